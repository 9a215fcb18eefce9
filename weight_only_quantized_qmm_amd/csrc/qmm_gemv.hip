// qmm_gemv.hip -- W4A16 group-128 matrix-vector kernel for decode (M <= 8) on gfx950.
//
// tiny-llm "Week 2 Day 7: Split-K Prefill", Benchmark Analysis: decode (M = 1) runs
// on a separate matvec kernel; the split-K matmul pads M up to its MFMA tile. This is
// that matvec for one to eight rows: no matrix cores, no padding, every packed weight
// read once per call, with the same split contract as the matmul kernels (Task 2:
// partition p = groups [p*gpp, (p+1)*gpp), bf16 plane p of `out`, or C when s = 1).
//
// Arithmetic: for a 16-byte chunk of a weight row (32 consecutive k, a quarter of a
// group, four packed words) a lane forms bf16 pairs (128 + q[k+i], 128 + q[k+i+4])
// straight from the nibbles (mask and or: 128 + q is exact in bf16) and takes
// v_dot2_f32_bf16 against A arranged in the same pairs, then applies the group's
// affine transform through the chunk's A sum S:
//     sum_k A*(scale*q + bias) = scale * (sum_k A*(128 + q) - 128*S) + bias*S.
// A's pairs and chunk sums are staged in LDS once per workgroup and shared by its 16
// weight rows; the group's scale and bias likewise.
//
// Work decomposition: a workgroup of 4 waves computes 16 output columns (4 per wave)
// over one partition; lane l of a wave takes chunks l, l+64, ..., issuing all of its
// weight loads (NCH chunks x 4 rows) before any arithmetic. Lane partial sums are
// reduced across the wave in a fixed order (deterministic).
#include "qmm_device.h"
#include "qmm_launch.h"

using namespace qmm_dev;

namespace {

constexpr int ROWS_PER_WAVE = 4;
constexpr int ROWS_PER_WG = 16;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2(uint32_t x, uint32_t y, float acc)
{
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, x), __builtin_bit_cast(bf16x2_t, y), acc,
                                           false);
}

// Pair k (0..3) of a packed word: bf16 (128 + q[k]) in the low half, (128 + q[k+4]) in the high.
__device__ __forceinline__ uint32_t nib_pair(uint32_t w, int k)
{
    return ((w >> (4 * k)) & 0x000F000Fu) | 0x43004300u;
}

template <int MM, int NCH>
__global__ void __launch_bounds__(256)
gemv_kernel(const uint16_t *__restrict__ A, const uint32_t *__restrict__ Wq, const uint16_t *__restrict__ scale,
            const uint16_t *__restrict__ bias, uint16_t *__restrict__ out, int M, int N, int K, int gpp)
{
    extern __shared__ __attribute__((aligned(16))) char lds[];
    const int G = K >> 7;
    const int p = blockIdx.y;
    const int g0 = p * gpp;
    const int k0 = g0 * 128;
    const int WP = gpp * 16;  // packed words of a row in the partition
    const int CP = gpp * 4;   // 16-byte chunks of a row in the partition
    const int n_blk = blockIdx.x * ROWS_PER_WG;
    uint4 *apair = reinterpret_cast<uint4 *>(lds);                       // [MM][WP]: pairs of word w
    float *asum = reinterpret_cast<float *>(apair + MM * WP);            // [MM][CP]
    uint32_t *sb = reinterpret_cast<uint32_t *>(asum + MM * CP);         // [16][gpp]: scale | bias << 16

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    // Weight loads first: rows past N re-read row N-1, chunks past the partition re-read
    // its last chunk (neither is used).
    uint4 wr[ROWS_PER_WAVE][NCH];
#pragma unroll
    for (int r = 0; r < ROWS_PER_WAVE; ++r) {
        const int n = min(n_blk + ROWS_PER_WAVE * wave + r, N - 1);
        const uint4 *row = reinterpret_cast<const uint4 *>(Wq + (size_t)n * (size_t)(K >> 3) + (k0 >> 3));
#pragma unroll
        for (int i = 0; i < NCH; ++i) wr[r][i] = row[min(lane + 64 * i, CP - 1)];
    }

    // A in pair order and its chunk sums (rows m >= M are zero), then scale and bias.
    // Each thread owns up to ITEMS (row, chunk) items and issues all of their loads
    // before converting any, so the staging costs one memory round trip.
    constexpr int ITEMS = (MM * 10240 / 32 + 255) / 256 < 4 ? (MM * 10240 / 32 + 255) / 256 : 4;
    {
        uint4 av[ITEMS][4];
#pragma unroll
        for (int it = 0; it < ITEMS; ++it) {
            const int idx = threadIdx.x + 256 * it;
            const int m = idx / CP, c = idx - m * CP;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                av[it][w] = make_uint4(0u, 0u, 0u, 0u);
                if (idx < MM * CP && m < M)
                    av[it][w] = *reinterpret_cast<const uint4 *>(A + (size_t)m * (size_t)K + k0 + 32 * c + 8 * w);
            }
        }
#pragma unroll
        for (int it = 0; it < ITEMS; ++it) {
            const int idx = threadIdx.x + 256 * it;
            if (idx >= MM * CP) break;
            const int m = idx / CP, c = idx - m * CP;
            float s = 0.f;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const uint32_t e[4] = {av[it][w].x, av[it][w].y, av[it][w].z, av[it][w].w};
                // e[j]: values 2j (low half) and 2j+1 (high half); pair i = (a[i], a[i+4])
                uint4 pr;
                pr.x = (e[0] & 0xFFFFu) | (e[2] << 16);
                pr.y = (e[0] >> 16) | (e[2] & 0xFFFF0000u);
                pr.z = (e[1] & 0xFFFFu) | (e[3] << 16);
                pr.w = (e[1] >> 16) | (e[3] & 0xFFFF0000u);
                apair[m * WP + 4 * c + w] = pr;
#pragma unroll
                for (int j = 0; j < 4; ++j) s += bf16_to_f32(e[j] & 0xFFFFu) + bf16_to_f32(e[j] >> 16);
            }
            asum[m * CP + c] = s;
        }
    }
    for (int idx = threadIdx.x; idx < ROWS_PER_WG * gpp; idx += blockDim.x) {
        const int r = idx / gpp, g = idx - r * gpp;
        const int n = min(n_blk + r, N - 1);
        sb[idx] = (uint32_t)scale[(size_t)n * G + g0 + g] | ((uint32_t)bias[(size_t)n * G + g0 + g] << 16);
    }
    __syncthreads();

    float acc[ROWS_PER_WAVE][MM];
#pragma unroll
    for (int r = 0; r < ROWS_PER_WAVE; ++r)
#pragma unroll
        for (int m = 0; m < MM; ++m) acc[r][m] = 0.f;

#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int c = lane + 64 * i;
        if (c >= CP) break;  // the lane's remaining chunks are all past the partition
        uint32_t pr[ROWS_PER_WAVE][16];
        float sc[ROWS_PER_WAVE], bi[ROWS_PER_WAVE];
#pragma unroll
        for (int r = 0; r < ROWS_PER_WAVE; ++r) {
            const uint32_t wv[4] = {wr[r][i].x, wr[r][i].y, wr[r][i].z, wr[r][i].w};
#pragma unroll
            for (int w = 0; w < 4; ++w)
#pragma unroll
                for (int k = 0; k < 4; ++k) pr[r][4 * w + k] = nib_pair(wv[w], k);
            const uint32_t v = sb[(ROWS_PER_WAVE * wave + r) * gpp + (c >> 2)];
            sc[r] = bf16_to_f32(v & 0xFFFFu);
            bi[r] = bf16_to_f32(v >> 16);
        }
#pragma unroll
        for (int m = 0; m < MM; ++m) {
            uint4 ap[4];
#pragma unroll
            for (int w = 0; w < 4; ++w) ap[w] = apair[m * WP + 4 * c + w];
            const float s = asum[m * CP + c];
#pragma unroll
            for (int r = 0; r < ROWS_PER_WAVE; ++r) {
                float q = 0.f;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    q = dot2(pr[r][4 * w + 0], ap[w].x, q);
                    q = dot2(pr[r][4 * w + 1], ap[w].y, q);
                    q = dot2(pr[r][4 * w + 2], ap[w].z, q);
                    q = dot2(pr[r][4 * w + 3], ap[w].w, q);
                }
                acc[r][m] += sc[r] * (q - 128.f * s) + bi[r] * s;
            }
        }
    }

    // Wave sums, butterfly in a fixed order; lane 0 stores.
#pragma unroll
    for (int r = 0; r < ROWS_PER_WAVE; ++r)
#pragma unroll
        for (int m = 0; m < MM; ++m) {
            float v = acc[r][m];
#pragma unroll
            for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
            acc[r][m] = v;
        }
    if (lane == 0) {
        uint16_t *dst = out + (size_t)p * (size_t)M * (size_t)N;
#pragma unroll
        for (int r = 0; r < ROWS_PER_WAVE; ++r) {
            const int n = n_blk + ROWS_PER_WAVE * wave + r;
            if (n >= N) continue;
#pragma unroll
            for (int m = 0; m < MM; ++m)
                if (m < M) dst[(size_t)m * (size_t)N + n] = (uint16_t)f32_to_bf16(acc[r][m]);
        }
    }
}

template <int MM, int NCH>
hipError_t launch_cfg(const void *A, const void *Wq, const void *scale, const void *bias, void *out, int M, int N,
                      int K, int s, hipStream_t stream)
{
    const int gpp = (K / 128) / s;
    const size_t lds = (size_t)MM * gpp * 16 * 16 + (size_t)MM * gpp * 4 * 4 + (size_t)ROWS_PER_WG * gpp * 4;
    const dim3 grid((N + ROWS_PER_WG - 1) / ROWS_PER_WG, s);
    (void)hipGetLastError();
    hipLaunchKernelGGL((gemv_kernel<MM, NCH>), grid, dim3(256), lds, stream, static_cast<const uint16_t *>(A),
                       static_cast<const uint32_t *>(Wq), static_cast<const uint16_t *>(scale),
                       static_cast<const uint16_t *>(bias), static_cast<uint16_t *>(out), M, N, K, gpp);
    return hipGetLastError();
}

}  // namespace

namespace qmm_impl {

hipError_t launch_w4a16_gemv(const void *A, const void *Wq, const void *scale, const void *bias, void *out, int M,
                             int N, int K, int s, hipStream_t stream)
{
    if (M < 1 || M > 8 || s < 1) return hipErrorInvalidValue;
    const int kp = K / s;
    const int mm = M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : 8;
    if (!gemv_split_fits(mm, kp)) return hipErrorInvalidValue;
    const int nch = (kp / 32 + 63) / 64;
#define QMM_G(MM_, NCH_)                                                                                         \
    if (mm == MM_ && nch == NCH_) return launch_cfg<MM_, NCH_>(A, Wq, scale, bias, out, M, N, K, s, stream);
    QMM_G(1, 1) QMM_G(1, 2) QMM_G(1, 3) QMM_G(1, 4) QMM_G(1, 5)
    QMM_G(2, 1) QMM_G(2, 2) QMM_G(2, 3) QMM_G(2, 4) QMM_G(2, 5)
    QMM_G(4, 1) QMM_G(4, 2) QMM_G(4, 3) QMM_G(4, 4)
    QMM_G(8, 1) QMM_G(8, 2)
#undef QMM_G
    return hipErrorInvalidValue;
}

}  // namespace qmm_impl
