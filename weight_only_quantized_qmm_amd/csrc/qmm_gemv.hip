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
// Work decomposition: a workgroup computes 16 output columns with 4 waves of 4, or 10 with
// 5 waves of 2, over one partition. A workgroup's time follows the weight bytes it
// streams, so the host takes the layout whose busiest CU holds fewer rows (for one or two
// activation rows; down at M = 1 on MI355X: 256 workgroups of 10 rows instead of 160 of
// 16, 7.6 -> 6.5 us). A wave's work is split into items of RG rows (4 or 2) by one
// chunk; lane l takes items l, l+64, ..., so consecutive lanes read consecutive 16 bytes
// of a row (whole cache lines) and every lane gets the same number of items to within
// one. Per-lane sums are reduced across the wave in a fixed order (deterministic).
//
// Schedule: the dispatch is over before the first weight byte arrives unless every load
// is in flight early, so a thread issues its activation loads, then the scale and bias of
// its items, then all of its weight loads, before any arithmetic. The activation staging
// waits only for the activation loads (they return first) and the barrier after it waits
// only for the LDS writes, so both overlap the weight stream; each item's arithmetic then
// waits for its own weights. Issued after the weights, the staging loads had cost a
// second and third memory round trip per call (decode shapes of Qwen3-4B on MI355X:
// 15-35 % of the call at M = 1).
#include "qmm_device.h"
#include "qmm_launch.h"

using namespace qmm_dev;

namespace {


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

// LDS writes of this wave done, then the workgroup barrier; the memory clobber keeps the
// compiler from moving LDS accesses across it. Unlike __syncthreads() it does not wait for
// the weight loads still in flight.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// RPW rows (output columns) per wave, NW waves per workgroup: 4 x 4 or 2 x 5.
template <int MM, int RG, int NCHM, int RPW, int NW>
__global__ void __launch_bounds__(64 * NW)
gemv_kernel(const uint16_t *__restrict__ A, const uint32_t *__restrict__ Wq, const uint16_t *__restrict__ scale,
            const uint16_t *__restrict__ bias, uint16_t *__restrict__ out, int M, int N, int K, int gpp)
{
    extern __shared__ __attribute__((aligned(16))) char lds[];
    asm volatile("" ::"s"(A), "s"(Wq), "s"(scale), "s"(bias), "s"(out));
    constexpr int NT = 64 * NW;            // threads of the workgroup
    constexpr int NRG = RPW / RG;          // row groups of a wave
    const int G = K >> 7;
    const int p = blockIdx.y;
    const int g0 = p * gpp;
    const int k0 = g0 * 128;
    const int WP = gpp * 16;  // packed words of a row in the partition
    const int CP = gpp * 4;   // 16-byte chunks of a row in the partition
    const int n_blk = blockIdx.x * (RPW * NW);
    uint4 *apair = reinterpret_cast<uint4 *>(lds);             // [MM][WP]: pairs of word w
    float *asum = reinterpret_cast<float *>(apair + MM * WP);  // [MM][CP]

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    // 1. Activation loads: each thread owns up to ITEMS (row, chunk) items of the partition
    // (rows m >= M stage zeros). CPMAX: the most chunks a row's partition has
    // (gemv_split_fits).
    constexpr int CPMAX = MM == 1 || MM == 2 ? 320 : MM == 4 ? 240 : 128;
    constexpr int ITEMS = (MM * CPMAX + NT - 1) / NT;
    uint4 av[ITEMS][4];
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
        const int idx = threadIdx.x + NT * it;
        const int m = idx / CP, c = idx - m * CP;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            av[it][w] = make_uint4(0u, 0u, 0u, 0u);
            if (idx < MM * CP && m < M)
                av[it][w] = *reinterpret_cast<const uint4 *>(A + (size_t)m * (size_t)K + k0 + 32 * c + 8 * w);
        }
    }
    // 2. Scale/bias, then weights, of the lane's items: item idx of the wave is row group
    // idx / CP (rows RG*rg .. RG*rg + RG-1 of the wave), chunk idx % CP. Items past the
    // wave's last re-read its last one, rows past N re-read row N-1 (neither is used).
    const int nit = NRG * CP;
    uint32_t sbv[NCHM][RG];
    uint4 wr[NCHM][RG];
#pragma unroll
    for (int i = 0; i < NCHM; ++i) {
        const int idx = min(lane + 64 * i, nit - 1);
        const int rg = idx / CP, c = idx - rg * CP;
#pragma unroll
        for (int rr = 0; rr < RG; ++rr) {
            const int n = min(n_blk + RPW * wave + RG * rg + rr, N - 1);
            const size_t e = (size_t)n * G + g0 + (c >> 2);
            sbv[i][rr] = (uint32_t)scale[e] | ((uint32_t)bias[e] << 16);
        }
    }
#pragma unroll
    for (int i = 0; i < NCHM; ++i) {
        const int idx = min(lane + 64 * i, nit - 1);
        const int rg = idx / CP, c = idx - rg * CP;
#pragma unroll
        for (int rr = 0; rr < RG; ++rr) {
            const int n = min(n_blk + RPW * wave + RG * rg + rr, N - 1);
            wr[i][rr] = reinterpret_cast<const uint4 *>(Wq + (size_t)n * (size_t)(K >> 3) + (k0 >> 3))[c];
        }
    }
    // Without the fence the compiler sinks each load next to its first use.
    __builtin_amdgcn_sched_barrier(0);

    // 3. Activation pairs (a[i], a[i+4]) of each packed word and the chunk sums into LDS.
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
        const int idx = threadIdx.x + NT * it;
        if (idx >= MM * CP) break;
        const int m = idx / CP, c = idx - m * CP;
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const uint32_t e[4] = {av[it][w].x, av[it][w].y, av[it][w].z, av[it][w].w};
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
    lds_barrier();

    // 4. Each item as its weights arrive.
    float acc[RPW][MM];
#pragma unroll
    for (int r = 0; r < RPW; ++r)
#pragma unroll
        for (int m = 0; m < MM; ++m) acc[r][m] = 0.f;
#pragma unroll
    for (int i = 0; i < NCHM; ++i) {
        const int idx = lane + 64 * i;
        if (idx >= nit) break;
        const int rg = idx / CP, c = idx - rg * CP;
        uint32_t pr[RG][16];
        float sc[RG], bi[RG];
#pragma unroll
        for (int rr = 0; rr < RG; ++rr) {
            const uint32_t wv[4] = {wr[i][rr].x, wr[i][rr].y, wr[i][rr].z, wr[i][rr].w};
#pragma unroll
            for (int w = 0; w < 4; ++w)
#pragma unroll
                for (int k = 0; k < 4; ++k) pr[rr][4 * w + k] = nib_pair(wv[w], k);
            sc[rr] = bf16_to_f32(sbv[i][rr] & 0xFFFFu);
            bi[rr] = bf16_to_f32(sbv[i][rr] >> 16);
        }
#pragma unroll
        for (int m = 0; m < MM; ++m) {
            uint4 ap[4];
#pragma unroll
            for (int w = 0; w < 4; ++w) ap[w] = apair[m * WP + 4 * c + w];
            const float s = asum[m * CP + c];
#pragma unroll
            for (int rr = 0; rr < RG; ++rr) {
                float q = 0.f;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    q = dot2(pr[rr][4 * w + 0], ap[w].x, q);
                    q = dot2(pr[rr][4 * w + 1], ap[w].y, q);
                    q = dot2(pr[rr][4 * w + 2], ap[w].z, q);
                    q = dot2(pr[rr][4 * w + 3], ap[w].w, q);
                }
                const float v = sc[rr] * (q - 128.f * s) + bi[rr] * s;
#pragma unroll
                for (int g = 0; g < NRG; ++g)
                    if (NRG == 1 || rg == g) acc[RG * g + rr][m] += v;
            }
        }
    }

    // Wave sums in a fixed order (within rows of 16 lanes, then across them); lane 0 stores.
#pragma unroll
    for (int r = 0; r < RPW; ++r)
#pragma unroll
        for (int m = 0; m < MM; ++m) {
            float v = acc[r][m];
            v = xor32_add(xor16_add(row16_sum(v)));
            acc[r][m] = v;
        }
    if (lane == 0) {
        uint16_t *dst = out + (size_t)p * (size_t)M * (size_t)N;
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
            const int n = n_blk + RPW * wave + r;
            if (n >= N) continue;
#pragma unroll
            for (int m = 0; m < MM; ++m)
                if (m < M) dst[(size_t)m * (size_t)N + n] = (uint16_t)f32_to_bf16(acc[r][m]);
        }
    }
}

template <int MM, int RG, int NCHM, int RPW, int NW>
hipError_t launch_cfg(const void *A, const void *Wq, const void *scale, const void *bias, void *out, int M, int N,
                      int K, int s, hipStream_t stream)
{
    const int gpp = (K / 128) / s;
    const size_t lds = (size_t)MM * gpp * 16 * 16 + (size_t)MM * gpp * 4 * 4;
    const dim3 grid((N + RPW * NW - 1) / (RPW * NW), s);
    (void)hipGetLastError();
    hipLaunchKernelGGL((gemv_kernel<MM, RG, NCHM, RPW, NW>), grid, dim3(64 * NW), lds, stream,
                       static_cast<const uint16_t *>(A), static_cast<const uint32_t *>(Wq),
                       static_cast<const uint16_t *>(scale), static_cast<const uint16_t *>(bias),
                       static_cast<uint16_t *>(out), M, N, K, gpp);
    return hipGetLastError();
}

// Rows of the busiest CU when ceil(N / rows) * s workgroups of `rows` rows spread evenly.
long long busiest_rows(int N, int s, int rows)
{
    const long long wgs = (long long)((N + rows - 1) / rows) * s;
    return (wgs + 255) / 256 * rows;
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
    const int cp = kp / 32;
    const int it4 = (cp + 63) / 64, it2 = (2 * cp + 63) / 64;
    const auto bucket = [](int nch) { return nch <= 2 ? 2 : nch <= 3 ? 3 : nch <= 5 ? 5 : 10; };
    // Workgroup layout: 16 rows (4 waves of 4) or 10 rows (5 waves of 2). A workgroup's time
    // follows the weight bytes it streams, so for one or two activation rows the layout whose
    // busiest CU holds fewer rows wins (down at M = 1: 256 workgroups of 10 rows instead of
    // 160 of 16). The 2-row waves take items of one row pair and one chunk.
    if (mm <= 2 && busiest_rows(N, s, 10) < busiest_rows(N, s, 16)) {
        const int nchm = bucket(it4);
#define QMM_G10(MM_, NCH_)                                                                                       \
    if (mm == MM_ && nchm == NCH_) return launch_cfg<MM_, 2, NCH_, 2, 5>(A, Wq, scale, bias, out, M, N, K, s, stream);
        QMM_G10(1, 2) QMM_G10(1, 3) QMM_G10(1, 5) QMM_G10(2, 2) QMM_G10(2, 3) QMM_G10(2, 5)
#undef QMM_G10
        return hipErrorInvalidValue;
    }
    // Rows per lane item: RG = 4 shares each chunk's activation reads over 4 rows; RG = 2
    // makes the items half as large, which evens out the lanes' work when a row's chunks are
    // not a multiple of 64 (K = 2560: 80 chunks, 2 items of 4 rows on some lanes, 1 on the
    // others). Per lane the cost is about items * (RG + MM/2) row-chunks of arithmetic;
    // ties go to 4 (decode sweeps of the Qwen3-4B projections on MI355X).
    const int rg = it2 * (4 + mm) < it4 * (8 + mm) ? 2 : 4;
    const int nchm = bucket(rg == 4 ? it4 : it2);
#define QMM_G(MM_, RG_, NCH_)                                                                                    \
    if (mm == MM_ && rg == RG_ && nchm == NCH_)                                                                  \
        return launch_cfg<MM_, RG_, NCH_, 4, 4>(A, Wq, scale, bias, out, M, N, K, s, stream);
#define QMM_GM(MM_) QMM_G(MM_, 4, 2) QMM_G(MM_, 4, 3) QMM_G(MM_, 4, 5) \
                    QMM_G(MM_, 2, 2) QMM_G(MM_, 2, 3) QMM_G(MM_, 2, 5) QMM_G(MM_, 2, 10)
    QMM_GM(1) QMM_GM(2) QMM_GM(4)
    QMM_G(8, 4, 2) QMM_G(8, 2, 2) QMM_G(8, 2, 3) QMM_G(8, 2, 5)
#undef QMM_GM
#undef QMM_G
    return hipErrorInvalidValue;
}

}  // namespace qmm_impl
