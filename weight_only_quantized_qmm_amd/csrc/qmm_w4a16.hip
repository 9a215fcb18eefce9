// qmm_w4a16.hip -- W4A16 group-128 matmul kernel for gfx950, unsplit and split-K.
//
// One kernel serves both forms (tiny-llm "Week 2 Day 7: Split-K Prefill",
// Task 2: each partition reuses the unsplit tile, loader and dequantizer):
// blockIdx.z is the partition index p, the partition covers groups
// [p*gpp, (p+1)*gpp) of the reduction, and the block writes its tile into plane
// p of `out`. With s = 1 the single plane is C itself, so the unsplit kernel and
// the split kernel are one code path and the s = 1 result is the same launch
// however it was requested. Planes are written with plain stores, no atomics.
//
// Work decomposition (MI355X): a workgroup is 4 wave64s side by side along N.
// Each wave owns 16*NS output columns and all 16*MT rows of the block, so every
// weight element is loaded and dequantised exactly once per block. Weights are
// loaded straight from global memory into registers with 128-bit loads: lane l
// holds row n = l%16 of a 16-column subtile and the 32 reduction values
// 32*(l/16) .. +31 of the current group (one uint4 = four packed words). Word t
// of that uint4 becomes the lane's eight bf16 operand values for the t-th
// 32-deep MFMA of the group, and the activation fragment the lane supplies for
// that MFMA is the same eight k values of its row m (one 16-byte load). The
// next group's weights are prefetched into registers while the current group
// is computed.
//
// Dequantisation: w = scale * q + bias in fp32 (one FMA per value), rounded to
// bf16 for the MFMA; the accumulator is fp32. The output is rounded once to
// bf16 (round to nearest even).
#include "qmm_device.h"
#include "qmm_launch.h"

using namespace qmm_dev;

namespace {

__device__ __forceinline__ bf16x8 dequant_word(uint32_t x, float sc, float bi) {
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        r[i] = (__bf16)__builtin_fmaf((float)((x >> (4 * i)) & 0xFu), sc, bi);
    return r;
}

template <int MT, int NS>
__global__ void __launch_bounds__(256)
w4a16_kernel(const uint16_t *__restrict__ A, const uint32_t *__restrict__ Wq,
             const uint16_t *__restrict__ scale, const uint16_t *__restrict__ bias,
             uint16_t *__restrict__ out, int M, int N, int K, int gpp, int vec_store)
{
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    const int r = lane & 15;
    const int slot = lane >> 4;
    const int n_wave = (blockIdx.x * 4 + wave) * (16 * NS);
    if (n_wave >= N) return;  // no block-wide synchronisation follows
    const int m_blk = blockIdx.y * (16 * MT);
    const int G = K >> 7;
    const int g_begin = blockIdx.z * gpp;
    const int g_end = g_begin + gpp;
    uint16_t *dst = out + (size_t)blockIdx.z * (size_t)M * (size_t)N;

    // Rows beyond N or M read a valid row (the last one); their results land in
    // output rows / columns that are never stored.
    const uint4 *wptr[NS];
    const uint16_t *sptr[NS];
    const uint16_t *bptr[NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) {
        const int n = min(n_wave + 16 * j + r, N - 1);
        wptr[j] = reinterpret_cast<const uint4 *>(Wq + (size_t)n * (size_t)(K >> 3)) + slot;
        sptr[j] = scale + (size_t)n * G;
        bptr[j] = bias + (size_t)n * G;
    }
    const uint4 *aptr[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
        const int m = min(m_blk + 16 * i + r, M - 1);
        aptr[i] = reinterpret_cast<const uint4 *>(A + (size_t)m * (size_t)K) + 4 * slot;
    }

    f32x4 acc[MT][NS];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NS; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    uint4 wnext[NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) wnext[j] = wptr[j][4 * g_begin];

    for (int g = g_begin; g < g_end; ++g) {
        uint4 wcur[NS];
#pragma unroll
        for (int j = 0; j < NS; ++j) wcur[j] = wnext[j];
        if (g + 1 < g_end) {
#pragma unroll
            for (int j = 0; j < NS; ++j) wnext[j] = wptr[j][4 * (g + 1)];
        }
        float sc[NS], bi[NS];
#pragma unroll
        for (int j = 0; j < NS; ++j) {
            sc[j] = bf16_to_f32(sptr[j][g]);
            bi[j] = bf16_to_f32(bptr[j][g]);
        }
        uint4 av[MT][4];
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int t = 0; t < 4; ++t) av[i][t] = aptr[i][16 * g + t];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
#pragma unroll
            for (int j = 0; j < NS; ++j) {
                const bf16x8 b = dequant_word(word_of(wcur[j], t), sc[j], bi[j]);
#pragma unroll
                for (int i = 0; i < MT; ++i) acc[i][j] = mfma16x16x32(b, as_bf16x8(av[i][t]), acc[i][j]);
            }
        }
    }

    // Lane holds C[m_blk + 16i + r][n_wave + 16j + 4*slot + e], e = 0..3.
#pragma unroll
    for (int i = 0; i < MT; ++i) {
        const int m = m_blk + 16 * i + r;
        if (m >= M) continue;
#pragma unroll
        for (int j = 0; j < NS; ++j) {
            const int n0 = n_wave + 16 * j + 4 * slot;
            uint16_t *p = dst + (size_t)m * (size_t)N + n0;
            if (vec_store && n0 + 3 < N) {
                uint2 v;
                v.x = pack_bf16x2(acc[i][j][0], acc[i][j][1]);
                v.y = pack_bf16x2(acc[i][j][2], acc[i][j][3]);
                *reinterpret_cast<uint2 *>(p) = v;
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (n0 + e < N) p[e] = (uint16_t)f32_to_bf16(acc[i][j][e]);
            }
        }
    }
}

template <int MT, int NS>
hipError_t launch_tile(const void *A, const void *Wq, const void *scale, const void *bias, void *out,
                       int M, int N, int K, int s, bool vec_store, hipStream_t stream)
{
    const int block_n = 4 * 16 * NS, block_m = 16 * MT;
    dim3 grid((N + block_n - 1) / block_n, (M + block_m - 1) / block_m, s);
    const int gpp = (K / 128) / s;
    (void)hipGetLastError();  // launches report through the thread's last-error slot
    hipLaunchKernelGGL((w4a16_kernel<MT, NS>), grid, dim3(256), 0, stream,
                       static_cast<const uint16_t *>(A), static_cast<const uint32_t *>(Wq),
                       static_cast<const uint16_t *>(scale), static_cast<const uint16_t *>(bias),
                       static_cast<uint16_t *>(out), M, N, K, gpp, vec_store ? 1 : 0);
    return hipGetLastError();
}

}  // namespace

namespace qmm_impl {

hipError_t launch_w4a16(W4A16Tile tile, const void *A, const void *Wq, const void *scale,
                        const void *bias, void *out, int M, int N, int K, int s, bool vec_store,
                        hipStream_t stream)
{
#define QMM_TILE(MT_, NS_)                                                               \
    if (tile.mt == MT_ && tile.ns == NS_)                                                \
        return launch_tile<MT_, NS_>(A, Wq, scale, bias, out, M, N, K, s, vec_store, stream);
    QMM_TILE(1, 1) QMM_TILE(1, 2) QMM_TILE(1, 4)
    QMM_TILE(2, 1) QMM_TILE(2, 2) QMM_TILE(2, 4)
    QMM_TILE(4, 1) QMM_TILE(4, 2) QMM_TILE(4, 4)
    QMM_TILE(8, 1) QMM_TILE(8, 2) QMM_TILE(8, 4)
#undef QMM_TILE
    return hipErrorInvalidValue;
}

}  // namespace qmm_impl
