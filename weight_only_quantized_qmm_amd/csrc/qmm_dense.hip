// qmm_dense.hip -- dense bf16 split-K matmul C = A . B^T for gfx950.
//
// gpu-kernels-explained "Split-K, streams and overlap", Concept: a small output
// with a long reduction gives too few output tiles to fill the GPU; cutting k
// into s slices multiplies the blocks by s, each block computes one tile over
// one slice, and a second pass adds the s partial sums. Here the slices are
// near-equal runs of 32-value granules (one MFMA depth): partition p covers
// granules [floor(p*U/s), floor((p+1)*U/s)), U = K/32. Each partition writes
// an fp32 partial plane (plain stores, no atomics); with s = 1 the block writes
// the bf16 result directly.
//
// Work decomposition: a workgroup is 2 x 2 wave64s; each wave owns a
// (16*MT) x (16*NS) output tile and streams its A rows and B rows straight from
// global memory with 128-bit loads (lane l: row l%16 of a subtile, eight k
// values of slot l/16 of the current 32-deep granule), prefetching the next
// granule while the MFMAs of the current one run.
#include "qmm_device.h"
#include "qmm_launch.h"

using namespace qmm_dev;

namespace {

template <int MT, int NS, bool F32_OUT>
__global__ void __launch_bounds__(256)
dense_kernel(const uint16_t *__restrict__ A, const uint16_t *__restrict__ B, void *__restrict__ out,
             int M, int N, int K, int s, int vec_store)
{
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    const int r = lane & 15;
    const int slot = lane >> 4;
    const int m_wave = blockIdx.y * (2 * 16 * MT) + (wave >> 1) * (16 * MT);
    const int n_wave = blockIdx.x * (2 * 16 * NS) + (wave & 1) * (16 * NS);
    if (m_wave >= M || n_wave >= N) return;  // no block-wide synchronisation follows
    const int p = blockIdx.z;
    const long long U = K >> 5;
    const int u_begin = (int)(((long long)p * U) / s);
    const int u_end = (int)(((long long)(p + 1) * U) / s);

    const uint4 *bptr[NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) {
        const int n = min(n_wave + 16 * j + r, N - 1);
        bptr[j] = reinterpret_cast<const uint4 *>(B + (size_t)n * (size_t)K) + slot;
    }
    const uint4 *aptr[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
        const int m = min(m_wave + 16 * i + r, M - 1);
        aptr[i] = reinterpret_cast<const uint4 *>(A + (size_t)m * (size_t)K) + slot;
    }

    f32x4 acc[MT][NS];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NS; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    uint4 bn[NS], an[MT];
    if (u_begin < u_end) {
#pragma unroll
        for (int j = 0; j < NS; ++j) bn[j] = bptr[j][4 * u_begin];
#pragma unroll
        for (int i = 0; i < MT; ++i) an[i] = aptr[i][4 * u_begin];
    }
    for (int u = u_begin; u < u_end; ++u) {
        uint4 bc[NS], ac[MT];
#pragma unroll
        for (int j = 0; j < NS; ++j) bc[j] = bn[j];
#pragma unroll
        for (int i = 0; i < MT; ++i) ac[i] = an[i];
        if (u + 1 < u_end) {
#pragma unroll
            for (int j = 0; j < NS; ++j) bn[j] = bptr[j][4 * (u + 1)];
#pragma unroll
            for (int i = 0; i < MT; ++i) an[i] = aptr[i][4 * (u + 1)];
        }
#pragma unroll
        for (int j = 0; j < NS; ++j)
#pragma unroll
            for (int i = 0; i < MT; ++i)
                acc[i][j] = mfma16x16x32(as_bf16x8(bc[j]), as_bf16x8(ac[i]), acc[i][j]);
    }

    // Lane holds C[m_wave + 16i + r][n_wave + 16j + 4*slot + e], e = 0..3.
#pragma unroll
    for (int i = 0; i < MT; ++i) {
        const int m = m_wave + 16 * i + r;
        if (m >= M) continue;
#pragma unroll
        for (int j = 0; j < NS; ++j) {
            const int n0 = n_wave + 16 * j + 4 * slot;
            const size_t off = (size_t)m * (size_t)N + n0;
            if (F32_OUT) {
                float *dst = static_cast<float *>(out) + (size_t)p * (size_t)M * (size_t)N + off;
                if (vec_store && n0 + 3 < N) {
                    *reinterpret_cast<float4 *>(dst) =
                        make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (n0 + e < N) dst[e] = acc[i][j][e];
                }
            } else {
                uint16_t *dst = static_cast<uint16_t *>(out) + off;
                if (vec_store && n0 + 3 < N) {
                    uint2 v;
                    v.x = pack_bf16x2(acc[i][j][0], acc[i][j][1]);
                    v.y = pack_bf16x2(acc[i][j][2], acc[i][j][3]);
                    *reinterpret_cast<uint2 *>(dst) = v;
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (n0 + e < N) dst[e] = (uint16_t)f32_to_bf16(acc[i][j][e]);
                }
            }
        }
    }
}

template <int MT, int NS>
hipError_t launch_tile(const void *A, const void *B, void *out, bool f32_out, int M, int N, int K,
                       int s, bool vec_store, hipStream_t stream)
{
    const int block_m = 2 * 16 * MT, block_n = 2 * 16 * NS;
    dim3 grid((N + block_n - 1) / block_n, (M + block_m - 1) / block_m, s);
    (void)hipGetLastError();
    if (f32_out)
        hipLaunchKernelGGL((dense_kernel<MT, NS, true>), grid, dim3(256), 0, stream,
                           static_cast<const uint16_t *>(A), static_cast<const uint16_t *>(B), out,
                           M, N, K, s, vec_store ? 1 : 0);
    else
        hipLaunchKernelGGL((dense_kernel<MT, NS, false>), grid, dim3(256), 0, stream,
                           static_cast<const uint16_t *>(A), static_cast<const uint16_t *>(B), out,
                           M, N, K, s, vec_store ? 1 : 0);
    return hipGetLastError();
}

}  // namespace

namespace qmm_impl {

hipError_t launch_dense(DenseTile tile, const void *A, const void *B, void *out, bool f32_out,
                        int M, int N, int K, int s, bool vec_store, hipStream_t stream)
{
    if (tile.mt == 4 && tile.ns == 4)
        return launch_tile<4, 4>(A, B, out, f32_out, M, N, K, s, vec_store, stream);
    if (tile.mt == 2 && tile.ns == 2)
        return launch_tile<2, 2>(A, B, out, f32_out, M, N, K, s, vec_store, stream);
    return hipErrorInvalidValue;
}

}  // namespace qmm_impl
