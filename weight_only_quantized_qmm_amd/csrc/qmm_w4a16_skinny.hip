// qmm_w4a16_skinny.hip -- weight-only quantized matmul kernel for few rows (M <= 64) on gfx950:
// W4A16 group 128, and the other formats of the library (4- or 8-bit codes, groups of
// 32, 64 or 128 values).
//
// Same contract as the other W4A16 kernels (tiny-llm "Week 2 Day 7: Split-K
// Prefill", Task 2): blockIdx.z is the partition p, the workgroup covers groups
// [p*gpp, (p+1)*gpp) of the reduction and writes its tile into plane p of `out`
// (C itself when s = 1), with plain stores and no atomics.
//
// With few rows the op streams the packed weights once and is bound by memory
// latency and bandwidth, not by the matrix cores (a dispatch on MI355X costs about
// 1.6 us before the first byte arrives). The design therefore maximises the bytes
// in flight per wave and keeps the work in one dispatch where possible:
//   * a workgroup owns a (16*MT) x (16*NS) output tile and up to 16 waves; the
//     waves split the tile's reduction range, wave w taking groups g0 + w,
//     g0 + w + WAVES, ... of its partition;
//   * each wave issues all loads of a round of up to GPW groups at once -- per
//     group and lane one 16-byte load of packed weights per 16-column subtile, four
//     16-byte loads of activations per 16-row subtile, and the scale/bias of its
//     rows -- then waits once and runs the MFMAs of the round;
//   * the waves' fp32 tiles meet in LDS and are summed in ascending wave order
//     (deterministic), rounded once to bf16 and stored with 8-byte stores.
// Weights are dequantised in registers: w = scale*q + bias in fp32, rounded to
// bf16 (each weight is used by all 16*MT rows of the tile from the same registers).
// A lane's share of a 128-value block is 32 consecutive values of one row: 16 bytes of
// 4-bit codes or 32 bytes of 8-bit codes, and the scale/bias of the group holding them
// (block g, lane slot c: group (4g + c) * 32 / group_size).
// The 16x16x32 MFMA takes the weights as its first operand, so a lane's result is
// four consecutive output columns of one row.
#include "qmm_device.h"
#include "qmm_launch.h"

using namespace qmm_dev;

namespace {

constexpr int MAX_WAVES = 16;

template <int BITS, int MT, int NS, int GPW, int MAXW>
__global__ void __launch_bounds__(64 * MAXW)
w4a16_skinny_kernel(const uint16_t *__restrict__ A, const uint32_t *__restrict__ Wq,
                    const uint16_t *__restrict__ scale, const uint16_t *__restrict__ bias,
                    void *__restrict__ out, int M, int N, int K, int gpp, int sub_shift, int vec_store,
                    int f32_part)
{
    constexpr int WV = BITS / 4;  // 16-byte weight loads per lane, group and 16-column subtile
    extern __shared__ __attribute__((aligned(16))) char red[];  // [WAVES][MT][NS][64] float4
    // Fetch every pointer argument up front, in the kernel's first scalar loads: left to
    // itself the compiler loads them after the first branch, one more dependent memory
    // round trip before the first weight load.
    asm volatile("" ::"s"(A), "s"(Wq), "s"(scale), "s"(bias), "s"(out));
    const int waves = __builtin_amdgcn_readfirstlane(blockDim.x >> 6);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    const int r = lane & 15;
    const int slot = lane >> 4;
    const int n_blk = blockIdx.x * (16 * NS);
    const int m_blk = blockIdx.y * (16 * MT);
    const int GG = (K >> 7) << sub_shift;  // scale/bias entries per row (128 / group_size per block)
    const int g0 = blockIdx.z * gpp;
    // this wave's groups: g0 + wave + waves*i, i < n_w
    const int n_w = (gpp - wave + waves - 1) / waves;

    const uint4 *wptr[NS];
    const uint16_t *sptr[NS];
    const uint16_t *bptr[NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) {
        const int n = min(n_blk + 16 * j + r, N - 1);  // rows past N read row N-1, never stored
        wptr[j] = reinterpret_cast<const uint4 *>(Wq + (size_t)n * (size_t)(K * BITS / 32)) + WV * slot;
        sptr[j] = scale + (size_t)n * GG + (slot >> (2 - sub_shift));
        bptr[j] = bias + (size_t)n * GG + (slot >> (2 - sub_shift));
    }
    const uint4 *aptr[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
        const int m = min(m_blk + 16 * i + r, M - 1);  // rows past M read row M-1, never stored
        aptr[i] = reinterpret_cast<const uint4 *>(A + (size_t)m * (size_t)K) + 4 * slot;
    }

    f32x4 acc[MT][NS];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NS; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int base = 0; base < n_w; base += GPW) {
        uint4 wv[GPW][NS][WV];
        uint4 av[GPW][MT][4];
        uint32_t sc[GPW][NS], bi[GPW][NS];
        // issue every load of the round before the first use
#pragma unroll
        for (int q = 0; q < GPW; ++q) {
            if (base + q >= n_w) break;  // uniform across the wave
            const int g = g0 + wave + waves * (base + q);
#pragma unroll
            for (int j = 0; j < NS; ++j) {
#pragma unroll
                for (int u = 0; u < WV; ++u) wv[q][j][u] = wptr[j][4 * WV * g + u];
                sc[q][j] = sptr[j][g << sub_shift];
                bi[q][j] = bptr[j][g << sub_shift];
            }
#pragma unroll
            for (int i = 0; i < MT; ++i)
#pragma unroll
                for (int t = 0; t < 4; ++t) av[q][i][t] = aptr[i][16 * g + t];
        }
        // Keep all of the round's loads ahead of the first MFMA: without this the
        // compiler sinks each group's loads next to its use, one round trip per group.
        asm volatile("" ::: "memory");
#pragma unroll
        for (int q = 0; q < GPW; ++q) {
            if (base + q >= n_w) break;  // uniform across the wave
#pragma unroll
            for (int j = 0; j < NS; ++j) {
                const float s_ = bf16_to_f32(sc[q][j]);
                const float b_ = bf16_to_f32(bi[q][j]);
                const float s512 = s_ * 512.f;
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    // step t: values 8t .. 8t+7 of the lane's 32 (one word of 4-bit codes,
                    // two words of 8-bit codes)
                    const bf16x8 b = as_bf16x8(
                        BITS == 4 ? dequant8(word_of(wv[q][j][0], t), s512, b_)
                                  : dequant8_u8(word_of(wv[q][j][(t >> 1) % WV], 2 * (t & 1)),
                                                word_of(wv[q][j][(t >> 1) % WV], 2 * (t & 1) + 1), s_, b_));
#pragma unroll
                    for (int i = 0; i < MT; ++i) acc[i][j] = mfma16x16x32(b, as_bf16x8(av[q][i][t]), acc[i][j]);
                }
            }
        }
    }

    // Cross-wave sum in LDS: wave w stores its tiles, then each of the MT*NS*64 lane-quads
    // (i, j, lane) is owned by one thread (strided over the workgroup), which adds the
    // waves' values in order w = 0, 1, ...
    f32x4 *red4 = reinterpret_cast<f32x4 *>(red);
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NS; ++j) red4[((wave * MT + i) * NS + j) * 64 + lane] = acc[i][j];
    __syncthreads();
    for (int t = threadIdx.x; t < MT * NS * 64; t += blockDim.x) {
        f32x4 sum = red4[t];
        for (int w = 1; w < waves; ++w) sum += red4[w * MT * NS * 64 + t];
        const int l = t & 63;
        const int j = (t >> 6) % NS;
        const int i = (t >> 6) / NS;
        const int m = m_blk + 16 * i + (l & 15);
        const int n = n_blk + 16 * j + 4 * (l >> 4);
        if (m < M) {
            // C (bf16) when unsplit, else plane blockIdx.z of bf16 or (f32_part) fp32 partials
            const size_t e = (size_t)blockIdx.z * (size_t)M * (size_t)N + (size_t)m * (size_t)N + n;
            if (f32_part && gridDim.z > 1) {
                float *dst = static_cast<float *>(out) + e;
                if (vec_store && n + 3 < N) {
                    *reinterpret_cast<float4 *>(dst) = make_float4(sum[0], sum[1], sum[2], sum[3]);
                } else {
#pragma unroll
                    for (int e2 = 0; e2 < 4; ++e2)
                        if (n + e2 < N) dst[e2] = sum[e2];
                }
            } else {
                uint16_t *dst = static_cast<uint16_t *>(out) + e;
                if (vec_store && n + 3 < N) {
                    uint2 v;
                    v.x = pack_bf16x2(sum[0], sum[1]);
                    v.y = pack_bf16x2(sum[2], sum[3]);
                    *reinterpret_cast<uint2 *>(dst) = v;
                } else {
#pragma unroll
                    for (int e2 = 0; e2 < 4; ++e2)
                        if (n + e2 < N) dst[e2] = (uint16_t)f32_to_bf16(sum[e2]);
                }
            }
        }
    }
}

template <int BITS, int MT, int NS, int GPW, int MAXW>
hipError_t launch_cfg(const void *A, const void *Wq, const void *scale, const void *bias, void *out, bool f32_part,
                      int M, int N, int K, int s, int sub_shift, int waves, bool vec_store, hipStream_t stream)
{
    const dim3 grid((N + 16 * NS - 1) / (16 * NS), (M + 16 * MT - 1) / (16 * MT), s);
    const int gpp = (K / 128) / s;
    const size_t lds = (size_t)waves * MT * NS * 64 * 16;
    if (waves > MAXW) return hipErrorInvalidValue;
    (void)hipGetLastError();
    hipLaunchKernelGGL((w4a16_skinny_kernel<BITS, MT, NS, GPW, MAXW>), grid, dim3(64 * waves), lds, stream,
                       static_cast<const uint16_t *>(A), static_cast<const uint32_t *>(Wq),
                       static_cast<const uint16_t *>(scale), static_cast<const uint16_t *>(bias),
                       out, M, N, K, gpp, sub_shift, vec_store ? 1 : 0, f32_part ? 1 : 0);
    return hipGetLastError();
}

}  // namespace

namespace qmm_impl {

// The host picks (mt, ns, gpw, waves) with SkinnyShape (qmm_launch.h). 32-column tiles
// (ns 2): mt 1 with up to 16 waves and gpw <= 3; mt 2 with up to 8 waves and gpw <= 3;
// mt 4 with up to 8 waves and gpw <= 2. 64-column tiles (ns 4), used when the 32-column
// grid would not fit on the GPU in one round: up to 8 waves, gpw <= 3, 2, 1 for mt 1, 2,
// 4 (register budgets of 128 VGPRs per lane at 16 waves, 256 at 8). 8-bit codes take one
// group less per round where the 4-bit limit is above one.
hipError_t launch_w4a16_skinny(WFormat fmt, int mt, int ns, int gpw, int waves, const void *A, const void *Wq,
                               const void *scale, const void *bias, void *out, bool f32_part, int M, int N, int K,
                               int s, bool vec_store, hipStream_t stream)
{
    if (waves < 1 || waves > MAX_WAVES || !format_supported(fmt)) return hipErrorInvalidValue;
    const int sub_shift = fmt.group == 128 ? 0 : fmt.group == 64 ? 1 : 2;
#define QMM_CFG(B_, MT_, NS_, GPW_, MAXW_)                                                                     \
    if (fmt.bits == B_ && mt == MT_ && ns == NS_ && gpw == GPW_)                                               \
        return launch_cfg<B_, MT_, NS_, GPW_, MAXW_>(A, Wq, scale, bias, out, f32_part, M, N, K, s, sub_shift,  \
                                                     waves, vec_store, stream);
    QMM_CFG(4, 1, 2, 1, 16) QMM_CFG(4, 1, 2, 2, 16) QMM_CFG(4, 1, 2, 3, 16)
    QMM_CFG(4, 2, 2, 1, 8) QMM_CFG(4, 2, 2, 2, 8) QMM_CFG(4, 2, 2, 3, 8)
    QMM_CFG(4, 4, 2, 1, 8) QMM_CFG(4, 4, 2, 2, 8)
    QMM_CFG(4, 1, 4, 1, 8) QMM_CFG(4, 1, 4, 2, 8) QMM_CFG(4, 1, 4, 3, 8)
    QMM_CFG(4, 2, 4, 1, 8) QMM_CFG(4, 2, 4, 2, 8)
    QMM_CFG(4, 4, 4, 1, 8)
    QMM_CFG(8, 1, 2, 1, 16) QMM_CFG(8, 1, 2, 2, 16)
    QMM_CFG(8, 2, 2, 1, 8) QMM_CFG(8, 2, 2, 2, 8)
    QMM_CFG(8, 4, 2, 1, 8)
    QMM_CFG(8, 1, 4, 1, 8) QMM_CFG(8, 1, 4, 2, 8)
    QMM_CFG(8, 2, 4, 1, 8)
    QMM_CFG(8, 4, 4, 1, 8)
#undef QMM_CFG
    return hipErrorInvalidValue;
}

}  // namespace qmm_impl
