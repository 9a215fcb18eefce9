// qmm_dense.hip -- dense bf16 split-K matmul C = A . B^T for gfx950.
//
// gpu-kernels-explained "Split-K, streams and overlap", Concept and Maths: a small
// output with a long reduction gives too few output tiles to fill the GPU; cutting k
// into s slices multiplies the workgroups by s, each computes one tile over one slice,
// and a second pass adds the s partial sums. Here the slices are near-equal runs of
// 64-value units when K is a multiple of 64 (32-value granules otherwise): partition p
// covers units [floor(p*U/s), floor((p+1)*U/s)), U = K/64 (K/32). Each partition writes an fp32 partial plane (plain stores, no atomics);
// with s = 1 the workgroup writes the bf16 result directly.
//
// Structure (the same pipeline as the large-M W4A16 kernel, without the dequant):
//   * a workgroup of 8 wave64s (two per SIMD) owns a 128 x 128 output tile (2 x 4 waves,
//     each a 64 x 32 block of 2 x 1 v_mfma_f32_32x32x16_bf16 accumulators);
//   * the partition is walked in stages of 64 reduction values; A and B rows of a stage
//     (128 bytes each) are copied global -> LDS by global_load_lds_dwordx4, two stages
//     ahead, into rings of three 16 KB slots each (96 KB); each wave waits for its own
//     copies of the next stage (s_waitcnt vmcnt) before the barrier that ends a stage;
//   * a partition with an odd number of 32-value granules ends with a half stage (32 values):
//     its copies re-read the first half of the row instead of reading past it, and
//     the two reduction steps of the missing half are skipped;
//   * LDS rows are 128 bytes, 16-byte chunk c of row r stored at c ^ ((r >> 1) & 7);
//   * B is the MFMA's first operand, so a lane's results are four consecutive output
//     columns of one row; the tile is then written through LDS as whole rows;
//   * workgroups are ordered so that each XCD computes whole partitions (see below).
#include "qmm_device.h"
#include "qmm_launch.h"

using namespace qmm_dev;

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int TM = 128, TN = 128, SK = 64;
constexpr int SLOT = TM * SK * 2;  // 16 KB per operand per stage
// Waves per workgroup: NW = 4 (2 x 2 waves of 64 x 64) or 8 (2 x 4 waves of 64 x 32, two per
// SIMD); each stage's 16 A and 16 B copies are shared out evenly.
template <int NW> struct DGeom {
    static constexpr int WN = NW / 2;        // waves along N
    static constexpr int NJ = 2 * 2 / WN;    // 32-column MFMA blocks per wave: 2 or 1
    static constexpr int CP = 16 / NW;       // copies of A (and of B) per wave and stage: 4 or 2
    static constexpr int NCOPY = 2 * CP;     // copies per wave per stage
};

typedef __attribute__((address_space(3))) void lds_void;

#define QMM_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (((n) >> 4) << 14) | (0x7 << 4) | (0xF << 8))

__device__ __forceinline__ uint32_t lds_addr(const void *p) { return (uint32_t)(uintptr_t)(const lds_void *)p; }

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// One 16-byte global -> LDS copy per lane (lane i lands at lds_off + 16*i), scalar base
// plus 32-bit lane offset; inline assembly so that the compiler does not wait for it.
__device__ __forceinline__ void copy16(uint32_t lds_off, uint32_t voff, const void *sbase)
{
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds_off), "v"(voff), "s"(sbase)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// Slots per operand: stage x in slot x % RING, copied RING - 1 stages ahead. Four or five
// slots (three or four stages in flight, 128 or 160 KB) were no faster on MI355X (cfg3, every s).
constexpr int RING = 3;
constexpr int AHEAD = RING - 1;

struct DenseLds {
    char a[RING * SLOT];
    char b[RING * SLOT];
};
static_assert(TM * TN * 4 <= sizeof(DenseLds), "the fp32 output tile is staged in the stage slots");

template <int NW>
struct DCtx {
    using GE = DGeom<NW>;
    const char *A, *B;     // A + m0*K, B + n0*K (bytes)
    int k_begin, k_end;    // reduction range of the partition
    uint32_t a_off[GE::CP][2];  // per-lane byte offsets of the A copies: full / half stage
    uint32_t b_off[GE::CP][2];
    uint32_t a_lds, b_lds; // this wave's copy destinations inside slot 0
    uint32_t a_rd[4], b_rd[4];  // operand read offsets, reduction step t
};

// Copies of stage x (k0 = k_begin + 64x) into slot `slot`: NCOPY instructions per wave.
template <int NW>
__device__ __forceinline__ void issue(const DCtx<NW> &c, int x, int slot)
{
    const int k0 = c.k_begin + SK * x;
    const int half = (c.k_end - k0) < SK ? 1 : 0;
    const char *Ab = c.A + 2 * (size_t)k0;
    const char *Bb = c.B + 2 * (size_t)k0;
#pragma unroll
    for (int j = 0; j < DGeom<NW>::CP; ++j) copy16(c.a_lds + (uint32_t)slot * SLOT + 1024u * j, c.a_off[j][half], Ab);
#pragma unroll
    for (int j = 0; j < DGeom<NW>::CP; ++j) copy16(c.b_lds + (uint32_t)slot * SLOT + 1024u * j, c.b_off[j][half], Bb);
}

template <int NW>
__device__ __forceinline__ void compute(const DCtx<NW> &c, const DenseLds &L, int slot, bool half,
                                        f32x16 (&acc)[2][DGeom<NW>::NJ])
{
    constexpr int NJ = DGeom<NW>::NJ;
    const char *As = L.a + slot * SLOT;
    const char *Bs = L.b + slot * SLOT;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        if (half && t >= 2) break;  // uniform: the missing half of a half stage
        bf16x8 af[2], bf[NJ];
#pragma unroll
        for (int i = 0; i < 2; ++i) af[i] = as_bf16x8(*reinterpret_cast<const uint4 *>(As + c.a_rd[t] + 4096 * i));
#pragma unroll
        for (int j = 0; j < NJ; ++j) bf[j] = as_bf16x8(*reinterpret_cast<const uint4 *>(Bs + c.b_rd[t] + 4096 * j));
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j) acc[i][j] = mfma32x32x16(bf[j], af[i], acc[i][j]);
    }
}

template <bool F32_OUT, int NW>
__global__ void __launch_bounds__(64 * NW, 1)
dense_kernel(const uint16_t *__restrict__ A, const uint16_t *__restrict__ B, void *__restrict__ out,
             int M, int N, int K, int s, int vec_store)
{
    using GE = DGeom<NW>;
    constexpr int NJ = GE::NJ;
    __shared__ __attribute__((aligned(1024))) DenseLds L;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    const int wm = wave / GE::WN, wn = wave % GE::WN;  // 64-row block, 32*NJ-column block
    const int num_m = (M + TM - 1) / TM;
    const int tiles = num_m * ((N + TN - 1) / TN);
    // XCD-aware order: the dispatcher sends workgroup b to XCD b % 8, so when the grid
    // is a multiple of 8 XCD x gets the contiguous run [x*G/8, (x+1)*G/8) of the
    // (partition, tile) list in partition-major order: whole partitions per XCD, whose
    // A and B slices are then read into that XCD's L2 once instead of once per XCD.
    const int total = tiles * s;
    const int b = blockIdx.x;
    const int L_idx = (total % 8 == 0) ? (b % 8) * (total / 8) + b / 8 : b;
    const int tile = L_idx % tiles;
    const int p = L_idx / tiles;
    const int m0 = (tile % num_m) * TM;
    const int n0 = (tile / num_m) * TN;
    // Partition bounds in units of 64 values (one stage, a whole 128-byte line of every row)
    // when K allows, else of 32-value granules: bounds off the 64-value grid make every
    // stage's 128 bytes of a row straddle two lines (cfg3 at s = 6 and 12: 49 and 33 us on
    // granule bounds, 34 and 24 us on 64-value bounds).
    const int UNIT = (K & 63) == 0 ? 64 : 32;
    const long long U = K / UNIT;
    const int u_lo = (int)(((long long)p * U) / s);
    const int u_hi = (int)(((long long)(p + 1) * U) / s);

    DCtx<NW> c;
    c.A = reinterpret_cast<const char *>(A) + 2 * (size_t)m0 * (size_t)K;
    c.B = reinterpret_cast<const char *>(B) + 2 * (size_t)n0 * (size_t)K;
    c.k_begin = UNIT * u_lo;
    c.k_end = UNIT * u_hi;
    // Copy j of wave w fills LDS rows 8q .. 8q+7, q = CP*w + j; lane i -> row 8q + i/8,
    // stored chunk i%8, logical chunk (i%8) ^ ((r>>1)&7); a half stage reads logical
    // chunk & 3 (the stage's valid half). Rows past M (N) re-read the last row.
#pragma unroll
    for (int j = 0; j < GE::CP; ++j) {
        const int r = 8 * (GE::CP * wave + j) + (lane >> 3);
        const int chunk = (lane & 7) ^ ((r >> 1) & 7);
        const int ra = min(m0 + r, M - 1) - m0;
        const int rb = min(n0 + r, N - 1) - n0;
        c.a_off[j][0] = 2u * ((uint32_t)ra * (uint32_t)K + 8u * (uint32_t)chunk);
        c.a_off[j][1] = 2u * ((uint32_t)ra * (uint32_t)K + 8u * (uint32_t)(chunk & 3));
        c.b_off[j][0] = 2u * ((uint32_t)rb * (uint32_t)K + 8u * (uint32_t)chunk);
        c.b_off[j][1] = 2u * ((uint32_t)rb * (uint32_t)K + 8u * (uint32_t)(chunk & 3));
    }
    c.a_lds = lds_addr(L.a) + 1024u * GE::CP * (uint32_t)wave;
    c.b_lds = lds_addr(L.b) + 1024u * GE::CP * (uint32_t)wave;
    {
        // Reduction step t, lane half h: logical chunk 2t + h (eight values) of the row.
        const int r32 = lane & 31, h = lane >> 5;
        const int arow = wm * 64 + r32;  // + 32 i: same swizzle
        const int brow = wn * 32 * NJ + r32;  // + 32 j
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            c.a_rd[t] = (uint32_t)(arow * 128 + 16 * ((2 * t + h) ^ ((arow >> 1) & 7)));
            c.b_rd[t] = (uint32_t)(brow * 128 + 16 * ((2 * t + h) ^ ((brow >> 1) & 7)));
        }
    }

    f32x16 acc[2][NJ];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    // Stages of the partition (the last one may be a half stage); past the last stage
    // the copies repeat it into a slot that is never read again, so every stage issues
    // NCOPY copies and the waits below are exact.
    const int nst = (c.k_end - c.k_begin + SK - 1) / SK;  // >= 1
#pragma unroll
    for (int x = 0; x < AHEAD; ++x) issue(c, min(x, nst - 1), x);
    QMM_WAIT_VMCNT(GE::NCOPY * (AHEAD - 1));  // stage 0 landed
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    int slot = 0;  // st % RING
    for (int st = 0; st < nst; ++st) {
        const int slot_issue = slot == 0 ? RING - 1 : slot - 1;  // (st + AHEAD) % RING: the slot stage st-1 used
        issue(c, min(st + AHEAD, nst - 1), slot_issue);
        compute(c, L, slot, (c.k_end - (c.k_begin + SK * st)) < SK, acc);
        QMM_WAIT_VMCNT(GE::NCOPY * (AHEAD - 1));  // the copies of stage st+1 landed; later stages' may remain
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
        slot = slot == RING - 1 ? 0 : slot + 1;
    }
    QMM_WAIT_VMCNT(0);  // no copy may still be writing LDS when the workgroup ends

    // Lane holds, for tile (i, j), C[m][n..n+3] with m = m0 + wm*64 + 32i + (lane % 32)
    // and n = n0 + wn*32*NJ + 32j + 8*vq + 4*(lane / 32), values 4vq .. 4vq+3.
    // The tile goes out through LDS (free now): the waves write it row-major, 128 values
    // per row (512 bytes of fp32 or 256 of bf16) with 16-byte chunk c of row x stored at
    // chunk c ^ (x % chunks per row), and then every store instruction writes whole rows.
    // Stored straight from the accumulators, each instruction would write 16 or 8 bytes
    // into each of 32 rows.
    constexpr int ES = F32_OUT ? 4 : 2;    // bytes per element
    constexpr int CPR = TN * ES / 16;      // 16-byte chunks per row: 32 or 16
    char *T = reinterpret_cast<char *>(&L);
    const int r = lane & 31, sl = lane >> 5;
    __syncthreads();  // every wave is done with the stage slots
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int x = wm * 64 + 32 * i + r;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
#pragma unroll
            for (int vq = 0; vq < 4; ++vq) {
                const float v0 = acc[i][j][4 * vq], v1 = acc[i][j][4 * vq + 1];
                const float v2 = acc[i][j][4 * vq + 2], v3 = acc[i][j][4 * vq + 3];
                const int col = wn * 32 * NJ + 32 * j + 8 * vq + 4 * sl;  // first of the four columns
                if (F32_OUT) {
                    const int cc = col >> 2;
                    *reinterpret_cast<float4 *>(T + x * (CPR * 16) + 16 * (cc ^ (x & (CPR - 1)))) =
                        make_float4(v0, v1, v2, v3);
                } else {
                    const int cc = col >> 3;
                    uint2 v;
                    v.x = pack_bf16x2(v0, v1);
                    v.y = pack_bf16x2(v2, v3);
                    *reinterpret_cast<uint2 *>(T + x * (CPR * 16) + 16 * (cc ^ (x & (CPR - 1))) + 8 * sl) = v;
                }
            }
        }
    }
    __syncthreads();
    char *base = static_cast<char *>(out) + (F32_OUT ? (size_t)p * (size_t)M * (size_t)N * ES : 0);
    const bool v16 = vec_store && (N % (16 / ES)) == 0 && (reinterpret_cast<uintptr_t>(base) & 15) == 0;
    for (int k = threadIdx.x; k < TM * CPR; k += 64 * NW) {
        const int x = k / CPR, cc = k % CPR;
        const int m = m0 + x, n = n0 + cc * (16 / ES);
        if (m >= M || n >= N) continue;
        const uint4 v = *reinterpret_cast<const uint4 *>(T + x * (CPR * 16) + 16 * (cc ^ (x & (CPR - 1))));
        char *g = base + ((size_t)m * (size_t)N + n) * ES;
        if (v16 && n + 16 / ES - 1 < N) {
            // Non-temporal (streaming) store: lines left dirty in the XCD's L2 are written
            // back before the kernel completes (cfg3 at s = 16: 5 % faster with the hint).
            __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4 *>(g));
        } else {
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 16 / ES; ++e) {
                if (n + e >= N) break;
                if (F32_OUT)
                    reinterpret_cast<uint32_t *>(g)[e] = w[e];
                else
                    reinterpret_cast<uint16_t *>(g)[e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
            }
        }
    }
}

}  // namespace

namespace qmm_impl {

// K < 2^22 (32-bit copy offsets over 128 rows); s <= K/64 when K % 64 == 0, else s <= K/32
// (no empty partition). vec_store: N % 4 == 0 and
// the output 16-byte (fp32 planes) or 8-byte (bf16 C) aligned.
hipError_t launch_dense(DenseTile tile, const void *A, const void *B, void *out, bool f32_out,
                        int M, int N, int K, int s, bool vec_store, hipStream_t stream)
{
    if (tile.block_m() != TM || tile.block_n() != TN) return hipErrorInvalidValue;
    if (K >= (1 << 22) || s < 1 || s > K / ((K & 63) == 0 ? 64 : 32)) return hipErrorInvalidValue;
    const int tiles = ((M + TM - 1) / TM) * ((N + TN - 1) / TN);
    const dim3 grid(tiles * s);
    // eight 64 x 32 waves, two per SIMD, so that one wave's LDS reads and copy waits hide under
    // the other's MFMAs (cfg3 on MI355X: 8 % faster than four 64 x 64 waves at s = 1..8, 5 % at
    // s = 12, 1 % at s = 16)
    constexpr int NW = 8;
    (void)hipGetLastError();
    if (f32_out)
        hipLaunchKernelGGL((dense_kernel<true, NW>), grid, dim3(64 * NW), 0, stream, static_cast<const uint16_t *>(A),
                           static_cast<const uint16_t *>(B), out, M, N, K, s, vec_store ? 1 : 0);
    else
        hipLaunchKernelGGL((dense_kernel<false, NW>), grid, dim3(64 * NW), 0, stream,
                           static_cast<const uint16_t *>(A), static_cast<const uint16_t *>(B), out, M, N, K, s,
                           vec_store ? 1 : 0);
    return hipGetLastError();
}

}  // namespace qmm_impl
