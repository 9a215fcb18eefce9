// qmm_w4a16_wide.hip -- W4A16 group-128 matmul kernel for many rows (M > 128) on gfx950.
//
// Same contract as the small-M kernel (tiny-llm "Week 2 Day 7: Split-K Prefill",
// Task 2): blockIdx.z is the partition p, the block covers groups
// [p*gpp, (p+1)*gpp) of the reduction and writes plane p of `out` (C itself when
// s = 1), with plain stores and no atomics.
//
// This regime is bound by the bf16 matrix cores, so the design maximises MFMA
// issue: a 256 x 128 output tile per workgroup of 4 wave64s (2 x 2, each wave a
// 128 x 64 tile of 4 x 2 v_mfma_f32_32x32x16_bf16 accumulators), the reduction
// walked in stages of 32 values.
//
// Data movement per stage:
//   A: 256 rows x 32 k of bf16 (16 KB), copied global -> LDS by the direct
//      load-to-LDS instruction (global_load_lds_dwordx4: lane i of an
//      instruction lands at LDS base + 16*i), three stages ahead of its use;
//   W: 128 rows x 32 k of packed nibbles (2 KB) plus the group's scale and bias,
//      loaded into registers four stages ahead, dequantised ONCE per workgroup
//      (w = scale*q + bias in fp32, rounded to bf16) into a bf16 LDS tile (8 KB)
//      one stage ahead of its use.
// LDS holds a ring of four A slots (16 KB each) and two dequantised-W buffers
// (8 KB each): 80 KB per workgroup, two workgroups per CU. The matrix cores work
// on stage i while stage i+1 is dequantised, A of stages i+2, i+3 is in flight
// and W of stages i+2 .. i+5 is in flight in a four-set register ring.
//
// The compiler does not track the LDS writes of the load-to-LDS instruction, so
// the kernel waits for them itself: before the barrier that ends stage i, each
// wave waits (s_waitcnt vmcnt) until the copies it issued for stage i+1 have
// landed; the barrier then publishes them to the whole workgroup.
//
// LDS rows are 64 bytes (four 16-byte chunks); chunk c of row r is stored at
// chunk c ^ ((r >> 2) & 3), which keeps the 16-byte fragment reads (rows r..r+15
// at one chunk) and the tile writes free of bank conflicts.
//
// Block order: tiles are numbered with the M-block fastest, so with 8 M-blocks
// (M = 2048) the workgroups that the round-robin dispatch sends to one XCD share
// the same 256 rows of A, which then stay in that XCD's L2.
#include "qmm_device.h"
#include "qmm_launch.h"

using namespace qmm_dev;

namespace {

constexpr int BM = 256;
constexpr int BN = 128;
constexpr int BK = 32;
constexpr int A_BYTES = BM * BK * 2;        // 16 KB per A slot, 4 slots
constexpr int B_BYTES = BN * BK * 2;        // 8 KB per dequantised W buffer, 2 buffers

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ int swz(int row, int chunk) { return row * 64 + ((chunk ^ ((row >> 2) & 3)) << 4); }

// s_waitcnt with only the vector-memory counter limited to n (n < 64; the count's
// low four bits sit in bits 3:0 of the immediate, its high two bits in bits 15:14).
#define QMM_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (((n) >> 4) << 14) | (0x7 << 4) | (0xF << 8))

struct WRegs {
    u32x2 w;          // 16 packed weights of row n = tid/2, k half tid%2
    uint32_t sc, bi;  // bf16 bits of the group's scale and bias for row n
};

struct Ctx {
    int rot, nst;  // k-stage rotation of this workgroup, stages in its partition
    const uint16_t *A;
    const uint32_t *Wq;
    const uint16_t *scale;
    const uint16_t *bias;
    int M, N, K, G;
    int m0, n0, k_begin;
    int tid, lane, wave, wm, wn;
};

// LDS: four A slots (a ring, stage st in slot st % 4) and two dequantised-W buffers
// (stage st in buffer st % 2): 80 KB per workgroup, two workgroups per CU.
__shared__ __attribute__((aligned(1024))) char lds_a[4][A_BYTES];
__shared__ __attribute__((aligned(1024))) char lds_b[2][B_BYTES];

template <int S>
__device__ __forceinline__ char *a_slot() { return lds_a[S]; }
template <int S>
__device__ __forceinline__ char *b_buf() { return lds_b[S]; }

// W and the group's scale/bias for stage st: 3 vector-memory instructions.
// Reduction offset of pipeline stage st: the workgroup walks its partition's stages
// starting at a per-workgroup rotation (see the kernel), wrapping around.
__device__ __forceinline__ int stage_k(const Ctx &c, int st) { return c.k_begin + ((st + c.rot) % c.nst) * BK; }

__device__ __forceinline__ WRegs load_w(const Ctx &c, int st)
{
    WRegs R;
    const int k0 = stage_k(c, st);
    const int n = min(c.n0 + (c.tid >> 1), c.N - 1);
    const int h = c.tid & 1;
    R.w = *reinterpret_cast<const u32x2 *>(c.Wq + (size_t)n * (size_t)(c.K >> 3) + (k0 >> 3) + 2 * h);
    const int g = k0 >> 7;
    R.sc = c.scale[(size_t)n * c.G + g];
    R.bi = c.bias[(size_t)n * c.G + g];
    return R;
}

// One 16-byte global -> LDS copy per lane: lane i's bytes land at LDS byte
// address lds_off + 16*i (lds_off is wave-uniform, passed in M0). Issued as inline
// assembly so that the compiler neither tracks nor waits for it: the kernel orders
// these copies itself with explicit s_waitcnt vmcnt and workgroup barriers.
__device__ __forceinline__ void copy16_to_lds(const void *gsrc, uint32_t lds_off)
{
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds_off), "v"(gsrc) : "memory", "m0");
#pragma clang diagnostic pop
}

template <int S>
__device__ __forceinline__ uint32_t a_slot_lds_offset() { return (uint32_t)(uintptr_t)(lds_void *)a_slot<S>(); }

// A tile of stage st into LDS slot S: 4 copy instructions per wave.
// Instruction q = 4*wave + j fills LDS bytes [1024q, 1024q + 1024) of the A region,
// i.e. rows 16q .. 16q+15; lane i carries LDS 16-byte position 64q + i, which is
// row r = 16q + i/4, stored chunk i%4, so it fetches logical chunk (i%4) ^ ((r>>2)&3).
template <int S>
__device__ __forceinline__ void dma_a(const Ctx &c, int st)
{
    const int k0 = stage_k(c, st);
    const uint32_t base = a_slot_lds_offset<S>() + 4096u * (uint32_t)__builtin_amdgcn_readfirstlane(c.wave);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int q = 4 * c.wave + j;
        const int r = 16 * q + (c.lane >> 2);
        const int chunk = (c.lane & 3) ^ ((r >> 2) & 3);
        const int m = min(c.m0 + r, c.M - 1);
        copy16_to_lds(c.A + (size_t)m * (size_t)c.K + k0 + 8 * chunk, base + 1024u * j);
    }
}

// Dequantise stage registers into dequantised-W buffer S (row n = tid/2, chunks 2h
// and 2h+1 of its 64-byte row).
template <int S>
__device__ __forceinline__ void dequant_w(const Ctx &c, const WRegs &R)
{
    char *Bs = b_buf<S>();
    const int n = c.tid >> 1;
    const int h = c.tid & 1;
    const float sc = bf16_to_f32(R.sc);
    const float bi = bf16_to_f32(R.bi);
    const float sc16 = sc * 0.0625f;
    *reinterpret_cast<uint4 *>(Bs + swz(n, 2 * h)) = dequant8(R.w[0], sc, sc16, bi);
    *reinterpret_cast<uint4 *>(Bs + swz(n, 2 * h + 1)) = dequant8(R.w[1], sc, sc16, bi);
}

// sched_group_barrier masks (instruction classes the scheduler may place in a group)
constexpr int SG_VALU = 0x002;
constexpr int SG_MFMA = 0x008;
constexpr int SG_DS_READ = 0x100;

// The MFMAs of one stage (2 x 8 per wave) with the dequantisation of the next stage's
// W (2 x 22 VALU instructions) and the second half's LDS reads woven between them,
// so the vector ALU work runs in the shadow of the matrix cores instead of before them.
template <int SA, int SB>
__device__ __forceinline__ void compute_and_dequant(const Ctx &c, f32x16 (&acc)[4][2], const WRegs &wn,
                                                    uint4 &d0, uint4 &d1)
{
    const char *As = a_slot<SA>();
    const char *Bs = b_buf<SB>();
    const int r = c.lane & 31;
    const int sl = c.lane >> 5;
    const float sc = bf16_to_f32(wn.sc);
    const float bi = bf16_to_f32(wn.bi);
    const float sc16 = sc * 0.0625f;
    bf16x8 af[2][4], bfr[2][2];
#pragma unroll
    for (int k16 = 0; k16 < 2; ++k16) {
        const int chunk = 2 * k16 + sl;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            af[k16][i] = as_bf16x8(*reinterpret_cast<const uint4 *>(As + swz(c.wm * 128 + i * 32 + r, chunk)));
#pragma unroll
        for (int j = 0; j < 2; ++j)
            bfr[k16][j] = as_bf16x8(*reinterpret_cast<const uint4 *>(Bs + swz(c.wn * 64 + j * 32 + r, chunk)));
    }
    d0 = dequant8(wn.w[0], sc, sc16, bi);
    d1 = dequant8(wn.w[1], sc, sc16, bi);
#pragma unroll
    for (int k16 = 0; k16 < 2; ++k16)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) acc[i][j] = mfma32x32x16(bfr[k16][j], af[k16][i], acc[i][j]);
    // Schedule: the first half's 6 LDS reads, then 8 MFMAs each followed by 3 VALU,
    // with the second half's 6 reads issued after the second MFMA; then 8 more MFMAs
    // each followed by 3 VALU.
    __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 6, 0);
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
        __builtin_amdgcn_sched_group_barrier(SG_VALU, 3, 0);
        if (q == 1) __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 6, 0);
    }
}

// One stage: st is computed from A slot CUR = st % 4 and W buffer st % 2, while the
// W registers `wr` (stage st+1) are dequantised into buffer (st+1) % 2 and then
// refilled with stage st+5. The body is branch-free: past the last stage the
// indices are clamped, so the extra loads only touch slots and buffers that are
// never read again, and every stage issues exactly 7 vector-memory instructions
// (A: 4 copies first, W: 3 loads last).
template <int CUR>
__device__ __forceinline__ void stage(const Ctx &c, int st, int nst, WRegs &wr, f32x16 (&acc)[4][2])
{
    dma_a<(CUR + 3) % 4>(c, min(st + 3, nst - 1));
    uint4 d0, d1;
    compute_and_dequant<CUR, CUR % 2>(c, acc, wr, d0, d1);
    {
        char *Bs = b_buf<(CUR + 1) % 2>();
        const int n = c.tid >> 1;
        const int h = c.tid & 1;
        *reinterpret_cast<uint4 *>(Bs + swz(n, 2 * h)) = d0;
        *reinterpret_cast<uint4 *>(Bs + swz(n, 2 * h + 1)) = d1;
    }
    wr = load_w(c, min(st + 5, nst - 1));
    // The A copies of stage st+1 were the first 4 instructions of stage st-2; issued
    // after them: 3 + 7 + 7 = 17. Waiting until at most 17 are outstanding retires
    // them, whatever order the instructions have within a stage.
    QMM_WAIT_VMCNT(17);
    __syncthreads();
    // Keep the next stage's instructions below the barrier.
    __builtin_amdgcn_sched_barrier(0);
}

__global__ void __launch_bounds__(256, 2)
w4a16_wide_kernel(const uint16_t *__restrict__ A, const uint32_t *__restrict__ Wq,
                  const uint16_t *__restrict__ scale, const uint16_t *__restrict__ bias,
                  uint16_t *__restrict__ out, int M, int N, int K, int gpp, int vec_store)
{
    Ctx c;
    c.A = A;
    c.Wq = Wq;
    c.scale = scale;
    c.bias = bias;
    c.M = M;
    c.N = N;
    c.K = K;
    c.G = K >> 7;
    c.tid = threadIdx.x;
    c.lane = c.tid & 63;
    c.wave = __builtin_amdgcn_readfirstlane(c.tid >> 6);  // wave-uniform
    c.wm = c.wave >> 1;
    c.wn = c.wave & 1;
    const int num_m = (M + BM - 1) / BM;
    c.m0 = (blockIdx.x % num_m) * BM;
    c.n0 = (blockIdx.x / num_m) * BN;
    c.k_begin = blockIdx.z * gpp * 128;
    const int nst = gpp * (128 / BK);  // a multiple of 4, at least 4
    // Workgroups that run side by side on one XCD share rows of A; starting each at a
    // different group (4 stages) of the partition spreads their simultaneous reads of
    // A over more L2 channels. The order of the fp32 sums depends only on the tile.
    c.nst = nst;
    c.rot = ((blockIdx.x / num_m) * 4) % nst;
    uint16_t *dst = out + (size_t)blockIdx.z * (size_t)M * (size_t)N;

    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    // Prologue: W of stages 0..3 into the register ring, A of stages 0..2 into
    // slots 0..2, W of stage 0 dequantised into buffer 0, W of stage 4 loaded.
    dma_a<0>(c, 0);
    WRegs w0 = load_w(c, 0);
    dma_a<1>(c, 1);
    WRegs w1 = load_w(c, 1);
    dma_a<2>(c, 2);
    WRegs w2 = load_w(c, 2);
    WRegs w3 = load_w(c, 3);
    dequant_w<0>(c, w0);
    w0 = load_w(c, min(4, nst - 1));
    // A of stage 0 landed: issued after it are W0 (3), A1 (4), W1 (3), A2 (4), W2, W3, W4 (9) = 23;
    // the A copies of stages 1 and 2 are then retired by the waits of stages 0 and 1.
    QMM_WAIT_VMCNT(23);
    __syncthreads();

    // Stage st uses A slot st % 4, W buffer st % 2 and W register set st % 4
    // (w0 holds stages 0, 4, 8, ...; w1 holds 1, 5, ...). nst is a multiple of 4.
    for (int st = 0; st < nst; st += 4) {
        stage<0>(c, st, nst, w1, acc);
        stage<1>(c, st + 1, nst, w2, acc);
        stage<2>(c, st + 2, nst, w3, acc);
        stage<3>(c, st + 3, nst, w0, acc);
    }

    // Lane holds, for tile (i, j), C[m][n..n+3] with m = m0 + wm*128 + 32i + (lane % 32)
    // and n = n0 + wn*64 + 32j + 8*vq + 4*(lane / 32), values 4vq .. 4vq+3.
    const int r = c.lane & 31;
    const int sl = c.lane >> 5;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = c.m0 + c.wm * 128 + 32 * i + r;
        const bool row_ok = m < M;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
#pragma unroll
            for (int vq = 0; vq < 4; ++vq) {
                const int n = c.n0 + c.wn * 64 + 32 * j + 8 * vq + 4 * sl;
                uint16_t *p = dst + (size_t)m * (size_t)N + n;
                const float v0 = acc[i][j][4 * vq], v1 = acc[i][j][4 * vq + 1];
                const float v2 = acc[i][j][4 * vq + 2], v3 = acc[i][j][4 * vq + 3];
                if (vec_store && n + 3 < N) {
                    if (row_ok) {
                        uint2 v;
                        v.x = pack_bf16x2(v0, v1);
                        v.y = pack_bf16x2(v2, v3);
                        *reinterpret_cast<uint2 *>(p) = v;
                    }
                } else if (row_ok) {
                    if (n < N) p[0] = (uint16_t)f32_to_bf16(v0);
                    if (n + 1 < N) p[1] = (uint16_t)f32_to_bf16(v1);
                    if (n + 2 < N) p[2] = (uint16_t)f32_to_bf16(v2);
                    if (n + 3 < N) p[3] = (uint16_t)f32_to_bf16(v3);
                }
            }
        }
    }
}

}  // namespace

namespace qmm_impl {

hipError_t launch_w4a16_wide(const void *A, const void *Wq, const void *scale, const void *bias, void *out,
                             int M, int N, int K, int s, bool vec_store, hipStream_t stream)
{
    const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    const int gpp = (K / 128) / s;
    (void)hipGetLastError();
    hipLaunchKernelGGL(w4a16_wide_kernel, dim3(tiles, 1, s), dim3(256), 0, stream,
                       static_cast<const uint16_t *>(A), static_cast<const uint32_t *>(Wq),
                       static_cast<const uint16_t *>(scale), static_cast<const uint16_t *>(bias),
                       static_cast<uint16_t *>(out), M, N, K, gpp, vec_store ? 1 : 0);
    return hipGetLastError();
}

}  // namespace qmm_impl
