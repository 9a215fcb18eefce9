// qmm_w4a16_wide.hip -- weight-only quantized matmul kernel for many rows (M > 64) on gfx950:
// W4A16 group 128, and the library's other formats (4- or 8-bit codes, groups of 32, 64
// or 128 values; skillsdirectory "Optimize Prefill vs Decode Kernels", step 6, names
// W4A16 and W8A16 with the dequantisation fused into the main loop).
//
// Split contract of tiny-llm "Week 2 Day 7: Split-K Prefill", Task 2: a workgroup
// computes one output tile over one group-aligned partition of the reduction and
// writes its bf16 result into that partition's plane (C itself when unsplit), with
// plain stores and no atomics. Beyond the page's uniform split, the grid may run the
// first tiles unsplit and split only the remaining ones, and the partitions may differ
// by one group (see the work decomposition above the kernel): on 256 CUs this fills
// the last wave of workgroups instead of leaving it mostly idle.
//
// This regime is bound by the bf16 matrix cores. A workgroup owns a 128 x 256 tile (variant
// 0: 4 wave64s, each 128 x 64, 4 x 2 v_mfma_f32_32x32x16_bf16 accumulators), a 128 x 128
// tile (variant 1: 4 wave64s, each 128 x 32, 4 x 1 accumulators; for shapes whose 256-column
// tiles would need a deep split) or a 256 x 256 tile (variant 2: 8 wave64s, each 256 x 32,
// 8 x 1 accumulators), and walks its partition
// in stages of 64 reduction values. Tall wave tiles spread each dequantised weight over
// 4 or 8 MFMAs, and 64-value stages make every row of A a whole 128-byte line.
//
// Data movement: every global read of the kernel is a direct global -> LDS copy
// (global_load_lds_*), issued one to one and a half stages ahead of its use, into rings of three slots:
//   A:  BM rows x 64 bf16 (16 or 32 KB per stage), 1 KB per copy;
//   W:  BN (256 or 128) rows x 32 bytes of packed nibbles (8 or 4 KB per stage; rows of
//       64 bytes for 8-bit codes), 1 KB per copy;
//   scale/bias: the 128-value block's BN + BN bf16 values per group it holds (one, two
//       or four), one 2-byte copy per lane (zero-extended into a dword), once per block,
//       in a ring of two.
// The compiler neither sees nor waits for these copies; the kernel retires them
// itself: in the middle of stage i each wave waits (s_waitcnt vmcnt) until the copies
// it issued for stage i+1 have landed, and the barrier that follows publishes them
// to the whole workgroup; the A copies of stage i+2 are issued right after it, its W
// and scale/bias copies during the stage's last step. No other vector-memory
// instruction is issued in the loop, so the counter arithmetic is exact. In the 8-wave
// variant only waves 0-3, one per SIMD, issue copies (twice the share each): while a
// copying wave issues them, the other wave of its SIMD keeps the matrix core busy
// (2-4 % faster than copies from every wave).
// The next stage's first operands are read during the last step of the current one,
// so the matrix pipeline does not drain at stage boundaries.
//
// Dequantisation: each wave turns its 64 or 32 columns' packed words straight into MFMA
// operands (w = scale*q + bias in fp32, rounded to bf16). One packed 32-bit word is
// eight consecutive reduction values, i.e. one lane's operand of one
// 32x32x16 MFMA. For reduction step t of a stage, lane l (half h = l / 32) takes word
// 4h + t of its row, so one 16-byte LDS read gives a lane its words for all four
// steps; its A operand is the matching 8 values (16-byte chunk 4h + t of the row).
// With 8-bit codes the same eight values are two words and a lane reads 32 bytes. A
// lane's 32 values of a stage lie in one scale/bias group for every group size.
// The MFMA takes the weights as its first operand, so a lane's results are four
// consecutive output columns of one row. Results leave through LDS as whole rows (see the
// end of segment): bf16 tiles in one or two passes, fp32 planes in passes of 64 rows.
//
// LDS layouts: A rows are 128 bytes (eight 16-byte chunks), chunk c of row r stored
// at chunk c ^ ((r >> 1) & 7); W rows of 32 bytes store chunk h of row r at
// h ^ ((r >> 3) & 1), rows of 64 bytes chunk h at h ^ ((r >> 2) & 3). Each keeps the
// 16-lane phases of the 16-byte reads on distinct banks.
//
// Block order: tiles are numbered with the M-block fastest, so with 8 M-blocks the
// workgroups that the round-robin dispatch sends to one XCD share the same BM rows
// of A in that XCD's L2.
#include "qmm_device.h"
#include "qmm_launch.h"

using namespace qmm_dev;

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int BK = 64;
constexpr int ROT_GROUPS = 8;        // k-start spread of the workgroups sharing A rows

typedef __attribute__((address_space(3))) void lds_void;

// Tile geometry of a variant and weight format: 128*WM rows x BN columns per workgroup,
// each wave a (32*MI) x (32*NJ) block of 32x32 MFMA tiles, waves side by side along N
// first; BITS-wide codes, SUB scale/bias groups per 128-value block.
template <int WM_, int MI_, int NJ_, int BITS_, int SUB_, int BN_ = 256>
struct Cfg {
    static constexpr int WM = WM_, MI = MI_, NJ = NJ_, BITS = BITS_, SUB = SUB_, BN = BN_;
    static constexpr int BM = 128 * WM;             // rows per tile
    static constexpr int NWN = BN / (32 * NJ);      // waves along N
    static constexpr int NWM = BM / (32 * MI);      // waves along M
    static constexpr int NW = NWM * NWN;            // waves per workgroup
    static constexpr int CW = NW == 8 ? 4 : NW;      // waves that issue the copies (one per SIMD for 8)
    static constexpr int A_SLOT = BM * BK * 2;      // 16 or 32 KB
    static constexpr int WROW = BK * BITS / 8;      // bytes of one W row per stage: 32 or 64
    static constexpr int WCH = WROW / 16;           // 16-byte chunks per W row: 2 or 4
    static constexpr int WSW = WCH == 2 ? 3 : 2;    // W row swizzle: chunk ^ ((r >> WSW) & (WCH-1))
    static constexpr int WV = BITS / 4;             // 16-byte W reads per lane per stage
    static constexpr int W_SLOT = BN * WROW;        // 8 or 16 KB
    static constexpr int SB_SLOT = 2 * SUB * BN * 4;  // scale then bias dwords of one block
    static constexpr int AC = (BM / 8) / CW;        // A copies (1 KB each) per copying wave per stage
    static constexpr int WC = W_SLOT / 1024 / CW;   // W copies (1 KB each) per copying wave per stage
    static constexpr int SC = SB_SLOT / 256 / CW;   // scale/bias copies (64 values) per copying wave per block
    static constexpr int N_EVEN = AC + WC + SC;     // copies a copying wave issues in an even stage
    static constexpr int N_ODD = AC + WC;           // ... in an odd stage
    static constexpr int LDS = 3 * A_SLOT + 3 * W_SLOT + 2 * SB_SLOT;
    static constexpr int SBQ = BN / 64;             // scale/bias copies per array and group
    static constexpr int OCC = 2 * LDS <= qmm_impl::kLdsPerCU ? 2 : 1;  // workgroups one CU holds
    static_assert(LDS == qmm_impl::wide_lds_bytes(BM, BITS, SUB, BN), "LDS size differs from the host's");
    static_assert(AC * CW * 8 == BM && WC * CW * 1024 == W_SLOT && SC * CW * 256 == SB_SLOT, "copy split");
};

// LDS of one workgroup: three A slots, three W slots, two scale/bias slots.
template <class CF>
struct Lds {
    char a[3 * CF::A_SLOT];
    char w[3 * CF::W_SLOT];
    char sb[2 * CF::SB_SLOT];
};

// s_waitcnt with only the vector-memory counter limited to n (n < 64; the count's
// low four bits sit in bits 3:0 of the immediate, its high two bits in bits 15:14).
#define QMM_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (((n) >> 4) << 14) | (0x7 << 4) | (0xF << 8))

__device__ __forceinline__ uint32_t lds_addr(const void *p) { return (uint32_t)(uintptr_t)(const lds_void *)p; }

// Global -> LDS copies (global_load_lds_*, address = scalar base + 32-bit lane offset).
// Lane i's data lands at LDS byte lds_off + 16*i (dwordx4) or lds_off + 4*i (ushort,
// zero-extended to a dword); lds_off is wave-uniform and travels in M0. Inline assembly,
// so that the compiler neither tracks nor waits for them.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void copy16(uint32_t lds_off, uint32_t voff, const void *sbase)
{
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds_off), "v"(voff), "s"(sbase)
                 : "memory", "m0");
}
__device__ __forceinline__ void copy2(uint32_t lds_off, uint32_t voff, const void *sbase)
{
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_ushort %1, %2" ::"s"(lds_off), "v"(voff), "s"(sbase)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

template <class CF>
struct Ctx {
    const char *A;      // A + m0*K (bytes), wave-uniform
    const char *Wq;     // Wq + n0*K/8 words (bytes)
    const char *sb[CF::SC];  // scale/bias source of this wave's copies (scale or bias, + n0*GG + sub)
    int gpp, rot, g_begin;
    int copier;  // this wave issues copies (wave < CW; wave-uniform)
    uint32_t a_off[CF::AC];    // per-lane byte offsets of the A copies (stage k excluded)
    uint32_t w_off[CF::WC];    // per-lane byte offsets of the W copies
    uint32_t sb_off[CF::SC];   // per-lane byte offsets of the scale/bias copies
    uint32_t a_lds, w_lds, sb_lds;  // this wave's destinations inside slot 0
    uint32_t a_rd[4];   // per-lane LDS byte offsets of the A operand reads, step t
    uint32_t w_rd[CF::WV];
    uint32_t sb_rd[2];  // scale read offset for an even / odd stage (its group in the block)
};

// Group of stage x (two stages per group), rotated per workgroup.
template <class CF>
__device__ __forceinline__ int stage_group(const Ctx<CF> &c, int x)
{
    int g = (x >> 1) + c.rot;
    if (g >= c.gpp) g -= c.gpp;
    return c.g_begin + g;
}

// The copies of stage x into A/W slot `slot3` (and its group's scale/bias into
// slot `sbslot` when WITH_SB): AC + WC (+ SC) vector-memory instructions per copying
// wave, none for the others. PART 0 issues them all, PART 1 the A copies, PART 2 the
// W and scale/bias copies.
template <class CF, bool WITH_SB, int PART = 0>
__device__ __forceinline__ void issue(const Ctx<CF> &c, int x, int slot3, int sbslot)
{
    typedef CF GE;
    if (GE::CW < GE::NW && !c.copier) return;
    const int g = __builtin_amdgcn_readfirstlane(stage_group(c, x));
    const int k0 = g * 128 + (x & 1) * BK;
    const char *Ab = c.A + 2 * (size_t)k0;
    const uint32_t a_dst = c.a_lds + (uint32_t)slot3 * GE::A_SLOT;
    if (PART != 2) {
#pragma unroll
        for (int j = 0; j < GE::AC; ++j) copy16(a_dst + 1024u * j, c.a_off[j], Ab);
    }
    if (PART == 1) return;
    const uint32_t w_dst = c.w_lds + (uint32_t)slot3 * GE::W_SLOT;
#pragma unroll
    for (int j = 0; j < GE::WC; ++j)
        copy16(w_dst + 1024u * j, c.w_off[j], c.Wq + (size_t)k0 * GE::BITS / 8);
    if (WITH_SB) {
        const uint32_t sb_dst = c.sb_lds + (uint32_t)sbslot * GE::SB_SLOT;
#pragma unroll
        for (int j = 0; j < GE::SC; ++j)
            copy2(sb_dst + 256u * j, c.sb_off[j], c.sb[j] + 2 * (size_t)g * GE::SUB);
    }
}

// Eight dequantised weights of reduction step t (0..3) from a lane's W words of a stage.
template <class CF>
__device__ __forceinline__ bf16x8 weights_of_step(const uint4 (&wpk)[CF::WV], int t, float sc, float sc512,
                                                  float bi)
{
    if (CF::BITS == 4) return as_bf16x8(dequant8(word_of(wpk[0], t), sc512, bi));
    const uint4 &v = wpk[(t >> 1) % CF::WV];
    return as_bf16x8(dequant8_u8(word_of(v, 2 * (t & 1)), word_of(v, 2 * (t & 1) + 1), sc, bi));
}

// Operands carried from one stage into the next: the stage's W words and scale/bias,
// and the A operands and dequantised weights of the step about to run.
template <class CF>
struct Ops {
    uint4 wpk[CF::NJ][CF::WV];
    float sc[CF::NJ], sc512[CF::NJ], bi[CF::NJ];
    bf16x8 af[CF::MI];
    bf16x8 bw[CF::NJ];
};

// The A operands (rows of this wave) and dequantised weights of reduction step t of a
// stage whose A slot starts at As.
template <class CF>
__device__ __forceinline__ void step_operands(const Ctx<CF> &c, const char *As, const Ops<CF> &o, int t,
                                              bf16x8 (&af)[CF::MI], bf16x8 (&bw)[CF::NJ])
{
#pragma unroll
    for (int i = 0; i < CF::MI; ++i) af[i] = as_bf16x8(*reinterpret_cast<const uint4 *>(As + c.a_rd[t] + 4096 * i));
#pragma unroll
    for (int j = 0; j < CF::NJ; ++j) bw[j] = weights_of_step<CF>(o.wpk[j], t, o.sc[j], o.sc512[j], o.bi[j]);
}

// The head of a stage (A/W slot `slot3`, scale/bias slot `sbslot`; ODD: the second half
// of its 128-value block): its W words, scale/bias and the operands of its step 0.
template <class CF, int ODD>
__device__ __forceinline__ void load_head(const Ctx<CF> &c, const Lds<CF> &L, int slot3, int sbslot, Ops<CF> &o)
{
    const char *Ws = L.w + slot3 * CF::W_SLOT;
    const char *Ss = L.sb + sbslot * CF::SB_SLOT;
#pragma unroll
    for (int j = 0; j < CF::NJ; ++j) {
#pragma unroll
        for (int u = 0; u < CF::WV; ++u)
            o.wpk[j][u] = *reinterpret_cast<const uint4 *>(Ws + c.w_rd[u] + 32 * CF::WROW * j);
        o.sc[j] = bf16_to_f32(*reinterpret_cast<const uint32_t *>(Ss + c.sb_rd[ODD] + 128 * j));
        o.bi[j] = bf16_to_f32(*reinterpret_cast<const uint32_t *>(Ss + 4 * CF::BN * CF::SUB + c.sb_rd[ODD] + 128 * j));
        o.sc512[j] = o.sc[j] * 512.f;
    }
    step_operands<CF>(c, L.a + slot3 * CF::A_SLOT, o, 0, o.af, o.bw);
}

// The 32 MFMAs of one stage (A slot `slot3`) whose head is in `o`, software-pipelined:
// the operands of step t+1 are read and dequantised while the MFMAs of step t run.
// Between steps 1 and 2 it calls mid() (the workgroup's stage barrier and the copies it
// frees a slot for); during step 3 it calls next(o) to read the next stage's head, so
// no stage starts with an empty matrix pipeline. The scheduling fences keep the
// compiler from sinking the reads down to their use or hoisting them above mid().
template <class CF, class Mid, class Next>
__device__ __forceinline__ void run_stage(const Ctx<CF> &c, const Lds<CF> &L, int slot3, Ops<CF> &o,
                                          f32x16 (&acc)[CF::MI][CF::NJ], Mid mid, Next next)
{
    constexpr int MI = CF::MI, NJ = CF::NJ;
    const char *As = L.a + slot3 * CF::A_SLOT;
    bf16x8 af2[MI], bw2[NJ];
    __builtin_amdgcn_sched_barrier(0);
    step_operands<CF>(c, As, o, 1, af2, bw2);
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = mfma32x32x16(o.bw[j], o.af[i], acc[i][j]);
    __builtin_amdgcn_sched_barrier(0);
    step_operands<CF>(c, As, o, 2, o.af, o.bw);
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = mfma32x32x16(bw2[j], af2[i], acc[i][j]);
    __builtin_amdgcn_sched_barrier(0);
    mid();
    __builtin_amdgcn_sched_barrier(0);
    step_operands<CF>(c, As, o, 3, af2, bw2);
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = mfma32x32x16(o.bw[j], o.af[i], acc[i][j]);
    __builtin_amdgcn_sched_barrier(0);
    next(o);
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = mfma32x32x16(bw2[j], af2[i], acc[i][j]);
    __builtin_amdgcn_sched_barrier(0);
}

// Where a segment's results go: element (m, n) of the tile is stored at
// base + ((m - r0) * ld + (n - c0)) elements, bf16 or (f32) fp32, rows m < M and
// columns n < N only.
struct Dest {
    char *base;
    size_t ld;
    int r0, c0;
    bool f32;
    int vec;  // 8/16-byte stores where four columns are in range
};

// One segment: tile `tile` (M-block fastest) over the 128-value blocks [g_lo, g_hi) of
// the reduction, from its first copy to its last store. Every wave of the workgroup
// calls it with the same arguments.
template <class CF>
__device__ __forceinline__ void segment(Lds<CF> &L, const uint16_t *__restrict__ A, const uint32_t *__restrict__ Wq,
                                        const uint16_t *__restrict__ scale, const uint16_t *__restrict__ bias, int M,
                                        int N, int K, int tile, int g_lo, int g_hi, const Dest &dst)
{
    typedef CF GE;
    constexpr int MI = CF::MI, NJ = CF::NJ;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    const int wm = wave / CF::NWN;  // row block of the wave (32*MI rows)
    const int wn = wave % CF::NWN;  // column block of the wave (32*NJ columns)
    const int G = K >> 7;                  // 128-value blocks
    const int GG = G * CF::SUB;            // scale/bias entries per row
    const int gpp = g_hi - g_lo;           // >= 1
    const int num_m = (M + GE::BM - 1) / GE::BM;
    const int m_idx = tile % num_m;
    const int n_idx = tile / num_m;
    const int m0 = m_idx * GE::BM;
    const int n0 = n_idx * CF::BN;

    Ctx<CF> c;
    c.gpp = gpp;
    c.g_begin = g_lo;
    c.copier = wave < CF::CW;
    // Workgroups that run side by side on one XCD share rows of A; starting them at
    // different groups (within a window of ROT_GROUPS) spreads their simultaneous
    // reads of A over more L2 channels. The fp32 sums' order depends only on the tile
    // and the block range.
    c.rot = (n_idx % ROT_GROUPS) % gpp;
    c.A = reinterpret_cast<const char *>(A) + 2 * (size_t)m0 * (size_t)K;
    c.Wq = reinterpret_cast<const char *>(Wq) + (size_t)n0 * (size_t)K * CF::BITS / 8;

    // Copy lanes (copying waves, w < CW). A: copy j of wave w fills rows 8q .. 8q+7, q = AC*w + j; lane i
    // lands at row r = 8q + i/8, stored chunk i%8, so it fetches logical chunk
    // (i%8) ^ ((r>>1)&7). Rows past M re-read row M-1 (never stored).
#pragma unroll
    for (int j = 0; j < GE::AC; ++j) {
        const int r = 8 * (GE::AC * wave + j) + (lane >> 3);
        const int chunk = (lane & 7) ^ ((r >> 1) & 7);
        const int rr = min(m0 + r, M - 1) - m0;
        c.a_off[j] = 2u * ((uint32_t)rr * (uint32_t)K + 8u * (uint32_t)chunk);
    }
#pragma unroll
    for (int j = 0; j < GE::WC; ++j) {
        // W: copy q = w*WC + j fills 1 KB of rows (32 rows of 32 bytes, or 16 of 64); lane
        // i -> row (1024/WROW)*q + i/WCH, stored chunk i%WCH, logical chunk
        // (i%WCH) ^ ((r>>WSW)&(WCH-1)). Rows past N re-read N-1.
        const int q = wave * GE::WC + j;
        const int r = (1024 / GE::WROW) * q + lane / GE::WCH;
        const int h = (lane % GE::WCH) ^ ((r >> GE::WSW) & (GE::WCH - 1));
        const int rr = min(n0 + r, N - 1) - n0;
        c.w_off[j] = (uint32_t)(rr * (K * GE::BITS / 8) + 16 * h);
    }
#pragma unroll
    for (int j = 0; j < GE::SC; ++j) {
        // scale/bias: copy q = w*SC + j carries 64 rows (lane i -> row 64*(q%4) + i) of
        // group (q/4) % SUB of the block, from scale (q < 4*SUB) or bias.
        const int q = wave * GE::SC + j;
        const int rs = min(n0 + 64 * (q % GE::SBQ) + lane, N - 1) - n0;
        const int sub = (q / GE::SBQ) % GE::SUB;
        c.sb_off[j] = (uint32_t)(2 * rs * GG);
        c.sb[j] = reinterpret_cast<const char *>(q < GE::SBQ * GE::SUB ? scale : bias) +
                  2 * (size_t)n0 * (size_t)GG + 2 * sub;
    }
    c.a_lds = lds_addr(L.a) + 1024u * (uint32_t)(GE::AC * wave);
    c.w_lds = lds_addr(L.w) + 1024u * (uint32_t)(wave * GE::WC);
    c.sb_lds = lds_addr(L.sb) + 256u * (uint32_t)(wave * GE::SC);
    // Operand reads: lane (r32 = lane % 32, half h = lane / 32).
    {
        const int r32 = lane & 31;
        const int h = lane >> 5;
        const int arow = wm * 32 * MI + r32;  // + 32 i (leaves the swizzle bits unchanged)
#pragma unroll
        for (int t = 0; t < 4; ++t) c.a_rd[t] = (uint32_t)(arow * 128 + 16 * ((4 * h + t) ^ ((arow >> 1) & 7)));
        const int nrow = wn * 32 * NJ + r32;  // + 32 j (likewise)
#pragma unroll
        for (int u = 0; u < GE::WV; ++u)
            c.w_rd[u] = (uint32_t)(nrow * GE::WROW +
                                   16 * ((GE::WV * h + u) ^ ((nrow >> GE::WSW) & (GE::WCH - 1))));
        // the lane's 32 values of an even (odd) stage are values 32h (64 + 32h) of the
        // block: group (32h) * SUB / 128 (and (64 + 32h) * SUB / 128) of the block
#pragma unroll
        for (int odd = 0; odd < 2; ++odd)
            c.sb_rd[odd] = (uint32_t)(4 * nrow + 4 * GE::BN * (((2 * odd + h) * GE::SUB) >> 2));
    }

    f32x16 acc[MI][NJ];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    const int nst = 2 * gpp;  // stages in the segment, even
    // Prologue: stage 0 (A, W, group 0's scale/bias) and stage 1 (A, W); wait for stage 0
    // and read its head.
    issue<CF, true>(c, 0, 0, 0);
    issue<CF, false>(c, 1, 1, 0);
    QMM_WAIT_VMCNT(GE::N_ODD);
    __syncthreads();
    Ops<CF> o;
    load_head<CF, 0>(c, L, 0, 0, o);

    // Stage x uses A/W slot x % 3 and scale/bias slot (x/2) % 2. In the middle of stage x
    // each wave waits for its copies of stage x+1 (issued during stage x-1, the only ones
    // outstanding), the barrier publishes them and certifies that every wave has left
    // stage x-1, and the copies of stage x+2 go into stage x-1's slot (with the next
    // group's scale/bias when x is even, whose slot the group of stages x-2 and x-1 has
    // left): the A copies at once, the W and scale/bias copies during the last step of
    // stage x, before the head of stage x+1 is read. Past the last stage the copies
    // repeat stage nst-1 into slots that are never read again.
    int s3 = 0;  // st % 3
    for (int st = 0; st < nst; st += 2) {
        const int s3n = s3 == 2 ? 0 : s3 + 1;    // (st+1) % 3
        const int s3p = s3 == 0 ? 2 : s3 - 1;    // (st+2) % 3
        const int sbs = (st >> 1) & 1;
        const bool more = st + 2 < nst;
        run_stage<CF>(
            c, L, s3, o, acc,
            [&] {
                QMM_WAIT_VMCNT(0);
                __syncthreads();
                issue<CF, true, 1>(c, min(st + 2, nst - 1), s3p, sbs ^ 1);
            },
            [&](Ops<CF> &n) {
                issue<CF, true, 2>(c, min(st + 2, nst - 1), s3p, sbs ^ 1);
                load_head<CF, 1>(c, L, s3n, sbs, n);
            });
        run_stage<CF>(
            c, L, s3n, o, acc,
            [&] {
                QMM_WAIT_VMCNT(0);
                __syncthreads();
                issue<CF, false, 1>(c, min(st + 3, nst - 1), s3, 0);  // (st+3) % 3 == st % 3
            },
            [&](Ops<CF> &n) {
                issue<CF, false, 2>(c, min(st + 3, nst - 1), s3, 0);
                if (more) load_head<CF, 0>(c, L, s3p, sbs ^ 1, n);
            });
        s3 = s3p;
    }
    // No copy may still be writing LDS when the segment ends (the next segment, or the
    // end of the workgroup, follows).
    QMM_WAIT_VMCNT(0);

    // Lane holds, for tile (i, j), C[m][n..n+3] with m = m0 + wm*32*MI + 32i + (lane % 32)
    // and n = n0 + wn*32*NJ + 32j + 8*vq + 4*(lane / 32), values 4vq .. 4vq+3.
    const int r = lane & 31;
    const int sl = lane >> 5;
    char *T = reinterpret_cast<char *>(&L);
    if (dst.f32) {
        // fp32 planes go out through LDS like the bf16 results below: 4*BN bytes per row,
        // chunk c of row x at chunk c ^ (x % (BN/4)), as many rows per pass as the LDS
        // holds (a multiple of 32, so that each 32-row block of a wave lies in one pass),
        // then whole rows per store instruction. Stored straight from the accumulators,
        // every instruction wrote 16 bytes into each of 32 rows.
        constexpr int CPR4 = CF::BN / 4;  // 16-byte chunks per row
        constexpr int RB4 = CF::BN * 4;   // bytes per row
        constexpr int PR4 = CF::BM * RB4 <= CF::LDS ? CF::BM : (CF::BM / 2) * RB4 <= CF::LDS ? CF::BM / 2 : CF::BM / 4;
        static_assert(PR4 >= 32 && PR4 % 32 == 0 && PR4 * RB4 <= CF::LDS, "fp32 epilogue pass");
        const bool v16f = dst.vec && (dst.ld % 4) == 0 && (reinterpret_cast<uintptr_t>(dst.base) & 15) == 0;
#pragma unroll
        for (int h = 0; h < CF::BM / PR4; ++h) {
            __syncthreads();  // every wave is done with the stage slots, or with the previous pass
#pragma unroll
            for (int i = 0; i < MI; ++i) {
                const int rb = wm * 32 * MI + 32 * i;
                if (rb / PR4 != h) continue;  // wave-uniform
                const int x = rb - h * PR4 + r;
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
#pragma unroll
                    for (int vq = 0; vq < 4; ++vq) {
                        const int cc = 8 * (wn * NJ + j) + 2 * vq + sl;  // columns 4cc .. 4cc+3 of the tile
                        *reinterpret_cast<float4 *>(T + x * RB4 + 16 * (cc ^ (x & (CPR4 - 1)))) =
                            make_float4(acc[i][j][4 * vq], acc[i][j][4 * vq + 1], acc[i][j][4 * vq + 2],
                                        acc[i][j][4 * vq + 3]);
                    }
                }
            }
            __syncthreads();
            for (int k = threadIdx.x; k < PR4 * CPR4; k += 64 * CF::NW) {
                const int x = k / CPR4, cc = k % CPR4;
                const int m = m0 + h * PR4 + x, n = n0 + 4 * cc;
                if (m >= M || n >= N) continue;
                const float4 v = *reinterpret_cast<const float4 *>(T + x * RB4 + 16 * (cc ^ (x & (CPR4 - 1))));
                float *g = reinterpret_cast<float *>(dst.base) + (size_t)(m - dst.r0) * dst.ld + (size_t)(n - dst.c0);
                if (v16f && n + 3 < N) {
                    __builtin_nontemporal_store(
                        u32x4{__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z), __float_as_uint(v.w)},
                        reinterpret_cast<u32x4 *>(g));
                } else {
                    const float w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (n + e < N) g[e] = w[e];
                }
            }
        }
        return;
    }
    // bf16 results go out through LDS, whose stage slots are free now: the waves write the
    // rounded tile (or, when it does not fit, half of its rows at a time) row-major, 2*BN
    // bytes per row with 16-byte chunk c of row x stored at chunk c ^ (x % (BN/8)), and then
    // every store instruction writes whole rows of contiguous bytes. Stored
    // straight from the accumulators, each instruction would write 16 bytes into each of
    // 32 rows (32 partly written lines), which took 4-5 us per tile.
    constexpr int PR = CF::BM * CF::BN * 2 <= CF::LDS ? CF::BM : CF::BM / 2;  // rows per pass
    constexpr int CPR = CF::BN / 8;  // 16-byte chunks per row
    constexpr int RB = CF::BN * 2;   // bytes per row
    const bool v16 = dst.vec && (dst.ld % 8) == 0 && (reinterpret_cast<uintptr_t>(dst.base) & 15) == 0;
#pragma unroll
    for (int h = 0; h < CF::BM / PR; ++h) {
        __syncthreads();  // every wave is done with the stage slots, or with the previous pass
#pragma unroll
        for (int i = 0; i < MI; ++i) {
            const int rb = wm * 32 * MI + 32 * i;  // first tile row of block i (PR is a multiple of 32)
            if (rb / PR != h) continue;            // wave-uniform
            const int x = rb - h * PR + r;
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
#pragma unroll
                for (int vq = 0; vq < 4; ++vq) {
                    const int cc = 4 * (wn * NJ + j) + vq;  // 16-byte chunk of the row
                    uint2 v;
                    v.x = pack_bf16x2(acc[i][j][4 * vq], acc[i][j][4 * vq + 1]);
                    v.y = pack_bf16x2(acc[i][j][4 * vq + 2], acc[i][j][4 * vq + 3]);
                    *reinterpret_cast<uint2 *>(T + x * RB + 16 * (cc ^ (x & (CPR - 1))) + 8 * sl) = v;
                }
            }
        }
        __syncthreads();
        for (int k = threadIdx.x; k < PR * CPR; k += 64 * CF::NW) {
            const int x = k / CPR, cc = k % CPR;
            const int m = m0 + h * PR + x, n = n0 + 8 * cc;
            if (m >= M || n >= N) continue;
            const uint4 v = *reinterpret_cast<const uint4 *>(T + x * RB + 16 * (cc ^ (x & (CPR - 1))));
            uint16_t *g = reinterpret_cast<uint16_t *>(dst.base) + (size_t)(m - dst.r0) * dst.ld + (size_t)(n - dst.c0);
            if (v16 && n + 7 < N) {
                // Non-temporal (streaming) store: the tile is not read again by this kernel,
                // and lines left dirty in the XCD's L2 are written back before the kernel
                // completes. A/B on MI355X, whole calls with the reduce: 1-3 % at M = 2048
                // (k: 5 %), 5.5 % for gate at M = 128.
                __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4 *>(g));
            } else {
                const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (n + e < N) g[e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
            }
        }
    }
}

// Work decomposition, one-dimensional grid.
//   streamk == 0: full_tiles + tail_tiles * split workgroups. The first full_tiles
//     compute the tiles 0 .. full_tiles-1 over the whole reduction and write C; the
//     others compute each of the tiles full_tiles .. full_tiles+tail_tiles-1 over each
//     partition p, the blocks [floor(p*G/split), floor((p+1)*G/split)), and write plane
//     p of `part` (C itself when split = 1). Within each of the two regions the host
//     chooses the order: wide_item's XCD runs (the whole tiles being whole columns of
//     tiles), or workgroup q of the region taking tile q % tiles over partition
//     q / tiles. With full_tiles = 0 this is the plain split into `split` partitions
//     (equal ones when split divides G).
//   streamk == P > 0 (stream-K): the T*G (tile, block) units, tile-major, are cut into
//     P near-equal ranges, workgroup w taking units [floor(w*U/P), floor((w+1)*U/P)).
//     It walks them tile by tile: a tile it covers whole goes to C; the piece of a
//     tile it shares with other workgroups goes to its own slot of `part` (slot 2w for
//     its first tile, 2w+1 for its last; each a BM x BN tile, row-major), which the
//     fix-up kernel adds in workgroup order.
template <class CF, bool SK>
__global__ void __launch_bounds__(64 * CF::NW, CF::OCC)
w4a16_wide_kernel(const uint16_t *__restrict__ A, const uint32_t *__restrict__ Wq,
                  const uint16_t *__restrict__ scale, const uint16_t *__restrict__ bias,
                  uint16_t *__restrict__ C, void *__restrict__ part, int M, int N, int K,
                  int full_tiles, int tail_tiles, int split, int vec_store, int f32_part, int streamk,
                  int pm_full, int pm_tail)
{
    __shared__ __attribute__((aligned(1024))) Lds<CF> L;
    const int G = K >> 7;
    const int b = blockIdx.x;
    if (!SK) {
        // The whole tiles, then the split ones; within each region, in the XCD order of
        // wide_item when the host gives a panel height (pm > 0, whole columns of tiles), else
        // workgroup q of the region takes tile q % tiles over partition q / tiles.
        const bool whole = b < full_tiles;
        const int q = whole ? b : b - full_tiles;
        const int rt = whole ? full_tiles : tail_tiles;  // tiles of the region
        const int nparts = whole ? 1 : split;
        const int pm = whole ? pm_full : pm_tail;
        int tile, p;
        if (pm > 0) {
            const int num_m = (M + CF::BM - 1) / CF::BM;
            const qmm_impl::WideItem it = qmm_impl::wide_item(q, rt * nparts, num_m, rt / num_m, pm);
            tile = (whole ? 0 : full_tiles) + it.m + num_m * it.n;
            p = it.p;
        } else {
            tile = (whole ? 0 : full_tiles) + q % rt;
            p = q / rt;
        }
        const int g_lo = (int)(((long long)p * G) / nparts);
        const int g_hi = (int)(((long long)(p + 1) * G) / nparts);
        // C for an unsplit tile; else plane p of `part`, bf16 or (f32_part) fp32.
        Dest d;
        d.base = nparts > 1 ? static_cast<char *>(part) + (size_t)p * (size_t)M * (size_t)N * (f32_part ? 4 : 2)
                            : reinterpret_cast<char *>(C);
        d.ld = (size_t)N;
        d.r0 = d.c0 = 0;
        d.f32 = nparts > 1 && f32_part;
        d.vec = vec_store;
        segment<CF>(L, A, Wq, scale, bias, M, N, K, tile, g_lo, g_hi, d);
        return;
    }
    const int P = streamk;
    const int T = full_tiles + tail_tiles;  // every tile
    const long long U = (long long)T * G;
    const long long u0 = ((long long)b * U) / P;
    const long long u1 = ((long long)(b + 1) * U) / P;
    const int num_m = (M + CF::BM - 1) / CF::BM;
    for (long long u = u0; u < u1;) {
        const int tile = (int)(u / G);
        const int g_lo = (int)(u - (long long)tile * G);
        const int g_hi = (int)min((long long)G, u1 - (long long)tile * G);
        Dest d;
        if (g_lo == 0 && g_hi == G) {
            d.base = reinterpret_cast<char *>(C);
            d.ld = (size_t)N;
            d.r0 = d.c0 = 0;
            d.f32 = false;
            d.vec = vec_store;
        } else {
            const size_t slot = 2 * (size_t)b + (u == u0 ? 0 : 1);
            d.base = static_cast<char *>(part) + slot * (size_t)CF::BM * CF::BN * (f32_part ? 4 : 2);
            d.ld = CF::BN;
            d.r0 = (tile % num_m) * CF::BM;
            d.c0 = (tile / num_m) * CF::BN;
            d.f32 = f32_part;
            d.vec = 1;
        }
        if (u != u0) __syncthreads();  // every wave has left the previous segment's LDS
        segment<CF>(L, A, Wq, scale, bias, M, N, K, tile, g_lo, g_hi, d);
        u = (long long)tile * G + g_hi;
    }
}

// Stream-K fix-up: workgroup (t, chunk) merges 2048 elements (8 rows of 256) of tile t if
// the stream-K ranges split it. The workgroups that touch tile t are those whose unit
// ranges meet [t*G, (t+1)*G); their pieces sit in slot 2w (when the tile is w's first) or
// 2w+1 (its last), and are added in ascending w (ascending reduction order) in fp32,
// with one cast to bf16 into C. A lane owns eight consecutive columns (16-byte loads of
// bf16 slots, two of fp32 ones).
template <int BM, typename T>
__global__ void __launch_bounds__(256)
streamk_fixup(const T *__restrict__ part, uint16_t *__restrict__ C, int M, int N, int G, int T_tiles, int P,
              int vec)
{
    const int t = blockIdx.x;
    const long long U = (long long)T_tiles * G;
    const long long lo = (long long)t * G, hi = lo + G;  // the tile's units
    // first workgroup whose range contains unit lo: the largest w with floor(w*U/P) <= lo
    int w0 = (int)((lo * P) / U);
    while (w0 + 1 < P && ((long long)(w0 + 1) * U) / P <= lo) ++w0;
    while (w0 > 0 && ((long long)w0 * U) / P > lo) --w0;
    int w1 = w0;  // last workgroup whose range starts before hi
    while (w1 + 1 < P && ((long long)(w1 + 1) * U) / P < hi) ++w1;
    const long long s0 = ((long long)w0 * U) / P, e0 = ((long long)(w0 + 1) * U) / P;
    if (w0 == w1 && s0 <= lo && e0 >= hi) return;  // one workgroup covered it whole: already in C
    const int num_m = (M + BM - 1) / BM;
    const int idx = blockIdx.y * 256 + threadIdx.x;  // 8-column group of the tile
    const int rr = idx >> 5, cc = 8 * (idx & 31);
    const int m = (t % num_m) * BM + rr, n = (t / num_m) * 256 + cc;
    if (rr >= BM || m >= M || n >= N) return;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int w = w0; w <= w1; ++w) {
        const size_t slot = 2 * (size_t)w + ((((long long)w * U) / P >= lo) ? 0 : 1);
        const T *src = part + slot * (size_t)BM * 256 + (size_t)rr * 256 + cc;
        float v[8];
        if constexpr (sizeof(T) == 4) {
            const float4 a = *reinterpret_cast<const float4 *>(src);
            const float4 b = *reinterpret_cast<const float4 *>(src + 4);
            v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
        } else {
            const uint4 x = *reinterpret_cast<const uint4 *>(src);
            const uint32_t wd[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[2 * e] = bf16_to_f32(wd[e] & 0xFFFFu);
                v[2 * e + 1] = bf16_to_f32(wd[e] >> 16);
            }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = acc[e] + v[e];
    }
    uint16_t *dst = C + (size_t)m * N + n;
    if (vec && n + 7 < N) {
        uint4 o;
        o.x = pack_bf16x2(acc[0], acc[1]);
        o.y = pack_bf16x2(acc[2], acc[3]);
        o.z = pack_bf16x2(acc[4], acc[5]);
        o.w = pack_bf16x2(acc[6], acc[7]);
        *reinterpret_cast<uint4 *>(dst) = o;
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (n + e < N) dst[e] = (uint16_t)f32_to_bf16(acc[e]);
    }
}

template <int BITS, int SUB>
using CfgV0 = Cfg<1, 4, 2, BITS, SUB>;  // 128 x 256 tile, 4 waves of 128 x 64
template <int BITS, int SUB>
using CfgV2 = Cfg<2, 8, 1, BITS, SUB>;  // 256 x 256 tile, 8 waves of 256 x 32
template <int BITS, int SUB>
using CfgV1 = Cfg<1, 4, 1, BITS, SUB, 128>;  // 128 x 128 tile, 4 waves of 128 x 32

template <class CF>
void launch_cfg(dim3 grid, hipStream_t stream, const uint16_t *a, const uint32_t *w, const uint16_t *sc,
                const uint16_t *bi, uint16_t *c, void *pt, int M, int N, int K, int full_tiles, int tail_tiles,
                int split, int vec, int f32p, int streamk)
{
    if (streamk == 0) {
        // XCD order of each region (whole columns of 256-column tiles): A's row block and W's
        // column block (packed codes plus scale and bias) over one partition of the region.
        // MI355X, M = 2048 Qwen3-4B projections, same results: down 2-3 % faster, gate and up
        // 0.2-0.7 %, q and o unchanged; on the 128 x 128 tiles (k and v) 3 % slower, so those
        // keep the plain order.
        const int num_m = (M + CF::BM - 1) / CF::BM;
        const int G = K >> 7;
        int pm_full = 0, pm_tail = 0;
        if (CF::BN == 256 && full_tiles % num_m == 0) {
            const double gf = (double)G, gt = (double)G / split;
            const double a_blk = (double)CF::BM * 256.0, w_blk = (double)CF::BN * (64.0 * CF::BITS / 4.0 + 4.0 * CF::SUB);
            if (full_tiles > 0) pm_full = qmm_impl::wide_panel(1, full_tiles / num_m, num_m, gf * a_blk, gf * w_blk);
            if (tail_tiles > 0) pm_tail = qmm_impl::wide_panel(split, tail_tiles / num_m, num_m, gt * a_blk, gt * w_blk);
        }
        hipLaunchKernelGGL((w4a16_wide_kernel<CF, false>), grid, dim3(64 * CF::NW), 0, stream, a, w, sc, bi, c, pt,
                           M, N, K, full_tiles, tail_tiles, split, vec, f32p, 0, pm_full, pm_tail);
    } else if constexpr (CF::BITS == 4 && CF::SUB == 1 && CF::BN == 256) {  // stream-K: W4A16 g128, 256 columns
        hipLaunchKernelGGL((w4a16_wide_kernel<CF, true>), grid, dim3(64 * CF::NW), 0, stream, a, w, sc, bi, c, pt,
                           M, N, K, full_tiles, tail_tiles, split, vec, f32p, streamk, 0, 0);
        const int T = full_tiles + tail_tiles;
        const dim3 fgrid(T, CF::BM * 256 / (256 * 8));
        // 16-byte stores into C need N % 8 == 0 and a 16-byte aligned C
        const int cvec = (N % 8 == 0 && (reinterpret_cast<uintptr_t>(c) & 15) == 0) ? 1 : 0;
        if (f32p)
            hipLaunchKernelGGL((streamk_fixup<CF::BM, float>), fgrid, dim3(256), 0, stream,
                               static_cast<const float *>(pt), c, M, N, K >> 7, T, streamk, cvec);
        else
            hipLaunchKernelGGL((streamk_fixup<CF::BM, uint16_t>), fgrid, dim3(256), 0, stream,
                               static_cast<const uint16_t *>(pt), c, M, N, K >> 7, T, streamk, cvec);
    }
}

template <int BITS, int SUB>
void launch_variant(int variant, dim3 grid, hipStream_t stream, const uint16_t *a, const uint32_t *w,
                    const uint16_t *sc, const uint16_t *bi, uint16_t *c, void *pt, int M, int N, int K,
                    int full_tiles, int tail_tiles, int split, int vec, int f32p, int streamk)
{
    if (variant == 0)
        launch_cfg<CfgV0<BITS, SUB>>(grid, stream, a, w, sc, bi, c, pt, M, N, K, full_tiles, tail_tiles, split, vec,
                                     f32p, streamk);
    else if (variant == 1)
        launch_cfg<CfgV1<BITS, SUB>>(grid, stream, a, w, sc, bi, c, pt, M, N, K, full_tiles, tail_tiles, split, vec,
                                     f32p, streamk);
    else
        launch_cfg<CfgV2<BITS, SUB>>(grid, stream, a, w, sc, bi, c, pt, M, N, K, full_tiles, tail_tiles, split, vec,
                                     f32p, streamk);
}

}  // namespace

namespace qmm_impl {

// The per-lane copy offsets are 32-bit byte offsets within 256 rows of A: K < 2^22.
hipError_t launch_w4a16_wide(WFormat fmt, int variant, const void *A, const void *Wq, const void *scale,
                             const void *bias, void *C, void *part, bool f32_part, int M, int N, int K,
                             int full_tiles, int split, bool vec_store, hipStream_t stream, int streamk)
{
    if (K >= (1 << 22) || variant < 0 || variant > 2 || !format_supported(fmt)) return hipErrorInvalidValue;
    const int rows = wide_rows(variant), cols = wide_cols(variant);
    const int tiles = ((M + rows - 1) / rows) * ((N + cols - 1) / cols);
    if (streamk > 0 && variant == 1) return hipErrorInvalidValue;
    if (streamk < 0 || (streamk > 0 && (!part || (long long)streamk > (long long)tiles * (K / 128))))
        return hipErrorInvalidValue;
    if (streamk > 0 && (fmt.bits != 4 || fmt.group != 128)) return hipErrorInvalidValue;
    if (streamk > 0) {
        full_tiles = tiles;  // T = full_tiles + tail_tiles for the kernel
        split = 1;
    }
    if (full_tiles < 0 || full_tiles > tiles || split < 1 || split > K / 128) return hipErrorInvalidValue;
    if (split > 1 && !part) return hipErrorInvalidValue;
    const int tail_tiles = tiles - full_tiles;
    const dim3 grid(streamk > 0 ? streamk : full_tiles + tail_tiles * split);
    const uint16_t *a = static_cast<const uint16_t *>(A);
    const uint32_t *w = static_cast<const uint32_t *>(Wq);
    const uint16_t *sc = static_cast<const uint16_t *>(scale);
    const uint16_t *bi = static_cast<const uint16_t *>(bias);
    uint16_t *c = static_cast<uint16_t *>(C);
    const int vec = vec_store ? 1 : 0;
    const int f32p = f32_part ? 1 : 0;
    (void)hipGetLastError();
#define QMM_FMT(B_, S_)                                                                                          \
    if (fmt.bits == B_ && fmt.sub() == S_)                                                                       \
        launch_variant<B_, S_>(variant, grid, stream, a, w, sc, bi, c, part, M, N, K, full_tiles, tail_tiles,    \
                               split, vec, f32p, streamk);
    QMM_FMT(4, 1) QMM_FMT(4, 2) QMM_FMT(4, 4) QMM_FMT(8, 1) QMM_FMT(8, 2) QMM_FMT(8, 4)
#undef QMM_FMT
    return hipGetLastError();
}

}  // namespace qmm_impl
