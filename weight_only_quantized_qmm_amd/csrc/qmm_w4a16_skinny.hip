// qmm_w4a16_skinny.hip -- weight-only quantized matmul kernel for few rows (M <= 64, and up to
// 128 rows over small weight matrices) on gfx950: W4A16 group 128, and the other formats of
// the library (4- or 8-bit codes, groups of 32, 64 or 128 values).
//
// Same contract as the other W4A16 kernels (tiny-llm "Week 2 Day 7: Split-K
// Prefill", Task 2): blockIdx.z is the partition p of s = gridDim.z, the workgroup covers
// the 128-value blocks [floor(p*G/s), floor((p+1)*G/s)) of the reduction (the page's equal
// partitions when s divides G) and writes its tile into plane p of `out` (C itself when
// s = 1), with plain stores and no atomics.
//
// With few rows the op streams the packed weights once and is bound by memory
// latency and bandwidth, not by the matrix cores (a dispatch on MI355X costs about
// 1.6 us before the first byte arrives). The design therefore maximises the bytes
// in flight per wave and keeps the work in one dispatch where possible:
//   * a workgroup owns a (16*MT) x tw output tile (tw <= 16*NS columns: the host narrows
//     an unsplit grid of 16-column tiles that has fewer tiles than CUs, and the subtile's
//     columns past tw re-read the tile's last weight row and are not stored) and up to 16
//     waves; the waves split the tile's reduction range, wave w taking groups g0 + w,
//     g0 + w + WAVES, ... of its partition;
//   * each wave issues every load of a round of up to GPW groups before it computes:
//     the round's activations go straight into the wave's own LDS staging slots
//     (global_load_lds, 1 KB per instruction: four rows of 256 bytes, so each copy
//     touches 8 whole cache lines), the scale/bias entries of its rows into the wave's
//     own LDS arrays (global_load_lds, 64 entries per instruction), and the packed
//     weights into registers (one 16-byte load per lane and 16-column subtile; 16 rows
//     of 64 bytes); then it waits once and runs the MFMAs of the round, reading its
//     activation operands and scale/bias from LDS; with one group per round the next
//     round's weights and scale/bias go out before those MFMAs, the activations after;
//   * the waves' fp32 tiles meet in LDS and are summed in ascending wave order
//     (deterministic), rounded once to bf16 and stored with 8-byte stores (4-byte pairs
//     where a tile's width is not a multiple of 4).
// Loading the activations in MFMA operand order straight into registers instead touches
// four times as many cache lines per byte (16 rows x 4 pieces per instruction); on the
// Qwen3-4B projections at M = 16..64 the staged copies are 5-15 % faster.
// Weights are dequantised in registers: w = scale*q + bias in fp32, rounded to
// bf16 (each weight is used by all 16*MT rows of the tile from the same registers).
// A lane's share of a 128-value block is 32 consecutive values of one row: 16 bytes of
// 4-bit codes or 32 bytes of 8-bit codes, and the scale/bias of the group holding them
// (block g, lane slot c: group (4g + c) * 32 / group_size).
// The 16x16x32 MFMA takes the weights as its first operand, so a lane's result is
// four consecutive output columns of one row.
//
// LDS: wave w's staging slots are [GPW][RS rows][256 bytes] at w*GPW*RS*256 (RS = 16*MT, or
// 4 or 8 for decode, whose 16 operand rows then read the staged rows cyclically); chunk c
// (16 bytes) of row r is stored at chunk c ^ (r % 16), so the 16 rows that one 16-lane
// phase of an operand read touches fall on distinct banks. The waves' scale and bias
// arrays follow the staging slots. The waves' fp32 tiles for the cross-wave sum follow
// those when everything fits in the LDS, else reuse the staging memory after the main loop.
#include "qmm_device.h"
#include "qmm_launch.h"

using namespace qmm_dev;

namespace {

constexpr int MAX_WAVES = 16;

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ uint32_t lds_addr(const void *p) { return (uint32_t)(uintptr_t)(const lds_void *)p; }

// Global -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4): lane i's data lands at
// LDS byte lds_off + 16*i (lds_off wave-uniform, in M0); global address = scalar base +
// 32-bit lane offset. Inline assembly: the compiler neither tracks nor waits for it.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void copy16(uint32_t lds_off, uint32_t voff, const void *sbase)
{
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds_off), "v"(voff), "s"(sbase)
                 : "memory", "m0");
}
// The same for 2 bytes per lane (global_load_lds_ushort), zero-extended into the dword at
// LDS byte lds_off + 4*i.
__device__ __forceinline__ void copy2(uint32_t lds_off, uint32_t voff, const void *sbase)
{
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_ushort %1, %2" ::"s"(lds_off), "v"(voff), "s"(sbase)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

template <int BITS, int MT, int NS, int GPW, int MAXW, int RS>
__global__ void __launch_bounds__(64 * MAXW)
w4a16_skinny_kernel(const uint16_t *__restrict__ A, const uint32_t *__restrict__ Wq,
                    const uint16_t *__restrict__ scale, const uint16_t *__restrict__ bias,
                    void *__restrict__ out, int M, int N, int K, int tw, int sub_shift, int vec_store,
                    int f32_part, int sum_off)
{
    constexpr int WV = BITS / 4;  // 16-byte weight loads per lane, group and 16-column subtile
    // RS staged activation rows per group (16*MT, or 4 or 8 for decode: MT = 1, M <= RS); one
    // staged group is RS rows x 128 values
    static_assert(RS == 16 * MT || (MT == 1 && (RS == 4 || RS == 8)), "staged rows");
    constexpr int ABYTES = RS * 256;
    constexpr int NCPY = RS / 4;  // activation copies per group
    extern __shared__ __attribute__((aligned(1024))) char smem[];  // staging, then [WAVES][MT][NS][64] float4
    // Fetch every argument (and the grid's partition count and workgroup size) up front,
    // in one batch of scalar loads: left to itself the compiler loads the pointers after
    // the first branch, and a use of the pointers alone splits the loads into two
    // dependent memory round trips before the first weight load.
    const unsigned nz = gridDim.z, nt = blockDim.x;
    asm volatile("" ::"s"(A), "s"(Wq), "s"(scale), "s"(bias), "s"(out), "s"(M), "s"(N), "s"(K), "s"(tw),
                 "s"(sub_shift), "s"(vec_store), "s"(f32_part), "s"(sum_off), "s"(nz), "s"(nt));
    const int waves = __builtin_amdgcn_readfirstlane(nt >> 6);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    const int r = lane & 15;
    const int slot = lane >> 4;
    // The workgroup's columns: [n_blk, n_end), tw of them (tw <= 16*NS; fewer than the
    // subtiles hold when the host narrows the tiles to spread the grid over every CU).
    const int n_blk = blockIdx.x * tw;
    const int n_end = min(N, n_blk + tw);
    const int m_blk = blockIdx.y * (16 * MT);
    const int GG = (K >> 7) << sub_shift;  // scale/bias entries per row (128 / group_size per block)
    const int G = K >> 7;  // 128-value blocks of the reduction
    // Partition bounds floor(p*G/s) in 32-bit unsigned arithmetic ((p+1)*G < 2^31: the host
    // keeps K below 2^22), and none at all when unsplit: every wave evaluates them on the
    // CU's shared scalar unit before its first load, and a 64-bit division is a software
    // routine of over a hundred scalar instructions.
    const unsigned Gu = (unsigned)G, S = nz, Z = blockIdx.z;
    const int g0 = S == 1 ? 0 : (int)((Z * Gu) / S);
    const int gpp = S == 1 ? G : (int)(((Z + 1) * Gu) / S) - g0;  // this partition's blocks
    // this wave's groups: g0 + wave + waves*i for the i with has(i), i.e. i < ceil((gpp -
    // wave) / waves), tested without the division (a few dozen scalar instructions per wave,
    // on the CU's shared scalar unit, before the first load)
    auto has = [&](const int i) { return wave + waves * i < gpp; };

    const uint4 *wptr[NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) {
        const int n = min(n_blk + 16 * j + r, n_end - 1);  // rows past the tile re-read its last row, never stored
        wptr[j] = reinterpret_cast<const uint4 *>(Wq + (size_t)n * (size_t)(K * BITS / 32)) + WV * slot;
    }
    // Activation copies: copy c (0 .. 4*MT-1) of a group fills staging rows 4c .. 4c+3; lane i
    // lands at row 4c + i/16, stored chunk i%16, so it fetches chunk (i%16) ^ (row%16) of the
    // group's 256 bytes of that row. Rows past M re-read row M-1; a copy whose rows all lie
    // past M is not issued at all, and its staging rows keep whatever they held. An MFMA
    // output row depends only on its own activation row, so such rows reach only output rows
    // past M, which are never stored (decode with M = 1..8 saves up to 15 of 16 copies).
    uint32_t a_voff[NCPY];
#pragma unroll
    for (int c = 0; c < NCPY; ++c) {
        const int row = 4 * c + (lane >> 4);
        const int m = min(m_blk + row, M - 1);
        a_voff[c] = (uint32_t)m * (uint32_t)K * 2u + 16u * (uint32_t)((lane & 15) ^ (row & 15));
    }
    char *stage = smem + (size_t)wave * GPW * ABYTES;
    const uint32_t stage_lds = lds_addr(stage);
    // Operand reads: lane (r, slot), step t, row tile i: staging row 16i + r, chunk 4*slot + t
    // (values 32*slot + 8t .. +7 of the group). With fewer staged rows (RS < 16) operand row r
    // reads staging row r % RS: rows from RS on are copies that reach only output rows past
    // M, never stored.
    const int rr = RS < 16 ? (r & (RS - 1)) : r;
    uint32_t a_rd[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) a_rd[t] = (uint32_t)(rr * 256 + 16 * ((4 * slot + t) ^ rr));

    // Scale/bias: each round also copies, next to its activations, the scale and bias
    // entries its groups need into the wave's own dword arrays [16*NS rows][GPW*SUB] (SUB =
    // entries per 128-value block): entry (row, q, e) at row*GPW*SUB + q*SUB + e, the bias
    // array AW dwords (whole copies) after the scale array. One copy moves 64 entries;
    // per-group loads of 16 rows each would touch four times the cache lines.
    const int RW = GPW << sub_shift;            // dwords per row of a wave's arrays
    const int EW = 16 * NS * RW;                // entries per array
    const int ncp = (EW + 63) >> 6;             // copies per array and round
    const int AW = ncp << 6;
    uint32_t *sbw = reinterpret_cast<uint32_t *>(smem + (size_t)waves * GPW * ABYTES) + (size_t)wave * 2 * AW;
    const uint32_t sbw_lds = lds_addr(sbw);
    const int sub_e = slot >> (2 - sub_shift);  // the lane's entry within a block
    f32x4 acc[MT][NS];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NS; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const char *Abase = reinterpret_cast<const char *>(A);
    // The loads of the round starting at group index base (of this wave's groups):
    // activation copies into the staging slots, scale/bias copies into the wave's arrays,
    // packed weights into registers.
    auto issue_a = [&](const int base) {
#pragma unroll
        for (int q = 0; q < GPW; ++q) {
            if (!has(base + q)) break;  // uniform across the wave
            const char *Ag = Abase + (size_t)(g0 + wave + waves * (base + q)) * 256;
#pragma unroll
            for (int c = 0; c < NCPY; ++c)
                if (m_blk + 4 * c < M)  // a copy whose four rows all lie past M is skipped (see below)
                    copy16(stage_lds + (uint32_t)(q * ABYTES + 1024 * c), a_voff[c], Ag);
        }
    };
    auto issue_sb = [&](const int base) {
        int nq = 1;  // groups of this round (has(base) holds)
#pragma unroll
        for (int q = 1; q < GPW; ++q)
            if (has(base + q)) nq = q + 1;
        for (int c = 0; c < ncp; ++c) {
            const int e = min(64 * c + lane, EW - 1);  // past the array: re-read its last entry
            const int row_e = (e >> sub_shift) / GPW;  // = e / RW
            const int rem = e - row_e * RW;
            const int row = min(row_e, n_end - 1 - n_blk);  // rows past the tile re-read its last row (never used)
            const int q = min(rem >> sub_shift, nq - 1);  // slots past the round re-read its last group
            const int g = g0 + wave + waves * (base + q);
            const uint32_t voff = 2u * (uint32_t)(row * GG + (g << sub_shift) + (rem & ((1 << sub_shift) - 1)));
            copy2(sbw_lds + 256u * (uint32_t)c, voff, scale + (size_t)n_blk * GG);
            copy2(sbw_lds + 4u * (uint32_t)AW + 256u * (uint32_t)c, voff, bias + (size_t)n_blk * GG);
        }
    };
    uint4 wn[GPW][NS][WV];  // the packed weights of the next round, in flight
    auto issue_w = [&](const int base) {
#pragma unroll
        for (int q = 0; q < GPW; ++q) {
            if (!has(base + q)) break;  // uniform across the wave
            const int g = g0 + wave + waves * (base + q);
#pragma unroll
            for (int j = 0; j < NS; ++j) {
#pragma unroll
                for (int u = 0; u < WV; ++u) wn[q][j][u] = wptr[j][4 * WV * g + u];
            }
        }
    };
    // A wave may have no groups at all (a partition with fewer groups than the workgroup
    // has waves); it issues nothing and contributes zeros to the sum.
    if (has(0)) {
        issue_a(0);
        issue_sb(0);
        issue_w(0);
    }
    for (int base = 0; has(base); base += GPW) {
        // Without the scheduling fences the compiler sinks each load next to its first use,
        // one memory round trip per load. The copies are invisible to the compiler, so
        // the wave waits for all of its loads itself before it reads the staging slots.
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        uint4 wv[GPW][NS][WV];
        uint32_t sc[GPW][NS], bi[GPW][NS];
#pragma unroll
        for (int q = 0; q < GPW; ++q)
#pragma unroll
            for (int j = 0; j < NS; ++j)
#pragma unroll
                for (int u = 0; u < WV; ++u) wv[q][j][u] = wn[q][j][u];
#pragma unroll
        for (int q = 0; q < GPW; ++q) {
            if (!has(base + q)) break;
#pragma unroll
            for (int j = 0; j < NS; ++j) {
                sc[q][j] = sbw[(16 * j + r) * RW + (q << sub_shift) + sub_e];
                bi[q][j] = sbw[AW + (16 * j + r) * RW + (q << sub_shift) + sub_e];
            }
        }
        // With one group per round, the next round's weights and scale/bias entries go out
        // before this round's MFMAs (the scale/bias arrays are free once read), so their
        // memory latency overlaps this round's arithmetic and the next round's activation
        // copies, which wait for the staging slots that this round's operand reads still
        // use. With two or three groups per round the early loads were slower (MI355X, the
        // Qwen3-4B projections at M = 1..64), and the whole next round goes out after the
        // MFMAs.
        constexpr bool kEarly = GPW == 1;
        const bool more = has(base + GPW);  // uniform across the wave
        if (kEarly && more) {
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            issue_sb(base + GPW);
            issue_w(base + GPW);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < GPW; ++q) {
            if (!has(base + q)) break;  // uniform across the wave
            const char *As = stage + q * ABYTES;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                // step t: values 8t .. 8t+7 of the lane's 32 (one word of 4-bit codes, two
                // words of 8-bit codes); the activation operands of the MT row tiles
                uint4 av[MT];
#pragma unroll
                for (int i = 0; i < MT; ++i) av[i] = *reinterpret_cast<const uint4 *>(As + 4096 * i + a_rd[t]);
#pragma unroll
                for (int j = 0; j < NS; ++j) {
                    const float s_ = bf16_to_f32(sc[q][j]);
                    const float b_ = bf16_to_f32(bi[q][j]);
                    const bf16x8 b = as_bf16x8(
                        BITS == 4 ? dequant8(word_of(wv[q][j][0], t), s_ * 512.f, b_)
                                  : dequant8_u8(word_of(wv[q][j][(t >> 1) % WV], 2 * (t & 1)),
                                                word_of(wv[q][j][(t >> 1) % WV], 2 * (t & 1) + 1), s_, b_));
#pragma unroll
                    for (int i = 0; i < MT; ++i) acc[i][j] = mfma16x16x32(b, as_bf16x8(av[i]), acc[i][j]);
                }
            }
        }
        if (more) {
            // every operand read of the staging slots (and of the scale/bias arrays) has
            // returned before they are refilled
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            issue_a(base + GPW);
            if (!kEarly) {
                issue_sb(base + GPW);
                issue_w(base + GPW);
            }
        }
    }

    // Cross-wave sum in LDS: wave w stores its tiles, then each of the MT*NS*64 lane-quads
    // (i, j, lane) is owned by one thread (strided over the workgroup), which adds the
    // waves' values in order w = 0, 1, ... The tiles sit at byte sum_off: past the staging
    // memory when both fit (a wave stores as soon as it is done), else over it (sum_off = 0:
    // every wave must first have left its staging slots).
    if (sum_off == 0) __syncthreads();  // uniform: a kernel argument
    f32x4 *red4 = reinterpret_cast<f32x4 *>(smem + sum_off);
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NS; ++j) red4[((wave * MT + i) * NS + j) * 64 + lane] = acc[i][j];
    __syncthreads();
    for (int t = threadIdx.x; t < MT * NS * 64; t += (int)nt) {
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
            // vec_store (N % 4 == 0, aligned buffers): a whole quad starting on a multiple of 4
            // in one store, else pairs starting on an even column (tiles of a width that is
            // not a multiple of 4 start on any even column), else single elements
            const bool quad = vec_store && (n & 3) == 0 && n + 3 < n_end;
            if (f32_part && nz > 1) {
                float *dst = static_cast<float *>(out) + e;
                if (quad) {
                    *reinterpret_cast<float4 *>(dst) = make_float4(sum[0], sum[1], sum[2], sum[3]);
                } else {
#pragma unroll
                    for (int e2 = 0; e2 < 4; e2 += 2) {
                        const int c = n + e2;
                        if (vec_store && (c & 1) == 0 && c + 1 < n_end) {
                            *reinterpret_cast<float2 *>(dst + e2) = make_float2(sum[e2], sum[e2 + 1]);
                        } else {
                            if (c < n_end) dst[e2] = sum[e2];
                            if (c + 1 < n_end) dst[e2 + 1] = sum[e2 + 1];
                        }
                    }
                }
            } else {
                uint16_t *dst = static_cast<uint16_t *>(out) + e;
                if (quad) {
                    uint2 v;
                    v.x = pack_bf16x2(sum[0], sum[1]);
                    v.y = pack_bf16x2(sum[2], sum[3]);
                    *reinterpret_cast<uint2 *>(dst) = v;
                } else {
#pragma unroll
                    for (int e2 = 0; e2 < 4; e2 += 2) {
                        const int c = n + e2;
                        if (vec_store && (c & 1) == 0 && c + 1 < n_end) {
                            *reinterpret_cast<uint32_t *>(dst + e2) = pack_bf16x2(sum[e2], sum[e2 + 1]);
                        } else {
                            if (c < n_end) dst[e2] = (uint16_t)f32_to_bf16(sum[e2]);
                            if (c + 1 < n_end) dst[e2 + 1] = (uint16_t)f32_to_bf16(sum[e2 + 1]);
                        }
                    }
                }
            }
        }
    }
}

template <int BITS, int MT, int NS, int GPW, int MAXW, int RS>
hipError_t launch_cfg(const void *A, const void *Wq, const void *scale, const void *bias, void *out, bool f32_part,
                      int M, int N, int K, int tw, int s, int sub_shift, int waves, bool vec_store,
                      hipStream_t stream)
{
    if (tw < 1 || tw > 16 * NS) return hipErrorInvalidValue;
    const dim3 grid((N + tw - 1) / tw, (M + 16 * MT - 1) / (16 * MT), s);
    const size_t stage = qmm_impl::skinny_stage_bytes(MT, NS, waves, GPW, 1 << sub_shift, RS);
    const size_t sums = qmm_impl::skinny_sum_bytes(MT, NS, waves);
    // the waves' tiles beside the staging memory when both fit (16-byte aligned: stage is a
    // multiple of 256), else over it
    const bool apart = stage + sums <= (size_t)qmm_impl::kLdsPerCU;
    const size_t lds = apart ? stage + sums : qmm_impl::skinny_lds_bytes(MT, NS, waves, GPW, 1 << sub_shift, RS);
    if (RS < 16 && M > RS) return hipErrorInvalidValue;
    if (waves > MAXW || lds > (size_t)qmm_impl::kLdsPerCU) return hipErrorInvalidValue;
    // the activation copies take 32-bit byte offsets into A
    if ((size_t)M * (size_t)K * 2 >= ((size_t)1 << 32)) return hipErrorInvalidValue;
    (void)hipGetLastError();
    hipLaunchKernelGGL((w4a16_skinny_kernel<BITS, MT, NS, GPW, MAXW, RS>), grid, dim3(64 * waves), lds, stream,
                       static_cast<const uint16_t *>(A), static_cast<const uint32_t *>(Wq),
                       static_cast<const uint16_t *>(scale), static_cast<const uint16_t *>(bias),
                       out, M, N, K, tw, sub_shift, vec_store ? 1 : 0, f32_part ? 1 : 0, apart ? (int)stage : 0);
    return hipGetLastError();
}

}  // namespace

namespace qmm_impl {

// The host picks (mt, ns, gpw, waves) with skinny_shape (qmm_launch.h); these are the
// configurations it can return: 16-column tiles (ns 1, mt 1 or 2) with up to 12 waves and gpw <= 3;
// 32-column tiles (ns 2) with up to 16 waves (mt 1) or 8 (mt 2, 4) and gpw <= 3, 3, 2;
// 48- and 64-column tiles (ns 3, 4) with up to 8 waves and gpw <= 2, 2, 1 for mt 1, 2, 4 (register
// budgets of 128 VGPRs per lane at 16 waves, 256 at 8). 8-bit codes take one group less per
// round where the 4-bit limit is above one. Decode with 4-bit codes on 16- and 48-column
// tiles of one 16-row block stages 4 or 8 activation rows per group instead of 16 (skinny_rows).
hipError_t launch_w4a16_skinny(WFormat fmt, int mt, int ns, int tw, int gpw, int waves, const void *A,
                               const void *Wq, const void *scale, const void *bias, void *out, bool f32_part, int M,
                               int N, int K, int s, bool vec_store, hipStream_t stream)
{
    if (waves < 1 || waves > MAX_WAVES || !format_supported(fmt)) return hipErrorInvalidValue;
    const int sub_shift = fmt.group == 128 ? 0 : fmt.group == 64 ? 1 : 2;
    const int rows = skinny_rows(mt, ns, fmt.bits, M);
#define QMM_CFGR(B_, MT_, NS_, GPW_, MAXW_, RS_)                                                               \
    if (fmt.bits == B_ && mt == MT_ && ns == NS_ && gpw == GPW_ && rows == RS_)                                \
        return launch_cfg<B_, MT_, NS_, GPW_, MAXW_, RS_>(A, Wq, scale, bias, out, f32_part, M, N, K, tw, s,    \
                                                          sub_shift, waves, vec_store, stream);
#define QMM_CFG(B_, MT_, NS_, GPW_, MAXW_) QMM_CFGR(B_, MT_, NS_, GPW_, MAXW_, 16 * MT_)
    QMM_CFG(4, 1, 1, 1, 16) QMM_CFG(4, 1, 1, 2, 16) QMM_CFG(4, 1, 1, 3, 16)
    QMM_CFG(4, 1, 2, 1, 16) QMM_CFG(4, 1, 2, 2, 16) QMM_CFG(4, 1, 2, 3, 16)
    QMM_CFG(4, 2, 2, 1, 8) QMM_CFG(4, 2, 2, 2, 8) QMM_CFG(4, 2, 2, 3, 8)
    QMM_CFG(4, 4, 2, 1, 8) QMM_CFG(4, 4, 2, 2, 8)
    QMM_CFG(4, 1, 4, 1, 8) QMM_CFG(4, 1, 4, 2, 8)
    QMM_CFG(4, 2, 4, 1, 8) QMM_CFG(4, 2, 4, 2, 8)
    QMM_CFG(4, 4, 4, 1, 8)
    QMM_CFG(4, 1, 3, 1, 8) QMM_CFG(4, 1, 3, 2, 8)
    QMM_CFG(4, 2, 3, 1, 8) QMM_CFG(4, 2, 3, 2, 8)
    QMM_CFG(4, 4, 3, 1, 8)
    QMM_CFG(4, 2, 1, 1, 16) QMM_CFG(4, 2, 1, 2, 16) QMM_CFG(4, 2, 1, 3, 16)
    QMM_CFG(8, 1, 1, 1, 16) QMM_CFG(8, 1, 1, 2, 16)
    QMM_CFG(8, 2, 1, 1, 16) QMM_CFG(8, 2, 1, 2, 16)
    QMM_CFG(8, 1, 2, 1, 16) QMM_CFG(8, 1, 2, 2, 16)
    QMM_CFG(8, 2, 2, 1, 8) QMM_CFG(8, 2, 2, 2, 8)
    QMM_CFG(8, 4, 2, 1, 8)
    QMM_CFG(8, 1, 4, 1, 8)
    QMM_CFG(8, 2, 4, 1, 8)
    QMM_CFG(8, 4, 4, 1, 8)
    QMM_CFG(8, 1, 3, 1, 8) QMM_CFG(8, 2, 3, 1, 8) QMM_CFG(8, 4, 3, 1, 8)
    // decode: 4 or 8 staged activation rows (skinny_rows)
    QMM_CFGR(4, 1, 1, 1, 16, 4) QMM_CFGR(4, 1, 1, 2, 16, 4) QMM_CFGR(4, 1, 1, 3, 16, 4)
    QMM_CFGR(4, 1, 1, 1, 16, 8) QMM_CFGR(4, 1, 1, 2, 16, 8) QMM_CFGR(4, 1, 1, 3, 16, 8)
    QMM_CFGR(4, 1, 3, 1, 8, 8) QMM_CFGR(4, 1, 3, 2, 8, 8)
#undef QMM_CFG
#undef QMM_CFGR
    return hipErrorInvalidValue;
}

}  // namespace qmm_impl
