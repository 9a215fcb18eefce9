// qmm_launch.h -- internal interface between the C-ABI host code (qmm_api.cpp)
// and the gfx950 kernels (*.hip). Not installed; the public ABI is include/qmm.h.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>

namespace qmm_impl {

// Which W4A16 kernel runs a problem, and the output tile of one workgroup.
//   SKINNY (M <= 64, or M <= 128 with N*K <= 2^24): a (16*mt) x tw tile (tw = 16*ns, ns 1 to 4,
//          or fewer columns for a narrowed unsplit grid of 16-column tiles),
//          up to 16 waves splitting its reduction;
//   WIDE   (otherwise): a 128 x 256 (variant 0), 128 x 128 (variant 1) or 256 x 256
//          (variant 2) tile; mt = 8 or 16.
enum W4A16Kind { W4A16_SKINNY = 0, W4A16_WIDE = 2 };

// Rows and columns of a large-M kernel tile.
inline int wide_rows(int variant) { return variant == 2 ? 256 : 128; }
inline int wide_cols(int variant) { return variant == 1 ? 128 : 256; }

struct W4A16Tile {
    W4A16Kind kind;
    int mt;  // 16-row MFMA subtiles per block (SKINNY: 1, 2, 4; WIDE: 8, 16)
    int ns;  // SKINNY: 16-column MFMA subtiles per block (1 to 4); WIDE: kernel variant
    int tw;  // SKINNY: columns per workgroup, 1 to 16*ns (the last subtile may be partly idle)
    int block_m() const { return 16 * mt; }
    int block_n() const { return kind == W4A16_WIDE ? wide_cols(ns) : tw; }
};

// Weight format: `bits`-wide unsigned codes (4 or 8) packed 32/bits per 32-bit word along K,
// lowest field first, and one bf16 scale and bias per `group` consecutive values of a row
// (32, 64 or 128). The kernels walk K in blocks of 128 values, so 128 % group == 0.
struct WFormat {
    int bits;
    int group;
    int sub() const { return 128 / group; }  // scale/bias groups per 128-value block
};

inline bool format_supported(WFormat f)
{
    return (f.bits == 4 || f.bits == 8) && (f.group == 32 || f.group == 64 || f.group == 128);
}

constexpr int kLdsPerCU = 160 * 1024;  // LDS bytes of one CU (and the most one workgroup may take)

// Wave count and groups per load round of the SKINNY kernel for partitions of at most gpp groups
// (128-value blocks). A wave stages a round's activations in LDS (256 bytes per staged row and
// group: 16 rows per 16-row tile, or only 4 or 8 with at most that many rows, see skinny_rows)
// and its scale/bias entries (two dword arrays of 16*ns rows x gpw*sub entries, each rounded
// up to 64); the workgroup's LDS is at most 160 KB.
struct SkinnyShape {
    int waves;  // waves per workgroup, each taking every waves-th group of the partition
    int gpw;    // groups whose loads one wave issues together
};

// Activation rows a wave stages per group. Decode (at most 8 rows, 4-bit codes, one 16-row
// tile of 16 or 48 columns) stages only 4 or 8 rows, and the MFMA's 16 operand rows read
// them cyclically (rows past M reach only output rows that are never stored): a quarter or
// half of the LDS per group, which leaves room for the waves' fp32 tiles beside the staging
// memory (A/B on MI355X, same waves and groups per round: down at M = 1 and 4, gate, up, q,
// k, v and o at M = 1..8 3-4.5 % faster, down at M = 8 unchanged). More groups per round
// in the freed LDS (4..8 on 16-column tiles, 3 on 48-column ones) were 2-7 % slower.
inline int skinny_rows(int mt, int ns, int bits, int M)
{
    if (bits == 4 && mt == 1 && ns == 1 && M <= 8) return M <= 4 ? 4 : 8;
    if (bits == 4 && mt == 1 && ns == 3 && M <= 8) return 8;  // 5..8 rows: up to 4 take 16-column tiles
    return 16 * mt;
}

inline size_t skinny_stage_bytes(int mt, int ns, int waves, int gpw, int sub, int rows)
{
    (void)mt;
    const size_t ew = (size_t)16 * ns * gpw * sub;
    return (size_t)waves * gpw * rows * 256 + (size_t)waves * 2 * ((ew + 63) & ~(size_t)63) * 4;
}
inline size_t skinny_sum_bytes(int mt, int ns, int waves) { return (size_t)waves * mt * ns * 1024; }
// The least LDS a configuration needs: the waves' fp32 tiles reuse the staging memory once
// every wave has left it. (When staging and tiles fit side by side, the kernel keeps them
// apart instead, so that a wave can store its tile without waiting for the others.)
inline size_t skinny_lds_bytes(int mt, int ns, int waves, int gpw, int sub, int rows)
{
    const size_t stage = skinny_stage_bytes(mt, ns, waves, gpw, sub, rows);
    const size_t sums = skinny_sum_bytes(mt, ns, waves);
    return stage > sums ? stage : sums;
}

inline SkinnyShape skinny_shape(int mt, int ns, int gpp, int bits, int sub, int rows)
{
    // 16-column tiles: up to 12 waves; 32-column tiles of one 16-row block: 16; else 8.
    // Groups per round: up to 3, 2 for 48- and 64-column tiles of 16 or 32 rows, 1 for them
    // with 64 rows (config sweeps of the Qwen3-4B projections at M = 16..64 on MI355X; the
    // same limits with decode's fewer staged rows, see skinny_rows).
    const int max_waves = ns == 1 ? 12 : (mt == 1 && ns == 2) ? 16 : 8;
    int max_gpw = ns >= 3 ? (mt == 4 ? 1 : 2) : (mt == 4 ? 2 : 3);
    if (bits == 8 && max_gpw > 1) max_gpw -= 1;  // twice the weight registers per group
    SkinnyShape sh;
    sh.waves = gpp < max_waves ? gpp : max_waves;
    const int per_wave = (gpp + sh.waves - 1) / sh.waves;
    sh.gpw = per_wave < max_gpw ? per_wave : max_gpw;
    while (skinny_lds_bytes(mt, ns, sh.waves, sh.gpw, sub, rows) > (size_t)kLdsPerCU) {
        if (sh.gpw > 1) --sh.gpw;
        else --sh.waves;
    }
    return sh;
}

// Dense bf16 kernel tile: 32*mt rows by 32*ns columns (the kernel has 128 x 128 only).
struct DenseTile {
    int mt;
    int ns;
    int block_m() const { return 2 * 16 * mt; }
    int block_n() const { return 2 * 16 * ns; }
};

// out: C (bf16) when s = 1, else the partial planes [s][M][N], bf16 or (f32_part) fp32.
// Workgroup (x, y, z) computes columns [x*tw, x*tw + tw) of rows [16*mt*y, 16*mt*(y+1)).
hipError_t launch_w4a16_skinny(WFormat fmt, int mt, int ns, int tw, int gpw, int waves, const void *A,
                               const void *Wq, const void *scale, const void *bias, void *out, bool f32_part, int M,
                               int N, int K, int s, bool vec_store, hipStream_t stream);

// Large-M kernel variants: 0 = 128 x 256 tiles of 4 waves of 128 x 64; 1 = 128 x 128
// tiles of 4 waves of 128 x 32; 2 = 256 x 256 tiles of 8 waves of 256 x 32. LDS bytes of
// one workgroup (three stage slots of A, 64 values per row, and of W, 64 codes per
// column, and two scale/bias slots of one 128-value block); workgroups one CU holds
// (160 KB of LDS).
constexpr int kWideCols = 256;  // columns of the stream-K variants (0 and 2)
constexpr int wide_lds_bytes(int rows, int bits, int sub, int cols = kWideCols)
{
    return 3 * rows * 64 * 2 + 3 * cols * 64 * bits / 8 + 2 * 2 * cols * 4 * sub;
}
inline int wide_wgs_per_cu(int variant, WFormat f = WFormat{4, 128})
{
    return variant != 2 && 2 * wide_lds_bytes(128, f.bits, f.sub(), wide_cols(variant)) <= kLdsPerCU ? 2 : 1;
}

// Large-M kernel: the first full_tiles tiles (M-block fastest) unsplit into C, the
// remaining ones in `split` near-equal group partitions into the planes of `part`
// ([split][M][N], bf16 or (f32_part) fp32; unused when split = 1).
// streamk = P > 0 instead runs the stream-K decomposition on P workgroups (near-equal
// ranges of the (tile, 128-value block) units; full_tiles and split are ignored), with
// `part` holding 2P tile slots (wide_streamk_bytes) and a fix-up launch after it;
// variants 0 and 2 only.
hipError_t launch_w4a16_wide(WFormat fmt, int variant, const void *A, const void *Wq, const void *scale,
                             const void *bias, void *C, void *part, bool f32_part, int M, int N, int K,
                             int full_tiles, int split, bool vec_store, hipStream_t stream, int streamk = 0);

// Order of the large-M kernel's work items over the XCDs. The grid has one or two regions:
// the whole tiles (one partition), then the split ones (split partitions); a region holds
// wr = P * nb * num_m items, P partitions of nb column blocks of num_m row blocks. The
// dispatcher deals workgroups round-robin over the 8 XCDs, so the workgroups r, r + 8,
// r + 16, ... of a region share an L2; they get one contiguous run of items, read in
// panels of pm row blocks:
//   L = k*(wr/8) + min(k, wr%8) + j  for workgroup r = 8j + k of the region (a bijection
//       onto 0 .. wr-1: run k holds wr/8 items, one more for k < wr%8),
//   p = L / (nb*num_m); within the partition, panel = l / (pm*nb) covers row blocks
//   panel*pm .. panel*pm + pm-1, and l % (pm*nb) walks them row block fastest, then the
//   column blocks.
// So one XCD's workgroups read a few row blocks of A against a few column blocks of W
// (about pm x (wr/8)/pm tiles) instead of one row block of A against every column block.
// pm divides num_m. Each workgroup still computes one whole tile over one partition.
struct WideItem {
    int p, n, m;  // partition, column block, row block
};
constexpr WideItem wide_item(int r, int wr, int num_m, int nb, int pm)
{
    const int k = r & 7, j = r >> 3;
    const int q = wr >> 3, rem = wr & 7;
    const int L = k * q + (k < rem ? k : rem) + j;
    const int per_p = nb * num_m;
    const int p = L / per_p;
    const int l = L - p * per_p;
    const int panel = l / (pm * nb);
    const int w = l - panel * pm * nb;
    return WideItem{p, w / pm, panel * pm + w % pm};
}

// The panel height for a region (0: the plain order, workgroup r taking item r, row block
// fastest): the divisor of num_m whose XCD runs read the fewest bytes, A's row blocks at
// a_mp bytes each and W's column blocks (with their scale/bias) at w_np bytes each, per
// partition. A run of c = ceil(wr/8) items covers min(pm, c) row blocks by ceil(c/pm)
// column blocks while it fits one panel, else whole panels; the plain order gives an XCD
// every eighth item: num_m/8 row blocks by all nb column blocks of every partition when 8
// divides num_m, one row block by nb*num_m/8 column blocks when num_m divides 8.
inline int wide_panel(int P, int nb, int num_m, double a_mp, double w_np)
{
    if (P < 1 || nb < 1 || num_m < 1) return 0;
    const long long wr = (long long)P * nb * num_m;
    const long long c = (wr + 7) / 8;
    double plain;
    if (num_m % 8 == 0)
        plain = P * (num_m / 8 * a_mp + nb * w_np);
    else if (8 % num_m == 0)
        plain = P * (a_mp + ((nb * num_m + 7) / 8) * w_np);
    else
        plain = P * (num_m * a_mp + nb * w_np);
    int best = 0;
    double best_cost = plain;
    for (int pm = 1; pm <= num_m; ++pm) {
        if (num_m % pm) continue;
        double cost;
        if (c <= (long long)pm * nb)
            cost = (double)(c < pm ? c : pm) * a_mp + (double)((c + pm - 1) / pm) * w_np;
        else if (c <= (long long)nb * num_m)
            cost = (double)((c + nb - 1) / nb) * a_mp + nb * w_np;
        else
            cost = (double)((c + nb * num_m - 1) / (nb * num_m)) * (num_m * a_mp + nb * w_np);
        if (cost < best_cost * 0.98) {  // a clear gain over the best so far, else keep it
            best_cost = cost;
            best = pm;
        }
    }
    return best;
}

inline size_t wide_streamk_bytes(int variant, int P, bool f32_part)
{
    return (size_t)2 * (size_t)P * (size_t)wide_rows(variant) * (size_t)kWideCols * (f32_part ? 4 : 2);
}

// Decode matrix-vector kernel (M <= 8): a partition of kp reduction values fits its A
// staging when kp <= 10240 (at most 5 chunks of 32 per lane) and m8 * kp <= 30720
// (m8 = M rounded up to 1, 2, 4 or 8; LDS), and for m8 = 8 kp <= 4096 as well.
inline bool gemv_split_fits(int m8, int kp) { return kp <= 10240 && m8 * kp <= 30720 && (m8 < 8 || kp <= 4096); }

hipError_t launch_w4a16_gemv(const void *A, const void *Wq, const void *scale, const void *bias, void *out, int M,
                             int N, int K, int s, hipStream_t stream);

hipError_t launch_reduce(const void *partials, bool f32_partials, int s, size_t MN, void *C,
                         bool vec, hipStream_t stream);

// The same merge restricted to columns [n_lo, N) of planes [s][M][N] (bf16 or fp32).
hipError_t launch_reduce_cols(const void *partials, bool f32_partials, int s, int M, int N, int n_lo, void *C,
                              bool vec, hipStream_t stream);

// Split-KV decode attention (head dimension 128, G*Mq <= 16 query rows per key/value
// head): S splits of every request's keys; S > 1 needs the workspace (fp32
// accumulators [S][B*Mq*Hq][128], then max and sum [S][B*Mq*Hq][2]) and runs the merge.
hipError_t launch_attn_decode(const void *Q, const void *K, const void *V, const int *lengths, void *O,
                              void *workspace, int B, int Mq, int Hq, int Hkv, int Lmax, float scale, int S,
                              hipStream_t stream);

hipError_t launch_dense(DenseTile tile, const void *A, const void *B, void *out, bool f32_out,
                        int M, int N, int K, int s, bool vec_store, hipStream_t stream);

}  // namespace qmm_impl
