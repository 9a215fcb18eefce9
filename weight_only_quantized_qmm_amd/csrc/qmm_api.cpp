// qmm_api.cpp -- the C ABI declared in include/qmm.h: argument checks, the split
// policy, and the dispatch of the gfx950 kernels.
//
// tiny-llm "Week 2 Day 7: Split-K Prefill", Task 3 and Task 4: the dispatcher
// picks the partition count from occupancy, dispatches the partition kernel and
// then the reduction, and uses the unsplit kernel unchanged when the count is 1.
// Every check below runs on the host before any launch, so an error return has
// no device side effect.
#include "qmm.h"

#include <limits.h>
#include <stdint.h>

#include "qmm_launch.h"

using qmm_impl::DenseTile;
using qmm_impl::W4A16Tile;
using qmm_impl::WFormat;

extern "C" {
const qmm_policy QMM_POLICY_PAGE = {32, 32, 320, 16, 128};
// Tile 0 x 0 = the output tile of the kernel that runs the shape; 256 target blocks = the CU
// count (times two for the large-M kernel, which holds two workgroups per CU); cap and minimum
// K per partition fitted to per-shape split sweeps on MI355X (split never slower than unsplit;
// a cap of 20 rather than 16 lets down at M = 96..128 take 19 even partitions of four groups,
// 5 % faster than 16 uneven ones).
const qmm_policy QMM_POLICY_MI355X = {0, 0, 256, 20, 512};
}

namespace {

constexpr int kGroup = 128;
constexpr int kGranule = 32;
constexpr int kCUs = 256;  // MI355X compute units
constexpr int kSkinnyMinK = 2048;  // shortest partition of the small-M kernel up to 32 rows (preset)

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

long long ceil_div(long long a, long long b) { return (a + b - 1) / b; }

// The large-M kernel's decomposition under a kernel-tile policy: (s, full_tiles).
struct Decomp {
    int s;
    int full_tiles;
};

Decomp wide_rule(long long T, long long num_m, int G, int K, long long target, const qmm_policy &pol) {
    long long smax = pol.cap;
    if (G < smax) smax = G;
    const long long by_k = K / pol.min_k_per_split;
    if (by_k < smax) smax = by_k;
    Decomp d = {1, (int)T};
    if (smax <= 1 || target <= 0) return d;
    if (T >= target) {
        long long full = (T / target) * target;
        full -= full % num_m;
        const long long tail = T - full;
        if (tail == 0) return d;
        long long s = target / tail;
        if (smax < s) s = smax;
        if (s <= 1) return d;
        d.s = (int)s;
        d.full_tiles = (int)full;
        return d;
    }
    long long s = target / T;
    if (smax < s) s = smax;
    if (s <= 1) return d;
    d.s = (int)s;
    d.full_tiles = 0;
    return d;
}

// Critical path of a large-M decomposition of T tiles of rows x cols (one workgroup per
// CU, the unsplit rounds first, then the split tail) in units of one 128-row x 256-column x
// 128-value block, plus half a unit per partition of a split for its planes and reduce.
double wide_cost(long long T, int rows, int cols, const Decomp &d, int G)
{
    const double blk = rows / 128.0 * cols / 256.0;
    const long long full = d.full_tiles, tail = T - full;
    double t = (double)ceil_div(full, kCUs) * G * blk;
    if (tail > 0 && d.s > 1) t += (double)ceil_div(tail * d.s, kCUs) * ceil_div(G, d.s) * blk + 0.5 * d.s;
    return t;
}

// Large-M variant: each candidate under the preset's split rule over its own tiles, the
// smallest critical path winning:
//   variant 0, 128 x 256 tiles (two workgroups per CU up to M = 128, one above);
//   variant 2, 256 x 256 tiles, above M = 128;
//   variant 1, 128 x 128 tiles, only while they are fewer than the CUs (a pure split, one
//   workgroup per CU): it halves the split of shapes whose 256-column tiles must split
//   deeply. Ties go to the larger tiles (2, then 0, then 1).
// On the Qwen3-4B shapes this takes 128 x 256 tiles for q at M = 2048 (256 tiles, no split),
// 128 x 128 tiles for k and v at M = 2048 (128 tiles in two partitions instead of 64 in
// four) and for gate, up and down at M = 128 (three and twelve partitions instead of five
// and nineteen), and 256 x 256 tiles for o, gate, up and down at M = 2048. Split sweeps on
// MI355X: k, v 8 %, gate, up 13 %, down 9 % faster than on 128 x 256 tiles.
int wide_variant(int M, int N, int K)
{
    const qmm_policy &pol = QMM_POLICY_MI355X;
    const int G = K / kGroup;
    int best = -1;
    double best_cost = 0;
    for (int v : {2, 0, 1}) {
        if (v == 2 && M <= 128) continue;
        const int rows = qmm_impl::wide_rows(v), cols = qmm_impl::wide_cols(v);
        const long long num_m = ceil_div(M, rows), T = num_m * ceil_div(N, cols);
        if (v == 1 && T >= kCUs) continue;
        const long long slots = (long long)pol.target_blocks * (v == 0 && M <= 128 ? qmm_impl::wide_wgs_per_cu(0) : 1);
        const double c = wide_cost(T, rows, cols, wide_rule(T, num_m, G, K, slots, pol), G);
        if (best < 0 || c < best_cost) {
            best = v;
            best_cost = c;
        }
    }
    return best;
}

// An unsplit grid of 16-column small-M tiles with fewer tiles than CUs leaves CUs idle, and
// a workgroup's time grows with the weight bytes it streams: narrow the tiles to
// ceil(N / tiles-per-row-block) columns so that the grid covers every CU once (the MFMA
// subtile keeps 16 columns, the ones past the tile idle). Each workgroup still reads all of
// A, so this pays where the weights are a large share of its bytes (A/B on MI355X: down at
// M = 4 and 8 6-8 % faster, k and v at M = 32 3 %, o at M = 32 2 %; 48-column tiles of gate
// and up narrowed to 38 or 40 columns were unchanged, so wider tiles are left as they are).
W4A16Tile narrow_skinny(W4A16Tile t, int M, int N, int s)
{
    t.tw = 16 * t.ns;
    if (s != 1 || t.ns != 1) return t;
    const long long per_row = kCUs / ceil_div(M, t.block_m());  // column tiles one round holds
    if (per_row < 1 || ceil_div(N, t.tw) >= per_row) return t;
    const long long tw = ceil_div(N, per_row);
    if (tw < t.tw) t.tw = (int)tw;
    return t;
}

// Kernel and block tile for an (M, N, K) problem. The small-M kernel takes up to 64 rows
// in one block row, and 65..128 rows in 64-row blocks when the packed weights are at
// most 8 MB (N*K <= 2^24): there the large-M kernel has too few 256-column tiles and must
// split deeply, while reading the weights twice costs less (split sweeps of the Qwen3-4B
// q, k and v projections at M = 128 on MI355X: 25-45 % faster; gate, up and down stay on
// the large-M kernel). Otherwise the large-M kernel, in the tile variant wide_variant picks.
W4A16Tile w4a16_tile(int M, int N, int K, int s) {
    W4A16Tile t;
    t.tw = 0;
    if (M <= 64 || (M <= 128 && (long long)N * K <= (1LL << 24))) {
        t.kind = qmm_impl::W4A16_SKINNY;
        // Narrow projections up to 64 rows whose 16-row, 16-column tiles fit one round of
        // workgroups (k and v at M = 17..64): 16-row tiles, so that each workgroup reads 16
        // rows of A instead of all M, unsplit (no second pass). A/B on MI355X: k and v at
        // M = 24, 32, 48, 64 4.83, 5.10, 5.17, 5.07 us against 5.68, 6.07, 7.64, 7.96 on the
        // 32- or 64-row tiles (split at M = 48 and 64); with two rounds of such tiles (q and
        // o at M = 32, k at M = 128) 0-30 % slower, so only one round.
        if (M <= 64 && ceil_div(M, 16) * ceil_div(N, 16) <= kCUs && (long long)N * K <= (1LL << 24)) {
            t.mt = 1;
            t.ns = 1;
            return narrow_skinny(t, M, N, s);
        }
        // Likewise 16-row tiles of 64 columns when those fill at least three quarters of one
        // round (q at M = 48..64, N = 3072..4096): unsplit instead of 32- or 64-row tiles in
        // two partitions plus the merge. A/B on MI355X: q at M = 48, 56, 64 8.36, 8.22, 8.33 us
        // against 9.40, 9.73, 10.05, N = 3072 at M = 64 8.30 against 9.96. With 32 or 48
        // columns, or filling fewer CUs (o at M = 32 and 64, q at M = 24 and 32), 0-7 % slower.
        if (M <= 64 && (long long)N * K <= (1LL << 24) && ceil_div(M, 16) * ceil_div(N, 64) <= kCUs &&
            4 * ceil_div(M, 16) * ceil_div(N, 64) >= 3 * kCUs) {
            t.mt = 1;
            t.ns = 4;
            return narrow_skinny(t, M, N, s);
        }
        // Past 64 rows the same holds with 32-row tiles of 16 columns (k and v at M = 65..128):
        // unsplit, each workgroup reading 32 rows of A instead of 64 in split 64-row tiles.
        // A/B on MI355X: k and v at M = 80, 96, 128 6.13, 6.25, 6.10 us against 8.28, 8.31,
        // 8.43 (4 partitions plus the merge).
        if (M > 64 && ceil_div(M, 32) * ceil_div(N, 16) <= kCUs && (long long)N * K <= (1LL << 24)) {
            t.mt = 2;
            t.ns = 1;
            return narrow_skinny(t, M, N, s);
        }
        t.mt = M <= 16 ? 1 : M <= 32 ? 2 : 4;
        // Up to 32 rows over at most 2^24 weights: 16-column tiles, so that the unsplit grid
        // has N/16 workgroups of up to 12 waves (config sweeps of q, k, v and o on MI355X:
        // at M = 16 20-30 % faster than split 32-column tiles, whose second pass costs more
        // than the spread saves; at M = 32 11-15 % faster than 32-column tiles). Decode (up
        // to 8 rows) also over more weights while those tiles fit one round of workgroups
        // (N <= 4096): the long reduction then runs unsplit instead of in split 48-column
        // tiles plus a second pass (down at M = 1, 4, 8 on MI355X: 8.6, 9.2, 10.2 us against
        // 10.3, 10.6, 10.9). Up to 4 rows at any N: their staging (4 rows per group) is small
        // enough for two or three workgroups per CU (gate at M = 1 and 4 on 608 16-column
        // tiles: 6.67 and 6.65 us against 6.90 and 7.01 on 203 48-column tiles; at M = 8,
        // with 8 staged rows, 7.95 against 7.18).
        if (M <= 32 && ((long long)N * K <= (1LL << 24) || (M <= 8 && N <= 16 * kCUs) || M <= 4)) {
            t.ns = 1;
            return narrow_skinny(t, M, N, s);
        }
        // 32-column tiles while they fit one workgroup per CU (one workgroup of the
        // small-M kernel fills a CU's wave slots) over a reduction shorter than 8192;
        // otherwise the widest tile that still spreads over the most CUs: 48 columns when
        // those tiles fit one per CU, else 64. Wider tiles feed each staged activation group
        // to more columns (config sweeps of the Qwen3-4B projections on MI355X: gate and up
        // at M = 16..64 on 203 48-column tiles 10-12 % faster than on 152 64-column ones;
        // down (K = 9728) 11-16 % faster on 48 columns in 4 partitions than on 32 or 64).
        const long long rows = ceil_div(M, 16 * t.mt);
        if (rows * ceil_div(N, 32) <= kCUs && K < 8192)
            t.ns = 2;
        else
            t.ns = rows * ceil_div(N, 48) <= kCUs ? 3 : 4;
        return narrow_skinny(t, M, N, s);
    } else {
        t.kind = qmm_impl::W4A16_WIDE;
        t.ns = wide_variant(M, N, K);
        t.mt = qmm_impl::wide_rows(t.ns) / 16;
    }
    return t;
}

// The large-M kernel's tile for M > 64, whichever kernel the plan picks (stream-K runs it).
W4A16Tile wide_tile(int M) {
    W4A16Tile t;
    t.tw = 0;
    t.kind = qmm_impl::W4A16_WIDE;
    t.mt = M <= 128 ? 8 : 16;
    t.ns = M <= 128 ? 0 : 2;
    return t;
}

hipError_t dispatch_skinny(WFormat fmt, const W4A16Tile &tile, const void *A, const void *Wq, const void *scale,
                           const void *bias, void *out, bool f32_part, int M, int N, int K, int s, bool vec,
                           hipStream_t st) {
    // the longest partition: ceil(G / s) blocks (near-equal partitions differ by at most one)
    const int G = K / kGroup;
    const int rows = qmm_impl::skinny_rows(tile.mt, tile.ns, fmt.bits, M);
    const qmm_impl::SkinnyShape sh =
        qmm_impl::skinny_shape(tile.mt, tile.ns, (G + s - 1) / s, fmt.bits, fmt.sub(), rows);
    return qmm_impl::launch_w4a16_skinny(fmt, tile.mt, tile.ns, tile.tw, sh.gpw, sh.waves, A, Wq, scale, bias, out,
                                         f32_part, M, N, K, s, vec, st);
}

DenseTile dense_tile(int /*M*/, int /*N*/) {
    DenseTile t;
    t.mt = 4;
    t.ns = 4;
    return t;
}

// Sizes the kernels index with 32-bit row/column counters and 64-bit offsets; the
// reduction length also bounds the large-M kernel's 32-bit per-lane copy offsets
// (256 rows of A: 512*K bytes < 2^31).
bool sizes_ok(int M, int N, int K) {
    if ((long long)M * (long long)N > (long long)INT_MAX * 64) return false;
    if ((long long)N * (long long)K > (long long)INT_MAX * 64) return false;
    if ((long long)M * (long long)K > (long long)INT_MAX * 64) return false;
    if (K >= (1 << 22)) return false;
    return true;
}

// The page's rule (Task 3); with divisor = false the last step, which lowers s to a divisor
// of G so that the partitions are equal (Task 2), is left out and the partitions are the
// near-equal floor(p*G/s) ranges.
int split_rule(long long base, int G, int K, const qmm_policy &pol, bool divisor = true) {
    long long s = pol.cap;
    const long long by_target = pol.target_blocks / base;
    if (by_target < s) s = by_target;
    const long long by_k = K / pol.min_k_per_split;
    if (by_k < s) s = by_k;
    if (G < s) s = G;
    while (divisor && s > 1 && G % s != 0) --s;
    return s < 1 ? 1 : (int)s;
}

bool policy_ok(const qmm_policy &p) {
    return p.tile_m >= 0 && p.tile_n >= 0 && p.target_blocks >= 0 && p.cap >= 1 && p.min_k_per_split >= 1;
}

int hip_status(hipError_t e) { return e == hipSuccess ? QMM_OK : QMM_ERR_HIP; }

}  // namespace

namespace {

// The plan of an (M, N, K) product in weight format fmt (the split rule is the same for
// every format; the large-M kernel's workgroups per CU depend on the format's LDS).
int plan_format(WFormat fmt, int M, int N, int K, const qmm_policy *policy, qmm_plan *out)
{
    if (!out || M <= 0 || N <= 0 || K <= 0 || !qmm_impl::format_supported(fmt)) return QMM_ERR_ARG;
    if (K % kGroup != 0) return QMM_ERR_SHAPE;
    if (!sizes_ok(M, N, K)) return QMM_ERR_SIZE;
    const qmm_policy pol = policy ? *policy : QMM_POLICY_MI355X;
    if (!policy_ok(pol)) return QMM_ERR_ARG;
    // the split rule counts the kernel's full-width tiles; an unsplit plan then narrows them
    const W4A16Tile tile = w4a16_tile(M, N, K, 0);
    const int tm = pol.tile_m > 0 ? pol.tile_m : tile.block_m();
    const int tn = pol.tile_n > 0 ? pol.tile_n : tile.block_n();
    const long long base = ceil_div(M, tm) * ceil_div(N, tn);
    const int G = K / kGroup;
    const long long kernel_tiles = ceil_div(M, tile.block_m()) * ceil_div(N, tile.block_n());
    Decomp d;
    if (tile.kind == qmm_impl::W4A16_WIDE && pol.tile_m == 0 && pol.tile_n == 0) {
        // slots: target_blocks times the workgroups of this kernel one CU holds; 128 x 256
        // tiles above M = 128 and 128 x 128 tiles count one per CU, as the variant choice does
        const long long slots =
            (long long)pol.target_blocks * (M > 128 || tile.ns == 1 ? 1 : qmm_impl::wide_wgs_per_cu(tile.ns, fmt));
        d = wide_rule(kernel_tiles, ceil_div(M, tile.block_m()), G, K, slots, pol);
    } else {
        qmm_policy p = pol;
        const bool own_tile = tile.kind == qmm_impl::W4A16_SKINNY && pol.tile_m == 0 && pol.tile_n == 0;
        // The small-M kernel under the preset's own tiles, up to 32 rows: a partition shorter
        // than kSkinnyMinK reduction values saves less than the second pass costs (a launch
        // and a round trip through HBM, about 3 us on MI355X).
        if (own_tile && M <= 32 && p.min_k_per_split < kSkinnyMinK) p.min_k_per_split = kSkinnyMinK;
        // Under its own tiles the small-M kernel takes near-equal partitions, as the large-M
        // plan does: o at M = 64 (80 tiles, G = 32) in 3 partitions instead of 2 (the largest
        // divisor) fills 240 CUs instead of 160, 12.1 -> 10.7 us on MI355X.
        d.s = split_rule(base, G, K, p, !own_tile);
        d.full_tiles = 0;
    }
    const int s = d.s;
    const W4A16Tile run = w4a16_tile(M, N, K, s);
    if (s == 1) d.full_tiles = (int)(ceil_div(M, run.block_m()) * ceil_div(N, run.block_n()));
    out->s = s;
    out->base_tiles = base > INT_MAX ? INT_MAX : (int)base;
    out->tile_m = tm;
    out->tile_n = tn;
    out->full_tiles = d.full_tiles;
    if (tile.kind == qmm_impl::W4A16_WIDE) {  // one-dimensional grid: full tiles, then (tile, partition)
        out->grid_x = (int)(d.full_tiles + (kernel_tiles - d.full_tiles) * s);
        out->grid_y = 1;
        out->grid_z = 1;
    } else {
        out->grid_x = (int)ceil_div(N, run.block_n());
        out->grid_y = (int)ceil_div(M, run.block_m());
        out->grid_z = s;
    }
    out->block_m = run.block_m();
    out->block_n = run.block_n();
    out->workspace_bytes = s > 1 ? (size_t)2 * (size_t)s * (size_t)M * (size_t)N : 0;
    return QMM_OK;
}

}  // namespace

extern "C" int qmm_splitk_plan(int M, int N, int K, int group_size, const qmm_policy *policy,
                               qmm_plan *out)
{
    if (group_size != kGroup) return QMM_ERR_ARG;
    return plan_format(WFormat{4, kGroup}, M, N, K, policy, out);
}

extern "C" int qmm_wna16_plan(int bits, int group_size, int M, int N, int K, const qmm_policy *policy,
                              qmm_plan *out)
{
    return plan_format(WFormat{bits, group_size}, M, N, K, policy, out);
}

namespace {

// The weight-only matmul in format fmt with partial planes of element size 2 (bf16) or
// 4 (fp32, f32_part). With pass1 != nullptr only the matmul launch runs; pass1[0] receives
// the effective split and pass1[1] the first column whose outputs are left in the planes.
int wq_run(WFormat fmt, const void *A, const void *Wq, const void *scale, const void *bias, void *C, int M, int N,
           int K, int s, void *workspace, size_t workspace_bytes, bool f32_part, void *stream,
           int *pass1 = nullptr)
{
    if (!A || !Wq || !scale || !bias || !C || !qmm_impl::format_supported(fmt)) return QMM_ERR_ARG;
    if (M <= 0 || N <= 0 || K <= 0 || s < 0) return QMM_ERR_ARG;
    if (K % kGroup != 0) return QMM_ERR_SHAPE;
    if (!sizes_ok(M, N, K)) return QMM_ERR_SIZE;
    if (!aligned(A, 16) || !aligned(Wq, 16) || !aligned(scale, 2) || !aligned(bias, 2) || !aligned(C, 2))
        return QMM_ERR_ALIGN;
    const int G = K / kGroup;
    int full_tiles = 0;
    if (s == 0) {
        qmm_plan plan;
        const int rc = plan_format(fmt, M, N, K, nullptr, &plan);
        if (rc != QMM_OK) return rc;
        s = plan.s;
        full_tiles = plan.full_tiles;
    } else if (s > G) {
        return QMM_ERR_SHAPE;
    }
    const W4A16Tile tile = w4a16_tile(M, N, K, s);
    const size_t MN = (size_t)M * (size_t)N;
    const size_t esz = f32_part ? 4 : 2;
    if (s > 1) {
        if (!workspace || workspace_bytes < esz * (size_t)s * MN) return QMM_ERR_WORKSPACE;
        if (!aligned(workspace, 16)) return QMM_ERR_ALIGN;
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    const bool vec_c = (N % 4 == 0) && aligned(C, 8);
    if (tile.kind == qmm_impl::W4A16_WIDE) {
        const int num_m = (int)ceil_div(M, tile.block_m());
        const int tiles = num_m * (int)ceil_div(N, tile.block_n());
        if (s == 1) full_tiles = tiles;
        // Partial planes and C share one store-width decision (N % 4 == 0 and 8-byte C).
        int rc = hip_status(qmm_impl::launch_w4a16_wide(fmt, tile.ns, A, Wq, scale, bias, C,
                                                        s > 1 ? workspace : nullptr, f32_part, M, N, K, full_tiles,
                                                        s, vec_c, st));
        const int n_lo = s == 1 ? N : (full_tiles / num_m) * tile.block_n();
        if (pass1) {
            pass1[0] = s;
            pass1[1] = n_lo;
        }
        if (rc != QMM_OK || s == 1 || pass1) return rc;
        if (full_tiles == 0) {
            const bool vec_red = (MN % 8 == 0) && aligned(C, 16);
            return hip_status(qmm_impl::launch_reduce(workspace, f32_part, s, MN, C, vec_red, st));
        }
        const bool vec_red = (N % 8 == 0) && aligned(C, 16);
        return hip_status(qmm_impl::launch_reduce_cols(workspace, f32_part, s, M, N, n_lo, C, vec_red, st));
    }
    if (pass1) {
        pass1[0] = s;
        pass1[1] = s == 1 ? N : 0;
    }
    if (s == 1) return hip_status(dispatch_skinny(fmt, tile, A, Wq, scale, bias, C, false, M, N, K, 1, vec_c, st));
    const bool vec_ws = (N % 4 == 0);
    int rc = hip_status(dispatch_skinny(fmt, tile, A, Wq, scale, bias, workspace, f32_part, M, N, K, s, vec_ws, st));
    if (rc != QMM_OK || pass1) return rc;
    const bool vec_red = (MN % 8 == 0) && aligned(C, 16);
    return hip_status(qmm_impl::launch_reduce(workspace, f32_part, s, MN, C, vec_red, st));
}

}  // namespace

extern "C" int qmm_w4a16_g128(const void *A, const void *Wq, const void *scale, const void *bias,
                              void *C, int M, int N, int K, int s, void *workspace,
                              size_t workspace_bytes, void *stream)
{
    return wq_run(WFormat{4, kGroup}, A, Wq, scale, bias, C, M, N, K, s, workspace, workspace_bytes, false, stream);
}

extern "C" int qmm_w4a16_g128_pass1(const void *A, const void *Wq, const void *scale, const void *bias, void *C,
                                    int M, int N, int K, int s, void *workspace, size_t workspace_bytes, int *s_out,
                                    int *n_lo_out, void *stream)
{
    if (!s_out || !n_lo_out) return QMM_ERR_ARG;
    int out[2] = {0, 0};
    const int rc = wq_run(WFormat{4, kGroup}, A, Wq, scale, bias, C, M, N, K, s, workspace, workspace_bytes, false,
                          stream, out);
    if (rc == QMM_OK) {
        *s_out = out[0];
        *n_lo_out = out[1];
    }
    return rc;
}

extern "C" int qmm_w4a16_g128_f32p(const void *A, const void *Wq, const void *scale, const void *bias,
                                   void *C, int M, int N, int K, int s, void *workspace,
                                   size_t workspace_bytes, void *stream)
{
    return wq_run(WFormat{4, kGroup}, A, Wq, scale, bias, C, M, N, K, s, workspace, workspace_bytes, true, stream);
}

extern "C" int qmm_wna16(int bits, int group_size, int partial_dtype, const void *A, const void *Wq,
                         const void *scale, const void *bias, void *C, int M, int N, int K, int s, void *workspace,
                         size_t workspace_bytes, void *stream)
{
    if (partial_dtype != QMM_PARTIAL_BF16 && partial_dtype != QMM_PARTIAL_F32) return QMM_ERR_ARG;
    return wq_run(WFormat{bits, group_size}, A, Wq, scale, bias, C, M, N, K, s, workspace, workspace_bytes,
                  partial_dtype == QMM_PARTIAL_F32, stream);
}

namespace {

// Workgroups of the stream-K decomposition for workgroups = 0: one per workgroup slot,
// and no more than leave each at least min_k_per_split reduction values (the MI355X
// preset's floor on a partition) of units.
long long streamk_default_wgs(WFormat fmt, int variant, long long units, int K)
{
    long long P = (long long)kCUs * qmm_impl::wide_wgs_per_cu(variant, fmt);
    const long long min_units = QMM_POLICY_MI355X.min_k_per_split / kGroup;  // 4 blocks
    const long long G = K / kGroup;
    const long long cap = units / (min_units < G ? min_units : G);
    if (cap < P) P = cap;
    return P < 1 ? 1 : P;
}

}  // namespace

extern "C" size_t qmm_streamk_workspace_bytes(int M, int N, int K, int workgroups)
{
    if (M <= 64 || N <= 0 || K <= 0 || K % kGroup != 0 || workgroups < 0) return 0;
    const W4A16Tile tile = wide_tile(M);
    const long long units = ceil_div(M, tile.block_m()) * ceil_div(N, tile.block_n()) * (long long)(K / kGroup);
    long long P = workgroups ? workgroups : streamk_default_wgs(WFormat{4, kGroup}, tile.ns, units, K);
    if (P > units) P = units;
    return qmm_impl::wide_streamk_bytes(tile.ns, (int)P, false);
}

extern "C" int qmm_w4a16_g128_streamk(const void *A, const void *Wq, const void *scale, const void *bias, void *C,
                                      int M, int N, int K, int workgroups, void *workspace, size_t workspace_bytes,
                                      void *stream)
{
    if (!A || !Wq || !scale || !bias || !C) return QMM_ERR_ARG;
    if (M <= 0 || N <= 0 || K <= 0 || workgroups < 0) return QMM_ERR_ARG;
    if (K % kGroup != 0 || M <= 64) return QMM_ERR_SHAPE;
    if (!sizes_ok(M, N, K)) return QMM_ERR_SIZE;
    if (!aligned(A, 16) || !aligned(Wq, 16) || !aligned(scale, 2) || !aligned(bias, 2) || !aligned(C, 2))
        return QMM_ERR_ALIGN;
    const WFormat fmt{4, kGroup};
    const W4A16Tile tile = wide_tile(M);
    const long long units = ceil_div(M, tile.block_m()) * ceil_div(N, tile.block_n()) * (long long)(K / kGroup);
    long long P = workgroups ? workgroups : streamk_default_wgs(fmt, tile.ns, units, K);
    if (workgroups && P > units) return QMM_ERR_SHAPE;
    if (P > units) P = units;
    if (P > INT_MAX / 2) return QMM_ERR_SIZE;
    if (!workspace || workspace_bytes < qmm_impl::wide_streamk_bytes(tile.ns, (int)P, false)) return QMM_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return QMM_ERR_ALIGN;
    const bool vec_c = (N % 4 == 0) && aligned(C, 8);
    return hip_status(qmm_impl::launch_w4a16_wide(fmt, tile.ns, A, Wq, scale, bias, C, workspace, false, M, N, K, 0,
                                                  1, vec_c, static_cast<hipStream_t>(stream), (int)P));
}

namespace {
int gemv_m8(int M) { return M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : 8; }
}  // namespace

extern "C" int qmm_gemv_min_split(int M, int K)
{
    if (M < 1 || K <= 0) return QMM_ERR_ARG;
    if (M > 8) return QMM_ERR_SHAPE;
    if (K % kGroup != 0) return QMM_ERR_SHAPE;
    if (!sizes_ok(1, 1, K)) return QMM_ERR_SIZE;
    const int G = K / kGroup;
    for (int s = 1; s <= G; ++s)
        if (G % s == 0 && qmm_impl::gemv_split_fits(gemv_m8(M), K / s)) return s;
    return QMM_ERR_SHAPE;
}

extern "C" int qmm_w4a16_gemv(const void *A, const void *Wq, const void *scale, const void *bias, void *C, int M,
                              int N, int K, int s, void *workspace, size_t workspace_bytes, void *stream)
{
    if (!A || !Wq || !scale || !bias || !C) return QMM_ERR_ARG;
    if (M <= 0 || N <= 0 || K <= 0 || s < 0) return QMM_ERR_ARG;
    if (M > 8 || K % kGroup != 0) return QMM_ERR_SHAPE;
    if (!sizes_ok(M, N, K)) return QMM_ERR_SIZE;
    if (!aligned(A, 16) || !aligned(Wq, 16) || !aligned(scale, 2) || !aligned(bias, 2) || !aligned(C, 2))
        return QMM_ERR_ALIGN;
    const int G = K / kGroup;
    if (s == 0) {
        s = qmm_gemv_min_split(M, K);
        if (s < 0) return s;
    } else if (s > G || G % s != 0 || !qmm_impl::gemv_split_fits(gemv_m8(M), K / s)) {
        return QMM_ERR_SHAPE;
    }
    const size_t MN = (size_t)M * (size_t)N;
    if (s > 1) {
        if (!workspace || workspace_bytes < 2 * (size_t)s * MN) return QMM_ERR_WORKSPACE;
        if (!aligned(workspace, 16)) return QMM_ERR_ALIGN;
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (s == 1) return hip_status(qmm_impl::launch_w4a16_gemv(A, Wq, scale, bias, C, M, N, K, 1, st));
    int rc = hip_status(qmm_impl::launch_w4a16_gemv(A, Wq, scale, bias, workspace, M, N, K, s, st));
    if (rc != QMM_OK) return rc;
    const bool vec_red = (MN % 8 == 0) && aligned(C, 16);
    return hip_status(qmm_impl::launch_reduce(workspace, false, s, MN, C, vec_red, st));
}

extern "C" int qmm_splitk_reduce(const void *partials, int partial_dtype, int s, int M, int N, void *C,
                                 void *stream)
{
    if (!partials || !C || s < 1 || M <= 0 || N <= 0) return QMM_ERR_ARG;
    if (partial_dtype != QMM_PARTIAL_BF16 && partial_dtype != QMM_PARTIAL_F32) return QMM_ERR_ARG;
    if ((long long)M * (long long)N > (long long)INT_MAX * 64) return QMM_ERR_SIZE;
    const bool f32 = partial_dtype == QMM_PARTIAL_F32;
    if (!aligned(partials, f32 ? 4 : 2) || !aligned(C, 2)) return QMM_ERR_ALIGN;
    const size_t MN = (size_t)M * (size_t)N;
    const bool vec = (MN % 8 == 0) && aligned(partials, 16) && aligned(C, 16);
    return hip_status(qmm_impl::launch_reduce(partials, f32, s, MN, C, vec, static_cast<hipStream_t>(stream)));
}

extern "C" int qmm_splitk_reduce_cols(const void *partials, int partial_dtype, int s, int M, int N, int n_lo,
                                      void *C, void *stream)
{
    if (!partials || !C || s < 1 || M <= 0 || N <= 0 || n_lo < 0 || n_lo >= N) return QMM_ERR_ARG;
    if (partial_dtype != QMM_PARTIAL_BF16 && partial_dtype != QMM_PARTIAL_F32) return QMM_ERR_ARG;
    if ((long long)M * (long long)N > (long long)INT_MAX * 64) return QMM_ERR_SIZE;
    const bool f32 = partial_dtype == QMM_PARTIAL_F32;
    if (!aligned(partials, f32 ? 4 : 2) || !aligned(C, 2)) return QMM_ERR_ALIGN;
    // eight columns per thread when every row's run [n_lo, N) starts and ends on 8-element
    // boundaries of 16-byte aligned buffers
    const bool vec = (N % 8 == 0) && (n_lo % 8 == 0) && aligned(partials, 16) && aligned(C, 16);
    return hip_status(qmm_impl::launch_reduce_cols(partials, f32, s, M, N, n_lo, C, vec,
                                                   static_cast<hipStream_t>(stream)));
}

extern "C" int qmm_bf16_splitk(const void *A, const void *B, void *C, int M, int N, int K, int s,
                               void *workspace, size_t workspace_bytes, void *stream)
{
    if (!A || !B || !C) return QMM_ERR_ARG;
    if (M <= 0 || N <= 0 || K <= 0 || s < 0) return QMM_ERR_ARG;
    if (K % kGranule != 0) return QMM_ERR_SHAPE;
    if (!sizes_ok(M, N, K)) return QMM_ERR_SIZE;
    if (!aligned(A, 16) || !aligned(B, 16) || !aligned(C, 2)) return QMM_ERR_ALIGN;
    // partition units: 64 values when K is a multiple of 64 (whole 128-byte lines per stage),
    // else 32-value granules
    const int U = K / ((K % 64) == 0 ? 64 : kGranule);
    const DenseTile tile = dense_tile(M, N);
    if (s == 0) {
        // The occupancy rule over this kernel's tile: fill one wave of workgroups.
        const long long base = ceil_div(M, tile.block_m()) * ceil_div(N, tile.block_n());
        long long t = 256 / base;
        if (t > 32) t = 32;
        if (t > U) t = U;
        s = t < 1 ? 1 : (int)t;
    } else if (s > U) {
        return QMM_ERR_SHAPE;
    }
    const size_t MN = (size_t)M * (size_t)N;
    if (s > 1) {
        if (!workspace || workspace_bytes < 4 * (size_t)s * MN) return QMM_ERR_WORKSPACE;
        if (!aligned(workspace, 16)) return QMM_ERR_ALIGN;
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (s == 1) {
        const bool vec = (N % 4 == 0) && aligned(C, 8);
        return hip_status(qmm_impl::launch_dense(tile, A, B, C, false, M, N, K, 1, vec, st));
    }
    int rc = hip_status(qmm_impl::launch_dense(tile, A, B, workspace, true, M, N, K, s, N % 4 == 0, st));
    if (rc != QMM_OK) return rc;
    const bool vec_red = (MN % 8 == 0) && aligned(C, 16);
    return hip_status(qmm_impl::launch_reduce(workspace, true, s, MN, C, vec_red, st));
}

namespace {
constexpr int kAttnHeadDim = 128;
constexpr int kAttnMaxSplit = 64;
constexpr int kAttnPlanCap = 32;
constexpr int kAttnTargetWgs = 256;  // one workgroup per CU
constexpr int kAttnTileKeys = 64;    // keys of one wave's tile: the shortest useful split
constexpr int kAttnOneBatch = 16;    // splits the merge reads in one round trip
}  // namespace

// Split-count rule of decode attention: enough workgroups for one per CU, at most one split
// per 64-key tile, and beyond the merge's one-batch 16 splits only while every split keeps
// at least 512 keys (two tiles per wave). Split sweeps of Qwen3-4B's heads on MI355X: a
// single request takes 16 splits from 1024 to 4096 keys (64-256 keys each: 12 and 7 %
// faster than the 4 and 8 of a 256-key minimum at 1024 and 2048 keys, 8-13 % faster than
// 32), and 32 at 16384 keys.
extern "C" int qmm_attn_decode_split(int B, int Hkv, int Lmax)
{
    if (B <= 0 || Hkv <= 0 || Lmax <= 0) return QMM_ERR_ARG;
    long long s = ceil_div(kAttnTargetWgs, (long long)B * Hkv);
    const long long by_tile = Lmax / kAttnTileKeys;
    if (by_tile < s) s = by_tile;
    const long long long_split = Lmax / (8 * kAttnTileKeys);
    const long long by_batch = long_split > kAttnOneBatch ? long_split : kAttnOneBatch;
    if (by_batch < s) s = by_batch;
    if (s > kAttnPlanCap) s = kAttnPlanCap;
    return s < 1 ? 1 : (int)s;
}

extern "C" size_t qmm_attn_decode_workspace_bytes(int B, int Mq, int Hq, int s)
{
    if (B <= 0 || Mq <= 0 || Hq <= 0 || s <= 1) return 0;
    return (size_t)s * (size_t)B * (size_t)Mq * (size_t)Hq * (size_t)(kAttnHeadDim + 2) * 4;
}

extern "C" int qmm_attn_decode(const void *Q, const void *K, const void *V, const int *lengths, void *O, int B,
                               int Mq, int Hq, int Hkv, int Lmax, int head_dim, float scale, int s, void *workspace,
                               size_t workspace_bytes, void *stream)
{
    if (!Q || !K || !V || !lengths || !O) return QMM_ERR_ARG;
    if (B <= 0 || Mq <= 0 || Hq <= 0 || Hkv <= 0 || Lmax <= 0 || head_dim <= 0 || s < 0) return QMM_ERR_ARG;
    if (!(scale == scale) || scale == __builtin_inff() || scale == -__builtin_inff()) return QMM_ERR_ARG;
    if (head_dim != kAttnHeadDim || Hq % Hkv != 0 || (Hq / Hkv) * Mq > 16 || Mq > Lmax) return QMM_ERR_SHAPE;
    if (s > kAttnMaxSplit) return QMM_ERR_SHAPE;
    if ((long long)B * Hkv * Lmax > (long long)INT_MAX || (long long)B * Mq * Hq > (long long)INT_MAX / 64 ||
        (long long)B * Hkv * kAttnMaxSplit > (long long)INT_MAX)
        return QMM_ERR_SIZE;
    if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(O, 16) || !aligned(lengths, 4))
        return QMM_ERR_ALIGN;
    if (s == 0) s = qmm_attn_decode_split(B, Hkv, Lmax);
    if (s > 1) {
        if (!workspace || workspace_bytes < qmm_attn_decode_workspace_bytes(B, Mq, Hq, s)) return QMM_ERR_WORKSPACE;
        if (!aligned(workspace, 16)) return QMM_ERR_ALIGN;
    }
    return hip_status(qmm_impl::launch_attn_decode(Q, K, V, lengths, O, s > 1 ? workspace : nullptr, B, Mq, Hq, Hkv,
                                                   Lmax, scale, s, static_cast<hipStream_t>(stream)));
}

extern "C" const char *qmm_status_string(int status)
{
    switch (status) {
    case QMM_OK: return "QMM_OK";
    case QMM_ERR_ARG: return "QMM_ERR_ARG: null pointer, non-positive size or bad argument";
    case QMM_ERR_SHAPE: return "QMM_ERR_SHAPE: K not a multiple of the group/granule, or split not allowed";
    case QMM_ERR_ALIGN: return "QMM_ERR_ALIGN: pointer not aligned as required";
    case QMM_ERR_WORKSPACE: return "QMM_ERR_WORKSPACE: workspace missing or too small for the split";
    case QMM_ERR_HIP: return "QMM_ERR_HIP: kernel launch failed";
    case QMM_ERR_SIZE: return "QMM_ERR_SIZE: problem too large for the library's indexing";
    case QMM_ERR_SCRATCH: return "QMM_ERR_SCRATCH: the split's partial planes exceed the library's static scratch";
    default: return "QMM: unknown status";
    }
}
