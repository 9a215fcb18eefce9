// host_checks.cpp -- the C-ABI host code (qmm_api.cpp) built for the CPU alone, under
// AddressSanitizer and UndefinedBehaviorSanitizer, with the kernel launchers replaced by
// recording stubs. It runs every entry point's argument checks and plans over a grid of
// shapes, and checks that a rejected call launches nothing and an accepted one launches the
// kernels its documentation names. No GPU, no HIP runtime: the pointers handed to the
// entry points are host addresses that the host code only inspects for alignment.
//
// Built and run by tests/test_sanitizers.py (g++ -fsanitize=address,undefined).
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <set>
#include <vector>
#include <tuple>

#include "qmm.h"
#include "qmm_launch.h"

namespace {
int g_launches = 0;       // launches recorded since the last reset
int g_last_split = -1;    // split of the last matmul launch
// (bits, mt, ns, gpw, waves, staged rows) of every small-M launch: printed at the end, checked
// by the test against the configurations the kernel source instantiates
std::set<std::tuple<int, int, int, int, int, int>> g_skinny_cfgs;
}  // namespace

// Every global load the small-M kernel issues, its offsets computed as the kernel computes
// them (partition bounds, each wave's groups and rounds, the activation copies, the weight
// loads and the scale/bias copies), for the first and the last workgroup of each grid
// dimension and every partition and wave: each must fall inside A, Wq or the scale/bias
// arrays. A wave with no groups (a partition with fewer groups than waves) issues nothing.
void check_skinny_offsets(qmm_impl::WFormat fmt, int mt, int ns, int tw, int gpw, int waves, int M, int N, int K,
                          int s)
{
    const int sub_shift = fmt.group == 128 ? 0 : fmt.group == 64 ? 1 : 2;
    const int G = K >> 7, GG = G << sub_shift;
    const int WV = fmt.bits / 4;
    const long long row_u4 = (long long)K * fmt.bits / 128;  // 16-byte units per weight row
    const int RW = gpw << sub_shift, EW = 16 * ns * RW, ncp = (EW + 63) >> 6;
    const int gx = (N + tw - 1) / tw, gy = (M + 16 * mt - 1) / (16 * mt);
    for (int bx : {0, gx - 1})
        for (int by : {0, gy - 1})
            for (int z = 0; z < s; ++z)
                for (int wave = 0; wave < waves; ++wave) {
                    const int n_blk = bx * tw, n_end = std::min(N, n_blk + tw), m_blk = by * 16 * mt;
                    if (n_blk >= N || m_blk >= M) abort();
                    const unsigned Gu = (unsigned)G, S = (unsigned)s, Z = (unsigned)z;
                    const int g0 = S == 1 ? 0 : (int)((Z * Gu) / S);
                    const int gpp = S == 1 ? G : (int)(((Z + 1) * Gu) / S) - g0;
                    if (gpp < 1) abort();
                    const int n_w = (int)((unsigned)(gpp - wave + waves - 1) / (unsigned)waves);
                    if (n_w < 1) continue;
                    for (int base = 0; base < n_w; base += gpw) {
                        for (int q = 0; q < gpw && base + q < n_w; ++q) {
                            const int g = g0 + wave + waves * (base + q);
                            if (g < g0 || g >= g0 + gpp) abort();
                            for (int r = 0; r < 16; ++r)
                                for (int j = 0; j < ns; ++j) {
                                    const int n = std::min(n_blk + 16 * j + r, n_end - 1);
                                    for (int slot = 0; slot < 4; ++slot)
                                        for (int u = 0; u < WV; ++u) {
                                            const long long i4 = (long long)WV * slot + 4LL * WV * g + u;
                                            if (n < 0 || n >= N || i4 < 0 || i4 >= row_u4) abort();
                                        }
                                }
                            for (int c = 0; c < qmm_impl::skinny_rows(mt, ns, fmt.bits, M) / 4; ++c)
                                for (int lane = 0; lane < 64; ++lane) {
                                    const int row = 4 * c + (lane >> 4);
                                    if (m_blk + 4 * c >= M) continue;  // copy not issued
                                    const long long m = std::min(m_blk + row, M - 1);
                                    const long long off = m * K * 2 + 16LL * ((lane & 15) ^ (row & 15)) + 256LL * g;
                                    if (off < 0 || off + 16 > 2LL * M * K || off >= (1LL << 32)) abort();
                                }
                        }
                        const int nq = std::min(gpw, n_w - base);
                        for (int c = 0; c < ncp; ++c)
                            for (int lane = 0; lane < 64; ++lane) {
                                const int e = std::min(64 * c + lane, EW - 1);
                                const int row_e = (e >> sub_shift) / gpw;
                                const int rem = e - row_e * RW;
                                const int row = std::min(row_e, n_end - 1 - n_blk);
                                const int q = std::min(rem >> sub_shift, nq - 1);
                                const long long g = g0 + wave + (long long)waves * (base + q);
                                const long long idx =
                                    (long long)row * GG + (g << sub_shift) + (rem & ((1 << sub_shift) - 1));
                                if (idx < 0 || (long long)n_blk * GG + idx >= (long long)N * GG ||
                                    2 * idx >= (1LL << 32))
                                    abort();
                            }
                    }
                }
}

namespace qmm_impl {
hipError_t launch_w4a16_skinny(WFormat fmt, int mt, int ns, int tw, int gpw, int waves, const void *,
                               const void *, const void *, const void *, void *, bool, int M, int N, int K, int s, bool,
                               hipStream_t)
{
    if (waves < 1 || waves > 16) abort();
    if (tw < 1 || tw > 16 * ns || (tw < 16 * ns && (ns != 1 || s != 1))) abort();  // narrowed: unsplit 16-column only
    if ((long long)(N + tw - 1) / tw > 65535) abort();  // grid x
    const int rows = skinny_rows(mt, ns, fmt.bits, M);
    if (M < 1 || (rows < 16 * mt && M > rows)) abort();
    if (skinny_lds_bytes(mt, ns, waves, gpw, fmt.sub(), rows) > (size_t)kLdsPerCU) abort();
    g_skinny_cfgs.insert(std::make_tuple(fmt.bits, mt, ns, gpw, waves, rows));
    check_skinny_offsets(fmt, mt, ns, tw, gpw, waves, M, N, K, s);
    ++g_launches;
    g_last_split = s;
    return hipSuccess;
}
hipError_t launch_w4a16_wide(WFormat, int variant, const void *, const void *, const void *, const void *, void *,
                             void *, bool, int, int, int, int, int split, bool, hipStream_t, int)
{
    if (variant < 0 || variant > 2) abort();
    ++g_launches;
    g_last_split = split;
    return hipSuccess;
}
hipError_t launch_w4a16_gemv(const void *, const void *, const void *, const void *, void *, int, int, int, int s,
                             hipStream_t)
{
    ++g_launches;
    g_last_split = s;
    return hipSuccess;
}
hipError_t launch_reduce(const void *, bool, int, size_t, void *, bool, hipStream_t)
{
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_reduce_cols(const void *, bool, int, int, int, int, void *, bool, hipStream_t)
{
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_attn_decode(const void *, const void *, const void *, const int *, void *, void *, int, int, int,
                              int, int, float, int S, hipStream_t)
{
    ++g_launches;
    g_last_split = S;
    return hipSuccess;
}
hipError_t launch_dense(DenseTile, const void *, const void *, void *, bool, int, int, int, int s, bool, hipStream_t)
{
    ++g_launches;
    g_last_split = s;
    return hipSuccess;
}
}  // namespace qmm_impl

namespace {

int failures = 0;

void expect(bool ok, const char *what, int line)
{
    if (!ok) {
        fprintf(stderr, "FAIL line %d: %s\n", line, what);
        ++failures;
    }
}
#define EXPECT(c) expect((c), #c, __LINE__)

// An aligned host arena standing in for device buffers (never dereferenced by the host code).
alignas(256) unsigned char arena[1 << 16];
void *P(size_t off) { return arena + off; }

int call_w4a16(int M, int N, int K, int s, void *ws, size_t wsb, const void *A = P(0), const void *W = P(256),
               void *C = P(1024))
{
    g_launches = 0;
    return qmm_w4a16_g128(A, W, P(512), P(768), C, M, N, K, s, ws, wsb, nullptr);
}

}  // namespace

// The large-M kernel's XCD order: for every region shape and every panel height that divides
// the row blocks, wide_item maps the region's workgroups one to one onto its (partition,
// column block, row block) items; wide_panel returns 0 or such a divisor.
void check_wide_order()
{
    long regions = 0;
    std::vector<char> seen;
    for (int P = 1; P <= 7; ++P)
        for (int nb = 1; nb <= 40; nb += (nb < 12 ? 1 : 7))
            for (int num_m = 1; num_m <= 17; ++num_m) {
                const int wr = P * nb * num_m;
                for (int pm = 1; pm <= num_m; ++pm) {
                    if (num_m % pm) continue;
                    seen.assign((size_t)wr, 0);
                    for (int r = 0; r < wr; ++r) {
                        const qmm_impl::WideItem it = qmm_impl::wide_item(r, wr, num_m, nb, pm);
                        EXPECT(it.p >= 0 && it.p < P && it.n >= 0 && it.n < nb && it.m >= 0 && it.m < num_m);
                        const size_t idx = ((size_t)it.p * nb + it.n) * num_m + it.m;
                        EXPECT(!seen[idx]);
                        seen[idx] = 1;
                    }
                    ++regions;
                }
                for (double ratio : {0.05, 0.3, 1.0, 3.0, 20.0}) {
                    const int pm = qmm_impl::wide_panel(P, nb, num_m, 1.0, ratio);
                    EXPECT(pm == 0 || (pm >= 1 && pm <= num_m && num_m % pm == 0));
                }
            }
    // the Qwen3-4B M = 2048 regions: an XCD-blocked order where one XCD would otherwise read
    // every column block (gate's whole tiles: 8 x 32 tiles of 256 x 256; o and down: 3
    // partitions of 8 x 10)
    EXPECT(qmm_impl::wide_panel(1, 32, 8, 20 * 65536.0, 20 * 256 * 68.0) > 0);
    EXPECT(qmm_impl::wide_panel(3, 10, 8, 76 / 3.0 * 65536.0, 76 / 3.0 * 256 * 68.0) > 0);
    printf("wide order regions %ld\n", regions);
}

int main()
{
    check_wide_order();
    // ---- plans over a grid of shapes, every preset and a few tunables
    const int Ms[] = {1, 2, 7, 16, 31, 32, 33, 48, 64, 65, 100, 128, 129, 255, 256, 300, 1000, 2048, 4096};
    const int Ns[] = {1, 17, 100, 1000, 1024, 2560, 4096, 9728, 16484};
    const int Ks[] = {128, 256, 1024, 2560, 4096, 9728, 16384};
    const qmm_policy pols[] = {QMM_POLICY_PAGE, QMM_POLICY_MI355X, {16, 64, 512, 4, 256}, {0, 0, 1, 1, 128},
                               {0, 0, 100000, 64, 128}};
    long plans = 0;
    for (int M : Ms)
        for (int N : Ns)
            for (int K : Ks)
                for (const qmm_policy &pol : pols) {
                    qmm_plan p;
                    memset(&p, 0xA5, sizeof p);
                    const int rc = qmm_splitk_plan(M, N, K, 128, &pol, &p);
                    EXPECT(rc == QMM_OK);
                    EXPECT(p.s >= 1 && p.s <= K / 128);
                    EXPECT(p.workspace_bytes == (p.s > 1 ? (size_t)2 * p.s * M * N : 0));
                    EXPECT(p.full_tiles >= 0 && p.full_tiles <= p.base_tiles || p.block_m < 128);
                    for (int bits : {4, 8})
                        for (int g : {32, 64, 128}) {
                            qmm_plan pf;
                            EXPECT(qmm_wna16_plan(bits, g, M, N, K, &pol, &pf) == QMM_OK);
                        }
                    ++plans;
                }

    // ---- plan errors
    qmm_plan p;
    EXPECT(qmm_splitk_plan(0, 8, 128, 128, nullptr, &p) == QMM_ERR_ARG);
    EXPECT(qmm_splitk_plan(8, 8, 200, 128, nullptr, &p) == QMM_ERR_SHAPE);
    EXPECT(qmm_splitk_plan(8, 8, 128, 64, nullptr, &p) == QMM_ERR_ARG);
    EXPECT(qmm_splitk_plan(8, 8, 128, 128, nullptr, nullptr) == QMM_ERR_ARG);
    EXPECT(qmm_splitk_plan(8, 8, 1 << 22, 128, nullptr, &p) == QMM_ERR_SIZE);
    EXPECT(qmm_wna16_plan(5, 128, 8, 8, 128, nullptr, &p) == QMM_ERR_ARG);
    const qmm_policy bad = {0, 0, 256, 0, 512};
    EXPECT(qmm_splitk_plan(8, 8, 128, 128, &bad, &p) == QMM_ERR_ARG);

    // ---- the matmul: rejected calls launch nothing
    char ws_small[64];
    (void)ws_small;
    EXPECT(call_w4a16(32, 1024, 2560, 1, nullptr, 0, nullptr) == QMM_ERR_ARG && g_launches == 0);
    EXPECT(call_w4a16(0, 1024, 2560, 1, nullptr, 0) == QMM_ERR_ARG && g_launches == 0);
    EXPECT(call_w4a16(32, 1024, 2500, 1, nullptr, 0) == QMM_ERR_SHAPE && g_launches == 0);
    EXPECT(call_w4a16(32, 1024, 2560, 21, P(4096), 1 << 20) == QMM_ERR_SHAPE && g_launches == 0);  // 21 > 20 groups
    // a split that does not divide the 20 groups: near-equal partitions, accepted
    EXPECT(call_w4a16(32, 1024, 2560, 3, P(4096), 1 << 20) == QMM_OK && g_launches == 2 && g_last_split == 3);
    EXPECT(call_w4a16(128, 9728, 2560, 3, P(4096), 1 << 24) == QMM_OK && g_launches == 2 && g_last_split == 3);
    EXPECT(call_w4a16(32, 1024, 2560, 40, P(4096), 1 << 20) == QMM_ERR_SHAPE && g_launches == 0);
    EXPECT(call_w4a16(32, 1024, 2560, 4, nullptr, 0) == QMM_ERR_WORKSPACE && g_launches == 0);
    EXPECT(call_w4a16(32, 1024, 2560, 4, P(4096), 2 * 4 * 32 * 1024 - 1) == QMM_ERR_WORKSPACE && g_launches == 0);
    EXPECT(call_w4a16(32, 1024, 2560, 4, P(4100), 1 << 20) == QMM_ERR_ALIGN && g_launches == 0);
    EXPECT(call_w4a16(32, 1024, 2560, 1, nullptr, 0, P(2)) == QMM_ERR_ALIGN && g_launches == 0);
    EXPECT(call_w4a16(32, 1024, 2560, 1, nullptr, 0, P(0), P(8)) == QMM_ERR_ALIGN && g_launches == 0);
    EXPECT(call_w4a16(32, 1024, 2560, 1, nullptr, 0, P(0), P(256), P(1025)) == QMM_ERR_ALIGN && g_launches == 0);
    EXPECT(call_w4a16(1 << 20, 1 << 20, 1 << 14, 1, nullptr, 0) == QMM_ERR_SIZE && g_launches == 0);

    // ---- accepted calls launch the matmul, plus the merge when split
    EXPECT(call_w4a16(32, 1024, 2560, 1, nullptr, 0) == QMM_OK && g_launches == 1 && g_last_split == 1);
    EXPECT(call_w4a16(32, 1024, 2560, 4, P(4096), 1 << 20) == QMM_OK && g_launches == 2 && g_last_split == 4);
    for (int M : {1, 16, 32, 64, 128, 2048})
        for (int N : {1000, 1024, 2560, 9728})
            for (int K : {2560, 4096, 9728}) {
                qmm_plan pl;
                EXPECT(qmm_splitk_plan(M, N, K, 128, nullptr, &pl) == QMM_OK);
                const int rc = call_w4a16(M, N, K, 0, pl.s > 1 ? P(4096) : nullptr, pl.workspace_bytes);
                EXPECT(rc == QMM_OK && g_launches == (pl.s > 1 ? 2 : 1) && g_last_split == pl.s);
                int s_out = 0, n_lo = -1;
                g_launches = 0;
                EXPECT(qmm_w4a16_g128_pass1(P(0), P(256), P(512), P(768), P(1024), M, N, K, 0,
                                            pl.s > 1 ? P(4096) : nullptr, pl.workspace_bytes, &s_out, &n_lo,
                                            nullptr) == QMM_OK);
                EXPECT(g_launches == 1 && s_out == pl.s && n_lo >= 0 && n_lo <= N);
                EXPECT((pl.s == 1) == (n_lo == N));
            }

    // ---- the other entry points: argument errors launch nothing
    g_launches = 0;
    EXPECT(qmm_w4a16_gemv(P(0), P(256), P(512), P(768), P(1024), 9, 100, 256, 1, nullptr, 0, nullptr) ==
           QMM_ERR_SHAPE);
    EXPECT(qmm_w4a16_gemv(P(0), P(256), P(512), P(768), P(1024), 1, 100, 256, 3, nullptr, 0, nullptr) ==
           QMM_ERR_SHAPE);
    EXPECT(qmm_gemv_min_split(0, 256) == QMM_ERR_ARG && qmm_gemv_min_split(9, 256) == QMM_ERR_SHAPE);
    EXPECT(qmm_splitk_reduce(nullptr, QMM_PARTIAL_BF16, 2, 4, 4, P(0), nullptr) == QMM_ERR_ARG);
    EXPECT(qmm_splitk_reduce(P(0), 7, 2, 4, 4, P(64), nullptr) == QMM_ERR_ARG);
    EXPECT(qmm_splitk_reduce(P(1), QMM_PARTIAL_F32, 2, 4, 4, P(64), nullptr) == QMM_ERR_ALIGN);
    EXPECT(qmm_splitk_reduce_cols(P(0), QMM_PARTIAL_BF16, 2, 4, 4, 4, P(64), nullptr) == QMM_ERR_ARG);
    EXPECT(qmm_bf16_splitk(P(0), P(256), P(1024), 512, 512, 100, 2, P(4096), 1 << 20, nullptr) == QMM_ERR_SHAPE);
    EXPECT(qmm_bf16_splitk(P(0), P(256), P(1024), 512, 512, 16384, 600, P(4096), 1 << 24, nullptr) ==
           QMM_ERR_SHAPE);
    EXPECT(qmm_bf16_splitk(P(0), P(256), P(1024), 512, 512, 16384, 4, P(4096), 100, nullptr) ==
           QMM_ERR_WORKSPACE);
    EXPECT(qmm_w4a16_g128_streamk(P(0), P(256), P(512), P(768), P(1024), 64, 1024, 2560, 0, P(4096), 1 << 20,
                                  nullptr) == QMM_ERR_SHAPE);
    EXPECT(qmm_wna16(5, 128, QMM_PARTIAL_BF16, P(0), P(256), P(512), P(768), P(1024), 32, 1024, 2560, 1, nullptr, 0,
                     nullptr) == QMM_ERR_ARG);
    EXPECT(qmm_wna16(4, 128, 3, P(0), P(256), P(512), P(768), P(1024), 32, 1024, 2560, 1, nullptr, 0, nullptr) ==
           QMM_ERR_ARG);
    const int lengths[4] = {8, 8, 8, 8};
    EXPECT(qmm_attn_decode(P(0), P(256), P(512), lengths, P(1024), 1, 1, 32, 8, 64, 64, 0.1f, 1, nullptr, 0,
                           nullptr) == QMM_ERR_SHAPE);
    EXPECT(qmm_attn_decode(P(0), P(256), P(512), lengths, P(1024), 1, 1, 32, 8, 64, 128, __builtin_nanf(""), 1,
                           nullptr, 0, nullptr) == QMM_ERR_ARG);
    EXPECT(qmm_attn_decode(P(0), P(256), P(512), lengths, P(1024), 1, 1, 32, 8, 64, 128, 0.1f, 65, nullptr, 0,
                           nullptr) == QMM_ERR_SHAPE);
    EXPECT(g_launches == 0);

    // ---- accepted calls of the other entry points
    g_launches = 0;
    EXPECT(qmm_bf16_splitk(P(0), P(256), P(1024), 512, 512, 16384, 6, P(4096), 4 * 6 * 512 * 512, nullptr) ==
           QMM_OK && g_launches == 2 && g_last_split == 6);
    g_launches = 0;
    EXPECT(qmm_w4a16_gemv(P(0), P(256), P(512), P(768), P(1024), 1, 2560, 9728, 0, P(4096), 1 << 20, nullptr) ==
           QMM_OK && g_launches >= 1);
    g_launches = 0;
    EXPECT(qmm_attn_decode(P(0), P(256), P(512), lengths, P(1024), 1, 1, 32, 8, 1024, 128, 0.1f, 4, P(4096),
                           qmm_attn_decode_workspace_bytes(1, 1, 32, 4), nullptr) == QMM_OK && g_launches == 1);
    for (int st = -7; st <= 1; ++st) EXPECT(qmm_status_string(st) != nullptr);

    // ---- every small-M configuration the host can pick: decode and small rows, every
    // format, plan and explicit splits
    for (int M : {1, 2, 3, 4, 5, 7, 8, 9, 12, 16, 20, 24, 32, 40, 48, 64, 80, 100, 128})
        for (int N : {16, 100, 1000, 1024, 2560, 4096, 5000, 9728})
            for (int K : {128, 384, 1024, 2560, 4096, 9728, 16384})
                for (int bits : {4, 8})
                    for (int g : {32, 64, 128})
                        for (int s : {0, 1, 2, 3, 5}) {
                            if (s > K / 128) continue;
                            qmm_plan pl;
                            if (qmm_wna16_plan(bits, g, M, N, K, nullptr, &pl) != QMM_OK) continue;
                            const int s_eff = s ? s : pl.s;
                            const size_t ws = (size_t)4 * s_eff * M * N;
                            static unsigned char *big = nullptr;
                            (void)big;
                            g_launches = 0;
                            const int rc = qmm_wna16(bits, g, QMM_PARTIAL_BF16, P(0), P(256), P(512), P(768), P(1024),
                                                     M, N, K, s, s_eff > 1 ? P(4096) : nullptr, ws, nullptr);
                            EXPECT(rc == QMM_OK);
                        }
    for (const auto &c : g_skinny_cfgs)
        printf("skinny config %d %d %d %d %d %d\n", std::get<0>(c), std::get<1>(c), std::get<2>(c), std::get<3>(c),
               std::get<4>(c), std::get<5>(c));

    if (failures) {
        fprintf(stderr, "%d host checks failed\n", failures);
        return 1;
    }
    printf("host checks ok: %ld plans\n", plans);
    return 0;
}
