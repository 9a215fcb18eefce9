"""Host-side tests of the C-ABI library (no GPU needed).

They load libqmm.so, check that it exports every symbol include/qmm.h declares,
exercise the host-only split plan against the oracle's statement of the page's
rule, and check that every invalid call returns its error code before any
launch. No call here reaches a kernel launch: each one fails validation first.
"""
import ctypes
import os
import re

import pytest

import qmm_synth as syn
import weight_only_quantized_qmm_amd as q
from oracle import policy as opolicy

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qmm.h")

# Fake, never-dereferenced device addresses for validation-only calls.
ADDR = 0x7f0000000000
ADDR2 = 0x7f0010000000
ADDR3 = 0x7f0020000000


def header_symbols():
    text = open(HEADER).read()
    funcs = set(re.findall(r"^\s*(?:int|size_t|const char \*)\s*(qmm_\w+)\s*\(", text, re.M))
    data = set(re.findall(r"^extern const qmm_policy (\w+);", text, re.M))
    return funcs, data


def test_library_exports_every_declared_symbol():
    funcs, data = header_symbols()
    assert funcs == set(q.EXPORTED_FUNCTIONS)
    assert data == set(q.EXPORTED_DATA)
    L = q.lib()
    for f in funcs:
        assert hasattr(L, f), f
    for d in data:
        ctypes.c_int.in_dll(L, d)  # resolves the data symbol


def test_calibration_library_exports_what_the_bench_binds():
    # libqmm_calib.so holds only the benchmark's measurement kernels; bench.py binds
    # these entry points by name (loading it initialises no GPU)
    import bench
    L = bench.calib_lib()
    for f in ("qmm_calib_empty", "qmm_calib_read", "qmm_calib_read_grid", "qmm_calib_chain", "qmm_calib_copy",
              "qmm_calib_mfma", "qmm_calib_step"):
        assert hasattr(L, f), f


def test_status_strings():
    for code in (q.QMM_OK, q.QMM_ERR_ARG, q.QMM_ERR_SHAPE, q.QMM_ERR_ALIGN, q.QMM_ERR_WORKSPACE,
                 q.QMM_ERR_HIP, q.QMM_ERR_SIZE, q.QMM_ERR_SCRATCH):
        assert q.qmm_status_string(code).startswith("QMM")
    assert "unknown" in q.qmm_status_string(12345)


def test_page_preset_values():
    assert q.policy_preset("QMM_POLICY_PAGE").as_dict() == dict(
        tile_m=32, tile_n=32, target_blocks=320, cap=16, min_k_per_split=128)


def _page_split_oracle(M, N, K, **kw):
    r = dict(opolicy.PAGE_PRESET)
    r.update(kw)
    return opolicy.split_count(M, N, K, **r)


ALL_SHAPES = ([(32, 1024, 2560), (48, 1000, 2560), (512, 512, 16384)]
              + [(M, N, K) for _, M, N, K, _ in syn.projection_sweep()]
              + [(M, N, K) for _, M, N, K, _ in syn.decode_sweep()]
              + [(1, 1, 128), (3, 17, 256), (129, 4096, 9728), (7, 100000, 128)])


@pytest.mark.parametrize("M,N,K", ALL_SHAPES)
def test_plan_page_preset_matches_oracle_rule(M, N, K):
    pol = q.policy_preset("QMM_POLICY_PAGE")
    plan = q.qmm_splitk_plan(M, N, K, policy=pol)
    assert plan.s == _page_split_oracle(M, N, K)
    assert plan.base_tiles == opolicy.base_tiles(M, N, 32, 32)
    assert plan.workspace_bytes == (2 * plan.s * M * N if plan.s > 1 else 0)


def test_plan_tunables_follow_oracle_rule():
    for target in (64, 320, 512, 1024, 4096):
        for cap in (1, 4, 16, 32):
            for min_k in (128, 256, 512, 1024):
                pol = q.qmm_policy(16, 64, target, cap, min_k)
                for M, N, K in ALL_SHAPES:
                    got = q.qmm_splitk_plan(M, N, K, policy=pol).s
                    assert got == opolicy.split_count(M, N, K, tile_m=16, tile_n=64, target=target, cap=cap,
                                                      min_k_per_split=min_k), (M, N, K, target, cap, min_k)


@pytest.mark.parametrize("M,N,K", ALL_SHAPES)
def test_plan_mi355x_preset_is_valid(M, N, K):
    pol = q.policy_preset("QMM_POLICY_MI355X")
    plan = q.qmm_splitk_plan(M, N, K)
    G = K // 128
    # the occupancy count uses the kernel's tile; only an unsplit small-M grid narrows it
    assert plan.tile_m == plan.block_m and (plan.tile_n == plan.block_n or plan.s == 1)
    tiles = -(-M // plan.tile_m) * -(-N // plan.tile_n)
    assert plan.base_tiles == tiles
    assert 1 <= plan.s <= min(pol.cap, G)
    assert plan.s == 1 or K // plan.s >= pol.min_k_per_split
    assert plan.workspace_bytes == (2 * plan.s * M * N if plan.s > 1 else 0)
    # the small-M kernel runs M <= 64, and M <= 128 with N*K <= 2^24 (64-row blocks)
    wide = plan.block_m >= 128
    assert wide == (M > 64 and not (M <= 128 and N * K <= 1 << 24))
    if wide:  # the large-M kernel: slot-filling rule over its tiles (128 x 256, 128 x 128, 256 x 256)
        assert (plan.block_m, plan.block_n) in ((128, 256), (128, 128), (256, 256))
        # two 128 x 256 workgroups per CU up to M = 128; every other tile counts one per CU
        slots = pol.target_blocks * (2 if (plan.block_m, plan.block_n) == (128, 256) and M <= 128 else 1)
        check_slot_filling(plan, M, K, slots, pol)
    else:  # the page's rule over the kernel's tile without its divisor step (near-equal
        # partitions); partitions of at least 2048 values up to M = 32
        # 16-column tiles for up to 32 rows over at most 2^24 weights (and for up to 8 rows
        # with at most 4096 columns, and up to 4 rows at any width); else 32 columns while
        # they fit one workgroup per CU over K < 8192, else 48 when those fit, else 64
        rows = -(-M // plan.block_m)
        one_round_16 = M <= 64 and -(-M // 16) * -(-N // 16) <= 256 and N * K <= 1 << 24
        t64 = -(-M // 16) * -(-N // 64)
        one_round_64 = M <= 64 and N * K <= 1 << 24 and 3 * 256 <= 4 * t64 <= 4 * 256
        one_round_32 = 64 < M and -(-M // 32) * -(-N // 16) <= 256 and N * K <= 1 << 24
        if one_round_16:  # narrow projections: 16-row, 16-column tiles in one round
            assert plan.block_m == 16 and plan.tile_n == 16
        elif one_round_64:  # 16-row, 64-column tiles filling at least 3/4 of one round
            assert plan.block_m == 16 and plan.tile_n == 64
        elif one_round_32:  # past 64 rows: 32-row, 16-column tiles in one round
            assert plan.block_m == 32 and plan.tile_n == 16
        elif M <= 32 and (N * K <= 1 << 24 or (M <= 8 and N <= 4096) or M <= 4):
            assert plan.tile_n == 16
        elif rows * -(-N // 32) <= 256 and K < 8192:
            assert plan.tile_n == 32
        else:
            assert plan.tile_n == (48 if rows * -(-N // 48) <= 256 else 64)
        min_k = max(pol.min_k_per_split, 2048) if M <= 32 else pol.min_k_per_split
        assert plan.s == max(1, min(pol.cap, pol.target_blocks // tiles, K // min_k, G))
        # the page's rule would lower that to a divisor of G
        page_s = opolicy.split_count(M, N, K, tile_m=plan.block_m, tile_n=plan.tile_n, target=pol.target_blocks,
                                     cap=pol.cap, min_k_per_split=min_k)
        assert page_s <= plan.s and G % page_s == 0
        # an unsplit grid of 16-column tiles with fewer tiles than CUs runs narrower tiles,
        # ceil(N / (256 // rows)) columns, so that it covers every CU once
        if plan.s == 1 and plan.tile_n == 16 and tiles < 256:
            assert plan.block_n == -(-N // (256 // rows))
        else:
            assert plan.block_n == plan.tile_n
        run_tiles = rows * -(-N // plan.block_n)
        assert run_tiles <= max(tiles, 256)
        assert plan.grid_z == plan.s
        assert (plan.grid_x, plan.grid_y) == (-(-N // plan.block_n), rows)
        assert plan.full_tiles == (run_tiles if plan.s == 1 else 0)


FORMATS = [(4, 32), (4, 64), (4, 128), (8, 32), (8, 64), (8, 128)]


def _wide_lds_bytes(rows, bits, group, cols=256):
    # three stage slots of A (rows x 64 bf16) and of W (cols rows x 64 codes), two of the
    # 128-value block's scale and bias dwords (cols rows x 128/group groups each)
    return 3 * rows * 128 + 3 * cols * 64 * bits // 8 + 2 * 2 * cols * 4 * (128 // group)


@pytest.mark.parametrize("bits,group", FORMATS)
def test_wna16_plan_follows_the_rule_for_each_format(bits, group):
    pol = q.policy_preset("QMM_POLICY_MI355X")
    for M, N, K in ALL_SHAPES:
        name = "%dx%dx%d" % (M, N, K)
        plan = q.qmm_wna16_plan(bits, group, M, N, K)
        ref = q.qmm_splitk_plan(M, N, K)
        assert (plan.block_m, plan.block_n, plan.base_tiles) == (ref.block_m, ref.block_n, ref.base_tiles)
        if plan.block_m < 128 or (bits, group) == (4, 128):
            assert (plan.s, plan.full_tiles, plan.grid_x) == (ref.s, ref.full_tiles, ref.grid_x), (name, M)
            continue
        wgs = 2 if ((plan.block_m, plan.block_n) == (128, 256) and M <= 128
                    and 2 * _wide_lds_bytes(128, bits, group) <= 160 * 1024) else 1
        check_slot_filling(plan, M, K, pol.target_blocks * wgs, pol, what=name)


def test_wna16_plan_lds_budget():
    # 128-row tiles keep two workgroups per CU only for 4-bit codes in groups of 64 or 128
    two = [f for f in FORMATS if 2 * _wide_lds_bytes(128, *f) <= 160 * 1024]
    assert two == [(4, 64), (4, 128)]
    assert max(_wide_lds_bytes(256, *f) for f in FORMATS) <= 160 * 1024


@pytest.mark.parametrize("M,N,K", [(M, N, K) for M, N, K in ALL_SHAPES
                                   if M > 64 and not (M <= 128 and N * K <= 1 << 24)])
def test_large_m_tile_choice_is_admissible(M, N, K):
    # the large-M kernel's three tiles: 256 x 256 only above 128 rows, 128 x 128 only while
    # its tiles are fewer than the CUs (a pure split at one workgroup per CU)
    plan = q.qmm_splitk_plan(M, N, K)
    assert (plan.block_m, plan.block_n) in ((128, 256), (128, 128), (256, 256))
    if plan.block_m == 256:
        assert M > 128
    if plan.block_n == 128:
        assert -(-M // 128) * -(-N // 128) < 256 and plan.full_tiles == 0


def test_large_m_variant_on_the_sweep():
    # M = 2048: q on 128 x 256 tiles, k/v on 128 x 128, the rest on 256 x 256; M = 128:
    # gate, up and down on 128 x 128 (q, k, v, o run the small-M kernel)
    got = {(n, M): (p.block_m, p.block_n) for n, M, N, K, _ in syn.projection_sweep() if M in (128, 2048)
           for p in [q.qmm_splitk_plan(M, N, K)]}
    big = {n: got[(n, 2048)] for n in ("q", "k", "v", "o", "gate", "up", "down")}
    assert big == {"q": (128, 256), "k": (128, 128), "v": (128, 128), "o": (256, 256), "gate": (256, 256),
                   "up": (256, 256), "down": (256, 256)}
    assert all(got[(n, 128)] == (128, 128) for n in ("gate", "up", "down"))
    assert all(got[(n, 128)][0] == 64 for n in ("q", "o"))
    assert all(got[(n, 128)] == (32, 16) for n in ("k", "v"))  # 32-row tiles of 16 columns, one round


def check_slot_filling(plan, M, K, slots, pol, what=""):
    """Properties of the large-M kernel's slot-filling decomposition (the library's own
    rule for that kernel, stated in qmm.h), checked without restating the rule:
      * the split respects the cap, the group count and the shortest partition;
      * the unsplit tiles are whole columns of tiles and come first;
      * a split's last round fits the workgroup slots, and one more partition would not
        (the split is as deep as the slots allow, unless capped);
      * with the tiles already filling whole rounds of slots, nothing is split."""
    G = K // 128
    T = plan.base_tiles
    num_m = -(-M // plan.block_m)
    smax = min(pol.cap, G, K // pol.min_k_per_split)
    assert 1 <= plan.s <= max(1, smax), what
    assert plan.grid_x == plan.full_tiles + (T - plan.full_tiles) * plan.s, what
    assert plan.grid_y == 1 and plan.grid_z == 1, what
    if plan.s == 1:
        assert plan.full_tiles == T, what
        if T < slots:  # an unsplit pure grid: two partitions would not fit, or splitting is barred
            assert 2 * T > slots or smax <= 1, what
        else:  # full rounds: the columns left after whole rounds do not fit two partitions
            full = (T // slots) * slots
            full -= full % num_m
            assert T - full == 0 or 2 * (T - full) > slots or smax <= 1, what
        return
    assert plan.full_tiles % num_m == 0 and 0 <= plan.full_tiles < T, what
    tail = T - plan.full_tiles
    assert tail * plan.s <= slots, what  # the split tiles' workgroups fit one round of slots
    assert plan.s == smax or tail * (plan.s + 1) > slots, what
    if plan.full_tiles:
        assert plan.full_tiles >= slots - num_m and T >= slots, what  # only past whole rounds


# Hand-derived decompositions of the Qwen3-4B sweep under the MI355X preset {0, 0, 256, 20, 512}
# (G = K/128 groups; smax = min(20, G, K/512)):
#   gate/up M=2048: 256 x 256 tiles, 8 x 38 = 304 >= 256 slots; 256 whole (a multiple of 8 rows
#                   of tiles) unsplit, the 48 left in min(5, 256 // 48 = 5) = 5 partitions
#   down M=2048:    8 x 10 = 80 tiles, s = min(19, 256 // 80 = 3) = 3
#   o M=2048:       8 x 10 = 80 tiles, s = min(8, 3) = 3
#   q M=2048:       128 x 256 tiles, 16 x 16 = 256 = the slots: one full round, no split
#   k/v M=2048:     128 x 128 tiles, 16 x 8 = 128, s = min(5, 256 // 128 = 2) = 2
#   gate/up M=128:  128 x 128 tiles, 76, s = min(5, 256 // 76 = 3) = 3
#   down M=128:     128 x 128 tiles, 20, s = min(19, 256 // 20 = 12) = 12
HAND_PLANS = {("gate", 2048): (5, 256), ("up", 2048): (5, 256), ("down", 2048): (3, 0), ("o", 2048): (3, 0),
              ("q", 2048): (1, 256), ("k", 2048): (2, 0), ("v", 2048): (2, 0),
              ("gate", 128): (3, 0), ("up", 128): (3, 0), ("down", 128): (12, 0)}


def test_large_m_plan_hand_derived_cases():
    got = {(n, M): (p.s, p.full_tiles) for n, M, N, K, _ in syn.projection_sweep() if (n, M) in HAND_PLANS
           for p in [q.qmm_splitk_plan(M, N, K)]}
    assert got == HAND_PLANS


def test_large_m_plan_split_tail_hand_derived():
    # 1000 x (64*256 + 100) x 2560 on 128 x 256 tiles: 8 x 65 = 520 >= 256 slots; 512 whole
    # tiles (two rounds, a multiple of 8) unsplit, the last column of 8 tiles in
    # min(5, 256 // 8) = 5 partitions
    p = q.qmm_splitk_plan(1000, 64 * 256 + 100, 2560)
    assert (p.block_m, p.block_n, p.s, p.full_tiles, p.grid_x) == (128, 256, 5, 512, 512 + 8 * 5)
    # whole columns: 300 x (342*256) x 2560 on 128 x 256 tiles: 3 x 342 = 1026 tiles; four
    # rounds are 1024, rounded down to 1023 (a multiple of 3); 3 left in min(5, 256 // 3) = 5
    p = q.qmm_splitk_plan(300, 342 * 256, 2560)
    assert (p.block_m, p.block_n, p.s, p.full_tiles) == (128, 256, 5, 1023)
    # 300 x 100000: 3 x 391 = 1173 tiles, 1023 whole, the 150 left fit only one partition each
    p = q.qmm_splitk_plan(300, 100000, 2560)
    assert (p.s, p.full_tiles) == (1, p.base_tiles)
    # K below two shortest partitions (512 values): never split
    assert q.qmm_splitk_plan(2048, 256, 768).s == 1


def test_plan_rejects_bad_arguments():
    for args, code in [((0, 8, 128), q.QMM_ERR_ARG), ((8, 0, 128), q.QMM_ERR_ARG), ((8, 8, 0), q.QMM_ERR_ARG),
                       ((8, 8, 200), q.QMM_ERR_SHAPE)]:
        with pytest.raises(q.QmmError) as e:
            q.qmm_splitk_plan(*args)
        assert e.value.status == code
    with pytest.raises(q.QmmError) as e:
        q.qmm_splitk_plan(8, 8, 128, group_size=64)
    assert e.value.status == q.QMM_ERR_ARG
    with pytest.raises(q.QmmError) as e:
        q.qmm_splitk_plan(8, 8, 128, policy=q.qmm_policy(32, 32, 320, 0, 128))
    assert e.value.status == q.QMM_ERR_ARG


def _w4(**kw):
    a = dict(A=ADDR, Wq=ADDR2, scale=ADDR3, bias=ADDR3 + 4096, C=ADDR + 0x100000, M=32, N=1024, K=2560, s=1,
             workspace=None, workspace_bytes=0)
    a.update(kw)
    return q.qmm_w4a16_g128(a["A"], a["Wq"], a["scale"], a["bias"], a["C"], a["M"], a["N"], a["K"], a["s"],
                            a["workspace"], a["workspace_bytes"], stream=0, check=False)


@pytest.mark.parametrize("kw,code", [
    (dict(A=None), q.QMM_ERR_ARG), (dict(Wq=None), q.QMM_ERR_ARG), (dict(scale=None), q.QMM_ERR_ARG),
    (dict(bias=None), q.QMM_ERR_ARG), (dict(C=None), q.QMM_ERR_ARG),
    (dict(M=0), q.QMM_ERR_ARG), (dict(N=-1), q.QMM_ERR_ARG), (dict(K=0), q.QMM_ERR_ARG), (dict(s=-1), q.QMM_ERR_ARG),
    (dict(K=2500), q.QMM_ERR_SHAPE), (dict(s=21), q.QMM_ERR_SHAPE), (dict(s=40), q.QMM_ERR_SHAPE),
    (dict(A=ADDR + 8), q.QMM_ERR_ALIGN), (dict(Wq=ADDR2 + 4), q.QMM_ERR_ALIGN), (dict(C=ADDR + 1), q.QMM_ERR_ALIGN),
    (dict(scale=ADDR3 + 1), q.QMM_ERR_ALIGN),
    (dict(s=4), q.QMM_ERR_WORKSPACE),
    (dict(s=4, workspace=ADDR + 0x200000, workspace_bytes=2 * 4 * 32 * 1024 - 2), q.QMM_ERR_WORKSPACE),
    (dict(s=4, workspace=ADDR + 0x200008, workspace_bytes=2 * 4 * 32 * 1024), q.QMM_ERR_ALIGN),
    (dict(M=1 << 30, N=1 << 30), q.QMM_ERR_SIZE),
])
def test_w4a16_rejects_before_launch(kw, code):
    assert _w4(**kw) == code


def _w4f(**kw):
    a = dict(A=ADDR, Wq=ADDR2, scale=ADDR3, bias=ADDR3 + 4096, C=ADDR + 0x100000, M=32, N=1024, K=2560, s=1,
             workspace=None, workspace_bytes=0)
    a.update(kw)
    return q.qmm_w4a16_g128_f32p(a["A"], a["Wq"], a["scale"], a["bias"], a["C"], a["M"], a["N"], a["K"], a["s"],
                                 a["workspace"], a["workspace_bytes"], stream=0, check=False)


@pytest.mark.parametrize("kw,code", [
    (dict(A=None), q.QMM_ERR_ARG), (dict(s=-1), q.QMM_ERR_ARG), (dict(K=2500), q.QMM_ERR_SHAPE),
    (dict(s=21), q.QMM_ERR_SHAPE), (dict(A=ADDR + 8), q.QMM_ERR_ALIGN), (dict(s=4), q.QMM_ERR_WORKSPACE),
    # fp32 planes: the bf16-sized workspace is too small by half
    (dict(s=4, workspace=ADDR + 0x200000, workspace_bytes=2 * 4 * 32 * 1024), q.QMM_ERR_WORKSPACE),
    (dict(s=4, workspace=ADDR + 0x200000, workspace_bytes=4 * 4 * 32 * 1024 - 4), q.QMM_ERR_WORKSPACE),
    (dict(s=4, workspace=ADDR + 0x200008, workspace_bytes=4 * 4 * 32 * 1024), q.QMM_ERR_ALIGN),
    (dict(M=1 << 30, N=1 << 30), q.QMM_ERR_SIZE),
])
def test_w4a16_f32p_rejects_before_launch(kw, code):
    assert _w4f(**kw) == code


def _w4p(**kw):
    a = dict(A=ADDR, Wq=ADDR2, scale=ADDR3, bias=ADDR3 + 4096, C=ADDR + 0x100000, M=32, N=1024, K=2560, s=1,
             workspace=None, workspace_bytes=0)
    a.update(kw)
    rc, _, _ = q.qmm_w4a16_g128_pass1(a["A"], a["Wq"], a["scale"], a["bias"], a["C"], a["M"], a["N"], a["K"],
                                      a["s"], a["workspace"], a["workspace_bytes"], stream=0, check=False)
    return rc


@pytest.mark.parametrize("kw,code", [
    (dict(A=None), q.QMM_ERR_ARG), (dict(s=-1), q.QMM_ERR_ARG), (dict(K=2500), q.QMM_ERR_SHAPE),
    (dict(s=21), q.QMM_ERR_SHAPE), (dict(A=ADDR + 8), q.QMM_ERR_ALIGN), (dict(s=4), q.QMM_ERR_WORKSPACE),
    (dict(s=4, workspace=ADDR2 + 8, workspace_bytes=1 << 30), q.QMM_ERR_ALIGN), (dict(K=1 << 22), q.QMM_ERR_SIZE),
])
def test_w4a16_pass1_rejects_before_launch(kw, code):
    # the same checks as qmm_w4a16_g128, all on the host
    assert _w4p(**kw) == code


def test_w4a16_pass1_needs_its_outputs():
    f = q.lib().qmm_w4a16_g128_pass1
    rc = f(ADDR, ADDR2, ADDR3, ADDR3 + 4096, ADDR + 0x100000, 32, 1024, 2560, 1, None, 0, None, None, None)
    assert rc == q.QMM_ERR_ARG


@pytest.mark.parametrize("args,code", [
    ((None, 0, 2, 4, 64, 0, ADDR), q.QMM_ERR_ARG), ((ADDR, 2, 2, 4, 64, 0, ADDR), q.QMM_ERR_ARG),
    ((ADDR, 0, 0, 4, 64, 0, ADDR), q.QMM_ERR_ARG), ((ADDR, 0, 2, 4, 64, -1, ADDR), q.QMM_ERR_ARG),
    ((ADDR, 0, 2, 4, 64, 64, ADDR), q.QMM_ERR_ARG), ((ADDR, 0, 2, 0, 64, 0, ADDR), q.QMM_ERR_ARG),
    ((ADDR + 1, 0, 2, 4, 64, 0, ADDR), q.QMM_ERR_ALIGN), ((ADDR + 2, 1, 2, 4, 64, 0, ADDR), q.QMM_ERR_ALIGN),
    ((ADDR, 0, 2, 4, 64, 0, ADDR + 1), q.QMM_ERR_ALIGN),
])
def test_reduce_cols_rejects_before_launch(args, code):
    assert q.qmm_splitk_reduce_cols(*args, stream=0, check=False) == code


def _wn(bits=8, group=64, dt=0, **kw):
    a = dict(A=ADDR, Wq=ADDR2, scale=ADDR3, bias=ADDR3 + 4096, C=ADDR + 0x100000, M=32, N=1024, K=2560, s=1,
             workspace=None, workspace_bytes=0)
    a.update(kw)
    return q.qmm_wna16(bits, group, dt, a["A"], a["Wq"], a["scale"], a["bias"], a["C"], a["M"], a["N"], a["K"],
                       a["s"], a["workspace"], a["workspace_bytes"], stream=0, check=False)


@pytest.mark.parametrize("fmt,kw,code", [
    (dict(bits=5), {}, q.QMM_ERR_ARG), (dict(bits=2), {}, q.QMM_ERR_ARG), (dict(group=16), {}, q.QMM_ERR_ARG),
    (dict(group=256), {}, q.QMM_ERR_ARG), (dict(group=96), {}, q.QMM_ERR_ARG), (dict(dt=2), {}, q.QMM_ERR_ARG),
    ({}, dict(A=None), q.QMM_ERR_ARG), ({}, dict(K=2560 + 64), q.QMM_ERR_SHAPE), ({}, dict(s=21), q.QMM_ERR_SHAPE),
    ({}, dict(A=ADDR + 8), q.QMM_ERR_ALIGN), ({}, dict(s=4), q.QMM_ERR_WORKSPACE),
    (dict(dt=1), dict(s=4, workspace=ADDR + 0x200000, workspace_bytes=2 * 4 * 32 * 1024), q.QMM_ERR_WORKSPACE),
    ({}, dict(s=4, workspace=ADDR + 0x200000, workspace_bytes=2 * 4 * 32 * 1024 - 2), q.QMM_ERR_WORKSPACE),
    ({}, dict(M=1 << 30, N=1 << 30), q.QMM_ERR_SIZE),
])
def test_wna16_rejects_before_launch(fmt, kw, code):
    assert _wn(**fmt, **kw) == code


def test_wna16_plan_rejects_unsupported_formats():
    for bits, group in [(5, 128), (8, 16), (4, 256), (16, 128)]:
        with pytest.raises(q.QmmError) as e:
            q.qmm_wna16_plan(bits, group, 16, 1024, 2560)
        assert e.value.status == q.QMM_ERR_ARG


def test_attn_split_rule():
    # one workgroup per CU, at most one split per 64-key tile, past 16 splits (one merge
    # batch) only with 512 keys per split, at most 32
    for B, Hkv, L in [(1, 8, 4096), (1, 8, 1024), (1, 8, 2048), (1, 8, 16384), (2, 8, 2048), (4, 8, 1024),
                      (8, 8, 4096), (32, 8, 16384), (1, 1, 100), (1, 1, 63), (64, 8, 65536), (1, 2, 12800)]:
        want = max(1, min(32, -(-256 // (B * Hkv)), L // 64, max(16, L // 512)))
        assert q.qmm_attn_decode_split(B, Hkv, L) == want, (B, Hkv, L)
    # the Qwen3-4B single-request cases the rule was fitted on
    assert [q.qmm_attn_decode_split(1, 8, L) for L in (1024, 2048, 4096, 16384)] == [16, 16, 16, 32]
    assert q.qmm_attn_decode_workspace_bytes(2, 1, 32, 4) == 4 * 2 * 32 * 130 * 4
    assert q.qmm_attn_decode_workspace_bytes(2, 1, 32, 1) == 0


def _at(**kw):
    a = dict(Q=ADDR, K=ADDR2, V=ADDR3, lengths=ADDR + 0x400000, O=ADDR + 0x100000, B=2, Mq=1, Hq=32, Hkv=8,
             Lmax=1024, D=128, scale=0.088, s=1, workspace=None, workspace_bytes=0)
    a.update(kw)
    return q.qmm_attn_decode(a["Q"], a["K"], a["V"], a["lengths"], a["O"], a["B"], a["Mq"], a["Hq"], a["Hkv"],
                             a["Lmax"], a["D"], a["scale"], a["s"], a["workspace"], a["workspace_bytes"], stream=0,
                             check=False)


@pytest.mark.parametrize("kw,code", [
    (dict(Q=None), q.QMM_ERR_ARG), (dict(lengths=None), q.QMM_ERR_ARG), (dict(B=0), q.QMM_ERR_ARG),
    (dict(s=-1), q.QMM_ERR_ARG), (dict(scale=float("nan")), q.QMM_ERR_ARG), (dict(scale=float("inf")), q.QMM_ERR_ARG),
    (dict(D=64), q.QMM_ERR_SHAPE), (dict(Hq=30), q.QMM_ERR_SHAPE), (dict(Mq=5), q.QMM_ERR_SHAPE),
    (dict(Mq=4, Lmax=3), q.QMM_ERR_SHAPE), (dict(s=65), q.QMM_ERR_SHAPE),
    (dict(Q=ADDR + 8), q.QMM_ERR_ALIGN), (dict(O=ADDR + 0x100002), q.QMM_ERR_ALIGN),
    (dict(lengths=ADDR + 0x400002), q.QMM_ERR_ALIGN), (dict(s=4), q.QMM_ERR_WORKSPACE),
    (dict(s=4, workspace=ADDR + 0x800000, workspace_bytes=4 * 2 * 32 * 130 * 4 - 4), q.QMM_ERR_WORKSPACE),
    (dict(s=4, workspace=ADDR + 0x800008, workspace_bytes=4 * 2 * 32 * 130 * 4), q.QMM_ERR_ALIGN),
    (dict(B=1 << 20, Lmax=1 << 12), q.QMM_ERR_SIZE),
])
def test_attn_rejects_before_launch(kw, code):
    assert _at(**kw) == code


def _sk(**kw):
    a = dict(A=ADDR, Wq=ADDR2, scale=ADDR3, bias=ADDR3 + 4096, C=ADDR + 0x100000, M=300, N=520, K=1024, P=0,
             workspace=ADDR + 0x2000000, workspace_bytes=1 << 30)
    a.update(kw)
    return q.qmm_w4a16_g128_streamk(a["A"], a["Wq"], a["scale"], a["bias"], a["C"], a["M"], a["N"], a["K"], a["P"],
                                    a["workspace"], a["workspace_bytes"], stream=0, check=False)


@pytest.mark.parametrize("kw,code", [
    (dict(A=None), q.QMM_ERR_ARG), (dict(P=-1), q.QMM_ERR_ARG), (dict(M=0), q.QMM_ERR_ARG),
    (dict(M=64), q.QMM_ERR_SHAPE), (dict(K=1000), q.QMM_ERR_SHAPE),
    (dict(P=2 * 3 * 8 + 1), q.QMM_ERR_SHAPE),  # 2 x 3 tiles of 256 x 256, 8 blocks: 48 units
    (dict(workspace=None), q.QMM_ERR_WORKSPACE),
    (dict(P=7, workspace_bytes=2 * 7 * 256 * 256 * 2 - 2), q.QMM_ERR_WORKSPACE),
    (dict(workspace=ADDR + 0x2000008), q.QMM_ERR_ALIGN), (dict(A=ADDR + 8), q.QMM_ERR_ALIGN),
])
def test_streamk_rejects_before_launch(kw, code):
    assert _sk(**kw) == code


def test_streamk_workspace_sizes():
    assert q.qmm_streamk_workspace_bytes(300, 520, 1024, 7) == 2 * 7 * 256 * 256 * 2
    assert q.qmm_streamk_workspace_bytes(300, 520, 1024, 0) == 2 * 12 * 256 * 256 * 2  # 48 units, 4 per group
    assert q.qmm_streamk_workspace_bytes(100, 4096, 2560, 0) == 2 * 80 * 128 * 256 * 2  # 16 tiles x 20 blocks / 4
    assert q.qmm_streamk_workspace_bytes(100, 9728, 2560, 0) == 2 * 190 * 128 * 256 * 2  # 760 units / 4
    assert q.qmm_streamk_workspace_bytes(2048, 9728, 2560, 0) == 2 * 256 * 256 * 256 * 2
    assert q.qmm_streamk_workspace_bytes(64, 1024, 2560, 0) == 0
    assert _sk(P=7, workspace_bytes=2 * 7 * 256 * 256 * 2, C=None) == q.QMM_ERR_ARG


def test_w4a16_workspace_sizes():
    assert q.w4a16_workspace_bytes(32, 1024, 1) == 0
    assert q.w4a16_workspace_bytes(32, 1024, 4) == 2 * 4 * 32 * 1024
    assert q.w4a16_workspace_bytes(32, 1024, 4, f32_partials=True) == 4 * 4 * 32 * 1024


def test_w4a16_policy_split_needs_workspace():
    # s = 0 resolves through the MI355X plan; where it splits, no workspace is an error
    M, N, K = 16, 1024, 2560
    if q.qmm_splitk_plan(M, N, K).s > 1:
        assert _w4(M=M, N=N, K=K, s=0) == q.QMM_ERR_WORKSPACE


@pytest.mark.parametrize("args,code", [
    ((None, 0, 2, 4, 4, ADDR), q.QMM_ERR_ARG), ((ADDR, 0, 2, 4, 4, None), q.QMM_ERR_ARG),
    ((ADDR, 2, 2, 4, 4, ADDR2), q.QMM_ERR_ARG), ((ADDR, 0, 0, 4, 4, ADDR2), q.QMM_ERR_ARG),
    ((ADDR, 0, 2, 0, 4, ADDR2), q.QMM_ERR_ARG), ((ADDR + 1, 0, 2, 4, 4, ADDR2), q.QMM_ERR_ALIGN),
    ((ADDR + 2, 1, 2, 4, 4, ADDR2), q.QMM_ERR_ALIGN), ((ADDR, 0, 2, 4, 4, ADDR2 + 1), q.QMM_ERR_ALIGN),
])
def test_reduce_rejects_before_launch(args, code):
    assert q.qmm_splitk_reduce(*args, stream=0, check=False) == code


def _gemv_min_split_rule(M, K):
    """The documented rule of qmm_gemv_min_split, restated."""
    m8 = 1 if M <= 1 else 2 if M <= 2 else 4 if M <= 4 else 8
    G = K // 128
    for s in range(1, G + 1):
        kp = K // s
        if G % s == 0 and kp <= 10240 and m8 * kp <= 30720 and (m8 < 8 or kp <= 4096):
            return s
    return None


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 8])
@pytest.mark.parametrize("K", [128, 2560, 4096, 9728, 12288, 30720, 65536])
def test_gemv_min_split_rule(M, K):
    want = _gemv_min_split_rule(M, K)
    if want is None:
        with pytest.raises(q.QmmError):
            q.qmm_gemv_min_split(M, K)
    else:
        assert q.qmm_gemv_min_split(M, K) == want


def test_gemv_min_split_cases():
    # decode shapes: down (K 9728) and gate (K 2560) at M = 1, 4, 8
    assert [q.qmm_gemv_min_split(M, 9728) for M in (1, 4, 8)] == [1, 2, 4]
    assert [q.qmm_gemv_min_split(M, 2560) for M in (1, 4, 8)] == [1, 1, 1]
    for args, code in [((0, 256), q.QMM_ERR_ARG), ((9, 256), q.QMM_ERR_SHAPE), ((1, 200), q.QMM_ERR_SHAPE)]:
        assert q.lib().qmm_gemv_min_split(*args) == code


@pytest.mark.parametrize("kw,code", [
    (dict(A=None), q.QMM_ERR_ARG), (dict(C=None), q.QMM_ERR_ARG), (dict(M=0), q.QMM_ERR_ARG),
    (dict(M=9), q.QMM_ERR_SHAPE), (dict(K=200), q.QMM_ERR_SHAPE), (dict(s=3), q.QMM_ERR_SHAPE),
    (dict(M=8, K=9728, s=1), q.QMM_ERR_SHAPE),  # 9728 values do not fit for 8 rows
    (dict(s=2), q.QMM_ERR_WORKSPACE), (dict(A=ADDR + 2), q.QMM_ERR_ALIGN),
    (dict(s=2, workspace=ADDR3, workspace_bytes=2 * 2 * 4 * 1024 - 2), q.QMM_ERR_WORKSPACE),
])
def test_gemv_rejects_before_launch(kw, code):
    a = dict(A=ADDR, Wq=ADDR2, scale=ADDR3, bias=ADDR3 + 4096, C=ADDR + 0x100000, M=4, N=1024, K=2560, s=1,
             workspace=None, workspace_bytes=0)
    a.update(kw)
    rc = q.qmm_w4a16_gemv(a["A"], a["Wq"], a["scale"], a["bias"], a["C"], a["M"], a["N"], a["K"], a["s"],
                          a["workspace"], a["workspace_bytes"], stream=0, check=False)
    assert rc == code


@pytest.mark.parametrize("kw,code", [
    (dict(A=None), q.QMM_ERR_ARG), (dict(B=None), q.QMM_ERR_ARG), (dict(C=None), q.QMM_ERR_ARG),
    (dict(K=100), q.QMM_ERR_SHAPE), (dict(s=257), q.QMM_ERR_SHAPE), (dict(K=32 * 71, s=72), q.QMM_ERR_SHAPE),
    (dict(M=-2), q.QMM_ERR_ARG),
    (dict(A=ADDR + 4), q.QMM_ERR_ALIGN), (dict(s=4), q.QMM_ERR_WORKSPACE),
    (dict(s=4, workspace=ADDR3, workspace_bytes=4 * 4 * 512 * 512 - 4), q.QMM_ERR_WORKSPACE),
])
def test_dense_rejects_before_launch(kw, code):
    a = dict(A=ADDR, B=ADDR2, C=ADDR + 0x100000, M=512, N=512, K=16384, s=1, workspace=None, workspace_bytes=0)
    a.update(kw)
    rc = q.qmm_bf16_splitk(a["A"], a["B"], a["C"], a["M"], a["N"], a["K"], a["s"], a["workspace"],
                           a["workspace_bytes"], stream=0, check=False)
    assert rc == code


def test_decode_tile_rule_edges():
    """The plan's tile at the decode rule's edges (the GPU edge-shape tests run these shapes against the oracle)."""
    tiles = {(M, N, K): (p.block_m, p.tile_n, p.s, p.block_n) for M, N, K in [(8, 4096, 8192), (9, 4096, 8192),
                                                                            (5, 4097, 8192), (7, 2500, 9728)]
             for p in [q.qmm_splitk_plan(M, N, K)]}
    assert tiles[(8, 4096, 8192)][:2] == (16, 16) and tiles[(7, 2500, 9728)][:2] == (16, 16)
    assert tiles[(9, 4096, 8192)][1] != 16 and tiles[(5, 4097, 8192)][1] != 16
    # 256 16-column tiles fill the CUs as they are; 157 of them run as 250 tiles of 10 columns
    assert tiles[(8, 4096, 8192)][3] == 16 and tiles[(7, 2500, 9728)][2:] == (1, 10)


# Small-M tile choices around the 16-row rules, derived by hand (T16 = ceil(M/16) * ceil(N/16)
# and T64 = ceil(M/16) * ceil(N/64) 16-row tiles; one round = 256 workgroups):
#   (64, 1024, 2560): T16 = 4 * 64 = 256 <= 256          -> 16 x 16 tiles, unsplit, 256 workgroups
#   (32, 1024, 2560): T16 = 2 * 64 = 128, narrowed to 256 // 2 = 128 tiles per row block of
#                     ceil(1024 / 128) = 8 columns            -> 16 x 8, unsplit
#   (65, 1024, 2560): M > 64                              -> not a 16-row tile (32 x 16)
#   (64, 4096, 2560): T16 = 1024; T64 = 4 * 64 = 256 >= 192 -> 16 x 64 tiles, unsplit
#   (48, 4096, 2560): T64 = 3 * 64 = 192 = 3/4 of a round  -> 16 x 64 tiles, unsplit
#   (32, 4096, 2560): T64 = 2 * 64 = 128 < 192             -> 32-row tiles of 16 columns (256 of them)
#   (64, 4160, 2560): T64 = 4 * 65 = 260 > 256             -> not a 16-row tile
#   (64, 9728, 2560): N*K > 2^24                           -> not a 16-row tile
#   (128, 1024, 2560): M > 64, ceil(128/32) * 64 = 256 <= 256  -> 32 x 16 tiles, unsplit
#   (96, 1024, 2560): 3 * 64 = 192, narrowed to 256 // 3 = 85 tiles per row block of
#                     ceil(1024 / 85) = 13 columns           -> 32 x 13, unsplit
SMALL_HAND = [((128, 1024, 2560), (32, 16, 1, 64, 4)), ((96, 1024, 2560), (32, 13, 1, 79, 3)),
              ((64, 1024, 2560), (16, 16, 1, 64, 4)), ((32, 1024, 2560), (16, 8, 1, 128, 2)),
              ((64, 4096, 2560), (16, 64, 1, 64, 4)), ((48, 4096, 2560), (16, 64, 1, 64, 3)),
              ((32, 4096, 2560), (32, 16, 1, 256, 1))]


def test_small_m_sixteen_row_tiles_hand_derived():
    for (M, N, K), want in SMALL_HAND:
        p = q.qmm_splitk_plan(M, N, K)
        assert (p.block_m, p.block_n, p.s, p.grid_x, p.grid_y) == want, (M, N, K, p.as_dict())
    for M, N, K in ((65, 1024, 2560), (64, 4160, 2560), (64, 9728, 2560)):
        assert q.qmm_splitk_plan(M, N, K).block_m != 16, (M, N, K)
    assert q.qmm_splitk_plan(129, 1024, 2560).block_m >= 128  # past 128 rows: the large-M kernel
