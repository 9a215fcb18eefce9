"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Every case uses the seeded inputs of qmm_synth, runs the library through its
ctypes binding on the current torch stream, and compares with the oracle:
  * split and unsplit W4A16 results within |gpu-ref| <= 0.02|ref| + 0.02 rms(ref);
  * the s = 1 fallback bitwise equal to the explicit unsplit kernel;
  * the reduce kernel bitwise equal to the oracle's fp32 sum + one bf16 cast;
  * closed forms that are exact in bf16 (zero weights, one-hot rows) bitwise;
  * determinism and untouched guard bands around C and the workspace.
"""
import numpy as np
import pytest
import torch

import oracle
import qmm_synth as syn
import weight_only_quantized_qmm_amd as q
from gpu_util import check_tolerance, dev_bf16, dev_u32, host_bits, host_f64, w4a16_device

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)


def run_w4a16(dv, M, N, K, s, guard=0, f32p=False):
    """Run the library (qmm_w4a16_g128, or qmm_w4a16_g128_f32p when f32p); returns C (bf16
    device tensor). guard > 0 wraps C and the workspace in canary regions of that many
    elements and checks them afterwards."""
    s_eff = q.effective_split(M, N, K, s)
    Cbuf = torch.full((M * N + 2 * guard,), -12345.0, dtype=torch.bfloat16, device="cuda")
    C = Cbuf[guard:guard + M * N].view(M, N)
    ws = None
    wbuf = None
    wdt = torch.float32 if f32p else torch.bfloat16
    if s_eff > 1:
        nws = s_eff * M * N
        gw = ((guard + 7) // 8) * 8  # keep the workspace 16-byte aligned
        wbuf = torch.full((nws + 2 * gw,), -777.0, dtype=wdt, device="cuda")
        ws = wbuf[gw:gw + nws]
    fn = q.qmm_w4a16_g128_f32p if f32p else q.qmm_w4a16_g128
    fn(dv["A"], dv["Wq"], dv["scale"], dv["bias"], C, M, N, K, s, ws)
    torch.cuda.synchronize()
    if guard:
        g = host_bits(Cbuf)
        canary = host_bits(torch.tensor([-12345.0], dtype=torch.bfloat16))[0]
        assert np.all(g[:guard] == canary) and np.all(g[guard + M * N:] == canary), "C guard band written"
        if wbuf is not None:
            w = wbuf.cpu().numpy() if f32p else host_bits(wbuf)
            wc = (np.float32(-777.0) if f32p else host_bits(torch.tensor([-777.0], dtype=torch.bfloat16))[0])
            assert np.all(w[:gw] == wc) and np.all(w[gw + s_eff * M * N:] == wc), "workspace guard written"
    return C


# ------------------------------------------------------------------ config 0 / 1

@pytest.fixture(scope="module")
def cfg0():
    M, N, K = 32, 1024, 2560
    d = syn.w4a16_inputs(M, N, K, seed=0)
    return M, N, K, d, oracle.qmm_w4a16(d["A"], d["Wq"], d["scale"], d["bias"], M, N, K)


@pytest.mark.parametrize("s", [1, 4, 0])
def test_cfg0_k_projection(cfg0, s):
    M, N, K, d, ref = cfg0
    say("cfg0 M=%d N=%d K=%d s=%d" % (M, N, K, s))
    C = run_w4a16(w4a16_device(d), M, N, K, s, guard=64)
    check_tolerance(host_f64(C), ref, what="cfg0 s=%d" % s)


@pytest.fixture(scope="module")
def cfg1():
    M, N, K = 48, 1000, 2560
    d = syn.w4a16_inputs(M, N, K, seed=1000)
    return M, N, K, d, oracle.qmm_w4a16(d["A"], d["Wq"], d["scale"], d["bias"], M, N, K)


@pytest.mark.parametrize("s", [1, 2, 4, 5, 10, 20])
def test_cfg1_partial_tile_split_sweep(cfg1, s):
    M, N, K, d, ref = cfg1
    say("cfg1 M=%d N=%d K=%d s=%d" % (M, N, K, s))
    C = run_w4a16(w4a16_device(d), M, N, K, s, guard=64)
    check_tolerance(host_f64(C), ref, what="cfg1 s=%d" % s)


def test_cfg1_unsplit_equals_policy_when_policy_is_one(cfg1):
    M, N, K, d, _ = cfg1
    dv = w4a16_device(d)
    a = host_bits(run_w4a16(dv, M, N, K, 1))
    b = host_bits(run_w4a16(dv, M, N, K, 1))
    assert np.array_equal(a, b)


# ------------------------------------------------------------- config 2 (sweep)

SWEEP = syn.projection_sweep()


@pytest.mark.parametrize("name,M,N,K,idx", SWEEP, ids=["%s-M%d" % (n, m) for n, m, _, _, _ in SWEEP])
def test_cfg2_projection_sweep(name, M, N, K, idx):
    seed = 2000 + idx
    d = syn.w4a16_inputs(M, N, K, seed=seed)
    dv = w4a16_device(d)
    s_pol = q.effective_split(M, N, K, 0)
    say("cfg2 %s M=%d N=%d K=%d policy s=%d" % (name, M, N, K, s_pol))
    C = run_w4a16(dv, M, N, K, 0)
    C1 = run_w4a16(dv, M, N, K, 1)
    got, got1 = host_f64(C), host_f64(C1)
    # every output element against the oracle, at full size (M = 2048 included)
    ref = oracle.qmm_w4a16(d["A"], d["Wq"], d["scale"], d["bias"], M, N, K)
    check_tolerance(got, ref, what="%s M=%d policy" % (name, M))
    check_tolerance(got1, ref, what="%s M=%d unsplit" % (name, M))
    if s_pol == 1:
        # the policy's fallback is the unsplit kernel, bit for bit
        assert np.array_equal(host_bits(C), host_bits(C1))


# Explicit splits that do not divide the group count: partition p covers groups
# [floor(p*G/s), floor((p+1)*G/s)) on both matmul kernels (small-M kernel: 48 and 100 rows;
# large-M kernel: 128 x 128 tiles at 128 rows, 256 x 256 tiles at 300 rows).
NONDIV_CASES = [(48, 1000, 2560, (3, 7, 9, 13)), (100, 1000, 2560, (3, 6)), (128, 9728, 2560, (3, 7)),
                (300, 520, 1024, (3, 5))]


@pytest.mark.parametrize("M,N,K,splits", NONDIV_CASES)
def test_non_divisor_splits_match_oracle(M, N, K, splits):
    d = syn.w4a16_inputs(M, N, K, seed=18500 + M)
    ref = oracle.qmm_w4a16(d["A"], d["Wq"], d["scale"], d["bias"], M, N, K)
    dv = w4a16_device(d)
    G = K // 128
    for s in splits:
        assert G % s != 0
        for f32p in (False, True):
            say("non-divisor split M=%d N=%d K=%d s=%d f32p=%d" % (M, N, K, s, f32p))
            C = run_w4a16(dv, M, N, K, s, guard=40, f32p=f32p)
            check_tolerance(host_f64(C), ref, what="%dx%dx%d s=%d f32p=%d" % (M, N, K, s, f32p))


def test_explicit_split_reproduces_the_plan():
    """gate at M = 128: the plan splits every 128 x 128 tile in 3 (20 groups: 6, 7, 7);
    the same s passed explicitly is the same launch, bit for bit."""
    M, N, K = 128, 9728, 2560
    plan = q.qmm_splitk_plan(M, N, K)
    assert (plan.s, plan.full_tiles) == (3, 0)
    dv = w4a16_device(syn.w4a16_inputs(M, N, K, seed=18600))
    say("explicit s=3 against the plan M=%d N=%d K=%d" % (M, N, K))
    a = host_bits(run_w4a16(dv, M, N, K, 0))
    b = host_bits(run_w4a16(dv, M, N, K, 3))
    assert np.array_equal(a, b)


# Shapes the plan runs on 128 x 128 tiles of the large-M kernel (a pure split): ragged M
# below and above 128 rows, N not a multiple of 128 (and of 8: element-wise stores).
TILE128_CASES = [(100, 7000, 2560), (300, 300, 1024), (256, 520, 4096), (130, 1000, 3072)]


@pytest.mark.parametrize("M,N,K", TILE128_CASES)
def test_128x128_tiles_match_oracle(M, N, K):
    plan = q.qmm_splitk_plan(M, N, K)
    assert (plan.block_m, plan.block_n, plan.full_tiles) == (128, 128, 0) and plan.s > 1, plan.as_dict()
    d = syn.w4a16_inputs(M, N, K, seed=18000 + M + N)
    ref = oracle.qmm_w4a16(d["A"], d["Wq"], d["scale"], d["bias"], M, N, K)
    dv = w4a16_device(d)
    for s, f32p in ((0, False), (1, False), (2, False), (4, False), (0, True)):
        say("128x128 tiles M=%d N=%d K=%d s=%d f32p=%d" % (M, N, K, s, f32p))
        C = run_w4a16(dv, M, N, K, s, guard=40, f32p=f32p)
        check_tolerance(host_f64(C), ref, what="128x128 tiles %dx%dx%d s=%d f32p=%d" % (M, N, K, s, f32p))


def test_split_tail_decomposition():
    """Large-M plan that runs most tiles unsplit and splits only the last column of tiles
    (ragged in N): the unsplit columns equal the s = 1 kernel bit for bit, the split tail
    is within tolerance of the oracle, and nothing outside C is written."""
    M, N, K = 1000, 64 * 256 + 100, 2560
    plan = q.qmm_splitk_plan(M, N, K)
    say("split tail M=%d N=%d K=%d s=%d full_tiles=%d" % (M, N, K, plan.s, plan.full_tiles))
    assert plan.s > 1 and 0 < plan.full_tiles < plan.base_tiles
    n_lo = (plan.full_tiles // -(-M // plan.block_m)) * plan.block_n
    d = syn.w4a16_inputs(M, N, K, seed=7200)
    dv = w4a16_device(d)
    C = run_w4a16(dv, M, N, K, 0, guard=64)
    C1 = run_w4a16(dv, M, N, K, 1)
    bits, bits1 = host_bits(C), host_bits(C1)
    assert np.array_equal(bits[:, :n_lo], bits1[:, :n_lo])
    ref = oracle.qmm_w4a16(d["A"], d["Wq"], d["scale"], d["bias"], M, N, K)
    got = host_f64(C)
    check_tolerance(got[:, n_lo:], ref[:, n_lo:], rms=float(np.sqrt(np.mean(ref * ref))), what="split tail columns")
    check_tolerance(got, ref, what="split tail, whole output")


# ------------------------------------------------------- stream-K decomposition

def streamk_whole_tiles(T, G, P):
    """Tiles a single workgroup covers whole under the near-equal unit ranges."""
    U = T * G
    whole = []
    for w in range(P):
        u0, u1 = w * U // P, (w + 1) * U // P
        t_first = -(-u0 // G)              # first tile starting at or after u0
        t_last = u1 // G                   # tiles ending at or before u1
        whole += list(range(t_first, t_last))
    return sorted(set(whole))


def run_streamk(dv, M, N, K, P, guard=0):
    nbytes = q.qmm_streamk_workspace_bytes(M, N, K, P)
    Cbuf = torch.full((M * N + 2 * guard,), -12345.0, dtype=torch.bfloat16, device="cuda")
    C = Cbuf[guard:guard + M * N].view(M, N)
    gw = 64
    wbuf = torch.full((nbytes // 2 + 2 * gw,), -777.0, dtype=torch.bfloat16, device="cuda")
    q.qmm_w4a16_g128_streamk(dv["A"], dv["Wq"], dv["scale"], dv["bias"], C, M, N, K, P, wbuf[gw:gw + nbytes // 2],
                             nbytes)
    torch.cuda.synchronize()
    if guard:
        g = host_bits(Cbuf)
        canary = host_bits(torch.tensor([-12345.0], dtype=torch.bfloat16))[0]
        assert np.all(g[:guard] == canary) and np.all(g[guard + M * N:] == canary), "C guard band written"
        w = host_bits(wbuf)
        wc = host_bits(torch.tensor([-777.0], dtype=torch.bfloat16))[0]
        assert np.all(w[:gw] == wc) and np.all(w[gw + nbytes // 2:] == wc), "workspace guard written"
    return C


@pytest.mark.parametrize("M,N,K,Ps", [
    (100, 1000, 2560, (1, 7, 64, 80, 0)),      # 128-row tiles: 4 tiles x 20 blocks
    (300, 520, 1024, (1, 5, 13, 48, 0)),       # 256-row tiles, ragged M and N: 6 tiles x 8 blocks
    (520, 300, 1280, (3, 11, 29, 0)),
])
def test_streamk_matches_oracle(M, N, K, Ps):
    d = syn.w4a16_inputs(M, N, K, seed=17000 + M)
    ref = oracle.qmm_w4a16(d["A"], d["Wq"], d["scale"], d["bias"], M, N, K)
    dv = w4a16_device(d)
    BM = 128 if M <= 128 else 256
    num_m, num_n, G = -(-M // BM), -(-N // 256), K // 128
    # one workgroup per tile: every tile whole, the large-M kernel's unsplit decomposition
    # (the same launch as s = 1 where the plan runs that kernel)
    c1 = host_bits(run_streamk(dv, M, N, K, num_m * num_n))
    plan = q.qmm_splitk_plan(M, N, K)
    if (plan.block_m, plan.block_n) == (BM, 256):  # s = 1 runs the same tiles
        assert np.array_equal(c1, host_bits(run_w4a16(dv, M, N, K, 1)))
    for P in Ps:
        Peff = P or max(1, min(num_m * num_n * G // min(4, G), 256 * (2 if BM == 128 else 1)))
        say("streamk M=%d N=%d K=%d P=%d" % (M, N, K, Peff))
        C = run_streamk(dv, M, N, K, P, guard=64)
        check_tolerance(host_f64(C), ref, what="stream-K P=%d" % Peff)
        bits = host_bits(C)
        for t in streamk_whole_tiles(num_m * num_n, G, Peff):
            r0, c0 = (t % num_m) * BM, (t // num_m) * 256
            blk = (slice(r0, min(r0 + BM, M)), slice(c0, min(c0 + 256, N)))
            assert np.array_equal(bits[blk], c1[blk]), "tile %d covered whole differs from the unsplit kernel" % t


def test_streamk_full_size():
    M, N, K = 2048, 2560, 9728  # the down projection: 80 tiles x 76 blocks on 256 workgroups
    d = syn.w4a16_inputs(M, N, K, seed=17500)
    dv = w4a16_device(d)
    say("streamk full size M=%d N=%d K=%d" % (M, N, K))
    C = host_f64(run_streamk(dv, M, N, K, 0, guard=64))
    ref = oracle.qmm_w4a16(d["A"], d["Wq"], d["scale"], d["bias"], M, N, K)
    check_tolerance(C, ref, what="stream-K down M=2048")


@pytest.mark.parametrize("name,M,N,K", [("gate", 2048, 9728, 2560), ("down", 2048, 2560, 9728),
                                         ("down", 128, 2560, 9728)])
def test_f32p_full_size(name, M, N, K):
    """fp32 partial planes under the plan at full projection sizes (the split tail of gate
    at M = 2048, three and twelve partitions of down), every element against the oracle."""
    d = syn.w4a16_inputs(M, N, K, seed=17600 + M)
    dv = w4a16_device(d)
    say("f32p full size %s M=%d N=%d K=%d s=%d" % (name, M, N, K, q.effective_split(M, N, K, 0)))
    C = host_f64(run_w4a16(dv, M, N, K, 0, guard=64, f32p=True))
    ref = oracle.qmm_w4a16(d["A"], d["Wq"], d["scale"], d["bias"], M, N, K)
    check_tolerance(C, ref, what="f32p %s M=%d" % (name, M))


# --------------------------------------------------- fp32 partial planes (W4A16)

def check_single_cast(bits, ref, min_equal, what):
    """bits: bf16 result; ref: fp64 exact value. Every element lies within one bf16 spacing
    of ref (the correctly rounded value or its neighbour across a nearby midpoint), plus
    an absolute 1e-4*rms(ref) for the fp32 accumulation near zero (its typical size is
    about sqrt(K)*2^-24*rms(ref), 3e-6*rms at K = 2560), and at least min_equal of them
    are the correctly rounded value. Returns that fraction."""
    got = syn.bf16_bits_to_f32(bits).astype(np.float64)
    mag = np.maximum(np.abs(ref), np.abs(got))
    spacing = np.exp2(np.floor(np.log2(np.maximum(mag, 1e-30))) - 7)
    err = np.abs(got - ref)
    bad = err > spacing + 1e-4 * float(np.sqrt(np.mean(ref * ref)))
    assert not bad.any(), "%s: %d elements more than one bf16 spacing away; first got %s ref %s" % (
        what, int(bad.sum()), got[bad][:4].tolist(), ref[bad][:4].tolist())
    frac = float(np.mean(bits == oracle.bf16_round_array(ref)))
    say("%s: correctly rounded fraction %.4f" % (what, frac))
    assert frac >= min_equal, "%s: only %.4f correctly rounded" % (what, frac)
    return frac


F32P_CASES = [  # (M, N, K, explicit splits): small-M kernel (48 rows, and 100 rows in 64-row blocks),
    # 128-row and 256-row large-M kernels
    (48, 1000, 2560, (2, 5, 20)), (100, 1000, 2560, (4, 10)), (100, 7000, 2560, (4, 10)),
    (256, 520, 4096, (2, 8, 32))]


@pytest.mark.parametrize("M,N,K,splits", F32P_CASES)
def test_f32p_partials_round_once(M, N, K, splits):
    """Power-of-two scales make every dequantised weight and product exact, so a result
    rounded to bf16 once (unsplit, or fp32 planes) is correctly rounded but for fp32
    accumulation; bf16 planes round each partition first (printed for contrast)."""
    d = syn.w4a16_pow2_inputs(M, N, K, seed=9000 + M)
    ref = oracle.qmm_w4a16(d["A"], d["Wq"], d["scale"], d["bias"], M, N, K)
    dv = w4a16_device(d)
    say("f32p M=%d N=%d K=%d s=1" % (M, N, K))
    c1 = host_bits(run_w4a16(dv, M, N, K, 1))
    check_single_cast(c1, ref, 0.98, "unsplit %dx%dx%d" % (M, N, K))
    c1f = host_bits(run_w4a16(dv, M, N, K, 1, f32p=True))
    assert np.array_equal(c1, c1f), "f32p s=1 is not the unsplit launch"
    for s in splits + (0,):
        say("f32p M=%d N=%d K=%d s=%d" % (M, N, K, s))
        C = run_w4a16(dv, M, N, K, s, guard=64, f32p=True)
        check_tolerance(host_f64(C), ref, what="f32p s=%d" % s)
        check_single_cast(host_bits(C), ref, 0.98, "f32p %dx%dx%d s=%d" % (M, N, K, s))
    sb = max(splits)
    fb = float(np.mean(host_bits(run_w4a16(dv, M, N, K, sb)) == oracle.bf16_round_array(ref)))
    say("bf16 planes s=%d: correctly rounded fraction %.4f" % (sb, fb))


@pytest.mark.parametrize("M", [1, 4, 8])
def test_gemv_unsplit_rounds_once(M):
    N, K = 1000, 2560
    d = syn.w4a16_pow2_inputs(M, N, K, seed=9050 + M)
    ref = oracle.qmm_w4a16(d["A"], d["Wq"], d["scale"], d["bias"], M, N, K)
    say("gemv single cast M=%d N=%d K=%d" % (M, N, K))
    C = host_bits(run_gemv(w4a16_device(d), M, N, K, 1))
    check_single_cast(C, ref, 0.98, "gemv %dx%dx%d s=1" % (M, N, K))


def test_f32p_split_tail():
    """The large-M plan with unsplit leading columns and a split tail, fp32 planes: leading
    columns equal the unsplit kernel, tail columns round once (sampled by the oracle)."""
    M, N, K = 1000, 64 * 256 + 100, 2560
    plan = q.qmm_splitk_plan(M, N, K)
    assert plan.s > 1 and 0 < plan.full_tiles < plan.base_tiles
    n_lo = (plan.full_tiles // -(-M // plan.block_m)) * plan.block_n
    d = syn.w4a16_pow2_inputs(M, N, K, seed=9100)
    dv = w4a16_device(d)
    say("f32p split tail M=%d N=%d K=%d s=%d" % (M, N, K, plan.s))
    C = host_bits(run_w4a16(dv, M, N, K, 0, guard=64, f32p=True))
    C1 = host_bits(run_w4a16(dv, M, N, K, 1))
    assert np.array_equal(C[:, :n_lo], C1[:, :n_lo])
    ref = oracle.qmm_w4a16(d["A"], d["Wq"], d["scale"], d["bias"], M, N, K)
    check_single_cast(C[:, n_lo:], ref[:, n_lo:], 0.98, "f32p split tail")


def test_f32p_policy_fallback_is_unsplit():
    # shapes where the plan picks s = 1: the f32p entry runs the unsplit launch unchanged
    for M, N, K in [(2048, 9728, 2560), (64, 9728, 2560)]:
        if q.qmm_splitk_plan(M, N, K).s != 1:
            continue
        d = syn.w4a16_inputs(M, N, K, seed=9200 + M)
        dv = w4a16_device(d)
        say("f32p fallback M=%d N=%d K=%d" % (M, N, K))
        a = host_bits(run_w4a16(dv, M, N, K, 0, f32p=True))
        b = host_bits(run_w4a16(dv, M, N, K, 1))
        assert np.array_equal(a, b)


# ----------------------------------------------------------- config 3 (dense)

@pytest.fixture(scope="module")
def cfg3():
    M, N, K = 512, 512, 16384
    d = syn.dense_inputs(M, N, K, seed=3000)
    return M, N, K, d, oracle.qmm_dense(d["A"], d["B"], M, N, K)


@pytest.mark.parametrize("s", [1, 2, 4, 6, 8, 12, 16, 32])
def test_cfg3_dense_split_sweep(cfg3, s):
    M, N, K, d, ref = cfg3
    say("cfg3 dense M=%d N=%d K=%d s=%d" % (M, N, K, s))
    A, B = dev_bf16(d["A"]), dev_bf16(d["B"])
    C = q.bf16_splitk(A, B, s=s)
    torch.cuda.synchronize()
    check_tolerance(host_f64(C), ref, what="dense s=%d" % s)


@pytest.mark.parametrize("M,N,K,splits", [(37, 45, 32 * 71, (1, 3, 7, 71)), (37, 45, 64 * 35, (2, 3, 6, 35)),
                                          (200, 300, 2048, (1, 5, 16))])
def test_dense_ragged_and_reduce_fp32(M, N, K, splits):
    # K = 32 * 71: partitions of 32-value granules (half stages at the odd ones, one granule
    # each at s = 71); K = 64 * 35: 64-value units (one each at s = 35); 200 x 300: 2 x 3
    # tiles, the last row and column of tiles partial
    d = syn.dense_inputs(M, N, K, seed=3001 + K)
    ref = oracle.qmm_dense(d["A"], d["B"], M, N, K)
    A, B = dev_bf16(d["A"]), dev_bf16(d["B"])
    for s in splits:
        say("dense ragged M=%d N=%d K=%d s=%d" % (M, N, K, s))
        C = q.bf16_splitk(A, B, s=s)
        torch.cuda.synchronize()
        check_tolerance(host_f64(C), ref, what="dense ragged K=%d s=%d" % (K, s))


# ----------------------------------------------------------- config 4 (decode)

DECODE = syn.decode_sweep()


@pytest.mark.parametrize("name,M,N,K,idx", DECODE, ids=["%s-M%d" % (n, m) for n, m, _, _, _ in DECODE])
def test_cfg4_decode(name, M, N, K, idx):
    d = syn.w4a16_inputs(M, N, K, seed=4000 + idx)
    dv = w4a16_device(d)
    ref = oracle.qmm_w4a16(d["A"], d["Wq"], d["scale"], d["bias"], M, N, K)
    G = K // 128
    valid = [s for s in range(1, G + 1) if G % s == 0 and K // s >= 512]
    for s in valid + [0]:
        say("cfg4 %s M=%d N=%d K=%d s=%d" % (name, M, N, K, s))
        C = run_w4a16(dv, M, N, K, s, guard=32)
        check_tolerance(host_f64(C), ref, what="%s M=%d s=%d" % (name, M, s))


# ------------------------------------------------------ decode matrix-vector kernel

def run_gemv(dv, M, N, K, s, guard=0):
    s_eff = s or q.qmm_gemv_min_split(M, K)
    Cbuf = torch.full((M * N + 2 * guard,), -12345.0, dtype=torch.bfloat16, device="cuda")
    C = Cbuf[guard:guard + M * N].view(M, N)
    ws = torch.empty(2 * s_eff * M * N + 16, dtype=torch.uint8, device="cuda") if s_eff > 1 else None
    q.qmm_w4a16_gemv(dv["A"], dv["Wq"], dv["scale"], dv["bias"], C, M, N, K, s, ws)
    torch.cuda.synchronize()
    if guard:
        g = host_bits(Cbuf)
        canary = host_bits(torch.tensor([-12345.0], dtype=torch.bfloat16))[0]
        assert np.all(g[:guard] == canary) and np.all(g[guard + M * N:] == canary), "C guard band written"
    return C


def gemv_splits(M, K):
    """Every split the decode kernel accepts for (M, K)."""
    G = K // 128
    m8 = 1 if M <= 1 else 2 if M <= 2 else 4 if M <= 4 else 8
    return [s for s in range(1, G + 1) if G % s == 0 and K // s <= 10240 and m8 * (K // s) <= 30720
            and (m8 < 8 or K // s <= 4096)]


@pytest.mark.parametrize("name,M,N,K,idx", DECODE, ids=["%s-M%d" % (n, m) for n, m, _, _, _ in DECODE])
def test_gemv_decode_shapes(name, M, N, K, idx):
    d = syn.w4a16_inputs(M, N, K, seed=4000 + idx)
    ref = oracle.qmm_w4a16(d["A"], d["Wq"], d["scale"], d["bias"], M, N, K)
    dv = w4a16_device(d)
    for s in [0] + gemv_splits(M, K)[:4]:
        say("gemv %s M=%d N=%d K=%d s=%d" % (name, M, N, K, s))
        C = run_gemv(dv, M, N, K, s)
        check_tolerance(host_f64(C), ref, what="gemv %s M=%d s=%d" % (name, M, s))


# Covers both item sizes of the kernel (4 rows per item, or 2 where that evens out the
# lanes' work: K = 128, 256, 384, 2560 at M = 2, 6400 with up to 7 items per lane) and
# ragged N.
GEMV_EDGE = [(1, 1, 128), (3, 17, 256), (5, 100, 384), (8, 33, 4096), (2, 1000, 10240), (7, 4100, 1280),
             (4, 64, 7680), (6, 15, 3968), (1, 50, 6400), (2, 70, 2560),
             # 10-row workgroups with a ragged last one (5, 3 and 7 rows)
             (1, 2555, 9728), (2, 33, 1280), (1, 7, 2560)]


@pytest.mark.parametrize("M,N,K", GEMV_EDGE)
def test_gemv_edge_shapes(M, N, K):
    d = syn.w4a16_inputs(M, N, K, seed=4500 + M + N + K)
    ref = oracle.qmm_w4a16(d["A"], d["Wq"], d["scale"], d["bias"], M, N, K)
    dv = w4a16_device(d)
    splits = gemv_splits(M, K)
    for s in sorted({0, splits[0], splits[-1]}):
        say("gemv edge M=%d N=%d K=%d s=%d" % (M, N, K, s))
        C = run_gemv(dv, M, N, K, s, guard=24)
        check_tolerance(host_f64(C), ref, what="gemv edge %dx%dx%d s=%d" % (M, N, K, s))


def test_gemv_closed_forms():
    """Zero weights give zero up to the kernel's cancellation bound; one-hot rows of A
    give the dequantised weight, rounded once to bf16; two runs agree bit for bit.

    The kernel sums A*(128 + q) in fp32 and subtracts 128*sum(A) per chunk of 32 values
    (the products are exact, the sums round), so with q = 8 and bias = -8*scale the
    result is scale * (rounding residue), bounded by K fp32 additions of terms up to
    136*max|A|: |C| <= K * 2^-24 * 136 * max|A| * max(scale) * 4 (generous factor 4)."""
    M, N, K = 8, 96, 1024
    d = syn.w4a16_inputs(M, N, K, seed=4600)
    d["Wq"][:] = np.uint32(0x88888888)  # q = 8 and bias = -8*scale: w = 0
    dv = w4a16_device(d)
    C = run_gemv(dv, M, N, K, 0)
    amax = float(np.max(np.abs(syn.bf16_bits_to_f32(d["A"]))))
    smax = float(np.max(syn.bf16_bits_to_f32(d["scale"])))
    bound = K * 2.0 ** -24 * 136 * amax * smax * 4
    assert float(np.max(np.abs(host_f64(C)))) <= bound
    d = syn.w4a16_inputs(M, N, K, seed=4601)
    ks = np.random.default_rng(4601).integers(0, K, M)
    A = np.zeros((M, K), dtype=np.uint16)
    A[np.arange(M), ks] = 0x3F80  # 1.0
    d["A"] = A
    dv = w4a16_device(d)
    C = run_gemv(dv, M, N, K, 0)
    w = oracle.dequant_w4a16(d["Wq"], d["scale"], d["bias"], N, K)  # [N][K], exact
    want = oracle.bf16_round_array(w[:, ks].T)
    assert np.array_equal(host_bits(C), want)
    assert np.array_equal(host_bits(run_gemv(dv, M, N, K, 0)), host_bits(C))


# ---------------------------------------------------------------- reduce

@pytest.mark.parametrize("s,M,N", [(1, 16, 1024), (2, 32, 1024), (5, 48, 1000), (20, 7, 33), (32, 1, 9),
                                   (10, 128, 2560), (3, 2048, 1024)])
def test_reduce_bf16_bitexact(s, M, N):
    say("reduce bf16 s=%d M=%d N=%d" % (s, M, N))
    planes = syn.bf16_planes(s, M, N, seed=5000 + s + M + N, sigma=3.0)
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    q.qmm_splitk_reduce(dev_bf16(planes), q.QMM_PARTIAL_BF16, s, M, N, out)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(out).ravel(), oracle.reduce_bf16(planes, s, M * N))


@pytest.mark.parametrize("s,M,N", [(1, 8, 8), (6, 512, 512), (32, 5, 7), (12, 3, 1001)])
def test_reduce_f32_bitexact(s, M, N):
    say("reduce f32 s=%d M=%d N=%d" % (s, M, N))
    planes = syn.f32_planes(s, M, N, seed=5100 + s, sigma=40.0)
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    q.qmm_splitk_reduce(torch.from_numpy(planes).cuda(), q.QMM_PARTIAL_F32, s, M, N, out)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(out).ravel(), oracle.reduce_f32(planes, s, M * N))


# ---------------------------------------------------------- exact closed forms

@pytest.mark.parametrize("s", [1, 2, 4, 5, 10, 20])
def test_zero_weights_give_exact_zero(s):
    M, N, K = 24, 200, 2560
    d = syn.w4a16_inputs(M, N, K, seed=6000)
    d["Wq"] = np.full_like(d["Wq"], 0x88888888)  # q == 8, bias = -8*scale -> w == 0
    say("zero weights s=%d" % s)
    C = run_w4a16(w4a16_device(d), M, N, K, s)
    bits = host_bits(C)
    assert np.all((bits == 0) | (bits == 0x8000))


@pytest.mark.parametrize("s", [1, 2, 4, 5, 10, 20])
def test_one_hot_rows_give_exact_weights(s):
    """A[m, k_m] = 1: C[m, n] = w[n, k_m] exactly (one nonzero partial; bf16 of an exact
    fp32 value). Pins the nibble order, scale/bias indexing and the partition bounds."""
    M, N, K = 40, 130, 2560
    d = syn.w4a16_inputs(M, N, K, seed=6001)
    rng = np.random.default_rng(6001)
    ks = rng.choice(K, size=M, replace=False)
    ks[:8] = [0, 7, 8, 127, 128, 1279, 1280, 2559]
    A = np.zeros((M, K), dtype=np.uint16)
    A[np.arange(M), ks] = 0x3F80
    d["A"] = A
    say("one-hot s=%d" % s)
    C = run_w4a16(w4a16_device(d), M, N, K, s, guard=16)
    w = oracle.dequant_w4a16(d["Wq"], d["scale"], d["bias"], N, K)
    expect = oracle.bf16_round_array(w[:, ks].T)
    got = host_bits(C).copy()
    got[got == 0x8000] = 0  # the sign of an exact zero is not part of the definition
    expect[expect == 0x8000] = 0
    assert np.array_equal(got, expect)


def test_determinism_two_runs():
    M, N, K = 16, 9728, 2560
    d = syn.w4a16_inputs(M, N, K, seed=6002)
    dv = w4a16_device(d)
    for s in (1, 4, 10):
        say("determinism s=%d" % s)
        a = host_bits(run_w4a16(dv, M, N, K, s))
        b = host_bits(run_w4a16(dv, M, N, K, s))
        assert np.array_equal(a, b)


# ------------------------------------------- other weight formats (qmm_wna16)

FORMATS = [(4, 32), (4, 64), (8, 32), (8, 64), (8, 128)]


def run_wna16(dv, bits, group, M, N, K, s, guard=0, f32p=False):
    """qmm_wna16 through the C ABI; returns C (bf16 device tensor), checking guard bands
    around C and the workspace when guard > 0."""
    s_eff = q.qmm_wna16_plan(bits, group, M, N, K).s if s == 0 else s
    Cbuf = torch.full((M * N + 2 * guard,), -12345.0, dtype=torch.bfloat16, device="cuda")
    C = Cbuf[guard:guard + M * N].view(M, N)
    ws = wbuf = None
    wdt = torch.float32 if f32p else torch.bfloat16
    gw = ((guard + 7) // 8) * 8
    if s_eff > 1:
        wbuf = torch.full((s_eff * M * N + 2 * gw,), -777.0, dtype=wdt, device="cuda")
        ws = wbuf[gw:gw + s_eff * M * N]
    q.qmm_wna16(bits, group, q.QMM_PARTIAL_F32 if f32p else q.QMM_PARTIAL_BF16, dv["A"], dv["Wq"], dv["scale"],
                dv["bias"], C, M, N, K, s, ws)
    torch.cuda.synchronize()
    if guard:
        g = host_bits(Cbuf)
        canary = host_bits(torch.tensor([-12345.0], dtype=torch.bfloat16))[0]
        assert np.all(g[:guard] == canary) and np.all(g[guard + M * N:] == canary), "C guard band written"
        if wbuf is not None:
            w = wbuf.cpu().numpy() if f32p else host_bits(wbuf)
            wc = np.float32(-777.0) if f32p else host_bits(torch.tensor([-777.0], dtype=torch.bfloat16))[0]
            assert np.all(w[:gw] == wc) and np.all(w[gw + s_eff * M * N:] == wc), "workspace guard written"
    return C


# small-M kernel (M <= 64, ragged N; 100 rows in 64-row blocks), 128-row and 256-row
# large-M kernels; the last two split into partitions of unequal length (3 of 20 and 8 groups)
FORMAT_SHAPES = [(1, 1000, 2560, 4), (16, 1024, 2560, 5), (48, 1000, 1024, 2), (100, 1000, 2560, 4),
                 (100, 7000, 2560, 4), (300, 520, 1024, 8), (48, 1000, 2560, 3), (300, 520, 1024, 3)]


@pytest.mark.parametrize("bits,group", FORMATS)
@pytest.mark.parametrize("M,N,K,s", FORMAT_SHAPES)
def test_wna16_formats_match_oracle(bits, group, M, N, K, s):
    d = syn.wq_inputs(bits, group, M, N, K, seed=11000 + 7 * M + bits * 3 + group)
    ref = oracle.qmm_wq(bits, group, d["A"], d["Wq"], d["scale"], d["bias"], M, N, K)
    dv = w4a16_device(d)
    for ss in (1, s, 0):
        say("wna16 bits=%d group=%d M=%d N=%d K=%d s=%d" % (bits, group, M, N, K, ss))
        C = run_wna16(dv, bits, group, M, N, K, ss, guard=64)
        check_tolerance(host_f64(C), ref, what="w%da16 g%d %dx%dx%d s=%d" % (bits, group, M, N, K, ss))
    say("wna16 bits=%d group=%d M=%d fp32 partials s=%d" % (bits, group, M, s))
    C = run_wna16(dv, bits, group, M, N, K, s, guard=64, f32p=True)
    check_tolerance(host_f64(C), ref, what="w%da16 g%d %dx%dx%d s=%d fp32 partials" % (bits, group, M, N, K, s))


@pytest.mark.parametrize("bits,group", FORMATS)
@pytest.mark.parametrize("M,N,K", [(16, 300, 1024), (100, 300, 1024), (100, 7000, 2560), (300, 300, 1024)])
def test_wna16_one_hot_rows_exact(bits, group, M, N, K):
    """A row with a single 1 at k picks w[:, k] = scale*q + bias (exact in fp32, one
    rounding to bf16): every split gives the correctly rounded weights, bit for bit.
    This pins the code order, the group index and the partition bounds on the GPU
    (small-M kernel; 128-row and 256-row large-M kernels)."""
    d = syn.wq_inputs(bits, group, M, N, K, seed=12000 + M + N + bits + group)
    rng = np.random.default_rng(12000 + M + N)
    ks = rng.integers(0, K, M)
    A = np.zeros((M, K), dtype=np.uint16)
    A[np.arange(M), ks] = 0x3F80
    d["A"] = A
    ref_bits = oracle.bf16_round_array(oracle.qmm_wq(bits, group, A, d["Wq"], d["scale"], d["bias"], M, N, K))
    dv = w4a16_device(d)
    G = K // 128
    for s in (1, 2, max(x for x in range(1, 9) if G % x == 0)):
        say("wna16 one-hot bits=%d group=%d M=%d s=%d" % (bits, group, M, s))
        got = host_bits(run_wna16(dv, bits, group, M, N, K, s))
        assert np.array_equal(got, ref_bits), "s=%d: %d of %d differ" % (s, int((got != ref_bits).sum()), got.size)


@pytest.mark.parametrize("M", [16, 300])
def test_w8a16_rounds_once(M):
    """8-bit codes with power-of-two scales: exact dequantisation and products, so the
    unsplit kernel and fp32 planes round once (see check_single_cast)."""
    N, K = 520, 2560
    d = syn.wq_inputs(8, 128, M, N, K, seed=13000 + M)
    e = np.random.default_rng(13001 + M).integers(-11, -8, size=d["scale"].shape)
    sc = np.ldexp(np.float32(1.0), e).astype(np.float32)
    d["scale"] = syn.f32_to_bf16_bits(sc)
    d["bias"] = syn.f32_to_bf16_bits(np.float32(-128.0) * sc)
    ref = oracle.qmm_wq(8, 128, d["A"], d["Wq"], d["scale"], d["bias"], M, N, K)
    dv = w4a16_device(d)
    say("w8a16 single cast M=%d s=1" % M)
    check_single_cast(host_bits(run_wna16(dv, 8, 128, M, N, K, 1)), ref, 0.98, "w8a16 %d s=1" % M)
    say("w8a16 single cast M=%d s=4 fp32 partials" % M)
    check_single_cast(host_bits(run_wna16(dv, 8, 128, M, N, K, 4, f32p=True)), ref, 0.98, "w8a16 %d s=4 f32p" % M)


def test_wna16_w4_g128_is_the_w4a16_launch():
    for M, N, K in [(16, 1024, 2560), (300, 520, 1024)]:
        d = syn.w4a16_inputs(M, N, K, seed=14000 + M)
        dv = w4a16_device(d)
        for s in (1, 0, 4):
            say("wna16(4,128) vs w4a16 M=%d s=%d" % (M, s))
            a = host_bits(run_wna16(dv, 4, 128, M, N, K, s))
            b = host_bits(run_w4a16(dv, M, N, K, s))
            assert np.array_equal(a, b)


def test_w8a16_full_size():
    """W8A16 g128 at the gate projection's full size (M = 2048) under the plan."""
    M, N, K = 2048, 9728, 2560
    d = syn.wq_inputs(8, 128, M, N, K, seed=15000)
    dv = w4a16_device(d)
    say("w8a16 full size M=%d N=%d K=%d plan" % (M, N, K))
    C = host_f64(run_wna16(dv, 8, 128, M, N, K, 0))
    ref = oracle.qmm_wq(8, 128, d["A"], d["Wq"], d["scale"], d["bias"], M, N, K)
    check_tolerance(C, ref, what="w8a16 gate M=2048")


# ------------------------------------------------- split-KV decode attention

def run_attn(d, scale, s, guard=0):
    """qmm_attn_decode through the C ABI; returns O [B, Mq, Hq, D] bits, checking a guard
    band after O when guard > 0."""
    B, Mq, Hq, D = d["Q"].shape
    _, Hkv, Lmax, _ = d["K"].shape
    Q, K, V = dev_bf16(d["Q"]), dev_bf16(d["K"]), dev_bf16(d["V"])
    lengths = torch.from_numpy(d["lengths"].astype(np.int32)).cuda()
    n = B * Mq * Hq * D
    Obuf = torch.full((n + guard,), -12345.0, dtype=torch.bfloat16, device="cuda")
    s_eff = s or q.qmm_attn_decode_split(B, Hkv, Lmax)
    wb = q.qmm_attn_decode_workspace_bytes(B, Mq, Hq, s_eff)
    ws = torch.empty(max(wb, 16), dtype=torch.uint8, device="cuda") if wb else None
    q.qmm_attn_decode(Q, K, V, lengths, Obuf, B, Mq, Hq, Hkv, Lmax, D, scale, s, ws)
    torch.cuda.synchronize()
    bits = host_bits(Obuf)
    if guard:
        canary = host_bits(torch.tensor([-12345.0], dtype=torch.bfloat16))[0]
        assert np.all(bits[n:] == canary), "O guard band written"
    return bits[:n].reshape(B, Mq, Hq, D)


def check_attn(bits, ref, what):
    got = syn.bf16_bits_to_f32(bits).astype(np.float64)
    check_tolerance(got, ref, what=what)
    # fp32 probabilities and accumulators, one bf16 rounding: far inside the bf16 bar
    rms = float(np.sqrt(np.mean(ref * ref)))
    err = np.abs(got - ref)
    bound = 2.0 ** -8 * np.abs(ref) + 1e-3 * rms
    assert np.all(err <= bound), "%s: %d outside the tight bound, worst %.3g" % (
        what, int((err > bound).sum()), float(np.max(err - bound)))


ATTN_CASES = [  # (B, Mq, Hq, Hkv, Lmax, lengths, splits)
    (2, 1, 32, 8, 1024, (1000, 37), (1, 2, 3, 4, 8)),      # grouped heads, ragged lengths
    (2, 4, 32, 8, 320, (300, 4), (1, 5)),                  # four draft queries (16 rows), causal
    (3, 2, 4, 4, 200, (200, 2, 129), (1, 3, 7)),           # one head per group
    (1, 2, 16, 2, 512, (512,), (1, 2, 16)),                # eight heads per group, two queries
    (1, 1, 32, 8, 16384, (16384,), (1, 32)),               # a long history
    (4, 1, 8, 8, 64, (5, 64, 1, 63), (1, 8, 64)),          # empty splits (s > length)
]


@pytest.mark.parametrize("B,Mq,Hq,Hkv,Lmax,lengths,splits", ATTN_CASES)
def test_attn_decode_matches_oracle(B, Mq, Hq, Hkv, Lmax, lengths, splits):
    d = syn.attn_inputs(B, Mq, Hq, Hkv, Lmax, 128, list(lengths), seed=16000 + B * 100 + Mq * 10 + Hkv)
    scale = 1.0 / np.sqrt(128.0)
    ref = oracle.attn_decode(d["Q"], d["K"], d["V"], d["lengths"], scale)
    for s in splits + (0,):
        say("attn B=%d Mq=%d Hq=%d Hkv=%d L=%s s=%d" % (B, Mq, Hq, Hkv, lengths, s))
        check_attn(run_attn(d, scale, s, guard=64), ref, "attn %s s=%d" % (lengths, s))


def test_attn_single_key_is_exact():
    # each query sees exactly one key (lengths = Mq = 1): O is that key's value row, bit for bit
    B, Hq, Hkv, L = 3, 32, 8, 64
    d = syn.attn_inputs(B, 1, Hq, Hkv, L, 128, [1, 1, 1], seed=16500)
    for s in (1, 4):
        say("attn single key s=%d" % s)
        got = run_attn(d, 0.1, s)
        for h in range(Hq):
            assert np.array_equal(got[:, 0, h], d["V"][:, h // 4, 0]), (s, h)


def test_attn_uniform_weights_average_values():
    # zero queries: every allowed key has weight 1/len (exact for power-of-two lengths)
    B, Hq, Hkv, L = 2, 8, 2, 256
    d = syn.attn_inputs(B, 1, Hq, Hkv, L, 128, [256, 128], seed=16600)
    d["Q"][:] = 0
    V = syn.bf16_bits_to_f32(d["V"]).astype(np.float64)
    for s in (1, 2, 8):
        say("attn uniform s=%d" % s)
        got = syn.bf16_bits_to_f32(run_attn(d, 0.5, s)).astype(np.float64)
        for b, n in enumerate((256, 128)):
            for h in range(Hq):
                ref = V[b, h // 4, :n].mean(axis=0)
                assert np.all(np.abs(got[b, 0, h] - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-6), (s, b, h)


# ------------------------------------------------------------- edge shapes

EDGE = [(1, 1, 128, 1), (1, 17, 256, 2), (3, 33, 384, 3), (15, 100, 512, 4), (17, 64, 1024, 8),
        (129, 70, 256, 2), (130, 1001, 640, 5), (2048, 16, 128, 1), (8, 4100, 1280, 10),
        # the decode tile rule's edges: up to 8 rows and 4096 columns over more than 2^24 weights
        # run 16-column tiles (one 256-workgroup round), 9 rows or 4097 columns do not; ragged N
        (8, 4096, 8192, 2), (9, 4096, 8192, 2), (5, 4097, 8192, 3), (7, 2500, 9728, 4),
        # 16-row tiles of 64 columns (at least three quarters of one round), ragged M and N
        (50, 4000, 2560, 2), (33, 6000, 1280, 3),
        # past 64 rows, 32-row tiles of 16 columns in one round (narrowed to 13 at M = 80),
        # ragged M and N
        (100, 1000, 2560, 4), (80, 1024, 2560, 3)]


@pytest.mark.parametrize("M,N,K,s", EDGE)
def test_edge_shapes(M, N, K, s):
    d = syn.w4a16_inputs(M, N, K, seed=7000 + M + N + K)
    ref = oracle.qmm_w4a16(d["A"], d["Wq"], d["scale"], d["bias"], M, N, K)
    dv = w4a16_device(d)
    for ss in sorted({1, s, 0}):
        say("edge M=%d N=%d K=%d s=%d" % (M, N, K, ss))
        C = run_w4a16(dv, M, N, K, ss, guard=40)
        check_tolerance(host_f64(C), ref, what="edge %dx%dx%d s=%d" % (M, N, K, ss))


# Decode (up to 8 rows, 4-bit codes) stages 4 activation rows per group up to M = 4 and 8
# rows up to M = 8 instead of 16, on 16-column tiles (narrowed when unsplit; up to 4 rows at
# any N) and on 48-column tiles (5 to 8 rows, N above 8192 over more than 2^24 weights);
# every M from 1 to 9 (9: 16 rows again),
# ragged N, splits with one, two and three groups per round, and near-equal partitions.
DECODE_ROWS = [(M, 2560, 9728, (1, 4, 7)) for M in (1, 2, 3, 4, 5, 6, 7, 8, 9)] + \
    [(M, 8200, 2560, (1, 3, 20)) for M in (1, 4, 5, 8)] + [(3, 1001, 1280, (1, 2, 10)), (6, 33, 384, (1, 3))]


@pytest.mark.parametrize("M,N,K,splits", DECODE_ROWS)
def test_decode_staged_rows(M, N, K, splits):
    d = syn.w4a16_inputs(M, N, K, seed=7500 + M + N + K)
    ref = oracle.qmm_w4a16(d["A"], d["Wq"], d["scale"], d["bias"], M, N, K)
    dv = w4a16_device(d)
    for ss in sorted(set(splits) | {0}):
        say("decode rows M=%d N=%d K=%d s=%d" % (M, N, K, ss))
        C = run_w4a16(dv, M, N, K, ss, guard=40)
        check_tolerance(host_f64(C), ref, what="decode rows %dx%dx%d s=%d" % (M, N, K, ss))


def test_decode_staged_rows_one_hot_exact():
    """One-hot activation rows, A[m, k_m] = 1: C[m, n] = RNE_bf16(w[n, k_m]) exactly with 4 or
    8 staged rows, on 16- and 48-column tiles (each output row reads only its own staged row)."""
    for M, N, K in ((3, 2560, 2560), (8, 8200, 2560)):
        d = syn.w4a16_inputs(M, N, K, seed=7600 + M)
        ks = np.array([(37 * i + 5) % K for i in range(M)])
        A = np.zeros((M, K), dtype=np.uint16)
        A[np.arange(M), ks] = 0x3F80
        d["A"] = A
        say("decode rows one-hot M=%d N=%d" % (M, N))
        C = run_w4a16(w4a16_device(d), M, N, K, 1, guard=40)
        w = oracle.dequant_w4a16(d["Wq"], d["scale"], d["bias"], N, K)
        expect = oracle.bf16_round_array(w[:, ks].T)
        got = host_bits(C).copy()
        got[got == 0x8000] = 0  # the sign of an exact zero is not part of the definition
        expect[expect == 0x8000] = 0
        assert np.array_equal(got, expect), (M, N)


# Unsplit grids of 16-column small-M tiles with fewer tiles than CUs run narrower tiles of
# ceil(N / (256 // row blocks)) columns: widths of 1 (one column per workgroup), 2, 4 (whole
# 4-column stores), 8 (two 16-row blocks, the second ragged), 10 and 12 (pairs), 11 (odd:
# pairs and single columns), ragged last tiles, and a 256-tile grid that is left as it is.
NARROW = [(1, 1, 256, 1), (5, 40, 384, 1), (16, 300, 512, 2), (13, 1000, 640, 4), (29, 1000, 640, 8),
          (7, 2500, 9728, 10),
          (32, 2561, 1024, 11), (3, 3000, 1280, 12), (20, 4095, 256, 16)]


@pytest.mark.parametrize("M,N,K,tw", NARROW)
def test_narrowed_tiles(M, N, K, tw):
    plan = q.qmm_splitk_plan(M, N, K)
    assert (plan.s, plan.block_n) == (1, tw)
    d = syn.w4a16_inputs(M, N, K, seed=7100 + M + N)
    ref = oracle.qmm_w4a16(d["A"], d["Wq"], d["scale"], d["bias"], M, N, K)
    dv = w4a16_device(d)
    for f32p in (False, True):
        say("narrowed tiles M=%d N=%d K=%d width=%d f32p=%d" % (M, N, K, tw, f32p))
        C = run_w4a16(dv, M, N, K, 1, guard=40, f32p=f32p)
        check_tolerance(host_f64(C), ref, what="narrowed %dx%dx%d" % (M, N, K))
    # one-hot rows: every column of every narrowed tile is the correctly rounded weight
    rng = np.random.default_rng(7100 + N)
    ks = rng.integers(0, K, M)
    A = np.zeros((M, K), dtype=np.uint16)
    A[np.arange(M), ks] = 0x3F80
    dv["A"] = dev_bf16(A)
    say("narrowed tiles one-hot M=%d N=%d K=%d" % (M, N, K))
    got = host_bits(run_w4a16(dv, M, N, K, 1, guard=40)).copy()
    expect = oracle.bf16_round_array(oracle.dequant_w4a16(d["Wq"], d["scale"], d["bias"], N, K)[:, ks].T)
    got[got == 0x8000] = 0
    expect[expect == 0x8000] = 0
    assert np.array_equal(got, expect), "%d of %d differ" % (int((got != expect).sum()), got.size)


def test_narrowed_tiles_other_formats():
    # the 8-bit codes and groups of 32 take the same narrowed tiles (1000 columns: width 4)
    M, N, K = 16, 1000, 1024
    for bits, group in ((8, 128), (4, 32)):
        plan = q.qmm_wna16_plan(bits, group, M, N, K)
        assert (plan.s, plan.block_n) == (1, 4)
        d = syn.wq_inputs(bits, group, M, N, K, seed=7200 + bits + group)
        ref = oracle.qmm_wq(bits, group, d["A"], d["Wq"], d["scale"], d["bias"], M, N, K)
        say("narrowed tiles w%da16 g%d" % (bits, group))
        C = run_wna16(w4a16_device(d), bits, group, M, N, K, 1, guard=40)
        check_tolerance(host_f64(C), ref, what="narrowed w%da16 g%d" % (bits, group))


# 256 x 256 tiles of a split with ragged M and N (N % 4 = 2 and 1): the epilogues' whole-row
# stores through LDS, bf16 and fp32 planes, with the partial quads stored element by element.
@pytest.mark.parametrize("M,N,K", [(900, 4098, 1536), (1300, 3001, 1536)])
def test_256_row_tiles_ragged_planes(M, N, K):
    plan = q.qmm_splitk_plan(M, N, K)
    assert (plan.block_m, plan.block_n) == (256, 256) and plan.s > 1
    d = syn.w4a16_inputs(M, N, K, seed=7300 + N)
    ref = oracle.qmm_w4a16(d["A"], d["Wq"], d["scale"], d["bias"], M, N, K)
    dv = w4a16_device(d)
    for f32p in (False, True):
        say("256-row tiles ragged M=%d N=%d K=%d s=%d f32p=%d" % (M, N, K, plan.s, f32p))
        C = run_w4a16(dv, M, N, K, 0, guard=40, f32p=f32p)
        check_tolerance(host_f64(C), ref, what="256-row ragged %dx%dx%d f32p=%d" % (M, N, K, f32p))


def test_largest_k_partition_bounds():
    # K just under 2^22 (the host's limit: G = 32767 groups) on the small-M kernel, unsplit,
    # split 7 ways, 20000 ways (partitions of one or two groups: p*G up to 6.6e8) and one
    # group per partition: the partition bounds floor(p*G/s) at their largest values
    M, N, K = 3, 40, ((1 << 22) // 128 - 1) * 128
    d = syn.w4a16_inputs(M, N, K, seed=7050)
    ref = oracle.qmm_w4a16(d["A"], d["Wq"], d["scale"], d["bias"], M, N, K)
    dv = w4a16_device(d)
    for s in (1, 7, 20000, K // 128):
        say("largest K M=%d N=%d K=%d s=%d" % (M, N, K, s))
        C = run_w4a16(dv, M, N, K, s, guard=24)
        check_tolerance(host_f64(C), ref, what="largest K s=%d" % s)


def test_largest_k_large_m_kernel():
    # the large-M kernel (129 rows) at the largest K the host accepts (32767 groups): its
    # 32-bit per-lane copy offsets reach 2*255*K bytes; unsplit, split 7 ways, at the cap
    # and under the plan, on sampled outputs (every edge row and column among them).
    # Inputs: a seeded block of 151 groups repeated 217 times along K (generating 5.4e8
    # activations takes minutes); an offset that wrapped at 2^32 bytes would land at a
    # different position within the block.
    M, N, K = 129, 64, ((1 << 22) // 128 - 1) * 128
    kb = 151 * 128
    blk = syn.w4a16_inputs(M, N, kb, seed=7060)
    d = {key: np.tile(blk[key], (1, K // kb)) for key in ("A", "Wq", "scale", "bias")}
    rng = np.random.default_rng(7060)
    ms = np.concatenate([np.repeat([0, 1, 127, 128], 3), rng.integers(0, M, 60)]).astype(np.int32)
    ns = np.concatenate([np.tile([0, 31, 63], 4), rng.integers(0, N, 60)]).astype(np.int32)
    ref = oracle.qmm_w4a16_points(d["A"], d["Wq"], d["scale"], d["bias"], M, N, K, ms, ns)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    dv = w4a16_device(d)
    del d
    for s in (1, 7, 20, 0):
        say("largest K large-M kernel M=%d N=%d K=%d s=%d" % (M, N, K, s))
        C = host_f64(run_w4a16(dv, M, N, K, s, guard=24))
        check_tolerance(C[ms, ns], ref, rms=rms, what="largest K large-M s=%d" % s)


def test_error_leaves_output_untouched():
    M, N, K = 16, 64, 256
    d = syn.w4a16_inputs(M, N, K, seed=7100)
    dv = w4a16_device(d)
    C = torch.full((M, N), 3.0, dtype=torch.bfloat16, device="cuda")
    rc = q.qmm_w4a16_g128(dv["A"], dv["Wq"], dv["scale"], dv["bias"], C, M, N, K, 2, None, check=False)
    assert rc == q.QMM_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(C == 3.0)


# ------------------------------------------------------------ graph capture

def test_graph_capture_replays_match_eager():
    """The library enqueues only kernels (no memsets, no allocation), so a HIP graph of
    its calls replays to the eager result bit for bit, replay after replay."""
    cases = [(16, 1024, 2560, 5), (32, 9728, 2560, 1), (48, 1000, 2560, 4)]
    bufs = []
    for i, (M, N, K, s) in enumerate(cases):
        d = syn.w4a16_inputs(M, N, K, seed=8000 + i)
        dv = w4a16_device(d)
        C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(max(2 * s * M * N, 16), dtype=torch.uint8, device="cuda")
        bufs.append((M, N, K, s, dv, C, ws))

    def step():
        for M, N, K, s, dv, C, ws in bufs:
            q.qmm_w4a16_g128(dv["A"], dv["Wq"], dv["scale"], dv["bias"], C, M, N, K, s, ws if s > 1 else None)

    say("graph: eager reference")
    step()
    torch.cuda.synchronize()
    eager = [host_bits(b[5]).copy() for b in bufs]
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        for b in bufs:
            b[5].fill_(7.0)  # eager work between replays
        torch.cuda.synchronize()
        say("graph: replay %d" % rep)
        g.replay()
        torch.cuda.synchronize()
        for b, e in zip(bufs, eager):
            assert np.array_equal(host_bits(b[5]), e), "replay %d differs" % rep


def test_graph_capture_other_entry_points():
    """fp32 partials, another weight format, the matrix-vector path, stream-K, the dense
    variant and split-KV attention also enqueue kernels only: a graph of all of them
    replays to the eager bits, replay after replay."""
    torch.manual_seed(0)
    calls = []
    # fp32 partial planes, small M split
    d = syn.w4a16_inputs(48, 1000, 2560, seed=18000)
    dv = w4a16_device(d)
    C1 = torch.empty(48, 1000, dtype=torch.bfloat16, device="cuda")
    ws1 = torch.empty(4 * 5 * 48 * 1000, dtype=torch.uint8, device="cuda")
    calls.append((C1, lambda: q.qmm_w4a16_g128_f32p(dv["A"], dv["Wq"], dv["scale"], dv["bias"], C1, 48, 1000, 2560,
                                                    5, ws1)))
    # W8A16 in groups of 32 on the large-M kernel, split
    d8 = syn.wq_inputs(8, 32, 300, 520, 1024, seed=18001)
    dv8 = w4a16_device(d8)
    C2 = torch.empty(300, 520, dtype=torch.bfloat16, device="cuda")
    ws2 = torch.empty(2 * 4 * 300 * 520, dtype=torch.uint8, device="cuda")
    calls.append((C2, lambda: q.qmm_wna16(8, 32, q.QMM_PARTIAL_BF16, dv8["A"], dv8["Wq"], dv8["scale"], dv8["bias"],
                                          C2, 300, 520, 1024, 4, ws2)))
    # decode matrix-vector, split
    dg = syn.w4a16_inputs(4, 2560, 9728, seed=18002)
    dvg = w4a16_device(dg)
    C3 = torch.empty(4, 2560, dtype=torch.bfloat16, device="cuda")
    ws3 = torch.empty(2 * 4 * 4 * 2560, dtype=torch.uint8, device="cuda")
    calls.append((C3, lambda: q.qmm_w4a16_gemv(dvg["A"], dvg["Wq"], dvg["scale"], dvg["bias"], C3, 4, 2560, 9728, 4,
                                               ws3)))
    # stream-K
    ds = syn.w4a16_inputs(300, 520, 1024, seed=18003)
    dvs = w4a16_device(ds)
    C4 = torch.empty(300, 520, dtype=torch.bfloat16, device="cuda")
    nb = q.qmm_streamk_workspace_bytes(300, 520, 1024, 7)
    ws4 = torch.empty(nb, dtype=torch.uint8, device="cuda")
    calls.append((C4, lambda: q.qmm_w4a16_g128_streamk(dvs["A"], dvs["Wq"], dvs["scale"], dvs["bias"], C4, 300, 520,
                                                       1024, 7, ws4, nb)))
    # dense variant, split
    dd = syn.dense_inputs(64, 96, 2048, seed=18004)
    Ad, Bd = dev_bf16(dd["A"]), dev_bf16(dd["B"])
    C5 = torch.empty(64, 96, dtype=torch.bfloat16, device="cuda")
    ws5 = torch.empty(4 * 6 * 64 * 96, dtype=torch.uint8, device="cuda")
    calls.append((C5, lambda: q.qmm_bf16_splitk(Ad, Bd, C5, 64, 96, 2048, 6, ws5)))
    # split-KV attention with the merge
    da = syn.attn_inputs(2, 1, 32, 8, 1024, 128, [1000, 37], seed=18005)
    Qa, Ka, Va = dev_bf16(da["Q"]), dev_bf16(da["K"]), dev_bf16(da["V"])
    La = torch.from_numpy(da["lengths"]).cuda()
    C6 = torch.empty(2, 1, 32, 128, dtype=torch.bfloat16, device="cuda")
    ws6 = torch.empty(q.qmm_attn_decode_workspace_bytes(2, 1, 32, 4), dtype=torch.uint8, device="cuda")
    calls.append((C6, lambda: q.qmm_attn_decode(Qa, Ka, Va, La, C6, 2, 1, 32, 8, 1024, 128, 0.088, 4, ws6)))

    def step():
        for _, fn in calls:
            fn()

    say("graph (other entry points): eager reference")
    step()
    torch.cuda.synchronize()
    eager = [host_bits(c).copy() for c, _ in calls]
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for c, _ in calls:
            c.fill_(5.0)  # eager work between replays
        torch.cuda.synchronize()
        say("graph (other entry points): replay %d" % rep)
        g.replay()
        torch.cuda.synchronize()
        for (c, _), e in zip(calls, eager):
            assert np.array_equal(host_bits(c), e), "replay %d differs" % rep


# ------------------------------------------------------------------ the two passes as separate calls

PASS1_SHAPES = [(16, 1024, 2560, 0), (64, 4096, 2560, 0), (48, 1000, 2560, 4), (128, 9728, 2560, 0),
                (300, 300, 1024, 0), (256, 2560, 4096, 1), (2048, 9728, 2560, 0)]


@pytest.mark.parametrize("M,N,K,s", PASS1_SHAPES)
def test_pass1_then_reduce_cols_equals_the_whole_call(M, N, K, s):
    """qmm_w4a16_g128_pass1 + qmm_splitk_reduce_cols: the planes and columns the first pass
    reports, and C bitwise equal to qmm_w4a16_g128's (small- and large-M kernels, unsplit,
    fully split and the large-M split tail)."""
    say("pass1 M=%d N=%d K=%d s=%d" % (M, N, K, s))
    dv = w4a16_device(syn.w4a16_inputs(M, N, K, seed=4100 + M))
    whole = run_w4a16(dv, M, N, K, s)
    plan = q.qmm_splitk_plan(M, N, K)
    s_eff = q.effective_split(M, N, K, s)
    ws = torch.empty(max(s_eff * M * N, 8), dtype=torch.bfloat16, device="cuda")
    C = torch.full((M, N), -12345.0, dtype=torch.bfloat16, device="cuda")
    rc, s_out, n_lo = q.qmm_w4a16_g128_pass1(dv["A"], dv["Wq"], dv["scale"], dv["bias"], C, M, N, K, s, ws)
    torch.cuda.synchronize()
    assert rc == q.QMM_OK and s_out == s_eff
    if s_eff == 1:
        assert n_lo == N
    elif s == 0 and plan.block_n == 256 and plan.full_tiles > 0:
        assert n_lo == (plan.full_tiles // -(-M // plan.block_m)) * plan.block_n
    else:
        assert n_lo == 0
    got, ref = host_bits(C), host_bits(whole)
    canary = host_bits(torch.tensor([-12345.0], dtype=torch.bfloat16))[0]
    assert np.array_equal(got[:, :n_lo], ref[:, :n_lo]), "columns finished by the first pass"
    assert np.all(got[:, n_lo:] == canary), "the first pass wrote a column left to the planes"
    if s_eff > 1:
        q.qmm_splitk_reduce_cols(ws, q.QMM_PARTIAL_BF16, s_eff, M, N, n_lo, C)
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(C), ref)


# ------------------------------------------------------------ seeded random shapes

def _random_cases(n=24, seed=13000):
    """(bits, group, M, N, K, s) drawn from a fixed seed: every kernel and tile choice
    (16-, 32-, 64-column small-M tiles, 64-row blocks, 128- and 256-row large-M tiles),
    ragged M and N, and explicit splits that divide K/128."""
    rng = np.random.default_rng(seed)
    fmts = [(4, 128), (4, 64), (4, 32), (8, 128), (8, 64), (8, 32)]
    cases = []
    for i in range(n):
        bits, group = fmts[i % len(fmts)]
        M = int(rng.choice([1, 5, 16, 23, 32, 47, 64, 65, 100, 128, 131, 200, 257, 300]))
        N = int(rng.integers(1, 1200))
        G = int(rng.integers(1, 17))
        K = 128 * G
        divs = [d for d in range(1, G + 1) if G % d == 0]
        s = int(rng.choice(divs + [0, 0]))
        cases.append((bits, group, M, N, K, s))
    return cases


@pytest.mark.parametrize("bits,group,M,N,K,s", _random_cases())
def test_random_shapes_match_oracle(bits, group, M, N, K, s):
    """Seeded random shapes through qmm_wna16 (bf16 and fp32 partials) against the oracle,
    with guard bands around C and the workspace."""
    d = syn.wq_inputs(bits, group, M, N, K, seed=13100 + M + N + K + bits + group)
    ref = oracle.qmm_wq(bits, group, d["A"], d["Wq"], d["scale"], d["bias"], M, N, K)
    dv = w4a16_device(d)
    for f32p in (False, True):
        say("random bits=%d group=%d M=%d N=%d K=%d s=%d f32p=%d" % (bits, group, M, N, K, s, f32p))
        C = run_wna16(dv, bits, group, M, N, K, s, guard=48, f32p=f32p)
        check_tolerance(host_f64(C), ref, what="random w%da16 g%d %dx%dx%d s=%d f32p=%d" % (bits, group, M, N, K, s,
                                                                                           f32p))
