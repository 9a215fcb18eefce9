"""GPU test of qmm_w4a16_g128_noalloc (the entry point that allocates nothing: the split's
partial planes live in the library's static device scratch) through the C ABI, against
qmm_w4a16_g128 with a caller's workspace on the same inputs: bitwise equal, over calls in a
row whose planes shrink, so each call runs on the planes the previous one left behind."""
import numpy as np
import pytest
import torch

import qmm_synth as syn
import weight_only_quantized_qmm_amd as q
from gpu_util import host_bits, w4a16_device

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)


def with_workspace(dv, M, N, K, s):
    s_eff = q.effective_split(M, N, K, s)
    C = torch.full((M, N), -1.0, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(max(2 * s_eff * M * N, 16), dtype=torch.uint8, device="cuda") if s_eff > 1 else None
    q.qmm_w4a16_g128(dv["A"], dv["Wq"], dv["scale"], dv["bias"], C, M, N, K, s, ws)
    return C


def without_workspace(dv, M, N, K, s):
    C = torch.full((M, N), -2.0, dtype=torch.bfloat16, device="cuda")
    q.qmm_w4a16_g128_noalloc(dv["A"], dv["Wq"], dv["scale"], dv["bias"], C, M, N, K, s)
    return C


# calls in this order, each split's planes smaller than the previous call's (2*s*M*N bytes):
# o at M = 2048 (plan: 3 partitions, 31.5 MB), down at M = 128 (12, 7.9 MB), 48 x 1000 in 5
# (480 KB), the K projection at M = 32 in 4 (262 KB), 40 x 1000 in 3 unequal partitions
# (240 KB), then an unsplit call
CALLS = [(2048, 2560, 4096, 0), (128, 2560, 9728, 0), (48, 1000, 2560, 5), (32, 1024, 2560, 4), (40, 1000, 2560, 3),
         (64, 4096, 2560, 1)]


def test_noalloc_matches_the_workspace_entry_point():
    prev = None
    for i, (M, N, K, s) in enumerate(CALLS):
        s_eff = q.effective_split(M, N, K, s)
        need = 2 * s_eff * M * N if s_eff > 1 else 0
        assert need <= q.QMM_NOALLOC_SCRATCH_BYTES
        if prev is not None:
            assert need <= prev
        prev = need
        d = syn.w4a16_inputs(M, N, K, seed=19000 + i)
        dv = w4a16_device(d)
        say("noalloc M=%d N=%d K=%d s=%d (effective %d, planes %d bytes)" % (M, N, K, s, s_eff, need))
        a = host_bits(without_workspace(dv, M, N, K, s))
        torch.cuda.synchronize()
        b = host_bits(with_workspace(dv, M, N, K, s))
        torch.cuda.synchronize()
        assert np.array_equal(a, b), "noalloc differs from qmm_w4a16_g128 at %dx%dx%d s=%d" % (M, N, K, s)


def test_noalloc_rejects_planes_beyond_the_scratch():
    # gate at M = 2048 under the plan: 5 partitions of [2048][9728] bf16 planes, 199 MB
    M, N, K = 2048, 9728, 2560
    plan = q.qmm_splitk_plan(M, N, K)
    assert plan.workspace_bytes > q.QMM_NOALLOC_SCRATCH_BYTES
    A = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    W = torch.zeros((N, K // 8), dtype=torch.int32, device="cuda")
    S = torch.zeros((N, K // 128), dtype=torch.bfloat16, device="cuda")
    C = torch.full((M, N), 3.0, dtype=torch.bfloat16, device="cuda")
    say("noalloc rejects M=%d N=%d K=%d s=0" % (M, N, K))
    rc = q.qmm_w4a16_g128_noalloc(A, W, S, S, C, M, N, K, 0, check=False)
    assert rc == q.QMM_ERR_SCRATCH
    rc = q.qmm_w4a16_g128_noalloc(A, W, S, S, C, M, N, K, 20, check=False)
    assert rc == q.QMM_ERR_SCRATCH
    torch.cuda.synchronize()
    assert bool((C == 3.0).all()), "a rejected call wrote C"
    # the same shape unsplit needs no scratch
    say("noalloc M=%d N=%d K=%d s=1" % (M, N, K))
    assert q.qmm_w4a16_g128_noalloc(A, W, S, S, C, M, N, K, 1) == q.QMM_OK
    torch.cuda.synchronize()
    assert bool((C == 0.0).all())
