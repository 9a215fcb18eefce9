"""Helpers shared by the GPU parity tests: device copies of the seeded inputs,
the acceptance tolerance, and bf16 bit-pattern conversions."""
import numpy as np
import torch

import qmm_synth as syn

REL_TOL = 0.02  # |gpu - ref| <= 0.02*|ref| + 0.02*rms(ref)  (bf16-appropriate, per output element)
ABS_TOL_RMS = 0.02


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev_u32(words):
    return torch.from_numpy(np.ascontiguousarray(words).view(np.int32)).cuda()


def host_bits(t):
    """uint16 bit patterns of a bf16 device tensor."""
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def host_f64(t):
    return syn.bf16_bits_to_f32(host_bits(t)).astype(np.float64)


def w4a16_device(d):
    return dict(A=dev_bf16(d["A"]), Wq=dev_u32(d["Wq"]), scale=dev_bf16(d["scale"]), bias=dev_bf16(d["bias"]))


def check_tolerance(got, ref, rms=None, what=""):
    """Elementwise |got - ref| <= 0.02*|ref| + 0.02*rms(ref); returns the worst normalised error."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if rms is None:
        rms = float(np.sqrt(np.mean(ref * ref)))
    bound = REL_TOL * np.abs(ref) + ABS_TOL_RMS * rms
    err = np.abs(got - ref)
    bad = ~(err <= bound)
    if bad.any():
        idx = np.argwhere(bad)[:8]
        raise AssertionError("%s: %d of %d outside tolerance (rms %.4g); first %s: got %s ref %s" % (
            what, int(bad.sum()), bad.size, rms, idx.tolist(), got[bad][:8].tolist(), ref[bad][:8].tolist()))
    return float(np.max(err / np.maximum(bound, 1e-300)))


def expected_rms_w4a16(K, scale_lo=0.005, scale_hi=0.02):
    """sqrt(K * E[scale^2] * E[(q-8)^2]) for A ~ N(0,1), q ~ U{0..15}, scale ~ U[lo,hi]."""
    e_s2 = (scale_hi ** 3 - scale_lo ** 3) / (3 * (scale_hi - scale_lo))
    e_q2 = np.mean((np.arange(16) - 8.0) ** 2)
    return float(np.sqrt(K * e_s2 * e_q2))
