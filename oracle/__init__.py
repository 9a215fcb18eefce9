"""CPU oracle for the split-K W4A16 group-128 quantized matmul.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU
baseline may import this package. It shares no code with the GPU library
(``weight_only_quantized_qmm_amd``) and never imports it; the product path
never imports this package.

Contents
  * ``qmm_w4a16``, ``qmm_w4a16_points``, ``qmm_dense``, ``reduce_bf16``,
    ``reduce_f32``, ``dequant_w4a16``, ``bf16_round``, ``bf16_value``,
    ``nibble``, and for the other weight formats (4- or 8-bit codes, groups of
    32, 64 or 128) ``qmm_wq``, ``qmm_wq_points``, ``dequant_wq``, ``code``, and the
    decode attention ``attn_decode``: ctypes wrappers over the plain C definitions in qmm_oracle.c
    (fp64 products in ascending k, fp32 reduce, bf16 round-to-nearest-even).
  * ``policy``: the occupancy split rule of tiny-llm "Week 2 Day 7: Split-K
    Prefill", Task 3, in its plain form.
  * ``models``: the split-K wave model and the double-buffering schedule model
    of gpu-kernels-explained "Split-K, streams and overlap", Maths.

Every function is pinned by tests/test_oracle_pins.py; none is "parity
unpinned".
"""
import ctypes
import os

import numpy as np

from . import build as _build

_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        # QMM_ORACLE_LIB names another build of the same source (the sanitizer build of the tests)
        path = os.environ.get("QMM_ORACLE_LIB")
        if not path:
            path = _build.LIB
            if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_build.SRC):
                _build.build()
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        I = ctypes.c_int
        lib.oracle_bf16_value.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_value.restype = ctypes.c_double
        lib.oracle_bf16_round.argtypes = [ctypes.c_double]
        lib.oracle_bf16_round.restype = ctypes.c_uint16
        lib.oracle_nibble.argtypes = [P, I, I, I]
        lib.oracle_nibble.restype = I
        lib.oracle_dequant_w4a16.argtypes = [P, P, P, I, I, P]
        lib.oracle_dequant_w4a16.restype = None
        lib.oracle_partition_groups.argtypes = [I, I, I, ctypes.POINTER(I), ctypes.POINTER(I)]
        lib.oracle_partition_groups.restype = I
        lib.oracle_partition_granules.argtypes = [I, I, I, ctypes.POINTER(I), ctypes.POINTER(I)]
        lib.oracle_partition_granules.restype = I
        lib.oracle_qmm_w4a16.argtypes = [P, P, P, P, I, I, I, I, P, I]
        lib.oracle_qmm_w4a16.restype = I
        lib.oracle_qmm_w4a16_points.argtypes = [P, P, P, P, I, I, I, I, P, P, P]
        lib.oracle_qmm_w4a16_points.restype = I
        lib.oracle_qmm_dense.argtypes = [P, P, I, I, I, I, P, I]
        lib.oracle_qmm_dense.restype = I
        lib.oracle_code.argtypes = [P, I, I, I, I]
        lib.oracle_code.restype = I
        lib.oracle_dequant_wq.argtypes = [P, I, I, P, P, I, I, P]
        lib.oracle_dequant_wq.restype = I
        lib.oracle_qmm_wq.argtypes = [I, I, P, P, P, P, I, I, I, I, P, I]
        lib.oracle_qmm_wq.restype = I
        lib.oracle_qmm_wq_points.argtypes = [I, I, P, P, P, P, I, I, I, I, P, P, P]
        lib.oracle_qmm_wq_points.restype = I
        lib.oracle_attn_decode.argtypes = [P, P, P, P, I, I, I, I, I, I, ctypes.c_double, P]
        lib.oracle_attn_decode.restype = I
        lib.oracle_reduce_bf16.argtypes = [P, I, ctypes.c_size_t, P]
        lib.oracle_reduce_bf16.restype = None
        lib.oracle_reduce_f32.argtypes = [P, I, ctypes.c_size_t, P]
        lib.oracle_reduce_f32.restype = None
        _LIB = lib
    return _LIB


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data_as(ctypes.c_void_p)


def default_threads():
    """Host threads the oracle may use: the CPUs this process may run on."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def bf16_value(bits):
    """Real value of one bf16 bit pattern (exact, as a Python float)."""
    return _lib().oracle_bf16_value(int(bits))


def bf16_round(x):
    """bf16 bit pattern nearest to x, ties to even."""
    return int(_lib().oracle_bf16_round(float(x)))


def bf16_round_array(x):
    x = np.asarray(x, dtype=np.float64)
    f = _lib().oracle_bf16_round
    return np.array([f(float(v)) for v in x.ravel()], dtype=np.uint16).reshape(x.shape)


def nibble(Wq, K, n, k):
    Wq, p = _c(Wq, np.uint32)
    return _lib().oracle_nibble(p, K, n, k)


def dequant_w4a16(Wq, scale, bias, N, K):
    """w[n,k] = scale[n,k/128] * q[n,k] + bias[n,k/128] in fp64, shape [N, K]."""
    Wq, pw = _c(Wq, np.uint32)
    scale, ps = _c(scale, np.uint16)
    bias, pb = _c(bias, np.uint16)
    w = np.empty((N, K), dtype=np.float64)
    _lib().oracle_dequant_w4a16(pw, ps, pb, N, K, w.ctypes.data_as(ctypes.c_void_p))
    return w


def partition_groups(G, s, p):
    b, e = ctypes.c_int(), ctypes.c_int()
    rc = _lib().oracle_partition_groups(G, s, p, ctypes.byref(b), ctypes.byref(e))
    if rc != 0:
        raise ValueError("no equal group partition: G=%d s=%d p=%d" % (G, s, p))
    return b.value, e.value


def partition_granules(U, s, p):
    b, e = ctypes.c_int(), ctypes.c_int()
    rc = _lib().oracle_partition_granules(U, s, p, ctypes.byref(b), ctypes.byref(e))
    if rc != 0:
        raise ValueError("bad granule partition: U=%d s=%d p=%d" % (U, s, p))
    return b.value, e.value


def qmm_w4a16(A, Wq, scale, bias, M, N, K, s=1, nthreads=None):
    """fp64 C[M,N] of the W4A16 g128 product, summed per partition (s equal parts)."""
    A, pa = _c(A, np.uint16)
    Wq, pw = _c(Wq, np.uint32)
    scale, ps = _c(scale, np.uint16)
    bias, pb = _c(bias, np.uint16)
    C = np.empty((M, N), dtype=np.float64)
    rc = _lib().oracle_qmm_w4a16(pa, pw, ps, pb, M, N, K, s, C.ctypes.data_as(ctypes.c_void_p),
                                 nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle_qmm_w4a16 failed (%d) for M=%d N=%d K=%d s=%d" % (rc, M, N, K, s))
    return C


def qmm_w4a16_points(A, Wq, scale, bias, M, N, K, ms, ns):
    """fp64 C[ms[i], ns[i]] of the unsplit product, each output on its own."""
    A, pa = _c(A, np.uint16)
    Wq, pw = _c(Wq, np.uint32)
    scale, ps = _c(scale, np.uint16)
    bias, pb = _c(bias, np.uint16)
    ms, pm = _c(ms, np.int32)
    ns, pn = _c(ns, np.int32)
    out = np.empty(len(ms), dtype=np.float64)
    rc = _lib().oracle_qmm_w4a16_points(pa, pw, ps, pb, M, N, K, len(ms), pm, pn,
                                        out.ctypes.data_as(ctypes.c_void_p))
    if rc != 0:
        raise ValueError("oracle_qmm_w4a16_points failed (%d)" % rc)
    return out


def code(Wq, bits, K, n, k):
    """q[n, k] of a bits-wide code (4 or 8), lowest field of a word first."""
    Wq, p = _c(Wq, np.uint32)
    return _lib().oracle_code(p, bits, K, n, k)


def dequant_wq(Wq, bits, group, scale, bias, N, K):
    Wq, pw = _c(Wq, np.uint32)
    scale, ps = _c(scale, np.uint16)
    bias, pb = _c(bias, np.uint16)
    w = np.empty((N, K), dtype=np.float64)
    if _lib().oracle_dequant_wq(pw, bits, group, ps, pb, N, K, w.ctypes.data_as(ctypes.c_void_p)) != 0:
        raise ValueError("unsupported weight format bits=%d group=%d K=%d" % (bits, group, K))
    return w


def qmm_wq(bits, group, A, Wq, scale, bias, M, N, K, s=1, nthreads=None):
    """fp64 C[M,N] for a (bits, group) weight format, summed per partition (s equal
    parts of the K/128 blocks)."""
    A, pa = _c(A, np.uint16)
    Wq, pw = _c(Wq, np.uint32)
    scale, ps = _c(scale, np.uint16)
    bias, pb = _c(bias, np.uint16)
    C = np.empty((M, N), dtype=np.float64)
    rc = _lib().oracle_qmm_wq(bits, group, pa, pw, ps, pb, M, N, K, s, C.ctypes.data_as(ctypes.c_void_p),
                              nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle_qmm_wq failed (%d) for bits=%d group=%d M=%d N=%d K=%d s=%d"
                         % (rc, bits, group, M, N, K, s))
    return C


def qmm_wq_points(bits, group, A, Wq, scale, bias, M, N, K, ms, ns):
    """fp64 C[ms[i], ns[i]] of the unsplit product of a (bits, group) format."""
    A, pa = _c(A, np.uint16)
    Wq, pw = _c(Wq, np.uint32)
    scale, ps = _c(scale, np.uint16)
    bias, pb = _c(bias, np.uint16)
    ms, pm = _c(ms, np.int32)
    ns, pn = _c(ns, np.int32)
    out = np.empty(len(ms), dtype=np.float64)
    rc = _lib().oracle_qmm_wq_points(bits, group, pa, pw, ps, pb, M, N, K, len(ms), pm, pn,
                                     out.ctypes.data_as(ctypes.c_void_p))
    if rc != 0:
        raise ValueError("oracle_qmm_wq_points failed (%d)" % rc)
    return out


def attn_decode(Q, K, V, lengths, scale):
    """fp64 O[B, Mq, Hq, D] of decode attention: Q bf16 bits [B, Mq, Hq, D], K and V bf16
    bits [B, Hkv, Lmax, D], lengths int [B] (keys of each request, the Mq queries last)."""
    Q, pq = _c(Q, np.uint16)
    K, pk = _c(K, np.uint16)
    V, pv = _c(V, np.uint16)
    lengths, pl = _c(lengths, np.int32)
    B, Mq, Hq, D = Q.shape
    _, Hkv, Lmax, _ = K.shape
    O = np.empty((B, Mq, Hq, D), dtype=np.float64)
    rc = _lib().oracle_attn_decode(pq, pk, pv, pl, B, Mq, Hq, Hkv, Lmax, D, float(scale),
                                   O.ctypes.data_as(ctypes.c_void_p))
    if rc != 0:
        raise ValueError("oracle_attn_decode failed (%d)" % rc)
    return O


def qmm_dense(A, B, M, N, K, s=1, nthreads=None):
    """fp64 C[M,N] = A @ B.T over bf16 inputs, summed per partition (64-value units when K is a
    multiple of 64, else 32-value granules)."""
    A, pa = _c(A, np.uint16)
    B, pb = _c(B, np.uint16)
    C = np.empty((M, N), dtype=np.float64)
    rc = _lib().oracle_qmm_dense(pa, pb, M, N, K, s, C.ctypes.data_as(ctypes.c_void_p),
                                 nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle_qmm_dense failed (%d) for M=%d N=%d K=%d s=%d" % (rc, M, N, K, s))
    return C


def reduce_bf16(partials, s, MN):
    """bf16 bits of the fp32 ascending-p sum of s bf16 planes, cast once (RNE)."""
    partials, pp = _c(partials, np.uint16)
    C = np.empty(MN, dtype=np.uint16)
    _lib().oracle_reduce_bf16(pp, s, MN, C.ctypes.data_as(ctypes.c_void_p))
    return C


def reduce_f32(partials, s, MN):
    """bf16 bits of the fp32 ascending-p sum of s fp32 planes, cast once (RNE)."""
    partials, pp = _c(partials, np.float32)
    C = np.empty(MN, dtype=np.uint16)
    _lib().oracle_reduce_f32(pp, s, MN, C.ctypes.data_as(ctypes.c_void_p))
    return C
