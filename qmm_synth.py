"""Seeded synthetic inputs for the W4A16 g128 matmul and the dense bf16 matmul.

This module is the one thing the CPU oracle side and the GPU side of the tests
share: it produces the input bytes both consume. It holds none of the method's
arithmetic (no dequantisation, no product, no reduction); it draws random
numbers, rounds fp32 draws to bf16 bit patterns, and packs 4-bit values eight
to a 32-bit word along K, low nibble first.

Recipe (the workloads' stated distributions):
  A      ~ N(0, 1) drawn in fp32, rounded to bf16 (round-to-nearest-even)
  q      ~ uniform integers 0..15, packed eight per uint32 along K (nibble i of
           word j holds k = 8*j + i)
  scale  ~ U[0.005, 0.02] drawn in fp32, rounded to bf16, one per (row, 128-group)
  bias   = -8 * scale (exact in bf16)
  dense  A, B ~ N(0, 1) rounded to bf16
Other weight formats (wq_inputs): b-bit codes q ~ uniform 0..2^b-1 packed 32/b per
uint32 along K (lowest field first), one scale/bias per (row, group of gs values),
scale ~ U[lo, hi] with [0.005, 0.02] for b = 4 and [0.005, 0.02]/16 for b = 8 (so
the weights span the same range), bias = -2^(b-1) * scale (exact in bf16).
Generator: numpy PCG64 with the given seed; draws in the order A, q, scale.
Seeds used by the tests and the benchmark: 1000 * config + index of the shape
within its config.
"""
import numpy as np

GROUP = 128


def f32_to_bf16_bits(x):
    """Round finite fp32 values to bf16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b):
    """fp32 values of bf16 bit patterns (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def pack_nibbles(q):
    """uint8 q[N, K] with values 0..15 -> uint32 Wq[N, K/8], k = 8*j + i in bits 4i..4i+3."""
    q = np.asarray(q, dtype=np.uint32)
    N, K = q.shape
    if K % 8:
        raise ValueError("K must be a multiple of 8")
    q = q.reshape(N, K // 8, 8)
    word = np.zeros((N, K // 8), dtype=np.uint32)
    for i in range(8):
        word |= q[:, :, i] << np.uint32(4 * i)
    return word


def pack_codes(q, bits):
    """uint q[N, K] of `bits`-wide codes (4 or 8) -> uint32 Wq[N, K*bits/32], field i of
    word j holding k = (32/bits)*j + i in bits bits*i .. bits*i + bits - 1."""
    per = 32 // bits
    q = np.asarray(q, dtype=np.uint32)
    N, K = q.shape
    if K % per:
        raise ValueError("K must be a multiple of %d" % per)
    q = q.reshape(N, K // per, per)
    word = np.zeros((N, K // per), dtype=np.uint32)
    for i in range(per):
        word |= q[:, :, i] << np.uint32(bits * i)
    return word


def wq_inputs(bits, group, M, N, K, seed):
    """A bf16[M,K], Wq uint32[N, K*bits/32], scale/bias bf16[N, K/group], plus q."""
    if K % GROUP or K % group:
        raise ValueError("K must be a multiple of 128 and of the group size")
    rng = rng_for(seed)
    A = f32_to_bf16_bits(rng.standard_normal((M, K), dtype=np.float32))
    q = rng.integers(0, 1 << bits, size=(N, K), dtype=np.uint16)
    lo, hi = (0.005, 0.02) if bits == 4 else (0.005 / 16, 0.02 / 16)
    scale = f32_to_bf16_bits(rng.uniform(lo, hi, size=(N, K // group)).astype(np.float32))
    bias = f32_to_bf16_bits(np.float32(-(1 << (bits - 1))) * bf16_bits_to_f32(scale))
    return dict(A=A, Wq=pack_codes(q, bits), scale=scale, bias=bias, q=q)


def attn_inputs(B, Mq, Hq, Hkv, Lmax, D, lengths, seed):
    """Decode attention inputs: Q [B, Mq, Hq, D], K and V caches [B, Hkv, Lmax, D], all
    N(0, 1) rounded to bf16 (positions past a request's length hold data too, never
    read); lengths int32 [B]."""
    rng = rng_for(seed)
    Q = f32_to_bf16_bits(rng.standard_normal((B, Mq, Hq, D), dtype=np.float32))
    K = f32_to_bf16_bits(rng.standard_normal((B, Hkv, Lmax, D), dtype=np.float32))
    V = f32_to_bf16_bits(rng.standard_normal((B, Hkv, Lmax, D), dtype=np.float32))
    return dict(Q=Q, K=K, V=V, lengths=np.asarray(lengths, dtype=np.int32))


def rng_for(seed):
    return np.random.Generator(np.random.PCG64(seed))


def w4a16_inputs(M, N, K, seed, scale_lo=0.005, scale_hi=0.02):
    """A bf16[M,K], Wq uint32[N,K/8], scale/bias bf16[N,K/128] (bias = -8*scale), plus q."""
    if K % GROUP:
        raise ValueError("K must be a multiple of 128")
    rng = rng_for(seed)
    A = f32_to_bf16_bits(rng.standard_normal((M, K), dtype=np.float32))
    q = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    scale = f32_to_bf16_bits(rng.uniform(scale_lo, scale_hi, size=(N, K // GROUP)).astype(np.float32))
    bias = f32_to_bf16_bits(np.float32(-8.0) * bf16_bits_to_f32(scale))
    return dict(A=A, Wq=pack_nibbles(q), scale=scale, bias=bias, q=q)


def w4a16_pow2_inputs(M, N, K, seed):
    """Like w4a16_inputs, but every scale is a power of two (2^-7, 2^-6 or 2^-5) and
    bias = -8*scale, so each dequantised weight (q - 8)*scale is exact in bf16 and each
    product with A exact in fp32: a single-cast kernel then differs from the correctly
    rounded result only through its fp32 accumulation."""
    d = w4a16_inputs(M, N, K, seed)
    rng = rng_for(seed + 0x5EED)
    e = rng.integers(-7, -4, size=d["scale"].shape)
    scale = np.ldexp(np.float32(1.0), e).astype(np.float32)
    d["scale"] = f32_to_bf16_bits(scale)
    d["bias"] = f32_to_bf16_bits(np.float32(-8.0) * scale)
    return d


def w4a16_weights(N, K, seed, scale_lo=0.005, scale_hi=0.02):
    """Weights only (for shapes where several activation sets share one weight set)."""
    rng = rng_for(seed)
    q = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    scale = f32_to_bf16_bits(rng.uniform(scale_lo, scale_hi, size=(N, K // GROUP)).astype(np.float32))
    bias = f32_to_bf16_bits(np.float32(-8.0) * bf16_bits_to_f32(scale))
    return dict(Wq=pack_nibbles(q), scale=scale, bias=bias, q=q)


def normal_bf16(shape, seed):
    return f32_to_bf16_bits(rng_for(seed).standard_normal(shape, dtype=np.float32))


def dense_inputs(M, N, K, seed):
    rng = rng_for(seed)
    A = f32_to_bf16_bits(rng.standard_normal((M, K), dtype=np.float32))
    B = f32_to_bf16_bits(rng.standard_normal((N, K), dtype=np.float32))
    return dict(A=A, B=B)


def bf16_planes(s, M, N, seed, sigma=1.0):
    """s partial planes [s, M, N] of bf16 N(0, sigma^2) values (reduce tests)."""
    return f32_to_bf16_bits(sigma * rng_for(seed).standard_normal((s, M, N), dtype=np.float32))


def f32_planes(s, M, N, seed, sigma=1.0):
    return (sigma * rng_for(seed).standard_normal((s, M, N), dtype=np.float32)).astype(np.float32)


def random_bf16_any(shape, seed, lo_exp=-6, hi_exp=6):
    """bf16 values with random sign, exponent in [lo_exp, hi_exp] and random
    7-bit fraction (brute-force tests exercise arbitrary scale/bias bits)."""
    rng = rng_for(seed)
    sign = rng.integers(0, 2, size=shape, dtype=np.uint16)
    exp = rng.integers(lo_exp, hi_exp + 1, size=shape).astype(np.int32) + 127
    frac = rng.integers(0, 128, size=shape, dtype=np.uint16)
    return ((sign << 15) | (exp.astype(np.uint16) << 7) | frac).astype(np.uint16)


# Qwen3-4B projection shapes (output width N <- reduction length K).
QWEN3_4B_PROJECTIONS = {
    "q": (4096, 2560),
    "k": (1024, 2560),
    "v": (1024, 2560),
    "o": (2560, 4096),
    "gate": (9728, 2560),
    "up": (9728, 2560),
    "down": (2560, 9728),
}
PROJECTION_ORDER = ("q", "k", "v", "o", "gate", "up", "down")
PREFILL_ROWS = (16, 32, 64, 128, 2048)
DECODE_ROWS = (1, 4, 8)


def projection_sweep():
    """Shapes of the prefill projection sweep, in listed order: (name, M, N, K, index)."""
    out = []
    idx = 0
    for name in PROJECTION_ORDER:
        N, K = QWEN3_4B_PROJECTIONS[name]
        for M in PREFILL_ROWS:
            out.append((name, M, N, K, idx))
            idx += 1
    return out


def decode_sweep():
    """Decode / speculative-decode shapes: down and gate at M in {1, 4, 8}."""
    out = []
    idx = 0
    for name in ("down", "gate"):
        N, K = QWEN3_4B_PROJECTIONS[name]
        for M in DECODE_ROWS:
            out.append((name, M, N, K, idx))
            idx += 1
    return out
