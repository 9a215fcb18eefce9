"""Pins of the CPU oracle to facts fixed outside the oracle itself.

Each test checks the oracle against something it cannot agree with by
construction: exact rational arithmetic (brute force), closed forms, a library
routine (numpy / torch on the CPU), the values the pages print for their worked
examples (tests/golden/*.json), or an invariant of the mathematics. Together
they are chosen so that a plausible slip in the oracle (nibble order, group
index, a dropped bias, a transposed operand, a wrong partition bound, the
reduce order or rounding) fails at least one of them; test_oracle_mutants.py
plants such slips and checks that they are caught.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import qmm_synth as syn
from oracle import models, policy

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
U53 = 2.0 ** -53


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def gamma(n):
    """Higham's gamma_n for fp64: bound on the relative error of an n-term sum."""
    return n * U53 / (1 - n * U53)


def bf16_fraction(bits):
    """Exact rational value of a bf16 pattern, decoded field by field."""
    bits = int(bits)
    sign = -1 if bits & 0x8000 else 1
    exp = (bits >> 7) & 0xFF
    frac = bits & 0x7F
    if exp == 0:
        return sign * Fraction(frac, 128) * Fraction(2) ** -126
    assert exp != 0xFF
    return sign * (1 + Fraction(frac, 128)) * Fraction(2) ** (exp - 127)


# ---------------------------------------------------------------- bf16 helpers

def test_bf16_value_matches_torch():
    bits = np.arange(0, 1 << 16, 7, dtype=np.int64)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF].astype(np.uint16)  # finite only
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.bf16_value(b) for b in bits])
    assert np.array_equal(got, ref)


def test_bf16_round_matches_torch_on_fp32():
    rng = np.random.default_rng(11)
    x = np.concatenate([
        rng.standard_normal(4000).astype(np.float32) * np.float32(10.0) ** rng.integers(-30, 30, 4000).astype(np.float32),
        np.array([0.0, -0.0, 1.0, -1.0, 3.0e38, -3.0e38, 1e-39, -1e-39, 1e-44], dtype=np.float32),
    ]).astype(np.float32)
    # exact ties: a bf16 value plus half its spacing, both parities of the last bit
    base = syn.bf16_bits_to_f32(np.array([0x3F80, 0x3F81, 0x4120, 0x4121, 0xC2F7, 0xC2F8], dtype=np.uint16))
    _, e = np.frexp(base.astype(np.float64))
    spacing = np.ldexp(1.0, e - 8).astype(np.float32)  # bf16 spacing around |base|
    ties = (base + np.sign(base) * spacing / np.float32(2)).astype(np.float32)
    x = np.concatenate([x, ties]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.bf16_round(float(v)) for v in x], dtype=np.uint16)
    assert np.array_equal(got, ref)


def test_bf16_round_ties_to_even_by_hand():
    # 1 + 2^-8 lies halfway between 1 (even significand) and 1 + 2^-7 (odd): rounds to 1.
    assert oracle.bf16_round(1.0 + 2.0 ** -8) == 0x3F80
    # 1 + 3*2^-8 lies halfway between 1 + 2^-7 (odd) and 1 + 2^-6 (even): rounds up.
    assert oracle.bf16_round(1.0 + 3 * 2.0 ** -8) == 0x3F82
    assert oracle.bf16_round(-0.0) == 0x8000


# ---------------------------------------------------------- nibble / dequant

def test_nibble_order_golden():
    g = load_golden("nibble_order.json")
    Wq = np.array([g["words"]], dtype=np.uint32)  # one row, K = 8 * words
    K = 8 * Wq.shape[1]
    for j, expect in enumerate(g["q"]):
        got = [oracle.nibble(Wq, K, 0, 8 * j + i) for i in range(8)]
        assert got == expect
    assert [int(x) for x in g["words"]] == [int(h, 16) for h in g["words_hex"]]


def test_dequant_matches_generator_fields_exactly():
    d = syn.w4a16_inputs(3, 5, 256, seed=7)
    w = oracle.dequant_w4a16(d["Wq"], d["scale"], d["bias"], 5, 256)
    sc = syn.bf16_bits_to_f32(d["scale"]).astype(np.float64)
    bi = syn.bf16_bits_to_f32(d["bias"]).astype(np.float64)
    g = np.arange(256) // 128
    expect = sc[:, g] * d["q"].astype(np.float64) + bi[:, g]
    assert np.array_equal(w, expect)
    # with bias = -8*scale the weight is scale*(q-8) exactly
    assert np.array_equal(w, sc[:, g] * (d["q"].astype(np.float64) - 8.0))


# ------------------------------------------------------------- brute force

@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (2, 3, 256), (3, 5, 384), (1, 4, 128)])
def test_bruteforce_exact_rationals(M, N, K):
    seed = 100 + M * 10 + N + K
    d = syn.w4a16_inputs(M, N, K, seed=seed)
    G = K // 128
    # arbitrary scale and bias bit patterns, not tied to each other
    scale = syn.random_bf16_any((N, G), seed + 1, -8, 2)
    bias = syn.random_bf16_any((N, G), seed + 2, -8, 2)
    q = d["q"]
    A = d["A"]
    Af = [[bf16_fraction(A[m, k]) for k in range(K)] for m in range(M)]
    exact = [[None] * N for _ in range(M)]
    absum = [[None] * N for _ in range(M)]
    for n in range(N):
        w = [bf16_fraction(scale[n, k // 128]) * int(q[n, k]) + bf16_fraction(bias[n, k // 128])
             for k in range(K)]
        for m in range(M):
            terms = [Af[m][k] * w[k] for k in range(K)]
            exact[m][n] = sum(terms, Fraction(0))
            absum[m][n] = sum((abs(t) for t in terms), Fraction(0))
    for s in [x for x in range(1, G + 1) if G % x == 0]:
        C = oracle.qmm_w4a16(A, d["Wq"], scale, bias, M, N, K, s=s, nthreads=2)
        for m in range(M):
            for n in range(N):
                err = abs(Fraction(C[m, n]) - exact[m][n])
                assert err <= Fraction(gamma(K)) * absum[m][n], (m, n, s)


def test_bruteforce_dense_exact_rationals():
    M, N, K = 3, 2, 96
    d = syn.dense_inputs(M, N, K, seed=5)
    exact = [[sum((bf16_fraction(d["A"][m, k]) * bf16_fraction(d["B"][n, k]) for k in range(K)),
                  Fraction(0)) for n in range(N)] for m in range(M)]
    absum = [[sum((abs(bf16_fraction(d["A"][m, k]) * bf16_fraction(d["B"][n, k])) for k in range(K)),
                  Fraction(0)) for n in range(N)] for m in range(M)]
    for s in (1, 2, 3):
        C = oracle.qmm_dense(d["A"], d["B"], M, N, K, s=s, nthreads=1)
        for m in range(M):
            for n in range(N):
                assert abs(Fraction(C[m, n]) - exact[m][n]) <= Fraction(gamma(K)) * absum[m][n]


# -------------------------------------------------------------- invariants

def _abs_terms(d, N, K):
    w = np.abs(syn.bf16_bits_to_f32(d["scale"]).astype(np.float64)[:, np.arange(K) // 128]
               * (d["q"].astype(np.float64) - 8.0))
    a = np.abs(syn.bf16_bits_to_f32(d["A"]).astype(np.float64))
    return a @ w.T


@pytest.mark.parametrize("M,N,K,seed", [(32, 1024, 2560, 0), (48, 1000, 2560, 1000)])
def test_split_invariance_config_shapes(M, N, K, seed):
    d = syn.w4a16_inputs(M, N, K, seed=seed)
    G = K // 128
    C1 = oracle.qmm_w4a16(d["A"], d["Wq"], d["scale"], d["bias"], M, N, K, s=1)
    bound = 2 * gamma(K) * _abs_terms(d, N, K)
    for s in [x for x in range(2, G + 1) if G % x == 0]:
        Cs = oracle.qmm_w4a16(d["A"], d["Wq"], d["scale"], d["bias"], M, N, K, s=s)
        assert np.all(np.abs(Cs - C1) <= bound), s


def test_split_rejects_unequal_partitions():
    d = syn.w4a16_inputs(2, 3, 2560, seed=3)
    with pytest.raises(ValueError):
        oracle.qmm_w4a16(d["A"], d["Wq"], d["scale"], d["bias"], 2, 3, 2560, s=3)
    with pytest.raises(ValueError):
        oracle.qmm_w4a16(d["A"], d["Wq"], d["scale"], d["bias"], 2, 3, 2560, s=40)


# ------------------------------------------------------------ closed forms

def _const_words(N, K, nib):
    word = 0
    for i in range(8):
        word |= nib << (4 * i)
    return np.full((N, K // 8), word, dtype=np.uint32)


@pytest.mark.parametrize("s", [1, 2, 4, 5, 10, 20])
def test_closed_form_zero_weights(s):
    M, N, K = 5, 7, 2560
    d = syn.w4a16_inputs(M, N, K, seed=21)
    Wq = _const_words(N, K, 8)  # q == 8 with bias = -8*scale -> w == 0
    C = oracle.qmm_w4a16(d["A"], Wq, d["scale"], d["bias"], M, N, K, s=s)
    assert np.all(C == 0.0)


def test_closed_form_ones_times_nine():
    M, N, K = 3, 6, 1024
    d = syn.w4a16_inputs(M, N, K, seed=22)
    A = np.full((M, K), 0x3F80, dtype=np.uint16)  # 1.0
    Wq = _const_words(N, K, 9)  # q == 9 -> w = scale*(9-8) = scale
    C = oracle.qmm_w4a16(A, Wq, d["scale"], d["bias"], M, N, K, s=1)
    sc = syn.bf16_bits_to_f32(d["scale"]).astype(np.float64)
    expect = 128.0 * sc.sum(axis=1)
    assert np.array_equal(C, np.broadcast_to(expect, (M, N)))


@pytest.mark.parametrize("s", [1, 2, 4])
def test_closed_form_one_hot_rows(s):
    M, N, K = 9, 11, 512
    d = syn.w4a16_inputs(M, N, K, seed=23)
    A = np.zeros((M, K), dtype=np.uint16)
    ks = [0, 7, 8, 127, 128, 255, 300, 384, 511]
    for m, k in enumerate(ks):
        A[m, k] = 0x3F80
    C = oracle.qmm_w4a16(A, d["Wq"], d["scale"], d["bias"], M, N, K, s=s)
    sc = syn.bf16_bits_to_f32(d["scale"]).astype(np.float64)
    bi = syn.bf16_bits_to_f32(d["bias"]).astype(np.float64)
    for m, k in enumerate(ks):
        expect = sc[:, k // 128] * d["q"][:, k] + bi[:, k // 128]
        assert np.array_equal(C[m], expect)


def test_integer_weights_equal_numpy_matmul():
    M, N, K = 16, 40, 1024
    d = syn.w4a16_inputs(M, N, K, seed=24)
    ones = np.full((N, K // 128), 0x3F80, dtype=np.uint16)
    zeros = np.zeros((N, K // 128), dtype=np.uint16)
    C = oracle.qmm_w4a16(d["A"], d["Wq"], ones, zeros, M, N, K, s=1)
    a = syn.bf16_bits_to_f32(d["A"]).astype(np.float64)
    ref = a @ d["q"].astype(np.float64).T
    bound = gamma(K) * (np.abs(a) @ d["q"].astype(np.float64).T)
    assert np.all(np.abs(C - ref) <= 2 * bound)


def test_dense_equals_numpy_matmul_and_split_invariant():
    M, N, K = 24, 40, 2048
    d = syn.dense_inputs(M, N, K, seed=25)
    a = syn.bf16_bits_to_f32(d["A"]).astype(np.float64)
    b = syn.bf16_bits_to_f32(d["B"]).astype(np.float64)
    ref = a @ b.T
    bound = 2 * gamma(K) * (np.abs(a) @ np.abs(b).T)
    for s in (1, 2, 4, 6, 8, 12, 16, 32):
        C = oracle.qmm_dense(d["A"], d["B"], M, N, K, s=s)
        assert np.all(np.abs(C - ref) <= bound), s


def test_points_match_full_product():
    M, N, K = 7, 13, 768
    d = syn.w4a16_inputs(M, N, K, seed=26)
    C = oracle.qmm_w4a16(d["A"], d["Wq"], d["scale"], d["bias"], M, N, K, s=1)
    ms = np.array([0, 6, 3, 5, 1], dtype=np.int32)
    ns = np.array([0, 12, 7, 2, 11], dtype=np.int32)
    pts = oracle.qmm_w4a16_points(d["A"], d["Wq"], d["scale"], d["bias"], M, N, K, ms, ns)
    assert np.array_equal(pts, C[ms, ns])


# ------------------------------------------------- other weight formats

FORMATS = [(4, 32), (4, 64), (4, 128), (8, 32), (8, 64), (8, 128)]


def test_code_order_golden():
    g = load_golden("code_order.json")
    for bits, key in ((8, "w8"), (4, "w4")):
        Wq = np.array([[int(h, 16) for h in g[key]["words_hex"]]], dtype=np.uint32)
        per = 32 // bits
        K = per * Wq.shape[1]
        for j, expect in enumerate(g[key]["q"]):
            assert [oracle.code(Wq, bits, K, 0, per * j + i) for i in range(per)] == expect, (bits, j)


@pytest.mark.parametrize("bits,group", FORMATS)
def test_format_dequant_matches_generator_fields(bits, group):
    N, K = 5, 256
    d = syn.wq_inputs(bits, group, 2, N, K, seed=40 + bits + group)
    w = oracle.dequant_wq(d["Wq"], bits, group, d["scale"], d["bias"], N, K)
    sc = syn.bf16_bits_to_f32(d["scale"]).astype(np.float64)
    g = np.arange(K) // group
    # bias = -2^(bits-1) * scale, so the weight is scale * (q - 2^(bits-1)) exactly
    assert np.array_equal(w, sc[:, g] * (d["q"].astype(np.float64) - (1 << (bits - 1))))


@pytest.mark.parametrize("bits,group", [(4, 32), (4, 64), (8, 32), (8, 64), (8, 128)])
def test_format_bruteforce_exact_rationals(bits, group):
    M, N, K = 2, 3, 256
    seed = 300 + bits * 10 + group
    d = syn.wq_inputs(bits, group, M, N, K, seed=seed)
    scale = syn.random_bf16_any((N, K // group), seed + 1, -10, 0)
    bias = syn.random_bf16_any((N, K // group), seed + 2, -4, 4)
    q, A = d["q"], d["A"]
    Af = [[bf16_fraction(A[m, k]) for k in range(K)] for m in range(M)]
    for n in range(N):
        w = [bf16_fraction(scale[n, k // group]) * int(q[n, k]) + bf16_fraction(bias[n, k // group])
             for k in range(K)]
        for m in range(M):
            terms = [Af[m][k] * w[k] for k in range(K)]
            exact = sum(terms, Fraction(0))
            absum = sum((abs(t) for t in terms), Fraction(0))
            for s in (1, 2):
                C = oracle.qmm_wq(bits, group, A, d["Wq"], scale, bias, M, N, K, s=s, nthreads=1)
                assert abs(Fraction(C[m, n]) - exact) <= Fraction(gamma(K)) * absum, (m, n, s)


@pytest.mark.parametrize("bits,group", FORMATS)
def test_format_one_hot_rows(bits, group):
    M, N, K = 8, 7, 512
    d = syn.wq_inputs(bits, group, M, N, K, seed=50 + bits + group)
    ks = [0, 31, 32, 63, 64, 127, 200, 511]
    A = np.zeros((M, K), dtype=np.uint16)
    for m, k in enumerate(ks):
        A[m, k] = 0x3F80
    sc = syn.bf16_bits_to_f32(d["scale"]).astype(np.float64)
    bi = syn.bf16_bits_to_f32(d["bias"]).astype(np.float64)
    for s in (1, 4):
        C = oracle.qmm_wq(bits, group, A, d["Wq"], d["scale"], d["bias"], M, N, K, s=s)
        for m, k in enumerate(ks):
            assert np.array_equal(C[m], sc[:, k // group] * d["q"][:, k] + bi[:, k // group]), (m, s)


@pytest.mark.parametrize("bits", [4, 8])
def test_format_integer_weights_equal_numpy_matmul(bits):
    M, N, K = 12, 20, 512
    d = syn.wq_inputs(bits, 64, M, N, K, seed=60 + bits)
    ones = np.full((N, K // 64), 0x3F80, dtype=np.uint16)
    zeros = np.zeros((N, K // 64), dtype=np.uint16)
    C = oracle.qmm_wq(bits, 64, d["A"], d["Wq"], ones, zeros, M, N, K, s=1)
    a = syn.bf16_bits_to_f32(d["A"]).astype(np.float64)
    qf = d["q"].astype(np.float64)
    assert np.all(np.abs(C - a @ qf.T) <= 2 * gamma(K) * (np.abs(a) @ qf.T))


def test_format_w4_g128_is_the_w4a16_product():
    M, N, K = 6, 9, 640
    d = syn.w4a16_inputs(M, N, K, seed=70)
    for s in (1, 5):
        a = oracle.qmm_w4a16(d["A"], d["Wq"], d["scale"], d["bias"], M, N, K, s=s)
        b = oracle.qmm_wq(4, 128, d["A"], d["Wq"], d["scale"], d["bias"], M, N, K, s=s)
        assert np.array_equal(a, b)


def test_format_points_match_full_product_and_rejects():
    M, N, K = 5, 6, 384
    d = syn.wq_inputs(8, 32, M, N, K, seed=71)
    C = oracle.qmm_wq(8, 32, d["A"], d["Wq"], d["scale"], d["bias"], M, N, K)
    ms = np.array([0, 4, 2], dtype=np.int32)
    ns = np.array([5, 0, 3], dtype=np.int32)
    assert np.array_equal(oracle.qmm_wq_points(8, 32, d["A"], d["Wq"], d["scale"], d["bias"], M, N, K, ms, ns),
                          C[ms, ns])
    for bits, group, KK in ((5, 128, 384), (8, 16, 384), (8, 256, 512)):
        with pytest.raises(ValueError):
            oracle.qmm_wq(bits, group, d["A"], d["Wq"], d["scale"], d["bias"], M, N, KK)
    with pytest.raises(ValueError):  # 3 blocks of 128 do not split in two
        oracle.qmm_wq(8, 32, d["A"], d["Wq"], d["scale"], d["bias"], M, N, K, s=2)


# ------------------------------------------------------- decode attention

def _attn(B=2, Mq=1, Hq=8, Hkv=2, Lmax=40, D=16, lengths=(40, 17), seed=80):
    return syn.attn_inputs(B, Mq, Hq, Hkv, Lmax, D, list(lengths), seed)


def test_attn_single_key_returns_its_value_row():
    d = _attn(lengths=(1, 1))
    O = oracle.attn_decode(d["Q"], d["K"], d["V"], d["lengths"], 0.25)
    V = syn.bf16_bits_to_f32(d["V"]).astype(np.float64)
    for h in range(8):
        assert np.array_equal(O[:, 0, h], V[:, h // 4, 0])


def test_attn_zero_query_averages_the_allowed_values():
    d = _attn(lengths=(40, 17))
    d["Q"][:] = 0
    O = oracle.attn_decode(d["Q"], d["K"], d["V"], d["lengths"], 0.125)
    V = syn.bf16_bits_to_f32(d["V"]).astype(np.float64)
    for b, L in enumerate((40, 17)):
        for h in range(8):
            ref = V[b, h // 4, :L].mean(axis=0)
            assert np.all(np.abs(O[b, 0, h] - ref) <= 64 * U53 * np.abs(V[b, h // 4, :L]).mean(axis=0)), (b, h)


def test_attn_two_keys_closed_form():
    d = _attn(B=1, Hq=2, Hkv=1, Lmax=2, D=16, lengths=(2,), seed=81)
    scale = 0.3
    O = oracle.attn_decode(d["Q"], d["K"], d["V"], d["lengths"], scale)
    for h in range(2):
        q = [bf16_fraction(x) for x in d["Q"][0, 0, h]]
        s = [float(scale * sum(a * bf16_fraction(k) for a, k in zip(q, d["K"][0, 0, j]))) for j in range(2)]
        w1 = math.exp(s[1] - s[0])
        v = syn.bf16_bits_to_f32(d["V"][0, 0]).astype(np.float64)
        ref = (v[0] + w1 * v[1]) / (1.0 + w1)
        assert np.all(np.abs(O[0, 0, h] - ref) <= 1e-14 * (np.abs(v[0]) + np.abs(v[1]))), h


def test_attn_query_heads_share_their_group_key_value_head():
    # uniform weights (Q = 0) and value rows equal to the index of their key/value head
    d = _attn(B=1, Hq=12, Hkv=3, lengths=(40,))
    d["Q"][:] = 0
    for g in range(3):
        d["V"][0, g] = syn.f32_to_bf16_bits(np.full((40, 16), float(g), dtype=np.float32))
    O = oracle.attn_decode(d["Q"], d["K"], d["V"], d["lengths"], 1.0)
    for h in range(12):
        assert np.all(O[0, 0, h] == float(h // 4)), h


def test_attn_dominant_key_selects_its_value():
    d = _attn(B=1, Hq=4, Hkv=1, lengths=(40,), seed=82)
    q = syn.bf16_bits_to_f32(d["Q"][0, 0, 0]).astype(np.float64)
    d["Q"][0, 0, 1:] = d["Q"][0, 0, 0]
    # key 23 = 8 * q (bf16-exact): its score exceeds every other by > 30 at scale 1
    d["K"][0, 0, 23] = syn.f32_to_bf16_bits((8.0 * q).astype(np.float32))
    O = oracle.attn_decode(d["Q"], d["K"], d["V"], d["lengths"], 1.0)
    V = syn.bf16_bits_to_f32(d["V"][0, 0]).astype(np.float64)
    s = syn.bf16_bits_to_f32(d["K"][0, 0]).astype(np.float64) @ q
    gap = s[23] - np.max(np.delete(s, 23))
    assert gap > 30
    assert np.all(np.abs(O[0, 0, 0] - V[23]) <= 40 * math.exp(-gap) * np.abs(V).max())


def test_attn_causal_queries_match_shorter_histories():
    d = _attn(B=2, Mq=3, lengths=(40, 17), seed=83)
    O = oracle.attn_decode(d["Q"], d["K"], d["V"], d["lengths"], 0.25)
    for i in range(3):
        one = dict(d)
        one["Q"] = np.ascontiguousarray(d["Q"][:, i:i + 1])
        L = np.array([40 - 2 + i, 17 - 2 + i], dtype=np.int32)
        Oi = oracle.attn_decode(one["Q"], d["K"], d["V"], L, 0.25)
        assert np.array_equal(O[:, i], Oi[:, 0]), i


def test_attn_permuting_keys_with_values_changes_nothing():
    d = _attn(B=1, lengths=(40,), seed=84)
    O = oracle.attn_decode(d["Q"], d["K"], d["V"], d["lengths"], 0.25)
    perm = np.random.default_rng(84).permutation(40)
    d2 = dict(d)
    d2["K"] = np.ascontiguousarray(d["K"][:, :, perm])
    d2["V"] = np.ascontiguousarray(d["V"][:, :, perm])
    O2 = oracle.attn_decode(d2["Q"], d2["K"], d2["V"], d["lengths"], 0.25)
    V = syn.bf16_bits_to_f32(d["V"]).astype(np.float64)
    assert np.all(np.abs(O - O2) <= 1e-13 * np.abs(V).max())


def test_attn_rejects_bad_arguments():
    d = _attn(lengths=(40, 17))
    with pytest.raises(ValueError):
        oracle.attn_decode(d["Q"], d["K"], d["V"], np.array([41, 17], dtype=np.int32), 1.0)
    d3 = _attn(Mq=3, lengths=(40, 2))
    with pytest.raises(ValueError):  # fewer keys than queries
        oracle.attn_decode(d3["Q"], d3["K"], d3["V"], d3["lengths"], 1.0)


# ---------------------------------------------------------------- reduction

@pytest.mark.parametrize("s,M,N", [(1, 3, 5), (2, 16, 64), (5, 48, 1000), (20, 7, 33), (32, 4, 9)])
def test_reduce_bf16_matches_torch(s, M, N):
    planes = syn.bf16_planes(s, M, N, seed=s * 1000 + M + N)
    got = oracle.reduce_bf16(planes, s, M * N)
    t = torch.from_numpy(planes.reshape(s, -1).view(np.int16)).view(torch.bfloat16).to(torch.float32)
    acc = t[0].clone()
    for p in range(1, s):
        acc = acc + t[p]
    ref = acc.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)


def test_reduce_bf16_is_fp32_then_one_cast():
    # planes 1 + 2^-7, -2^-8, 2^-30: exact sum 1 + 2^-8 + 2^-30 lies just above the bf16 tie
    # between 1 and 1 + 2^-7 and would round up; in fp32 the 2^-30 term is lost (below half
    # an fp32 ulp of 1), leaving the exact tie 1 + 2^-8, which rounds to the even 1.0.
    vals = np.array([[0x3F81], [0xBB80], [0x3080]], dtype=np.uint16)
    assert oracle.reduce_bf16(vals, 3, 1)[0] == 0x3F80
    # planes 1 + 2^-7, -2^-8: the fp32 sum 1 + 2^-8 is a tie -> even significand (1.0)
    vals = np.array([[0x3F81], [0xBB80]], dtype=np.uint16)
    assert oracle.reduce_bf16(vals, 2, 1)[0] == 0x3F80
    # all-negative-zero planes keep the sign of zero (ascending sum starts at plane 0)
    vals = np.array([[0x8000], [0x8000]], dtype=np.uint16)
    assert oracle.reduce_bf16(vals, 2, 1)[0] == 0x8000


@pytest.mark.parametrize("s,M,N", [(1, 4, 8), (6, 32, 40), (32, 5, 7)])
def test_reduce_f32_matches_torch(s, M, N):
    planes = syn.f32_planes(s, M, N, seed=77 + s, sigma=50.0)
    got = oracle.reduce_f32(planes, s, M * N)
    t = torch.from_numpy(planes.reshape(s, -1))
    acc = t[0].clone()
    for p in range(1, s):
        acc = acc + t[p]
    ref = acc.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)


# --------------------------------------------------------------- partitions

def test_group_partitions_equal_and_covering():
    for G in (1, 20, 32, 76):
        for s in [x for x in range(1, G + 1) if G % x == 0]:
            bounds = [oracle.partition_groups(G, s, p) for p in range(s)]
            assert bounds[0][0] == 0 and bounds[-1][1] == G
            assert all(b[1] - b[0] == G // s for b in bounds)
            assert all(bounds[p][1] == bounds[p + 1][0] for p in range(s - 1))
    with pytest.raises(ValueError):
        oracle.partition_groups(20, 3, 0)


def test_granule_partitions_near_equal():
    U = 16384 // 32
    b = [oracle.partition_granules(U, 6, p) for p in range(6)]
    assert [e - s for s, e in b] == [85, 85, 86, 85, 85, 86]
    for s in (1, 2, 4, 6, 8, 12, 16, 32):
        b = [oracle.partition_granules(U, s, p) for p in range(s)]
        lens = [e - st for st, e in b]
        assert sum(lens) == U and max(lens) - min(lens) <= 1
        assert all(b[p][1] == b[p + 1][0] for p in range(s - 1))


# ----------------------------------------------------- the pages' examples

def test_policy_page_worked_example():
    g = load_golden("policy_page_worked_example.json")
    r = g["rule"]
    for M, expect in g["expected_split"].items():
        for name, s_expect in expect.items():
            N, K = g["projections"][name]
            s = policy.split_count(int(M), N, K, tile_m=r["tile_m"], tile_n=r["tile_n"],
                                   target=r["target"], cap=r["cap"],
                                   min_k_per_split=r["min_k_per_split"])
            assert s == s_expect, (M, name, s)
    for name, M in g["fallback_shapes_base_at_least_target"]:
        N, K = g["projections"][name]
        assert policy.base_tiles(M, N, r["tile_m"], r["tile_n"]) >= r["target"]
        assert policy.split_count(M, N, K, **{k: r[k] for k in ("tile_m", "tile_n", "target", "cap", "min_k_per_split")}) == 1


def test_policy_rule_details():
    # cfg shapes under the page rule: K projection at M=32 -> base 32 -> 10 ways;
    # the ragged N=1000 at M=48 -> base 2*32 = 64 -> 5 ways (20 groups).
    assert policy.split_count(32, 1024, 2560) == 10
    assert policy.split_count(48, 1000, 2560) == 5
    # divisibility walk: 76 groups, floor(320/20) = 16 -> 16, 15, ..., 4 divides 76
    assert policy.split_count(16, 640, 9728) == 4
    # never above the group count
    assert policy.split_count(1, 32, 256) == 2
    with pytest.raises(ValueError):
        policy.split_count(1, 32, 200)


def test_wave_model_golden():
    g = load_golden("a100_splitk_model.json")
    sh = g["shape"]
    for row in g["rows"]:
        r = models.splitk_wave_model(row["s"], m=sh["m"], n=sh["n"], k=sh["k"], tile_m=sh["tile_m"],
                                     tile_n=sh["tile_n"], sms=g["a100_sms"])
        assert r["blocks"] == row["blocks"]
        assert r["waves"] == row["waves"]
        tol = 10.0 ** -row["printed_decimals"]
        assert abs(r["time_s"] * 1e6 - row["time_us"]) <= tol, row
    # unsplit: 16 blocks on 108 SMs leave 85 % idle
    assert round(models.idle_fraction(16, g["a100_sms"]), 2) == g["idle_fraction_unsplit"]
    # the best split is the largest single-wave one: 6 on the A100, 8 on the H100
    for sms, best in ((g["a100_sms"], g["best_single_wave_split_a100"]),
                      (g["h100_sms"], g["h100_largest_single_wave_split"])):
        single = [s for s in range(1, 33) if models.splitk_wave_model(s, sms=sms)["waves"] == 1]
        assert max(single) == best
    times = {s: models.splitk_wave_model(s)["time_s"] for s in range(1, 13)}
    assert min(times, key=times.get) == g["best_single_wave_split_a100"]


def test_overlap_model_golden():
    g = load_golden("overlap_model.json")
    n, tl, tc, ts = g["tiles"], g["t_load"], g["t_comp"], g["t_store"]
    t1 = models.overlap_schedule(n, tl, tc, ts, buffers=1)
    t2 = models.overlap_schedule(n, tl, tc, ts, buffers=2)
    t3 = models.overlap_schedule(n, tl, tc, ts, buffers=3)
    assert t1 == g["single_buffer_time"] == models.single_buffer_closed_form(n, tl, tc, ts)
    assert t2 == g["double_buffer_time"] == models.overlap_closed_form(n, tl, tc, ts)
    assert round(t1 / t2, 2) == g["speedup"]
    assert (t3 == t2) == g["third_buffer_changes_nothing"]


def test_overlap_closed_form_exact_when_compute_slowest():
    rng = np.random.default_rng(3)
    for _ in range(200):
        tc = float(rng.integers(3, 9))
        tl = float(rng.integers(1, int(tc) + 1))
        ts = float(rng.integers(1, int(tc) + 1))
        n = int(rng.integers(1, 12))
        for b in (2, 3):
            assert models.overlap_schedule(n, tl, tc, ts, b) == models.overlap_closed_form(n, tl, tc, ts)
