"""Pins of the fp64 oracle against facts fixed outside the oracle itself:
values the pages print, closed forms, brute force on tiny inputs, special cases
that reduce to a textbook identity or a library routine, and invariants.
Each pin is chosen so that a plausible slip in the oracle (a dropped term, a
flipped sign, a wrong index, a transposed operand) fails at least one of them."""
import json
import math
import os

import numpy as np
import pytest

import datagen
import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# number formats
# ---------------------------------------------------------------------------

def test_round_bf16_matches_integer_rne_on_fp32_inputs():
    v = datagen.normal_f32((99, 0), (20000,), 3.0)
    v[:100] *= np.float32(1e-38)       # bf16 subnormal range
    v[100:200] *= np.float32(1e30)
    ref = datagen.bf16_bits_to_f32(datagen.bf16_bits_from_f32(v)).astype(np.float64)
    got = oracle.round_bf16(v.astype(np.float64))
    assert np.array_equal(got, ref)


def test_round_bf16_rounds_once_from_fp64():
    # exact midpoints go to the even neighbour
    lo = np.float64(1.0)
    mid = lo + 2.0 ** -8
    assert oracle.round_bf16(np.array([mid]))[0] == 1.0
    assert oracle.round_bf16(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2 * 2.0 ** -7
    # just above a midpoint by less than fp32 resolution: a route through fp32
    # would land on the midpoint and round to even (down); direct rounding goes up
    v = mid + 2.0 ** -40
    assert np.float32(v) == np.float32(mid)
    assert oracle.round_bf16(np.array([v]))[0] == 1.0 + 2.0 ** -7


def test_numpy_fp16_rounding_is_direct_nearest_even():
    # scales are rounded by numpy's fp64 -> fp16 cast; pin that it is a single
    # nearest-even rounding over every finite positive fp16 interval
    h = np.arange(1, 0x7BFF, dtype=np.uint16).view(np.float16).astype(np.float64)
    nxt = np.arange(2, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    mid = (h + nxt) / 2.0
    r_mid = mid.astype(np.float16).view(np.uint16)
    expect_mid = np.where(np.arange(1, 0x7BFF) % 2 == 0, np.arange(1, 0x7BFF), np.arange(2, 0x7C00)).astype(np.uint16)
    assert np.array_equal(r_mid, expect_mid)
    up = (mid + (nxt - h) * 2.0 ** -30).astype(np.float16).view(np.uint16)
    assert np.array_equal(up, np.arange(2, 0x7C00, dtype=np.uint16))
    dn = (mid - (nxt - h) * 2.0 ** -30).astype(np.float16).view(np.uint16)
    assert np.array_equal(dn, np.arange(1, 0x7BFF, dtype=np.uint16))


# ---------------------------------------------------------------------------
# S1 pack
# ---------------------------------------------------------------------------

def test_sign_convention_and_bit_order():
    g = _gold("sign1_format.json")
    w = np.ones((2, 128), dtype=np.float32)
    w[0, 0] = -1.0       # bit 0 of word 0
    w[0, 63] = -0.0      # IEEE sign bit set on negative zero
    w[0, 64] = -2.5      # bit 0 of word 1
    w[1, 127] = -1e-30   # bit 63 of word 1
    w[1, 5] = 0.0
    words, scales = oracle.pack_sign1(w)
    assert words.dtype == np.uint64 and words.shape == (2, 128 // g["signs_per_word"])
    assert int(words[0, 0]) == (1 << 0) | (1 << 63)
    assert int(words[0, 1]) == 1
    assert int(words[1, 0]) == 0
    assert int(words[1, 1]) == 1 << 63
    # +1 -> bit 0, -1 -> bit 1
    one = oracle.pack_sign1_only(np.full((1, 64), 1.0, np.float32))
    neg = oracle.pack_sign1_only(np.full((1, 64), -1.0, np.float32))
    assert int(one[0, 0]) == 0 if g["bit_for_plus_one"] == 0 else False
    assert int(neg[0, 0]) == (1 << 64) - 1 and g["bit_for_minus_one"] == 1
    # unpack is the inverse and maps bit 1 -> -1
    s = oracle.unpack_signs(words, 2, 128)
    assert s[0, 0] == -1 and s[0, 1] == 1 and s[0, 63] == -1 and s[0, 64] == -1 and s[1, 127] == -1


def test_scale_is_best_fp16_by_exhaustive_search():
    """The stored scale minimises sum (w - a*sign(w))^2 over every finite
    non-negative fp16 a (brute force over all 31744 candidates)."""
    cand = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    G = 8
    for i in range(200):
        w = datagen.normal_f32((98, i), (1, G), 0.02 * (1 + i % 7))
        s = np.where(np.signbit(w[0]), -1.0, 1.0)
        w64 = w[0].astype(np.float64)
        f = ((w64[None, :] - cand[:, None] * s[None, :]) ** 2).sum(axis=1)
        best = cand[np.argmin(f)]
        got = oracle.group_mean_abs(w, G).astype(np.float16).astype(np.float64)[0, 0]
        assert got == best, (i, got, best)


def test_signs_are_best_pattern_by_exhaustive_search():
    """Over all 2^G sign patterns, each with its own least-squares scale
    (numpy.linalg.lstsq), the best pattern is sign(w) and its scale mean|w|."""
    G = 10
    pats = 1.0 - 2.0 * ((np.arange(2 ** G)[:, None] >> np.arange(G)[None, :]) & 1)
    for i in range(20):
        w = datagen.normal_f32((97, i), (G,), 1.0).astype(np.float64)
        best_r, best_p, best_a = None, None, None
        for p in pats:
            a, res, *_ = np.linalg.lstsq(p[:, None], w, rcond=None)
            r = float(np.sum((w - a[0] * p) ** 2))
            if best_r is None or r < best_r - 1e-15:
                best_r, best_p, best_a = r, p, a[0]
        if best_a < 0:  # the pattern and its negation fit equally; keep a >= 0
            best_p, best_a = -best_p, -best_a
        assert np.array_equal(best_p, np.where(w < 0, -1.0, 1.0))
        assert abs(best_a - oracle.group_mean_abs(w[None, :].astype(np.float32), G)[0, 0]) < 1e-7


def test_round_trip_exact_on_pm_a_groups():
    N, K = 8, 512
    a = np.array([0.5, 0.015625, 3.0, 1e-3, 65504.0, 6.1035156e-05, 0.0123, 7.0], dtype=np.float16)
    sgn = datagen.pm1_f32((96, 0), (N, K))
    w = (sgn * np.repeat(a.astype(np.float32)[:, None], K, axis=1)).astype(np.float32)
    words, scales = oracle.pack_sign1(w)
    back = oracle.dequantize(words, scales, N, K)
    assert np.array_equal(back, w.astype(np.float64))


def test_gaussian_quantisation_error_law():
    """For Gaussian weights the expected relative squared error of sign+mean|w|
    per group of G is (1 - 1/G)(1 - 2/pi) = 0.360541 at G = 128."""
    w, _ = datagen.C1()
    words, scales = oracle.pack_sign1(w)
    wq = oracle.dequantize(words, scales, 1024, 1024)
    rel = np.sum((w - wq) ** 2) / np.sum(w.astype(np.float64) ** 2)
    law = (1 - 1 / 128) * (1 - 2 / math.pi)
    assert abs(law - 0.360541) < 1e-6
    assert abs(rel / law - 1) < 0.01


def test_bit_accounting():
    g = _gold("sign1_format.json")
    assert oracle.bits_per_weight() == g["bits_per_weight"]
    assert round(16 / oracle.bits_per_weight()) == g["fraction_of_16bit_about"]
    assert oracle.packed_bytes(1024, 1024) == 147456
    assert oracle.packed_bytes(4096, 14336) == 8257536
    assert oracle.packed_bytes(14336, 4096) == 8257536
    assert 3 * oracle.packed_bytes(512, 2048) == 442368
    w = datagen.normal_f32((95, 0), (64, 256), 0.02)
    words, scales = oracle.pack_sign1(w)
    assert words.nbytes + scales.nbytes == oracle.packed_bytes(64, 256)
    assert (words.nbytes + scales.nbytes) * 8 / w.size == 1.125


# ---------------------------------------------------------------------------
# S2/S3 products
# ---------------------------------------------------------------------------

def _packed(key, N, K):
    w = datagen.normal_f32(key, (N, K), 0.02)
    return (w,) + oracle.pack_sign1(w)


def test_gemm_one_hot_picks_signed_scale():
    N, K = 24, 384
    w, words, scales = _packed((94, 0), N, K)
    for k in (0, 1, 63, 64, 127, 128, 200, 383):
        x = np.zeros((1, K))
        x[0, k] = 1.0
        y = oracle.bin_gemm(x, words, scales, N, K)[0]
        expect = np.where(w[:, k] < 0, -1.0, 1.0) * scales[:, k // 128].astype(np.float64)
        assert np.array_equal(y, expect), k


def test_gemm_all_plus_and_all_minus_weights():
    N, K, M = 16, 512, 3
    w = np.abs(datagen.normal_f32((94, 1), (N, K), 0.02)) + np.float32(1e-6)
    x = oracle.bf16_to_f64(datagen.bf16_normal((94, 2), (M, K)))
    words, scales = oracle.pack_sign1(w)
    gsum = x.reshape(M, K // 128, 128).sum(axis=2)              # [M, G]
    expect = gsum @ scales.astype(np.float64).T                  # sum_g s[n,g] sum_k x
    assert np.allclose(oracle.bin_gemm(x, words, scales, N, K), expect, rtol=1e-13, atol=1e-15)
    words_n, scales_n = oracle.pack_sign1(-w)
    assert np.allclose(oracle.bin_gemm(x, words_n, scales_n, N, K), -expect, rtol=1e-13, atol=1e-15)


def test_gemm_matches_definitional_loops_and_columns():
    M, N, K = 2, 5, 256
    w, words, scales = _packed((94, 3), N, K)
    x = oracle.bf16_to_f64(datagen.bf16_normal((94, 4), (M, K)))
    y = oracle.bin_gemm(x, words, scales, N, K)
    yl = oracle.bin_gemm_loops(x, words, scales, N, K)
    assert np.allclose(y, yl, rtol=1e-13, atol=1e-16)
    cols = np.array([4, 0, 2])
    assert np.allclose(oracle.bin_gemm_cols(x, words, scales, N, K, cols), y[:, cols], rtol=1e-14)


def test_gemm_linear_and_row_independent():
    M, N, K = 4, 32, 256
    w, words, scales = _packed((94, 5), N, K)
    x = oracle.bf16_to_f64(datagen.bf16_normal((94, 6), (M, K)))
    y = oracle.bin_gemm(x, words, scales, N, K)
    for m in range(M):
        assert np.allclose(oracle.bin_gemm(x[m:m + 1], words, scales, N, K)[0], y[m], rtol=1e-14)
    y2 = oracle.bin_gemm(2.0 * x[:1] - 0.5 * x[1:2], words, scales, N, K)
    assert np.allclose(y2[0], 2.0 * y[0] - 0.5 * y[1], rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------------------
# binary product + low-rank correction (BWLA commentary, section 4)
# ---------------------------------------------------------------------------

def _f16(a):
    return np.asarray(a, dtype=np.float16)


def test_lowrank_zero_factors_reduce_to_bin_gemm():
    M, N, K, r = 3, 24, 256, 5
    w, words, scales = _packed((95, 0), N, K)
    x = oracle.bf16_to_f64(datagen.bf16_normal((95, 1), (M, K)))
    z = oracle.bin_gemm_lr(x, words, scales, _f16(np.zeros((r, K))), _f16(np.zeros((N, r))), N, K, r)
    assert np.array_equal(z, oracle.bin_gemm(x, words, scales, N, K))


def test_lowrank_one_hot_factors_closed_form():
    # V rows one-hot at k = j_i and U columns u_i: the correction is
    # sum_i x[:, j_i] (outer) u_i -- swapping the roles of U and V, or
    # transposing either, breaks it
    M, N, K = 4, 40, 384
    w, words, scales = _packed((95, 2), N, K)
    x = oracle.bf16_to_f64(datagen.bf16_normal((95, 3), (M, K)))
    js = [5, 200, 383]
    V = np.zeros((len(js), K))
    for i, jj in enumerate(js):
        V[i, jj] = 1.0
    U = np.asarray(datagen.normal_f32((95, 4), (N, len(js)), 0.5), dtype=np.float16).astype(np.float64)
    y = oracle.bin_gemm_lr(x, words, scales, _f16(V), _f16(U), N, K, len(js))
    corr = sum(np.outer(x[:, jj], U[:, i]) for i, jj in enumerate(js))
    assert np.allclose(y - oracle.bin_gemm(x, words, scales, N, K), corr, rtol=1e-12, atol=1e-14)


def test_lowrank_factored_equals_materialised_matrix():
    M, N, K, r = 5, 48, 512, 20
    w, words, scales = _packed((95, 5), N, K)
    x = oracle.bf16_to_f64(datagen.bf16_normal((95, 6), (M, K)))
    v = _f16(datagen.normal_f32((95, 7), (r, K), 0.05))
    u = _f16(datagen.normal_f32((95, 8), (N, r), 0.05))
    y = oracle.bin_gemm_lr(x, words, scales, v, u, N, K, r)
    # materialised from scratch: signs by the bit convention, scales per group
    bits = np.array([[(int(words[n, k // 64]) >> (k % 64)) & 1 for k in range(K)] for n in range(N)])
    Wq = np.where(bits == 1, -1.0, 1.0) * np.repeat(scales.astype(np.float64), 128, axis=1)
    W = Wq + u.astype(np.float64).reshape(N, r) @ v.astype(np.float64).reshape(r, K)
    assert np.allclose(y, x @ W.T, rtol=1e-12, atol=1e-13)
    assert np.allclose(oracle.bin_gemm_lr_dense(x, words, scales, v, u, N, K, r), x @ W.T, rtol=1e-12, atol=1e-13)
    cols = np.array([47, 0, 13])
    assert np.allclose(oracle.bin_gemm_lr_cols(x, words, scales, v, u, N, K, r, cols), y[:, cols], rtol=1e-14)


# ---------------------------------------------------------------------------
# S4 DBF
# ---------------------------------------------------------------------------

def test_dbf_chain_equals_dense_reconstruction():
    m, n, r, M = 96, 128, 64, 3
    v = datagen.pm1_f32((93, 0), (r, n))
    u = datagen.pm1_f32((93, 1), (m, r))
    d_in = datagen.f16_lognormal((93, 2), (n,))
    d_mid = datagen.f16_lognormal((93, 3), (r,))
    d_out = datagen.f16_lognormal((93, 4), (m,))
    x = oracle.bf16_to_f64(datagen.bf16_normal((93, 5), (M, n)))
    vw, uw = oracle.pack_sign1_only(v), oracle.pack_sign1_only(u)
    y = oracle.dbf_chain(x, d_in, vw, d_mid, uw, d_out, m, n, r)
    W = (d_out.astype(np.float64)[:, None] * u.astype(np.float64)) @ np.diag(d_mid.astype(np.float64)) @ \
        (v.astype(np.float64) * d_in.astype(np.float64)[None, :])
    assert np.allclose(y, x @ W.T, rtol=1e-12, atol=1e-12)
    assert np.allclose(oracle.dbf_dense(d_in, vw, d_mid, uw, d_out, m, n, r), W, rtol=1e-13, atol=1e-13)


def _sylvester(n):
    h = np.ones((1, 1))
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def test_dbf_hadamard_identity():
    """V = Hd P and U = P^T Hd with Sylvester Hadamard Hd (Hd Hd^T = n I) and a
    permutation P; with d_mid = 1/n the chain is D_out D_in exactly."""
    n = 256
    Hd = _sylvester(n)
    perm = datagen.rng(93, 9).permutation(n)
    P = np.eye(n)[:, perm]
    V = (Hd @ P).astype(np.float32)
    U = (P.T @ Hd).astype(np.float32)
    d_in = datagen.f16_lognormal((93, 10), (n,))
    d_out = datagen.f16_lognormal((93, 11), (n,))
    d_mid = np.full((n,), 1.0 / n, dtype=np.float16)
    x = oracle.bf16_to_f64(datagen.bf16_normal((93, 12), (2, n)))
    y = oracle.dbf_chain(x, d_in, oracle.pack_sign1_only(V), d_mid, oracle.pack_sign1_only(U), d_out, n, n, n)
    expect = x * d_in.astype(np.float64) * d_out.astype(np.float64)
    assert np.allclose(y, expect, rtol=1e-13, atol=1e-14)


# ---- Q8 activations (DBF post, section 5, item 4) --------------------------

def test_q8_rows_codes_and_exponents():
    """Rounding bound, minimal exponent, ties to even, zero row, exact codes
    of representable rows, over rows spanning many binades."""
    g = datagen.rng(95, 0)
    v = g.standard_normal((6, 300)) * np.exp2(g.integers(-30, 30, size=(6, 1)))
    v[2] = 0.0
    v[3, :5] = [63.5, -64.5, 2.5, -0.5, 127.0]   # ties at e = 0 (max 127)
    v[3, 5:] = 0.0
    q, e = oracle.q8_rows(v)
    for i in range(v.shape[0]):
        m = np.abs(v[i]).max()
        if m == 0:
            assert e[i] == 0 and not q[i].any()
            continue
        s = 2.0 ** e[i]
        assert m <= 127 * s and m > 127 * s / 2          # smallest exponent with |q| <= 127
        assert np.abs(q[i]).max() <= 127 and np.abs(q[i]).max() >= 64
        assert np.all(np.abs(v[i] - q[i] * s) <= s / 2)  # nearest code
        half = np.abs(v[i] / s - np.trunc(v[i] / s)) == 0.5
        assert np.all(q[i][half] % 2 == 0)               # ties to even
    assert list(q[3, :5]) == [64, -64, 2, 0, 127] and e[3] == 0
    # a row of codes times a power of two is reproduced exactly
    codes = g.integers(-127, 128, size=(1, 64))
    codes[0, 0] = 100
    q2, e2 = oracle.q8_rows(codes * 2.0 ** -9)
    assert e2[0] == -9 and np.array_equal(q2, codes)


def test_dbf_chain_q8_hadamard_closed_form():
    """V = U = Sylvester Hadamard H_n, unit diagonals, x = 127 e_k: every
    intermediate is an exact Q8 code, so y = H (127 H e_k) = 127 n e_k."""
    n = 128
    Hd = _sylvester(n).astype(np.float32)
    W = oracle.pack_sign1_only(Hd)
    one = np.ones(n, dtype=np.float16)
    x = np.zeros((3, n))
    for i, k in enumerate((0, 37, 127)):
        x[i, k] = 127.0 * (-1) ** i
    y = oracle.dbf_chain_q8(x, one, W, one, W, one, n, n, n)
    expect = 127.0 * n * x / 127.0
    assert np.array_equal(y, expect)


def test_dbf_chain_q8_symmetries_and_distance():
    """Odd symmetry (x -> -x), power-of-two equivariance (x -> 2^k x scales y by
    2^k exactly: the exponents shift, the codes stay), and the distance to
    the unquantised chain is that of two 8-bit roundings: nonzero, and a few
    percent in L2 with log-normal diagonals (a wrong exponent or a dropped
    scale would be off by a factor)."""
    n, r, m = 256, 128, 192
    v = datagen.pm1_f32((95, 1, 0), (r, n))
    u = datagen.pm1_f32((95, 1, 1), (m, r))
    d_in = datagen.f16_lognormal((95, 1, 2), (n,))
    d_mid = datagen.f16_lognormal((95, 1, 3), (r,))
    d_out = datagen.f16_lognormal((95, 1, 4), (m,))
    vw, uw = oracle.pack_sign1_only(v), oracle.pack_sign1_only(u)
    x = oracle.bf16_to_f64(datagen.bf16_normal((95, 1, 5), (4, n)))
    y = oracle.dbf_chain_q8(x, d_in, vw, d_mid, uw, d_out, m, n, r)
    assert np.array_equal(oracle.dbf_chain_q8(-x, d_in, vw, d_mid, uw, d_out, m, n, r), -y)
    assert np.array_equal(oracle.dbf_chain_q8(x * 2.0 ** 5, d_in, vw, d_mid, uw, d_out, m, n, r), y * 2.0 ** 5)
    ref = oracle.dbf_chain(x, d_in, vw, d_mid, uw, d_out, m, n, r)
    rel = np.linalg.norm(y - ref, axis=1) / np.linalg.norm(ref, axis=1)
    assert np.all(rel < 5e-2) and np.all(rel > 1e-3)


def test_dbf_chain_q8_rounds_h_s_once_to_fp32():
    """h_s = fp32(d_mid * h) before it is quantised, checked on a hand-built
    row whose codes differ under every other precision of that step.

    x = integer codes (max 127, so e1 = 0), d_in = 1, and three rows of V
    give h = 127, 20083 and 49. With d_mid = 1, 1723 * 2^-21 and
    1839 * 2^-14 the exact products are
      h_s[0] = 127                     (the row maximum: e2 = 0)
      h_s[1] = 16.5 + 2^-21            (fp64 -> code 17; fp32 rounds it to the
                                        midpoint 16.5 -> 16, ties to even;
                                        fp16 and bf16 also give 16.5 -> 16)
      h_s[2] = 5.5 - 2^-14             (exact in fp32 -> 5; fp16 and bf16
                                        round it to 5.5 -> 6; fp64 -> 5)
    so only fp32 gives the codes (127, 16, 5). Rows 0..2 of U read them out:
    y = (q0 + q1 + q2, q0 - q1 + q2, q0 + q1 - q2)."""
    n, r, m = 256, 64, 3
    q1 = np.array([127.0] * 248 + [64, 32, 16, 8, 4, 2, 1, 0])

    def v_row(h):
        # h = 127 * (2p - 248) + f with f odd in [-127, 127]: p coarse +1s, then
        # the binary expansion of f over the fine codes 64 .. 1
        k = int(round((h - 1) / 254.0)) * 2
        f = h - 127 * k
        assert f % 2 == 1 and -127 <= f <= 127
        p = (k + 248) // 2
        u = (f + 127) // 2
        row = np.array([1.0] * p + [-1.0] * (248 - p)
                       + [1.0 if (u >> i) & 1 else -1.0 for i in (6, 5, 4, 3, 2, 1, 0)] + [1.0])
        assert row @ q1 == h
        return row

    V = np.ones((r, n), dtype=np.float32)
    for j, h in enumerate((127, 20083, 49)):
        V[j] = v_row(h)
    d_mid = np.zeros(r, dtype=np.float16)
    d_mid[:3] = [1.0, 1723 * 2.0 ** -21, 1839 * 2.0 ** -14]
    assert d_mid[1] == 1723 * 2.0 ** -21 and d_mid[2] == 1839 * 2.0 ** -14   # exact fp16 values
    exact = np.array([127.0, 1723 * 20083 * 2.0 ** -21, 1839 * 49 * 2.0 ** -14])
    assert exact[1] == 16.5 + 2.0 ** -21 and exact[2] == 5.5 - 2.0 ** -14
    U = np.ones((m, r), dtype=np.float32)
    U[1, 1] = -1.0
    U[2, 2] = -1.0
    ones_n, ones_m = np.ones(n, np.float16), np.ones(m, np.float16)
    y = oracle.dbf_chain_q8(q1[None, :], ones_n, oracle.pack_sign1_only(V), d_mid,
                            oracle.pack_sign1_only(U), ones_m, m, n, r)
    assert np.array_equal(y[0], [127 + 16 + 5, 127 - 16 + 5, 127 + 16 - 5])
    # the codes the other precisions would give, for the record
    assert list(oracle.q8_rows(exact)[0]) == [127, 17, 5]                                    # fp64
    assert list(oracle.q8_rows(exact.astype(np.float16).astype(np.float64))[0]) == [127, 16, 6]  # fp16
    assert list(oracle.q8_rows(oracle.round_bf16(exact))[0]) == [127, 16, 6]                  # bf16


def test_dbf_bit_budget_worked_example():
    g = _gold("dbf_bit_budget.json")
    m, n, r = g["shape_m"], g["shape_n"], g["r"]
    assert r * (m + n) == g["binary_factor_bits"]
    assert 16 * (m + n + r) == g["fp16_diagonal_bits"]
    assert oracle.dbf_bits(m, n, r) == g["total_bits"]
    assert oracle.dbf_bpe(m, n, r) == g["bits_per_element"]
    q2k = int(g["q2k_bits_per_element"] * m * n)
    assert q2k == g["q2k_bits"]
    assert (q2k - oracle.dbf_bits(m, n, r)) // 8 == g["dbf_smaller_by_bytes"]
    tot = g["routed_matrices"]
    assert round(tot * oracle.dbf_bits(m, n, r) / 8 / 2 ** 30, 4) == g["dbf_payload_gib"]
    assert round(tot * q2k / 8 / 2 ** 30, 4) == g["q2k_payload_gib"]
    assert round(tot * (q2k - oracle.dbf_bits(m, n, r)) / 8 / 2 ** 20) == g["margin_mib"]
    # the shape benchmarked here
    assert oracle.dbf_bpe(4096, 4096, 2048) == 1.009765625


# ---------------------------------------------------------------------------
# S5/S6 MoE
# ---------------------------------------------------------------------------

def test_route_topk_brute_force_and_ties():
    T, E, k = 16, 256, 8
    lg = datagen.router_logits((92, 0), T, E)
    lg[3] = np.round(lg[3], 1)           # many exact ties
    lg[4, :] = 0.5                        # all tied: experts 0..7
    lg[5, 10] = lg[5, 200] = np.float32(9.0)
    ids, w = oracle.route_topk(lg, k)
    for t in range(T):
        exp_ids = sorted(range(E), key=lambda e: (-float(lg[t, e]), e))[:k]
        assert list(ids[t]) == exp_ids
    assert list(ids[4]) == list(range(8))
    assert list(ids[5][:2]) == [10, 200]
    assert np.allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-15)
    # equals the full softmax renormalised over the selected experts
    full = np.exp(lg.astype(np.float64) - lg.max(axis=1, keepdims=True))
    full /= full.sum(axis=1, keepdims=True)
    sel = np.take_along_axis(full, ids, axis=1)
    assert np.allclose(w, sel / sel.sum(axis=1, keepdims=True), rtol=1e-13)
    assert np.all(np.diff(w, axis=1) <= 0)


def _tiny_moe(E=4, H=256, I=128, seed=91):
    c = datagen.C4(E=E, H=H, I=I, top_k=2, layer=seed)
    packs = {}
    for e in range(E):
        gw, gs = oracle.pack_sign1(c.gate(e))
        uw, us = oracle.pack_sign1(c.up(e))
        dw, ds = oracle.pack_sign1(c.down(e))
        packs[e] = (gw, gs, uw, us, dw, ds)
    return c, packs


def _dense_ffn(p, x, H, I):
    gw, gs, uw, us, dw, ds = p
    Wg = oracle.dequantize(gw, gs, I, H)
    Wu = oracle.dequantize(uw, us, I, H)
    Wd = oracle.dequantize(dw, ds, H, I)
    g = x @ Wg.T
    return (g / (1 + np.exp(-g)) * (x @ Wu.T)) @ Wd.T


def test_silu_values_fixed_by_the_mathematics():
    """silu(z) = z * sigmoid(z), pinned by values that follow from the
    definition of the logistic function rather than by its formula:
    silu(0) = 0; silu(z) - silu(-z) = z (sigmoid(z) + sigmoid(-z) = 1);
    sigmoid(ln 3) = 3/4, so silu(ln 3) = (3/4) ln 3 and silu(-ln 3) = -(1/4) ln 3;
    slope 1/2 at 0; silu(z) -> z for large z and -> 0 from below for large -z."""
    assert oracle.silu(0.0) == 0.0
    z = np.linspace(-30.0, 30.0, 1201)
    assert np.allclose(oracle.silu(z) - oracle.silu(-z), z, rtol=1e-14, atol=1e-14)
    l3 = math.log(3.0)
    assert math.isclose(float(oracle.silu(l3)), 0.75 * l3, rel_tol=1e-15)
    assert math.isclose(float(oracle.silu(-l3)), -0.25 * l3, rel_tol=1e-15)
    assert math.isclose(float(oracle.silu(1e-9)) / 1e-9, 0.5, rel_tol=1e-9)
    assert float(oracle.silu(40.0)) == 40.0
    s = float(oracle.silu(-40.0))
    assert s < 0.0 and math.isclose(s, -40.0 * math.exp(-40.0), rel_tol=1e-12)
    # sigmoid(ln(p / (1 - p))) = p for any p in (0, 1)
    p = np.array([0.1, 0.2, 0.5, 0.9, 0.99])
    t = np.log(p / (1.0 - p))
    assert np.allclose(oracle.silu(t), t * p, rtol=1e-14, atol=1e-15)


def test_moe_identical_experts_and_single_route():
    E, H, I = 4, 256, 128
    c, packs = _tiny_moe(E, H, I)
    x = oracle.bf16_to_f64(c.x(3))
    lg = c.logits(3)
    same = {e: packs[0] for e in range(E)}
    y, ids, w = oracle.moe_ffn(x, lg, lambda e: same[e], H, I, 3)
    assert np.allclose(y, _dense_ffn(packs[0], x, H, I), rtol=1e-12, atol=1e-14)
    y1, ids1, w1 = oracle.moe_ffn(x, lg, lambda e: packs[e], H, I, 1)
    assert np.all(w1 == 1.0)
    for t in range(3):
        assert np.allclose(y1[t], _dense_ffn(packs[int(ids1[t, 0])], x[t:t + 1], H, I)[0], rtol=1e-12, atol=1e-14)


def test_moe_matches_definitional_loops():
    E, H, I = 4, 256, 128
    c, packs = _tiny_moe(E, H, I, seed=90)
    x = oracle.bf16_to_f64(c.x(2))
    lg = c.logits(2)
    y, ids, w = oracle.moe_ffn(x, lg, lambda e: packs[e], H, I, 2)
    yl, idl, wl = oracle.moe_ffn_loops(x, lg, lambda e: packs[e], H, I, 2)
    assert np.array_equal(ids, idl)
    assert np.allclose(y, yl, rtol=1e-12, atol=1e-15)


# ---------------------------------------------------------------------------
# S7 Kronecker rotation
# ---------------------------------------------------------------------------

# ---------------------------------------------------------------------------
# MoE with DBF experts (the DBF post's deployed layer)
# ---------------------------------------------------------------------------

def _dbf_experts(cfg):
    def rec(e, p):
        d = cfg.proj(e, p)
        return (d["d_in"], oracle.pack_sign1_only(d["v"]), d["d_mid"], oracle.pack_sign1_only(d["u"]), d["d_out"])

    return lambda e: (rec(e, 0), rec(e, 1), rec(e, 2))


def test_moe_dbf_equals_dense_reconstruction_and_sampling():
    cfg = datagen.C4D(E=6, H=256, I=128, r=128, top_k=2)
    x = oracle.bf16_to_f64(cfg.x(3))
    lg = cfg.logits(3)
    ex = _dbf_experts(cfg)
    y, ids, w = oracle.moe_dbf_ffn(x, lg, ex, cfg.H, cfg.I, cfg.r, cfg.top_k)
    yd, ids2, w2 = oracle.moe_dbf_dense(x, lg, ex, cfg.H, cfg.I, cfg.r, cfg.top_k)
    assert np.array_equal(ids, ids2)
    assert np.allclose(y, yd, rtol=1e-11, atol=1e-13 * np.abs(yd).max())
    ys, _, _ = oracle.moe_dbf_ffn(x, lg, ex, cfg.H, cfg.I, cfg.r, cfg.top_k, tokens=[2, 0])
    assert np.array_equal(ys[[0, 2]], y[[0, 2]]) and not ys[1].any()


def test_moe_dbf_identical_experts_and_single_route_from_raw_matrices():
    cfg = datagen.C4D(E=5, H=256, I=128, r=128, top_k=3)
    x = oracle.bf16_to_f64(cfg.x(4))
    lg = cfg.logits(4)
    one = _dbf_experts(cfg)(0)
    y, _, _ = oracle.moe_dbf_ffn(x, lg, lambda e: one, cfg.H, cfg.I, cfg.r, cfg.top_k)
    # expert 0 built from the raw +-1 arrays and fp16 diagonals (no unpacking)
    raw = [cfg.proj(0, p) for p in range(3)]

    def chain(d, v):
        h = d["v"].astype(np.float64) @ (d["d_in"].astype(np.float64) * v)
        return d["d_out"].astype(np.float64) * (d["u"].astype(np.float64) @ (d["d_mid"].astype(np.float64) * h))

    for t in range(4):
        g, u = chain(raw[0], x[t]), chain(raw[1], x[t])
        expect = chain(raw[2], g / (1.0 + np.exp(-g)) * u)
        assert np.allclose(y[t], expect, rtol=1e-11, atol=1e-13 * np.abs(expect).max())


def test_kron_rotate_is_kronecker_product():
    n1, n2, M = 8, 16, 5
    H = datagen.haar_orthogonal((89, 0), n1)
    R = datagen.haar_orthogonal((89, 1), n2)
    x = datagen.normal_f32((89, 2), (M, n1 * n2)).astype(np.float64)
    y = oracle.kron_rotate(x, H, R)
    assert np.allclose(y, x @ np.kron(H, R).T, rtol=1e-13, atol=1e-13)


def test_kron_rotate_invariants():
    d = datagen.C5(M=4)
    H, R = d["H"].astype(np.float64), d["R"].astype(np.float64)
    x = oracle.bf16_to_f64(d["x"][:4])
    y = oracle.kron_rotate(x, H, R)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-6)
    back = oracle.kron_rotate(y, H.T, R.T)
    assert np.allclose(back, x, rtol=1e-5, atol=1e-5)
    assert np.array_equal(oracle.kron_rotate(x, np.eye(64), np.eye(64)), x)
    # forward equivalence: W x = (W Q^T)(Q x)
    W = datagen.normal_f32((89, 3), (32, 4096), 0.02).astype(np.float64)
    Q = np.kron(H, R)
    # H and R are fp32 roundings of orthogonal matrices: orthogonal to ~1e-7
    assert np.allclose((W @ Q.T) @ y.T, W @ x.T, rtol=1e-5, atol=1e-5)
