"""GPU parity: every C-ABI call against the fp64 oracle on the same seeded
inputs, element by element.

Bars (see the header of include/brq.h for the numerics):
* sign planes bit-exact; fp16 scales within 1 ulp (counted; expected 0 off);
* products with fp32 output: max_i|g_i - o_i| / max_i|o_i| <= F32_TOL, small
  enough that one flipped sign or one dropped group fails;
* products with bf16 output: every element within 1 bf16 ulp of the oracle
  rounded to bf16 (or within 1e-5 of the largest output, for outputs so near
  zero that fp32 accumulation error spans several of their ulps), and l2 relative error <= 2e-3 (bf16 rounding alone reaches
  2^-8 relative per element, so the 2e-3 bar is applied normwise there);
* top-k expert ids bit-exact, route weights within 1e-6 relative.

Product parity feeds the oracle's packed bytes to the device, so a scale that
legitimately differs by one ulp cannot hide a product error; the end-to-end
cases use device-packed weights instead.
"""
import sys

import numpy as np
import pytest
import torch

import datagen
import oracle
from gpu_util import bf16_close, bf16_ulps, check_bf16, check_f32, dev, f16_ulps, f64, host_bits, l2rel, maxrel

pytestmark = pytest.mark.gpu

F32_TOL = 2e-5


def single_row_bound(xb, words, scales, N, K):
    """Error bound of the single-row path (M = 1, K % 512 == 0): it carries each
    activation as a 24-bit fixed-point field under the largest power of two of
    its slice of the row, so a value loses less than 2^-23 of that slice's
    maximum (taken here as the row maximum, which is larger), and the
    products and partial sums on the matrix cores are exact; the fp32 sums of
    the group results add at most a few dozen roundings of 2^-24 each."""
    x = oracle.bf16_to_f64(xb).reshape(-1)
    W = np.abs(oracle.dequantize(words, scales, N, K))
    rep = 2.0 ** -23 * np.abs(x).max() * W.sum(axis=1)
    acc = 64 * 2.0 ** -24 * (W @ np.abs(x))
    return rep + acc


def brq():
    import binary_weight_gemm_amd as b
    return b


def say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# S1 pack
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("rows,cols,key", [(1, 128, 1), (17, 384, 2), (1024, 1024, 3), (64, 2048, 4)])
def test_pack_small(rows, cols, key):
    say("pack", rows, cols)
    w = datagen.normal_f32((70, key), (rows, cols), 0.02)
    w[0, :5] = [0.0, -0.0, 1e-30, -1e-30, 0.5]
    ow, osc = oracle.pack_sign1(w)
    s, sc = brq().pack(dev(w))
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(s), ow)
    ul = f16_ulps(host_bits(sc), osc)
    assert ul.max() <= 1 and int((ul > 0).sum()) <= max(1, ul.size // 10000)


def test_pack_sign1_only_and_c2_full():
    say("pack sign1-only 2048x4096, pack C2 4096x14336")
    v = datagen.pm1_f32((3, 0, 2048), (2048, 4096))
    s, sc = brq().pack(dev(v), scales=False)
    assert sc is None
    assert np.array_equal(host_bits(s), oracle.pack_sign1_only(v))
    w = datagen.C2_weight(0)
    ow, osc = oracle.pack_sign1(w)
    s, sc = brq().pack(dev(w))
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(s), ow)
    ul = f16_ulps(host_bits(sc), osc)
    assert ul.max() <= 1
    assert int((ul > 0).sum()) <= 8, int((ul > 0).sum())


def test_pack_round_trip_exact_groups():
    say("pack round trip")
    N, K = 8, 512
    a = np.array([0.5, 0.015625, 3.0, 1e-3, 65504.0, 6.1035156e-05, 0.0123, 7.0], dtype=np.float16)
    w = (datagen.pm1_f32((96, 0), (N, K)) * np.repeat(a.astype(np.float32)[:, None], K, axis=1)).astype(np.float32)
    s, sc = brq().pack(dev(w))
    ow, osc = oracle.pack_sign1(w)
    assert np.array_equal(host_bits(s), ow)
    assert np.array_equal(host_bits(sc), osc.view(np.uint16))


# ---------------------------------------------------------------------------
# S2 / S3 products
# ---------------------------------------------------------------------------

def _gemm_case(M, N, K, key, out=torch.float32):
    w = datagen.normal_f32((71, key, 0), (N, K), 0.02)
    x = datagen.bf16_normal((71, key, 1), (M, K))
    ow, osc = oracle.pack_sign1(w)
    o = oracle.bin_gemm(oracle.bf16_to_f64(x), ow, osc, N, K)
    y = brq().gemm(dev(x), dev(ow), dev(osc), N, K, out_dtype=out)
    torch.cuda.synchronize()
    return y, o


@pytest.mark.parametrize("M,N,K", [(1, 16, 128), (1, 40, 640), (3, 48, 1024), (16, 33, 256), (17, 64, 512),
                                   (64, 32, 2048), (5, 16, 14336), (1, 1024, 1024), (9, 16, 128),
                                   (33, 130, 4480), (40, 2000, 3200), (20, 32768, 512), (64, 4100, 1280),
                                   (1, 48, 23552)])
def test_gemm_decode_f32(M, N, K):
    say("gemm decode f32", M, N, K)
    y, o = _gemm_case(M, N, K, M * 1000 + N)
    check_f32(f64(y), o, F32_TOL, f"gemm {M}x{N}x{K}")


# 9..64 rows over 64-column tiles: each wave of a workgroup takes every
# fourth k-step; these shapes give the waves 3, 4, 5 and 6 k-steps (ragged N,
# partial last row tile) where the cases above give 1, 2, 7 and 8
@pytest.mark.parametrize("M,N,K", [(64, 16384, 1536), (48, 16384, 2048), (30, 16400, 2560), (12, 16384, 3072)])
def test_gemm_mid_wave_steps(M, N, K):
    say("gemm mid wave steps", M, N, K)
    y, o = _gemm_case(M, N, K, M * 7 + N)
    check_f32(f64(y), o, F32_TOL, f"gemm {M}x{N}x{K}")
    yb, _ = _gemm_case(M, N, K, M * 7 + N, out=torch.bfloat16)
    check_bf16(yb, o, f"gemm {M}x{N}x{K} bf16")


@pytest.mark.parametrize("N,K", [(40, 512), (1000, 1536), (2049, 4096), (48, 23040), (40, 8704), (300, 9728),
                                 (64, 17920)])
def test_gemm_single_row_wide_range(N, K):
    """A single activation row with K % 512 == 0 runs on the fp8 x fp4 matrix
    cores with the activations as fixed-point digit rows: ragged column tiles,
    a row spanning 36 binades, an all-zero row and tiny values with one
    outlier. Those matrix cores truncate whatever lies more than 13 bits below
    the largest of 8 products; the digit rows keep every product an integer
    times one power of two, so nothing is truncated and each output is held to
    the fp32 bar and, element by element, to the bound single_row_bound
    derives from the representation. K = 23040 is the longest row the digit
    rows fit the LDS for (45 chunks, three per wave); 23552 takes the fp16
    one-launch path (test_gemm_decode_f32). K = 8704, 9728 and 17920 (17, 19
    and 35 chunks of 512) leave the last wave fewer chunks than the others,
    whose empty slots must add nothing."""
    say("gemm single row, wide range", N, K)
    w = datagen.normal_f32((73, N, K), (N, K), 0.02)
    ow, osc = oracle.pack_sign1(w)
    S, SC = dev(ow), dev(osc)
    g = datagen.rng(73, N, K, 1)
    base = g.standard_normal((4, K)).astype(np.float32)
    rows = [base[0],
            base[1] * np.exp2(g.integers(-24, 12, size=K)).astype(np.float32),
            np.zeros(K, np.float32),
            base[3] * np.float32(2.0 ** -20)]
    rows[3][K // 3] = 3000.0
    for i, r in enumerate(rows):
        xb = datagen.bf16_bits_from_f32(r.reshape(1, K))
        o = oracle.bin_gemm(oracle.bf16_to_f64(xb), ow, osc, N, K)
        y = brq().gemm(dev(xb), S, SC, N, K, out_dtype=torch.float32)
        if i == 2:
            assert not torch.any(y != 0)
        else:
            check_f32(f64(y), o, F32_TOL, f"single row {i} {N}x{K}")
            err = np.abs(f64(y)[0] - o[0])
            bound = single_row_bound(xb, ow, osc, N, K)
            assert np.all(err <= bound), f"row {i}: error above the derived bound at {int(np.argmax(err - bound))}"
        yb = brq().gemm(dev(xb), S, SC, N, K, out_dtype=torch.bfloat16)
        assert np.array_equal(host_bits(yb), oracle.bf16_bits(oracle.round_bf16(f64(y))))


@pytest.mark.parametrize("M,N,K", [(2, 40, 512), (5, 1000, 1536), (8, 2049, 4096), (4, 4096, 14336)])
def test_gemm_few_rows_wide_range(M, N, K):
    """2 to 8 activation rows of very different magnitude (1e4, 36 binades
    inside a row, all zero, 2^-20 with one outlier) in one product on the fp16
    matrix cores: the rows must not disturb each other, and values below
    fp16's normal range lose at most 2^-25 each (the activation-range
    precondition), far below the fp32 bar of each row."""
    say("gemm few rows, wide range", M, N, K)
    w = datagen.normal_f32((75, N, K), (N, K), 0.02)
    ow, osc = oracle.pack_sign1(w)
    g = datagen.rng(75, N, K, 1)
    base = g.standard_normal((M, K)).astype(np.float32)
    kinds = [lambda r: r * np.float32(1e4),
             lambda r: r * np.exp2(g.integers(-24, 12, size=K)).astype(np.float32),
             lambda r: np.zeros(K, np.float32),
             lambda r: r * np.float32(2.0 ** -20)]
    rows = np.stack([kinds[m % 4](base[m]) if m < 4 else base[m] for m in range(M)])
    if M > 3:
        rows[3, K // 3] = 3000.0
    xb = datagen.bf16_bits_from_f32(rows)
    o = oracle.bin_gemm(oracle.bf16_to_f64(xb), ow, osc, N, K)
    y = f64(brq().gemm(dev(xb), dev(ow), dev(osc), N, K, out_dtype=torch.float32))
    for m in range(M):
        if m == 2:
            assert not np.any(y[m] != 0)
        else:
            check_f32(y[m], o[m], F32_TOL, f"row {m} of {M}x{N}x{K}")


# activation rows far outside fp16's range (|x| ~ 1e5, 1e30, 1e-30) next to
# ordinary and all-zero rows: the paths that stage bf16 rows as fp16 (decode
# rows M <= 8, prefill M > 64) scale each row (or wave slice of a row) by a
# power of two first, so every row matches the oracle and the single-row path
# to the fp32 bar, whatever its magnitude
_RANGE_SCALES = (1e5, 1e30, 0.0, 1e-30, 1.0, 3e4, 2.0 ** -20, 1e-3)


# the routed layer's SwiGLU squares the magnitude: scales whose fp32
# intermediates stay finite and normal
_RANGE_SCALES_MOE = (1e5, 3e8, 0.0, 1e-10, 1.0, 3e4, 2.0 ** -20, 1e-3)


def _range_rows(M, K, key, scales=_RANGE_SCALES):
    g = datagen.rng(79, M, K, key)
    base = g.standard_normal((M, K)).astype(np.float32)
    rows = np.stack([base[m] * np.float32(scales[m % len(scales)]) for m in range(M)])
    return datagen.bf16_bits_from_f32(rows)


@pytest.mark.parametrize("M,N,K", [(2, 96, 1024), (8, 130, 2048), (16, 96, 1024), (64, 130, 2048),
                                   (300, 520, 1024), (100, 130, 33280)])
def test_gemm_activation_range(M, N, K):
    say("gemm activation range", M, N, K)
    w = datagen.normal_f32((79, N, K), (N, K), 0.02)
    ow, osc = oracle.pack_sign1(w)
    xb = _range_rows(M, K, 0)
    o = oracle.bin_gemm(oracle.bf16_to_f64(xb), ow, osc, N, K)
    S, SC = dev(ow), dev(osc)
    y = f64(brq().gemm(dev(xb), S, SC, N, K, out_dtype=torch.float32))
    assert np.all(np.isfinite(y))
    for m in range(M):
        if not np.any(o[m]):
            assert not np.any(y[m])
            continue
        check_f32(y[m], o[m], F32_TOL, f"row {m} (scale {_RANGE_SCALES[m % len(_RANGE_SCALES)]:g}) of {M}x{N}x{K}")
    # each row alone (the single-row path) agrees with its row of the batch
    for m in range(min(M, len(_RANGE_SCALES))):
        if not np.any(o[m]):
            continue
        y1 = f64(brq().gemm(dev(xb[m:m + 1]), S, SC, N, K, out_dtype=torch.float32))[0]
        assert maxrel(y1, y[m]) <= F32_TOL, f"row {m}: single-row and batch differ"


def test_dbf_and_moe_activation_range():
    say("dbf decode and tiled + moe small/grouped, activation range")
    m_, n_, r_ = 128, 512, 256
    v = datagen.pm1_f32((79, 1, 0), (r_, n_))
    u = datagen.pm1_f32((79, 1, 1), (m_, r_))
    d_in, d_mid, d_out = (datagen.f16_lognormal((79, 1, 2 + i), (s_,)) for i, s_ in enumerate((n_, r_, m_)))
    vw, uw = oracle.pack_sign1_only(v), oracle.pack_sign1_only(u)
    for M in (4, 16, 300):  # decode path, tiled path (x staged per row)
        xb = _range_rows(M, n_, M)
        o = oracle.dbf_chain(oracle.bf16_to_f64(xb), d_in, vw, d_mid, uw, d_out, m_, n_, r_)
        y = f64(brq().dbf_gemm(dev(xb), dev(d_in), dev(vw), dev(d_mid), dev(uw), dev(d_out), m_, n_, r_,
                               out_dtype=torch.float32))
        for t in range(M):
            if np.any(o[t]):
                check_f32(y[t], o[t], F32_TOL, f"dbf M={M} row {t}")
            else:
                assert not np.any(y[t])
    cfg = datagen.C4(E=16, H=256, I=128, top_k=4, layer=79)
    ex = _Experts(cfg)
    for T in (3, 9):  # few-token path, grouped path
        xt = _range_rows(T, cfg.H, 2 + T, _RANGE_SCALES_MOE)
        lg = cfg.logits(T)
        om, oids, _ = oracle.moe_ffn(oracle.bf16_to_f64(xt), lg, ex, cfg.H, cfg.I, cfg.top_k)
        ym, ids, _ = brq().moe_ffn(dev(xt), dev(lg), *ex.d, cfg.E, cfg.H, cfg.I, cfg.top_k, out_dtype=torch.float32,
                                   return_routing=True)
        ym = f64(ym)
        assert np.array_equal(ids.cpu().numpy().astype(np.int64), oids)
        for t in range(T):
            if np.any(om[t]):
                check_f32(ym[t], om[t], F32_TOL, f"moe T={T} token {t}")
            else:
                assert not np.any(ym[t])


def _exp25_rows(M, K, key):
    """Rows whose every value lies in [2^-102, 1.9 * 2^-102] with a random
    sign: every wave slice's largest |x| has biased exponent 25, where the
    digit operands' zero row would read the E8M0 NaN code if it took the
    digit rows' exponent formula."""
    g = datagen.rng(83, M, K, key)
    mag = (1.0 + 0.9 * g.random((M, K))) * 2.0 ** -102
    sgn = np.where(g.random((M, K)) < 0.5, -1.0, 1.0)
    return datagen.bf16_bits_from_f32((sgn * mag).astype(np.float32))


@pytest.mark.parametrize("N,K", [(96, 512), (520, 4096)])
def test_digit_paths_slice_exponent_25(N, K):
    """The fp8 x fp4 digit paths on activations whose slice maxima sit at
    biased exponent 25: the single-row product matches the oracle to the fp32
    bar; a routed token at that scale gives finite outputs (its SwiGLU product
    underflows fp32, so it is checked for finiteness and size) and leaves the
    other tokens' results at the bar, on the plain and the DBF-expert layers."""
    say("digit paths at slice exponent 25", N, K)
    w = datagen.normal_f32((83, N, K), (N, K), 0.02)
    ow, osc = oracle.pack_sign1(w)
    xb = _exp25_rows(1, K, 0)
    o = oracle.bin_gemm(oracle.bf16_to_f64(xb), ow, osc, N, K)
    y = f64(brq().gemm(dev(xb), dev(ow), dev(osc), N, K, out_dtype=torch.float32))
    assert np.all(np.isfinite(y))
    check_f32(y, o, F32_TOL, f"single row at 2^-102, {N}x{K}")
    if K != 512:
        return

    def mixed(cfg, T):
        x = cfg.x(T).copy()
        x[1] = _exp25_rows(1, cfg.H, T)[0]
        return x

    def check(y, o, T, what):
        assert np.all(np.isfinite(y)), f"{what} T={T}: non-finite output"
        assert np.abs(y[1]).max() <= 2.0 ** -120, f"{what} T={T}: tiny token's output too large"
        keep = [t for t in range(T) if t != 1]
        check_f32(y[keep], o[keep], F32_TOL, f"{what} T={T}, other tokens")

    cfg = datagen.C4(E=16, H=512, I=128, top_k=4, layer=83)
    ex = _Experts(cfg)
    for T in (3, 9):  # few-token path, grouped path
        x, lg = mixed(cfg, T), cfg.logits(T)
        om, oids, _ = oracle.moe_ffn(oracle.bf16_to_f64(x), lg, ex, cfg.H, cfg.I, cfg.top_k)
        ym, ids, _ = brq().moe_ffn(dev(x), dev(lg), *ex.d, cfg.E, cfg.H, cfg.I, cfg.top_k, out_dtype=torch.float32,
                                   return_routing=True)
        assert np.array_equal(ids.cpu().numpy().astype(np.int64), oids)
        check(f64(ym), om, T, "moe")
    cfg = datagen.C4D(E=16, H=512, I=128, r=256, top_k=4, layer=83)
    for T in (2, 24):
        x, lg = mixed(cfg, T), cfg.logits(T)
        ids_o, _ = oracle.route_topk(lg, cfg.top_k)
        recs = _dbf_moe_dev(cfg, sorted(set(int(e) for e in ids_o.ravel())))
        o, _, _ = oracle.moe_dbf_ffn(oracle.bf16_to_f64(x), lg, _dbf_moe_oracle_experts(cfg), cfg.H, cfg.I, cfg.r,
                                     cfg.top_k)
        y = brq().moe_dbf_ffn(dev(x), dev(lg), *recs, cfg.E, cfg.H, cfg.I, cfg.r, cfg.top_k, out_dtype=torch.float32)
        check(f64(y), o, T, "moe dbf")


@pytest.mark.parametrize("M,N,K", [(1, 40, 640), (64, 96, 1024)])
def test_gemm_decode_bf16(M, N, K):
    say("gemm decode bf16", M, N, K)
    y, o = _gemm_case(M, N, K, M * 1000 + N + 7, out=torch.bfloat16)
    check_bf16(y, o, f"gemm {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(65, 64, 256), (128, 128, 512), (300, 200, 384), (512, 1024, 1024)])
def test_gemm_tiled_f32(M, N, K):
    say("gemm tiled f32", M, N, K)
    y, o = _gemm_case(M, N, K, M * 1000 + N + 3)
    check_f32(f64(y), o, F32_TOL, f"gemm {M}x{N}x{K}")


# More 256-wide tiles than compute units with a last round at most half full:
# the last round's columns go to 128-wide tiles (a second launch). 256 x 65892:
# 256 tiles of 256 columns, then 3 of 128 (the last ragged); 300 x 33280: two
# row blocks (the second ragged), 128 + 4 column tiles.
@pytest.mark.parametrize("M,N,K", [(256, 65892, 128), (300, 33280, 256)])
def test_gemm_tiled_split_tail(M, N, K):
    say("gemm tiled split tail", M, N, K)
    y, o = _gemm_case(M, N, K, M * 7 + 1)
    check_f32(f64(y), o, F32_TOL, f"gemm {M}x{N}x{K}")


# ---------------------------------------------------------------------------
# binary product + rank-r correction: decode rows (correction added to the fp32
# product) and many rows (fused k-step in the prefill epilogue, incl. the
# split-tail launch)
# ---------------------------------------------------------------------------

def _lr_case(M, N, K, r, key, out=torch.float32):
    w = datagen.normal_f32((77, key, 0), (N, K), 0.02)
    x = datagen.bf16_normal((77, key, 1), (M, K))
    v = np.asarray(datagen.normal_f32((77, key, 2), (r, K), 0.05), dtype=np.float16)
    u = np.asarray(datagen.normal_f32((77, key, 3), (N, r), 0.05), dtype=np.float16)
    ow, osc = oracle.pack_sign1(w)
    o = oracle.bin_gemm_lr(oracle.bf16_to_f64(x), ow, osc, v, u, N, K, r)
    y = brq().gemm_lr(dev(x), dev(ow), dev(osc), dev(v), dev(u), N, K, r, out_dtype=out)
    torch.cuda.synchronize()
    return y, o


@pytest.mark.parametrize("M,N,K,r", [(1, 40, 640, 1), (1, 1000, 1536, 20), (4, 130, 1024, 20), (17, 200, 2048, 33),
                                     (64, 96, 1024, 64), (65, 64, 256, 20), (300, 200, 384, 7),
                                     (512, 1024, 1024, 64), (256, 65892, 128, 20)])
def test_gemm_lr(M, N, K, r):
    say("gemm lr", M, N, K, r)
    y, o = _lr_case(M, N, K, r, M * 31 + r)
    # M = 1 with K % 512 == 0 takes the single-row fp8 x fp4 product
    tol = F32_TOL
    check_f32(f64(y), o, tol, f"gemm lr {M}x{N}x{K} r={r}")


@pytest.mark.parametrize("M", [4, 16, 300])
def test_gemm_lr_activation_range(M):
    """The low-rank path's rows are staged with a power of two per row too:
    x V^T is formed from the same scaled rows (fp16 operands) and scaled back
    with the product, so rows at 1e5 or 1e30 (or 1e-30) match the oracle."""
    say("gemm lr activation range", M)
    N, K, r = 130, 1024, 20
    w = datagen.normal_f32((81, M, 0), (N, K), 0.02)
    v = np.asarray(datagen.normal_f32((81, M, 2), (r, K), 0.05), dtype=np.float16)
    u = np.asarray(datagen.normal_f32((81, M, 3), (N, r), 0.05), dtype=np.float16)
    ow, osc = oracle.pack_sign1(w)
    xb = _range_rows(M, K, 5)
    o = oracle.bin_gemm_lr(oracle.bf16_to_f64(xb), ow, osc, v, u, N, K, r)
    y = f64(brq().gemm_lr(dev(xb), dev(ow), dev(osc), dev(v), dev(u), N, K, r, out_dtype=torch.float32))
    assert np.all(np.isfinite(y))
    for m in range(M):
        if np.any(o[m]):
            check_f32(y[m], o[m], F32_TOL, f"lr M={M} row {m}")
        else:
            assert not np.any(y[m])


@pytest.mark.parametrize("M", [8, 300])
def test_gemm_lr_bf16(M):
    say("gemm lr bf16", M)
    y, o = _lr_case(M, 384, 1024, 20, 900 + M, out=torch.bfloat16)
    check_bf16(y, o, f"gemm lr bf16 M={M}")


def test_gemm_lr_c5_sampled_columns():
    say("gemm lr at the C5 shape, rank 20, sampled columns")
    d = datagen.C5()
    N, K, r = d["N"], d["K"], 20
    w = datagen.C5_weight(N, K)
    ow, osc = oracle.pack_sign1(w)
    v = np.asarray(datagen.normal_f32((78, 0), (r, K), 0.02), dtype=np.float16)
    u = np.asarray(datagen.normal_f32((78, 1), (N, r), 0.02), dtype=np.float16)
    x = datagen.bf16_normal((78, 2), (4096, K))
    y = brq().gemm_lr(dev(x), dev(ow), dev(osc), dev(v), dev(u), N, K, r, out_dtype=torch.float32)
    torch.cuda.synchronize()
    cols = np.sort(datagen.rng(79, 0).choice(N, size=64, replace=False))
    o = oracle.bin_gemm_lr_cols(oracle.bf16_to_f64(x), ow, osc, v, u, N, K, r, cols)
    check_f32(f64(y)[:, cols], o, F32_TOL, "C5 gemm lr")


def test_gemm_tiled_bf16():
    say("gemm tiled bf16 257x320x768")
    y, o = _gemm_case(257, 320, 768, 99, out=torch.bfloat16)
    check_bf16(y, o, "gemm tiled bf16")


def test_gemm_c1():
    say("C1 gemv")
    w, x = datagen.C1()
    ow, osc = oracle.pack_sign1(w)
    o = oracle.bin_gemm(oracle.bf16_to_f64(x), ow, osc, 1024, 1024)
    for out in (torch.float32, torch.bfloat16):
        y = brq().gemm(dev(x), dev(ow), dev(osc), 1024, 1024, out_dtype=out)
        if out == torch.float32:
            check_f32(f64(y), o, F32_TOL, "C1")
        else:
            check_bf16(y, o, "C1")


@pytest.fixture(scope="module")
def c2_packed():
    out = []
    for which in (0, 1):
        w = datagen.C2_weight(which)
        out.append(oracle.pack_sign1(w))
    return out


@pytest.mark.parametrize("which", [0, 1])
@pytest.mark.parametrize("M", [1, 4, 16, 64])
def test_gemm_c2_full(c2_packed, which, M):
    N, K = datagen.C2_SHAPES[which]
    say("C2 gemm", which, M, N, K)
    ow, osc = c2_packed[which]
    x = datagen.C2_x(which, M)
    o = oracle.bin_gemm(oracle.bf16_to_f64(x), ow, osc, N, K)
    y = brq().gemm(dev(x), dev(ow), dev(osc), N, K, out_dtype=torch.float32)
    check_f32(f64(y), o, F32_TOL, f"C2 {which} M={M}")
    yb = brq().gemm(dev(x), dev(ow), dev(osc), N, K, out_dtype=torch.bfloat16)
    # the bf16 output is the fp32 result rounded to nearest even
    assert np.array_equal(host_bits(yb), oracle.bf16_bits(oracle.round_bf16(f64(y))))
    check_bf16(yb, o, f"C2 {which} M={M} bf16")


def test_gemm_deterministic_and_batch_invariant(c2_packed):
    say("determinism + batch invariance")
    ow, osc = c2_packed[0]
    N, K = datagen.C2_SHAPES[0]
    x = dev(datagen.C2_x(0, 16))
    S, SC = dev(ow), dev(osc)
    a = brq().gemm(x, S, SC, N, K, out_dtype=torch.float32)
    b = brq().gemm(x, S, SC, N, K, out_dtype=torch.float32)
    assert torch.equal(a, b)
    # a single row takes the fp8 x fp4 matrix-core path (fixed-point digit
    # rows), several rows the fp16 one; both are exact up to fp32 sums, so
    # they agree to the fp32 bar, and the single-row path is deterministic
    for m in (0, 5, 15):
        xm = x[m:m + 1].contiguous()
        r = brq().gemm(xm, S, SC, N, K, out_dtype=torch.float32)
        assert torch.equal(r, brq().gemm(xm, S, SC, N, K, out_dtype=torch.float32))
        assert maxrel(f64(r[0]), f64(a[m])) <= F32_TOL


def test_gemm_end_to_end_device_packed():
    say("gemm with device-packed weights 1024x2048")
    N, K, M = 1024, 2048, 8
    w = datagen.normal_f32((72, 0), (N, K), 0.02)
    x = datagen.bf16_normal((72, 1), (M, K))
    ow, osc = oracle.pack_sign1(w)
    o = oracle.bin_gemm(oracle.bf16_to_f64(x), ow, osc, N, K)
    s, sc = brq().pack(dev(w))
    y = brq().gemm(dev(x), s, sc, N, K, out_dtype=torch.float32)
    check_f32(f64(y), o, 1e-3, "device-packed")   # scales may differ by one fp16 ulp


# ---------------------------------------------------------------------------
# S4 DBF
# ---------------------------------------------------------------------------

def _dbf_case(M, m, n, r, key, out=torch.float32):
    v = datagen.pm1_f32((73, key, 0), (r, n))
    u = datagen.pm1_f32((73, key, 1), (m, r))
    d_in = datagen.f16_lognormal((73, key, 2), (n,))
    d_mid = datagen.f16_lognormal((73, key, 3), (r,))
    d_out = datagen.f16_lognormal((73, key, 4), (m,))
    x = datagen.bf16_normal((73, key, 5), (M, n))
    vw, uw = oracle.pack_sign1_only(v), oracle.pack_sign1_only(u)
    o = oracle.dbf_chain(oracle.bf16_to_f64(x), d_in, vw, d_mid, uw, d_out, m, n, r)
    y = brq().dbf_gemm(dev(x), dev(d_in), dev(vw), dev(d_mid), dev(uw), dev(d_out), m, n, r, out_dtype=out)
    torch.cuda.synchronize()
    return y, o


# one row with n % 512 == 0: the first stage on the fp8 x fp4 matrix cores
# with x_s = D_in x as digit rows, one wave (n = 512), three (1536), 17 chunks
# in pairs with the last wave's second slot empty (8704), 16 waves of two
# (16384, beyond 64 KiB of LDS); ranks of 8 to 24 16-row tiles
@pytest.mark.parametrize("m,n,r", [(64, 512, 384), (40, 1536, 128), (130, 8704, 256), (48, 16384, 128)])
def test_dbf_single_row_digit_stage(m, n, r):
    say("dbf single row digit stage", m, n, r)
    for out in (torch.float32, torch.bfloat16):
        y, o = _dbf_case(1, m, n, r, m + n + r, out=out)
        if out == torch.float32:
            check_f32(f64(y), o, F32_TOL, f"dbf 1x{m}x{n} r={r}")
        else:
            check_bf16(y, o, f"dbf 1x{m}x{n} r={r} bf16")


def test_dbf_single_row_activation_range():
    """Single rows at 1e5, 1e30, 0, 1e-30, 2^-20 on the digit first stage:
    each matches the oracle to the fp32 bar, the zero row gives zeros."""
    say("dbf single row activation range")
    m_, n_, r_ = 64, 1024, 128
    v = datagen.pm1_f32((79, 2, 0), (r_, n_))
    u = datagen.pm1_f32((79, 2, 1), (m_, r_))
    d_in, d_mid, d_out = (datagen.f16_lognormal((79, 2, 2 + i), (s_,)) for i, s_ in enumerate((n_, r_, m_)))
    vw, uw = oracle.pack_sign1_only(v), oracle.pack_sign1_only(u)
    base = datagen.rng(79, 2, 3).standard_normal(n_).astype(np.float32)
    for sc in (1e5, 1e30, 0.0, 1e-30, 2.0 ** -20):
        xb = datagen.bf16_bits_from_f32((base * np.float32(sc))[None, :])
        o = oracle.dbf_chain(oracle.bf16_to_f64(xb), d_in, vw, d_mid, uw, d_out, m_, n_, r_)
        y = f64(brq().dbf_gemm(dev(xb), dev(d_in), dev(vw), dev(d_mid), dev(uw), dev(d_out), m_, n_, r_,
                               out_dtype=torch.float32))
        assert np.all(np.isfinite(y))
        if np.any(o):
            check_f32(y, o, F32_TOL, f"dbf single row at scale {sc:g}")
        else:
            assert not np.any(y)


def _signed(d, key):
    """The diagonal d with each entry's sign drawn at random (the diagonals
    are real-valued, so either sign is valid)."""
    g = datagen.rng(97, *key)
    return np.where(g.random(d.shape) < 0.5, -d, d).astype(np.float16)


# negative diagonal entries: D_in enters the first product as the weight
# operand's magnitude on the fp16 paths (one row with n = 640, three rows,
# the tiled path at M = 100, and the one-launch chain) and as x_s on the
# digit path (one row, n = 1024); D_mid and D_out scale in fp32
@pytest.mark.parametrize("M,m,n,r", [(1, 64, 640, 256), (1, 64, 1024, 128), (3, 200, 512, 256),
                                     (100, 256, 512, 384)])
def test_dbf_negative_diagonals(M, m, n, r):
    say("dbf negative diagonals", M, m, n, r)
    key = (M, m, n, r)
    v = datagen.pm1_f32((98,) + key + (0,), (r, n))
    u = datagen.pm1_f32((98,) + key + (1,), (m, r))
    d_in, d_mid, d_out = (_signed(datagen.f16_lognormal((98,) + key + (2 + i,), (s_,)), key + (i,))
                          for i, s_ in enumerate((n, r, m)))
    assert (d_in < 0).any() and (d_mid < 0).any() and (d_out < 0).any()
    x = datagen.bf16_normal((98,) + key + (5,), (M, n))
    vw, uw = oracle.pack_sign1_only(v), oracle.pack_sign1_only(u)
    o = oracle.dbf_chain(oracle.bf16_to_f64(x), d_in, vw, d_mid, uw, d_out, m, n, r)
    args = (dev(x), dev(d_in), dev(vw), dev(d_mid), dev(uw), dev(d_out), m, n, r)
    y = brq().dbf_gemm(*args, out_dtype=torch.float32)
    check_f32(f64(y), o, F32_TOL, f"dbf negative diagonals {key}")
    if M <= 8:
        brq().set_decode_fusion(brq().FUSION_ON)
        try:
            y1 = brq().dbf_gemm(*args, out_dtype=torch.float32)
            check_f32(f64(y1), o, F32_TOL, f"dbf negative diagonals, one launch {key}")
        finally:
            brq().set_decode_fusion(brq().FUSION_DEFAULT)
    # the Q8 chain quantises x_s = D_in x and h_s, signs included
    oq = oracle.dbf_chain_q8(oracle.bf16_to_f64(x), d_in, vw, d_mid, uw, d_out, m, n, r)
    check_q8(_q8_run(x, d_in, vw, d_mid, uw, d_out, m, n, r), oq, f"dbf q8 negative diagonals {key}")


class _SignedDiagonals:
    """A DBF-expert configuration whose three diagonals per projection take
    random signs."""

    def __init__(self, cfg):
        self.cfg = cfg

    def __getattr__(self, name):
        return getattr(self.cfg, name)

    def proj(self, e, p):
        d = dict(self.cfg.proj(e, p))
        for i, name in enumerate(("d_in", "d_mid", "d_out")):
            d[name] = _signed(d[name], (e, p, i))
        return d


# the routed DBF-expert layer with signed diagonals: stage 0 on fp16 tiles
# (H = 384) and on digit rows (H = 512), the down chain's D_in on the a rows,
# few-token (T = 2) and grouped (T = 7, 24) paths
@pytest.mark.parametrize("T,E,H,I,r,k", [(2, 8, 384, 256, 256, 3), (7, 8, 384, 256, 256, 3),
                                         (24, 16, 512, 128, 256, 4)])
def test_moe_dbf_negative_diagonals(T, E, H, I, r, k):
    say("moe dbf negative diagonals", T, E, H, I, r, k)
    cfg = _SignedDiagonals(datagen.C4D(E=E, H=H, I=I, r=r, top_k=k, layer=9))
    y, o = _dbf_moe_case(cfg, T)
    check_f32(f64(y), o, F32_TOL, f"moe dbf negative diagonals T={T} H={H}")


@pytest.mark.parametrize("M,m,n,r", [(1, 16, 128, 128), (1, 48, 256, 384), (3, 200, 512, 256), (32, 64, 640, 512),
                                     (33, 96, 256, 128), (100, 256, 512, 384)])
def test_dbf_small(M, m, n, r):
    say("dbf", M, m, n, r)
    y, o = _dbf_case(M, m, n, r, M + m + n + r)
    check_f32(f64(y), o, F32_TOL, f"dbf {M},{m},{n},{r}")


# long h_s rows on the tiled path: the row split keeps 1, 2, 4 or 8 quads of
# values per thread in registers (r up to 16384) and re-reads longer rows
@pytest.mark.parametrize("r", [4096, 8192, 16384, 16512])
def test_dbf_tiled_long_rank(r):
    say("dbf tiled, long rank", r)
    y, o = _dbf_case(9, 64, 256, r, 9000 + r)
    check_f32(f64(y), o, F32_TOL, f"dbf 9,64,256,{r}")


# h_s of small magnitude (d_mid at 2^-12 of its usual spread, so |h_s| ~ 1e-3
# and below): an unscaled fp16 hi/lo pair keeps few bits there (its lo piece is
# subnormal below 2^-3); the scaled pieces keep about 22. Decode (M <= 8) and
# tiled (M = 100) paths.
@pytest.mark.parametrize("M", [1, 5, 100])
def test_dbf_small_intermediates(M):
    say("dbf small h_s", M)
    m, n, r = 192, 512, 384
    key = (74, M)
    v = datagen.pm1_f32(key + (0,), (r, n))
    u = datagen.pm1_f32(key + (1,), (m, r))
    d_in = datagen.f16_lognormal(key + (2,), (n,))
    d_mid = (datagen.f16_lognormal(key + (3,), (r,)).astype(np.float32) * 2.0 ** -12).astype(np.float16)
    d_out = datagen.f16_lognormal(key + (4,), (m,))
    x = datagen.bf16_normal(key + (5,), (M, n))
    vw, uw = oracle.pack_sign1_only(v), oracle.pack_sign1_only(u)
    o = oracle.dbf_chain(oracle.bf16_to_f64(x), d_in, vw, d_mid, uw, d_out, m, n, r)
    y = brq().dbf_gemm(dev(x), dev(d_in), dev(vw), dev(d_mid), dev(uw), dev(d_out), m, n, r,
                       out_dtype=torch.float32)
    torch.cuda.synchronize()
    check_f32(f64(y), o, F32_TOL, f"dbf small h_s M={M}")


# the DBF workload at about 2 bits per element: r = 4096 on 4096 x 4096
# (2.0117 bpe, section 1.1's bit budget), decode and tiled paths
@pytest.mark.parametrize("M", [1, 512])
def test_dbf_c3_rank4096(M):
    say("C3 dbf r=4096", M)
    d = datagen.C3(M, r=4096)
    vw, uw = oracle.pack_sign1_only(d["v"]), oracle.pack_sign1_only(d["u"])
    m, n, r = d["m"], d["n"], d["r"]
    o = oracle.dbf_chain(oracle.bf16_to_f64(d["x"]), d["d_in"], vw, d["d_mid"], uw, d["d_out"], m, n, r)
    args = (dev(d["x"]), dev(d["d_in"]), dev(vw), dev(d["d_mid"]), dev(uw), dev(d["d_out"]), m, n, r)
    y = brq().dbf_gemm(*args, out_dtype=torch.float32)
    check_f32(f64(y), o, F32_TOL, f"C3 r=4096 M={M}")
    yb = brq().dbf_gemm(*args, out_dtype=torch.bfloat16)
    check_bf16(yb, o, f"C3 r=4096 M={M} bf16")


@pytest.mark.parametrize("M", [1, 512])
def test_dbf_c3(M):
    say("C3 dbf", M)
    d = datagen.C3(M)
    vw, uw = oracle.pack_sign1_only(d["v"]), oracle.pack_sign1_only(d["u"])
    m, n, r = d["m"], d["n"], d["r"]
    o = oracle.dbf_chain(oracle.bf16_to_f64(d["x"]), d["d_in"], vw, d["d_mid"], uw, d["d_out"], m, n, r)
    args = (dev(d["x"]), dev(d["d_in"]), dev(vw), dev(d["d_mid"]), dev(uw), dev(d["d_out"]), m, n, r)
    y = brq().dbf_gemm(*args, out_dtype=torch.float32)
    check_f32(f64(y), o, F32_TOL, f"C3 M={M}")
    yb = brq().dbf_gemm(*args, out_dtype=torch.bfloat16)
    check_bf16(yb, o, f"C3 M={M} bf16")


def test_dbf_device_packed_factors():
    say("dbf with device-packed SIGN1 factors")
    m, n, r, M = 128, 256, 128, 2
    v = datagen.pm1_f32((74, 0), (r, n))
    u = datagen.pm1_f32((74, 1), (m, r))
    d_in = datagen.f16_lognormal((74, 2), (n,))
    d_mid = datagen.f16_lognormal((74, 3), (r,))
    d_out = datagen.f16_lognormal((74, 4), (m,))
    x = datagen.bf16_normal((74, 5), (M, n))
    o = oracle.dbf_chain(oracle.bf16_to_f64(x), d_in, oracle.pack_sign1_only(v), d_mid, oracle.pack_sign1_only(u),
                         d_out, m, n, r)
    vs, _ = brq().pack(dev(v), scales=False)
    us, _ = brq().pack(dev(u), scales=False)
    y = brq().dbf_gemm(dev(x), dev(d_in), vs, dev(d_mid), us, dev(d_out), m, n, r, out_dtype=torch.float32)
    check_f32(f64(y), o, F32_TOL, "dbf device-packed")


# ---------------------------------------------------------------------------
# DBF chain over Q8 activation codes
# ---------------------------------------------------------------------------

# The codes and exponents are decided from values that are exact in fp32 on
# both sides, the integer reductions are exact, and the only roundings are
# h_s to fp32 (the same single rounding on both sides) and the final product
# with d_out: the fp32 output is within one rounding (2^-24, relative,
# elementwise) of the oracle's fp64 value.
Q8_REL = 2.0 ** -24 * 1.01


def check_q8(y, o, what):
    g = f64(y)
    err = np.abs(g - o)
    bad = err > Q8_REL * np.abs(o)
    assert not bad.any(), f"{what}: {int(bad.sum())} elements off, worst {float(err.max()):.3e}"


def _q8_inputs(M, m, n, r, key):
    v = datagen.pm1_f32((75, key, 0), (r, n))
    u = datagen.pm1_f32((75, key, 1), (m, r))
    d_in = datagen.f16_lognormal((75, key, 2), (n,))
    d_mid = datagen.f16_lognormal((75, key, 3), (r,))
    d_out = datagen.f16_lognormal((75, key, 4), (m,))
    x = datagen.bf16_normal((75, key, 5), (M, n))
    return x, d_in, oracle.pack_sign1_only(v), d_mid, oracle.pack_sign1_only(u), d_out


def _q8_run(x, d_in, vw, d_mid, uw, d_out, m, n, r, out=torch.float32):
    y = brq().dbf_gemm_q8(dev(x), dev(d_in), dev(vw), dev(d_mid), dev(uw), dev(d_out), m, n, r, out_dtype=out)
    torch.cuda.synchronize()
    return y


# several 128 x 128 tiles with ragged row and column tails, 64-wide k-steps;
# three with few tiles and long reductions, which split along k into 2 or 4
# int32 partial sums (m = 99: the output pass off 4-element rows, and bf16
# pairs that straddle 4-byte boundaries); rows longer than 16384 (n or r =
# 16512) take the quantiser that re-reads its row; M = 1000 with m = 4001
# gives the second product 8 x 32 tiles, enough for 128-row tiles, with a
# 104-row tail, an odd column count and bf16 pairs straddling 4-byte words
@pytest.mark.parametrize("M,m,n,r", [(1, 16, 128, 128), (5, 201, 384, 256), (127, 128, 256, 128),
                                     (130, 300, 640, 384), (300, 96, 512, 640), (3, 130, 1024, 1280),
                                     (70, 100, 2048, 1024), (9, 99, 1024, 1024), (3, 64, 16512, 256),
                                     (2, 64, 256, 16512), (1000, 4001, 256, 256)])
def test_dbf_q8_small(M, m, n, r):
    say("dbf q8", M, m, n, r)
    x, d_in, vw, d_mid, uw, d_out = _q8_inputs(M, m, n, r, M + m + n + r)
    if M > 1:
        x[M // 2] = 0                      # an all-zero row: exponent 0, codes 0, output 0
    o = oracle.dbf_chain_q8(oracle.bf16_to_f64(x), d_in, vw, d_mid, uw, d_out, m, n, r)
    y = _q8_run(x, d_in, vw, d_mid, uw, d_out, m, n, r)
    check_q8(y, o, f"dbf q8 {M},{m},{n},{r}")
    if M > 1:
        assert not f64(y)[M // 2].any()
    # bf16 output: the fp32 value (one rounding of the exact d_out * integer
    # * 2^e) rounded to nearest even bf16, bit for bit
    yb = _q8_run(x, d_in, vw, d_mid, uw, d_out, m, n, r, out=torch.bfloat16)
    want = datagen.bf16_bits_from_f32(o.astype(np.float32))
    assert np.array_equal(host_bits(yb), want), f"dbf q8 {M},{m},{n},{r} bf16"


def test_dbf_q8_ties_and_exponent_edges():
    """Rows whose values land exactly on half codes (round half to even), a row
    whose maximum is exactly 127 * 2^e (code 127 at that exponent) and one a
    half step above it (the next exponent up), with unit d_in so that x_s = x."""
    say("dbf q8 ties")
    M, m, n, r = 6, 128, 256, 128
    x, _, vw, d_mid, uw, d_out = _q8_inputs(M, m, n, r, 11)
    d_in = np.ones(n, np.float16)
    half = datagen.rng(75, 99).integers(-126, 127, size=(M, n)).astype(np.float32) + 0.5
    rows = np.zeros((M, n), np.float32)
    rows[0] = half[0] * 2.0 ** -3
    rows[0, 7] = 127 * 2.0 ** -3            # max exactly 127 * 2^-3: codes are half[0] rounded to even
    rows[1] = half[1] * 2.0 ** 5
    rows[1, 3] = -127 * 2.0 ** 5
    rows[2] = np.round(half[2]) * 2.0 ** -9
    rows[2, 0] = 127.5 * 2.0 ** -9           # just past 127 * 2^-9: exponent -8
    rows[3] = half[3]
    rows[3, 5] = 127                        # exponent 0: the ties themselves
    rows[4, 9] = -3.0                       # one non-zero value
    rows[5] = half[5] * 2.0 ** -20
    rows[5, 1] = 127 * 2.0 ** -20
    x = datagen.bf16_bits_from_f32(rows)
    assert np.array_equal(oracle.bf16_to_f64(x), rows.astype(np.float64))   # every value is exact in bf16
    o = oracle.dbf_chain_q8(oracle.bf16_to_f64(x), d_in, vw, d_mid, uw, d_out, m, n, r)
    y = _q8_run(x, d_in, vw, d_mid, uw, d_out, m, n, r)
    check_q8(y, o, "dbf q8 ties")


# the full-size case at the launch configuration the benchmark times (all 512
# rows computed), compared on sampled rows: rows are independent in the chain
# (each has its own exponents), so the oracle runs on those rows alone
# 1 and 512 rows are the DBF workload's sizes (64-row tiles; one row splits
# both reductions); 4096 rows run the 128-row tiles the benchmark times
@pytest.mark.parametrize("M", [1, 512, 4096])
def test_dbf_q8_c3_sampled_rows(M):
    say("C3 dbf q8 sampled rows", M)
    d = datagen.C3(M)
    vw, uw = oracle.pack_sign1_only(d["v"]), oracle.pack_sign1_only(d["u"])
    m, n, r = d["m"], d["n"], d["r"]
    y = _q8_run(d["x"], d["d_in"], vw, d["d_mid"], uw, d["d_out"], m, n, r)
    rows = {1: np.array([0]), 512: np.array([0, 1, 127, 128, 255, 300, 383, 511]),
            4096: np.array([0, 1, 127, 128, 2047, 2048, 4094, 4095])}[M]
    o = oracle.dbf_chain_q8(oracle.bf16_to_f64(d["x"][rows]), d["d_in"], vw, d["d_mid"], uw, d["d_out"], m, n, r)
    check_q8(y[torch.from_numpy(rows).to(y.device)], o, f"C3 q8 M={M} sampled")
    # and the distance to the unquantised chain stays at the level of two 7-bit
    # magnitude quantisations (a few percent; one row alone, measured: 5.1%)
    full = oracle.dbf_chain(oracle.bf16_to_f64(d["x"][rows]), d["d_in"], vw, d["d_mid"], uw, d["d_out"], m, n, r)
    assert 1e-3 < l2rel(f64(y)[rows], full) < 1e-1


# ---------------------------------------------------------------------------
# S5 / S6 MoE
# ---------------------------------------------------------------------------

class _Experts:
    def __init__(self, cfg: datagen.C4):
        self.cfg = cfg
        E, H, I = cfg.E, cfg.H, cfg.I
        self.gw = np.zeros((E, I, H // 64), np.uint64)
        self.gs = np.zeros((E, I, H // 128), np.float16)
        self.uw = np.zeros_like(self.gw)
        self.us = np.zeros_like(self.gs)
        self.dw = np.zeros((E, H, I // 64), np.uint64)
        self.ds = np.zeros((E, H, I // 128), np.float16)
        for e in range(E):
            self.gw[e], self.gs[e] = oracle.pack_sign1(cfg.gate(e))
            self.uw[e], self.us[e] = oracle.pack_sign1(cfg.up(e))
            self.dw[e], self.ds[e] = oracle.pack_sign1(cfg.down(e))
        self.d = [dev(a) for a in (self.gw, self.gs, self.uw, self.us, self.dw, self.ds)]

    def __call__(self, e):
        return self.gw[e], self.gs[e], self.uw[e], self.us[e], self.dw[e], self.ds[e]


@pytest.fixture(scope="module")
def c4_experts():
    return _Experts(datagen.C4())


def _moe_check(ex, T, it=0, out=torch.float32):
    c = ex.cfg
    x = c.x(T)
    lg = c.logits(T, it)
    o, oids, ow = oracle.moe_ffn(oracle.bf16_to_f64(x), lg, ex, c.H, c.I, c.top_k)
    y, ids, w = brq().moe_ffn(dev(x), dev(lg), *ex.d, c.E, c.H, c.I, c.top_k, out_dtype=out, return_routing=True)
    torch.cuda.synchronize()
    assert np.array_equal(ids.cpu().numpy().astype(np.int64), oids), "top-k ids differ"
    assert np.allclose(w.cpu().numpy(), ow, rtol=1e-6, atol=1e-7)
    return y, o


@pytest.mark.parametrize("T", [1, 4, 16, 64])
def test_moe_c4(c4_experts, T):
    say("C4 moe", T)
    y, o = _moe_check(c4_experts, T)
    check_f32(f64(y), o, F32_TOL, f"moe T={T}")


# activations at 2^-7 of the usual scale put the SwiGLU output near 1e-4,
# where an unscaled fp16 hi/lo pair is subnormal; the down launches stage it
# as scaled pieces. T = 2 takes the token path, T = 24 the grouped one.
@pytest.mark.parametrize("T", [2, 24])
def test_moe_small_intermediates(T):
    say("moe small SwiGLU output", T)
    cfg = datagen.C4(E=16, H=256, I=256, top_k=4, layer=7)
    ex = _Experts(cfg)
    xf = oracle.bf16_to_f64(cfg.x(T)) * 2.0 ** -7
    x = (xf.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)  # exact: a power-of-two scale
    lg = cfg.logits(T)
    o, _, _ = oracle.moe_ffn(oracle.bf16_to_f64(x), lg, ex, cfg.H, cfg.I, cfg.top_k)
    y = brq().moe_ffn(dev(x), dev(lg), *ex.d, cfg.E, cfg.H, cfg.I, cfg.top_k, out_dtype=torch.float32)
    torch.cuda.synchronize()
    check_f32(f64(y), o, F32_TOL, f"moe small a T={T}")


# hidden sizes on the digit path of the grouped gate/up (a multiple of 512):
# one wave (H = 512) and three (H = 1536), routes in pairs with an odd count
@pytest.mark.parametrize("T,H,I,k", [(24, 512, 256, 4), (9, 1536, 128, 3), (40, 512, 128, 1), (6, 512, 256, 4)])
def test_moe_digit_gateup_shapes(T, H, I, k):
    say("moe digit gate/up", T, H, I, k)
    cfg = datagen.C4(E=16, H=H, I=I, top_k=k, layer=13)
    ex = _Experts(cfg)
    x, lg = cfg.x(T), cfg.logits(T)
    o, oids, _ = oracle.moe_ffn(oracle.bf16_to_f64(x), lg, ex, cfg.H, cfg.I, cfg.top_k)
    y, ids, _ = brq().moe_ffn(dev(x), dev(lg), *ex.d, cfg.E, cfg.H, cfg.I, cfg.top_k, out_dtype=torch.float32,
                              return_routing=True)
    torch.cuda.synchronize()
    assert np.array_equal(ids.cpu().numpy().astype(np.int64), oids)
    check_f32(f64(y), o, F32_TOL, f"moe digit gate/up T={T} H={H}")


def test_moe_c4_bf16_and_fresh_logits(c4_experts):
    say("C4 moe bf16, several logit draws")
    for it in range(3):
        y, o = _moe_check(c4_experts, 4, it=it + 1, out=torch.bfloat16)
        check_bf16(y, o, f"moe bf16 it={it}")


# ---------------------------------------------------------------------------
# MoE with DBF experts (the DBF post's deployed layer): every projection a
# D_in V D_mid U D_out chain
# ---------------------------------------------------------------------------

def _dbf_moe_dev(cfg, experts):
    """Device records [E, ...] per projection: the configuration's factors for
    `experts`, zeros for the others (never selected by the logits used)."""
    E, H, I, r = cfg.E, cfg.H, cfg.I, cfg.r
    recs = []
    for p, (m, n) in enumerate(((I, H), (I, H), (H, I))):
        d_in = np.zeros((E, n), np.float16)
        v = np.zeros((E, r, n // 64), np.uint64)
        d_mid = np.zeros((E, r), np.float16)
        u = np.zeros((E, m, r // 64), np.uint64)
        d_out = np.zeros((E, m), np.float16)
        for e in experts:
            d = cfg.proj(e, p)
            d_in[e], d_mid[e], d_out[e] = d["d_in"], d["d_mid"], d["d_out"]
            v[e] = oracle.pack_sign1_only(d["v"]).reshape(r, n // 64)
            u[e] = oracle.pack_sign1_only(d["u"]).reshape(m, r // 64)
        recs.append(tuple(dev(a) for a in (d_in, v, d_mid, u, d_out)))
    return recs


def _dbf_moe_oracle_experts(cfg):
    def rec(e, p):
        d = cfg.proj(e, p)
        return (d["d_in"], oracle.pack_sign1_only(d["v"]), d["d_mid"], oracle.pack_sign1_only(d["u"]), d["d_out"])

    cache = {}

    def ex(e):
        if e not in cache:
            cache[e] = (rec(e, 0), rec(e, 1), rec(e, 2))
        return cache[e]

    return ex


def _dbf_moe_case(cfg, T, out=torch.float32, it=0):
    x = cfg.x(T)
    lg = cfg.logits(T, it)
    ids_o, _ = oracle.route_topk(lg, cfg.top_k)
    recs = _dbf_moe_dev(cfg, sorted(set(int(e) for e in ids_o.ravel())))
    o, oids, ow = oracle.moe_dbf_ffn(oracle.bf16_to_f64(x), lg, _dbf_moe_oracle_experts(cfg), cfg.H, cfg.I, cfg.r,
                                     cfg.top_k)
    y, ids, w = brq().moe_dbf_ffn(dev(x), dev(lg), *recs, cfg.E, cfg.H, cfg.I, cfg.r, cfg.top_k, out_dtype=out,
                                  return_routing=True)
    torch.cuda.synchronize()
    assert np.array_equal(ids.cpu().numpy().astype(np.int64), oids), "top-k ids differ"
    assert np.allclose(w.cpu().numpy(), ow, rtol=1e-6, atol=1e-7)
    return y, o


# small experts: T = 1 and 3 take the few-token path (one route per block, the
# last stage fused with the slot sum; r = 640 gives a ragged last chunk), T = 4
# with T*k > E and T = 5 the grouped one with 4-token tiles, T = 64 (16 routes
# per expert) 16-token tiles and several tiles per expert; odd sizes with
# ragged blocks
@pytest.mark.parametrize("T,E,H,I,r,k", [(1, 16, 256, 128, 128, 4), (3, 16, 256, 128, 640, 4),
                                         (4, 8, 256, 128, 128, 3), (5, 16, 256, 128, 128, 4),
                                         (64, 16, 256, 128, 128, 4), (7, 8, 384, 256, 256, 3),
                                         (2, 16, 512, 128, 256, 4), (24, 16, 512, 128, 256, 4),
                                         (9, 8, 1536, 256, 128, 3)])
def test_moe_dbf_small(T, E, H, I, r, k):
    say("moe dbf", T, E, H, I, r, k)
    cfg = datagen.C4D(E=E, H=H, I=I, r=r, top_k=k, layer=1)
    y, o = _dbf_moe_case(cfg, T)
    check_f32(f64(y), o, F32_TOL, f"moe dbf T={T}")


def test_moe_dbf_deployed_shape():
    # the deployed layer (256 experts, top-8, gate/up 512x2048, down 2048x512,
    # r = 1024) at T = 4: every selected expert built, fp32 and bf16 outputs
    say("moe dbf deployed shape T=4")
    cfg = datagen.C4D()
    T = 4
    x, lg = cfg.x(T), cfg.logits(T)
    ids_o, _ = oracle.route_topk(lg, cfg.top_k)
    recs = _dbf_moe_dev(cfg, sorted(set(int(e) for e in ids_o.ravel())))
    o, _, _ = oracle.moe_dbf_ffn(oracle.bf16_to_f64(x), lg, _dbf_moe_oracle_experts(cfg), cfg.H, cfg.I, cfg.r,
                                 cfg.top_k)
    for out in (torch.float32, torch.bfloat16):
        y = brq().moe_dbf_ffn(dev(x), dev(lg), *recs, cfg.E, cfg.H, cfg.I, cfg.r, cfg.top_k, out_dtype=out)
        torch.cuda.synchronize()
        if out == torch.float32:
            check_f32(f64(y), o, F32_TOL, "moe dbf deployed")
        else:
            check_bf16(y, o, "moe dbf deployed bf16")


def test_moe_dbf_deployed_shape_t64_sampled_tokens():
    # the deployed layer at T = 64 (the grouped path, every expert built),
    # checked on 8 sampled tokens (fp32) and on all of them for the routing
    say("moe dbf deployed shape T=64, sampled tokens")
    cfg = datagen.C4D()
    T = 64
    x, lg = cfg.x(T), cfg.logits(T)
    ids_o, _ = oracle.route_topk(lg, cfg.top_k)
    recs = _dbf_moe_dev(cfg, sorted(set(int(e) for e in ids_o.ravel())))
    toks = [0, 5, 17, 31, 32, 47, 58, 63]
    o, oids, ow = oracle.moe_dbf_ffn(oracle.bf16_to_f64(x), lg, _dbf_moe_oracle_experts(cfg), cfg.H, cfg.I, cfg.r,
                                     cfg.top_k, tokens=toks)
    y, ids, w = brq().moe_dbf_ffn(dev(x), dev(lg), *recs, cfg.E, cfg.H, cfg.I, cfg.r, cfg.top_k,
                                  out_dtype=torch.float32, return_routing=True)
    torch.cuda.synchronize()
    assert np.array_equal(ids.cpu().numpy().astype(np.int64), oids)
    check_f32(f64(y)[toks], o[toks], F32_TOL, "moe dbf deployed T=64")


def _dbf_moe_packed(cfg, experts):
    """Device records [E, ...] per projection (the experts' factors from
    C4D.proj_packed, zeros for the others) and the oracle's expert lookup,
    both from the same arrays."""
    E, H, I, r = cfg.E, cfg.H, cfg.I, cfg.r
    recs, host = [], {e: [] for e in experts}
    for p, (m, n) in enumerate(((I, H), (I, H), (H, I))):
        d_in = np.zeros((E, n), np.float16)
        v = np.zeros((E, r, n // 64), np.uint64)
        d_mid = np.zeros((E, r), np.float16)
        u = np.zeros((E, m, r // 64), np.uint64)
        d_out = np.zeros((E, m), np.float16)
        for e in experts:
            d = cfg.proj_packed(e, p)
            d_in[e], d_mid[e], d_out[e] = d["d_in"], d["d_mid"], d["d_out"]
            v[e] = d["v"].reshape(r, n // 64)
            u[e] = d["u"].reshape(m, r // 64)
            host[e].append((d["d_in"], d["v"], d["d_mid"], d["u"], d["d_out"]))
        recs.append(tuple(dev(a) for a in (d_in, v, d_mid, u, d_out)))
    return recs, lambda e: tuple(host[e])


# the other MoE geometries the DBF post names (its section 9), full projection
# shapes with top-8 routing and r = 2048 (the most the layer accepts); only
# the selected experts are built. T = 1 and 3 take the few-token path, T = 5
# and 6 the grouped one; GLM-5.2's hidden 6144 gives the gate/up V factors
# two 512-wide chunks per wave.
@pytest.mark.parametrize("name,T", [("GLM-4.5-Air", 1), ("MiniMax-M2.5", 3), ("DeepSeek-V4-Flash", 5),
                                    ("GLM-5.2", 1), ("GLM-5.2", 6)])
def test_moe_dbf_named_geometries(name, T):
    say("moe dbf geometry", name, T)
    g = {**datagen.MOE_GEOMETRIES, **datagen.MOE_GEOMETRY_WIDE}[name]
    cfg = datagen.C4D(E=g["E"], H=g["H"], I=g["I"], r=g["r"], top_k=8, layer=11)
    x, lg = cfg.x(T), cfg.logits(T)
    ids_o, _ = oracle.route_topk(lg, cfg.top_k)
    recs, ex = _dbf_moe_packed(cfg, sorted(set(int(e) for e in ids_o.ravel())))
    o, oids, ow = oracle.moe_dbf_ffn(oracle.bf16_to_f64(x), lg, ex, cfg.H, cfg.I, cfg.r, cfg.top_k)
    y, ids, w = brq().moe_dbf_ffn(dev(x), dev(lg), *recs, cfg.E, cfg.H, cfg.I, cfg.r, cfg.top_k,
                                  out_dtype=torch.float32, return_routing=True)
    yb = brq().moe_dbf_ffn(dev(x), dev(lg), *recs, cfg.E, cfg.H, cfg.I, cfg.r, cfg.top_k, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert np.array_equal(ids.cpu().numpy().astype(np.int64), oids)
    assert np.allclose(w.cpu().numpy(), ow, rtol=1e-6, atol=1e-7)
    check_f32(f64(y), o, F32_TOL, f"moe dbf {name} T={T}")
    check_bf16(yb, o, f"moe dbf {name} T={T} bf16")


def _moe_packed_selected(E, H, I, experts, key):
    """Group-128 experts at full projection shapes with only `experts` built
    (random sign words, fp16 scales in [0.01, 0.03), near the 0.016 of a
    packed N(0, 0.02^2) matrix), the others zero: device tensors in the
    order brq.moe_ffn takes them and the oracle's lookup, from the same arrays."""
    host = []
    for p, (n, k) in enumerate(((I, H), (I, H), (H, I))):
        w = np.zeros((E, n, k // 64), np.uint64)
        sc = np.zeros((E, n, k // 128), np.float16)
        for e in experts:
            w[e] = datagen.sign_words((97, key, e, p, 0), n, k).reshape(n, k // 64)
            sc[e] = (0.01 + 0.02 * datagen.rng(97, key, e, p, 1).random((n, k // 128))).astype(np.float16)
        host += [w, sc]
    return [dev(a) for a in host], (lambda e: tuple(a[e] for a in host))


# the group-128 layer at the named geometries, full projection shapes, top-8:
# the router logits favour ten experts so that the oracle's dense
# reconstructions stay few; T = 1 takes the few-token path, T = 6 the grouped
# one; GLM-5.2's hidden 6144 gives the gate/up reductions two chunks per wave
@pytest.mark.parametrize("name,T", [("GLM-4.5-Air", 6), ("MiniMax-M2.5", 1), ("DeepSeek-V4-Flash", 6),
                                    ("GLM-5.2", 1), ("GLM-5.2", 6)])
def test_moe_named_geometries(name, T):
    say("moe geometry", name, T)
    geo = {**datagen.MOE_GEOMETRIES, **datagen.MOE_GEOMETRY_WIDE}
    g = geo[name]
    E, H, I = g["E"], g["H"], g["I"]
    key = sorted(geo).index(name)
    x = datagen.bf16_normal((98, key, T), (T, H))
    lg = datagen.router_logits((99, key, T), T, E)
    favoured = datagen.rng(96, key).choice(E, size=10, replace=False)
    lg[:, favoured] += np.float32(8.0)
    ids_o, _ = oracle.route_topk(lg, 8)
    d, ex = _moe_packed_selected(E, H, I, sorted(set(int(e) for e in ids_o.ravel())), key)
    o, oids, ow = oracle.moe_ffn(oracle.bf16_to_f64(x), lg, ex, H, I, 8)
    y, ids, w = brq().moe_ffn(dev(x), dev(lg), *d, E, H, I, 8, out_dtype=torch.float32, return_routing=True)
    yb = brq().moe_ffn(dev(x), dev(lg), *d, E, H, I, 8, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert np.array_equal(ids.cpu().numpy().astype(np.int64), oids)
    assert np.allclose(w.cpu().numpy(), ow, rtol=1e-6, atol=1e-7)
    check_f32(f64(y), o, F32_TOL, f"moe {name} T={T}")
    check_bf16(yb, o, f"moe {name} T={T} bf16")


# the ABI limits of the routed layers: T = 256 tokens, E = 1024 experts,
# top-16, with small projections (H = I = r = 128) so that every expert fits
def test_moe_limits():
    say("moe limits T=256 E=1024 k=16")
    cfg = datagen.C4(E=1024, H=128, I=128, top_k=16, layer=9)
    ex = _Experts(cfg)
    T = 256
    x, lg = cfg.x(T), cfg.logits(T)
    o, oids, ow = oracle.moe_ffn(oracle.bf16_to_f64(x), lg, ex, cfg.H, cfg.I, cfg.top_k)
    y, ids, w = brq().moe_ffn(dev(x), dev(lg), *ex.d, cfg.E, cfg.H, cfg.I, cfg.top_k, out_dtype=torch.float32,
                              return_routing=True)
    torch.cuda.synchronize()
    assert np.array_equal(ids.cpu().numpy().astype(np.int64), oids)
    assert np.allclose(w.cpu().numpy(), ow, rtol=1e-6, atol=1e-7)
    check_f32(f64(y), o, F32_TOL, "moe limits")


def test_moe_dbf_limits():
    say("moe dbf limits T=256 E=1024 k=16")
    cfg = datagen.C4D(E=1024, H=128, I=128, r=128, top_k=16, layer=9)
    y, o = _dbf_moe_case(cfg, 256)
    check_f32(f64(y), o, F32_TOL, "moe dbf limits")


def test_moe_ties_and_small_shapes():
    say("moe ties, E=8 H=256 I=128 k=3")
    cfg = datagen.C4(E=8, H=256, I=128, top_k=3, layer=5)
    ex = _Experts(cfg)
    T = 5
    x = cfg.x(T)
    lg = np.zeros((T, 8), np.float32)
    lg[1] = np.round(cfg.logits(1)[0], 0)
    lg[2, [2, 6, 7]] = 1.5
    lg[3] = np.arange(8, dtype=np.float32)[::-1]
    lg[4] = cfg.logits(1, 9)[0]
    o, oids, ow = oracle.moe_ffn(oracle.bf16_to_f64(x), lg, ex, cfg.H, cfg.I, 3)
    y, ids, w = brq().moe_ffn(dev(x), dev(lg), *ex.d, 8, cfg.H, cfg.I, 3, out_dtype=torch.float32,
                              return_routing=True)
    assert np.array_equal(ids.cpu().numpy().astype(np.int64), oids)
    check_f32(f64(y), o, F32_TOL, "moe ties")


# ---------------------------------------------------------------------------
# S7 Kronecker rotation
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("M", [1, 7, 4096])
def test_kron(M):
    say("kron", M)
    d = datagen.C5(M=M)
    o = oracle.kron_rotate(oracle.bf16_to_f64(d["x"]), d["H"], d["R"])
    y = brq().kron_rotate(dev(d["x"]), dev(d["H"]), dev(d["R"]))
    torch.cuda.synchronize()
    assert bf16_close(host_bits(y), o).all()
    assert l2rel(f64(y), o) <= 2e-3


@pytest.mark.parametrize("n1,n2,M", [(32, 64, 9), (64, 32, 300), (32, 32, 5), (96, 32, 7), (32, 96, 66),
                                    (96, 64, 13), (64, 96, 1030), (64, 64, 3)])
def test_kron_factor_sizes(n1, n2, M):
    """Factor sizes 32, 64 and 96 (rows of 1024 .. 6144 values), square and
    not, token counts that leave the last workgroup's waves partly idle; each
    element within 1 bf16 ulp of the rounded fp64 result."""
    say("kron factor sizes", n1, n2, M)
    d = datagen.C5(M=M, K=n1 * n2, n1=n1, n2=n2)
    o = oracle.kron_rotate(oracle.bf16_to_f64(d["x"]), d["H"], d["R"])
    y = brq().kron_rotate(dev(d["x"]), dev(d["H"]), dev(d["R"]))
    torch.cuda.synchronize()
    assert bf16_close(host_bits(y), o).all()
    assert l2rel(f64(y), o) <= 2e-3


def test_c5_prefill_sampled_columns():
    say("C5 rotate + prefill gemm, sampled columns")
    d = datagen.C5()
    N, K = d["N"], d["K"]
    w = datagen.C5_weight(N, K)
    ow, osc = oracle.pack_sign1(w)
    xr = brq().kron_rotate(dev(d["x"]), dev(d["H"]), dev(d["R"]))
    y = brq().gemm(xr, dev(ow), dev(osc), N, K, out_dtype=torch.float32)
    torch.cuda.synchronize()
    cols = np.sort(datagen.rng(75, 0).choice(N, size=96, replace=False))
    xo = oracle.kron_rotate_bf16(oracle.bf16_to_f64(d["x"]), d["H"], d["R"])
    o = oracle.bin_gemm_cols(xo, ow, osc, N, K, cols)
    # end to end: the rotated activations may differ from the oracle's by one
    # bf16 ulp where fp32 and fp64 straddle a rounding midpoint
    # (per element the product is checked below, on the oracle's rotated input)
    check_f32(f64(y)[:, cols], o, 1e-4, "C5 e2e", elementwise=False)
    assert l2rel(f64(y)[:, cols], o) <= 1e-4
    # product parity on the oracle's rotated activations
    xo_bits = oracle.bf16_bits(xo)
    y2 = brq().gemm(dev(xo_bits), dev(ow), dev(osc), N, K, out_dtype=torch.float32)
    yb2 = brq().gemm(dev(xo_bits), dev(ow), dev(osc), N, K, out_dtype=torch.bfloat16)
    sel = torch.from_numpy(cols).cuda()
    check_f32(f64(y2)[:, cols], o, F32_TOL, "C5 gemm")
    check_bf16(yb2[:, sel].contiguous(), o, "C5 gemm bf16")


# ---------------------------------------------------------------------------
# HIP graph capture: the calls enqueue only kernels, so they can be captured
# and replayed; every replay must equal the eager result
# ---------------------------------------------------------------------------

def test_graph_capture_replay():
    say("graph capture of gemm (decode + tiled), dbf, dbf over Q8 codes, moe")
    b = brq()
    N, K = 1024, 2048
    w = datagen.normal_f32((76, 0), (N, K), 0.02)
    ow, osc = oracle.pack_sign1(w)
    S, SC = dev(ow), dev(osc)
    x1 = dev(datagen.bf16_normal((76, 1), (1, K)))
    x2 = dev(datagen.bf16_normal((76, 2), (96, K)))
    d = datagen.C3(1, m=256, n=512, r=256)
    vw, uw = oracle.pack_sign1_only(d["v"]), oracle.pack_sign1_only(d["u"])
    dargs = (dev(d["x"]), dev(d["d_in"]), dev(vw), dev(d["d_mid"]), dev(uw), dev(d["d_out"]), 256, 512, 256)
    cfg = datagen.C4(E=16, H=256, I=128, top_k=4, layer=76)
    packs = [[oracle.pack_sign1(f(e)) for f in (cfg.gate, cfg.up, cfg.down)] for e in range(cfg.E)]
    mw = [dev(np.stack([pk[p][i] for pk in packs])) for p in range(3) for i in range(2)]
    xm, lg = dev(cfg.x(2)), dev(cfg.logits(2))
    # Q8 chain with both reductions split into int32 slices (9 rows, 99 outputs)
    qx, qdi, qv, qdm, qu, qdo = _q8_inputs(9, 99, 1024, 1024, 76)
    qargs = (dev(qx), dev(qdi), dev(qv), dev(qdm), dev(qu), dev(qdo), 99, 1024, 1024)
    yq = torch.empty((9, 99), dtype=torch.bfloat16, device="cuda")
    wsq = torch.empty(b.dbf_q8_workspace_bytes(9, 99, 1024, 1024), dtype=torch.uint8, device="cuda")
    y1 = torch.empty((1, N), dtype=torch.float32, device="cuda")
    y2 = torch.empty((96, N), dtype=torch.float32, device="cuda")
    yd = torch.empty((1, 256), dtype=torch.float32, device="cuda")
    ym = torch.empty((2, 256), dtype=torch.float32, device="cuda")
    wsd = torch.empty(b.dbf_workspace_bytes(1, 256, 512, 256), dtype=torch.uint8, device="cuda")
    wsm = torch.empty(b.moe_workspace_bytes(2, 256, 128, 16, 4), dtype=torch.uint8, device="cuda")

    def work():
        b.gemm(x1, S, SC, N, K, out_dtype=torch.float32, y=y1)
        b.gemm(x2, S, SC, N, K, out_dtype=torch.float32, y=y2)
        b.dbf_gemm(*dargs, out_dtype=torch.float32, y=yd, ws=wsd)
        b.dbf_gemm_q8(*qargs, out_dtype=torch.bfloat16, y=yq, ws=wsq)
        b.moe_ffn(xm, lg, *mw, cfg.E, cfg.H, cfg.I, cfg.top_k, out_dtype=torch.float32, y=ym, ws=wsm)

    work()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (y1, y2, yd, ym, yq)]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        work()
    torch.cuda.current_stream().wait_stream(s)
    with torch.cuda.graph(g):
        work()
    for rep in range(3):
        for t in (y1, y2, yd, ym, yq):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, r in zip((y1, y2, yd, ym, yq), ref):
            assert torch.equal(a, r), f"replay {rep} differs"
        work()  # eager work between replays
        torch.cuda.synchronize()


def test_injected_launch_failure_leaves_outputs():
    """brq_debug_fail_launches on the device: the armed call raises the
    BRQ_E_HIP status with its text and leaves y as it was; the next call runs
    and matches the oracle."""
    say("injected launch failure")
    b = brq()
    N, K = 64, 1024
    w = datagen.normal_f32((79, 1), (N, K), 0.02)
    x = datagen.bf16_normal((79, 2), (1, K))
    ow, osc = oracle.pack_sign1(w)
    y = torch.full((1, N), 7.0, dtype=torch.float32, device="cuda")
    assert b.lib().brq_debug_fail_launches(1) == 0
    with pytest.raises(b.BrqError, match="injected launch failure"):
        b.gemm(dev(x), dev(ow), dev(osc), N, K, out_dtype=torch.float32, y=y)
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)
    b.gemm(dev(x), dev(ow), dev(osc), N, K, out_dtype=torch.float32, y=y)
    torch.cuda.synchronize()
    check_f32(f64(y), oracle.bin_gemm(oracle.bf16_to_f64(x), ow, osc, N, K), F32_TOL, "after injection")
