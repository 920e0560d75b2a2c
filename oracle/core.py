"""fp64 reference implementations (test infrastructure only; see package docstring)."""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "GROUP", "bf16_to_f64", "f16_to_f64", "round_bf16", "bf16_bits",
    "sign_bits", "pack_words", "unpack_signs", "group_mean_abs", "pack_sign1", "pack_sign1_only",
    "dequantize", "bin_gemm", "bin_gemm_cols", "bin_gemm_loops", "bin_gemm_lr", "bin_gemm_lr_cols", "bin_gemm_lr_dense",
    "dbf_chain", "dbf_dense", "dbf_bpe", "dbf_bits", "q8_rows", "dbf_chain_q8",
    "route_topk", "silu", "moe_ffn", "moe_ffn_loops", "moe_dbf_ffn", "moe_dbf_dense",
    "kron_rotate", "kron_rotate_bf16",
    "packed_bytes", "bits_per_weight",
]

#: weights per scale group along the reduction axis: one fp16 scale per 128 signs
#: ("Behaviour-Relearned Quantization", item 02)
GROUP = 128

PINS = {
    "pack_sign1": "closed form + brute-force scale search + brute-force sign search + round trip + Gaussian error law",
    "pack_sign1_only": "bit convention + round trip",
    "bin_gemm": "one-hot / all-plus / all-minus closed forms + definitional loops + linearity",
    "bin_gemm_lr": "dense materialisation of Wq + U.V + zero-factor reduction + one-hot rank-1 closed form",
    "dbf_chain": "dense reconstruction + Sylvester-Hadamard identity",
    "dbf_bpe": "worked example of the DBF post, section 1.1",
    "q8_rows": "rounding bound + minimal exponent + exact codes for representable rows + zero row",
    "dbf_chain_q8": "Sylvester-Hadamard closed form + odd symmetry + power-of-two equivariance + distance to the unquantised chain"
                    " + a hand-built row whose codes differ unless h_s is rounded once to fp32",
    "silu": "logistic identities: silu(0) = 0, silu(z) - silu(-z) = z, silu(ln 3) = (3/4) ln 3, slope 1/2 at 0, limits",
    "route_topk": "brute-force ordering + softmax invariants",
    "moe_ffn": "identical-experts reduction + single-route dense FFN + loops",
    "moe_dbf_ffn": "dense reconstruction of every chain + identical-experts reduction + single route",
    "kron_rotate": "numpy.kron identity + orthogonality invariants",
}


# ---------------------------------------------------------------------------
# number formats
# ---------------------------------------------------------------------------

def bf16_to_f64(bits) -> np.ndarray:
    """Exact fp64 value of bf16 bit patterns (uint16)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f16_to_f64(h) -> np.ndarray:
    return np.asarray(h, dtype=np.float16).astype(np.float64)


def round_bf16(v) -> np.ndarray:
    """Round fp64 values to the nearest bf16 value (ties to even), returned as fp64.

    bf16 keeps 8 significant bits and fp32's exponent range. Written with
    frexp/rint so the rounding is taken once, directly from fp64."""
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)                       # v = m * 2**e, 0.5 <= |m| < 1
    # below the smallest normal bf16 (2**-126) the grid spacing stays 2**-133
    e_eff = np.maximum(e, -125)
    q = np.rint(np.ldexp(m, e - e_eff + 8))  # significand scaled to an integer grid
    out = np.ldexp(q, e_eff - 8)
    out = np.where(np.abs(out) >= 2.0 ** 128, np.copysign(np.inf, v), out)
    return np.where(np.isfinite(v), out, v)


def bf16_bits(v) -> np.ndarray:
    """bf16 bits of fp64 values that are already exactly representable in bf16."""
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# ---------------------------------------------------------------------------
# S1: sign planes and group-128 scales
# ---------------------------------------------------------------------------

def sign_bits(w) -> np.ndarray:
    """Bit per weight: the IEEE sign bit, so +x -> 0 (+1) and -x -> 1 (-1).

    "LLM binarization, Episode 01: DBF", section 1: 0 means +1, 1 means -1,
    following the sign-bit convention of IEEE 754."""
    return np.signbit(np.asarray(w, dtype=np.float32))


def pack_words(bits) -> np.ndarray:
    """Pack a boolean [rows, cols] plane into uint64 words, 64 signs per word
    (DBF post, section 3). Element k of a row is bit (k % 64) of word (k // 64):
    least-significant bit first."""
    bits = np.asarray(bits, dtype=bool)
    rows, cols = bits.shape
    assert cols % 64 == 0, "a SIGN1 row holds whole 64-sign words"
    b = bits.reshape(rows, cols // 64, 64).astype(np.uint64)
    shifts = np.arange(64, dtype=np.uint64)
    return np.bitwise_or.reduce(b << shifts, axis=2).astype(np.uint64)


def unpack_signs(words, rows: int, cols: int) -> np.ndarray:
    """+-1.0 fp64 matrix [rows, cols] from packed words (inverse of pack_words)."""
    w = np.asarray(words, dtype=np.uint64).reshape(rows, cols // 64, 1)
    bits = (w >> np.arange(64, dtype=np.uint64)) & np.uint64(1)
    return 1.0 - 2.0 * bits.reshape(rows, cols).astype(np.float64)


def group_mean_abs(w, group: int = GROUP) -> np.ndarray:
    """mean |w| over each run of ``group`` consecutive weights of a row, in fp64.

    For fixed signs s the best scale a of ||w - a s||^2 is sum(w s)/G; with
    s = sign(w) that is mean|w|, and that choice of s maximises sum(w s), so the
    pair (mean|w|, sign(w)) is the joint least-squares optimum."""
    w = np.asarray(w, dtype=np.float32).astype(np.float64)
    rows, cols = w.shape
    assert cols % group == 0
    return np.abs(w).reshape(rows, cols // group, group).mean(axis=2)


def pack_sign1(w, group: int = GROUP):
    """Quantise fp32 weights [N, K] to group-128 sign bits plus one fp16 scale per
    group ("Behaviour-Relearned Quantization", item 02; "Banyan", Abstract).

    Returns (words uint64 [N, K/64], scales float16 [N, K/group]). The scale is
    mean|w| of the group rounded once from fp64 to fp16 (nearest, ties to even)."""
    w = np.asarray(w, dtype=np.float32)
    words = pack_words(sign_bits(w))
    scales = group_mean_abs(w, group).astype(np.float16)
    return words, scales


def pack_sign1_only(w):
    """SIGN1 plane without scales (the DBF factors U and V carry no group scale)."""
    return pack_words(sign_bits(w))


def dequantize(words, scales, N: int, K: int, group: int = GROUP) -> np.ndarray:
    """W_q[n, k] = (+1 or -1) * scale[n, k // group], fp64."""
    s = unpack_signs(words, N, K)
    return s * np.repeat(f16_to_f64(scales).reshape(N, K // group), group, axis=1)


def packed_bytes(N: int, K: int, group: int = GROUP) -> int:
    """Bytes of the packed form: N*K/8 sign bytes plus 2 bytes per group."""
    return N * K // 8 + 2 * (N * K // group)


def bits_per_weight(group: int = GROUP, scale_bits: int = 16) -> float:
    return 1.0 + scale_bits / group


# ---------------------------------------------------------------------------
# S2 / S3: activation x binary-weight product
# ---------------------------------------------------------------------------

def bin_gemm(x, words, scales, N: int, K: int) -> np.ndarray:
    """y[m, n] = sum_k x[m, k] * W_q[n, k] in fp64 (y = x . W_q^T)."""
    x = np.asarray(x, dtype=np.float64)
    return x @ dequantize(words, scales, N, K).T


def bin_gemm_cols(x, words, scales, N: int, K: int, cols) -> np.ndarray:
    """Only the output columns ``cols`` of bin_gemm (for sampled checks at full size)."""
    cols = np.asarray(cols)
    kw = K // 64
    kg = K // GROUP
    w = np.asarray(words, dtype=np.uint64).reshape(N, kw)[cols]
    s = np.asarray(scales).reshape(N, kg)[cols]
    return np.asarray(x, dtype=np.float64) @ dequantize(w, s, len(cols), K).T


def bin_gemm_loops(x, words, scales, N: int, K: int) -> np.ndarray:
    """Definitional tier: y[m, n] = sum_g scale[n, g] * sum_{k in g} (+-x[m, k]),
    every sum taken exactly with math.fsum. Tiny shapes only."""
    x = np.asarray(x, dtype=np.float64)
    M = x.shape[0]
    words = np.asarray(words, dtype=np.uint64).reshape(N, K // 64)
    sc = f16_to_f64(scales).reshape(N, K // GROUP)
    y = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            parts = []
            for g in range(K // GROUP):
                terms = []
                for k in range(g * GROUP, (g + 1) * GROUP):
                    bit = (int(words[n, k // 64]) >> (k % 64)) & 1
                    terms.append(-x[m, k] if bit else x[m, k])
                parts.append(sc[n, g] * math.fsum(terms))
            y[m, n] = math.fsum(parts)
    return y


# ---------------------------------------------------------------------------
# Binary product plus a low-rank correction ("BWLA" commentary, section 4:
# the residual that the binarised weights leave is approximated by a truncated
# SVD, a rank-r matrix added to the binarised weights as a correction term)
# ---------------------------------------------------------------------------

def bin_gemm_lr(x, words, scales, v, u, N: int, K: int, r: int) -> np.ndarray:
    """y = x . (W_q + U V)^T = x . W_q^T + (x . V^T) . U^T in fp64, with the
    correction in factored form: V is r x K, U is N x r, both fp16 arrays
    (like the group scales). The factored order is how the correction is applied at inference
    (r dot products per row, then r products per output)."""
    x = np.asarray(x, dtype=np.float64)
    V = f16_to_f64(v).reshape(r, K)
    U = f16_to_f64(u).reshape(N, r)
    t = x @ V.T
    return bin_gemm(x, words, scales, N, K) + t @ U.T


def bin_gemm_lr_cols(x, words, scales, v, u, N: int, K: int, r: int, cols) -> np.ndarray:
    """Only the output columns ``cols`` of bin_gemm_lr (for sampled checks at full size)."""
    cols = np.asarray(cols)
    x = np.asarray(x, dtype=np.float64)
    t = x @ f16_to_f64(v).reshape(r, K).T
    return bin_gemm_cols(x, words, scales, N, K, cols) + t @ f16_to_f64(u).reshape(N, r)[cols].T


def bin_gemm_lr_dense(x, words, scales, v, u, N: int, K: int, r: int) -> np.ndarray:
    """The same product through the materialised corrected matrix W_q + U V
    (N x K, fp64): the definition the factored form must equal."""
    x = np.asarray(x, dtype=np.float64)
    W = dequantize(words, scales, N, K) + f16_to_f64(u).reshape(N, r) @ f16_to_f64(v).reshape(r, K)
    return x @ W.T


# ---------------------------------------------------------------------------
# S4: Double Binary Factorization chain
# ---------------------------------------------------------------------------

def dbf_chain(x, d_in, v_words, d_mid, u_words, d_out, m: int, n: int, r: int) -> np.ndarray:
    """y = D_out . U . D_mid . V . D_in . x for every row of x, evaluated in the
    deployed order of the DBF post, section 4:
    x_s = D_in x; h = V x_s; h_s = D_mid h; y_core = U h_s; y = D_out y_core.
    V is r x n and U is m x r, both +-1 (section 1)."""
    x = np.asarray(x, dtype=np.float64)
    V = unpack_signs(v_words, r, n)
    U = unpack_signs(u_words, m, r)
    xs = x * f16_to_f64(d_in)[None, :]
    h = xs @ V.T
    hs = h * f16_to_f64(d_mid)[None, :]
    yc = hs @ U.T
    return yc * f16_to_f64(d_out)[None, :]


def q8_rows(v) -> tuple:
    """Sign-magnitude Q8 activations with one exponent per reduction row (DBF
    post, section 5, item 4: the row is denormalised to a shared exponent and
    encoded as a sign plane and seven magnitude planes). Reading: the exponent
    e of a row is the smallest integer with max|v| <= 127 * 2^e and
    q = round-half-even(v / 2^e), so |q| <= 127; an all-zero row takes e = 0.
    Returns (q int64 [rows, n], e int64 [rows])."""
    v = np.asarray(v, dtype=np.float64)
    v2 = v.reshape(-1, v.shape[-1])
    e = np.zeros(v2.shape[0], dtype=np.int64)
    for i, m in enumerate(np.abs(v2).max(axis=1)):
        if m == 0.0:
            continue
        k = int(np.floor(np.log2(m)))  # refined below against the exact bounds
        k -= 6
        while m > 127.0 * 2.0 ** k:
            k += 1
        while m <= 127.0 * 2.0 ** (k - 1):
            k -= 1
        e[i] = k
    q = np.rint(v2 / np.exp2(e.astype(np.float64))[:, None])
    return q.astype(np.int64).reshape(v.shape), e


def dbf_chain_q8(x, d_in, v_words, d_mid, u_words, d_out, m: int, n: int, r: int) -> np.ndarray:
    """The DBF chain of dbf_chain with both binary products taken over Q8
    activations (the prompt-processing formulation of the DBF post, section
    5, item 4: row-denormalised sign-magnitude activations, an exact integer
    reduction of signs times magnitudes, then one shared scale):
    x_s = D_in x -> (q1, e1) = q8_rows(x_s); h = 2^e1 (V q1);
    h_s = fp32(D_mid h) -> (q2, e2) = q8_rows(h_s); y = D_out 2^e2 (U q2).
    The quantised codes are integer decisions taken on floating-point values,
    so they follow the precision the products run in: x_s = d_in x is exact
    in fp32 and fp64 alike, and h_s is rounded once to fp32 (as the products'
    epilogue does) before it is quantised."""
    x = np.asarray(x, dtype=np.float64)
    V = unpack_signs(v_words, r, n).astype(np.int64)
    U = unpack_signs(u_words, m, r).astype(np.int64)
    xs = x * f16_to_f64(d_in)[None, :]
    q1, e1 = q8_rows(xs)
    h = (q1 @ V.T).astype(np.float64) * np.exp2(e1.astype(np.float64))[:, None]
    hs = (np.asarray(d_mid, dtype=np.float16).astype(np.float32)[None, :] * h.astype(np.float32)).astype(np.float64)
    q2, e2 = q8_rows(hs)
    yc = (q2 @ U.T).astype(np.float64) * np.exp2(e2.astype(np.float64))[:, None]
    return yc * f16_to_f64(d_out)[None, :]


def dbf_dense(d_in, v_words, d_mid, u_words, d_out, m: int, n: int, r: int) -> np.ndarray:
    """The reconstructed dense matrix D_out U D_mid V D_in (m x n), fp64."""
    V = unpack_signs(v_words, r, n)
    U = unpack_signs(u_words, m, r)
    return (f16_to_f64(d_out)[:, None] * U * f16_to_f64(d_mid)[None, :]) @ (V * f16_to_f64(d_in)[None, :])


def dbf_bits(m: int, n: int, r: int, diag_bits: int = 16) -> int:
    """Storage of one DBF projection: r*n + m*r sign bits plus three fp16 diagonals
    (DBF post, section 1.1)."""
    return r * (m + n) + diag_bits * (m + n + r)


def dbf_bpe(m: int, n: int, r: int) -> float:
    return dbf_bits(m, n, r) / (m * n)


# ---------------------------------------------------------------------------
# S5 / S6: routed mixture of experts
# ---------------------------------------------------------------------------

def route_topk(logits, k: int):
    """Top-k experts per token by descending fp32 logit, ties to the lower expert
    index; route weights are the softmax of the k selected logits (equal to the
    full softmax renormalised over the selected experts). Each (token, slot)
    carries an expert id and a weight (DBF post, section 4)."""
    lg = np.asarray(logits, dtype=np.float32)
    T, E = lg.shape
    ids = np.zeros((T, k), dtype=np.int64)
    for t in range(T):
        # stable sort on the negated values: equal logits keep ascending index order
        order = np.argsort(-lg[t].astype(np.float64), kind="stable")
        ids[t] = order[:k]
    sel = np.take_along_axis(lg.astype(np.float64), ids, axis=1)
    e = np.exp(sel - sel.max(axis=1, keepdims=True))
    return ids, e / e.sum(axis=1, keepdims=True)


def silu(z):
    """z * sigmoid(z) = z / (1 + e^-z); for z below about -709 e^-z overflows to
    inf and the quotient is the limit -0 (no warning raised for it)."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def moe_ffn(x, logits, expert, H: int, I: int, k: int):
    """y_t = sum_j w_tj * Wd_e (silu(Wg_e x_t) * (Wu_e x_t)), e = id_tj.

    ``expert(e)`` returns the packed (gate_words, gate_scales, up_words,
    up_scales, down_words, down_scales) of expert e. Gate and up are [I, H],
    down is [H, I]. Returns (y fp64 [T, H], ids, weights)."""
    x = np.asarray(x, dtype=np.float64)
    T = x.shape[0]
    ids, wts = route_topk(logits, k)
    y = np.zeros((T, H))
    cache = {}
    for t in range(T):
        for j in range(k):
            e = int(ids[t, j])
            if e not in cache:
                gw, gs, uw, us, dw, ds = expert(e)
                cache[e] = (dequantize(gw, gs, I, H), dequantize(uw, us, I, H), dequantize(dw, ds, H, I))
            Wg, Wu, Wd = cache[e]
            a = silu(Wg @ x[t]) * (Wu @ x[t])
            y[t] += wts[t, j] * (Wd @ a)
    return y, ids, wts


def moe_ffn_loops(x, logits, expert, H: int, I: int, k: int):
    """Definitional tier of moe_ffn for tiny shapes: every product through
    bin_gemm_loops and every sum through math.fsum."""
    x = np.asarray(x, dtype=np.float64)
    T = x.shape[0]
    ids, wts = route_topk(logits, k)
    y = np.zeros((T, H))
    for t in range(T):
        outs = []
        for j in range(k):
            gw, gs, uw, us, dw, ds = expert(int(ids[t, j]))
            g = bin_gemm_loops(x[t:t + 1], gw, gs, I, H)[0]
            u = bin_gemm_loops(x[t:t + 1], uw, us, I, H)[0]
            a = np.array([gi / (1.0 + math.exp(-gi)) * ui for gi, ui in zip(g, u)])
            outs.append(wts[t, j] * bin_gemm_loops(a[None, :], dw, ds, H, I)[0])
        for h in range(H):
            y[t, h] = math.fsum(o[h] for o in outs)
    return y, ids, wts


def moe_dbf_ffn(x, logits, expert, H: int, I: int, r: int, k: int, tokens=None):
    """The routed SwiGLU layer with DBF experts (the DBF post's deployed model:
    every routed gate, up and down projection is a D_in V D_mid U D_out chain,
    section 4, evaluated in the deployed order by dbf_chain):
    y_t = sum_j w_tj * down_e(silu(gate_e(x_t)) * up_e(x_t)), e = id_tj.

    ``expert(e)`` returns three records (gate, up, down), each a tuple
    (d_in, v_words, d_mid, u_words, d_out); gate and up map H -> I, down
    I -> H. ``tokens`` restricts the evaluation to those rows (sampled checks).
    Returns (y fp64 [T, H] (zero rows outside ``tokens``), ids, weights)."""
    x = np.asarray(x, dtype=np.float64)
    T = x.shape[0]
    ids, wts = route_topk(logits, k)
    y = np.zeros((T, H))
    cache = {}
    for t in (range(T) if tokens is None else tokens):
        for j in range(k):
            e = int(ids[t, j])
            if e not in cache:
                cache[e] = expert(e)
            g, u, d = cache[e]
            xt = x[t:t + 1]
            a = silu(dbf_chain(xt, *g, I, H, r)) * dbf_chain(xt, *u, I, H, r)
            y[t] += wts[t, j] * dbf_chain(a, *d, H, I, r)[0]
    return y, ids, wts


def moe_dbf_dense(x, logits, expert, H: int, I: int, r: int, k: int):
    """The same layer through the dense reconstructions D_out U D_mid V D_in of
    every chain (dbf_dense) and a plain dense SwiGLU."""
    x = np.asarray(x, dtype=np.float64)
    T = x.shape[0]
    ids, wts = route_topk(logits, k)
    y = np.zeros((T, H))
    for t in range(T):
        for j in range(k):
            g, u, d = expert(int(ids[t, j]))
            Wg, Wu, Wd = dbf_dense(*g, I, H, r), dbf_dense(*u, I, H, r), dbf_dense(*d, H, I, r)
            y[t] += wts[t, j] * (Wd @ (silu(Wg @ x[t]) * (Wu @ x[t])))
    return y, ids, wts


# ---------------------------------------------------------------------------
# S7: Kronecker-factored orthogonal activation rotation
# ---------------------------------------------------------------------------

def kron_rotate(x, H, R) -> np.ndarray:
    """x' = (H (x) R) x per token, computed as X' = H X R^T with X the token
    reshaped row-major to [n1, n2] (BWLA commentary, sections 3 and 5). fp64."""
    x = np.asarray(x, dtype=np.float64)
    H = np.asarray(H, dtype=np.float64)
    R = np.asarray(R, dtype=np.float64)
    n1, n2 = H.shape[0], R.shape[0]
    M = x.shape[0]
    X = x.reshape(M, n1, n2)
    return np.matmul(np.matmul(H[None], X), R.T[None]).reshape(M, n1 * n2)


def kron_rotate_bf16(x, H, R) -> np.ndarray:
    """kron_rotate followed by the bf16 rounding of the library's output."""
    return round_bf16(kron_rotate(x, H, R))
