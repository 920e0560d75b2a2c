"""Seeded synthetic inputs for the binary-weight products.

This module is shared by the oracle's tests, the GPU parity tests and the
benchmark. It holds random draws and the dtype rounding of those draws, and
nothing of the method's own arithmetic (no packing, no products, no routing).

Every tensor is drawn from ``numpy.random.default_rng(SeedSequence(key))``
with ``key`` a short list of small integers ``[config, tensor, sub...]``, so the
same key always gives the same bytes on any machine.

Shapes and distributions follow the workloads of the pages:
* LLM-style weights: fp32 ~ N(0, 0.02^2);
* activations: bf16, rounded to nearest-even from fp32 ~ N(0, 1);
* DBF diagonals: fp16 of exp(N(0, 0.5^2)) (log-normal), DBF signs uniform +-1;
* router logits: fp32 ~ N(0, 1);
* Kronecker factors: Haar-random orthogonal 64x64 from a QR decomposition.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "rng", "normal_f32", "bf16_bits_from_f32", "bf16_bits_to_f32", "bf16_normal",
    "f16_lognormal", "pm1_f32", "haar_orthogonal", "router_logits",
    "C1", "C2_SHAPES", "C2_MS", "C3", "C4", "C5",
]


def rng(*key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(k) for k in key]))


def normal_f32(key, shape, std: float = 1.0) -> np.ndarray:
    g = rng(*key)
    a = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even) and return the raw uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_normal(key, shape, std: float = 1.0) -> np.ndarray:
    """bf16 bits of N(0, std^2) draws."""
    return bf16_bits_from_f32(normal_f32(key, shape, std))


def f16_lognormal(key, shape, sigma: float = 0.5) -> np.ndarray:
    g = rng(*key)
    return np.exp(g.standard_normal(size=shape) * sigma).astype(np.float16)


def pm1_f32(key, shape) -> np.ndarray:
    g = rng(*key)
    return np.where(g.integers(0, 2, size=shape, dtype=np.int8) == 0, 1.0, -1.0).astype(np.float32)


def sign_words(key, rows: int, cols: int) -> np.ndarray:
    """Uniform random signs of a rows x cols matrix as SIGN1 words (uint64
    [rows * cols / 64], 64 signs per word): every bit an independent fair coin."""
    g = rng(*key)
    return g.integers(0, 2 ** 63, size=rows * cols // 64, dtype=np.int64).view(np.uint64) ^ \
        (g.integers(0, 2, size=rows * cols // 64, dtype=np.int64).view(np.uint64) << np.uint64(63))


def haar_orthogonal(key, n: int) -> np.ndarray:
    """Haar-distributed n x n orthogonal matrix (fp64): QR of a Gaussian matrix,
    with the columns' signs fixed by the signs of R's diagonal."""
    g = rng(*key)
    a = g.standard_normal(size=(n, n))
    q, r = np.linalg.qr(a)
    return q * np.sign(np.diag(r))[None, :]


def router_logits(key, T: int, E: int) -> np.ndarray:
    return normal_f32(key, (T, E), 1.0)


# ---------------------------------------------------------------------------
# The five workloads. Each builder returns plain numpy arrays: fp32 weights
# (to be packed), bf16 activations as uint16 bits, fp16 diagonals, fp32 logits.
# ---------------------------------------------------------------------------

def C1():
    """Single binary GEMV: W 1024x1024 fp32 ~N(0, 0.02^2), x 1x1024 bf16 ~N(0,1)."""
    w = normal_f32((1, 0), (1024, 1024), 0.02)
    x = bf16_normal((1, 1), (1, 1024))
    return w, x


#: the named MoE geometries (experts, hidden, expert intermediate) with the
#: DBF rank used for them here: r = 2048, the most the layer accepts
MOE_GEOMETRIES = {
    "GLM-4.5-Air": dict(E=128, H=4096, I=1408, r=2048),
    "MiniMax-M2.5": dict(E=256, H=3072, I=1536, r=2048),
    "DeepSeek-V4-Flash": dict(E=256, H=4096, I=2048, r=2048),
}

#: the widest named geometry (hidden 6144 x expert intermediate 2048, 256
#: experts), kept apart so that the table above keeps its seeds
MOE_GEOMETRY_WIDE = {"GLM-5.2": dict(E=256, H=6144, I=2048, r=2048)}

#: decode-shaped matrices, stored [N_out, K_in]
C2_SHAPES = ((4096, 14336), (14336, 4096))
C2_MS = (1, 4, 16, 64)


def C2_weight(which: int) -> np.ndarray:
    N, K = C2_SHAPES[which]
    return normal_f32((2, which), (N, K), 0.02)


def C2_x(which: int, M: int) -> np.ndarray:
    N, K = C2_SHAPES[which]
    return bf16_normal((2, 2, which, M), (M, K))


def C3(M: int, m: int = 4096, n: int = 4096, r: int = 2048):
    """DBF chain: U (m x r) and V (r x n) uniform +-1, three fp16 log-normal(0, 0.5)
    diagonals, x bf16 [M, n] ~N(0,1)."""
    v = pm1_f32((3, 0, r), (r, n))
    u = pm1_f32((3, 1, r), (m, r))
    d_in = f16_lognormal((3, 2, n), (n,))
    d_mid = f16_lognormal((3, 3, r), (r,))
    d_out = f16_lognormal((3, 4, m), (m,))
    x = bf16_normal((3, 5, M), (M, n))
    return dict(x=x, v=v, u=u, d_in=d_in, d_mid=d_mid, d_out=d_out, m=m, n=n, r=r)


class C4:
    """Routed MoE layer: E experts, hidden H, expert intermediate I, top-k routing.
    Expert weights are drawn lazily per (expert, projection) so a test can build
    only the experts it needs."""

    def __init__(self, E: int = 256, H: int = 2048, I: int = 512, top_k: int = 8, layer: int = 0):
        self.E, self.H, self.I, self.top_k, self.layer = E, H, I, top_k, layer

    def gate(self, e):
        return normal_f32((4, 0, self.layer, e, 0), (self.I, self.H), 0.02)

    def up(self, e):
        return normal_f32((4, 0, self.layer, e, 1), (self.I, self.H), 0.02)

    def down(self, e):
        return normal_f32((4, 0, self.layer, e, 2), (self.H, self.I), 0.02)

    def x(self, T):
        return bf16_normal((4, 2, T), (T, self.H))

    def logits(self, T, it: int = 0):
        return router_logits((4, 1, T, it), T, self.E)


class C4D:
    """Routed MoE layer whose experts are DBF chains (the deployed workload of
    the DBF post: gate/up 512x2048 and down 2048x512 per expert, r = 1024).
    Per (expert, projection): V r x n and U m x r uniform +-1, d_in and d_out
    fp16 log-normal(0, 0.5), d_mid fp16 log-normal(0, 0.5) * 2^-12 so that the
    reconstructed matrix has the spread of a trained projection (about 0.017)
    and every intermediate stays well inside fp16. Drawn lazily per expert."""

    def __init__(self, E: int = 256, H: int = 2048, I: int = 512, r: int = 1024, top_k: int = 8, layer: int = 0):
        self.E, self.H, self.I, self.r, self.top_k, self.layer = E, H, I, r, top_k, layer

    def proj(self, e: int, p: int):
        """p = 0 gate, 1 up (m = I, n = H), 2 down (m = H, n = I)."""
        m, n = (self.I, self.H) if p < 2 else (self.H, self.I)
        key = (6, self.layer, e, p)
        d_mid = (np.exp(rng(*key, 3).standard_normal(size=(self.r,)) * 0.5) * 2.0 ** -12).astype(np.float16)
        return dict(v=pm1_f32(key + (0,), (self.r, n)), u=pm1_f32(key + (1,), (m, self.r)),
                    d_in=f16_lognormal(key + (2,), (n,)), d_mid=d_mid, d_out=f16_lognormal(key + (4,), (m,)),
                    m=m, n=n)

    def proj_packed(self, e: int, p: int):
        """As proj, with V and U drawn directly as SIGN1 words (uniform random
        bits are uniform +-1 signs): the layer's named geometries have factors
        too large to draw as fp32 and pack on the host per test."""
        m, n = (self.I, self.H) if p < 2 else (self.H, self.I)
        key = (6, self.layer, e, p)
        d_mid = (np.exp(rng(*key, 3).standard_normal(size=(self.r,)) * 0.5) * 2.0 ** -12).astype(np.float16)
        return dict(v=sign_words((7,) + key + (0,), self.r, n), u=sign_words((7,) + key + (1,), m, self.r),
                    d_in=f16_lognormal(key + (2,), (n,)), d_mid=d_mid, d_out=f16_lognormal(key + (4,), (m,)),
                    m=m, n=n)

    def x(self, T):
        return bf16_normal((6, 100, T), (T, self.H))

    def logits(self, T, it: int = 0):
        return router_logits((6, 101, T, it), T, self.E)


def C5(M: int = 4096, K: int = 4096, N: int = 14336, n1: int = 64, n2: int = 64):
    """Prefill with a Kronecker rotation: x bf16 [M, K] ~N(0,1); H (n1 x n1) and
    R (n2 x n2) Haar orthogonal, handed to both sides as fp32; W fp32 [N, K]
    ~N(0, 0.02^2)."""
    H = haar_orthogonal((5, 0, n1), n1).astype(np.float32)
    R = haar_orthogonal((5, 1, n2), n2).astype(np.float32)
    x = bf16_normal((5, 3, M, K), (M, K))
    return dict(x=x, H=H, R=R, N=N, K=K)


def C5_weight(N: int = 14336, K: int = 4096) -> np.ndarray:
    return normal_f32((5, 2), (N, K), 0.02)
