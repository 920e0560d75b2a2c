"""Helpers for the GPU parity tests: moving seeded numpy inputs to the device
and comparing device results with the fp64 oracle."""
import os
import sys

import numpy as np
import torch

import oracle


def dev(a: np.ndarray) -> torch.Tensor:
    """numpy -> CUDA tensor, keeping the bits: uint64 -> int64, uint16 (bf16 bits) -> bfloat16."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint64:
        return torch.from_numpy(a.view(np.int64)).cuda()
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def host_bits(t: torch.Tensor) -> np.ndarray:
    """CUDA tensor -> numpy with the raw bits (bf16/fp16 -> uint16, int64 -> uint64)."""
    t = t.detach().cpu()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.int64:
        return t.numpy().view(np.uint64)
    return t.numpy()


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def maxrel(g: np.ndarray, o: np.ndarray) -> float:
    """max_i |g_i - o_i| / max_i |o_i|: the largest error relative to the largest reference magnitude."""
    g = np.asarray(g, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    den = np.max(np.abs(o))
    return float(np.max(np.abs(g - o)) / den) if den > 0 else float(np.max(np.abs(g - o)))


def _ordered(bits: np.ndarray) -> np.ndarray:
    b = bits.astype(np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def bf16_ulps(g_bits: np.ndarray, o64: np.ndarray) -> np.ndarray:
    """Distance in bf16 ulps between device bf16 bits and RNE_bf16 of the fp64 reference."""
    ref = oracle.bf16_bits(oracle.round_bf16(o64))
    return np.abs(_ordered(np.asarray(g_bits, dtype=np.uint16)) - _ordered(ref))


#: the products' specified accuracy, as a per-element relative error
SPEC_TOL = 2e-3


def elemrel(g: np.ndarray, o: np.ndarray, floor: float = 1e-3) -> float:
    """max_i |g_i - o_i| / max(|o_i|, floor * rms(o)): the error of every element
    relative to its own reference value, with a floor of 1e-3 of the rms so that
    outputs at (or crossing) zero do not divide by nothing."""
    g = np.asarray(g, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    rms = float(np.sqrt(np.mean(o * o))) if o.size else 0.0
    if rms == 0.0:
        return 0.0 if np.array_equal(g, o) else float("inf")
    den = np.maximum(np.abs(o), floor * rms)
    return float(np.max(np.abs(g - o) / den))


def check_f32(g, o, tol, what="", elementwise=True):
    """fp32 outputs: max_i |g_i - o_i| / max_i |o_i| <= tol (the tight bar that
    one flipped sign or one dropped group fails) and, element by element,
    |g_i - o_i| / max(|o_i|, 1e-3 rms(o)) <= SPEC_TOL. `elementwise=False`
    only where the device and the oracle legitimately start from different
    inputs (an end-to-end chain whose intermediate is an output rounded on
    each side), which a per-element bar on the product does not describe."""
    e = maxrel(g, o)
    ee = elemrel(g, o)
    if os.environ.get("BRQ_REPORT_ERRORS"):
        print(f"[err] {what}: maxrel {e:.3e} elemrel {ee:.3e}", file=sys.stderr, flush=True)
    assert e <= tol, f"{what}: max rel error {e:.3e} > {tol:.1e}"
    if elementwise:
        assert ee <= SPEC_TOL, f"{what}: per-element rel error {ee:.3e} > {SPEC_TOL:.1e}"
    return e


def l2rel(g: np.ndarray, o: np.ndarray) -> float:
    g = np.asarray(g, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    return float(np.linalg.norm(g - o) / np.linalg.norm(o))


def bf16_close(g_bits: np.ndarray, o64: np.ndarray, atol_rel: float = 1e-5) -> np.ndarray:
    """Elementwise: within 1 bf16 ulp of RNE_bf16(oracle), or within
    atol_rel * max|o| of the oracle. The second arm covers outputs near zero,
    where fp32 accumulation error (~1e-7 of the largest output) spans many
    ulps of the tiny bf16 value."""
    ul = bf16_ulps(g_bits, o64)
    g = oracle.bf16_to_f64(g_bits)
    atol = atol_rel * float(np.max(np.abs(o64)))
    return (ul <= 1) | (np.abs(g - o64) <= atol)


def check_bf16(y: torch.Tensor, o64: np.ndarray, what="", tol=2e-3):
    """bf16 outputs: every element within 1 ulp of the oracle rounded to bf16
    (or, near zero, within 1e-5 of the largest output), and
    ||g - o||_2 / ||o||_2 <= tol. (bf16's own rounding reaches 2^-8 relative per
    element, so an elementwise or max-normalised 2e-3 bar cannot hold for a
    correctly rounded bf16 result.)"""
    assert y.dtype == torch.bfloat16
    g = host_bits(y)
    ok = bf16_close(g, o64)
    assert ok.all(), f"{what}: {int((~ok).sum())} elements off by more than 1 bf16 ulp"
    e = l2rel(f64(y), o64)
    assert e <= tol, f"{what}: l2 relative error {e:.3e} > {tol:.1e}"
    return e


def f16_ulps(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    return np.abs(_ordered(np.asarray(a).view(np.uint16)) - _ordered(np.asarray(b).view(np.uint16)))
