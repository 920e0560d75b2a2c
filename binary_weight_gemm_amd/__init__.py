"""brq -- matrix products against binarized LLM weights on AMD MI355X (gfx950).

A thin ctypes binding over ``libbrq.so``: it checks that tensors live on the
GPU with the dtype and shape each call expects, allocates outputs and
workspaces with torch, and passes raw pointers plus torch's current stream to
the C ABI declared in ``include/brq.h``. Every step of every product runs in
the library's HIP kernels; there is no fallback path. If the library is not
built, every call raises.

Tensor conventions (torch dtypes carrying the ABI's formats):
  sign planes   torch.int64 [rows, cols/64]   (uint64 words, same bits)
  scales        torch.float16 [rows, cols/128]
  activations   torch.bfloat16
  DBF diagonals torch.float16
  router logits torch.float32
  outputs       torch.bfloat16 or torch.float32
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "BrqError", "lib", "library_path", "pack", "gemm", "gemm_lr", "dbf_gemm", "dbf_gemm_q8", "moe_ffn", "moe_dbf_ffn",
    "kron_rotate", "DbfFactors", "moe_dbf_workspace_bytes",
    "gemm_workspace_bytes", "gemm_lr_workspace_bytes", "dbf_workspace_bytes", "dbf_q8_workspace_bytes",
    "moe_workspace_bytes",
    "sign_words", "scale_count",
    "BRQ_BF16", "BRQ_F32", "ABI_FUNCTIONS", "set_decode_fusion", "FUSION_DEFAULT", "FUSION_OFF", "FUSION_ON",
]

BRQ_BF16 = 0
BRQ_F32 = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

from .abi_table import ABI_FUNCTIONS  # noqa: E402  (every function of include/brq.h)

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_sz = ctypes.c_size_t
_int = ctypes.c_int


class DbfFactors(ctypes.Structure):
    """brq_dbf_factors: device pointers of one DBF chain record (all experts)."""
    _fields_ = [("d_in", _vp), ("v", _vp), ("d_mid", _vp), ("u", _vp), ("d_out", _vp)]


class BrqError(RuntimeError):
    pass


def library_path() -> str:
    return os.path.join(_HERE, "libbrq.so")


def lib():
    """Load libbrq.so (built in-tree by ``python -m binary_weight_gemm_amd.build``)."""
    global _LIB
    if _LIB is None:
        path = library_path()
        if not os.path.exists(path):
            raise BrqError(f"{path} is not built; run `python -m binary_weight_gemm_amd.build`")
        L = ctypes.CDLL(path)
        for name, (res, args) in ABI_FUNCTIONS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _LIB = L
    return _LIB


def _check(status: int, what: str):
    if status != 0:
        L = lib()
        raise BrqError(f"{what}: {L.brq_status_str(status).decode()}: {L.brq_last_error().decode()}")


def _dev(t: torch.Tensor, name: str, dtype=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise BrqError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise BrqError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise BrqError(f"{name} must be {dtype}, got {t.dtype}")
    return _vp(t.data_ptr())


def _stream():
    return _vp(torch.cuda.current_stream().cuda_stream)


def _out_code(dtype) -> int:
    if dtype == torch.bfloat16:
        return BRQ_BF16
    if dtype == torch.float32:
        return BRQ_F32
    raise BrqError(f"output dtype must be torch.bfloat16 or torch.float32, got {dtype}")


def _ws(nbytes: int, device, ws):
    if nbytes == 0:
        return None, 0
    if ws is None:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    if ws.numel() * ws.element_size() < nbytes:
        raise BrqError(f"workspace of {ws.numel() * ws.element_size()} bytes, {nbytes} needed")
    return ws, nbytes


FUSION_DEFAULT, FUSION_OFF, FUSION_ON = 0, 1, 2


def set_decode_fusion(mode: int, spin_limit: int = 0) -> None:
    """brq_set_decode_fusion: single-launch decode chains (DBF at M <= 8, MoE at
    T <= 4): FUSION_DEFAULT (the library's per-path choice), FUSION_OFF or
    FUSION_ON; spin_limit bounds the grid-wide wait (0: default)."""
    _check(lib().brq_set_decode_fusion(int(mode), int(spin_limit)), "brq_set_decode_fusion")


def sign_words(rows: int, cols: int) -> int:
    return lib().brq_sign_words(rows, cols)


def scale_count(rows: int, cols: int) -> int:
    return lib().brq_scale_count(rows, cols)


def gemm_workspace_bytes(M: int, N: int, K: int) -> int:
    return lib().brq_gemm_workspace_bytes(M, N, K)


def dbf_workspace_bytes(M: int, m: int, n: int, r: int) -> int:
    return lib().brq_dbf_workspace_bytes(M, m, n, r)


def dbf_q8_workspace_bytes(M: int, m: int, n: int, r: int) -> int:
    return lib().brq_dbf_q8_workspace_bytes(M, m, n, r)


def moe_workspace_bytes(T: int, H: int, I: int, E: int, top_k: int) -> int:
    return lib().brq_moe_workspace_bytes(T, H, I, E, top_k)


def pack(w: torch.Tensor, scales: bool = True, out=None):
    """brq_pack: fp32 [rows, cols] -> (signs int64 [rows, cols/64], scales fp16 [rows, cols/128] or None)."""
    if w.dim() != 2:
        raise BrqError("w must be 2-D")
    rows, cols = w.shape
    if out is None:
        s = torch.empty((rows, max(cols // 64, 0)), dtype=torch.int64, device=w.device)
        sc = torch.empty((rows, max(cols // 128, 0)), dtype=torch.float16, device=w.device) if scales else None
    else:
        s, sc = out
    _check(lib().brq_pack(_dev(w, "w", torch.float32), rows, cols, _dev(s, "signs", torch.int64),
                          _dev(sc, "scales", torch.float16) if sc is not None else None, _stream()), "brq_pack")
    return s, sc


def gemm(x: torch.Tensor, signs: torch.Tensor, scales: torch.Tensor, N: int, K: int,
         out_dtype=torch.bfloat16, y=None, ws=None) -> torch.Tensor:
    """brq_gemm: y[M, N] = x[M, K] . Wq^T for the group-128 matrix (signs, scales)."""
    M = x.shape[0]
    if x.dim() != 2 or x.shape[1] != K:
        raise BrqError(f"x must be [M, {K}]")
    if signs.numel() != N * K // 64 or scales.numel() != N * K // 128:
        raise BrqError("signs/scales do not match N x K")
    code = _out_code(out_dtype)
    if y is None:
        y = torch.empty((M, N), dtype=out_dtype, device=x.device)
    ws, wsb = _ws(gemm_workspace_bytes(M, N, K), x.device, ws)
    _check(lib().brq_gemm(_dev(x, "x", torch.bfloat16), M, N, K, _dev(signs, "signs", torch.int64),
                          _dev(scales, "scales", torch.float16), _dev(y, "y", out_dtype), code,
                          _dev(ws, "ws") if ws is not None else None, wsb, _stream()), "brq_gemm")
    return y


def gemm_lr_workspace_bytes(M: int, N: int, K: int, r: int) -> int:
    return lib().brq_gemm_lr_workspace_bytes(M, N, K, r)


def gemm_lr(x: torch.Tensor, signs: torch.Tensor, scales: torch.Tensor, v: torch.Tensor, u: torch.Tensor,
            N: int, K: int, r: int, out_dtype=torch.bfloat16, y=None, ws=None) -> torch.Tensor:
    """brq_gemm_lr: y[M, N] = x . (Wq + U V)^T with V fp16 [r, K] and U fp16 [N, r]."""
    M = x.shape[0]
    if x.dim() != 2 or x.shape[1] != K:
        raise BrqError(f"x must be [M, {K}]")
    if signs.numel() != N * K // 64 or scales.numel() != N * K // 128:
        raise BrqError("signs/scales do not match N x K")
    if v.numel() != r * K or u.numel() != N * r:
        raise BrqError("v must be r x K and u N x r")
    code = _out_code(out_dtype)
    if y is None:
        y = torch.empty((M, N), dtype=out_dtype, device=x.device)
    ws, wsb = _ws(gemm_lr_workspace_bytes(M, N, K, r), x.device, ws)
    _check(lib().brq_gemm_lr(_dev(x, "x", torch.bfloat16), M, N, K, _dev(signs, "signs", torch.int64),
                             _dev(scales, "scales", torch.float16), _dev(v, "v", torch.float16),
                             _dev(u, "u", torch.float16), r, _dev(y, "y", out_dtype), code, _dev(ws, "ws"), wsb,
                             _stream()), "brq_gemm_lr")
    return y


def dbf_gemm(x, d_in, v, d_mid, u, d_out, m: int, n: int, r: int, out_dtype=torch.bfloat16, y=None, ws=None):
    """brq_dbf_gemm: y[M, m] = D_out U D_mid V D_in x for every row of x[M, n]."""
    M = x.shape[0]
    if x.dim() != 2 or x.shape[1] != n:
        raise BrqError(f"x must be [M, {n}]")
    if v.numel() != r * n // 64 or u.numel() != m * r // 64:
        raise BrqError("v must be r x n and u m x r sign planes")
    if d_in.numel() != n or d_mid.numel() != r or d_out.numel() != m:
        raise BrqError("diagonal lengths must be n, r, m")
    code = _out_code(out_dtype)
    if y is None:
        y = torch.empty((M, m), dtype=out_dtype, device=x.device)
    ws, wsb = _ws(dbf_workspace_bytes(M, m, n, r), x.device, ws)
    _check(lib().brq_dbf_gemm(_dev(x, "x", torch.bfloat16), M, m, n, r, _dev(d_in, "d_in", torch.float16),
                              _dev(v, "v", torch.int64), _dev(d_mid, "d_mid", torch.float16),
                              _dev(u, "u", torch.int64), _dev(d_out, "d_out", torch.float16),
                              _dev(y, "y", out_dtype), code, _dev(ws, "ws") if ws is not None else None, wsb,
                              _stream()), "brq_dbf_gemm")
    return y


def dbf_gemm_q8(x, d_in, v, d_mid, u, d_out, m: int, n: int, r: int, out_dtype=torch.bfloat16, y=None, ws=None):
    """brq_dbf_gemm_q8: the DBF chain with both binary products over per-row Q8 activation codes."""
    M = x.shape[0]
    if x.dim() != 2 or x.shape[1] != n:
        raise BrqError(f"x must be [M, {n}]")
    if v.numel() != r * n // 64 or u.numel() != m * r // 64:
        raise BrqError("v must be r x n and u m x r sign planes")
    if d_in.numel() != n or d_mid.numel() != r or d_out.numel() != m:
        raise BrqError("diagonal lengths must be n, r, m")
    code = _out_code(out_dtype)
    if y is None:
        y = torch.empty((M, m), dtype=out_dtype, device=x.device)
    ws, wsb = _ws(dbf_q8_workspace_bytes(M, m, n, r), x.device, ws)
    _check(lib().brq_dbf_gemm_q8(_dev(x, "x", torch.bfloat16), M, m, n, r, _dev(d_in, "d_in", torch.float16),
                                 _dev(v, "v", torch.int64), _dev(d_mid, "d_mid", torch.float16),
                                 _dev(u, "u", torch.int64), _dev(d_out, "d_out", torch.float16),
                                 _dev(y, "y", out_dtype), code, _dev(ws, "ws") if ws is not None else None, wsb,
                                 _stream()), "brq_dbf_gemm_q8")
    return y


def moe_ffn(x, logits, gate_s, gate_sc, up_s, up_sc, down_s, down_sc, E: int, H: int, I: int, top_k: int,
            out_dtype=torch.bfloat16, y=None, ws=None, return_routing: bool = False):
    """brq_moe_ffn: routed top-k SwiGLU layer. Returns y (and (ids, weights) if asked)."""
    T = x.shape[0]
    if x.dim() != 2 or x.shape[1] != H or logits.shape != (T, E):
        raise BrqError("x must be [T, H] and logits [T, E]")
    if gate_s.numel() != E * I * H // 64 or up_s.numel() != E * I * H // 64 or down_s.numel() != E * H * I // 64:
        raise BrqError("expert sign planes do not match E, H, I")
    if gate_sc.numel() != E * I * H // 128 or up_sc.numel() != E * I * H // 128 or down_sc.numel() != E * H * I // 128:
        raise BrqError("expert scales do not match E, H, I")
    code = _out_code(out_dtype)
    if y is None:
        y = torch.empty((T, H), dtype=out_dtype, device=x.device)
    ids = wts = None
    if return_routing:
        ids = torch.empty((T, top_k), dtype=torch.int32, device=x.device)
        wts = torch.empty((T, top_k), dtype=torch.float32, device=x.device)
    ws, wsb = _ws(moe_workspace_bytes(T, H, I, E, top_k), x.device, ws)
    if ws is None:
        raise BrqError("invalid MoE shape")
    _check(lib().brq_moe_ffn(_dev(x, "x", torch.bfloat16), _dev(logits, "logits", torch.float32), T, H, I, E, top_k,
                             _dev(gate_s, "gate_s", torch.int64), _dev(gate_sc, "gate_sc", torch.float16),
                             _dev(up_s, "up_s", torch.int64), _dev(up_sc, "up_sc", torch.float16),
                             _dev(down_s, "down_s", torch.int64), _dev(down_sc, "down_sc", torch.float16),
                             _dev(y, "y", out_dtype), code,
                             _dev(ids, "ids", torch.int32) if ids is not None else None,
                             _dev(wts, "w", torch.float32) if wts is not None else None,
                             _dev(ws, "ws"), wsb, _stream()), "brq_moe_ffn")
    if return_routing:
        return y, ids, wts
    return y


#: bytes of the scratch array brq_moe_ffn_noalloc uses (BRQ_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 16 << 20


def moe_ffn_noalloc(x, logits, gate_s, gate_sc, up_s, up_sc, down_s, down_sc, E: int, H: int, I: int, top_k: int,
                    out_dtype=torch.bfloat16, y=None, ids=None, wts=None):
    """brq_moe_ffn_noalloc: the routed layer of moe_ffn with the library's own
    scratch array as workspace (the call allocates no device memory; pass y,
    and ids / wts if the routing is wanted, to allocate nothing here either)."""
    T = x.shape[0]
    if x.dim() != 2 or x.shape[1] != H or logits.shape != (T, E):
        raise BrqError("x must be [T, H] and logits [T, E]")
    if gate_s.numel() != E * I * H // 64 or up_s.numel() != E * I * H // 64 or down_s.numel() != E * H * I // 64:
        raise BrqError("expert sign planes do not match E, H, I")
    if gate_sc.numel() != E * I * H // 128 or up_sc.numel() != E * I * H // 128 or down_sc.numel() != E * H * I // 128:
        raise BrqError("expert scales do not match E, H, I")
    code = _out_code(out_dtype)
    if y is None:
        y = torch.empty((T, H), dtype=out_dtype, device=x.device)
    if (ids is None) != (wts is None):
        raise BrqError("pass both ids and wts, or neither")
    if ids is not None and (ids.shape != (T, top_k) or wts.shape != (T, top_k)):
        raise BrqError("ids and wts must be [T, top_k]")
    _check(lib().brq_moe_ffn_noalloc(_dev(x, "x", torch.bfloat16), _dev(logits, "logits", torch.float32), T, H, I, E,
                                     top_k, _dev(gate_s, "gate_s", torch.int64),
                                     _dev(gate_sc, "gate_sc", torch.float16), _dev(up_s, "up_s", torch.int64),
                                     _dev(up_sc, "up_sc", torch.float16), _dev(down_s, "down_s", torch.int64),
                                     _dev(down_sc, "down_sc", torch.float16), _dev(y, "y", out_dtype), code,
                                     _dev(ids, "ids", torch.int32) if ids is not None else None,
                                     _dev(wts, "w", torch.float32) if wts is not None else None, _stream()),
           "brq_moe_ffn_noalloc")
    return y


def moe_dbf_workspace_bytes(T: int, H: int, I: int, E: int, top_k: int, r: int) -> int:
    return lib().brq_moe_dbf_workspace_bytes(T, H, I, E, top_k, r)


def moe_dbf_ffn(x, logits, gate, up, down, E: int, H: int, I: int, r: int, top_k: int,
                out_dtype=torch.bfloat16, y=None, ws=None, return_routing: bool = False):
    """brq_moe_dbf_ffn: the routed SwiGLU layer with DBF experts. gate, up, down
    are (d_in, v, d_mid, u, d_out) tensor tuples for all experts: d_in fp16
    [E, n], v int64 [E, r, n/64], d_mid fp16 [E, r], u int64 [E, m, r/64],
    d_out fp16 [E, m], with (m, n) = (I, H) for gate/up and (H, I) for down."""
    T = x.shape[0]
    if x.dim() != 2 or x.shape[1] != H or logits.shape != (T, E):
        raise BrqError("x must be [T, H] and logits [T, E]")

    def rec(t, m, n, name):
        d_in, v, d_mid, u, d_out = t
        if (d_in.numel() != E * n or v.numel() != E * r * n // 64 or d_mid.numel() != E * r
                or u.numel() != E * m * r // 64 or d_out.numel() != E * m):
            raise BrqError(f"{name} record does not match E={E}, m={m}, n={n}, r={r}")
        return DbfFactors(_dev(d_in, f"{name}.d_in", torch.float16), _dev(v, f"{name}.v", torch.int64),
                          _dev(d_mid, f"{name}.d_mid", torch.float16), _dev(u, f"{name}.u", torch.int64),
                          _dev(d_out, f"{name}.d_out", torch.float16))

    g, u_, d = rec(gate, I, H, "gate"), rec(up, I, H, "up"), rec(down, H, I, "down")
    code = _out_code(out_dtype)
    if y is None:
        y = torch.empty((T, H), dtype=out_dtype, device=x.device)
    ids = wts = None
    if return_routing:
        ids = torch.empty((T, top_k), dtype=torch.int32, device=x.device)
        wts = torch.empty((T, top_k), dtype=torch.float32, device=x.device)
    ws, wsb = _ws(moe_dbf_workspace_bytes(T, H, I, E, top_k, r), x.device, ws)
    if ws is None:
        raise BrqError("invalid DBF MoE shape")
    _check(lib().brq_moe_dbf_ffn(_dev(x, "x", torch.bfloat16), _dev(logits, "logits", torch.float32), T, H, I, E,
                                 top_k, r, ctypes.byref(g), ctypes.byref(u_), ctypes.byref(d),
                                 _dev(y, "y", out_dtype), code,
                                 _dev(ids, "ids", torch.int32) if ids is not None else None,
                                 _dev(wts, "w", torch.float32) if wts is not None else None,
                                 _dev(ws, "ws"), wsb, _stream()), "brq_moe_dbf_ffn")
    if return_routing:
        return y, ids, wts
    return y


def kron_rotate(x: torch.Tensor, H: torch.Tensor, R: torch.Tensor, y=None) -> torch.Tensor:
    """brq_kron_rotate: x'[t] = (H kron R) x[t], bf16 in and out, fp32 factors."""
    M = x.shape[0]
    n1, n2 = H.shape[0], R.shape[0]
    if x.dim() != 2 or x.shape[1] != n1 * n2 or H.shape != (n1, n1) or R.shape != (n2, n2):
        raise BrqError("x must be [M, n1*n2], H [n1, n1], R [n2, n2]")
    if y is None:
        y = torch.empty_like(x)
    _check(lib().brq_kron_rotate(_dev(x, "x", torch.bfloat16), M, _dev(H, "H", torch.float32), n1,
                                 _dev(R, "R", torch.float32), n2, _dev(y, "y", torch.bfloat16), _stream()),
           "brq_kron_rotate")
    return y
