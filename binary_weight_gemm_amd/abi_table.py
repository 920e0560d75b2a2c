"""The C ABI of libbrq.so as ctypes signatures: every function that
include/brq.h declares, name -> (restype, argtypes). Plain ctypes, no torch,
so that a host-only process (the sanitized host-layer test) can load the
library with it."""
import ctypes

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_sz = ctypes.c_size_t
_int = ctypes.c_int

#: every function of include/brq.h: name -> (restype, argtypes)
ABI_FUNCTIONS = {
    "brq_abi_version": (_int, []),
    "brq_status_str": (ctypes.c_char_p, [_int]),
    "brq_last_error": (ctypes.c_char_p, []),
    "brq_set_decode_fusion": (_int, [_int, ctypes.c_uint32]),
    "brq_debug_fail_launches": (_int, [ctypes.c_int32]),
    "brq_sign_words": (_sz, [_i64, _i64]),
    "brq_scale_count": (_sz, [_i64, _i64]),
    "brq_pack": (_int, [_vp, _i64, _i64, _vp, _vp, _vp]),
    "brq_gemm_workspace_bytes": (_sz, [_i64, _i64, _i64]),
    "brq_gemm": (_int, [_vp, _i64, _i64, _i64, _vp, _vp, _vp, _int, _vp, _sz, _vp]),
    "brq_gemm_lr_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64]),
    "brq_gemm_lr": (_int, [_vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _i64, _vp, _int, _vp, _sz, _vp]),
    "brq_dbf_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64]),
    "brq_dbf_gemm": (_int, [_vp, _i64, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _int, _vp, _sz, _vp]),
    "brq_dbf_q8_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64]),
    "brq_dbf_gemm_q8": (_int, [_vp, _i64, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _int, _vp, _sz, _vp]),
    "brq_moe_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64, _i64]),
    "brq_moe_ffn": (_int, [_vp, _vp, _i64, _i64, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _int,
                           _vp, _vp, _vp, _sz, _vp]),
    "brq_moe_ffn_noalloc": (_int, [_vp, _vp, _i64, _i64, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                   _int, _vp, _vp, _vp]),
    "brq_moe_dbf_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64, _i64, _i64]),
    "brq_moe_dbf_ffn": (_int, [_vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _int, _vp, _vp,
                               _vp, _sz, _vp]),
    "brq_kron_rotate": (_int, [_vp, _i64, _vp, _i64, _vp, _i64, _vp, _vp]),
}
