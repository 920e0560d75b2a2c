"""Host-side checks of the C ABI: the library loads, exports every function
include/brq.h declares, and rejects invalid arguments with the documented
status before touching a device. No compute call runs here."""
import ctypes
import os
import re

import pytest

import binary_weight_gemm_amd as brq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

OK, E_NULL, E_SHAPE, E_ALIGN, E_DTYPE, E_WORKSPACE, E_DEVICE, E_HIP = range(8)
P = ctypes.c_void_p(1 << 20)        # a non-NULL, aligned, never dereferenced address
PMIS = ctypes.c_void_p((1 << 20) + 2)


def header_functions():
    src = open(os.path.join(ROOT, "include", "brq.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(brq_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    return brq.lib()


def test_exports_every_declared_function(L):
    names = header_functions()
    assert len(names) == 22, names
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(brq.ABI_FUNCTIONS)


def test_version_and_status_strings(L):
    assert L.brq_abi_version() == 1
    assert L.brq_status_str(E_SHAPE) == b"BRQ_E_SHAPE"
    assert L.brq_status_str(OK) == b"BRQ_OK"
    assert L.brq_status_str(99) == b"BRQ_E_UNKNOWN"


def test_injected_launch_failure(L):
    """brq_debug_fail_launches: an armed call whose arguments pass returns
    BRQ_E_HIP with its text and enqueues nothing (it fails before the device
    check, so this runs without a GPU); invalid arguments still win and do not
    use up an injection."""
    x = ctypes.c_void_p(16)  # never dereferenced: every call below stops on the host
    assert L.brq_debug_fail_launches(-1) == E_SHAPE
    assert L.brq_debug_fail_launches(2) == OK
    # argument errors are reported first and do not consume the injection
    assert L.brq_gemm(None, 1, 16, 128, x, x, x, 0, None, 0, None) == E_NULL
    assert L.brq_gemm(x, 1, 16, 128, x, x, x, 0, None, 0, None) == E_HIP
    assert b"injected launch failure" in L.brq_last_error()
    assert L.brq_kron_rotate(x, 1, x, 64, x, 64, ctypes.c_void_p(1 << 20), None) == E_HIP
    # both injections spent; no further call with these placeholder pointers
    # here (past the hook a call would reach the device)
    assert L.brq_debug_fail_launches(0) == OK


def test_decode_fusion_setting(L):
    """brq_set_decode_fusion takes the three modes (host state only, no device
    call) and rejects any other value with BRQ_E_SHAPE."""
    for mode in (1, 2, 0):
        assert L.brq_set_decode_fusion(mode, 0) == OK
    assert L.brq_set_decode_fusion(2, 1000) == OK
    assert L.brq_set_decode_fusion(0, 0) == OK
    assert L.brq_set_decode_fusion(3, 0) == E_SHAPE
    assert b"unknown mode" in L.brq_last_error()
    assert L.brq_set_decode_fusion(-1, 0) == E_SHAPE


def test_size_queries(L):
    assert L.brq_sign_words(4096, 14336) == 4096 * 224
    assert L.brq_scale_count(4096, 14336) == 4096 * 112
    assert L.brq_sign_words(3, 65) == 0
    assert L.brq_scale_count(3, 64) == 0
    assert L.brq_gemm_workspace_bytes(1, 4096, 14336) == 0          # staged in LDS
    # 64-column tiles; K = 14336 split over 4 workgroups: 4 partial results of 64 x 4096 fp32
    assert L.brq_gemm_workspace_bytes(64, 4096, 14336) == 4 * 64 * 4096 * 4
    # one K-slice (K = 512 over 512 tiles of 64 columns): no workspace
    assert L.brq_gemm_workspace_bytes(64, 32768, 512) == 0
    assert L.brq_gemm_workspace_bytes(4096, 14336, 4096) == 4096 * 4096 * 2 + 4096 * 4   # staged rows, exponents
    assert L.brq_gemm_workspace_bytes(1, 16, 100) == 0
    assert L.brq_dbf_workspace_bytes(1, 4096, 4096, 2048) > 0
    assert L.brq_moe_workspace_bytes(1, 2048, 512, 256, 8) > 0
    assert L.brq_moe_workspace_bytes(300, 2048, 512, 256, 8) == 0
    assert L.brq_moe_workspace_bytes(1, 2048, 512, 256, 17) == 0


def _err(L):
    return L.brq_last_error().decode()


def test_pack_validation(L):
    assert L.brq_pack(None, 4, 128, P, P, None) == E_NULL
    assert "NULL" in _err(L)
    assert L.brq_pack(P, 0, 128, P, P, None) == E_SHAPE
    assert L.brq_pack(P, 4, 100, P, P, None) == E_SHAPE
    assert L.brq_pack(P, 4, 64, P, P, None) == E_SHAPE       # scales need cols % 128
    assert L.brq_pack(PMIS, 4, 128, P, P, None) == E_ALIGN


def test_gemm_validation(L):
    g = L.brq_gemm
    assert g(None, 1, 16, 128, P, P, P, 0, P, 1 << 20, None) == E_NULL
    assert g(P, 0, 16, 128, P, P, P, 0, P, 1 << 20, None) == E_SHAPE
    assert g(P, 1, 0, 128, P, P, P, 0, P, 1 << 20, None) == E_SHAPE
    assert g(P, 1, 16, 192, P, P, P, 0, P, 1 << 20, None) == E_SHAPE
    assert g(P, 1, 16, 128, P, P, P, 7, P, 1 << 20, None) == E_DTYPE
    assert g(P, 1, 16, 128, P, PMIS, P, 0, P, 1 << 20, None) == E_ALIGN
    assert g(P, 64, 16, 14336, P, P, P, 0, None, 0, None) == E_WORKSPACE
    assert g(P, 64, 16, 14336, P, P, P, 0, P, 10, None) == E_WORKSPACE
    assert "workspace" in _err(L)


def test_gemm_lr_validation(L):
    g = L.brq_gemm_lr
    ok = (P, 4, 16, 256, P, P, P, P, 20, P, 0, P, 1 << 22, None)
    assert g(None, *ok[1:]) == E_NULL
    assert g(*ok[:6], None, *ok[7:]) == E_NULL                        # v
    assert g(*ok[:8], 0, *ok[9:]) == E_SHAPE                           # rank 0
    assert g(*ok[:8], 65, *ok[9:]) == E_SHAPE                          # rank past 64
    assert "rank" in _err(L)
    assert g(*ok[:3], 200, *ok[4:]) == E_SHAPE                         # K % 128
    assert g(*ok[:10], 5, *ok[11:]) == E_DTYPE
    assert g(PMIS, *ok[1:]) == E_ALIGN
    assert g(*ok[:11], None, 0, None) == E_WORKSPACE
    assert L.brq_gemm_lr_workspace_bytes(4, 16, 256, 0) == 0
    assert L.brq_gemm_lr_workspace_bytes(4, 16, 256, 65) == 0
    # decode rows: padded V (64 x K fp16) + row exponents (256 B) + x V^T (fp32 [M][64]) + fp32 product
    # + the product's own workspace
    M, N, K = 4, 4096, 14336
    assert L.brq_gemm_lr_workspace_bytes(M, N, K, 20) == (64 * K * 2 + 256 + 1024 + M * N * 4
                                                          + L.brq_gemm_workspace_bytes(M, N, K))
    # many rows: padded V + row exponents + padded U (N x 64 fp16) + x V^T hi/lo (M x 128 fp16)
    # + staged activations
    M, N, K = 4096, 14336, 4096
    assert L.brq_gemm_lr_workspace_bytes(M, N, K, 20) == 64 * K * 2 + M * 4 + N * 128 + M * 256 + M * K * 2


def test_moe_dbf_validation(L):
    f = L.brq_moe_dbf_ffn
    rec = brq.DbfFactors(P, P, P, P, P)
    bad = brq.DbfFactors(P, None, P, P, P)
    mis = brq.DbfFactors(P, PMIS, P, P, P)
    R = ctypes.byref
    ok = [P, P, 4, 2048, 512, 256, 8, 1024, R(rec), R(rec), R(rec), P, 0, None, None, P, 1 << 30, None]

    def call(**kw):
        a = list(ok)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f(*a)

    assert call(a0=None) == E_NULL
    assert call(a9=R(bad)) == E_NULL                     # a missing tensor in the up record
    assert "record" in _err(L)
    assert call(a2=0) == E_SHAPE                          # T
    assert call(a7=100) == E_SHAPE                        # r % 128
    assert call(a3=8320) == E_SHAPE                       # H past 8192
    assert call(a7=4096) == E_SHAPE                       # r past 2048
    assert call(a6=300) == E_SHAPE                        # top_k past min(E, 16)
    assert call(a12=9) == E_DTYPE
    assert call(a10=R(mis)) == E_ALIGN
    assert call(a15=None) == E_WORKSPACE
    assert L.brq_moe_dbf_workspace_bytes(4, 2048, 512, 256, 8, 1024) == (
        L.brq_moe_workspace_bytes(4, 2048, 512, 256, 8) + 2 * 2 * 4 * 8 * 1024 * 2)
    assert L.brq_moe_dbf_workspace_bytes(4, 2048, 512, 256, 8, 100) == 0


def test_dbf_validation(L):
    f = L.brq_dbf_gemm
    args = [P, 1, 4096, 4096, 2048, P, P, P, P, P, P, 0, P, 1 << 30, None]
    bad = list(args); bad[5] = None
    assert f(*bad) == E_NULL
    bad = list(args); bad[3] = 4000
    assert f(*bad) == E_SHAPE
    bad = list(args); bad[4] = 100
    assert f(*bad) == E_SHAPE
    bad = list(args); bad[11] = 5
    assert f(*bad) == E_DTYPE
    bad = list(args); bad[13] = 16
    assert f(*bad) == E_WORKSPACE


def test_dbf_q8_validation(L):
    f = L.brq_dbf_gemm_q8
    args = [P, 1, 4096, 4096, 2048, P, P, P, P, P, P, 0, P, 1 << 30, None]
    bad = list(args); bad[6] = None
    assert f(*bad) == E_NULL
    bad = list(args); bad[1] = 0
    assert f(*bad) == E_SHAPE
    bad = list(args); bad[3] = 4000
    assert f(*bad) == E_SHAPE
    bad = list(args); bad[4] = 100
    assert f(*bad) == E_SHAPE
    bad = list(args); bad[3] = 131072 + 128                 # 127 n must stay below 2^24
    assert f(*bad) == E_SHAPE
    bad = list(args); bad[6] = PMIS
    assert f(*bad) == E_ALIGN
    bad = list(args); bad[7] = PMIS                         # d_mid is read 8 values at a time
    assert f(*bad) == E_ALIGN
    bad = list(args); bad[10] = PMIS; bad[11] = 1           # fp32 y needs 4-byte alignment
    assert f(*bad) == E_ALIGN
    bad = list(args); bad[11] = 5
    assert f(*bad) == E_DTYPE
    bad = list(args); bad[13] = 16
    assert f(*bad) == E_WORKSPACE
    bad = list(args); bad[12] = PMIS
    assert f(*bad) == E_WORKSPACE
    # codes [M][n] int8, exponents [M], h_s [M][r] fp32, codes [M][r], exponents [M]; 4096 rows fill
    # 512 tiles and split no reduction
    assert L.brq_dbf_q8_workspace_bytes(4096, 4096, 4096, 2048) == (4096 * 4096 + 4 * 4096 + 4096 * 2048 * 4
                                                                    + 4096 * 2048 + 4 * 4096)
    # 512 rows: 64-row tiles, 128 and 256 of them, no K-split
    assert L.brq_dbf_q8_workspace_bytes(512, 4096, 4096, 2048) == (512 * 4096 + 2048 + 512 * 2048 * 4
                                                                   + 512 * 2048 + 2048)
    # one row: 16 tiles of the first product in 8 K-slices, 32 of the second in 4 (int32 partials)
    assert L.brq_dbf_q8_workspace_bytes(1, 4096, 4096, 2048) == (4096 + 256 + 2048 * 4 + 2048 + 256
                                                                 + max(8 * 2048, 4 * 4096) * 4)
    assert L.brq_dbf_q8_workspace_bytes(1, 4096, 4096, 100) == 0


def test_moe_validation(L):
    f = L.brq_moe_ffn
    args = [P, P, 1, 2048, 512, 256, 8, P, P, P, P, P, P, P, 0, None, None, P, 1 << 30, None]
    bad = list(args); bad[1] = None
    assert f(*bad) == E_NULL
    bad = list(args); bad[2] = 0
    assert f(*bad) == E_SHAPE
    bad = list(args); bad[2] = 257
    assert f(*bad) == E_SHAPE
    bad = list(args); bad[6] = 300
    assert f(*bad) == E_SHAPE
    bad = list(args); bad[3] = 2000
    assert f(*bad) == E_SHAPE
    bad = list(args); bad[12] = PMIS
    assert f(*bad) == E_ALIGN
    bad = list(args); bad[18] = 8
    assert f(*bad) == E_WORKSPACE


def test_kron_validation(L):
    f = L.brq_kron_rotate
    assert f(None, 4, P, 64, P, 64, P, None) == E_NULL
    assert f(P, 4, P, 32, P, 128, ctypes.c_void_p(1 << 30), None) == E_SHAPE
    assert f(P, 4, P, 48, P, 64, ctypes.c_void_p(1 << 30), None) == E_SHAPE   # factor size not 32, 64 or 96
    assert f(P, 4, P, 96, P, 96, ctypes.c_void_p(1 << 30), None) == E_SHAPE   # n1 * n2 above 6144
    assert f(P, 4, P, 16, P, 64, ctypes.c_void_p(1 << 30), None) == E_SHAPE
    assert f(P, 4, P, 64, P, 64, P, None) == E_SHAPE         # x and y overlap
    assert f(PMIS, 4, P, 64, P, 64, ctypes.c_void_p(1 << 30), None) == E_ALIGN


def test_device_check_without_gpu(L):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; valid arguments would reach the device")
    assert L.brq_pack(P, 4, 128, P, P, None) == E_DEVICE
    assert L.brq_gemm(P, 1, 16, 128, P, P, P, 0, P, 1 << 20, None) == E_DEVICE


def test_binding_refuses_host_tensors():
    import torch
    w = torch.zeros((4, 128), dtype=torch.float32)
    with pytest.raises(brq.BrqError):
        brq.pack(w)


def test_moe_noalloc_validation(L):
    f = L.brq_moe_ffn_noalloc
    args = [P, P, 1, 2048, 512, 256, 8, P, P, P, P, P, P, P, 0, None, None, None]
    bad = list(args); bad[1] = None
    assert f(*bad) == E_NULL
    bad = list(args); bad[2] = 0
    assert f(*bad) == E_SHAPE
    bad = list(args); bad[3] = 2000
    assert f(*bad) == E_SHAPE
    # beyond the library's scratch array: refused before any device call
    big = list(args); big[2] = 256; big[3] = 4096; big[4] = 2048; big[6] = 16
    assert f(*big) == E_WORKSPACE
    assert b"scratch" in L.brq_last_error()
