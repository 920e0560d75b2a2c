"""The host layer of libbrq (argument checks, status codes and error text,
size queries, the process-wide settings) under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU.

binary_weight_gemm_amd.build also builds libbrq_hostsan.so: abi.hip,
noalloc.hip and gsync.hip with both sanitizers on their host code. A child
Python process loads it with the sanitizer runtime preloaded and drives every
entry point through its host-side paths (NULL, shape, alignment, dtype and
workspace errors, the injected launch failure, and the device check, which
finds no GPU here); any sanitizer report ends the child with a non-zero
status. Nothing reaches a device: every pointer below is a placeholder that
no path taken here dereferences.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "binary_weight_gemm_amd", "_build", "libbrq_hostsan.so")

CHILD = r'''
import ctypes, importlib.util, sys
spec = importlib.util.spec_from_file_location("abi_table", sys.argv[2])
tab = importlib.util.module_from_spec(spec); spec.loader.exec_module(tab)
L = ctypes.CDLL(sys.argv[1])
for name, (res, args) in tab.ABI_FUNCTIONS.items():
    f = getattr(L, name); f.restype = res; f.argtypes = args
P = ctypes.c_void_p
a, b, c, d = P(1 << 20), P(2 << 20), P(3 << 20), P(4 << 20)
mis = P((1 << 20) + 4)
big = 1 << 40
seen = set()
def call(name, *args):
    s = getattr(L, name)(*args)
    seen.add(name)
    assert L.brq_last_error() is not None
    seen.add("brq_last_error")
    return s
# status text, sizes (including values that would overflow a careless product)
for s in range(-3, 12):
    assert call("brq_status_str", s)
assert call("brq_abi_version") == 1
for r, cc in ((4096, 14336), (3, 65), (1, 0), (big, big), (-1, 128), (1 << 62, 1 << 62)):
    call("brq_sign_words", r, cc); call("brq_scale_count", r, cc)
for args in ((1, 4096, 14336), (64, 4096, 14336), (4096, 14336, 4096), (big, big, big), (0, 1, 128), (-5, 1, 128)):
    call("brq_gemm_workspace_bytes", *args)
    call("brq_gemm_lr_workspace_bytes", *args, 20)
    call("brq_dbf_workspace_bytes", *args, 2048)
    call("brq_dbf_q8_workspace_bytes", *args, 2048)
for args in ((1, 2048, 512, 256, 8), (256, 4096, 2048, 1024, 16), (big, big, big, big, big), (0, 0, 0, 0, 0)):
    call("brq_moe_workspace_bytes", *args)
    call("brq_moe_dbf_workspace_bytes", *args, 1024)
# argument errors of every entry point
assert call("brq_pack", None, 16, 128, a, b, None) == 1
assert call("brq_pack", a, 16, 100, b, c, None) == 2
assert call("brq_pack", mis, 16, 128, b, c, None) == 3
assert call("brq_gemm", None, 1, 16, 128, a, b, c, 0, None, 0, None) == 1
assert call("brq_gemm", a, 1, 16, 100, b, c, d, 0, None, 0, None) == 2
assert call("brq_gemm", a, 1, 16, 128, b, c, d, 7, None, 0, None) == 4
assert call("brq_gemm", mis, 1, 16, 128, b, c, d, 0, None, 0, None) == 3
assert call("brq_gemm", a, 65, 4096, 4096, b, c, d, 0, None, 0, None) == 5
assert call("brq_gemm_lr", a, 1, 16, 128, b, c, None, None, 20, d, 0, None, 0, None) == 1
assert call("brq_dbf_gemm", a, 1, 16, 128, 100, a, b, c, d, a, b, 0, None, 0, None) != 0
assert call("brq_dbf_gemm_q8", None, 1, 16, 128, 128, a, b, c, d, a, b, 0, None, 0, None) == 1
assert call("brq_moe_ffn", a, b, 1, 2048, 512, 256, 99, a, b, c, d, a, b, c, 0, None, None, d, 0, None) == 2
assert call("brq_moe_ffn_noalloc", a, b, 1, 2048, 512, 256, 99, a, b, c, d, a, b, c, 0, None, None, None) == 2
assert call("brq_moe_dbf_ffn", a, b, 1, 2048, 512, 256, 8, 1024, None, None, None, c, 0, None, None, d, 0, None) == 1
assert call("brq_kron_rotate", a, 1, b, 48, c, 64, d, None) == 2
assert call("brq_set_decode_fusion", 9, 0) == 2
assert call("brq_debug_fail_launches", -2) == 2
# the injected failure, then the device check (no GPU in this process)
assert call("brq_debug_fail_launches", 1) == 0
assert call("brq_gemm", a, 1, 16, 128, b, c, d, 0, None, 0, None) == 7
assert call("brq_set_decode_fusion", 2, 5) == 0 and call("brq_set_decode_fusion", 0, 0) == 0
assert call("brq_gemm", a, 1, 16, 128, b, c, d, 0, None, 0, None) == 6
assert call("brq_kron_rotate", a, 1, b, 64, c, 64, d, None) == 6
missing = set(tab.ABI_FUNCTIONS) - seen
assert not missing, missing
print("ok", len(seen))
'''


@pytest.mark.skipif(not os.path.exists(LIB), reason="libbrq_hostsan.so is built by binary_weight_gemm_amd.build")
def test_host_layer_under_address_and_ub_sanitizers():
    sys.path.insert(0, ROOT)
    from binary_weight_gemm_amd.build import sanitizer_runtime
    rt = sanitizer_runtime()
    assert os.path.exists(rt), rt
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", HIP_VISIBLE_DEVICES="")
    table = os.path.join(ROOT, "binary_weight_gemm_amd", "abi_table.py")
    r = subprocess.run([sys.executable, "-c", CHILD, LIB, table], env=env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert r.stdout.startswith("ok"), r.stdout
