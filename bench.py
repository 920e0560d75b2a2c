"""Benchmark of the binary-weight hot path on one MI355X.

Headline (value): decode-shaped binary GEMV at M=1 -- one step is y = x . Wq^T
for both decode matrices, W 4096x14336 and 14336x4096 in the group-128 sign +
fp16 scale format, bf16 activations, bf16 outputs. Throughput is algorithmic
HBM bytes (packed weights + activations in + outputs out) per second. The
timed steps walk a ring of distinct weight copies (larger than twice the 256 MB
Infinity Cache; a copy comes back only after more than 512 MB of others), and
the caches are scrubbed before every timed replay, so every call streams its
weights from HBM.

Also reported (extra): device facts and reference rates (a 1 GiB device copy,
the vendor library's bf16 GEMM); the 1024 x 1024 single GEMV (cache resident);
the same product at M = 4, 16, 64; the packing pass of
the 14336 x 4096 matrix; the routed MoE layer
(256 experts, top-8, hidden 2048, intermediate 512) at T = 1 and 64 decode
tokens, with group-128 experts and with DBF-chain experts (r = 1024); the DBF chain (4096x4096, r = 2048) at M = 1 and 512; the prefill
product at M = 4096 (4096 -> 14336) with the Kronecker rotation before it, and
the same product with a rank-20 weight correction fused into its epilogue.

The CPU baseline is the fp64 numpy oracle on the host cores, timed on a bounded
sample of the headline workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extra] [--no-cpu]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "binary GEMV/MoE decode HBM GB/s (% of peak) at M=1; prefill TFLOP/s at M=4096"
HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0
MALL_BYTES = 256 * 2 ** 20


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def packed_bytes(N, K):
    return N * K // 8 + 2 * (N * K // 128)


def dev_np(a):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def kernel_source_hash(files):
    """sha256 over the named kernel sources (csrc/), to tie counter readings to the code they came from."""
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "binary_weight_gemm_amd", "csrc", f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


# HBM traffic of the headline kernel, from rocprofv3 FETCH_SIZE / WRITE_SIZE runs
# (profiles/decode_m1_traffic.txt, a JSON record). It is reported only while the kernel
# sources still hash to the value recorded with the counters.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_m1_traffic.txt")
DECODE_SOURCES = ("common.h", "dec_core.h", "dec.hip", "abi.hip", "kernels.h")


def recorded_traffic():
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != kernel_source_hash(DECODE_SOURCES):
        return None
    return rec.get("bytes_per_launch")


def copy_calibration(torch, mib=512, reps=5):
    """Plain device-to-device copies of a known size: the reference reading that
    scales the FETCH_SIZE / WRITE_SIZE counters to bytes."""
    n = mib * 2 ** 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    return dict(copy_bytes=n, reps=reps)


def warm_gpu(torch, seconds=0.5):
    """Run dense matrix products for about `seconds` so that clocks and power
    reach their steady state before anything is timed (the first few hundred
    microseconds of work after an idle period run at lower clocks)."""
    a = torch.randn((8192, 8192), device="cuda", dtype=torch.float16)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            a = torch.matmul(a, a).mul_(1e-4)
        torch.cuda.synchronize()
    del a


def ring_copies(per_copy_bytes):
    return max(2, int(np.ceil(2 * MALL_BYTES / per_copy_bytes)))


# ---------------------------------------------------------------------------
# headline: C2 decode at M (default 1)
# ---------------------------------------------------------------------------

def setup_c2(brq, torch, M):
    import datagen
    mats = []
    for which in (0, 1):
        N, K = datagen.C2_SHAPES[which]
        w = torch.from_numpy(datagen.C2_weight(which)).cuda()
        s, sc = brq.pack(w)
        del w
        mats.append((N, K, s, sc))
    torch.cuda.synchronize()
    per_step = sum(packed_bytes(N, K) for N, K, _, _ in mats)
    copies = ring_copies(per_step)
    ring = []
    for c in range(copies):
        ring.append([(N, K, s.clone(), sc.clone()) for N, K, s, sc in mats])
    xs = [dev_np(datagen.C2_x(which, M)) for which in (0, 1)]
    ys = [torch.empty((M, N), dtype=torch.bfloat16, device="cuda") for N, K, _, _ in mats]
    wss = [torch.empty(max(brq.gemm_workspace_bytes(M, N, K), 256), dtype=torch.uint8, device="cuda")
           for N, K, _, _ in mats]
    step_bytes = sum(packed_bytes(N, K) + M * K * 2 + M * N * 2 for N, K, _, _ in mats)
    return ring, xs, ys, wss, step_bytes


_SCRUB = []


def scrub_caches(torch):
    """Read a buffer of twice the Infinity Cache's size (untimed), so that
    whatever an earlier replay left in the caches has been evicted: the next
    replay's first weight reads come from HBM."""
    if not _SCRUB:
        _SCRUB.append(torch.ones(2 * MALL_BYTES // 4, dtype=torch.float32, device="cuda"))
    _SCRUB.append(_SCRUB[0].sum())
    del _SCRUB[1:]


def graph_time(torch, fn, n_items, replays=5):
    """Capture fn() (which enqueues n_items kernel launches) in a HIP graph,
    replay it `replays` times and return ms per replay (median), GPU time only:
    no host submission gaps between the captured launches. Before each timed
    replay the caches are scrubbed (scrub_caches), so a replay never finds
    weights that the previous one left in the Infinity Cache; inside a replay
    the callers walk a ring of distinct weight copies."""
    warm_gpu(torch, 0.3)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # eager pass on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    times = []
    for _ in range(replays):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        scrub_caches(torch)
        torch.cuda.synchronize()
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    del g
    times.sort()
    return times[len(times) // 2]


def run_c2(brq, torch, M, steps, warmup):
    ring, xs, ys, wss, step_bytes = setup_c2(brq, torch, M)
    n = len(ring)

    def step(i):
        for j, (N, K, s, sc) in enumerate(ring[i % n]):
            brq.gemm(xs[j], s, sc, N, K, out_dtype=torch.bfloat16, y=ys[j], ws=wss[j])

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()

    def timed():
        for i in range(steps):
            step(warmup + i)

    ms = graph_time(torch, timed, 2 * steps)
    res = dict(M=M, ms_per_step=ms / steps, step_bytes=step_bytes, gbs=step_bytes * steps / (ms * 1e-3) / 1e9,
               tflops=2.0 * M * sum(N * K for N, K, _, _ in ring[0]) * steps / (ms * 1e-3) / 1e12,
               ring_copies=n, launch_ms=ms / (2 * steps))
    res["launch_gbs"] = (step_bytes / 2) / (res["launch_ms"] * 1e-3) / 1e9
    del ring
    torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------------------
# extras
# ---------------------------------------------------------------------------

def device_facts(torch):
    p = torch.cuda.get_device_properties(0)
    return dict(name=p.name, arch=getattr(p, "gcnArchName", ""), compute_units=p.multi_processor_count,
                memory_gib=round(p.total_memory / 2 ** 30, 1))


def achievable_peaks(torch, reps=10):
    """Reference rates on this device (not the product): a 1 GiB device copy
    (read + write) for HBM, and the vendor library's 8192^3 bf16 and fp16
    GEMMs (hipBLASLt through torch.matmul; fp16 is the operand type of the
    prefill product) for the matrix cores; back-to-back calls between two
    events."""
    n = 2 ** 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    a = torch.randn((8192, 8192), device="cuda", dtype=torch.bfloat16)
    b = torch.randn((8192, 8192), device="cuda", dtype=torch.bfloat16)
    c = torch.empty_like(a)
    ah, bh = a.to(torch.float16), b.to(torch.float16)
    ch = torch.empty_like(ah)
    warm_gpu(torch, 0.3)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    copy_ms = timed(lambda: dst.copy_(src))
    gemm_ms = timed(lambda: torch.matmul(a, b, out=c))
    gemm16_ms = timed(lambda: torch.matmul(ah, bh, out=ch))
    del src, dst, a, b, c, ah, bh, ch
    torch.cuda.empty_cache()
    copy_gbs = 2 * n / (copy_ms * 1e-3) / 1e9
    gemm_tflops = 2 * 8192 ** 3 / (gemm_ms * 1e-3) / 1e12
    gemm16_tflops = 2 * 8192 ** 3 / (gemm16_ms * 1e-3) / 1e12
    return dict(hbm_copy_gbs=copy_gbs, hbm_copy_frac=copy_gbs / HBM_PEAK_GBS,
                bf16_gemm_tflops=gemm_tflops, bf16_gemm_frac=gemm_tflops / MFMA_F16_PEAK_TFLOPS,
                f16_gemm_tflops=gemm16_tflops, f16_gemm_frac=gemm16_tflops / MFMA_F16_PEAK_TFLOPS)


def reference_kernels(torch, brq):
    """Rates of this device's own reference kernels (libbrq_ref.so, not the
    product): a plain streaming read of 8.26 MB (the packed size of one decode
    matrix) on a cold ring of copies, one launch per copy, graph-timed like the
    headline (launch overhead included); the same read of 1 GiB; and a loop of
    independent 32x32x16 fp16 matrix-core products (1024 workgroups of 4 waves)."""
    import ctypes
    L = ctypes.CDLL(os.path.join(ROOT, "binary_weight_gemm_amd", "libbrq_ref.so"))
    L.brq_ref_stream_blocks.restype = ctypes.c_uint
    L.brq_ref_stream_blocks.argtypes = [ctypes.c_size_t]
    L.brq_ref_stream_read.restype = ctypes.c_int
    L.brq_ref_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    L.brq_ref_mfma_loop.restype = ctypes.c_int
    L.brq_ref_mfma_loop.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    out = {}
    nbytes = packed_bytes(14336, 4096)
    nbytes -= nbytes % 16
    copies = ring_copies(nbytes)
    ring = [torch.ones(nbytes // 4, dtype=torch.int32, device="cuda") for _ in range(copies)]
    sink = torch.zeros(max(L.brq_ref_stream_blocks(nbytes), 1), dtype=torch.int32, device="cuda")

    def stream():
        st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        for t in ring:
            assert L.brq_ref_stream_read(ctypes.c_void_p(t.data_ptr()), nbytes, ctypes.c_void_p(sink.data_ptr()), st) == 0

    ms = graph_time(torch, stream, copies) / copies
    out["stream_read_8mb"] = dict(bytes=nbytes, us_per_launch=ms * 1e3, gbs=nbytes / (ms * 1e-3) / 1e9)
    del ring
    big = torch.ones((1 << 30) // 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(L.brq_ref_stream_blocks(1 << 30), dtype=torch.int32, device="cuda")

    def stream_big():
        st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        assert L.brq_ref_stream_read(ctypes.c_void_p(big.data_ptr()), 1 << 30, ctypes.c_void_p(sink.data_ptr()), st) == 0

    ms = graph_time(torch, stream_big, 1)
    out["stream_read_1gib"] = dict(us=ms * 1e3, gbs=(1 << 30) / (ms * 1e-3) / 1e9)
    del big
    blocks, iters = 1024, 4000
    fsink = torch.zeros(blocks, dtype=torch.float32, device="cuda")

    def mfma():
        st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        assert L.brq_ref_mfma_loop(blocks, iters, ctypes.c_void_p(fsink.data_ptr()), st) == 0

    ms = graph_time(torch, mfma, 1)
    flops = blocks * 4 * 8 * iters * 32768.0
    out["mfma_f16_loop"] = dict(us=ms * 1e3, tflops=flops / (ms * 1e-3) / 1e12,
                                frac_of_peak=flops / (ms * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS)
    torch.cuda.empty_cache()
    return out


def isolated_call_us(brq, torch, reps=20):
    """One decode product (M = 1, the 14336 x 4096 matrix) launched on its own
    between two synchronisations, median of `reps`: launch overhead included."""
    import datagen
    N, K = datagen.C2_SHAPES[1]
    s, sc = brq.pack(torch.from_numpy(datagen.C2_weight(1)).cuda())
    x = dev_np(datagen.C2_x(1, 1))
    y = torch.empty((1, N), dtype=torch.bfloat16, device="cuda")
    brq.gemm(x, s, sc, N, K, y=y)
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        brq.gemm(x, s, sc, N, K, y=y)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e3)
    ts.sort()
    return ts[len(ts) // 2]


def run_c1(brq, torch, iters=50):
    """C1, the single GEMV on a 1024 x 1024 matrix: its 151 KB stay in the
    caches, so this is a latency figure, not an HBM one."""
    import datagen
    w, xh = datagen.C1()
    s, sc = brq.pack(torch.from_numpy(w).cuda())
    x = dev_np(xh)
    y = torch.empty((1, 1024), dtype=torch.bfloat16, device="cuda")
    brq.gemm(x, s, sc, 1024, 1024, y=y)
    torch.cuda.synchronize()

    def timed():
        for _ in range(iters):
            brq.gemm(x, s, sc, 1024, 1024, y=y)

    ms = graph_time(torch, timed, iters) / iters
    nbytes = packed_bytes(1024, 1024) + 1024 * 2 * 2
    return dict(us=ms * 1e3, gbs=nbytes / (ms * 1e-3) / 1e9, note="cache-resident, latency-bound")


def run_pack(brq, torch, iters=10):
    """The packing pass (group-128 sign + fp16 scale) of the larger decode
    matrix, 14336 x 4096 fp32, graph-timed: algorithmic bytes are the fp32
    weights read and the packed bytes written."""
    import datagen
    N, K = datagen.C2_SHAPES[1]
    w = torch.from_numpy(datagen.C2_weight(1)).cuda()
    s = torch.empty((N, K // 64), dtype=torch.int64, device="cuda")
    sc = torch.empty((N, K // 128), dtype=torch.float16, device="cuda")
    brq.pack(w, out=(s, sc))
    torch.cuda.synchronize()

    def timed():
        for _ in range(iters):
            brq.pack(w, out=(s, sc))

    ms = graph_time(torch, timed, iters) / iters
    nbytes = 4 * N * K + packed_bytes(N, K)
    del w, s, sc
    torch.cuda.empty_cache()
    return dict(shape=[N, K], us=ms * 1e3, gbs=nbytes / (ms * 1e-3) / 1e9,
                frac_of_hbm=nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS)


def run_moe(brq, torch, Ts, iters=50, fusion=0):
    """The routed MoE layer at the C4 shape; fusion selects the single-launch
    setting (brq.set_decode_fusion) for the timed calls."""
    import datagen
    cfg = datagen.C4()
    E, H, I, k = cfg.E, cfg.H, cfg.I, cfg.top_k
    gs = torch.empty((E, I, H // 64), dtype=torch.int64, device="cuda")
    gsc = torch.empty((E, I, H // 128), dtype=torch.float16, device="cuda")
    us, usc = torch.empty_like(gs), torch.empty_like(gsc)
    ds = torch.empty((E, H, I // 64), dtype=torch.int64, device="cuda")
    dsc = torch.empty((E, H, I // 128), dtype=torch.float16, device="cuda")
    for e in range(E):
        for f, (a, b) in ((cfg.gate, (gs, gsc)), (cfg.up, (us, usc)), (cfg.down, (ds, dsc))):
            brq.pack(torch.from_numpy(f(e)).cuda(), out=(a[e], b[e]))
    torch.cuda.synchronize()
    layer_bytes = 3 * E * packed_bytes(I, H)
    copies = ring_copies(layer_bytes)
    ring = [(gs.clone(), gsc.clone(), us.clone(), usc.clone(), ds.clone(), dsc.clone()) for _ in range(copies)]
    out = {}
    for T in Ts:
        x = dev_np(cfg.x(T))
        lgs = [dev_np(cfg.logits(T, it)) for it in range(iters)]
        y = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(brq.moe_workspace_bytes(T, H, I, E, k), dtype=torch.uint8, device="cuda")
        # algorithmic bytes: distinct selected experts' packed weights + x + logits + y
        nbytes = 0
        for it in range(iters):
            ids = np.argsort(-cfg.logits(T, it), axis=1, kind="stable")[:, :k]
            nbytes += len(np.unique(ids)) * 3 * packed_bytes(I, H) + T * (H * 2 * 2 + E * 4)
        brq.set_decode_fusion(fusion)
        for it in range(5):
            brq.moe_ffn(x, lgs[it], *ring[it % copies], E, H, I, k, y=y, ws=ws)
        torch.cuda.synchronize()

        def timed():
            for it in range(iters):
                brq.moe_ffn(x, lgs[it], *ring[it % copies], E, H, I, k, y=y, ws=ws)

        ms = graph_time(torch, timed, iters) / iters
        brq.set_decode_fusion(brq.FUSION_DEFAULT)
        out[f"T={T}"] = dict(us_per_layer=ms * 1e3, gbs=nbytes / iters / (ms * 1e-3) / 1e9,
                             tokens_per_s=T / (ms * 1e-3), ring_copies=copies)
    del ring, gs, gsc, us, usc, ds, dsc
    torch.cuda.empty_cache()
    return out


def run_moe_dbf(brq, torch, Ts, iters=50, geometry=None):
    """The DBF-expert MoE layer at the deployed shape (256 experts, top-8,
    gate/up 512x2048, down 2048x512, r = 1024), or at one of the named
    geometries of datagen.MOE_GEOMETRIES: random sign words and fp16
    log-normal diagonals on the device (timing does not depend on their
    values), D_mid at 2^-12 as in the parity inputs."""
    import datagen
    cfg = datagen.C4D() if geometry is None else datagen.C4D(**datagen.MOE_GEOMETRIES[geometry], top_k=8)
    E, H, I, r, k = cfg.E, cfg.H, cfg.I, cfg.r, cfg.top_k
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7)

    def words(*shape):
        return torch.randint(-2 ** 62, 2 ** 62, shape, dtype=torch.int64, device="cuda", generator=gen)

    def diag(n, scale=1.0):
        g = torch.randn((E, n), device="cuda", generator=gen)
        return (torch.exp(0.5 * g) * scale).to(torch.float16)

    def rec(m, n):
        return (diag(n), words(E, r, n // 64), diag(r, 2.0 ** -12), words(E, m, r // 64), diag(m))

    base = (rec(I, H), rec(I, H), rec(H, I))
    exp_bytes = 2 * ((r * H + I * r) // 8 + 2 * (H + r + I)) + (r * I + H * r) // 8 + 2 * (I + r + H)
    copies = ring_copies(E * exp_bytes)
    ring = [base] + [tuple(tuple(t.clone() for t in rc) for rc in base) for _ in range(copies - 1)]
    out = {}
    for T in Ts:
        x = dev_np(cfg.x(T))
        lgs = [dev_np(cfg.logits(T, it)) for it in range(iters)]
        y = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(brq.moe_dbf_workspace_bytes(T, H, I, E, k, r), dtype=torch.uint8, device="cuda")
        # algorithmic bytes: distinct selected experts' factors + x + logits + y
        nbytes = 0
        for it in range(iters):
            ids = np.argsort(-cfg.logits(T, it), axis=1, kind="stable")[:, :k]
            nbytes += len(np.unique(ids)) * exp_bytes + T * (H * 2 * 2 + E * 4)
        for it in range(5):
            brq.moe_dbf_ffn(x, lgs[it], *ring[it % copies], E, H, I, r, k, y=y, ws=ws)
        torch.cuda.synchronize()

        def timed():
            for it in range(iters):
                brq.moe_dbf_ffn(x, lgs[it], *ring[it % copies], E, H, I, r, k, y=y, ws=ws)

        ms = graph_time(torch, timed, iters) / iters
        out[f"T={T}"] = dict(us_per_layer=ms * 1e3, gbs=nbytes / iters / (ms * 1e-3) / 1e9,
                             tokens_per_s=T / (ms * 1e-3), ring_copies=copies)
    del ring, base
    torch.cuda.empty_cache()
    return out


def run_dbf(brq, torch, Ms, iters=50, q8=False, r=2048, fusion=0):
    """The DBF chain at the DBF workload's shapes (rank r); q8 selects the path
    over Q8 activation codes (int8 matrix cores) instead of the fp16-piece path;
    fusion the single-launch setting (brq.set_decode_fusion)."""
    import datagen
    gemm = brq.dbf_gemm_q8 if q8 else brq.dbf_gemm
    ws_bytes = brq.dbf_q8_workspace_bytes if q8 else brq.dbf_workspace_bytes
    out = {}
    for M in Ms:
        d = datagen.C3(M, r=r)
        m, n, r = d["m"], d["n"], d["r"]
        v, _ = brq.pack(torch.from_numpy(d["v"]).cuda(), scales=False)
        u, _ = brq.pack(torch.from_numpy(d["u"]).cuda(), scales=False)
        wbytes = (r * n + m * r) // 8 + 2 * (n + r + m)
        copies = ring_copies(wbytes) if M == 1 else 1
        ring = [(v.clone(), u.clone()) for _ in range(copies)]
        x = dev_np(d["x"])
        di, dm, do = (torch.from_numpy(d[k]).cuda() for k in ("d_in", "d_mid", "d_out"))
        y = torch.empty((M, m), dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(ws_bytes(M, m, n, r), dtype=torch.uint8, device="cuda")
        brq.set_decode_fusion(fusion)
        for i in range(5):
            gemm(x, di, ring[i % copies][0], dm, ring[i % copies][1], do, m, n, r, y=y, ws=ws)
        torch.cuda.synchronize()

        def timed():
            for i in range(iters):
                gemm(x, di, ring[i % copies][0], dm, ring[i % copies][1], do, m, n, r, y=y, ws=ws)

        ms = graph_time(torch, timed, iters) / iters
        brq.set_decode_fusion(brq.FUSION_DEFAULT)
        nbytes = wbytes + M * n * 2 + M * m * 2
        flops = 2.0 * M * (r * n + m * r)
        out[f"M={M}"] = dict(us=ms * 1e3, gbs=nbytes / (ms * 1e-3) / 1e9, tflops=flops / (ms * 1e-3) / 1e12,
                             bpe=(r * (m + n) + 16 * (m + n + r)) / (m * n))
        del ring
    torch.cuda.empty_cache()
    return out


def run_prefill(brq, torch, iters=10):
    import datagen
    d = datagen.C5()
    N, K = d["N"], d["K"]
    w = torch.from_numpy(datagen.C5_weight(N, K)).cuda()
    s, sc = brq.pack(w)
    del w
    x = dev_np(d["x"])
    H, R = dev_np(d["H"]), dev_np(d["R"])
    xr = torch.empty_like(x)
    y = torch.empty((x.shape[0], N), dtype=torch.bfloat16, device="cuda")
    for _ in range(2):
        brq.kron_rotate(x, H, R, y=xr)
        brq.gemm(xr, s, sc, N, K, y=y)
    warm_gpu(torch)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    rot_ms = gemm_ms = 0.0
    for _ in range(iters):
        ev[0].record()
        brq.kron_rotate(x, H, R, y=xr)
        ev[1].record()
        brq.gemm(xr, s, sc, N, K, y=y)
        ev[2].record()
        torch.cuda.synchronize()
        rot_ms += ev[0].elapsed_time(ev[1])
        gemm_ms += ev[1].elapsed_time(ev[2])
    rot_ms /= iters
    gemm_ms /= iters
    # the same product with a rank-20 weight correction fused into its epilogue
    # (rank 0.005 of the dimension); factors are synthetic normal fp16
    r = 20
    g = torch.Generator(device="cuda")
    g.manual_seed(20)
    v = (torch.randn((r, K), device="cuda", generator=g) * 0.02).to(torch.float16)
    u = (torch.randn((N, r), device="cuda", generator=g) * 0.02).to(torch.float16)
    ws_lr = torch.empty(brq.gemm_lr_workspace_bytes(x.shape[0], N, K, r), dtype=torch.uint8, device="cuda")
    for _ in range(2):
        brq.gemm_lr(xr, s, sc, v, u, N, K, r, y=y, ws=ws_lr)
    torch.cuda.synchronize()

    # both products graph-replayed (the corrected one is five launches, two of
    # them short: eager timing would measure the host's launch gaps)
    ws_pf = torch.empty(brq.gemm_workspace_bytes(x.shape[0], N, K), dtype=torch.uint8, device="cuda")

    def plain():
        for _ in range(iters):
            brq.gemm(xr, s, sc, N, K, y=y, ws=ws_pf)

    def corrected():
        for _ in range(iters):
            brq.gemm_lr(xr, s, sc, v, u, N, K, r, y=y, ws=ws_lr)

    def rotations():
        for _ in range(iters):
            brq.kron_rotate(x, H, R, y=xr)

    gemm_graph_ms = graph_time(torch, plain, 3 * iters) / iters
    lr_ms = graph_time(torch, corrected, 5 * iters) / iters
    rot_graph_ms = graph_time(torch, rotations, iters) / iters
    M = x.shape[0]
    flops = 2.0 * M * N * K
    flops_lr = flops + 2.0 * M * r * (K + N)
    res = dict(M=M, N=N, K=K, gemm_us=gemm_ms * 1e3, gemm_tflops=flops / (gemm_ms * 1e-3) / 1e12,
               gemm_frac_of_f16_peak=flops / (gemm_ms * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS,
               gemm_graph_us=gemm_graph_ms * 1e3,
               gemm_lr20_us=lr_ms * 1e3, gemm_lr20_tflops=flops_lr / (lr_ms * 1e-3) / 1e12,
               rotate_us=rot_ms * 1e3, rotate_gbs=(2 * M * K * 2) / (rot_ms * 1e-3) / 1e9,
               rotate_graph_us=rot_graph_ms * 1e3,
               rotate_graph_tflops_f32=2.0 * 2 * 64 ** 3 * M / (rot_graph_ms * 1e-3) / 1e12,
               tokens_per_s=M / ((rot_ms + gemm_ms) * 1e-3))
    del s, sc, x, xr, y, v, u, ws_lr, ws_pf
    torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on the host cores, bounded sample
# ---------------------------------------------------------------------------

def cpu_baseline(budget_s=12.0):
    import datagen
    import oracle
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        ncores = len(os.sched_getaffinity(0))
        limiter = threadpool_limits(limits=ncores, user_api="blas")
        threads = max([d.get("num_threads", 1) for d in threadpool_info() if d.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        limiter, threads = None, os.cpu_count()
    mats = []
    for which in (0, 1):
        N, K = datagen.C2_SHAPES[which]
        words, scales = oracle.pack_sign1(datagen.C2_weight(which))
        x = oracle.bf16_to_f64(datagen.C2_x(which, 1))
        mats.append((N, K, words, scales, x))
    step_bytes = sum(packed_bytes(N, K) + K * 2 + N * 2 for N, K, _, _, _ in mats)
    steps = 0
    t0 = time.perf_counter()
    while True:
        for N, K, words, scales, x in mats:
            oracle.bin_gemm(x, words, scales, N, K)
        steps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    if limiter is not None:
        limiter.unregister() if hasattr(limiter, "unregister") else None
    # the same on one BLAS thread, a shorter sample
    one = None
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1, user_api="blas"):
            n1, t1 = 0, time.perf_counter()
            while time.perf_counter() - t1 < budget_s / 3:
                for N, K, words, scales, x in mats:
                    oracle.bin_gemm(x, words, scales, N, K)
                n1 += 1
            one = step_bytes * n1 / (time.perf_counter() - t1) / 1e9
    except Exception:  # pragma: no cover
        pass
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:  # pragma: no cover
        pass
    return dict(value=step_bytes * steps / el / 1e9, unit="GB/s", cores=int(threads), kind="oracle",
                sample=f"{steps} steps of the headline workload (both C2 matrices at M=1, fp64 numpy "
                       f"dequantise + matmul) in {el:.1f} s",
                one_thread_value=one, cpu_model=model)


# ---------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run plain 512 MiB device copies (counter calibration) and exit")
    ap.add_argument("--only", choices=["prefill", "decode64", "moe1", "dbf1", "q8", "fusion"],
                    help="run one extra section alone and print its result (for profiling runs)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (the library has no multi-GPU path); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import binary_weight_gemm_amd as brq
    brq.lib()
    torch.cuda.set_device(0)
    if args.copy_calibration:
        print(json.dumps(copy_calibration(torch)))
        return
    if args.only:
        sections = {
            "prefill": lambda: run_prefill(brq, torch),
            "decode64": lambda: run_c2(brq, torch, 64, 50, 10),
            "moe1": lambda: run_moe(brq, torch, (1,)),
            "dbf1": lambda: run_dbf(brq, torch, (1,)),
            "q8": lambda: run_dbf(brq, torch, (512,), q8=True),
            "fusion": lambda: {
                "moe_one_launch": run_moe(brq, torch, (1, 2, 4), fusion=brq.FUSION_ON),
                "moe_multi_launch": run_moe(brq, torch, (1, 2, 4), fusion=brq.FUSION_OFF),
                "dbf_one_launch": run_dbf(brq, torch, (1, 4), fusion=brq.FUSION_ON),
                "dbf_multi_launch": run_dbf(brq, torch, (1, 4), fusion=brq.FUSION_OFF)},
        }
        print(json.dumps({args.only: sections[args.only]()}, default=float))
        return

    log("[bench] headline C2 decode M=1")
    head = run_c2(brq, torch, 1, args.steps, args.warmup)
    log(f"[bench] headline {head}")
    extra = {}
    if not args.no_extra:
        extra["device"] = device_facts(torch)
        log("[bench] achievable peaks")
        extra["achievable"] = achievable_peaks(torch)
        log("[bench] reference kernels")
        extra["reference_kernels"] = reference_kernels(torch, brq)
        log("[bench] C1")
        extra["c1"] = run_c1(brq, torch)
        extra["isolated_decode_call_us"] = isolated_call_us(brq, torch)
        extra["c2"] = {}
        for M in (4, 16, 64):
            log(f"[bench] C2 M={M}")
            r = run_c2(brq, torch, M, 50, 10)
            extra["c2"][f"M={M}"] = {k: r[k] for k in ("ms_per_step", "gbs", "tflops")}
        log("[bench] pack")
        extra["pack"] = run_pack(brq, torch)
        log("[bench] MoE")
        extra["moe"] = run_moe(brq, torch, (1, 4, 16, 64))
        log("[bench] single-launch decode chains: MoE T = 1, 2, 4 and DBF M = 1, 4, one launch and multi-launch")
        extra["decode_fusion"] = {
            "moe_one_launch": run_moe(brq, torch, (1, 2, 4), fusion=brq.FUSION_ON),
            "moe_multi_launch": run_moe(brq, torch, (1, 2, 4), fusion=brq.FUSION_OFF),
            "dbf_one_launch": run_dbf(brq, torch, (1, 4), fusion=brq.FUSION_ON),
            "dbf_multi_launch": run_dbf(brq, torch, (1, 4), fusion=brq.FUSION_OFF),
        }
        log("[bench] MoE with DBF experts")
        extra["moe_dbf"] = run_moe_dbf(brq, torch, (1, 64))
        log("[bench] MoE with DBF experts, DeepSeek-V4-Flash geometry")
        extra["moe_dbf_deepseek_v4_flash"] = run_moe_dbf(brq, torch, (1, 4), geometry="DeepSeek-V4-Flash")
        log("[bench] DBF")
        extra["dbf"] = run_dbf(brq, torch, (1, 512))
        log("[bench] DBF, r = 4096")
        extra["dbf_r4096"] = run_dbf(brq, torch, (1, 512), r=4096)
        log("[bench] DBF over Q8 activation codes")
        extra["dbf_q8"] = run_dbf(brq, torch, (512, 4096), q8=True)
        log("[bench] prefill")
        extra["prefill"] = run_prefill(brq, torch)
    cpu = None
    if not args.no_cpu:
        log("[bench] cpu baseline")
        cpu = cpu_baseline()

    achieved = head["launch_gbs"]
    out = {
        "metric": METRIC,
        "value": round(head["gbs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8xfp4",
        "data": "synthetic",
        "config": {
            "workload": "decode binary GEMV: W 4096x14336 and 14336x4096 group-128 sign + fp16 scale, "
                        "x bf16 M=1, y bf16; one step = both matrices",
            "M": 1, "shapes_NxK": [[4096, 14336], [14336, 4096]], "ring_copies": head["ring_copies"],
            "step_bytes": head["step_bytes"],
        },
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": recorded_traffic(),
            "kernel": "k_gemm_dec (brq_gemm, M=1): one launch per matrix; HIP-graph replay of the timed steps, "
                      "HIP events around each replay, time / launches",
            "launch_us": round(head["launch_ms"] * 1e3, 3),
        },
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
