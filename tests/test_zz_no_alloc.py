"""brq_moe_ffn_noalloc (the MoE layer on the library's own scratch array)
against brq_moe_ffn with a caller-owned workspace: the same kernels, so the
outputs and the routing must be identical bit for bit, on two calls in a row
(the second smaller, through the other launch path), and a size beyond the
scratch array must be refused. Collected last: it runs on a fresh process or
after every other GPU test."""
import sys

import numpy as np
import pytest
import torch

import datagen

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


def test_moe_noalloc_matches_workspace_entry_point():
    import binary_weight_gemm_amd as brq
    cfg = datagen.C4(E=64, H=2048, I=512, top_k=8, layer=81)
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
    w = (gs, gsc, us, usc, ds, dsc)
    for T, dt in ((24, torch.float32), (3, torch.bfloat16)):   # T > 4 path, then the few-token path
        say("moe noalloc", T, dt)
        x = torch.from_numpy(cfg.x(T).view(np.int16)).cuda().view(torch.bfloat16)
        lg = torch.from_numpy(cfg.logits(T, 5)).cuda()
        ref, rid, rw = brq.moe_ffn(x, lg, *w, E, H, I, k, out_dtype=dt, return_routing=True)
        y = torch.full((T, H), float("nan"), dtype=dt, device="cuda")
        ids = torch.full((T, k), -1, dtype=torch.int32, device="cuda")
        wts = torch.full((T, k), float("nan"), dtype=torch.float32, device="cuda")
        brq.moe_ffn_noalloc(x, lg, *w, E, H, I, k, out_dtype=dt, y=y, ids=ids, wts=wts)
        torch.cuda.synchronize()
        assert torch.equal(ids, rid)
        assert torch.equal(wts.view(torch.int32), rw.view(torch.int32))
        assert torch.equal(y.view(torch.int16) if dt == torch.bfloat16 else y.view(torch.int32),
                           ref.view(torch.int16) if dt == torch.bfloat16 else ref.view(torch.int32))


def test_moe_noalloc_refuses_sizes_beyond_the_scratch_array():
    import binary_weight_gemm_amd as brq
    T, H, I, E, k = 256, 4096, 2048, 64, 16
    assert brq.moe_workspace_bytes(T, H, I, E, k) > brq.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((T, H), dtype=torch.bfloat16, device="cuda")
    lg = torch.zeros((T, E), dtype=torch.float32, device="cuda")
    gs = torch.zeros((E * I * H // 64,), dtype=torch.int64, device="cuda")
    gsc = torch.zeros((E * I * H // 128,), dtype=torch.float16, device="cuda")
    with pytest.raises(brq.BrqError, match="BRQ_E_WORKSPACE"):
        brq.moe_ffn_noalloc(x, lg, gs, gsc, gs, gsc, gs, gsc, E, H, I, k)
