"""moe_dispatch_noalloc (the dispatch for callers that cannot allocate) gives
the same results as moe_dispatch, through the C ABI, on two calls in a row
(the second smaller, so it runs on the scratch the first left behind), and
under HIP graph capture."""
import ctypes as C

import numpy as np
import pytest
import torch

import oracle
import routing_capacity_dispatch_amd as rcd
import synth
from routing_capacity_dispatch_amd import abi
from gpu_common import bank_valid, dev, np_i, say

pytestmark = pytest.mark.gpu


def _outputs(cfg, p, d):
    """Output buffers shaped as dispatch() returns them, zero-filled (so the
    slots neither call writes compare equal)."""
    T, k, W, P, E = cfg.T, cfg.top_k, cfg.n_waves, cfg.n_pools, cfg.n_experts
    i32 = dict(dtype=torch.int32, device=d)
    return dict(pools=torch.zeros(p["pools_bytes"], dtype=torch.uint8, device=d),
                pool_slot=torch.zeros((T, k), **i32), recv_slot=torch.zeros((T, k), **i32),
                bank_rows=torch.zeros((W, E, max(p["cap_recv"], 0)), **i32),
                pool_count=torch.zeros((W, P), **i32), expert_count=torch.zeros((W, E), **i32),
                counts=torch.zeros(3, dtype=torch.int64, device=d))


def _with_ws(cfg, p, topk, z, out, d):
    ws = torch.empty(max(p["dispatch_ws_bytes"], 256), dtype=torch.uint8, device=d)
    ptr = lambda t: C.c_void_p(t.data_ptr())
    abi.check("moe_dispatch", rcd.library().moe_dispatch(
        C.byref(cfg), ptr(topk), ptr(z), ptr(out["pools"]), ptr(out["pool_slot"]), ptr(out["recv_slot"]),
        ptr(out["bank_rows"]), ptr(out["pool_count"]), ptr(out["expert_count"]), ptr(out["counts"]),
        ptr(ws), ws.numel(), C.c_void_p(torch.cuda.current_stream(d).cuda_stream)))


# (T, E, P, k, W, L, skew): the Marin-shaped dispatch, then a smaller call
CASES = [(16384, 384, 64, 8, 3, 3072, 0.0), (2500, 384, 64, 8, 3, 3072, 0.3),
         (4096, 64, 16, 8, 3, 512, 0.05), (77, 16, 4, 2, 3, 128, 0.5)]


def test_dispatch_noalloc_matches_dispatch():
    d = dev()
    assert rcd.dispatch_noalloc_scratch_bytes() == 4 << 20
    for T, E, P, k, W, L, skew in CASES:
        say("dispatch noalloc", T, E, P, k, W, L)
        cfg = rcd.make_config(T, 64, L, E, P, k, 64, n_waves=W, dtype="bf16")
        p = rcd.plan(cfg)
        assert 0 < p["dispatch_ws_bytes"] <= rcd.dispatch_noalloc_scratch_bytes()
        topk = synth.topk_case(T, E, k, seed=41, skew=skew).to(d)
        z = synth.rows_case(T, L, seed=42, dtype="bf16").to(d)
        a = _outputs(cfg, p, d)
        b = _outputs(cfg, p, d)
        _with_ws(cfg, p, topk, z, a, d)
        rcd.dispatch_noalloc(cfg, topk, z, b)
        torch.cuda.synchronize()
        for name in a:
            assert torch.equal(a[name], b[name]), (T, name)
        # and the integer results against the oracle
        ref = oracle.assign_slots(topk.cpu().numpy(), E, P, W, p["cap_send"], p["cap_recv"])
        assert np.array_equal(np_i(b["pool_slot"]), ref["pool_slot"])
        assert np.array_equal(np_i(b["recv_slot"]), ref["recv_slot"])
        ec = np_i(b["expert_count"])
        assert np.array_equal(ec, ref["expert_count"])
        assert np.array_equal(bank_valid(np_i(b["bank_rows"]), ec), ref["bank_rows"])
        assert np_i(b["counts"]).tolist() == [ref["kept"], ref["sender_dropped"], ref["receiver_dropped"]]


def test_dispatch_noalloc_under_graph_capture():
    """The callers it is for include code under HIP graph capture: a captured
    moe_dispatch_noalloc replayed on other routings (copied into the
    captured input buffer, eager work and synchronisations between the
    replays) matches moe_dispatch on each, bit for bit."""
    d = dev()
    T, E, P, k, W, L = 4096, 64, 16, 8, 3, 512
    say("dispatch noalloc under graph capture", T, E, P, k, W, L)
    cfg = rcd.make_config(T, 64, L, E, P, k, 64, n_waves=W, dtype="bf16")
    p = rcd.plan(cfg)
    topks = [synth.topk_case(T, E, k, seed=s, skew=0.2).to(d) for s in (51, 52, 53)]
    z = synth.rows_case(T, L, seed=54, dtype="bf16").to(d)
    topk = topks[0].clone()
    b = _outputs(cfg, p, d)
    rcd.dispatch_noalloc(cfg, topk, z, b)  # first call on the device: its scratch address, outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        rcd.dispatch_noalloc(cfg, topk, z, b)
    torch.cuda.synchronize()
    for i, t in enumerate(topks + topks[:1]):
        topk.copy_(t)
        for v in b.values():
            v.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        a = _outputs(cfg, p, d)
        _with_ws(cfg, p, t, z, a, d)
        torch.cuda.synchronize()
        for name in a:
            assert torch.equal(a[name], b[name]), (i, name)
