"""GPU parity of the routed-path backward (moe_*_backward, moe_backward_routed)
against the fp64 oracle of oracle/moe_backward.py, on the routing, slots,
rows and saved expert outputs of a GPU forward run (the gradient of that
very forward call: its bf16 o rows are the backward's input, as a training
step saves them).

bf16 bar (2e-2 row-wise relative): dz [T, L], d_logits [T, E] (rows over
experts), d_gates [T, k] and every row of the weight gradients.  The
composition is checked against the four component entry points, bit for
bit, and two runs must agree bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import routing_capacity_dispatch_amd as rcd
import synth
from _util import f64, oracle_weights, rowwise_rel_err
from gpu_common import check_weight_grads, dev, np_f32, np_i, say, tol

pytestmark = pytest.mark.gpu


def _run(w, seed, d):
    cfg = rcd.config_of(w)
    inp = synth.make_inputs(w, seed, device=d)
    weights = {k: v for k, v in inp.items() if k != "x"}
    fwd = rcd.Forward(cfg, weights, d, taps=True)
    fwd(inp["x"])
    dy = synth.grad_latent(w, seed, device=d)
    bwd = rcd.BackwardRouted(fwd)
    dz, d_logits, dw = bwd(dy)
    torch.cuda.synchronize()
    return cfg, inp, fwd, bwd, dy, dz, d_logits, dw


def _saved_o(cfg, fwd, toks=None):
    """The forward's expert outputs o[t, j] (bf16 values, fp64), read from its
    expert_out buffer at each kept assignment's (wave, pool, slot): the saved
    activation the backward takes as input."""
    p, taps = fwd.p, fwd.tap_t
    T, k, L = cfg.T, cfg.top_k, cfg.d_latent
    toks = np.arange(T) if toks is None else np.asarray(toks)
    topk = np_i(taps["topk_idx"])[toks]
    ps = np_i(taps["pool_slot"])[toks]
    keep = np_i(taps["recv_slot"])[toks] >= 0
    if not keep.any():  # nothing kept (e.g. a zero capacity: the buffer may be empty)
        return np.zeros((len(toks), k, L))
    w = toks[:, None] // p["tokens_per_wave"]
    row = (w * cfg.n_pools + topk // (cfg.n_experts // cfg.n_pools)) * p["cap_send"] + np.maximum(ps, 0)
    eo = rcd.expert_out_view(cfg, taps["expert_out"]).reshape(-1, L)
    o = f64(eo[torch.from_numpy(np.where(keep, row, 0).reshape(-1)).to(eo.device)]).reshape(len(toks), k, L)
    return np.where(keep[:, :, None], o, 0.0)


def _oracle(w, inp, fwd, dy, experts=None):
    wt = oracle_weights(inp)
    taps = fwd.tap_t

    def ew(e):
        return wt["w_gate"][e], wt["w_up"][e], wt["w_down"][e]
    topk = np_i(taps["topk_idx"])
    gates = np_f32(taps["gates"]).astype(np.float64)
    recv = np_i(taps["recv_slot"])
    z = f64(taps["z"])
    return oracle.routed_backward(z, topk, gates, recv, ew, f64(dy), w.n_experts,
                                  o=_saved_o(fwd.cfg, fwd), experts=experts), topk, recv


def _check_all(w, seed, d):
    cfg, inp, fwd, bwd, dy, dz, d_logits, dw = _run(w, seed, d)
    ref, topk, recv = _oracle(w, inp, fwd, dy, experts=range(w.n_experts))
    t = tol(w.dtype)
    err = rowwise_rel_err(f64(dz), ref["dz"])
    assert err <= t, ("dz", err)
    err = rowwise_rel_err(np_f32(d_logits).astype(np.float64), ref["d_logits"])
    assert err <= t, ("d_logits", err)
    # unselected experts get exactly zero
    sel = np.zeros((w.T, w.n_experts), dtype=bool)
    np.put_along_axis(sel, topk, True, axis=1)
    assert np.all(np_f32(d_logits)[~sel] == 0)
    check_weight_grads(dw, ref["dw"], np_i(fwd.tap_t["expert_count"]).sum(axis=0), t)
    return cfg, inp, fwd, bwd, dy, ref


@pytest.mark.parametrize("seed", [0, 1])
def test_backward_routed_mid(seed):
    d = dev()
    say("backward mid_bf16", seed)
    _check_all(synth.workload("mid_bf16"), seed, d)


@pytest.mark.parametrize("over", [dict(recv_cap=(1, 2)), dict(send_cap=(1, 2)), dict(n_waves=1),
                                  dict(n_pools=1), dict(top_k=1), dict(top_k=2, T=1000),
                                  # every assignment dropped: zero-size pools (null buffers), zero gradients
                                  dict(send_cap=(0, 1)), dict(recv_cap=(0, 1))])
def test_backward_routed_special_cases(over):
    d = dev()
    say("backward special", over)
    w = synth.workload("mid_bf16", T=2048).replace(**over)
    _check_all(w, 3, d)


@pytest.mark.parametrize("seed", [5, 6, 7, 8, 9, 10])
def test_backward_with_empty_experts_and_ragged_tokens(seed):
    # 77 tokens, top-1 over 64 experts: most experts get no row, and their
    # weight gradients must be written as zeros; the others keep 1-4 rows
    d = dev()
    say("backward empty experts", seed)
    w = synth.workload("mid_bf16", T=77, top_k=1)
    cfg, inp, fwd, bwd, dy, ref = _check_all(w, seed, d)
    ec = np_i(fwd.tap_t["expert_count"]).sum(axis=0)
    assert (ec == 0).any()
    for e in np.nonzero(ec == 0)[0]:
        for g in bwd.dw:
            assert torch.count_nonzero(g[int(e)]) == 0


def test_components_compose_bitwise_and_runs_repeat():
    d = dev()
    w = synth.workload("mid_bf16")
    say("backward components")
    cfg, inp, fwd, bwd, dy, dz, d_logits, dw = _run(w, 2, d)
    dz1, dl1, dw1 = dz.clone(), d_logits.clone(), [g.clone() for g in dw]
    bwd(dy)
    torch.cuda.synchronize()
    assert torch.equal(bwd.dz.view(torch.int16), dz1.view(torch.int16))
    assert torch.equal(bwd.d_logits, dl1)
    for a, b in zip(bwd.dw, dw1):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    t = fwd.tap_t
    dg, deo = rcd.combine_backward(cfg, t["expert_out"], t["topk_idx"], t["pool_slot"], t["recv_slot"],
                                   t["gates"], dy)
    dpr, dwc = rcd.experts_backward(cfg, t["pools"], t["bank_rows"], t["expert_count"], fwd.w["w_gate"],
                                    fwd.w["w_up"], fwd.w["w_down"], deo)
    dzc = rcd.dispatch_backward(cfg, t["topk_idx"], t["pool_slot"], t["recv_slot"], dpr)
    dlc = rcd.route_backward(cfg, t["topk_idx"], t["gates"], dg)
    torch.cuda.synchronize()
    assert torch.equal(dzc.view(torch.int16), dz1.view(torch.int16))
    assert torch.equal(dlc, dl1)
    for a, b in zip(dwc, dw1):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    # d_gates: zero for dropped assignments, the oracle's value otherwise
    ref, topk, recv = _oracle(w, inp, fwd, dy)
    g = np_f32(dg).astype(np.float64)
    assert np.all(g[recv < 0] == 0)
    assert rowwise_rel_err(g, ref["d_gates"]) <= tol(w.dtype)


def test_backward_profiled_matches():
    d = dev()
    w = synth.workload("mid_bf16")
    say("backward profiled")
    cfg, inp, fwd, bwd, dy, dz, d_logits, dw = _run(w, 1, d)
    dz1 = dz.clone()
    n = rcd.backward_stage_count()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    for e in ev:
        e.record()  # torch creates the event handle at its first record
    bwd.profiled(dy, ev)
    torch.cuda.synchronize()
    assert torch.equal(bwd.dz.view(torch.int16), dz1.view(torch.int16))
    ms = [ev[i].elapsed_time(ev[i + 1]) for i in range(n)]
    assert all(m >= 0 for m in ms) and sum(ms) > 0


@pytest.mark.parametrize("name", ["marin_16k", "zipf_64k"])
def test_backward_full_size_sampled(name):
    """At the full workload: dz, d_gates and d_logits of sampled tokens from
    single-row oracle backwards, and the weight gradients of a few experts."""
    d = dev()
    w = synth.workload(name)
    say("backward full size", name)
    cfg, inp, fwd, bwd, dy, dz, d_logits, dw = _run(w, 0, d)
    taps = fwd.tap_t
    topk = np_i(taps["topk_idx"])
    recv = np_i(taps["recv_slot"])
    gates = np_f32(taps["gates"]).astype(np.float64)
    rng = np.random.default_rng(7)
    toks = np.sort(rng.choice(w.T, 24, replace=False))
    z = f64(taps["z"][torch.from_numpy(toks).to(d)])
    dyt = f64(dy[torch.from_numpy(toks).to(d)])
    wg, wu, wd = (bwd.fwd.w[n] for n in ("w_gate", "w_up", "w_down"))
    o_saved = _saved_o(cfg, fwd, toks)
    want_dz = np.zeros_like(z)
    want_dg = np.zeros((len(toks), w.top_k))
    for i, t in enumerate(toks):
        for j in range(w.top_k):
            if recv[t, j] < 0:
                continue
            e = int(topk[t, j])
            W3 = [f64(m[e]) for m in (wg, wu, wd)]
            want_dg[i, j] = dyt[i] @ o_saved[i, j]
            du, _, _, _ = oracle.swiglu_backward(z[i:i + 1], *W3, gates[t, j] * dyt[i:i + 1])
            want_dz[i] += du[0]
    t_ = tol(w.dtype)
    assert rowwise_rel_err(f64(dz[torch.from_numpy(toks).to(d)]), want_dz) <= t_
    want_dl = oracle.scatter_logit_grad(topk[toks], oracle.gates_backward(gates[toks], want_dg), w.n_experts)
    assert rowwise_rel_err(np_f32(d_logits[torch.from_numpy(toks).to(d)]).astype(np.float64), want_dl) <= t_
    # weight gradients of three experts: all their kept rows
    ec = np_i(taps["expert_count"]).sum(axis=0)
    for e in [int(np.argmax(ec)), int(np.argmin(ec)), 7]:
        rows, js = np.nonzero((topk == e) & (recv >= 0))
        if len(rows) == 0:
            for g in bwd.dw:
                assert torch.count_nonzero(g[e]) == 0
            continue
        zr = f64(taps["z"][torch.from_numpy(rows).to(d)])
        d_o = gates[rows, js][:, None] * f64(dy[torch.from_numpy(rows).to(d)])
        _, gg, gu, gd = oracle.swiglu_backward(zr, f64(wg[e]), f64(wu[e]), f64(wd[e]), d_o)
        for got, want in zip(bwd.dw, (gg, gu, gd)):
            assert rowwise_rel_err(f64(got[e]), want) <= t_, e


# ------------------------------------------------------------------ dropless
def _run_dropless(w, seed, d):
    cfg = rcd.config_of(w)
    inp = synth.make_inputs(w, seed, device=d)
    weights = {k: v for k, v in inp.items() if k != "x"}
    fwd = rcd.ForwardDropless(cfg, weights, d, taps=True)
    fwd(inp["x"])
    dy = synth.grad_latent(w, seed, device=d)
    bwd = rcd.BackwardRouted(fwd)
    dz, d_logits, dw = bwd(dy)
    torch.cuda.synchronize()
    return cfg, inp, fwd, bwd, dy, dz, d_logits, dw


def _saved_o_dropless(fwd, toks=None):
    taps = fwd.tap_t
    row_of = np_i(taps["row_of"])
    toks = np.arange(row_of.shape[0]) if toks is None else np.asarray(toks)
    r = row_of[toks]
    o = f64(taps["expert_out"][torch.from_numpy(np.maximum(r, 0).reshape(-1)).to(taps["expert_out"].device)])
    o = o.reshape(len(toks), r.shape[1], -1)
    return np.where((r >= 0)[:, :, None], o, 0.0)


@pytest.mark.parametrize("seed", [0, 1])
def test_backward_dropless_mid(seed):
    d = dev()
    w = synth.workload("mid_bf16")
    say("backward dropless mid_bf16", seed)
    cfg, inp, fwd, bwd, dy, dz, d_logits, dw = _run_dropless(w, seed, d)
    wt = oracle_weights(inp)
    taps = fwd.tap_t
    topk = np_i(taps["topk_idx"])
    keep = np.zeros(topk.shape, dtype=np.int64)   # every assignment kept
    ref = oracle.routed_backward(f64(taps["z"]), topk, np_f32(taps["gates"]).astype(np.float64), keep,
                                 lambda e: (wt["w_gate"][e], wt["w_up"][e], wt["w_down"][e]), f64(dy),
                                 w.n_experts, o=_saved_o_dropless(fwd), experts=range(w.n_experts))
    t = tol(w.dtype)
    assert rowwise_rel_err(f64(dz), ref["dz"]) <= t
    assert rowwise_rel_err(np_f32(d_logits).astype(np.float64), ref["d_logits"]) <= t
    check_weight_grads(dw, ref["dw"], np.bincount(topk.ravel(), minlength=w.n_experts), t)


def test_backward_dropless_components_compose_bitwise():
    d = dev()
    w = synth.workload("mid_bf16", T=1500)
    say("backward dropless components")
    cfg, inp, fwd, bwd, dy, dz, d_logits, dw = _run_dropless(w, 4, d)
    t = fwd.tap_t
    dg, deo = rcd.combine_backward_dropless(cfg, t["expert_out"], t["row_of"], t["gates"], dy)
    dxs, dwc = rcd.experts_backward_dropless(cfg, t["xs"], t["expert_offsets"], fwd.w["w_gate"],
                                             fwd.w["w_up"], fwd.w["w_down"], deo)
    dzc = rcd.dispatch_backward_dropless(cfg, t["row_of"], dxs)
    dlc = rcd.route_backward(cfg, t["topk_idx"], t["gates"], dg)
    torch.cuda.synchronize()
    assert torch.equal(dzc.view(torch.int16), dz.view(torch.int16))
    assert torch.equal(dlc, d_logits)
    for a, b in zip(dwc, dw):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_backward_dropless_full_size_sampled():
    d = dev()
    w = synth.workload("marin_16k")
    say("backward dropless full size")
    cfg, inp, fwd, bwd, dy, dz, d_logits, dw = _run_dropless(w, 0, d)
    taps = fwd.tap_t
    topk = np_i(taps["topk_idx"])
    gates = np_f32(taps["gates"]).astype(np.float64)
    toks = np.sort(np.random.default_rng(8).choice(w.T, 16, replace=False))
    z = f64(taps["z"][torch.from_numpy(toks).to(d)])
    dyt = f64(dy[torch.from_numpy(toks).to(d)])
    o_saved = _saved_o_dropless(fwd, toks)
    wg, wu, wd = (fwd.w[n] for n in ("w_gate", "w_up", "w_down"))
    want_dz = np.zeros_like(z)
    want_dg = np.zeros((len(toks), w.top_k))
    for i, t in enumerate(toks):
        for j in range(w.top_k):
            e = int(topk[t, j])
            W3 = [f64(m[e]) for m in (wg, wu, wd)]
            want_dg[i, j] = dyt[i] @ o_saved[i, j]
            du, _, _, _ = oracle.swiglu_backward(z[i:i + 1], *W3, gates[t, j] * dyt[i:i + 1])
            want_dz[i] += du[0]
    t_ = tol(w.dtype)
    assert rowwise_rel_err(f64(dz[torch.from_numpy(toks).to(d)]), want_dz) <= t_
    want_dl = oracle.scatter_logit_grad(topk[toks], oracle.gates_backward(gates[toks], want_dg), w.n_experts)
    assert rowwise_rel_err(np_f32(d_logits[torch.from_numpy(toks).to(d)]).astype(np.float64), want_dl) <= t_
    e = 11
    rows, js = np.nonzero(topk == e)
    zr = f64(taps["z"][torch.from_numpy(rows).to(d)])
    d_o = gates[rows, js][:, None] * f64(dy[torch.from_numpy(rows).to(d)])
    _, gg, gu, gd = oracle.swiglu_backward(zr, f64(wg[e]), f64(wu[e]), f64(wd[e]), d_o)
    for got, want in zip(dw, (gg, gu, gd)):
        assert rowwise_rel_err(f64(got[e]), want) <= t_
