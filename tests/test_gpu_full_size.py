"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (one moe_forward call).

Integer results (top-k, slots, counts, id columns, receiver lists) are
compared in full against the oracle's assignment from the same fp32 logits.
Values are compared on samples the fp64 oracle computes one by one: 64+
sampled tokens' z, logits and y (including tokens routed to the sampled
experts), and every kept row of sampled experts: one expert per M-tile count
at the Marin shape, the most loaded experts (multi-band tile order) at the
Zipf-skewed one.
"""
import numpy as np
import pytest
import torch

import oracle
import routing_capacity_dispatch_amd as rcd
import synth
from _util import f64, rowwise_rel_err
from gpu_common import GATE_ATOL, bank_valid, check_untapped, dev, np_f32, np_i, say, tol

pytestmark = pytest.mark.gpu


def _dense_weights(inp):
    out = {k: f64(inp[k]) for k in ("w_latent", "w_router", "w_up_proj", "ws_gate", "ws_up",
                                    "ws_down")}
    out["router_bias"] = inp["router_bias"].cpu().numpy().astype(np.float32)
    return out


def _expert_fn_uncached(inp):
    """Expert weights in fp64, converted on each call (the oracle asks for
    each expert once per call, and hundreds of experts would not fit)."""
    return lambda e: (f64(inp["w_gate"][e]), f64(inp["w_up"][e]), f64(inp["w_down"][e]))


GEMM_TILE_ROWS = 192  # M tile of the routed grouped GEMMs


def _checked_experts(name, rows, rng):
    """Experts whose every kept row is checked.  Zipf-skewed workload: the
    three most loaded (up to 9 M tiles: two bands of the tile order, the
    longest K loops' worth of tiles) and one other; otherwise one expert for
    each M-tile count present."""
    present = np.nonzero(rows > 0)[0]
    if name.startswith("zipf"):
        top = [int(e) for e in np.argsort(-rows, kind="stable")[:3]]
        rest = np.setdiff1d(present, top)
        return top + [int(rng.choice(rest))]
    tiles = -(-rows // GEMM_TILE_ROWS)
    return [int(rng.choice(np.nonzero(tiles == m)[0])) for m in np.unique(tiles[present])]


@pytest.mark.parametrize("name", ["marin_16k", "zipf_64k"])
def test_forward_full_size_sampled(name):
    d = dev()
    w = synth.workload(name)
    say("full-size forward", name)
    inp = synth.make_inputs(w, 0, device=d)
    weights = {k: v for k, v in inp.items() if k != "x"}
    cfg = rcd.config_of(w)
    y, counts, taps = rcd.forward(cfg, weights, inp["x"], taps=True)
    check_untapped(rcd.forward, cfg, weights, inp["x"], y)
    torch.cuda.synchronize()
    say("oracle", name)
    rng = np.random.default_rng(0)
    # sampled experts (chosen from the GPU's receiver counts, which are
    # checked against the oracle in full below) and 64+ sampled tokens:
    # 64 at random and 4 routed to (and kept by) each sampled expert
    kept_rows = np_i(taps["expert_count"]).sum(axis=0)
    experts = _checked_experts(name, kept_rows, rng)
    say("checked experts", name, [(e, int(kept_rows[e])) for e in experts])
    gtopk, grecv = np_i(taps["topk_idx"]), np_i(taps["recv_slot"])
    pick = set(rng.choice(w.T, 64, replace=False).tolist())
    for e in experts:
        cand = np.unique(np.nonzero((gtopk == e) & (grecv >= 0))[0])
        pick.update(rng.choice(cand, min(4, len(cand)), replace=False).tolist())
    toks = np.array(sorted(pick))
    assert len(toks) >= 64
    wt = _dense_weights(inp)
    wt["expert_weights"] = _expert_fn_uncached(inp)
    logits32 = np_f32(taps["logits"])
    ref = oracle.forward(np_f32(inp["x"]), wt, top_k=w.top_k, n_pools=w.n_pools,
                         n_waves=w.n_waves, routing_logits32=logits32, tokens=toks)
    t = tol(w.dtype)
    # whole-run integer results
    assert np.array_equal(np_i(taps["topk_idx"]), ref["topk_idx"])
    assert np.abs(np_f32(taps["gates"]) - ref["gates"]).max() <= GATE_ATOL
    a = ref["assignment"]
    assert np.array_equal(np_i(taps["pool_slot"]), a["pool_slot"])
    assert np.array_equal(np_i(taps["recv_slot"]), a["recv_slot"])
    assert np.array_equal(np_i(taps["pool_count"]), a["pool_count"])
    ec = np_i(taps["expert_count"])
    assert np.array_equal(ec, a["expert_count"])
    assert np.array_equal(bank_valid(np_i(taps["bank_rows"]), ec), a["bank_rows"])
    rows, ids = rcd.pool_views(cfg, taps["pools"])
    assert np.array_equal(np_i(ids), a["ids"])
    assert np_i(counts).tolist() == [a["kept"], a["sender_dropped"], a["receiver_dropped"]]
    fr = oracle.drop_fractions(a, w.T, w.top_k)
    say("drop fractions", name, fr)
    # sampled values
    tt = torch.from_numpy(toks).to(d)
    assert rowwise_rel_err(f64(taps["z"][tt]), ref["z"]) <= t
    assert rowwise_rel_err(logits32[toks].astype(np.float64), ref["logits"]) <= t
    assert rowwise_rel_err(f64(taps["y_latent"][tt]), ref["y_latent"]) <= t
    err = rowwise_rel_err(f64(y[tt]), ref["y"])
    say("y rel err", name, err)
    assert err <= t
    # every kept row of sampled experts, from the GPU's own z rows (bf16)
    view = rcd.expert_out_view(cfg, taps["expert_out"])
    Tw = -(-w.T // w.n_waves)
    epp = w.n_experts // w.n_pools
    topk = ref["topk_idx"]
    for e in experts:
        ti, ji = np.nonzero((topk == e) & (a["recv_slot"] >= 0))
        assert len(ti) == kept_rows[e]
        zr = f64(taps["z"][torch.from_numpy(ti).to(d)])
        o = oracle.swiglu(zr, *_expert_fn_uncached(inp)(int(e)))
        got = view[torch.from_numpy(ti // Tw).to(d), int(e) // epp,
                   torch.from_numpy(a["pool_slot"][ti, ji]).to(d)]
        assert rowwise_rel_err(f64(got), o) <= t


def test_recv_share_sampled():
    """One EP rank's receive side: 6 local experts, 3 wave slabs of 33,497
    rows, 65,536 tokens x 8 returning rows; grouped SwiGLU then combine."""
    d = dev()
    say("recv share")
    sh = synth.make_recv_share(seed=0, device=d)
    W, n_local, cw, L, F, T, k = (sh[x] for x in ("W", "n_local", "cap_wave", "L", "F", "T", "k"))
    cfg = rcd.make_config(T, 64, L, n_local, 1, k, F, n_waves=W, dtype="bf16",
                          cap_send_rows=n_local * cw, cap_recv_rows=cw)
    p = rcd.plan(cfg)
    pools = torch.empty(p["pools_bytes"], dtype=torch.uint8, device=d)
    rows, ids = rcd.pool_views(cfg, pools)
    rows[:, 0].copy_(sh["rows"])
    counts = sh["counts"]
    slot = torch.arange(n_local * cw, dtype=torch.int32)
    ids_host = torch.where((slot % cw)[None, :] < counts.repeat_interleave(cw, dim=1),
                           (slot // cw)[None, :].expand(W, -1), torch.full_like(slot, -1)[None, :])
    ids[:, 0].copy_(ids_host.to(d))
    bank_rows = (torch.arange(n_local, dtype=torch.int32)[:, None] * cw
                 + torch.arange(cw, dtype=torch.int32)[None, :]).expand(W, -1, -1).contiguous()
    eo = rcd.experts(cfg, pools, bank_rows.to(d), counts.to(d), sh["w_gate"], sh["w_up"],
                     sh["w_down"])
    rs = (sh["slot_of"] % cw).to(torch.int32)
    y = rcd.combine(cfg, eo, sh["expert_of"].to(d), sh["slot_of"].to(d), rs.to(d),
                    sh["gates"].to(d))
    torch.cuda.synchronize()
    say("oracle recv share")
    rng = np.random.default_rng(1)
    toks = np.sort(rng.choice(T, 64, replace=False))
    Tw = sh["Tw"]
    need = {}
    for t in toks:
        for j in range(k):
            e = int(sh["expert_of"][t, j])
            need.setdefault(e, set()).add((int(t // Tw), int(sh["slot_of"][t, j])))
    ew_cache = {}

    def ew(e):
        if e not in ew_cache:
            ew_cache[e] = (f64(sh["w_gate"][e]), f64(sh["w_up"][e]), f64(sh["w_down"][e]))
        return ew_cache[e]
    br = bank_rows.numpy()
    cn = counts.numpy()
    rows_host = {}
    for (wv, s) in {x for v in need.values() for x in v}:
        rows_host[(wv, s)] = f64(sh["rows"][wv, s])
    outs = {}
    for e, want in need.items():
        got = oracle.bank_expert_rows(
            {wv: {s: rows_host[(wv, s)] for (ww, s) in want if ww == wv} for wv in range(W)},
            br, cn, ew, [e], row_filter=lambda wv, s, want=want: (wv, s) in want)
        outs.update(got)
    o = np.stack([[outs[(int(t // Tw), int(sh["slot_of"][t, j]))] for j in range(k)] for t in toks])
    want = oracle.combine(f64(sh["gates"][torch.from_numpy(toks)]), np.zeros((len(toks), k)), o)
    err = rowwise_rel_err(f64(y[torch.from_numpy(toks).to(d)]), want)
    say("recv share y rel err", err)
    assert err <= 2e-2
    # expert_out rows of a few bank slots, directly
    view = rcd.expert_out_view(cfg, eo)
    for (wv, s) in list(rows_host)[:8]:
        e = s // cw
        assert rowwise_rel_err(f64(view[wv, 0, s])[None], outs[(wv, s)][None]) <= 2e-2
