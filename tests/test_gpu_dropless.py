"""GPU parity of the dropless ragged variant (every assignment kept, rows
ordered by expert) against the fp64 oracle, through the C ABI.

row_of, expert_offsets and counts must match bit-exactly; xs rows are bitwise
copies of z rows; values within the row-wise relative tolerance (2e-2 bf16).
"""
import numpy as np
import pytest
import torch

import oracle
import routing_capacity_dispatch_amd as rcd
import synth
from _util import f64, oracle_weights, rowwise_rel_err
from gpu_common import GATE_ATOL, TOL_BF16, check_logits, check_untapped, dev, np_f32, np_i, say

pytestmark = pytest.mark.gpu


# (name, T, E, k, skew, L, F)
DISPATCH_CASES = [
    ("tiny", 256, 16, 2, 0.1, 128, 128),
    ("mid", 4096, 64, 8, 0.01, 512, 512),
    ("marin", 16384, 384, 8, 0.0, 3072, 3072),
    ("one_token", 1, 16, 2, 0.0, 64, 64),
    ("skewed", 333, 12, 3, 2.0, 192, 320),      # empty experts and one large group
    ("k_equals_e", 64, 8, 8, 0.0, 64, 64),
    ("many_experts", 2048, 1024, 16, 0.002, 64, 64),
]


def _case(c, d):
    name, T, E, k, skew, L, F = c
    topk = synth.topk_case(T, E, k, seed=T + 3, skew=skew)
    z = synth.rows_case(T, L, seed=T + 1, dtype="bf16")
    cfg = rcd.make_config(T, 64, L, E, 1, k, F, n_waves=1, dtype="bf16")
    return cfg, topk, z


@pytest.mark.parametrize("case", DISPATCH_CASES, ids=[c[0] for c in DISPATCH_CASES])
def test_dispatch_dropless(case):
    d = dev()
    say("dispatch dropless", case)
    cfg, topk, z = _case(case, d)
    out = rcd.dispatch_dropless(cfg, topk.to(d), z.to(d))
    torch.cuda.synchronize()
    E = case[2]
    row_of, offsets = oracle.ragged_order(topk.numpy(), E)
    assert np.array_equal(np_i(out["row_of"]), row_of)
    assert np.array_equal(np_i(out["expert_offsets"]), offsets)
    assert np_i(out["counts"]).tolist() == [int(offsets[-1]), 0, 0]
    # every row is a bitwise copy of its token's z row
    t_idx, j_idx = np.nonzero(row_of >= 0)
    got = out["xs"][torch.from_numpy(row_of[t_idx, j_idx]).to(d)].cpu()
    assert torch.equal(got.view(torch.int16), z[torch.from_numpy(t_idx)].view(torch.int16))


def test_dispatch_dropless_invalid_ids_and_empty():
    d = dev()
    T, E, k = 64, 16, 2
    topk = synth.topk_case(T, E, k, seed=9)
    topk[3, 1] = 16
    topk[10, 0] = -2
    z = synth.rows_case(T, 64, seed=2, dtype="bf16")
    cfg = rcd.make_config(T, 64, 64, E, 1, k, 64, n_waves=1, dtype="bf16")
    say("dispatch dropless invalid ids")
    out = rcd.dispatch_dropless(cfg, topk.to(d), z.to(d))
    torch.cuda.synchronize()
    row_of, offsets = oracle.ragged_order(topk.numpy(), E)
    assert np.array_equal(np_i(out["row_of"]), row_of)
    assert np_i(out["counts"]).tolist() == [T * k - 2, 2, 0]
    cfg0 = rcd.make_config(0, 64, 64, E, 1, k, 64, n_waves=1, dtype="bf16")
    out0 = rcd.dispatch_dropless(cfg0, torch.empty((0, k), dtype=torch.int32, device=d),
                                 torch.empty((0, 64), dtype=torch.bfloat16, device=d))
    torch.cuda.synchronize()
    assert np_i(out0["expert_offsets"]).tolist() == [0] * (E + 1)
    assert np_i(out0["counts"]).tolist() == [0, 0, 0]


EXPERT_CASES = [
    ("mid", 4096, 64, 8, 0.01, 512, 512),     # ~512 rows per expert: 3 M tiles
    ("skewed", 333, 12, 3, 2.0, 192, 320),    # empty experts, partial feature tile
    ("marin", 16384, 384, 8, 0.0, 3072, 3072),
    ("tall", 16384, 4, 2, 0.0, 256, 256),     # 8192 rows per expert: 256-row expert tiles
]


@pytest.mark.parametrize("case", EXPERT_CASES, ids=[c[0] for c in EXPERT_CASES])
def test_experts_dropless(case):
    d = dev()
    say("experts dropless", case)
    name, T, E, k, skew, L, F = case
    cfg, topk, z = _case(case, d)
    wl = synth.Workload("x", T=T, d_model=64, d_latent=L, n_experts=E, n_pools=1, top_k=k, d_ff=F,
                        n_shared=0, d_ff_shared=64, n_waves=1, dtype="bf16", bias="zero")
    ew = synth.expert_weights(wl, seed=7, device=d)
    dsp = rcd.dispatch_dropless(cfg, topk.to(d), z.to(d))
    eo = rcd.experts_dropless(cfg, dsp["xs"], dsp["expert_offsets"], ew["w_gate"], ew["w_up"],
                              ew["w_down"])
    torch.cuda.synchronize()
    row_of, offsets = oracle.ragged_order(topk.numpy(), E)
    experts = range(E) if E <= 64 else np.random.default_rng(0).choice(E, 10, replace=False)
    zf = f64(z)
    worst = 0.0
    for e in experts:
        t_idx, j_idx = np.nonzero(topk.numpy() == e)
        if not len(t_idx):
            continue
        o = oracle.swiglu(zf[t_idx], f64(ew["w_gate"][e]), f64(ew["w_up"][e]), f64(ew["w_down"][e]))
        got = eo[torch.from_numpy(row_of[t_idx, j_idx]).to(d)]
        worst = max(worst, rowwise_rel_err(f64(got), o))
    assert worst <= TOL_BF16, worst


@pytest.mark.parametrize("T,E,k,L", [(256, 16, 2, 128), (4096, 64, 8, 512), (129, 8, 3, 4096 + 64)])
def test_combine_dropless(T, E, k, L):
    d = dev()
    say("combine dropless", T, E, k, L)
    topk = synth.topk_case(T, E, k, seed=31, skew=0.05)
    row_of, _ = oracle.ragged_order(topk.numpy(), E)
    rows = synth.rows_case(T * k, L, seed=32, dtype="bf16")
    gates = synth.gates_case(T, k, seed=33)
    cfg = rcd.make_config(T, 64, L, E, 1, k, 64, n_waves=1, dtype="bf16")
    ro = torch.from_numpy(row_of.astype(np.int32))
    ro[0, 0] = -1   # an assignment without a row adds nothing
    y = rcd.combine_dropless(cfg, rows.to(d), ro.to(d), gates.to(d))
    torch.cuda.synchronize()
    o = f64(rows[torch.from_numpy(np.maximum(ro.numpy(), 0))])
    keep = (ro.numpy() >= 0).astype(np.int64) - 1   # 0 kept, -1 dropped
    want = oracle.combine(f64(gates), keep, o)
    assert rowwise_rel_err(f64(y), want) <= 5e-3


def _check_forward_dropless(w, seed, d):
    cfg = rcd.config_of(w)
    inp = synth.make_inputs(w, seed, device=d)
    weights = {k: v for k, v in inp.items() if k != "x"}
    y, counts, taps = rcd.forward_dropless(cfg, weights, inp["x"], taps=True)
    torch.cuda.synchronize()
    logits32 = np_f32(taps["logits"])
    ref = oracle.forward_dropless(np_f32(inp["x"]), oracle_weights(inp), top_k=w.top_k,
                                  routing_logits32=logits32)
    assert np.array_equal(np_i(taps["topk_idx"]), ref["topk_idx"])
    assert np.abs(np_f32(taps["gates"]) - ref["gates"]).max() <= GATE_ATOL
    assert np.array_equal(np_i(taps["row_of"]), ref["row_of"])
    assert np.array_equal(np_i(taps["expert_offsets"]), ref["offsets"])
    assert np_i(counts).tolist() == [w.T * w.top_k, 0, 0]
    assert rowwise_rel_err(f64(taps["z"]), ref["z"]) <= TOL_BF16
    check_logits(logits32, f64(taps["z"]), f64(inp["w_router"]), ref["logits"], ref["z"], TOL_BF16)
    assert rowwise_rel_err(f64(taps["y_latent"]), ref["y_latent"]) <= TOL_BF16
    err = rowwise_rel_err(f64(y), ref["y"])
    assert err <= TOL_BF16, err
    check_untapped(rcd.forward_dropless, cfg, weights, inp["x"], y)
    return y


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_forward_dropless_mid(seed):
    d = dev()
    say("forward dropless mid", seed)
    _check_forward_dropless(synth.workload("mid_bf16"), seed, d)


@pytest.mark.parametrize("over", [dict(T=1), dict(T=257), dict(T=1000, n_experts=4, n_pools=1, top_k=1),
                                  dict(T=512, n_shared=0), dict(T=300, top_k=16),
                                  dict(T=8192, n_experts=4, n_pools=4, top_k=2)])  # 256-row expert tiles
def test_forward_dropless_special(over):
    d = dev()
    say("forward dropless special", over)
    _check_forward_dropless(synth.workload("mid_bf16").replace(**over), 4, d)


def test_forward_dropless_empty_and_f32_unsupported():
    d = dev()
    w0 = synth.workload("mid_bf16", T=0)
    inp = synth.make_inputs(w0, 0, device=d)
    y, counts, _ = rcd.forward_dropless(rcd.config_of(w0), {k: v for k, v in inp.items() if k != "x"},
                                        inp["x"])
    torch.cuda.synchronize()
    assert y.shape == (0, w0.d_model) and np_i(counts).tolist() == [0, 0, 0]
    wf = synth.workload("tiny_fp32")
    inp = synth.make_inputs(wf, 0, device=d)
    with pytest.raises(rcd.MoeError) as ex:
        rcd.forward_dropless(rcd.config_of(wf), {k: v for k, v in inp.items() if k != "x"}, inp["x"])
    assert ex.value.status == rcd.abi.MOE_ERR_UNSUPPORTED


def test_forward_dropless_deterministic_and_profiled():
    d = dev()
    w = synth.workload("mid_bf16")
    cfg = rcd.config_of(w)
    inp = synth.make_inputs(w, 1, device=d)
    f = rcd.ForwardDropless(cfg, {k: v for k, v in inp.items() if k != "x"}, d)
    say("forward dropless determinism")
    y1 = f(inp["x"]).clone()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(rcd.dropless_stage_count() + 1)]
    for e in ev:
        e.record()
    y2 = f.profiled(inp["x"], ev).clone()
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert all(ev[i].elapsed_time(ev[i + 1]) >= 0 for i in range(len(ev) - 1))


@pytest.mark.parametrize("name", ["marin_16k", "zipf_64k"])
def test_forward_dropless_full_size_sampled(name):
    """Full-size layers without caps: all integer results in full, values on
    sampled tokens.  Under the Zipf bias the head experts hold thousands of
    rows (many M tiles) and the tail experts few."""
    d = dev()
    w = synth.workload(name)
    say("forward dropless full size", name)
    inp = synth.make_inputs(w, 0, device=d)
    y, counts, taps = rcd.forward_dropless(rcd.config_of(w), {k: v for k, v in inp.items() if k != "x"},
                                           inp["x"], taps=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(2)
    toks = np.sort(rng.choice(w.T, 6, replace=False))
    offs = np_i(taps["expert_offsets"])
    say("largest expert group", int(np.diff(offs).max()), "rows")
    wt = {k: f64(inp[k]) for k in ("w_latent", "w_router", "w_up_proj", "ws_gate", "ws_up", "ws_down")}
    wt["router_bias"] = inp["router_bias"].cpu().numpy().astype(np.float32)
    cache = {}

    def ew(e):
        if e not in cache:
            cache[e] = (f64(inp["w_gate"][e]), f64(inp["w_up"][e]), f64(inp["w_down"][e]))
        return cache[e]
    wt["expert_weights"] = ew
    logits32 = np_f32(taps["logits"])
    ref = oracle.forward_dropless(np_f32(inp["x"]), wt, top_k=w.top_k, routing_logits32=logits32,
                                  tokens=toks)
    assert np.array_equal(np_i(taps["topk_idx"]), ref["topk_idx"])
    assert np.array_equal(np_i(taps["row_of"]), ref["row_of"])
    assert np.array_equal(np_i(taps["expert_offsets"]), ref["offsets"])
    assert np_i(counts).tolist() == [w.T * w.top_k, 0, 0]
    tt = torch.from_numpy(toks).to(d)
    assert rowwise_rel_err(f64(taps["y_latent"][tt]), ref["y_latent"]) <= TOL_BF16
    err = rowwise_rel_err(f64(y[tt]), ref["y"])
    say("dropless y rel err", err)
    assert err <= TOL_BF16
