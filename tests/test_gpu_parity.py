"""GPU parity of every entry point against the fp64 oracle, through the C ABI.

Indices, slots, counts and id columns must match bit-exactly; values within
the row-wise relative tolerance (1e-4 fp32, 2e-2 bf16), gates within 2e-6.
"""
import numpy as np
import pytest
import torch

import oracle
import routing_capacity_dispatch_amd as rcd
import synth
from _util import f64, oracle_weights, rowwise_rel_err
from gpu_common import GATE_ATOL, bank_valid, check_logits, check_untapped, dev, np_f32, np_i, say, tol

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------------ route
ROUTE_CASES = [
    # T, E, k, kind, bias std
    (1, 4, 1, "normal", 0.0),
    (256, 16, 2, "normal", 0.0),
    (256, 16, 2, "ties", 0.0),
    (4096, 64, 8, "normal", 0.01),
    (4096, 64, 8, "ties", 0.25),
    (1000, 100, 5, "tiny", 0.0),        # E not a multiple of 64
    (16384, 384, 8, "normal", 0.0),
    (5000, 384, 8, "ties", 0.0),
    (777, 384, 8, "tiny", 2.0 ** -22),  # selection decided in the last fp32 bits
    (300, 1024, 64, "normal", 0.1),     # largest E and k
    (300, 512, 33, "ties", 0.0),
    (64, 8, 8, "ties", 0.0),            # k == E
]


@pytest.mark.parametrize("T,E,k,kind,bstd", ROUTE_CASES)
def test_route(T, E, k, kind, bstd):
    d = dev()
    say("route", T, E, k, kind, bstd)
    logits = synth.logits_case(T, E, seed=T + E, kind=kind)
    bias = synth.bias_case(E, seed=E, std=bstd) if bstd else None
    cfg = rcd.make_config(T, 64, 64, E, 1, k, 64)
    topk, gates = rcd.route(cfg, logits.to(d), None if bias is None else bias.to(d))
    torch.cuda.synchronize()
    b = np.zeros(E, np.float32) if bias is None else bias.numpy()
    ref = oracle.route_topk(logits.numpy(), b, k)
    assert np.array_equal(np_i(topk), ref)
    g = oracle.gates(logits.numpy(), ref)
    assert np.abs(np_f32(gates) - g).max() <= GATE_ATOL


def test_route_empty():
    d = dev()
    cfg = rcd.make_config(0, 64, 64, 16, 1, 2, 64)
    topk, gates = rcd.route(cfg, torch.empty((0, 16), device=d))
    assert topk.shape == (0, 2)


# ------------------------------------------------------------------ dispatch
# (T, E, P, k, W, L, dtype, skew, send_cap, recv_cap, cap rows)
DISPATCH_CASES = [
    ("tiny", 256, 16, 4, 2, 3, 128, "f32", 0.1, (11, 10), (23, 20), (0, 0)),
    ("mid", 4096, 64, 16, 8, 3, 512, "bf16", 0.01, (11, 10), (23, 20), (0, 0)),
    ("marin", 16384, 384, 64, 8, 3, 3072, "bf16", 0.0, (11, 10), (23, 20), (0, 0)),
    ("marin_skew", 16384, 384, 64, 8, 3, 3072, "bf16", 0.01, (11, 10), (23, 20), (0, 0)),
    ("zipf", 65536, 384, 64, 8, 3, 3072, "bf16", 0.015, (11, 10), (23, 20), (0, 0)),
    ("one_token", 1, 16, 4, 2, 3, 64, "bf16", 0.0, (11, 10), (23, 20), (0, 0)),
    ("ragged_waves", 257, 16, 4, 3, 3, 64, "bf16", 0.2, (11, 10), (23, 20), (0, 0)),
    ("one_wave", 1000, 32, 8, 4, 1, 64, "bf16", 0.1, (11, 10), (23, 20), (0, 0)),
    ("one_pool", 1000, 32, 1, 4, 3, 64, "bf16", 0.1, (11, 10), (23, 20), (0, 0)),
    ("pool_per_expert", 1000, 32, 32, 4, 3, 64, "bf16", 0.1, (11, 10), (23, 20), (0, 0)),
    ("no_sender_cap", 500, 16, 4, 2, 3, 64, "f32", 0.3, (0, 1), (23, 20), (0, 0)),
    ("no_receiver_cap", 500, 16, 4, 2, 3, 64, "f32", 0.3, (11, 10), (0, 1), (0, 0)),
    ("dropless", 500, 16, 4, 2, 3, 64, "f32", 0.3, (11, 10), (23, 20), (4000, 4000)),
    ("many_experts", 2048, 1024, 1024, 16, 2, 64, "bf16", 0.002, (11, 10), (23, 20), (0, 0)),
    ("many_pools", 3000, 256, 128, 6, 5, 128, "bf16", 0.01, (11, 10), (23, 20), (0, 0)),
    ("wide_rows", 300, 16, 4, 2, 3, 8192, "f32", 0.1, (11, 10), (23, 20), (0, 0)),
    # the slot scan works in chunks of 1024 assignments per wave: a wave of
    # exactly one chunk, and waves one token past it (a chunk of 8)
    ("chunk_exact", 384, 64, 16, 8, 3, 64, "bf16", 0.3, (11, 10), (23, 20), (0, 0)),
    ("chunk_plus_one", 387, 64, 16, 8, 3, 64, "bf16", 0.3, (11, 10), (23, 20), (0, 0)),
    ("chunk_mixed", 386, 64, 16, 8, 3, 64, "bf16", 0.3, (11, 10), (23, 20), (0, 0)),  # waves 129, 129, 128
]


def _dispatch_case(case, device):
    name, T, E, P, k, W, L, dt, skew, sc, rc, rows = case
    topk = synth.topk_case(T, E, k, seed=T + 7, skew=skew)
    z = synth.rows_case(T, L, seed=T, dtype=dt)
    cfg = rcd.make_config(T, 64, L, E, P, k, 64, n_waves=W, dtype=dt, send_cap=sc,
                          recv_cap=rc, cap_send_rows=rows[0], cap_recv_rows=rows[1])
    out = rcd.dispatch(cfg, topk.to(device), z.to(device))
    return cfg, topk, z, out


@pytest.mark.parametrize("case", DISPATCH_CASES, ids=[c[0] for c in DISPATCH_CASES])
def test_dispatch(case):
    d = dev()
    say("dispatch", case)
    cfg, topk, z, out = _dispatch_case(case, d)
    torch.cuda.synchronize()
    name, T, E, P, k, W, L, dt = case[:8]
    p = out["plan"]
    ref = oracle.assign_slots(topk.numpy(), E, P, W, p["cap_send"], p["cap_recv"])
    assert np.array_equal(np_i(out["pool_slot"]), ref["pool_slot"])
    assert np.array_equal(np_i(out["recv_slot"]), ref["recv_slot"])
    assert np.array_equal(np_i(out["pool_count"]), ref["pool_count"])
    ec = np_i(out["expert_count"])
    assert np.array_equal(ec, ref["expert_count"])
    assert np.array_equal(bank_valid(np_i(out["bank_rows"]), ec), ref["bank_rows"])
    assert np_i(out["counts"]).tolist() == [ref["kept"], ref["sender_dropped"], ref["receiver_dropped"]]
    rows, ids = rcd.pool_views(cfg, out["pools"])
    assert np.array_equal(np_i(ids), ref["ids"])
    # every occupied slot holds a bitwise copy of its token's row
    ps = ref["pool_slot"]
    t_idx, j_idx = np.nonzero(ps >= 0)
    if len(t_idx):
        Tw = p["tokens_per_wave"]
        w_idx = t_idx // Tw
        p_idx = topk.numpy()[t_idx, j_idx] // (E // P)
        sel = torch.from_numpy(np.stack([w_idx, p_idx, ps[t_idx, j_idx]]))
        got = rows[sel[0].to(d), sel[1].to(d), sel[2].to(d)].cpu()
        want = z[torch.from_numpy(t_idx)]
        assert torch.equal(got.view(torch.int16) if dt == "bf16" else got.view(torch.int32),
                           want.view(torch.int16) if dt == "bf16" else want.view(torch.int32))


def _random_dispatch_cases(n=24, seed=20260):
    """Seeded random shapes for the slot scan: T, E (with P dividing it), k,
    W, the skew of the expert draw and the capacity factors or explicit
    capacities, so that sender and receiver drops fall at random places
    across chunk and wave boundaries."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        E = int(rng.choice([4, 12, 16, 48, 64, 96, 384, 1024]))
        divisors = [d for d in range(1, E + 1) if E % d == 0]
        P = int(rng.choice(divisors))
        k = int(rng.integers(1, min(E, 16) + 1))
        W = int(rng.integers(1, 6))
        T = int(rng.integers(1, 6000))
        skew = float(rng.choice([0.0, 0.01, 0.05, 0.3]))
        sc = (int(rng.integers(0, 16)), 10)
        rc = (int(rng.integers(0, 16)), 10)
        rows = (0, 0) if rng.random() < 0.7 else (int(rng.integers(1, 200)), int(rng.integers(1, 200)))
        cases.append((f"random{i}", T, E, P, k, W, 64, "bf16", skew, sc, rc, rows))
    return cases


@pytest.mark.parametrize("case", _random_dispatch_cases(), ids=lambda c: c[0])
def test_dispatch_random(case):
    d = dev()
    say("dispatch", case)
    cfg, topk, z, out = _dispatch_case(case, d)
    torch.cuda.synchronize()
    name, T, E, P, k, W = case[:6]
    p = out["plan"]
    ref = oracle.assign_slots(topk.numpy(), E, P, W, p["cap_send"], p["cap_recv"])
    assert np.array_equal(np_i(out["pool_slot"]), ref["pool_slot"])
    assert np.array_equal(np_i(out["recv_slot"]), ref["recv_slot"])
    assert np.array_equal(np_i(out["pool_count"]), ref["pool_count"])
    ec = np_i(out["expert_count"])
    assert np.array_equal(ec, ref["expert_count"])
    assert np.array_equal(bank_valid(np_i(out["bank_rows"]), ec), ref["bank_rows"])
    assert np_i(out["counts"]).tolist() == [ref["kept"], ref["sender_dropped"], ref["receiver_dropped"]]
    _, ids = rcd.pool_views(cfg, out["pools"])
    assert np.array_equal(np_i(ids), ref["ids"])


def test_dispatch_out_of_range_ids_are_dropped():
    d = dev()
    T, E, P, k = 64, 16, 4, 2
    topk = synth.topk_case(T, E, k, seed=3)
    topk[5, 1] = 16
    topk[9, 0] = -3
    z = synth.rows_case(T, 64, seed=1, dtype="bf16")
    cfg = rcd.make_config(T, 64, 64, E, P, k, 64, n_waves=1, dtype="bf16")
    say("dispatch out-of-range ids")
    out = rcd.dispatch(cfg, topk.to(d), z.to(d))
    torch.cuda.synchronize()
    c = np_i(out["counts"])
    assert c.sum() == T * k and c[1] >= 2
    assert np_i(out["pool_slot"])[5, 1] == -1 and np_i(out["pool_slot"])[9, 0] == -1


# ------------------------------------------------------------------ experts
EXPERT_CASES = [
    ("tiny_f32", 256, 16, 4, 2, 3, 128, 128, "f32", 0.1),
    ("mid_bf16", 4096, 64, 16, 8, 3, 512, 512, "bf16", 0.01),
    ("ragged", 333, 12, 4, 3, 2, 192, 320, "bf16", 0.2),
    ("marin", 16384, 384, 64, 8, 3, 3072, 3072, "bf16", 0.0),
    # few experts with many rows: 11 M tiles of 192 rows per expert (a band of
    # 8 M tiles, then a partial band of 3) ...
    ("bands", 4096, 2, 1, 1, 1, 256, 256, "bf16", 0.0),
    # ... and 12, 18 and 16 M tiles over three waves, with receiver drops
    ("bands_w3", 9000, 3, 1, 1, 3, 128, 256, "bf16", 0.3),
    # ceil(T k / E) >= 4096 expected rows per expert: the 256-row expert tile
    ("tall", 16384, 4, 1, 2, 1, 256, 256, "bf16", 0.0),
    ("tall_w3", 12288, 3, 1, 1, 3, 128, 256, "bf16", 0.3),
]


@pytest.mark.parametrize("case", EXPERT_CASES, ids=[c[0] for c in EXPERT_CASES])
def test_experts(case):
    d = dev()
    say("experts", case)
    name, T, E, P, k, W, L, F, dt, skew = case
    topk = synth.topk_case(T, E, k, seed=11, skew=skew)
    z = synth.rows_case(T, L, seed=12, dtype=dt)
    wl = synth.Workload("x", T=T, d_model=64, d_latent=L, n_experts=E, n_pools=P, top_k=k,
                        d_ff=F, n_shared=0, d_ff_shared=64, n_waves=W, dtype=dt, bias="zero")
    ew = synth.expert_weights(wl, seed=5, device=d)
    cfg = rcd.make_config(T, 64, L, E, P, k, F, n_waves=W, dtype=dt)
    dsp = rcd.dispatch(cfg, topk.to(d), z.to(d))
    eo = rcd.experts(cfg, dsp["pools"], dsp["bank_rows"], dsp["expert_count"], ew["w_gate"],
                     ew["w_up"], ew["w_down"])
    torch.cuda.synchronize()
    p = dsp["plan"]
    ref = oracle.assign_slots(topk.numpy(), E, P, W, p["cap_send"], p["cap_recv"])
    view = rcd.expert_out_view(cfg, eo)
    # check every kept row of a sample of experts (all experts when small)
    experts = range(E) if E <= 64 else np.random.default_rng(0).choice(E, 12, replace=False)
    Tw = p["tokens_per_wave"]
    zf = f64(z)
    worst = 0.0
    for e in experts:
        t_idx, j_idx = np.nonzero((topk.numpy() == e) & (ref["recv_slot"] >= 0))
        if not len(t_idx):
            continue
        o = oracle.swiglu(zf[t_idx], f64(ew["w_gate"][e]), f64(ew["w_up"][e]), f64(ew["w_down"][e]))
        got = view[torch.from_numpy(t_idx // Tw).to(d), e // (E // P),
                   torch.from_numpy(ref["pool_slot"][t_idx, j_idx]).to(d)]
        worst = max(worst, rowwise_rel_err(f64(got), o))
    assert worst <= tol(dt), worst


@pytest.mark.parametrize("dt,T,E,P,k,W,L,F", [("f32", 256, 16, 4, 2, 3, 128, 128),
                                              ("bf16", 512, 8, 2, 2, 1, 256, 256)])
def test_experts_saturating_preactivations(dt, T, E, P, k, W, L, F):
    """Gate weights scaled by 200, so gate pre-activations reach |a| of several
    hundred: the sigmoid's e^-a overflows to inf (its reciprocal 0, silu(a) a
    signed zero) or underflows to 0 (silu(a) = a), and the experts' outputs
    still match the fp64 SwiGLU row-wise."""
    d = dev()
    say("experts, saturating pre-activations", dt, T, E, P, k, W, L, F)
    topk = synth.topk_case(T, E, k, seed=13, skew=0.0)
    z = synth.rows_case(T, L, seed=14, dtype=dt)
    wl = synth.Workload("x", T=T, d_model=64, d_latent=L, n_experts=E, n_pools=P, top_k=k,
                        d_ff=F, n_shared=0, d_ff_shared=64, n_waves=W, dtype=dt, bias="zero")
    ew = synth.expert_weights(wl, seed=6, device=d)
    ew["w_gate"] = ew["w_gate"] * 200
    cfg = rcd.make_config(T, 64, L, E, P, k, F, n_waves=W, dtype=dt)
    dsp = rcd.dispatch(cfg, topk.to(d), z.to(d))
    eo = rcd.experts(cfg, dsp["pools"], dsp["bank_rows"], dsp["expert_count"], ew["w_gate"],
                     ew["w_up"], ew["w_down"])
    torch.cuda.synchronize()
    p = dsp["plan"]
    ref = oracle.assign_slots(topk.numpy(), E, P, W, p["cap_send"], p["cap_recv"])
    view = rcd.expert_out_view(cfg, eo)
    Tw = p["tokens_per_wave"]
    zf = f64(z)
    worst, saturated = 0.0, 0
    for e in range(E):
        t_idx, j_idx = np.nonzero((topk.numpy() == e) & (ref["recv_slot"] >= 0))
        if not len(t_idx):
            continue
        a = zf[t_idx] @ f64(ew["w_gate"][e]).T
        saturated += int((np.abs(a) > 100).sum())
        o = oracle.swiglu(zf[t_idx], f64(ew["w_gate"][e]), f64(ew["w_up"][e]), f64(ew["w_down"][e]))
        got = f64(view[torch.from_numpy(t_idx // Tw).to(d), e // (E // P),
                       torch.from_numpy(ref["pool_slot"][t_idx, j_idx]).to(d)])
        assert np.isfinite(got).all()
        worst = max(worst, rowwise_rel_err(got, o))
    assert saturated > 1000, saturated  # the case reaches the saturated range
    assert worst <= tol(dt), worst


# ------------------------------------------------------------------ combine
@pytest.mark.parametrize("dt,T,E,P,k,W,L", [("f32", 256, 16, 4, 2, 3, 128),
                                            ("bf16", 4096, 64, 16, 8, 3, 512),
                                            ("bf16", 16384, 384, 64, 8, 3, 3072),
                                            ("bf16", 129, 8, 2, 3, 2, 4096 + 64)])
def test_combine(dt, T, E, P, k, W, L):
    d = dev()
    say("combine", dt, T, E, P, k, W, L)
    topk = synth.topk_case(T, E, k, seed=21, skew=0.05)
    cfg = rcd.make_config(T, 64, L, E, P, k, 64, n_waves=W, dtype=dt)
    p = rcd.plan(cfg)
    nrows = W * P * p["cap_send"]
    eo_rows = synth.rows_case(nrows, L, seed=22, dtype=dt)
    gates = synth.gates_case(T, k, seed=23)
    z = synth.rows_case(T, L, seed=24, dtype=dt)
    dsp = rcd.dispatch(cfg, topk.to(d), z.to(d))
    eo = torch.zeros(p["expert_out_bytes"], dtype=torch.uint8, device=d)
    rcd.expert_out_view(cfg, eo).view(nrows, L).copy_(eo_rows.to(d))
    y = rcd.combine(cfg, eo, topk.to(d), dsp["pool_slot"], dsp["recv_slot"], gates.to(d))
    torch.cuda.synchronize()
    ref = oracle.assign_slots(topk.numpy(), E, P, W, p["cap_send"], p["cap_recv"])
    Tw = p["tokens_per_wave"]
    ts = np.arange(T) if T <= 4096 else np.sort(np.random.default_rng(1).choice(T, 1024, replace=False))
    row = ((ts[:, None] // Tw) * P + topk.numpy()[ts] // (E // P)) * p["cap_send"] \
        + np.maximum(ref["pool_slot"][ts], 0)
    o = f64(eo_rows[torch.from_numpy(row)])
    want = oracle.combine(f64(gates[torch.from_numpy(ts)]), ref["recv_slot"][ts], o)
    # one rounding of the output: 2^-8 relative for bf16
    assert rowwise_rel_err(f64(y[torch.from_numpy(ts).to(d)]), want) <= (5e-3 if dt == "bf16" else 1e-6)


# ------------------------------------------------------------------ forward
FORWARD_CASES = [("tiny_fp32", 0), ("tiny_fp32", 1), ("tiny_fp32", 2),
                 ("mid_bf16", 0), ("mid_bf16", 1), ("mid_bf16", 2)]


def _check_forward(w, seed, d, **over):
    cfg = rcd.config_of(w, **over)
    inp = synth.make_inputs(w, seed, device=d)
    weights = {k: v for k, v in inp.items() if k != "x"}
    y, counts, taps = rcd.forward(cfg, weights, inp["x"], taps=True)
    torch.cuda.synchronize()
    wt = oracle_weights(inp)
    logits32 = np_f32(taps["logits"])
    ref = oracle.forward(np_f32(inp["x"]), wt, top_k=w.top_k, n_pools=w.n_pools,
                         n_waves=w.n_waves, send_cap=w.send_cap, recv_cap=w.recv_cap,
                         cap_send_rows=w.cap_send_rows, cap_recv_rows=w.cap_recv_rows,
                         routing_logits32=logits32)
    t = tol(w.dtype)
    assert rowwise_rel_err(f64(taps["z"]), ref["z"]) <= t
    check_logits(logits32, f64(taps["z"]), wt["w_router"], ref["logits"], ref["z"], t)
    assert np.array_equal(np_i(taps["topk_idx"]), ref["topk_idx"])
    assert np.abs(np_f32(taps["gates"]) - ref["gates"]).max() <= GATE_ATOL
    a = ref["assignment"]
    assert np.array_equal(np_i(taps["pool_slot"]), a["pool_slot"])
    assert np.array_equal(np_i(taps["recv_slot"]), a["recv_slot"])
    assert np.array_equal(np_i(taps["pool_count"]), a["pool_count"])
    ec = np_i(taps["expert_count"])
    assert np.array_equal(ec, a["expert_count"])
    assert np.array_equal(bank_valid(np_i(taps["bank_rows"]), ec), a["bank_rows"])
    assert np_i(counts).tolist() == [a["kept"], a["sender_dropped"], a["receiver_dropped"]]
    assert rowwise_rel_err(f64(taps["y_latent"]), ref["y_latent"]) <= t
    err = rowwise_rel_err(f64(y), ref["y"])
    assert err <= t, err
    check_untapped(rcd.forward, cfg, weights, inp["x"], y)
    return y, ref



@pytest.mark.parametrize("name,seed", FORWARD_CASES)
def test_forward(name, seed):
    d = dev()
    say("forward", name, seed)
    _check_forward(synth.workload(name), seed, d)


@pytest.mark.parametrize("T", [1, 2, 3, 129, 257, 1000])
def test_forward_ragged_token_counts(T):
    d = dev()
    say("forward ragged T", T)
    _check_forward(synth.workload("tiny_fp32", T=T), 3, d)


@pytest.mark.parametrize("over", [dict(n_waves=1), dict(n_pools=1), dict(n_pools=16),
                                  dict(send_cap=(0, 1)), dict(recv_cap=(0, 1)),
                                  dict(cap_send_rows=10 ** 5, cap_recv_rows=10 ** 5),
                                  dict(n_shared=0), dict(n_shared=1), dict(n_shared=3),
                                  dict(top_k=16), dict(top_k=1)])
def test_forward_special_cases(over):
    d = dev()
    say("forward special", over)
    w = synth.workload("tiny_fp32").replace(**over)
    y, ref = _check_forward(w, 4, d)
    a = ref["assignment"]
    if over.get("send_cap") == (0, 1):
        assert a["sender_dropped"] == w.T * w.top_k
    if over.get("recv_cap") == (0, 1):
        assert a["receiver_dropped"] == w.T * w.top_k


def test_forward_bf16_tall_expert_tiles():
    # 8192 tokens x top-2 over 4 experts: 4096 expected rows per expert, so the
    # routed GEMMs run on 256-row tiles
    d = dev()
    say("forward bf16 tall expert tiles")
    _check_forward(synth.workload("mid_bf16").replace(T=8192, n_experts=4, n_pools=4, top_k=2), 5, d)


def test_forward_bf16_single_expert_and_empty():
    d = dev()
    w = synth.workload("mid_bf16", T=512, n_experts=4, n_pools=2, top_k=1)
    say("forward bf16 small E")
    _check_forward(w, 6, d)
    w0 = synth.workload("tiny_fp32", T=0)
    cfg = rcd.config_of(w0)
    inp = synth.make_inputs(w0, 0, device=d)
    y, counts, _ = rcd.forward(cfg, {k: v for k, v in inp.items() if k != "x"}, inp["x"])
    torch.cuda.synchronize()
    assert y.shape == (0, w0.d_model) and np_i(counts).tolist() == [0, 0, 0]


def test_forward_is_deterministic():
    d = dev()
    w = synth.workload("mid_bf16")
    cfg = rcd.config_of(w)
    inp = synth.make_inputs(w, 0, device=d)
    weights = {k: v for k, v in inp.items() if k != "x"}
    say("forward determinism")
    f = rcd.Forward(cfg, weights, d, taps=True)
    y1 = f(inp["x"]).clone()
    t1 = {k: v.clone() for k, v in f.tap_t.items() if k not in ("pools", "expert_out")}
    y2 = f(inp["x"]).clone()
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    for k, v in t1.items():
        a, b = v, f.tap_t[k]
        if a.dtype == torch.bfloat16:
            a, b = a.view(torch.int16), b.view(torch.int16)
        assert torch.equal(a, b), k


def test_forward_profiled_matches_and_times_stages():
    d = dev()
    w = synth.workload("mid_bf16")
    cfg = rcd.config_of(w)
    inp = synth.make_inputs(w, 1, device=d)
    f = rcd.Forward(cfg, {k: v for k, v in inp.items() if k != "x"}, d)
    say("forward profiled")
    y1 = f(inp["x"]).clone()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(rcd.stage_count() + 1)]
    for e in ev:
        e.record()
    y2 = f.profiled(inp["x"], ev).clone()
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    ms = [ev[i].elapsed_time(ev[i + 1]) for i in range(len(ev) - 1)]
    assert all(m >= 0 for m in ms) and sum(ms) > 0
