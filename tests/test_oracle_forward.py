"""Pins of the oracle's dense numerics and of the workload shapes (CPU only)."""
import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as Fn

import oracle
import synth
from _util import f64, oracle_weights

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _small(E=8, P=2, k=2, T=48, D=32, L=16, F=24, S=2, Fs=20, W=3, seed=0, bias="zero"):
    w = synth.Workload("t", T=T, d_model=D, d_latent=L, n_experts=E, n_pools=P,
                       top_k=k, d_ff=F, n_shared=S, d_ff_shared=Fs, n_waves=W,
                       dtype="f32", bias=bias, bias_std=0.5)
    inp = synth.make_inputs(w, seed)
    return w, inp, f64(inp["x"]), oracle_weights(inp)


def _lib_swiglu(u, wg, wu, wd):
    """torch.nn.functional in float64: silu(u Wg^T) * (u Wu^T), then Wd."""
    u, wg, wu, wd = (torch.from_numpy(np.asarray(a, dtype=np.float64)) for a in (u, wg, wu, wd))
    return Fn.linear(Fn.silu(Fn.linear(u, wg)) * Fn.linear(u, wu), wd).numpy()


def test_swiglu_matches_library():
    rng = np.random.default_rng(0)
    u = rng.standard_normal((7, 10))
    wg, wu, wd = rng.standard_normal((6, 10)), rng.standard_normal((6, 10)), rng.standard_normal((10, 6))
    assert np.allclose(oracle.swiglu(u, wg, wu, wd), _lib_swiglu(u, wg, wu, wd), rtol=1e-12, atol=1e-12)
    # silu(0) = 0: a zero gate matrix switches the expert off
    assert (oracle.swiglu(u, 0 * wg, wu, wd) == 0).all()
    # silu closed values
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    assert np.isclose(oracle.silu(np.array([1.0]))[0], 1 / (1 + np.exp(-1)))
    assert oracle.silu(np.array([-1000.0]))[0] == 0.0


def test_single_expert_is_a_dense_mlp_stack():
    """E = k = 1, one pool, no drops: y = W_up(SwiGLU(x W_lat^T)) + shared(x),
    evaluated with torch.nn.functional."""
    w, inp, x, wt = _small(E=1, P=1, k=1, T=40)
    r = oracle.forward(x, wt, top_k=1, n_pools=1, n_waves=3)
    assert r["assignment"]["kept"] == 40 and (r["gates"] == 1).all()
    X = torch.from_numpy(x)
    z = Fn.linear(X, torch.from_numpy(wt["w_latent"]))
    h = _lib_swiglu(z.numpy(), wt["w_gate"][0], wt["w_up"][0], wt["w_down"][0])
    y = Fn.linear(torch.from_numpy(h), torch.from_numpy(wt["w_up_proj"])).numpy()
    for s in range(2):
        y = y + _lib_swiglu(x, wt["ws_gate"][s], wt["ws_up"][s], wt["ws_down"][s])
    assert np.allclose(r["y"], y, rtol=1e-12, atol=1e-12)
    assert np.allclose(r["z"], z.numpy(), rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("seed", range(3))
def test_dropless_equals_dense_per_token_mixture(seed):
    """Caps large enough for every row: the branch equals, token by token,
    sum_j g_j * Expert_{e_j}(z_t) projected up, plus the shared experts."""
    w, inp, x, wt = _small(seed=seed, bias="normal")
    big = w.T * w.top_k
    r = oracle.forward(x, wt, top_k=w.top_k, n_pools=w.n_pools, n_waves=w.n_waves,
                       cap_send_rows=big, cap_recv_rows=big)
    assert r["assignment"]["kept"] == big
    z = Fn.linear(torch.from_numpy(x), torch.from_numpy(wt["w_latent"])).numpy()
    logits = z @ wt["w_router"].T
    s = logits.astype(np.float32) + wt["router_bias"]
    for t in range(w.T):
        order = sorted(range(w.n_experts), key=lambda e: (-float(s[t, e]), e))[:w.top_k]
        sel = np.array([float(np.float32(logits[t, e])) for e in order])
        g = np.exp(sel - sel.max())
        g /= g.sum()
        yl = sum(g[j] * _lib_swiglu(z[t:t + 1], wt["w_gate"][e], wt["w_up"][e], wt["w_down"][e])[0]
                 for j, e in enumerate(order))
        y = yl @ wt["w_up_proj"].T
        for sh in range(w.n_shared):
            y = y + _lib_swiglu(x[t:t + 1], wt["ws_gate"][sh], wt["ws_up"][sh], wt["ws_down"][sh])[0]
        assert np.allclose(r["y"][t], y, rtol=1e-11, atol=1e-11)


def test_zero_sender_capacity_leaves_shared_path():
    w, inp, x, wt = _small()
    r = oracle.forward(x, wt, top_k=w.top_k, n_pools=w.n_pools, n_waves=w.n_waves,
                       send_cap=(0, 1))
    assert r["assignment"]["sender_dropped"] == w.T * w.top_k
    sh = sum(_lib_swiglu(x, wt["ws_gate"][s], wt["ws_up"][s], wt["ws_down"][s]) for s in range(2))
    assert np.allclose(r["y"], sh, rtol=1e-12, atol=1e-12)
    assert (r["y_latent"] == 0).all()


def test_combine_then_project_is_project_then_combine():
    w, inp, x, wt = _small(seed=4, T=60, E=6, P=3, k=3)
    r = oracle.forward(x, wt, top_k=3, n_pools=3, n_waves=3)
    keep = (r["assignment"]["recv_slot"] >= 0)
    assert 0 < keep.sum() < keep.size
    proj = np.einsum("tjl,dl->tjd", r["expert_out"], wt["w_up_proj"])
    alt = np.einsum("tj,tjd->td", r["gates"] * keep, proj)
    assert np.allclose(r["y_latent"] @ wt["w_up_proj"].T, alt, rtol=1e-11, atol=1e-12)


def test_token_subset_matches_full():
    w, inp, x, wt = _small(seed=1, T=64)
    full = oracle.forward(x, wt, top_k=w.top_k, n_pools=w.n_pools, n_waves=w.n_waves)
    toks = np.array([0, 5, 21, 22, 63])
    sub = oracle.forward(x, wt, top_k=w.top_k, n_pools=w.n_pools, n_waves=w.n_waves,
                         routing_logits32=full["logits"].astype(np.float32), tokens=toks)
    assert np.allclose(sub["y"], full["y"][toks], rtol=1e-13, atol=1e-13)
    assert (sub["assignment"]["recv_slot"] == full["assignment"]["recv_slot"]).all()


def test_expert_out_pool_layout_places_rows():
    w, inp, x, wt = _small(seed=2, T=30, E=4, P=2, k=2)
    r = oracle.forward(x, wt, top_k=2, n_pools=2, n_waves=3)
    rows, index = oracle.expert_out_pool_layout(
        r["expert_out"], r["topk_idx"], r["assignment"], 4, 2, 3, r["plan"]["cap_send"])
    a = r["assignment"]
    assert len(rows) == a["kept"]
    for (wv, p, s), v in zip(index, rows):
        e = a["ids"][wv, p, s]
        assert e >= 0 and e // 2 == p
        assert s in a["bank_rows"][wv, e]


def test_marin_shapes_match_the_pages():
    c = json.load(open(os.path.join(GOLD, "page_constants.json")))
    w = synth.workload("marin_16k")
    assert (w.d_model, w.d_latent, w.d_ff, w.n_shared, w.d_ff_shared) == (
        c["d_model"]["value"], c["d_latent"]["value"], c["routed_expert_width"]["value"],
        c["shared_experts"]["value"], c["shared_expert_width"]["value"])
    k8, f, act, four, d = c["active_width_identity"]["value"]
    assert w.top_k * w.d_ff == k8 * f == act == four * w.d_model == four * d
    # the shared experts' share of the active expert compute: 2 x 6144-wide
    # input vs 8 x 3072-wide routed rows, each SwiGLU of width 3072
    shared = w.n_shared * 3 * w.d_model * w.d_ff_shared
    routed = w.top_k * 3 * w.d_latent * w.d_ff
    num, den = c["shared_share_of_active"]["value"]
    assert shared * den == num * (shared + routed)
    # parameter count: the MoE branch of 48 layers accounts for all but a few
    # percent of the 535.3B total (attention and embeddings take the rest)
    per_layer = (w.d_latent * w.d_model + w.n_experts * w.d_latent
                 + w.n_experts * 3 * w.d_latent * w.d_ff + w.d_model * w.d_latent
                 + w.n_shared * 3 * w.d_model * w.d_ff_shared)
    total = per_layer * c["n_layers"]["value"] / 1e9
    assert 0.97 * c["total_params_billion"]["value"] < total < c["total_params_billion"]["value"]
    active = (w.d_latent * w.d_model + w.n_experts * w.d_latent
              + w.top_k * 3 * w.d_latent * w.d_ff + w.d_model * w.d_latent
              + w.n_shared * 3 * w.d_model * w.d_ff_shared) * c["n_layers"]["value"] / 1e9
    assert 0.7 * c["active_params_billion"]["value"] < active < c["active_params_billion"]["value"]


def test_recv_share_generator_is_consistent():
    sh = synth.make_recv_share(seed=0, T=600, n_local=3, d_latent=8, d_ff=8, cap_wave=700)
    W, k = sh["W"], sh["k"]
    for wv in range(W):
        t0, t1 = wv * sh["Tw"], min(sh["T"], (wv + 1) * sh["Tw"])
        ex = sh["expert_of"][t0:t1].reshape(-1).numpy()
        sl = sh["slot_of"][t0:t1].reshape(-1).numpy()
        assert (np.bincount(ex, minlength=3) == sh["counts"][wv].numpy()).all()
        # every used slot exactly once, inside its expert's range
        assert len(set(sl.tolist())) == len(sl)
        assert ((sl // 700) == ex).all()
        assert ((sl % 700) < sh["counts"][wv].numpy()[ex]).all()
    assert np.allclose(sh["gates"].sum(1).numpy(), 1.0, atol=1e-6)
