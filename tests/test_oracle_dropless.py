"""CPU pins of the oracle's dropless ragged variant (lamjinlab.com section 4,
ranhao.site section 3.3: the fallback that keeps every routed assignment).

ragged_order is checked against a brute-force count of what precedes each
assignment; forward_dropless against the capped forward with caps that hold
every row and against the dense per-token mixture."""
import numpy as np
import pytest

import oracle
import synth
from _util import oracle_weights


def _brute_rows(topk, E):
    """row of (t, j) = assignments with a smaller valid expert id, plus earlier
    (t', j') assignments (token-major order) with the same expert."""
    flat = topk.reshape(-1)
    rows = np.full(flat.shape, -1)
    for i, e in enumerate(flat):
        if not 0 <= e < E:
            continue
        smaller = sum(1 for f in flat if 0 <= f < e)
        earlier = sum(1 for f in flat[:i] if f == e)
        rows[i] = smaller + earlier
    return rows.reshape(topk.shape)


@pytest.mark.parametrize("seed,T,E,k", [(0, 7, 5, 2), (1, 13, 9, 3), (2, 1, 4, 4), (3, 20, 16, 1),
                                        (4, 11, 3, 3)])
def test_ragged_order_brute_force(seed, T, E, k):
    rng = np.random.default_rng(seed)
    topk = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    row_of, offsets = oracle.ragged_order(topk, E)
    assert np.array_equal(row_of, _brute_rows(topk, E))
    assert np.array_equal(np.diff(offsets), np.bincount(topk.reshape(-1), minlength=E))
    assert offsets[0] == 0 and offsets[-1] == T * k


def test_ragged_order_is_a_bijection_sorted_by_expert():
    rng = np.random.default_rng(5)
    T, E, k = 300, 40, 6
    topk = np.stack([rng.choice(E, k, replace=False, p=None) for _ in range(T)])
    row_of, offsets = oracle.ragged_order(topk, E)
    flat_rows = row_of.reshape(-1)
    assert np.array_equal(np.sort(flat_rows), np.arange(T * k))
    # rows of expert e are exactly [offsets[e], offsets[e+1]), in token order
    for e in range(E):
        t, j = np.nonzero(topk == e)
        r = row_of[t, j]
        assert np.array_equal(r, np.arange(offsets[e], offsets[e + 1]))


def test_ragged_order_skips_invalid_ids():
    topk = np.array([[0, 5], [7, 1], [-1, 0]])
    row_of, offsets = oracle.ragged_order(topk, 6)
    assert row_of.tolist() == [[0, 3], [-1, 2], [-1, 1]]
    assert offsets.tolist() == [0, 2, 3, 3, 3, 3, 4]


@pytest.mark.parametrize("seed", [0, 1])
def test_forward_dropless_equals_uncapped_forward(seed):
    w = synth.workload("tiny_fp32", T=40)
    inp = synth.make_inputs(w, seed)
    wt = oracle_weights(inp)
    x = inp["x"].numpy().astype(np.float64)
    d = oracle.forward_dropless(x, wt, top_k=w.top_k)
    big = w.T * w.top_k
    c = oracle.forward(x, wt, top_k=w.top_k, n_pools=w.n_pools, n_waves=w.n_waves,
                       cap_send_rows=big, cap_recv_rows=big)
    assert c["assignment"]["sender_dropped"] == 0 and c["assignment"]["receiver_dropped"] == 0
    assert np.array_equal(d["topk_idx"], c["topk_idx"])
    assert np.allclose(d["y"], c["y"], rtol=1e-12, atol=1e-12)


def test_forward_dropless_is_the_dense_mixture():
    """Per token: y = W_up (sum_j g_j SwiGLU_{e_j}(z_t)) + shared(x_t), written
    out without any dispatch."""
    w = synth.workload("tiny_fp32", T=9)
    inp = synth.make_inputs(w, 3)
    wt = oracle_weights(inp)
    x = inp["x"].numpy().astype(np.float64)
    d = oracle.forward_dropless(x, wt, top_k=w.top_k)
    for t in range(w.T):
        z = x[t] @ wt["w_latent"].T
        acc = np.zeros(w.d_latent)
        for j, e in enumerate(d["topk_idx"][t]):
            h = oracle.silu(z @ wt["w_gate"][e].T) * (z @ wt["w_up"][e].T)
            acc += d["gates"][t, j] * (h @ wt["w_down"][e].T)
        y = acc @ wt["w_up_proj"].T
        for s in range(w.n_shared):
            h = oracle.silu(x[t] @ wt["ws_gate"][s].T) * (x[t] @ wt["ws_up"][s].T)
            y += h @ wt["ws_down"][s].T
        assert np.allclose(d["y"][t], y, rtol=1e-10, atol=1e-10)
