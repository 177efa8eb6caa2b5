"""CPU pins of the backward oracle of the routed path.

The backward is the chain rule applied to the forward the pages define
(lamjinlab.com section 2, ranhao.site section 2.2), so it is pinned against
things that do not share its formulas:
  * central finite differences of the (separately pinned) forward oracle on
    tiny inputs with drops, for z, the logits and every expert weight;
  * torch.autograd on the CPU in float64, differentiating the same SwiGLU;
  * closed forms: a token's logit gradient sums to zero (softmax is shift
    invariant), k = 1 gives zero, a dropped assignment gets nothing, one row
    gives rank-one weight gradients.
"""
import numpy as np
import pytest
import torch

import oracle


def _tiny(seed, T=10, L=6, F=5, E=6, P=3, k=2, W=2, cap_send=3, cap_recv=2):
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((T, L))
    wg = rng.standard_normal((E, F, L)) / np.sqrt(L)
    wu = rng.standard_normal((E, F, L)) / np.sqrt(L)
    wd = rng.standard_normal((E, L, F)) / np.sqrt(F)
    # logits on a 2^-6 grid: fp32-exact, and so are +-2^-10 steps
    logits = np.round(rng.standard_normal((T, E)) * 64) / 64
    bias = np.zeros(E, dtype=np.float32)
    topk = oracle.route_topk(logits.astype(np.float32), bias, k)
    asg = oracle.assign_slots(topk, E, P, W, cap_send, cap_recv)
    dy = rng.standard_normal((T, L))
    return dict(z=z, wg=wg, wu=wu, wd=wd, logits=logits, topk=topk, asg=asg, dy=dy, E=E)


def _loss(c, z=None, logits=None, wg=None, wu=None, wd=None):
    """<dy, y_lat> for a fixed routing (top-k and slots held)."""
    z = c["z"] if z is None else z
    logits = c["logits"] if logits is None else logits
    wg = c["wg"] if wg is None else wg
    wu = c["wu"] if wu is None else wu
    wd = c["wd"] if wd is None else wd
    g = oracle.gates(logits, c["topk"])
    o = oracle.expert_outputs(z, c["topk"], c["asg"]["recv_slot"], lambda e: (wg[e], wu[e], wd[e]))
    return float((c["dy"] * oracle.combine(g, c["asg"]["recv_slot"], o)).sum())


def _grads(c):
    g = oracle.gates(c["logits"], c["topk"])
    return oracle.routed_backward(c["z"], c["topk"], g, c["asg"]["recv_slot"],
                                  lambda e: (c["wg"][e], c["wu"][e], c["wd"][e]), c["dy"], c["E"],
                                  experts=range(c["E"]))


def _fd(f, x, eps):
    out = np.zeros_like(x)
    for i in np.ndindex(x.shape):
        xp = x.copy()
        xm = x.copy()
        xp[i] += eps
        xm[i] -= eps
        out[i] = (f(xp) - f(xm)) / (2 * eps)
    return out


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_dz_matches_finite_differences(seed):
    c = _tiny(seed)
    assert c["asg"]["sender_dropped"] + c["asg"]["receiver_dropped"] > 0  # drops are exercised
    fd = _fd(lambda z: _loss(c, z=z), c["z"], 1e-6)
    np.testing.assert_allclose(_grads(c)["dz"], fd, rtol=1e-6, atol=1e-8)


@pytest.mark.parametrize("seed", [0, 3])
def test_logit_gradient_matches_finite_differences(seed):
    c = _tiny(seed)
    eps = 2.0 ** -10  # exact in fp32 at these magnitudes, so the gate softmax sees it
    fd = _fd(lambda l: _loss(c, logits=l), c["logits"], eps)
    np.testing.assert_allclose(_grads(c)["d_logits"], fd, rtol=1e-4, atol=1e-7)


@pytest.mark.parametrize("which", ["wg", "wu", "wd"])
def test_weight_gradients_match_finite_differences(which):
    c = _tiny(4)
    gr = _grads(c)
    pos = {"wg": 0, "wu": 1, "wd": 2}[which]
    for e in range(c["E"]):
        def f(w_e, e=e):
            w = c[which].copy()
            w[e] = w_e
            return _loss(c, **{which: w})
        fd = _fd(f, c[which][e], 1e-6)
        np.testing.assert_allclose(gr["dw"][e][pos], fd, rtol=1e-6, atol=1e-8)


def test_swiglu_backward_matches_torch_autograd():
    rng = np.random.default_rng(5)
    n, L, F = 7, 9, 11
    u = rng.standard_normal((n, L))
    wg = rng.standard_normal((F, L)) / 3
    wu = rng.standard_normal((F, L)) / 3
    wd = rng.standard_normal((L, F)) / 3
    d_o = rng.standard_normal((n, L))
    tu, tg, tup, td = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (u, wg, wu, wd))
    o = torch.matmul(torch.nn.functional.silu(tu @ tg.T) * (tu @ tup.T), td.T)
    o.backward(torch.tensor(d_o))
    du, dwg, dwu, dwd = oracle.swiglu_backward(u, wg, wu, wd, d_o)
    for mine, ref in ((du, tu), (dwg, tg), (dwu, tup), (dwd, td)):
        np.testing.assert_allclose(mine, ref.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_logit_gradient_closed_forms():
    rng = np.random.default_rng(6)
    g = rng.dirichlet(np.ones(4), size=9)
    dg = rng.standard_normal((9, 4))
    d = oracle.gates_backward(g, dg)
    np.testing.assert_allclose(d.sum(axis=1), 0.0, atol=1e-14)      # shift invariance
    one = oracle.gates_backward(np.ones((5, 1)), rng.standard_normal((5, 1)))
    assert np.all(one == 0.0)                                          # k = 1: the gate is 1
    # equal gates 1/k: d_j = (dg_j - mean dg) / k
    k = 4
    eq = oracle.gates_backward(np.full((3, k), 1.0 / k), dg[:3])
    np.testing.assert_allclose(eq, (dg[:3] - dg[:3].mean(axis=1, keepdims=True)) / k, atol=1e-15)
    full = oracle.scatter_logit_grad(np.array([[2, 0], [1, 3]]), np.array([[1.0, 2.0], [3.0, 4.0]]), 5)
    assert np.array_equal(full, [[2.0, 0, 1.0, 0, 0], [0, 3.0, 0, 4.0, 0]])


def test_dropped_assignments_get_nothing():
    c = _tiny(7)
    gr = _grads(c)
    drop = c["asg"]["recv_slot"] < 0
    assert drop.any()
    assert np.all(gr["d_gates"][drop] == 0) and np.all(gr["d_o"][drop] == 0) and np.all(gr["du"][drop] == 0)
    # an expert that no kept row reached has zero weight gradients
    kept_e = set(c["topk"][~drop].tolist())
    for e in range(c["E"]):
        if e not in kept_e:
            assert all(np.all(x == 0) for x in gr["dw"][e])


def test_single_row_weight_gradients_are_rank_one():
    rng = np.random.default_rng(8)
    L, F = 6, 4
    u = rng.standard_normal((1, L))
    wg, wu, wd = rng.standard_normal((F, L)), rng.standard_normal((F, L)), rng.standard_normal((L, F))
    d_o = rng.standard_normal((1, L))
    _, dwg, dwu, dwd = oracle.swiglu_backward(u, wg, wu, wd, d_o)
    for m in (dwg, dwu, dwd):
        assert np.linalg.matrix_rank(m, tol=1e-10) == 1
    # every row of dW_g and dW_u is a multiple of u
    assert np.linalg.matrix_rank(np.vstack([dwg, u]), tol=1e-10) == 1
    assert np.linalg.matrix_rank(np.vstack([dwu, u]), tol=1e-10) == 1
