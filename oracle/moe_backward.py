"""fp64 CPU oracle for the backward pass of the routed path of one
pooled-wave, capacity-bounded fine-grained MoE branch.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test suite, the smoke check and the benchmark's
CPU-baseline leg use it.  It shares no code with the HIP library.

The pages train this branch ([LJ §2]: the model is trained in the open, with
the routed experts behind the exchange); they print no backward pass, so the
backward here is the plain derivative of the forward they define, written
out step by step with the chain rule:

  forward (per receiver-kept assignment (t, j) of expert e = topk[t, j]):
      u = z[t];  a = u W_g[e]^T;  b = u W_u[e]^T;  h = silu(a) * b
      o[t, j] = h W_d[e]^T
      y_lat[t] = sum over kept j of g[t, j] * o[t, j]
      g[t, :] = softmax of the k selected raw logits
  backward, given dy_lat = dL/dy_lat:
      dg[t, j]  = <dy_lat[t], o[t, j]>                 (kept; 0 if dropped)
      do[t, j]  = g[t, j] * dy_lat[t]                  (kept; 0 if dropped)
      dh        = do W_d[e]                            (W_d is [out=L, in=F])
      dW_d[e]  += do^T h
      da        = dh * b * silu'(a),  db = dh * silu(a)
      silu'(a)  = s (1 + a (1 - s)),  s = 1 / (1 + exp(-a))
      dW_g[e]  += da^T u,  dW_u[e] += db^T u
      du        = da W_g[e] + db W_u[e]
      dz[t]     = sum over kept j of du[t, j]           (the transpose of dispatch)
      dlogit[t, e_j] = g_j (dg_j - sum_i g_i dg_i)     (softmax over the k selected)
  Unselected experts and the balancing bias get no gradient: the selection is
  piecewise constant and the bias enters only the selection ([RH §2.2]).
  Dropped assignments contribute nothing forward, so they get nothing back
  ([LJ §4]: gates are not renormalised).

Citations name the page and its section (see moe_oracle.py for the pages):
  [LJ] lamjinlab.com, §2 (how the sparse model is organised), §4 (dropping);
  [RH] ranhao.site, §2.2 (MoE details).

Pinned by CPU tests against central finite differences of the pinned forward
oracle on tiny inputs, against torch.autograd on the CPU in float64 (a
library differentiation of the same SwiGLU), and against closed forms (the
logit gradient of a token sums to zero; k = 1 gives zero; dropped rows give
zero; one row gives rank-one weight gradients).
"""
from __future__ import annotations

import numpy as np

from .moe_oracle import expert_outputs


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def sigmoid(a):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-a))


# ---------------------------------------------------------------------------
# gate gradients: through the softmax over the k selected raw logits
# ---------------------------------------------------------------------------


def gates_backward(gate_w, d_gates):
    """dL/d(selected logit) from dL/dgate: g_j (dg_j - sum_i g_i dg_i)."""
    g = _f64(gate_w)
    dg = _f64(d_gates)
    return g * (dg - (g * dg).sum(axis=1, keepdims=True))


def scatter_logit_grad(topk_idx, d_sel, n_experts):
    """[T, E] logit gradient: the selected experts' values, 0 elsewhere."""
    topk_idx = np.asarray(topk_idx, dtype=np.int64)
    out = np.zeros((topk_idx.shape[0], n_experts), dtype=np.float64)
    np.put_along_axis(out, topk_idx, _f64(d_sel), axis=1)
    return out


# ---------------------------------------------------------------------------
# the transposes of combine and dispatch
# ---------------------------------------------------------------------------


def combine_backward(gate_w, recv_slot, o, dy_lat):
    """(d_gates [T, k], d_o [T, k, L]) of y_lat = sum_kept g o."""
    keep = (np.asarray(recv_slot) >= 0).astype(np.float64)
    dy = _f64(dy_lat)
    d_gates = np.einsum("tl,tjl->tj", dy, _f64(o)) * keep
    d_o = (_f64(gate_w) * keep)[:, :, None] * dy[:, None, :]
    return d_gates, d_o


def dispatch_backward(recv_slot, du):
    """dz[t] = sum over receiver-kept j of du[t, j]: every kept assignment
    read z[t] once, a dropped one never reached an expert."""
    keep = (np.asarray(recv_slot) >= 0).astype(np.float64)
    return np.einsum("tj,tjl->tl", keep, _f64(du))


# ---------------------------------------------------------------------------
# grouped expert backward: dgrad and wgrad of each expert's SwiGLU
# ---------------------------------------------------------------------------


def swiglu_backward(u, w_gate, w_up, w_down, d_o):
    """Gradients of o = (silu(u W_g^T) * (u W_u^T)) W_d^T for rows u [n, L]
    given d_o [n, L]: returns (du [n, L], dW_g [F, L], dW_u [F, L],
    dW_d [L, F]), the weight gradients in the weights' own [out, in] layout."""
    u = _f64(u)
    wg, wu, wd = _f64(w_gate), _f64(w_up), _f64(w_down)
    d_o = _f64(d_o)
    a = u @ wg.T
    b = u @ wu.T
    s = sigmoid(a)
    silu_a = a * s
    h = silu_a * b
    dw_d = d_o.T @ h
    dh = d_o @ wd
    da = dh * b * s * (1.0 + a * (1.0 - s))
    db = dh * silu_a
    dw_g = da.T @ u
    dw_u = db.T @ u
    du = da @ wg + db @ wu
    return du, dw_g, dw_u, dw_d


def experts_backward(z, topk_idx, recv_slot, expert_weights, d_o, experts=None):
    """du [T, k, L] for every receiver-kept assignment (0 where dropped) and
    {e: (dW_g, dW_u, dW_d)} for the listed experts (default: every expert
    that received a row; an expert without rows has zero gradients)."""
    topk_idx = np.asarray(topk_idx)
    keep = np.asarray(recv_slot) >= 0
    z = _f64(z)
    d_o = _f64(d_o)
    du = np.zeros(d_o.shape, dtype=np.float64)
    present = np.unique(topk_idx[keep])
    wanted = set(int(e) for e in (present if experts is None else experts))
    dw = {}
    for e in sorted(set(int(e) for e in present) | wanted):
        wg, wu, wd = expert_weights(e)
        rows, js = np.nonzero((topk_idx == e) & keep)
        if len(rows) == 0:
            dw[e] = (np.zeros(np.shape(wg)), np.zeros(np.shape(wu)), np.zeros(np.shape(wd)))
            continue
        g_u, g_wg, g_wu, g_wd = swiglu_backward(z[rows], wg, wu, wd, d_o[rows, js])
        du[rows, js] = g_u
        if e in wanted:   # the others' gradients are computed, not kept
            dw[e] = (g_wg, g_wu, g_wd)
    return du, dw


# ---------------------------------------------------------------------------
# the routed path
# ---------------------------------------------------------------------------


def routed_backward(z, topk_idx, gate_w, recv_slot, expert_weights, dy_lat,
                    n_experts, o=None, experts=None):
    """Backward of y_lat(z, logits, W) for a fixed routing.

    z [T, L]; topk_idx, gate_w, recv_slot [T, k]; dy_lat [T, L];
    expert_weights(e) -> (w_gate [F, L], w_up [F, L], w_down [L, F]).
    o: the forward's expert outputs [T, k, L] (recomputed in fp64 if None).
    Returns d_gates [T, k], d_logits [T, E], d_o [T, k, L], du [T, k, L],
    dz [T, L] and dw {e: (dW_g, dW_u, dW_d)} for `experts` (default: all
    experts that received rows).
    """
    if o is None:
        o = expert_outputs(z, topk_idx, recv_slot, expert_weights)
    d_gates, d_o = combine_backward(gate_w, recv_slot, o, dy_lat)
    du, dw = experts_backward(z, topk_idx, recv_slot, expert_weights, d_o, experts)
    dz = dispatch_backward(recv_slot, du)
    d_logits = scatter_logit_grad(topk_idx, gates_backward(gate_w, d_gates), n_experts)
    return dict(d_gates=d_gates, d_logits=d_logits, d_o=d_o, du=du, dz=dz, dw=dw)
