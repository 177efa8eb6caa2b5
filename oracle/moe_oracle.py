"""fp64 CPU oracle for the forward pass of one pooled-wave, capacity-bounded
fine-grained MoE branch.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test suite, the smoke check and the benchmark's
CPU-baseline leg use it.  It shares no code with the HIP library.

It is deliberately plain: numpy in float64, a Python loop for the slot
assignment, one library matmul per contraction, no blocking or fusion.

Citations name the page and its section:
  [LJ]  lamjinlab.com, "Marin начинает открытое обучение MoE-модели с 535 млрд
        параметров" (Russian; the Korean page is a translation of it),
        §2 "Как организована разреженная модель" (how the sparse model is
        organised), §4 "Длинный контекст зависит от решения проблемы
        отбрасывания токенов" (long context and token dropping).
  [RH]  ranhao.site, "Marin 535B-A23B：一场完全公开的前沿 MoE 训练直播",
        §2.2 "MoE 详解" (MoE details), §3.2 "三 wave 固定 buffer" (three-wave
        fixed buffers), §3.3 "Token dropping".
  [AY]  aoyii.com, "Treinamento aberto do Marin 535B", section "A matemática
        do MoE".

Readings of points the pages leave open (each is also listed with its reason
in the design notes of the repository):
  * the router reads the latent z, not x (the routed path works in latent
    space, [RH §2.2] diagram);
  * gates are a softmax over the k selected raw logits; the balancing bias
    enters only the selection ([RH §2.2]: the bias is a heuristic outside the
    gradient);
  * top-k order is by score descending, ties to the lower expert index;
  * waves are contiguous token chunks of Tw = ceil(T/W) tokens, each with its
    own pools and caps ([LJ §2]: sequential transfers of identical shape;
    [RH §3.2]: the receive buffer is the expected load *in that wave* x 1.15);
  * capacity = ceil(factor x expected load) in exact rational arithmetic;
  * the sender cap is applied first; a receiver-dropped row still occupies
    its pool slot ("either fixed buffer", [LJ §2]);
  * priority is token order, then the rank j inside the token's top-k;
  * expert e lives in pool e div (E/P) (contiguous blocks, [LJ §2]: 384
    experts over 64 GPUs = 6 per destination);
  * dropped assignments contribute zero and the gates are not renormalised;
    the shared experts remain ([LJ §4]);
  * routed and shared experts are SwiGLU without biases; shared experts read
    x at model width and are added without scaling ([LJ §2], [RH §2.2]).
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

# ---------------------------------------------------------------------------
# capacity plan   [LJ §2] sender factor 1.10, receiver factor 1.15;
#                 [RH §3.2] receiver buffer = expected tokens in the wave x 1.15
# ---------------------------------------------------------------------------


def capacity_plan(T, top_k, n_experts, n_pools, n_waves,
                  send_cap=(11, 10), recv_cap=(23, 20),
                  cap_send_rows=0, cap_recv_rows=0):
    """Return dict(Tw, cap_send, cap_recv, experts_per_pool).

    Tw = ceil(T / W) tokens per wave (the static wave size).
    cap_send = ceil(send_factor * Tw * k / P): rows one wave may send to one pool.
    cap_recv = ceil(recv_factor * Tw * k / E): rows one wave may bin to one expert.
    Explicit row counts (non-zero cap_*_rows) replace the derived ones.
    """
    if n_waves < 1 or n_pools < 1 or n_experts < 1 or top_k < 1:
        raise ValueError("bad sizes")
    if n_experts % n_pools:
        raise ValueError("n_experts must be a multiple of n_pools")
    Tw = math.ceil(Fraction(T, n_waves))
    pool_load = Fraction(Tw * top_k, n_pools)      # expected rows per (wave, pool)
    expert_load = Fraction(Tw * top_k, n_experts)  # expected rows per (wave, expert)
    c_send = math.ceil(Fraction(*send_cap) * pool_load)
    c_recv = math.ceil(Fraction(*recv_cap) * expert_load)
    if cap_send_rows:
        c_send = int(cap_send_rows)
    if cap_recv_rows:
        c_recv = int(cap_recv_rows)
    return dict(Tw=Tw, cap_send=c_send, cap_recv=c_recv,
                experts_per_pool=n_experts // n_pools)


def wave_ranges(T, n_waves):
    """Token ranges [t0, t1) of the waves: contiguous chunks of ceil(T/W)."""
    Tw = math.ceil(Fraction(T, n_waves))
    return [(w * Tw, min(T, (w + 1) * Tw)) for w in range(n_waves)]


def pool_of(e, n_experts, n_pools):
    """Destination pool of expert e: contiguous blocks of E/P experts [LJ §2]."""
    return e // (n_experts // n_pools)


# ---------------------------------------------------------------------------
# router   [RH §2.2] top-8 routing with a zero-mean balancing bias that gets no
#          gradient; [LJ §2] eight of 384 routed experts per token
# ---------------------------------------------------------------------------


def selection_scores(logits32, bias32):
    """s[t, e] = fl32(logit[t, e] + bias[e]): one IEEE fp32 add (round to
    nearest even), the precision the selection is decided in."""
    l = np.asarray(logits32, dtype=np.float32)
    b = np.asarray(bias32, dtype=np.float32)
    return (l + b[None, :]).astype(np.float32)


def route_topk(logits32, bias32, top_k):
    """Top-k expert indices per token, ordered by (score desc, index asc).

    Scores compare as real numbers, so -0 and +0 tie and the lower index
    wins.  Inputs must be finite.
    """
    s = selection_scores(logits32, bias32).astype(np.float64)
    T, E = s.shape
    if not 1 <= top_k <= E:
        raise ValueError("top_k out of range")
    idx = np.broadcast_to(np.arange(E), (T, E))
    order = np.lexsort((idx, -s), axis=-1)        # primary key: -s; then e
    return order[:, :top_k].astype(np.int64)


def gates(logits32, topk_idx):
    """Softmax over the k selected *raw* logits (bias excluded), in fp64."""
    l = np.asarray(logits32, dtype=np.float32).astype(np.float64)
    sel = np.take_along_axis(l, np.asarray(topk_idx, dtype=np.int64), axis=1)
    m = sel.max(axis=1, keepdims=True)
    ex = np.exp(sel - m)
    return ex / ex.sum(axis=1, keepdims=True)


# ---------------------------------------------------------------------------
# pooled-wave slot assignment   [LJ §2]: one fixed pool per destination, three
# waves of identical shape, expert id packed with the row, overflow past
# either fixed buffer dropped and counted separately
# ---------------------------------------------------------------------------


def assign_slots(topk_idx, n_experts, n_pools, n_waves, cap_send, cap_recv):
    """Walk each wave's assignments in (token, j) order.

    For assignment (t, j) with expert e in pool p:
      * if pool p already holds cap_send rows this wave: sender drop;
      * else it takes pool slot pc[p] (pc[p] += 1) and the id column of that
        slot records e; then if expert e already holds cap_recv rows this
        wave: receiver drop (the pool slot stays occupied);
      * else it takes receiver slot ec[e] (ec[e] += 1) and the receiver bank
        row list records the pool slot.
    """
    topk_idx = np.asarray(topk_idx, dtype=np.int64)
    T, k = topk_idx.shape
    E, P, W = n_experts, n_pools, n_waves
    epp = E // P
    pool_slot = np.full((T, k), -1, dtype=np.int64)
    recv_slot = np.full((T, k), -1, dtype=np.int64)
    pool_count = np.zeros((W, P), dtype=np.int64)
    expert_count = np.zeros((W, E), dtype=np.int64)
    bank_rows = np.full((W, E, max(cap_recv, 0)), -1, dtype=np.int64)
    ids = np.full((W, P, max(cap_send, 0)), -1, dtype=np.int64)
    sender_dropped = 0
    receiver_dropped = 0
    for w, (t0, t1) in enumerate(wave_ranges(T, W)):
        pc = [0] * P
        ec = [0] * E
        for t in range(t0, t1):
            for j in range(k):
                e = int(topk_idx[t, j])
                p = e // epp
                if pc[p] >= cap_send:
                    sender_dropped += 1
                    continue
                s = pc[p]
                pc[p] += 1
                pool_slot[t, j] = s
                ids[w, p, s] = e
                if ec[e] >= cap_recv:
                    receiver_dropped += 1
                    continue
                r = ec[e]
                ec[e] += 1
                recv_slot[t, j] = r
                bank_rows[w, e, r] = s
        pool_count[w] = pc
        expert_count[w] = ec
    kept = int((recv_slot >= 0).sum())
    return dict(pool_slot=pool_slot, recv_slot=recv_slot,
                pool_count=pool_count, expert_count=expert_count,
                bank_rows=bank_rows, ids=ids, kept=kept,
                sender_dropped=sender_dropped,
                receiver_dropped=receiver_dropped)


def drop_fractions(assignment, T, top_k):
    """Sender, receiver and total drop fractions over the T*k assignments
    ([RH §3.3]: both ends are tracked separately)."""
    n = T * top_k
    sd = assignment["sender_dropped"]
    rd = assignment["receiver_dropped"]
    return dict(sender=sd / n, receiver=rd / n, total=(sd + rd) / n)


# ---------------------------------------------------------------------------
# expert compute   SwiGLU without biases ([RH §2.2] names dense SwiGLU for the
#                  shared experts; the routed experts take the same form)
# ---------------------------------------------------------------------------


def silu(a):
    with np.errstate(over="ignore"):
        return a / (1.0 + np.exp(-a))


def swiglu(u, w_gate, w_up, w_down):
    """(silu(u W_g^T) * (u W_u^T)) W_d^T for u [n, in]; weights [out, in]."""
    u = np.asarray(u, dtype=np.float64)
    g = u @ np.asarray(w_gate, dtype=np.float64).T
    v = u @ np.asarray(w_up, dtype=np.float64).T
    return (silu(g) * v) @ np.asarray(w_down, dtype=np.float64).T


def expert_outputs(z, topk_idx, recv_slot, expert_weights, tokens=None):
    """o[i, j, :] = SwiGLU_e(z[t]) for each receiver-kept assignment (t, j)
    of the listed tokens (all tokens by default); zero where dropped.

    expert_weights(e) -> (w_gate [F, L], w_up [F, L], w_down [L, F]).
    z holds the rows of the listed tokens, in that order.
    """
    topk_idx = np.asarray(topk_idx)
    recv_slot = np.asarray(recv_slot)
    toks = np.arange(topk_idx.shape[0]) if tokens is None else np.asarray(tokens)
    sub_idx = topk_idx[toks]
    sub_keep = recv_slot[toks] >= 0
    z = np.asarray(z, dtype=np.float64)
    out = np.zeros(sub_idx.shape + (z.shape[1],), dtype=np.float64)
    for e in np.unique(sub_idx[sub_keep]):
        rows, js = np.nonzero((sub_idx == e) & sub_keep)
        wg, wu, wd = expert_weights(int(e))
        out[rows, js] = swiglu(z[rows], wg, wu, wd)
    return out


def combine(gate_w, recv_slot, o):
    """y_lat[t] = sum over receiver-kept j of g[t, j] * o[t, j]; dropped
    assignments add nothing and the gates are not renormalised ([LJ §4])."""
    keep = (np.asarray(recv_slot) >= 0).astype(np.float64)
    return np.einsum("tj,tjl->tl", np.asarray(gate_w, dtype=np.float64) * keep, o)


def shared_experts(x, ws_gate, ws_up, ws_down):
    """Sum over the always-on shared experts of SwiGLU_s(x) at model width."""
    x = np.asarray(x, dtype=np.float64)
    y = np.zeros((x.shape[0], np.asarray(ws_down).shape[1]), dtype=np.float64)
    for s in range(np.asarray(ws_gate).shape[0]):
        y += swiglu(x, ws_gate[s], ws_up[s], ws_down[s])
    return y


# ---------------------------------------------------------------------------
# the whole branch
# ---------------------------------------------------------------------------


def latent(x, w_latent):
    """z = x W_lat^T: the 6144 -> 3072 compression before the exchange [LJ §2]."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(w_latent, dtype=np.float64).T


def router_logits(z, w_router):
    """logits = z W_r^T (fp64)."""
    return np.asarray(z, dtype=np.float64) @ np.asarray(w_router, dtype=np.float64).T


def up_project(y_lat, w_up_proj):
    """Back to model width, 3072 -> 6144, before the merge with the shared
    path [LJ §2]."""
    return np.asarray(y_lat, dtype=np.float64) @ np.asarray(w_up_proj, dtype=np.float64).T


def forward(x, w, *, top_k, n_pools, n_waves, send_cap=(11, 10),
            recv_cap=(23, 20), cap_send_rows=0, cap_recv_rows=0,
            routing_logits32=None, tokens=None):
    """Forward pass of the branch.

    x [T, D]; w: dict with w_latent [L, D], w_router [E, L], router_bias [E]
    (fp32), w_gate/w_up [E, F, L], w_down [E, L, F], w_up_proj [D, L],
    ws_gate/ws_up [S, Fs, D], ws_down [S, D, Fs]; any of the expert tensors
    may instead be given as expert_weights(e) -> (w_gate, w_up, w_down).

    Routing uses routing_logits32 if given (the fp32 logits of the run being
    checked), else fl32 of the fp64 logits.  `tokens` restricts the dense
    numerics (z, logits, y) to a subset of tokens; routing and slot
    assignment always cover all T tokens and then need routing_logits32.
    """
    x = np.asarray(x)
    T = x.shape[0]
    E = np.asarray(w["w_router"]).shape[0]
    toks = np.arange(T) if tokens is None else np.asarray(tokens)
    z = latent(x[toks], w["w_latent"])
    logits = router_logits(z, w["w_router"])
    if routing_logits32 is None:
        if tokens is not None:
            raise ValueError("a token subset needs the full routing logits")
        routing_logits32 = logits.astype(np.float32)
    topk_idx = route_topk(routing_logits32, w["router_bias"], top_k)
    g = gates(routing_logits32, topk_idx)
    plan = capacity_plan(T, top_k, E, n_pools, n_waves, send_cap, recv_cap,
                         cap_send_rows, cap_recv_rows)
    asg = assign_slots(topk_idx, E, n_pools, n_waves, plan["cap_send"],
                       plan["cap_recv"])
    ew = w.get("expert_weights")
    if ew is None:
        def ew(e):
            return w["w_gate"][e], w["w_up"][e], w["w_down"][e]
    o = expert_outputs(z, topk_idx, asg["recv_slot"], ew, tokens=toks)
    y_lat = combine(g[toks], asg["recv_slot"][toks], o)
    y = up_project(y_lat, w["w_up_proj"]) + shared_experts(
        x[toks], w["ws_gate"], w["ws_up"], w["ws_down"])
    return dict(plan=plan, z=z, logits=logits, topk_idx=topk_idx, gates=g,
                assignment=asg, expert_out=o, y_latent=y_lat, y=y,
                tokens=toks)


def expert_out_pool_layout(o, topk_idx, assignment, n_experts, n_pools,
                           n_waves, cap_send, tokens=None):
    """Place per-assignment expert outputs at their (wave, pool, slot) rows.

    Returns (rows [n, L], index [n, 3]) for every receiver-kept assignment of
    the listed tokens: index = (w, p, s)."""
    topk_idx = np.asarray(topk_idx)
    T = topk_idx.shape[0]
    toks = np.arange(T) if tokens is None else np.asarray(tokens)
    Tw = math.ceil(Fraction(T, n_waves))
    rows, index = [], []
    for i, t in enumerate(toks):
        for j in range(topk_idx.shape[1]):
            if assignment["recv_slot"][t, j] >= 0:
                e = int(topk_idx[t, j])
                rows.append(o[i, j])
                index.append((t // Tw, pool_of(e, n_experts, n_pools),
                              int(assignment["pool_slot"][t, j])))
    L = o.shape[-1]
    return (np.asarray(rows).reshape(-1, L), np.asarray(index).reshape(-1, 3))


# ---------------------------------------------------------------------------
# dropless ragged variant   [LJ §4] and [RH §3.3]: the fallback that keeps
# every routed assignment (a ragged all-to-all instead of fixed capped pools)
# ---------------------------------------------------------------------------


def ragged_order(topk_idx, n_experts):
    """Order of the T*k assignments by expert, stable in (token, j) order.

    Returns (row_of [T, k], offsets [E+1]): expert e's assignments take rows
    [offsets[e], offsets[e+1]); an id outside [0, E) takes no row (-1).
    The order is a stable sort of the flattened expert ids (a library sort).
    """
    topk_idx = np.asarray(topk_idx, dtype=np.int64)
    flat = topk_idx.reshape(-1)
    valid = (flat >= 0) & (flat < n_experts)
    counts = np.bincount(flat[valid], minlength=n_experts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    order = np.argsort(np.where(valid, flat, n_experts), kind="stable")
    row_of = np.full(flat.shape, -1, dtype=np.int64)
    nv = int(valid.sum())
    row_of[order[:nv]] = np.arange(nv)
    return row_of.reshape(topk_idx.shape), offsets


def forward_dropless(x, w, *, top_k, routing_logits32=None, tokens=None):
    """The branch with every assignment kept: top-k, gates, every selected
    expert's SwiGLU, the unrenormalised gate-weighted sum, up-projection and
    shared experts.  Equal to forward() with caps that hold every row."""
    x = np.asarray(x)
    T = x.shape[0]
    toks = np.arange(T) if tokens is None else np.asarray(tokens)
    z = latent(x[toks], w["w_latent"])
    logits = router_logits(z, w["w_router"])
    if routing_logits32 is None:
        if tokens is not None:
            raise ValueError("a token subset needs the full routing logits")
        routing_logits32 = logits.astype(np.float32)
    topk_idx = route_topk(routing_logits32, w["router_bias"], top_k)
    g = gates(routing_logits32, topk_idx)
    E = np.asarray(w["w_router"]).shape[0]
    row_of, offsets = ragged_order(topk_idx, E)
    ew = w.get("expert_weights")
    if ew is None:
        def ew(e):
            return w["w_gate"][e], w["w_up"][e], w["w_down"][e]
    kept = np.zeros(topk_idx.shape, dtype=np.int64)   # every row is kept
    o = expert_outputs(z, topk_idx, kept, ew, tokens=toks)
    y_lat = combine(g[toks], kept[toks], o)
    y = up_project(y_lat, w["w_up_proj"]) + shared_experts(
        x[toks], w["ws_gate"], w["ws_up"], w["ws_down"])
    return dict(z=z, logits=logits, topk_idx=topk_idx, gates=g, row_of=row_of,
                offsets=offsets, expert_out=o, y_latent=y_lat, y=y, tokens=toks)


# ---------------------------------------------------------------------------
# receive-side share of one rank: experts over a given bank, then combine
# ---------------------------------------------------------------------------


def bank_expert_rows(rows, bank_rows, expert_count, expert_weights, experts,
                     row_filter=None):
    """SwiGLU_e of the bank rows binned to expert e, for e in `experts`: the
    receiver side of one destination ([LJ §2]: the receiver cap bounds the
    rows of one local expert; [RH §3.2]: each wave's receive buffer holds
    the expected rows of that wave x 1.15).

    rows[w][s] is the row in slot s of the destination's block of wave w;
    bank_rows[w, e, r] is the pool slot of the r-th row wave w binned to
    expert e, for r < expert_count[w, e] (later entries are not read).
    Returns {(w, s): o}.  row_filter(w, s) -> bool restricts the computed
    rows.
    """
    out = {}
    W = bank_rows.shape[0]
    for e in experts:
        wg, wu, wd = expert_weights(int(e))
        sel = []
        for w in range(W):
            for r in range(int(expert_count[w, e])):
                s = int(bank_rows[w, e, r])
                if row_filter is None or row_filter(w, s):
                    sel.append((w, s))
        if not sel:
            continue
        u = np.stack([np.asarray(rows[w][s], dtype=np.float64) for w, s in sel])
        o = swiglu(u, wg, wu, wd)
        for (w, s), v in zip(sel, o):
            out[(w, s)] = v
    return out
