"""Pins of the oracle's pooled-wave slot assignment (CPU only)."""
import numpy as np
import pytest

import oracle


def _random_topk(rng, T, E, k, skew=0.0):
    """Distinct experts per token, optionally skewed towards low indices."""
    w = np.exp(-skew * np.arange(E))
    w /= w.sum()
    return np.stack([rng.choice(E, size=k, replace=False, p=w) for _ in range(T)])


def _check_closed_forms(idx, E, P, W, cs, cr, a):
    T, k = idx.shape
    epp = E // P
    # row conservation
    assert a["kept"] + a["sender_dropped"] + a["receiver_dropped"] == T * k
    assert a["kept"] == int((a["recv_slot"] >= 0).sum())
    assert a["sender_dropped"] == int((a["pool_slot"] < 0).sum())
    assert a["receiver_dropped"] == int(((a["pool_slot"] >= 0) & (a["recv_slot"] < 0)).sum())
    for w, (t0, t1) in enumerate(oracle.wave_ranges(T, W)):
        flat = idx[t0:t1].reshape(-1)              # (t, j) order
        pools = flat // epp
        ps = a["pool_slot"][t0:t1].reshape(-1)
        rs = a["recv_slot"][t0:t1].reshape(-1)
        demand = np.bincount(pools, minlength=P)
        # pool_count = min(cap_send, demand)
        assert (a["pool_count"][w] == np.minimum(cs, demand)).all()
        for p in range(P):
            pos = np.nonzero(pools == p)[0]
            # the first cap_send of pool p in (t, j) order are sent, in order
            sent = pos[:cs]
            assert (ps[sent] == np.arange(len(sent))).all()
            assert (ps[pos[cs:]] == -1).all()
            # ids column: expert of each occupied slot, -1 after
            assert (a["ids"][w, p, :len(sent)] == flat[sent]).all()
            assert (a["ids"][w, p, len(sent):] == -1).all()
            # expert_count = min(cap_recv, # of e among pool p's first cap_send)
            for e in range(p * epp, (p + 1) * epp):
                mine = sent[flat[sent] == e]
                assert a["expert_count"][w, e] == min(cr, len(mine))
                kept = mine[:cr]
                assert (rs[kept] == np.arange(len(kept))).all()
                assert (rs[mine[cr:]] == -1).all()
                assert (a["bank_rows"][w, e, :len(kept)] == ps[kept]).all()
                assert (a["bank_rows"][w, e, len(kept):] == -1).all()
        assert a["pool_count"][w].max(initial=0) <= cs
        assert a["expert_count"][w].max(initial=0) <= cr


def _brute(idx, E, P, W, cs, cr):
    """O(n^2) re-derivation: an assignment's pool rank is the number of
    earlier assignments of the wave to the same pool; its receive rank is the
    number of earlier assignments to the same expert (all sent when it is)."""
    T, k = idx.shape
    epp = E // P
    ps = np.full((T, k), -1)
    rs = np.full((T, k), -1)
    for t0, t1 in oracle.wave_ranges(T, W):
        order = [(t, j) for t in range(t0, t1) for j in range(k)]
        for n, (t, j) in enumerate(order):
            e = idx[t, j]
            prank = sum(1 for (u, i) in order[:n] if idx[u, i] // epp == e // epp)
            erank = sum(1 for (u, i) in order[:n] if idx[u, i] == e)
            if prank < cs:
                ps[t, j] = prank
                if erank < cr:
                    rs[t, j] = erank
    return ps, rs


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("E,P,k,W", [(16, 4, 2, 3), (8, 2, 3, 1), (12, 12, 2, 2), (6, 1, 2, 3)])
def test_brute_force_tiny(seed, E, P, k, W):
    rng = np.random.default_rng(seed)
    T = 13
    idx = _random_topk(rng, T, E, k, skew=0.5)
    for cs, cr in [(1, 1), (2, 1), (3, 2), (4, 4), (100, 100), (0, 5), (5, 0)]:
        a = oracle.assign_slots(idx, E, P, W, cs, cr)
        ps, rs = _brute(idx, E, P, W, cs, cr)
        assert (a["pool_slot"] == ps).all() and (a["recv_slot"] == rs).all()
        _check_closed_forms(idx, E, P, W, cs, cr, a)


@pytest.mark.parametrize("seed", range(3))
def test_closed_forms_tiny_workload(seed):
    rng = np.random.default_rng(seed)
    T, E, P, k, W = 256, 16, 4, 2, 3
    plan = oracle.capacity_plan(T, k, E, P, W)
    idx = _random_topk(rng, T, E, k, skew=0.3)
    a = oracle.assign_slots(idx, E, P, W, plan["cap_send"], plan["cap_recv"])
    _check_closed_forms(idx, E, P, W, plan["cap_send"], plan["cap_recv"], a)
    assert a["sender_dropped"] > 0 and a["receiver_dropped"] > 0


def test_one_pool_is_per_expert_capacity_routing():
    """P = 1: the sender cap (1.10 x all of the wave's rows) never binds, and
    the result is textbook per-expert capacity routing: in each wave the first
    cap_recv assignments of every expert, in token order, are kept."""
    rng = np.random.default_rng(11)
    T, E, k, W = 300, 10, 3, 3
    idx = _random_topk(rng, T, E, k, skew=0.4)
    plan = oracle.capacity_plan(T, k, E, 1, W)
    a = oracle.assign_slots(idx, E, 1, W, plan["cap_send"], plan["cap_recv"])
    assert a["sender_dropped"] == 0
    keep = np.zeros((T, k), dtype=bool)
    for t0, t1 in oracle.wave_ranges(T, W):
        flat = idx[t0:t1].reshape(-1)
        order = np.argsort(flat, kind="stable")
        starts = np.searchsorted(flat[order], np.arange(E))
        rank = np.empty_like(order)
        rank[order] = np.arange(len(flat)) - starts[flat[order]]
        keep[t0:t1] = (rank < plan["cap_recv"]).reshape(t1 - t0, k)
    assert ((a["recv_slot"] >= 0) == keep).all()
    assert a["receiver_dropped"] > 0


def test_one_expert_per_pool_has_no_receiver_drops():
    # P = E: cap_send = ceil(1.10 x load) <= cap_recv = ceil(1.15 x load)
    rng = np.random.default_rng(5)
    T, E, k, W = 400, 8, 2, 3
    idx = _random_topk(rng, T, E, k, skew=0.6)
    plan = oracle.capacity_plan(T, k, E, E, W)
    assert plan["cap_send"] <= plan["cap_recv"]
    a = oracle.assign_slots(idx, E, E, W, plan["cap_send"], plan["cap_recv"])
    assert a["receiver_dropped"] == 0 and a["sender_dropped"] > 0


def test_dropless_and_zero_caps():
    rng = np.random.default_rng(2)
    T, E, P, k, W = 90, 12, 3, 4, 3
    idx = _random_topk(rng, T, E, k)
    a = oracle.assign_slots(idx, E, P, W, T * k, T * k)
    assert a["kept"] == T * k
    a = oracle.assign_slots(idx, E, P, W, 0, T * k)
    assert a["sender_dropped"] == T * k and (a["ids"].size == 0)
    a = oracle.assign_slots(idx, E, P, W, T * k, 0)
    assert a["receiver_dropped"] == T * k and a["kept"] == 0


def test_waves_are_independent_chunks():
    """A W-wave assignment equals W one-wave assignments of its chunks with
    the same per-wave caps."""
    rng = np.random.default_rng(9)
    T, E, P, k, W = 100, 8, 4, 2, 3
    idx = _random_topk(rng, T, E, k, skew=0.5)
    cs, cr = 12, 5
    a = oracle.assign_slots(idx, E, P, W, cs, cr)
    for w, (t0, t1) in enumerate(oracle.wave_ranges(T, W)):
        b = oracle.assign_slots(idx[t0:t1], E, P, 1, cs, cr)
        assert (a["pool_slot"][t0:t1] == b["pool_slot"]).all()
        assert (a["recv_slot"][t0:t1] == b["recv_slot"]).all()
        assert (a["bank_rows"][w] == b["bank_rows"][0]).all()
        assert (a["ids"][w] == b["ids"][0]).all()


def test_priority_inside_a_token():
    # one token whose two experts share a pool with room for one row: j = 0
    # (its higher-scoring expert) takes the slot
    idx = np.array([[1, 0]])
    a = oracle.assign_slots(idx, 2, 1, 1, 1, 1)
    assert list(a["pool_slot"][0]) == [0, -1]
    assert a["ids"][0, 0, 0] == 1
