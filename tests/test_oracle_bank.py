"""Pins of the receiver-side oracle (bank_expert_rows) and of the drop
fractions, on the CPU.

bank_expert_rows computes each local expert's SwiGLU from the destination's
pool block and its receiver row lists ([LJ §2]: the receiver cap bounds one
local expert's rows; [RH §3.2]: per-wave receive buffers).  It is pinned
against the per-assignment expert outputs of the forward oracle, placed at
their (wave, pool, slot) rows, on tiny multi-wave inputs with receiver drops:
the two reach the same rows by different routes (token order against the
receiver's slot lists), so a wrong wave, a wrong slot map or a row list read
past its count disagrees.  drop_fractions is pinned by a count worked by
hand and by row conservation ([RH §3.3]: sender and receiver drops are
counted separately).
"""
from fractions import Fraction

import numpy as np

import oracle


def _weights(E, L, F, seed):
    rng = np.random.default_rng(seed)
    ws = [(rng.standard_normal((F, L)) / np.sqrt(L), rng.standard_normal((F, L)) / np.sqrt(L),
           rng.standard_normal((L, F)) / np.sqrt(F)) for _ in range(E)]
    return lambda e: ws[e]


def _bank_case(seed, T=31, E=6, k=2, W=3, L=8, F=12, recv_num=2, recv_den=3):
    """One destination (P = 1) holding E local experts, as one EP rank's
    receive side; receiver factor below 1 so that receiver drops occur."""
    rng = np.random.default_rng(seed)
    # skewed popularity so a few experts overflow their receiver capacity
    pop = rng.dirichlet(np.full(E, 0.7))
    topk = np.stack([rng.choice(E, k, replace=False, p=pop) for _ in range(T)])
    plan = oracle.capacity_plan(T, k, E, 1, W, recv_cap=(recv_num, recv_den))
    a = oracle.assign_slots(topk, E, 1, W, plan["cap_send"], plan["cap_recv"])
    z = rng.standard_normal((T, L))
    # the destination's pool block per wave, as the sender fills it
    Tw = plan["Tw"]
    rows = np.full((W, plan["cap_send"], L), np.nan)
    for t in range(T):
        for j in range(k):
            if a["pool_slot"][t, j] >= 0:
                rows[t // Tw, a["pool_slot"][t, j]] = z[t]
    return topk, z, a, plan, rows



def test_bank_rows_equal_forward_expert_outputs():
    E, L, F = 6, 8, 12
    ew = _weights(E, L, F, seed=3)
    for seed in range(6):
        topk, z, a, plan, rows = _bank_case(seed)
        assert a["receiver_dropped"] > 0 and a["kept"] > 0
        o = oracle.expert_outputs(z, topk, a["recv_slot"], ew)
        vals, index = oracle.expert_out_pool_layout(o, topk, a, E, 1, 3, plan["cap_send"])
        want = {(int(w), int(s)): v for (w, _, s), v in zip(index, vals)}
        got = oracle.bank_expert_rows(rows, a["bank_rows"], a["expert_count"], ew, range(E))
        assert set(got) == set(want), seed
        for key in want:
            np.testing.assert_allclose(got[key], want[key], rtol=1e-12, atol=1e-14)
        # receiver-dropped rows occupy a pool slot but get no output
        Tw = plan["Tw"]
        for t, j in zip(*np.nonzero((a["pool_slot"] >= 0) & (a["recv_slot"] < 0))):
            assert (t // Tw, int(a["pool_slot"][t, j])) not in got


def test_bank_rows_row_filter_and_expert_subset():
    E, L, F = 6, 8, 12
    ew = _weights(E, L, F, seed=4)
    topk, z, a, plan, rows = _bank_case(11)
    full = oracle.bank_expert_rows(rows, a["bank_rows"], a["expert_count"], ew, range(E))
    sub = oracle.bank_expert_rows(rows, a["bank_rows"], a["expert_count"], ew, [1, 4],
                                  row_filter=lambda w, s: w != 1)
    ids = a["ids"][:, 0]
    assert sub and set(sub) == {(w, s) for (w, s) in full if w != 1 and ids[w, s] in (1, 4)}
    for key, v in sub.items():
        np.testing.assert_array_equal(v, full[key])


def test_bank_rows_single_wave_by_hand():
    # one wave, two experts, receiver capacity 1: rows worked out by hand.
    # assignments in (t, j) order: (0,0)->e1 slot 0, (0,1)->e0 slot 1,
    # (1,0)->e1 slot 2 (receiver-dropped: e1 already holds 1 row),
    # (1,1)->e0 slot 3 (receiver-dropped)
    topk = np.array([[1, 0], [1, 0]])
    a = oracle.assign_slots(topk, 2, 1, 1, 4, 1)
    assert a["pool_slot"].tolist() == [[0, 1], [2, 3]]
    assert a["recv_slot"].tolist() == [[0, 0], [-1, -1]]
    assert a["bank_rows"][0].tolist() == [[1], [0]]
    z = np.array([[1.0, -2.0], [0.5, 3.0]])
    rows = np.array([[z[0], z[0], z[1], z[1]]])
    ew = _weights(2, 2, 3, seed=9)
    got = oracle.bank_expert_rows(rows, a["bank_rows"], a["expert_count"], ew, [0, 1])
    assert set(got) == {(0, 0), (0, 1)}
    np.testing.assert_allclose(got[(0, 0)], oracle.swiglu(z[:1], *ew(1))[0], rtol=1e-13)
    np.testing.assert_allclose(got[(0, 1)], oracle.swiglu(z[:1], *ew(0))[0], rtol=1e-13)


def test_drop_fractions_hand_count():
    # T = 4 tokens, k = 2, E = 2 experts in one pool, one wave, caps 3 / 1.
    # In (t, j) order the pool takes the first 3 of the 8 assignments and
    # drops 5 at the sender; of those 3, e0 keeps (0,0), e1 keeps (0,1), and
    # (1,0) -> e0 is dropped at the receiver: kept 2, sd 5, rd 1.
    topk = np.array([[0, 1], [0, 1], [0, 1], [1, 0]])
    a = oracle.assign_slots(topk, 2, 1, 1, 3, 1)
    assert (a["kept"], a["sender_dropped"], a["receiver_dropped"]) == (2, 5, 1)
    f = oracle.drop_fractions(a, 4, 2)
    assert f == dict(sender=5 / 8, receiver=1 / 8, total=6 / 8)


def test_drop_fractions_conservation():
    rng = np.random.default_rng(5)
    for _ in range(20):
        T, E, k, W = int(rng.integers(1, 60)), 8, int(rng.integers(1, 4)), int(rng.integers(1, 4))
        P = int(rng.choice([1, 2, 4, 8]))
        topk = np.stack([rng.choice(E, k, replace=False) for _ in range(T)])
        cs, cr = int(rng.integers(0, 6)), int(rng.integers(0, 4))
        a = oracle.assign_slots(topk, E, P, W, cs, cr)
        f = oracle.drop_fractions(a, T, k)
        n = T * k
        assert Fraction(f["total"]).limit_denominator(n) == 1 - Fraction(a["kept"], n)
        assert f["sender"] == a["sender_dropped"] / n and f["receiver"] == a["receiver_dropped"] / n
        assert f["sender"] == np.count_nonzero(a["pool_slot"] < 0) / n
        assert f["receiver"] == np.count_nonzero((a["pool_slot"] >= 0) & (a["recv_slot"] < 0)) / n
