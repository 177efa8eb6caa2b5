"""Pins of the oracle's top-k selection and gates (CPU only)."""
import itertools

import numpy as np
import pytest
import torch

import oracle


def _brute_topk(l, b, k):
    """Rank of e = number of experts that beat it: higher fl32 score, or an
    equal score and a lower index.  The top-k are ranks 0..k-1 in order."""
    T, E = l.shape
    out = np.empty((T, k), dtype=np.int64)
    for t in range(T):
        s = [float(np.float32(l[t, e]) + np.float32(b[e])) for e in range(E)]
        rank = [sum(1 for f in range(E) if s[f] > s[e] or (s[f] == s[e] and f < e))
                for e in range(E)]
        for e in range(E):
            if rank[e] < k:
                out[t, rank[e]] = e
    return out


@pytest.mark.parametrize("seed", range(6))
def test_topk_bruteforce_with_ties(seed):
    rng = np.random.default_rng(seed)
    T = 16
    for E in [1, 2, 3, 5, 8, 12]:
        # few distinct values, so ties are common; signed zeros included
        vals = np.array([-1.5, -0.0, 0.0, 0.25, 0.25, 1.0, 3.0], dtype=np.float32)
        l = rng.choice(vals, size=(T, E)).astype(np.float32)
        b = rng.choice(np.array([0.0, -0.0, 0.25], dtype=np.float32), size=E)
        for k in range(1, E + 1):
            got = oracle.route_topk(l, b, k)
            assert np.array_equal(got, _brute_topk(l, b, k)), (E, k)


def test_topk_is_a_stable_sort_on_minus_score():
    # textbook routine: Python's stable sort by (-score, index)
    rng = np.random.default_rng(7)
    l = rng.standard_normal((32, 24)).astype(np.float32)
    b = (0.1 * rng.standard_normal(24)).astype(np.float32)
    s = l + b
    got = oracle.route_topk(l, b, 5)
    for t in range(32):
        ref = sorted(range(24), key=lambda e: (-float(s[t, e]), e))[:5]
        assert list(got[t]) == ref


def test_all_equal_logits_pick_lowest_indices():
    l = np.full((4, 10), 0.5, dtype=np.float32)
    assert (oracle.route_topk(l, np.zeros(10, np.float32), 3) == [0, 1, 2]).all()


def test_signed_zero_ties():
    l = np.array([[-0.0, 0.0, -0.0]], dtype=np.float32)
    assert list(oracle.route_topk(l, np.zeros(3, np.float32), 3)[0]) == [0, 1, 2]
    l = np.array([[0.0, -0.0]], dtype=np.float32)
    assert list(oracle.route_topk(l, np.zeros(2, np.float32), 1)[0]) == [0]


def test_selection_decided_in_fp32():
    # 1 + 2^-25 rounds to 1 in fp32: experts 0 and 1 tie, the lower index wins,
    # although in exact arithmetic expert 1 scores higher
    l = np.array([[1.0, 1.0]], dtype=np.float32)
    b = np.array([0.0, 2.0 ** -25], dtype=np.float32)
    assert oracle.route_topk(l, b, 1)[0, 0] == 0
    # 2^-23 survives the rounding and expert 1 wins
    b = np.array([0.0, 2.0 ** -23], dtype=np.float32)
    assert oracle.route_topk(l, b, 1)[0, 0] == 1


def test_bias_moves_selection_not_gates():
    l = np.array([[2.0, 1.0, 0.0, -1.0]], dtype=np.float32)
    b = np.array([0.0, 0.0, 3.0, 0.0], dtype=np.float32)
    idx = oracle.route_topk(l, b, 2)
    assert list(idx[0]) == [2, 0]
    g = oracle.gates(l, idx)
    # softmax of the raw logits 0 and 2 (bias excluded)
    e = np.exp([0.0 - 2.0, 0.0])
    assert np.allclose(g[0], e / e.sum(), rtol=0, atol=1e-15)


def test_gates_closed_forms():
    rng = np.random.default_rng(3)
    l = rng.standard_normal((50, 16)).astype(np.float32)
    idx = oracle.route_topk(l, np.zeros(16, np.float32), 4)
    g = oracle.gates(l, idx)
    assert np.allclose(g.sum(axis=1), 1.0, rtol=0, atol=1e-15)
    assert (g > 0).all()
    # ordered by score, so gates are non-increasing along j
    assert (np.diff(g, axis=1) <= 1e-15).all()
    # ratio identity g_i / g_j = exp(l_i - l_j)
    sel = np.take_along_axis(l.astype(np.float64), idx, axis=1)
    for i, j in itertools.combinations(range(4), 2):
        assert np.allclose(g[:, i] / g[:, j], np.exp(sel[:, i] - sel[:, j]), rtol=1e-13)
    # library routine: torch softmax in float64 over the selected logits
    ref = torch.softmax(torch.from_numpy(sel), dim=1).numpy()
    assert np.allclose(g, ref, rtol=1e-14, atol=1e-16)
    # k = 1 -> gate 1; equal selected logits -> 1/k
    idx1 = oracle.route_topk(l, np.zeros(16, np.float32), 1)
    assert (oracle.gates(l, idx1) == 1.0).all()
    le = np.zeros((3, 8), dtype=np.float32)
    assert np.allclose(oracle.gates(le, oracle.route_topk(le, np.zeros(8, np.float32), 8)), 1 / 8)


def test_gates_shift_invariant_and_large_logits():
    l = np.array([[1000.0, 999.0, -1000.0]], dtype=np.float32)
    idx = oracle.route_topk(l, np.zeros(3, np.float32), 2)
    g = oracle.gates(l, idx)
    assert np.isfinite(g).all()
    assert np.allclose(g[0], [1 / (1 + np.exp(-1.0)), np.exp(-1.0) / (1 + np.exp(-1.0))])
