"""Pins of the oracle's capacity plan (CPU only)."""
import json
import math
import os

import pytest

import oracle
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def test_recv_share_printed_capacity():
    # ceil(1.15 x 87381) = 100489: one EP64 rank's per-expert row capacity
    # for a 4,194,304-token step, all of it one wave.
    c = _load("page_constants.json")["recv_share_capacity"]
    plan = oracle.capacity_plan(c["tokens_per_step"], 8, 384, 64, 1)
    assert plan["cap_recv"] == c["value"] == 100489
    assert c["tokens_per_step"] * 8 // 384 == c["expected_load"]
    # the per-wave slab of the receive share
    assert synth.RECV_SHARE["cap_wave"] == 33497
    assert 3 * 33497 >= 100489 > 3 * 33496


@pytest.mark.parametrize("name", ["tiny_fp32", "mid_bf16", "marin_16k", "zipf_64k"])
def test_workload_caps_table(name):
    g = _load("workload_caps.json")[name]
    w = synth.workload(name)
    assert (w.T, w.top_k, w.n_experts, w.n_pools, w.n_waves) == (
        g["T"], g["k"], g["E"], g["P"], g["W"])
    plan = oracle.capacity_plan(w.T, w.top_k, w.n_experts, w.n_pools, w.n_waves)
    assert (plan["Tw"], plan["cap_send"], plan["cap_recv"]) == (
        g["Tw"], g["cap_send"], g["cap_recv"])


def test_factors_are_the_pages():
    c = _load("page_constants.json")
    w = synth.workload("marin_16k")
    assert tuple(c["sender_capacity_factor"]["value"]) == w.send_cap
    assert tuple(c["receiver_capacity_factor"]["value"]) == w.recv_cap
    assert c["n_waves"]["value"] == w.n_waves
    assert c["routed_experts"]["value"] == w.n_experts
    assert c["top_k"]["value"] == w.top_k
    assert c["ep_degree"]["value"] == w.n_pools
    plan = oracle.capacity_plan(w.T, w.top_k, w.n_experts, w.n_pools, w.n_waves)
    assert plan["experts_per_pool"] == c["experts_per_destination"]["value"]


def test_exact_rational_not_float():
    # expected load exactly 100 rows: 1.10 x 100 = 110 exactly, while the
    # binary-float product 1.1 * 100 = 110.00000000000001 would ceil to 111
    assert math.ceil(1.1 * 100) == 111
    plan = oracle.capacity_plan(100, 1, 1, 1, 1)
    assert plan["cap_send"] == 110
    assert plan["cap_recv"] == 115


@pytest.mark.parametrize("T", [1, 2, 7, 86, 100, 255, 256, 1000, 4096, 5461, 16384])
@pytest.mark.parametrize("k,E,P,W", [(1, 1, 1, 1), (2, 16, 4, 3), (8, 64, 16, 3),
                                     (8, 384, 64, 3), (8, 384, 384, 2), (3, 9, 3, 5)])
def test_ceil_defining_property(T, k, E, P, W):
    """cap is the least integer >= factor x expected load, checked with
    integer cross-multiplication (no division, no rounding)."""
    plan = oracle.capacity_plan(T, k, E, P, W)
    Tw = plan["Tw"]
    assert W * Tw >= T > W * (Tw - 1)
    cs, cr = plan["cap_send"], plan["cap_recv"]
    # 10 P cs >= 11 Tw k > 10 P (cs - 1)
    assert 10 * P * cs >= 11 * Tw * k > 10 * P * (cs - 1)
    assert 20 * E * cr >= 23 * Tw * k > 20 * E * (cr - 1)


def test_overrides_and_errors():
    p = oracle.capacity_plan(65536, 8, 6, 1, 3, cap_send_rows=6 * 33497,
                             cap_recv_rows=33497)
    assert p["cap_send"] == 200982 and p["cap_recv"] == 33497
    with pytest.raises(ValueError):
        oracle.capacity_plan(10, 2, 10, 3, 1)      # E not a multiple of P
    with pytest.raises(ValueError):
        oracle.capacity_plan(10, 2, 8, 4, 0)       # no waves


def test_wave_ranges_cover_tokens():
    for T in [1, 2, 3, 4, 86, 256, 16384]:
        for W in [1, 2, 3, 7]:
            r = oracle.wave_ranges(T, W)
            assert len(r) == W
            toks = [t for a, b in r for t in range(a, b)]
            assert toks == list(range(T))
            Tw = -(-T // W)
            assert all(b - a <= Tw for a, b in r)
