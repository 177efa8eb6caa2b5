"""Seeded random shapes through the GPU path against the fp64 oracle.

Forward (capped and dropless), the routed-path backward (capped and
dropless) and the router bias update over random token counts, expert and
pool counts (4 experts included), top-k, wave counts, widths, shared experts
and capacity factors (including a zero factor), with the same bars as the
fixed cases: indices, slots, counts and histograms bit-exact, values within
the row-wise tolerance.

Two kinds of value are compared with the condition-aware bars of readings
R21 and B7 (the row-wise bar measures their conditioning, not the kernels):
router logits in rows of fewer than 8 experts (each element within the
tolerance of its magnitude bound sum_l |z_l| |W_el|, and the router GEMM of
the path's own z within 1e-5 of it), and the weight gradients of experts
that kept 1 to 31 rows (each expert's gradient matrix within the tolerance
in max-norm; experts with no row get exact zeros).  The row-wise bar on
those gradients is kept as an expected failure that records the class.
"""
import random

import numpy as np
import pytest
import torch

import oracle
import synth
from _util import f64, oracle_weights, rowwise_rel_err
from gpu_common import check_weight_grads, dev, np_f32, np_i, say, tol
import test_gpu_backward as gb
import test_gpu_bias as gbias
import test_gpu_dropless as gd
import test_gpu_parity as gp

pytestmark = pytest.mark.gpu

N_CASES = 16


def _shape(i, backward=False):
    rng = random.Random(1000 + i)
    E = rng.choice([8, 12, 16, 24, 32, 48, 64])
    P = rng.choice([p for p in (1, 2, 4, 8, 16) if E % p == 0])
    k = rng.randint(1, min(8, E))
    W = rng.randint(1, 3)
    T = rng.choice([1, 5, 63, 65, 300, 777, 1500, 2500])
    dt = "bf16" if backward else rng.choice(["bf16", "bf16", "f32"])
    if backward or rng.random() < 0.5:
        L, F = 256 * rng.randint(1, 2), 256 * rng.randint(1, 2)
    else:
        L, F = 64 * rng.randint(1, 6), 64 * rng.randint(1, 6)
    D = 64 * rng.randint(1, 6)
    S, Fs = rng.randint(0, 2), 64 * rng.randint(1, 4)
    sc = rng.choice([(11, 10), (1, 2), (3, 1), (0, 1)])
    rc = rng.choice([(23, 20), (1, 3), (5, 1), (0, 1)])
    return synth.Workload(f"random{i}", T=T, d_model=D, d_latent=L, n_experts=E, n_pools=P, top_k=k, d_ff=F,
                          n_shared=S, d_ff_shared=Fs, n_waves=W, dtype=dt, bias="normal",
                          bias_std=rng.choice([0.0, 0.01, 0.5]), send_cap=sc, recv_cap=rc)


@pytest.mark.parametrize("i", range(N_CASES))
def test_forward_random(i):
    w = _shape(i)
    say("random forward", w)
    gp._check_forward(w, 100 + i, dev())
    if w.dtype == "bf16":
        gd._check_forward_dropless(w, 200 + i, dev())


def _check_backward(w, seed, dropless):
    d = dev()
    if dropless:
        cfg, inp, fwd, bwd, dy, dz, d_logits, dw = gb._run_dropless(w, seed, d)
        taps = fwd.tap_t
        topk = np_i(taps["topk_idx"])
        wt = oracle_weights(inp)
        ref = oracle.routed_backward(f64(taps["z"]), topk, np_f32(taps["gates"]).astype(np.float64),
                                     np.zeros(topk.shape, dtype=np.int64),
                                     lambda e: (wt["w_gate"][e], wt["w_up"][e], wt["w_down"][e]), f64(dy),
                                     w.n_experts, o=gb._saved_o_dropless(fwd), experts=range(w.n_experts))
        rows = np.bincount(topk.ravel(), minlength=w.n_experts)
    else:
        cfg, inp, fwd, bwd, dy, dz, d_logits, dw = gb._run(w, seed, d)
        ref, topk, recv = gb._oracle(w, inp, fwd, dy, experts=range(w.n_experts))
        rows = np_i(fwd.tap_t["expert_count"]).sum(axis=0)
    t = tol(w.dtype)
    assert rowwise_rel_err(f64(dz), ref["dz"]) <= t
    assert rowwise_rel_err(np_f32(d_logits).astype(np.float64), ref["d_logits"]) <= t
    check_weight_grads(dw, ref["dw"], rows, t)
    return dw, ref, rows


def _four_experts(i):
    rng = random.Random(3000 + i)
    return synth.Workload(f"random_e4_{i}", T=rng.choice([1, 63, 300, 1500, 2500]), d_model=64 * rng.randint(1, 4),
                          d_latent=256 * rng.randint(1, 2), n_experts=4, n_pools=rng.choice([1, 2, 4]),
                          top_k=rng.randint(1, 4), d_ff=256, n_shared=rng.randint(0, 2), d_ff_shared=128,
                          n_waves=rng.randint(1, 3), dtype=rng.choice(["bf16", "bf16", "f32"]), bias="normal",
                          bias_std=rng.choice([0.0, 0.01]), send_cap=rng.choice([(11, 10), (1, 2)]),
                          recv_cap=rng.choice([(23, 20), (1, 3)]))


@pytest.mark.parametrize("i", range(8))
def test_forward_random_four_experts(i):
    w = _four_experts(i)
    say("random forward, 4 experts", w)
    gp._check_forward(w, 600 + i, dev())
    if w.dtype == "bf16":
        gd._check_forward_dropless(w, 700 + i, dev())


@pytest.mark.parametrize("i", range(N_CASES // 2))
def test_backward_random(i):
    w = _shape(50 + i, backward=True)
    say("random backward", w)
    _check_backward(w, 300 + i, dropless=False)
    _check_backward(w, 400 + i, dropless=True)


@pytest.mark.parametrize("dropless", [False, True])
def test_backward_weight_grads_many_tiles_per_workgroup(dropless):
    """More weight-gradient tiles than CUs (64 experts x 4 x 4 tiles of
    256 x 256 at L = F = 1024), so each persistent workgroup walks several
    tiles through one pipeline; a strongly biased router leaves some experts
    empty and, in the dropless variant, gives others many times the mean row
    count, so tiles of different K follow one another.  Every expert's gradients
    against the oracle."""
    w = synth.Workload("wgrad_many_tiles", T=1500, d_model=256, d_latent=1024, n_experts=64, n_pools=8,
                       top_k=2, d_ff=1024, n_shared=0, d_ff_shared=128, n_waves=2, dtype="bf16",
                       bias="normal", bias_std=2.0, send_cap=(11, 10), recv_cap=(23, 20))
    say("backward, weight-gradient tiles beyond one per CU", w, "dropless" if dropless else "capped")
    dw, ref, rows = _check_backward(w, 900 + int(dropless), dropless=dropless)
    # (capped: the receiver cap keeps every expert below 64 rows)
    assert (rows == 0).any() and (rows.max() > 64 or not dropless)


@pytest.mark.xfail(strict=False, reason=(
    "row-wise weight gradients of experts with 1-31 rows: a row is a short sum of rank-one terms "
    "whose size can rest on cancelling dh values and on silu'(a) near its zero, so its relative "
    "error is the elementwise error of da / db (do and dh are stored bf16, reading B5); reading B7 "
    "compares these experts in max-norm instead"))
def test_backward_rowwise_small_experts():
    worst = 0.0
    for i in range(4):
        w = _shape(50 + i, backward=True)
        say("random backward, row-wise on small experts", w)
        dw, ref, rows = _check_backward(w, 300 + i, dropless=False)
        for e in np.nonzero((rows > 0) & (rows < 32))[0]:
            for m in range(3):
                worst = max(worst, rowwise_rel_err(f64(dw[m][e]), ref["dw"][e][m]))
    assert worst <= tol("bf16"), worst


@pytest.mark.parametrize("i", range(N_CASES))
def test_bias_update_random(i):
    rng = random.Random(2000 + i)
    T = rng.choice([1, 2, 63, 1025, 5000, 20000])
    E = rng.choice([1, 3, 4, 31, 64, 100, 384, 1000, 1024])
    k = rng.randint(1, min(64, E))
    nb = rng.choice([1, 2, 7, 64, 256, 1000, 1024])
    g = torch.Generator().manual_seed(500 + i)
    kind = rng.choice(["normal", "ties", "shift"])
    if kind == "normal":
        lg = torch.randn(T, E, generator=g) * rng.choice([1e-3, 1.0, 30.0])
    elif kind == "ties":
        lg = torch.randint(-3, 4, (T, E), generator=g).float()
    else:
        lg = torch.randn(T, E, generator=g) + torch.randint(-50, 50, (1, E), generator=g).float()
    gbias._check(lg.contiguous(), k, nb)
