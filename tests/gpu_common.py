"""Shared helpers of the GPU parity tests (no method arithmetic)."""
import sys

import numpy as np
import pytest
import torch

import routing_capacity_dispatch_amd as rcd

TOL_F32 = 1e-4   # max row-wise relative error, fp32 workloads
TOL_BF16 = 2e-2  # bf16 inputs, fp32 accumulation
GATE_ATOL = 2e-6


def dev():
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")
    return torch.device("cuda:0")


def say(*a):
    """Name the case before a GPU step, flushed, so a crash log shows it."""
    print("[gpu]", *a, flush=True)
    sys.stdout.flush()


def np_i(t):
    return t.detach().cpu().numpy().astype(np.int64)


def np_f32(t):
    return t.detach().to("cpu", torch.float32).numpy()


def tol(dtype):
    return TOL_BF16 if dtype == "bf16" else TOL_F32


def bank_valid(bank_rows, expert_count):
    """bank_rows entries r < expert_count[w, e] (the rest are unspecified)."""
    W, E, C = bank_rows.shape
    r = np.arange(C)[None, None, :]
    return np.where(r < expert_count[:, :, None], bank_rows, -1)


def check_untapped(fwd, cfg, weights, x, y_tapped):
    # Without taps, y_lat and the shared hidden rows share one buffer and the
    # output projection runs as one K range (bf16 with d_latent == d_ff_shared:
    # the joined-range kernel); with taps they are separate K ranges.  Both
    # accumulate every output in the same K order, so y is the same bits.
    y2, _, _ = fwd(cfg, weights, x)
    torch.cuda.synchronize()
    a, b = y_tapped, y2
    if a.dtype == torch.bfloat16:
        a, b = a.view(torch.int16), b.view(torch.int16)
    assert torch.equal(a, b)


def check_weight_grads(dw, ref_dw, rows, t):
    """Weight gradients of every expert against the oracle (reading B7): an
    expert that kept no row must get exact zeros; every other expert's
    gradient matrix must be within t in max-norm (max |diff| / max |ref|);
    experts with at least 32 rows must also be within t row by row.
    dw: the three [E, out, in] gradients in the order the backward returns
    them; ref_dw[e]: the oracle's three for expert e in the same order, fp64.
    Returns the worst max-norm and row-wise errors."""
    from _util import f64, rowwise_rel_err
    worst_mx, worst_rw = 0.0, 0.0
    for e in range(len(rows)):
        for i in range(3):
            if rows[e] == 0:
                assert torch.count_nonzero(dw[i][e]) == 0, (e, i)
                continue
            g, r = f64(dw[i][e]), ref_dw[e][i]
            mx = float(np.abs(g - r).max() / np.abs(r).max())
            assert mx <= t, ("max-norm", e, i, int(rows[e]), mx)
            worst_mx = max(worst_mx, mx)
            if rows[e] >= 32:
                rw = rowwise_rel_err(g, r)
                assert rw <= t, ("row-wise", e, i, int(rows[e]), rw)
                worst_rw = max(worst_rw, rw)
    return worst_mx, worst_rw


def check_logits(logits32, z, w_router, ref_logits, ref_z, t):
    """Router logits (reading R21): against the router GEMM of the path's own
    z (fp64 over the same stored operands) within 1e-5 of each element's
    magnitude bound sum_l |z_l| |W_el|; against the fp64 oracle row by row
    within t when a row holds at least 8 experts, and within t of that
    magnitude bound for every element (rows of 4 experts included)."""
    from _util import rowwise_rel_err
    lg = np.asarray(logits32, dtype=np.float64)
    own = z @ w_router.T
    bound = np.abs(z) @ np.abs(w_router).T
    with np.errstate(invalid="ignore", divide="ignore"):
        q = np.where(bound > 0, np.abs(lg - own) / np.where(bound > 0, bound, 1.0), np.abs(lg - own))
    assert float(q.max(initial=0.0)) <= 1e-5, ("logits vs own z", float(q.max()))
    bref = np.abs(ref_z) @ np.abs(w_router).T
    with np.errstate(invalid="ignore", divide="ignore"):
        q = np.where(bref > 0, np.abs(lg - ref_logits) / np.where(bref > 0, bref, 1.0), np.abs(lg - ref_logits))
    assert float(q.max(initial=0.0)) <= t, ("logits vs oracle, element bound", float(q.max()))
    if lg.shape[1] >= 8:
        err = rowwise_rel_err(lg, ref_logits)
        assert err <= t, ("logits vs oracle, row-wise", err)
