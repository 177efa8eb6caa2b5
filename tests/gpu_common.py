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
