"""GPU parity of the router-bias update (moe_router_bias_update) against the
oracle, through the C ABI.

Ranges and histogram counts must match bit for bit (the bin of every logit
is decided in fp32 on both sides with the same operations).  The bias is
fp64 arithmetic on those counts and ranges, rounded to fp32; the two sides
sum the mean of the quantiles in different orders, so the bias may differ in
its last bits: |diff| <= 1e-6 * (1 + max |Q|).
"""
import numpy as np
import pytest
import torch

import oracle
import routing_capacity_dispatch_amd as rcd
import synth
from oracle import router_bias as rb
from gpu_common import dev, np_f32, np_i, say

pytestmark = pytest.mark.gpu


def _cfg(T, E, k):
    return rcd.make_config(T, 64, 64, E, 1, k, 64)


def _check(l_cpu, k, nb, logits_dev=None):
    T, E = l_cpu.shape
    d = dev()
    say("bias update", T, E, k, nb)
    lg = logits_dev if logits_dev is not None else l_cpu.to(d)
    bias, hist, lohi = rcd.router_bias_update(_cfg(T, E, k), lg, nb, with_hist=True)
    torch.cuda.synchronize()
    rb_bias, rb_hist, lo, hi, q = rb.bias_update(l_cpu.numpy(), k, nb)
    lohi = np_f32(lohi)
    assert np.array_equal(lohi[:, 0], lo) and np.array_equal(lohi[:, 1], hi)
    assert np.array_equal(np_i(hist), rb_hist)
    atol = 1e-6 * (1.0 + float(np.abs(q).max()))
    err = np.abs(np_f32(bias).astype(np.float64) - rb_bias.astype(np.float64)).max()
    assert err <= atol, (err, atol)
    return np_f32(bias)


CASES = [
    # T, E, k, nb, kind
    (1, 4, 1, 16, "normal"),            # one token: lo = hi, scale 0
    (7, 3, 2, 4, "normal"),             # E not a multiple of 4: scalar lanes
    (1000, 16, 2, 1, "normal"),         # one bin
    (1000, 16, 16, 64, "normal"),       # k = E: level 0
    (3000, 48, 8, 7, "ties"),           # many equal logits, odd bin count
    (5000, 100, 5, 256, "tiny"),        # ranges of a few hundred ulps
    (4097, 64, 8, 1024, "normal"),      # ragged last chunk, largest bin count
    (2049, 384, 8, 256, "normal"),
    (9000, 385, 8, 300, "ties"),        # partial last expert group, scalar lanes
    (300, 1024, 64, 512, "normal"),     # largest E and k
]


@pytest.mark.parametrize("T,E,k,nb,kind", CASES)
def test_bias_update(T, E, k, nb, kind):
    _check(synth.logits_case(T, E, seed=1, kind=kind), k, nb)


def test_misaligned_logits_take_the_scalar_path():
    # a view starting one float into its buffer: rows are not 16-byte aligned
    d = dev()
    T, E = 2000, 64
    l = synth.logits_case(T, E, seed=2)
    buf = torch.empty(T * E + 4, dtype=torch.float32, device=d)
    view = buf[1:1 + T * E].view(T, E)
    view.copy_(l.to(d))
    _check(l, 8, 128, logits_dev=view)


def test_values_on_bin_edges():
    # a grid of multiples of 1/8 over [0, 16] with 128 bins: every scaled
    # value lands on or next to an integer, where fp32 decides the bin; plus
    # the neighbours one ulp either side of each grid point
    g = np.arange(0, 129, dtype=np.float32) / 8
    up = np.nextafter(g, np.float32(np.inf))
    dn = np.nextafter(g, np.float32(-np.inf))
    col = np.concatenate([g, up[:-1], dn[1:]]).astype(np.float32)
    rng = np.random.default_rng(0)
    l = np.stack([rng.permutation(col) for _ in range(12)], axis=1)
    l[:, 5] *= np.float32(3.0)          # a range whose scale is not a power of two
    l[:, 7] += np.float32(0.1)
    _check(torch.from_numpy(np.ascontiguousarray(l)), 2, 128)


@pytest.mark.parametrize("name,nb", [("marin_16k", 256), ("marin_16k", 1024), ("zipf_64k", 256)])
def test_full_size(name, nb):
    w = synth.workload(name)
    l = synth.logits_case(w.T, w.n_experts, seed=0)
    l = (l + synth.router_bias(w, 0)[None, :]).contiguous()   # zipf_64k: skewed popularity
    _check(l, w.top_k, nb)


def test_deterministic_and_balancing():
    # the same call twice gives the same bits; the bias from skewed logits
    # evens the top-k loads out when routed with moe_route
    d = dev()
    T, E, k = 16384, 384, 8
    skew = synth.zipf_bias(E, seed=0).to(d)
    l = (synth.logits_case(T, E, seed=4).to(d) + skew[None, :]).contiguous()
    cfg = _cfg(T, E, k)
    say("bias update determinism", T, E, k)
    b0 = rcd.router_bias_update(cfg, l, 512)
    b1 = rcd.router_bias_update(cfg, l, 512)
    assert torch.equal(b0, b1)
    assert abs(float(b0.double().sum())) < 1e-3
    before = np.bincount(np_i(rcd.route(cfg, l)[0]).ravel(), minlength=E)
    after = np.bincount(np_i(rcd.route(cfg, l, b0)[0]).ravel(), minlength=E)
    fair = T * k / E
    assert before.max() > 2 * fair
    assert after.max() < 1.3 * fair
