"""Pins of the oracle's router-bias update (CPU only).

The reading under test: per-expert equal-width histograms of this step's
logits over each expert's own range, the quantile of level 1 - k/E read off
each histogram by linear interpolation inside its bin, and the zero-mean bias
that moves every expert's quantile onto their common mean (ranhao.site notes,
section 2.2: a histogram-based quantile router whose next-step bias is
zero-mean and outside the gradient).
"""
from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import router_bias as rb


def _col(*vals):
    return np.asarray(vals, dtype=np.float32)


def test_worked_example_by_hand():
    # T = 10 tokens, E = 3 experts, k = 1, 4 bins: level q = 2/3, r = 20/3.
    # e0 = 0..9: range [0, 9], scale fl32(4/9); the bins of 0..9 are
    #    0 0 0 1 1 2 2 3 3 3 (9 * scale rounds to 4.0, clamped to 3);
    #    counts 3 2 2 3, cumulative 3 5 7 10; the first C_j >= 20/3 is j = 2;
    #    Q0 = 0 + (2 + (20/3 - 5)/2) * 9/4 = 153/24.
    # e1 = nine 0s and one 8: range [0, 8], scale 1/2; counts 9 0 0 1;
    #    j = 0; Q1 = 0 + (20/3)/9 * 2 = 40/27.
    # e2 = constant 5: scale 0, every value in bin 0; Q2 = 5 + x * 0 = 5.
    # b = mean(Q) - Q.
    l = np.stack([np.arange(10, dtype=np.float32), _col(0, 0, 0, 0, 0, 0, 0, 0, 0, 8),
                  np.full(10, 5.0, np.float32)], axis=1)
    bias, hist, lo, hi, q = rb.bias_update(l, 1, 4)
    assert hist.tolist() == [[3, 2, 2, 3], [9, 0, 0, 1], [10, 0, 0, 0]]
    assert lo.tolist() == [0, 0, 5] and hi.tolist() == [9, 8, 5]
    Q = [Fraction(153, 24), Fraction(40, 27), Fraction(5)]
    mean = sum(Q) / 3
    assert np.allclose(q, [float(x) for x in Q], rtol=0, atol=1e-15)
    assert np.allclose(bias, [float(mean - x) for x in Q], rtol=0, atol=1e-6)


def test_rank_on_a_bin_edge_takes_that_bin():
    # T = 8, E = 2, k = 1: r = 4 exactly.  e0 = 0 1 2 3 | 4 5 6 7 over two bins
    # of width 7/2: cumulative 4 8, so C_0 = r and j = 0 with the whole bin
    # consumed: Q0 = 0 + (0 + 4/4) * 7/2 = 3.5 (the edge itself).
    l = np.stack([np.arange(8, dtype=np.float32), np.arange(8, dtype=np.float32) * 2], axis=1)
    _, hist, _, _, q = rb.bias_update(l, 1, 2)
    assert hist[0].tolist() == [4, 4]
    assert q[0] == 3.5 and q[1] == 7.0


def test_rank_before_an_empty_bin_is_the_generalised_inverse():
    # counts 4 0 4 over [0, 8] in 3 bins and r = 4: the interpolated CDF is
    # flat at 1/2 across the empty middle bin; the quantile is the generalised
    # inverse inf{x : F(x) >= 1/2}, the left end of the flat stretch, 8/3
    l = np.stack([_col(0, 0, 0, 0, 8, 8, 8, 8), _col(0, 1, 2, 3, 4, 5, 6, 7)], axis=1)
    _, hist, _, _, q = rb.bias_update(l, 1, 3)
    assert hist[0].tolist() == [4, 0, 4]
    assert np.isclose(q[0], 8 / 3, rtol=0, atol=1e-15)


def _interp_quantile(hist, lo, hi, level):
    """Inverse of the piecewise-linear CDF through the bin edges (np.interp).
    Empty bins make flat steps; keeping the first edge of each distinct
    cumulative value leaves a strictly increasing CDF with the same inverse
    at every level strictly between its steps."""
    E, nb = hist.shape
    out = np.empty(E)
    for e in range(E):
        x = lo[e] + (hi[e] - float(lo[e])) * np.arange(nb + 1) / nb
        y = np.concatenate([[0], np.cumsum(hist[e])]) / hist[e].sum()
        y, first = np.unique(y, return_index=True)
        out[e] = np.interp(level, y, x[first])
    return out


@pytest.mark.parametrize("T,E,k,nb", [(4096, 16, 2, 16), (20000, 48, 8, 32), (3000, 7, 3, 8)])
def test_quantile_inverts_the_interpolated_cdf(T, E, k, nb):
    l = synth.logits_case(T, E, seed=3).numpy()
    _, hist, lo, hi, q = rb.bias_update(l, k, nb)
    ref = _interp_quantile(hist, lo.astype(np.float64), hi.astype(np.float64), 1 - k / E)
    assert np.allclose(q, ref, rtol=0, atol=1e-9)


def test_histogram_matches_numpy_on_exact_edges():
    # integer values over a power-of-two range: every edge and scale is exact,
    # so numpy's equal-width histogram (last bin closed) is the same thing
    rng = np.random.default_rng(1)
    T, E, nb = 500, 6, 16
    l = rng.integers(0, 129, size=(T, E)).astype(np.float32)
    l[0], l[1] = 0, 128                      # range [0, 128] in every column
    hist, lo, hi = rb.histograms(l, nb)
    for e in range(E):
        ref, _ = np.histogram(l[:, e], bins=nb, range=(0, 128))
        assert hist[e].tolist() == ref.tolist()


def test_histogram_near_numpy_on_random_data():
    # with arbitrary fp32 values the two differ only where a value sits within
    # rounding of an edge: a handful of moves by one bin
    l = synth.logits_case(50000, 4, seed=5).numpy()
    hist, lo, hi = rb.histograms(l, 64)
    for e in range(4):
        ref, _ = np.histogram(l[:, e].astype(np.float64), bins=64, range=(float(lo[e]), float(hi[e])))
        assert np.abs(hist[e] - ref).sum() <= 4
        assert hist[e].sum() == 50000


def test_quantile_within_one_bin_of_the_sample_quantile():
    l = synth.logits_case(16384, 32, seed=2).numpy()
    k, nb = 4, 256
    _, hist, lo, hi, q = rb.bias_update(l, k, nb)
    r = (32 - k) * 16384 / 32
    srt = np.sort(l.astype(np.float64), axis=0)
    exact = srt[int(np.ceil(r)) - 1]          # the value of rank ceil(r)
    width = (hi.astype(np.float64) - lo) / nb
    assert (np.abs(q - exact) <= width * 1.0001).all()


def test_shift_equivariance_is_exact():
    # every column is one integer-valued base column plus an integer shift:
    # the quantiles move by the shifts and the bias is minus the centred shifts
    rng = np.random.default_rng(4)
    base = rng.integers(0, 65, size=300).astype(np.float32)
    base[:2] = [0, 64]
    c = np.array([0, 3, -7, 12, 5, -2], dtype=np.float32)
    l = base[:, None] + c[None, :]
    bias, _, _, _, q = rb.bias_update(l, 2, 32)
    assert np.all(q - c == q[0] - c[0])
    c64 = c.astype(np.float64)
    assert np.allclose(bias, -(c64 - c64.mean()), rtol=0, atol=1e-6)


def test_narrow_range_with_an_infinite_scale():
    # a range of one fp32 denormal step: n_bins / width overflows fp32; the
    # minimum stays in bin 0 and the maximum goes to the last bin
    tiny = np.float32(1e-40)
    l = np.stack([_col(0, tiny, 0, tiny, tiny), _col(1, 2, 3, 4, 5)], axis=1)
    hist, lo, hi = rb.histograms(l, 64)
    assert rb.bin_scale(lo, hi, 64)[0] == np.inf
    assert hist[0, 0] == 2 and hist[0, 63] == 3 and hist[0].sum() == 5


def test_adding_a_constant_to_every_logit_leaves_the_bias():
    rng = np.random.default_rng(6)
    l = rng.integers(-40, 41, size=(400, 9)).astype(np.float32)
    b0 = rb.bias_update(l, 2, 16)[0]
    b1 = rb.bias_update(l + 256, 2, 16)[0]
    assert np.array_equal(b0, b1)


def test_zero_mean():
    l = synth.logits_case(4096, 64, seed=8).numpy()
    bias = rb.bias_update(l, 8, 128)[0]
    assert abs(float(bias.astype(np.float64).sum())) <= 1e-5 * float(np.abs(bias).max()) * 64


def test_special_levels():
    l = synth.logits_case(1000, 6, seed=9).numpy()
    # k = E: level 0, the quantile is each expert's minimum
    _, _, lo, hi, q = rb.bias_update(l, 6, 32)
    assert np.array_equal(q, lo.astype(np.float64))
    # one bin: the quantile interpolates linearly between min and max
    _, _, lo, hi, q = rb.bias_update(l, 2, 1)
    ref = lo.astype(np.float64) + (1000 * 4 / 6) / 1000 * (hi.astype(np.float64) - lo)
    assert np.allclose(q, ref, rtol=0, atol=1e-12)


def test_the_bias_balances_a_skewed_router():
    # the purpose: logits with a Zipf-like per-expert offset load the experts
    # very unevenly; adding the next-step bias evens the top-k counts out
    T, E, k = 16384, 64, 4
    skew = synth.zipf_bias(E, seed=0, beta=1.0).numpy()
    l = (synth.logits_case(T, E, seed=11).numpy() + skew[None, :]).astype(np.float32)
    import oracle
    zero = np.zeros(E, np.float32)
    before = np.bincount(oracle.route_topk(l, zero, k).ravel(), minlength=E)
    bias = rb.bias_update(l, k, 512)[0]
    after = np.bincount(oracle.route_topk(l, bias, k).ravel(), minlength=E)
    fair = T * k / E
    assert before.max() > 3 * fair
    assert after.max() < 1.25 * fair and after.min() > 0.75 * fair
    # and the bias undoes the offset up to a constant
    d = bias + (skew - skew.mean())
    assert np.abs(d - d.mean()).max() < 0.1


def test_bad_arguments():
    l = synth.logits_case(8, 4, seed=0).numpy()
    with pytest.raises(ValueError):
        rb.bias_update(l, 5, 4)
    with pytest.raises(ValueError):
        rb.bias_update(l, 0, 4)
    with pytest.raises(ValueError):
        rb.bias_update(l, 2, 0)
    with pytest.raises(ValueError):
        rb.bias_update(l[:0], 2, 4)
