"""CPU oracle of the router's balancing-bias update: the next step's
zero-mean bias from a histogram-based quantile of each expert's logits.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test suite, the smoke check and the benchmark's
CPU-baseline leg use it.  It shares no code with the HIP library.

Source: [RH] ranhao.site, "Marin 535B-A23B：一场完全公开的前沿 MoE 训练直播",
§2.2 "MoE 详解" (the routing box of the MoE diagram and the last design
point): top-8 routing is done by a quantile router built on histograms; the
bias it adds is zero-mean, is computed for the next step, is a heuristic that
balances expert selection, and receives no gradient.

The page names the ingredients but not the rule.  The reading implemented
here (each step is also listed, with its reason, in the repository's design
notes):
  1. per expert e, the range [lo_e, hi_e] of its logit over the step's T
     tokens;
  2. an n_bins-bin equal-width histogram of that column over its range.  The
     bin of a value v is decided in fp32: scale_e = fl32(n_bins / (hi_e -
     lo_e)) (the quotient of the exact difference, rounded once in fp64 and
     then to fp32; 0 when hi_e = lo_e), bin = min(n_bins - 1,
     trunc(fl32(fl32(v - lo_e) * scale_e)));
  3. the quantile of level q = 1 - k/E read off the histogram with linear
     interpolation inside the bin that holds rank r = q * T (the
     grouped-data quantile: values spread uniformly across a bin).  At level
     q an expert's logit exceeds Q_e on a k/E share of the tokens, which is
     its fair share of the T*k assignments;
  4. b_e = -(Q_e - mean_e' Q_e'): shifting every expert's quantile onto the
     common mean makes the shares equal under a threshold view of top-k, and
     the mean is removed so the bias is zero-mean.  The new bias depends
     only on this step's raw logits; an incremental update from the biased
     scores gives the same value in exact arithmetic, since a shift of a
     column shifts its quantile by the same amount.

Parity: the histogram counts and ranges are integers or exact fp32 values and
are compared bit for bit; the quantile and the bias are fp64 arithmetic on
them, rounded to fp32 at the end.
"""
from __future__ import annotations

import numpy as np


def logit_range(logits32):
    """Per-expert (lo, hi) = (min, max) over tokens, fp32 (exact)."""
    l = np.asarray(logits32, dtype=np.float32)
    if l.ndim != 2 or l.shape[0] < 1:
        raise ValueError("logits must be [T >= 1, E]")
    return l.min(axis=0), l.max(axis=0)


def bin_scale(lo, hi, n_bins):
    """scale_e = fl32(n_bins / (hi_e - lo_e)), 0 for a constant column.

    The difference of two fp32 values is exact in fp64; the quotient is
    rounded to fp64 and then to fp32 (inf when a range is narrower than
    n_bins / FLT_MAX)."""
    lo64 = np.asarray(lo, dtype=np.float32).astype(np.float64)
    hi64 = np.asarray(hi, dtype=np.float32).astype(np.float64)
    width = hi64 - lo64
    out = np.zeros_like(width)
    nz = width > 0
    out[nz] = float(n_bins) / width[nz]
    with np.errstate(over="ignore"):
        return out.astype(np.float32)


def bin_index(logits32, lo, scale, n_bins):
    """bin[t, e] = min(n_bins - 1, trunc(fl32(fl32(v - lo_e) * scale_e))).

    v >= lo_e, so the product is >= 0 and truncation is the floor; a value
    equal to lo_e is in bin 0 whatever the scale (also an infinite one)."""
    l = np.asarray(logits32, dtype=np.float32)
    d = (l - np.asarray(lo, dtype=np.float32)[None, :]).astype(np.float32)
    with np.errstate(invalid="ignore", over="ignore"):
        p = (d * np.asarray(scale, dtype=np.float32)[None, :]).astype(np.float32)
    b = np.where(p >= n_bins, np.float32(n_bins - 1), p)
    b = np.where(d == 0, np.float32(0), b)
    return b.astype(np.int64)


def histograms(logits32, n_bins):
    """[E][n_bins] int64 counts of each expert's logits over its own range,
    with the (lo, hi) the bins were drawn over."""
    if n_bins < 1:
        raise ValueError("n_bins >= 1")
    lo, hi = logit_range(logits32)
    scale = bin_scale(lo, hi, n_bins)
    b = bin_index(logits32, lo, scale, n_bins)
    E = b.shape[1]
    h = np.zeros((E, n_bins), dtype=np.int64)
    for e in range(E):
        h[e] = np.bincount(b[:, e], minlength=n_bins)
    return h, lo, hi


def histogram_quantile(hist, lo, hi, T, top_k):
    """Q_e at level q = 1 - k/E by linear interpolation inside the bin.

    r = (E - k) * T / E is the target rank.  j is the first bin whose
    cumulative count C_j satisfies C_j >= r (decided exactly in integers:
    C_j * E >= (E - k) * T).  Then
        Q_e = lo_e + (j + (r - C_{j-1}) / h_j) * (hi_e - lo_e) / n_bins
    in fp64, with C_{-1} = 0."""
    hist = np.asarray(hist, dtype=np.int64)
    E, n_bins = hist.shape
    if not 1 <= top_k <= E:
        raise ValueError("top_k out of range")
    r_num = (E - top_k) * T            # r * E, exact
    r = r_num / E
    lo64 = np.asarray(lo, dtype=np.float32).astype(np.float64)
    hi64 = np.asarray(hi, dtype=np.float32).astype(np.float64)
    q = np.empty(E, dtype=np.float64)
    for e in range(E):
        c = np.cumsum(hist[e])
        if c[-1] != T:
            raise ValueError("histogram does not hold T values")
        j = int(np.argmax(c * E >= r_num))
        c_prev = int(c[j - 1]) if j > 0 else 0
        frac = (r - c_prev) / int(hist[e, j])
        width = (hi64[e] - lo64[e]) / n_bins
        q[e] = lo64[e] + (j + frac) * width
    return q


def bias_update(logits32, top_k, n_bins):
    """Next step's router bias [E] fp32 from this step's logits [T][E] fp32.

    Returns (bias, hist, lo, hi, q): the bias and the intermediate results
    (integer counts, fp32 ranges and fp64 quantiles) that parity compares."""
    l = np.asarray(logits32, dtype=np.float32)
    T = l.shape[0]
    hist, lo, hi = histograms(l, n_bins)
    q = histogram_quantile(hist, lo, hi, T, top_k)
    bias = (-(q - q.mean())).astype(np.float32)
    return bias, hist, lo, hi, q
