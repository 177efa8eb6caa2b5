"""Small helpers shared by the tests (no method arithmetic)."""
import numpy as np
import torch


def f64(t):
    """torch tensor (any float dtype, any device) -> numpy float64, exactly."""
    if isinstance(t, np.ndarray):
        return t.astype(np.float64)
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)


def oracle_weights(inp):
    """The input dict as numpy fp64 arrays (router bias kept fp32)."""
    out = {}
    for k, v in inp.items():
        if k == "router_bias":
            out[k] = v.detach().cpu().numpy().astype(np.float32)
        elif k != "x":
            out[k] = f64(v)
    return out


def rowwise_rel_err(y, r):
    """max over rows of ||y_t - r_t||_inf / ||r_t||_inf (0/0 = 0)."""
    y = np.asarray(y, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    num = np.abs(y - r).max(axis=-1)
    den = np.abs(r).max(axis=-1)
    bad = (den == 0) & (num != 0)
    if bad.any():
        return float("inf")
    with np.errstate(invalid="ignore", divide="ignore"):
        q = np.where(den == 0, 0.0, num / np.where(den == 0, 1.0, den))
    return float(q.max()) if q.size else 0.0
