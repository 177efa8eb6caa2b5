"""Seeded synthetic inputs for the pooled-wave MoE branch.

This module is the only code that both the fp64 oracle side and the GPU side
use.  It builds workload shapes and draws random tensors; it performs none of
the method's arithmetic (no routing, no capacity math, no expert compute).

Every tensor is drawn from its own seeded torch generator, so a tensor does
not change when another tensor's shape changes.  Values are drawn in fp32 and
cast (round-to-nearest-even) to bf16 for bf16 workloads.  Weights W of shape
[out, in] are N(0,1)/sqrt(in); activations x are N(0,1).

The workloads stand in for the pages' training data (a trained router on real
text), which is not available: the tokens are iid, so they carry no sequence
structure.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import torch

# --------------------------------------------------------------------------
# workload shapes
# --------------------------------------------------------------------------


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d_model: int
    d_latent: int
    n_experts: int
    n_pools: int
    top_k: int
    d_ff: int
    n_shared: int
    d_ff_shared: int
    n_waves: int
    dtype: str                 # "f32" or "bf16"
    bias: str                  # "zero", "normal", "zipf"
    bias_std: float = 0.0
    send_cap: tuple = (11, 10)  # sender capacity factor 1.10 as a rational
    recv_cap: tuple = (23, 20)  # receiver capacity factor 1.15 as a rational
    cap_send_rows: int = 0      # explicit per-(wave, pool) rows, 0 = derived
    cap_recv_rows: int = 0      # explicit per-(wave, expert) rows, 0 = derived

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS: Dict[str, Workload] = {
    # tiny fp32 case: 16 experts in 4 pools, top-2
    "tiny_fp32": Workload("tiny_fp32", T=256, d_model=256, d_latent=128,
                          n_experts=16, n_pools=4, top_k=2, d_ff=128,
                          n_shared=2, d_ff_shared=128, n_waves=3,
                          dtype="f32", bias="zero"),
    # mid-size bf16 case: one 4K sequence, 64 experts in 16 pools, top-8
    "mid_bf16": Workload("mid_bf16", T=4096, d_model=1024, d_latent=512,
                         n_experts=64, n_pools=16, top_k=8, d_ff=512,
                         n_shared=2, d_ff_shared=512, n_waves=3,
                         dtype="bf16", bias="normal", bias_std=0.01),
    # Marin-shaped layer: 4 x 4096 tokens, 6144 -> 3072 latent, 384 experts
    # in 64 pools of 6, top-8, 2 shared experts
    "marin_16k": Workload("marin_16k", T=16384, d_model=6144, d_latent=3072,
                          n_experts=384, n_pools=64, top_k=8, d_ff=3072,
                          n_shared=2, d_ff_shared=3072, n_waves=3,
                          dtype="bf16", bias="zero"),
    # long-context stress: one 65536-token sequence, Zipf-skewed popularity
    "zipf_64k": Workload("zipf_64k", T=65536, d_model=6144, d_latent=3072,
                         n_experts=384, n_pools=64, top_k=8, d_ff=3072,
                         n_shared=2, d_ff_shared=3072, n_waves=3,
                         dtype="bf16", bias="zipf"),
}

# The receive-side share of one EP64 rank: 6 local experts, 3 wave slabs of
# ceil(100489 / 3) = 33497 rows each, 65536 tokens x top-8 returning to it.
RECV_SHARE = dict(name="recv_share", T=65536, top_k=8, n_local=6, n_waves=3,
                  d_latent=3072, d_ff=3072, cap_total=100489,
                  cap_wave=-(-100489 // 3), dtype="bf16")

# Zipf exponent-matching bias scale for the skewed workload.  Derived by
# tests/golden/calibrate_zipf_beta.py (bisection so that the log-log slope of
# per-expert top-8 counts vs popularity rank is -1.1 for iid N(0,1) logits);
# the stored result lives in tests/golden/zipf_beta.json.
ZIPF_BETA = 0.474


def workload(name: str, **overrides) -> Workload:
    w = WORKLOADS[name]
    return w.replace(**overrides) if overrides else w


# --------------------------------------------------------------------------
# generators
# --------------------------------------------------------------------------

# tensor ids: one independent stream per tensor
_TID = dict(x=1, w_latent=2, w_router=3, router_bias=4, w_gate=5, w_up=6,
            w_down=7, w_up_proj=8, ws_gate=9, ws_up=10, ws_down=11,
            zipf_perm=12, share_rows=13, share_counts=14, share_perm=15,
            share_logits=16, dy_latent=17)


def _seed(seed: int, tid: int, sub: int = 0) -> int:
    # a fixed, collision-free packing of (seed, tensor, sub-stream)
    return (int(seed) & 0xFFFF) << 40 | (tid & 0xFF) << 32 | (sub & 0xFFFFFFFF)


def _gen(device, seed, tid, sub=0) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed(seed, tid, sub))
    return g


def torch_dtype(dtype: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]


def normal(shape, seed, tid, device="cpu", scale=1.0, dtype="f32", sub=0):
    g = _gen(device, seed, tid, sub)
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if scale != 1.0:
        t.mul_(scale)
    return t.to(torch_dtype(dtype))


def _weight(shape, seed, name, device, dtype):
    fan_in = shape[-1]
    return normal(shape, seed, _TID[name], device, 1.0 / math.sqrt(fan_in), dtype)


def zipf_bias(E: int, seed: int, beta: float = ZIPF_BETA) -> torch.Tensor:
    """b_e = -beta * ln(r_e), r a seeded permutation of 1..E (fp32, CPU)."""
    g = _gen("cpu", seed, _TID["zipf_perm"])
    r = torch.randperm(E, generator=g).to(torch.float64) + 1.0
    return (-beta * torch.log(r)).to(torch.float32)


def router_bias(w: Workload, seed: int, device="cpu") -> torch.Tensor:
    if w.bias == "zero":
        b = torch.zeros(w.n_experts, dtype=torch.float32)
    elif w.bias == "normal":
        b = normal((w.n_experts,), seed, _TID["router_bias"], "cpu", w.bias_std)
    elif w.bias == "zipf":
        b = zipf_bias(w.n_experts, seed)
    else:
        raise ValueError(w.bias)
    return b.to(device)


def make_inputs(w: Workload, seed: int = 0, device="cpu",
                with_experts: bool = True) -> Dict[str, torch.Tensor]:
    """All tensors of one forward call.

    Layouts (row-major, [out, in] for every weight, as torch.nn.Linear):
      x [T, D]; w_latent [L, D]; w_router [E, L]; router_bias [E] (fp32);
      w_gate, w_up [E, F, L]; w_down [E, L, F]; w_up_proj [D, L];
      ws_gate, ws_up [S, Fs, D]; ws_down [S, D, Fs].
    """
    dt = w.dtype
    T, D, L, E, F = w.T, w.d_model, w.d_latent, w.n_experts, w.d_ff
    S, Fs = w.n_shared, w.d_ff_shared
    out = dict(
        x=normal((T, D), seed, _TID["x"], device, 1.0, dt),
        w_latent=_weight((L, D), seed, "w_latent", device, dt),
        w_router=_weight((E, L), seed, "w_router", device, dt),
        router_bias=router_bias(w, seed, device),
        w_up_proj=_weight((D, L), seed, "w_up_proj", device, dt),
        ws_gate=_weight((S, Fs, D), seed, "ws_gate", device, dt),
        ws_up=_weight((S, Fs, D), seed, "ws_up", device, dt),
        ws_down=_weight((S, D, Fs), seed, "ws_down", device, dt),
    )
    if with_experts:
        out.update(expert_weights(w, seed, device))
    return out


def grad_latent(w: Workload, seed: int = 0, device="cpu") -> torch.Tensor:
    """dL/dy_latent [T, L] for the routed-path backward: N(0, 1) rows in the
    workload's dtype (a stand-in for the gradient a training step brings)."""
    return normal((w.T, w.d_latent), seed, _TID["dy_latent"], device, 1.0, w.dtype)


def expert_weights(w: Workload, seed: int, device="cpu"):
    dt = w.dtype
    E, F, L = w.n_experts, w.d_ff, w.d_latent
    return dict(
        w_gate=_weight((E, F, L), seed, "w_gate", device, dt),
        w_up=_weight((E, F, L), seed, "w_up", device, dt),
        w_down=_weight((E, L, F), seed, "w_down", device, dt),
    )


# --------------------------------------------------------------------------
# receive-side share of one EP rank
# --------------------------------------------------------------------------


def make_recv_share(seed: int = 0, device="cpu", T: Optional[int] = None,
                    n_local: Optional[int] = None, d_latent: Optional[int] = None,
                    d_ff: Optional[int] = None, cap_wave: Optional[int] = None,
                    top_k: int = 8, n_waves: int = 3):
    """Synthetic receive bank of one EP rank (inputs only).

    The bank holds, per wave, one block of n_local * cap_wave rows: local
    expert e owns slots [e*cap_wave, (e+1)*cap_wave).  Each of the rank's T
    tokens x top_k assignments is mapped to exactly one bank row: the
    assignments of wave w (tokens [w*Tw, (w+1)*Tw), Tw = ceil(T/n_waves)) are
    dealt to local experts with multinomial counts (equal probabilities) and
    placed in a seeded random order.  Returned index tensors describe that
    placement; rows beyond an expert's count are unused (id -1).
    """
    R = RECV_SHARE
    T = R["T"] if T is None else T
    n_local = R["n_local"] if n_local is None else n_local
    L = R["d_latent"] if d_latent is None else d_latent
    F = R["d_ff"] if d_ff is None else d_ff
    cw = R["cap_wave"] if cap_wave is None else cap_wave
    W, k = n_waves, top_k
    Tw = -(-T // W)
    gcpu = _gen("cpu", seed, _TID["share_counts"])
    expert_of = torch.empty((T, k), dtype=torch.int32)
    slot_of = torch.empty((T, k), dtype=torch.int32)
    counts = torch.zeros((W, n_local), dtype=torch.int32)
    for wv in range(W):
        t0, t1 = wv * Tw, min(T, (wv + 1) * Tw)
        n = (t1 - t0) * k
        # multinomial deal of the wave's n assignments over local experts
        probs = torch.full((n_local,), 1.0 / n_local, dtype=torch.float64)
        draw = torch.multinomial(probs, n, replacement=True, generator=gcpu)
        c = torch.bincount(draw, minlength=n_local).to(torch.int32)
        if int(c.max()) > cw:
            raise ValueError("multinomial draw exceeds the wave capacity")
        counts[wv] = c
        # seeded placement: assignment a of the wave gets expert draw[a] and
        # that expert's next free slot in a random order of the slots
        perm = torch.randperm(n, generator=gcpu)
        e_sorted = draw[perm]
        order = torch.argsort(e_sorted, stable=True)
        rank = torch.empty(n, dtype=torch.int64)
        starts = torch.cumsum(torch.cat([torch.zeros(1, dtype=torch.int64),
                                         c.to(torch.int64)]), 0)
        rank[order] = torch.arange(n) - starts[e_sorted[order]]
        ex = torch.empty(n, dtype=torch.int32)
        sl = torch.empty(n, dtype=torch.int32)
        ex[perm] = e_sorted.to(torch.int32)
        sl[perm] = (e_sorted.to(torch.int64) * cw + rank).to(torch.int32)
        expert_of[t0:t1] = ex.view(t1 - t0, k)
        slot_of[t0:t1] = sl.view(t1 - t0, k)
    rows = normal((W, n_local * cw, L), seed, _TID["share_rows"], device, 1.0, "bf16")
    # gate weights: Dirichlet(1, ..., 1) per token (normalised exponential
    # spacings), i.e. positive weights summing to one
    gu = _gen("cpu", seed, _TID["share_logits"])
    spac = -torch.log1p(-torch.rand((T, k), generator=gu, dtype=torch.float64))
    gates = (spac / spac.sum(dim=1, keepdim=True)).to(torch.float32)
    wts = dict(
        w_gate=_weight((n_local, F, L), seed, "w_gate", device, "bf16"),
        w_up=_weight((n_local, F, L), seed, "w_up", device, "bf16"),
        w_down=_weight((n_local, L, F), seed, "w_down", device, "bf16"),
    )
    return dict(T=T, k=k, W=W, Tw=Tw, n_local=n_local, L=L, F=F, cap_wave=cw,
                rows=rows, counts=counts, expert_of=expert_of, slot_of=slot_of,
                gates=gates, **wts)


# --------------------------------------------------------------------------
# inputs of single-step cases
# --------------------------------------------------------------------------

_CASE = dict(logits=20, topk=21, rows=22, gates=23, bias=24)


def logits_case(T: int, E: int, seed: int, kind: str = "normal") -> torch.Tensor:
    """fp32 router logits [T, E] (CPU).

    normal: N(0, 1).  ties: multiples of 0.5 in [-1.5, 1.0] with signed zeros,
    so equal scores are common.  tiny: N(0, 1) * 2^-20 plus 1.0, so scores
    differ in the last bits of fp32.
    """
    g = _gen("cpu", seed, _CASE["logits"], T * 4096 + E)
    if kind == "normal":
        return torch.randn((T, E), generator=g, dtype=torch.float32)
    if kind == "ties":
        v = torch.randint(-3, 3, (T, E), generator=g).to(torch.float32) * 0.5
        neg = torch.rand((T, E), generator=g) < 0.5
        return torch.where((v == 0) & neg, torch.full_like(v, -0.0), v)
    if kind == "tiny":
        return 1.0 + torch.randn((T, E), generator=g, dtype=torch.float32) * 2.0 ** -20
    raise ValueError(kind)


def bias_case(E: int, seed: int, std: float) -> torch.Tensor:
    g = _gen("cpu", seed, _CASE["bias"], E)
    return torch.randn(E, generator=g, dtype=torch.float32) * std


def topk_case(T: int, E: int, k: int, seed: int, skew: float = 0.0) -> torch.Tensor:
    """int32 [T, k]: k distinct experts per token, drawn without replacement
    with probabilities proportional to exp(-skew * rank(e)) for a seeded
    popularity order (Gumbel-top-k sampling)."""
    g = _gen("cpu", seed, _CASE["topk"], T * 4096 + E * 64 + k)
    order = torch.randperm(E, generator=g)
    logp = torch.empty(E, dtype=torch.float64)
    logp[order] = -skew * torch.arange(E, dtype=torch.float64)
    u = torch.rand((T, E), generator=g, dtype=torch.float64).clamp_min(1e-300)
    keys = logp[None, :] - torch.log(-torch.log(u))
    return torch.topk(keys, k, dim=1).indices.to(torch.int32)


def rows_case(n: int, L: int, seed: int, dtype: str, sub: int = 0) -> torch.Tensor:
    """[n, L] N(0, 1) rows (CPU), e.g. activations or expert outputs."""
    return normal((n, L), seed, _CASE["rows"], "cpu", 1.0, dtype, sub=sub)


def gates_case(T: int, k: int, seed: int) -> torch.Tensor:
    """fp32 [T, k] positive weights summing to one (Dirichlet(1))."""
    g = _gen("cpu", seed, _CASE["gates"], T * 64 + k)
    spac = -torch.log1p(-torch.rand((T, k), generator=g, dtype=torch.float64))
    return (spac / spac.sum(dim=1, keepdim=True)).to(torch.float32)
