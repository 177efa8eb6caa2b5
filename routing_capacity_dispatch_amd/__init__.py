"""Pooled-wave capacity-dispatch MoE branch (forward, and the backward of its
routed path) for MI355X / gfx950.

Thin torch binding over the C ABI in include/moe.h (libmoe.so).  torch only
provides device memory and the current stream; every step of the branch runs
in the HIP kernels of the library.  The same names as the C entry points:
route, dispatch, experts, combine, forward, their *_backward transposes and
BackwardRouted (moe_backward_routed), plus make_config / plan.
"""
from __future__ import annotations

import ctypes as C
from typing import Dict, Optional

import torch

from . import abi

__all__ = ["make_config", "plan", "route", "dispatch", "experts", "combine", "forward",
           "dispatch_dropless", "experts_dropless", "combine_dropless", "forward_dropless",
           "combine_backward", "experts_backward", "dispatch_backward", "route_backward",
           "combine_backward_dropless", "experts_backward_dropless", "dispatch_backward_dropless",
           "BackwardRouted", "library", "MoeError"]

MoeError = abi.MoeError
_DT = {"f32": abi.MOE_F32, "bf16": abi.MOE_BF16, torch.float32: abi.MOE_F32,
       torch.bfloat16: abi.MOE_BF16}


def library():
    return abi.load()


def make_config(T, d_model, d_latent, n_experts, n_pools, top_k, d_ff, n_shared=0,
                d_ff_shared=0, n_waves=3, dtype="bf16", send_cap=(11, 10), recv_cap=(23, 20),
                cap_send_rows=0, cap_recv_rows=0) -> abi.MoeConfig:
    return abi.MoeConfig(
        T=T, d_model=d_model, d_latent=d_latent, n_experts=n_experts, n_pools=n_pools,
        top_k=top_k, d_ff=d_ff, n_shared=n_shared, d_ff_shared=d_ff_shared, n_waves=n_waves,
        send_cap_num=send_cap[0], send_cap_den=send_cap[1], recv_cap_num=recv_cap[0],
        recv_cap_den=recv_cap[1], cap_send_rows=cap_send_rows, cap_recv_rows=cap_recv_rows,
        dtype=_DT[dtype], reserved=0)


def config_of(w, **over) -> abi.MoeConfig:
    """Config from any object with the workload attribute names."""
    f = dict(T=w.T, d_model=w.d_model, d_latent=w.d_latent, n_experts=w.n_experts,
             n_pools=w.n_pools, top_k=w.top_k, d_ff=w.d_ff, n_shared=w.n_shared,
             d_ff_shared=w.d_ff_shared, n_waves=w.n_waves, dtype=w.dtype,
             send_cap=tuple(w.send_cap), recv_cap=tuple(w.recv_cap),
             cap_send_rows=getattr(w, "cap_send_rows", 0),
             cap_recv_rows=getattr(w, "cap_recv_rows", 0))
    f.update(over)
    return make_config(**f)


def plan(cfg: abi.MoeConfig) -> Dict[str, int]:
    p = abi.MoePlan()
    abi.check("moe_make_plan", library().moe_make_plan(C.byref(cfg), C.byref(p)))
    return p.as_dict()


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(device=None):
    return C.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _tdt(cfg):
    return torch.bfloat16 if cfg.dtype == abi.MOE_BF16 else torch.float32


def _ws(nbytes, device):
    # 256-byte aligned: torch's caching allocator returns 512-byte aligned blocks
    t = torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)
    assert t.data_ptr() % 256 == 0
    return t


def route(cfg, logits: torch.Tensor, bias: Optional[torch.Tensor] = None, out=None):
    T, k = cfg.T, cfg.top_k
    dev = logits.device
    topk = out["topk_idx"] if out else torch.empty((T, k), dtype=torch.int32, device=dev)
    gates = out["gates"] if out else torch.empty((T, k), dtype=torch.float32, device=dev)
    abi.check("moe_route", library().moe_route(
        C.byref(cfg), _ptr(logits), _ptr(bias), _ptr(topk), _ptr(gates), _stream(dev)))
    return topk, gates


def router_bias_ws_bytes(cfg, n_bins: int) -> int:
    n = C.c_size_t(0)
    abi.check("moe_router_bias_ws_bytes", library().moe_router_bias_ws_bytes(C.byref(cfg), n_bins, C.byref(n)))
    return int(n.value)


def router_bias_update(cfg, logits: torch.Tensor, n_bins: int, with_hist: bool = False, ws=None, out=None):
    """Next step's zero-mean router bias [E] fp32 from this step's logits
    [T][E] fp32 (moe_router_bias_update).  With with_hist, also the
    per-expert counts [E][n_bins] int32 and ranges [E][2] fp32."""
    dev = logits.device
    E = cfg.n_experts
    bias = out if out is not None else torch.empty(E, dtype=torch.float32, device=dev)
    hist = torch.empty((E, n_bins), dtype=torch.int32, device=dev) if with_hist else None
    lohi = torch.empty((E, 2), dtype=torch.float32, device=dev) if with_hist else None
    if ws is None:
        ws = _ws(router_bias_ws_bytes(cfg, n_bins), dev)
    abi.check("moe_router_bias_update", library().moe_router_bias_update(
        C.byref(cfg), _ptr(logits), n_bins, _ptr(bias), _ptr(hist), _ptr(lohi), _ptr(ws), ws.numel(),
        _stream(dev)))
    return (bias, hist, lohi) if with_hist else bias


class RouterBias:
    """moe_router_bias_update with its workspace and output allocated once:
    call it with each step's logits [T][E] fp32; it returns the next step's
    bias [E] fp32 (the same tensor every call)."""

    def __init__(self, cfg, n_bins: int, device):
        self.cfg, self.n_bins = cfg, n_bins
        self.ws = _ws(router_bias_ws_bytes(cfg, n_bins), device)
        self.bias = torch.empty(cfg.n_experts, dtype=torch.float32, device=device)

    def __call__(self, logits: torch.Tensor):
        return router_bias_update(self.cfg, logits, self.n_bins, ws=self.ws, out=self.bias)

    def profiled(self, logits: torch.Tensor, events):
        arr = (C.c_void_p * len(events))(*[C.c_void_p(e.cuda_event) for e in events])
        abi.check("moe_router_bias_update_profiled", library().moe_router_bias_update_profiled(
            C.byref(self.cfg), _ptr(logits), self.n_bins, _ptr(self.bias), None, None, _ptr(self.ws),
            self.ws.numel(), _stream(logits.device), arr, len(events)))
        return self.bias


def router_bias_stage_count() -> int:
    return library().moe_router_bias_stage_count()


def dispatch(cfg, topk_idx: torch.Tensor, z: torch.Tensor) -> Dict[str, torch.Tensor]:
    p = plan(cfg)
    dev = z.device
    T, k, W, P, E = cfg.T, cfg.top_k, cfg.n_waves, cfg.n_pools, cfg.n_experts
    out = dict(
        pools=torch.empty(p["pools_bytes"], dtype=torch.uint8, device=dev),
        pool_slot=torch.empty((T, k), dtype=torch.int32, device=dev),
        recv_slot=torch.empty((T, k), dtype=torch.int32, device=dev),
        bank_rows=torch.full((W, E, max(p["cap_recv"], 0)), -1, dtype=torch.int32, device=dev),
        pool_count=torch.empty((W, P), dtype=torch.int32, device=dev),
        expert_count=torch.empty((W, E), dtype=torch.int32, device=dev),
        counts=torch.empty(3, dtype=torch.int64, device=dev),
    )
    ws = _ws(p["dispatch_ws_bytes"], dev)
    abi.check("moe_dispatch", library().moe_dispatch(
        C.byref(cfg), _ptr(topk_idx), _ptr(z), _ptr(out["pools"]), _ptr(out["pool_slot"]),
        _ptr(out["recv_slot"]), _ptr(out["bank_rows"]), _ptr(out["pool_count"]),
        _ptr(out["expert_count"]), _ptr(out["counts"]), _ptr(ws), ws.numel(), _stream(dev)))
    out["plan"] = p
    return out


def dispatch_noalloc(cfg, topk_idx: torch.Tensor, z: torch.Tensor, out: Dict[str, torch.Tensor]):
    """moe_dispatch_noalloc into caller-provided outputs (the dict that
    dispatch() returns, or one shaped like it); allocates nothing."""
    abi.check("moe_dispatch_noalloc", library().moe_dispatch_noalloc(
        C.byref(cfg), _ptr(topk_idx), _ptr(z), _ptr(out["pools"]), _ptr(out["pool_slot"]),
        _ptr(out["recv_slot"]), _ptr(out["bank_rows"]), _ptr(out["pool_count"]),
        _ptr(out["expert_count"]), _ptr(out["counts"]), _stream(z.device)))
    return out


def dispatch_noalloc_scratch_bytes() -> int:
    return library().moe_dispatch_noalloc_scratch_bytes()


def pool_views(cfg, pools: torch.Tensor):
    """(rows [W, P, C_send, L], ids [W, P, C_send]) views of a pools buffer."""
    p = plan(cfg)
    W, P = cfg.n_waves, cfg.n_pools
    cs, blk = p["cap_send"], p["pool_block_bytes"]
    if cs == 0:
        return (torch.empty((W, P, 0, cfg.d_latent), dtype=_tdt(cfg), device=pools.device),
                torch.empty((W, P, 0), dtype=torch.int32, device=pools.device))
    b = pools.view(W, P, blk)
    rows = b[:, :, :p["ids_offset"]].view(_tdt(cfg)).view(W, P, cs, cfg.d_latent)
    ids = b[:, :, p["ids_offset"]:p["ids_offset"] + 4 * cs].view(torch.int32).view(W, P, cs)
    return rows, ids


def experts(cfg, pools, bank_rows, expert_count, w_gate, w_up, w_down, expert_out=None):
    p = plan(cfg)
    dev = pools.device
    if expert_out is None:
        expert_out = torch.empty(p["expert_out_bytes"], dtype=torch.uint8, device=dev)
    ws = _ws(p["experts_ws_bytes"], dev)
    abi.check("moe_experts", library().moe_experts(
        C.byref(cfg), _ptr(pools), _ptr(bank_rows), _ptr(expert_count), _ptr(w_gate),
        _ptr(w_up), _ptr(w_down), _ptr(expert_out), _ptr(ws), ws.numel(), _stream(dev)))
    return expert_out


def expert_out_view(cfg, expert_out: torch.Tensor):
    p = plan(cfg)
    n = cfg.n_waves * cfg.n_pools * p["cap_send"] * cfg.d_latent
    return expert_out.view(_tdt(cfg))[:n].view(cfg.n_waves, cfg.n_pools, p["cap_send"],
                                                 cfg.d_latent)


def combine(cfg, expert_out, topk_idx, pool_slot, recv_slot, gates, y_latent=None):
    dev = expert_out.device
    if y_latent is None:
        y_latent = torch.empty((cfg.T, cfg.d_latent), dtype=_tdt(cfg), device=dev)
    abi.check("moe_combine", library().moe_combine(
        C.byref(cfg), _ptr(expert_out), _ptr(topk_idx), _ptr(pool_slot), _ptr(recv_slot),
        _ptr(gates), _ptr(y_latent), _stream(dev)))
    return y_latent


class Forward:
    """Reusable forward call: weights, workspace and outputs bound once, so a
    timed loop only enqueues kernels."""

    def __init__(self, cfg, weights: Dict[str, torch.Tensor], device, taps=False):
        self.cfg = cfg
        self.p = plan(cfg)
        self.w = weights
        self.wstruct = abi.MoeWeights(**{n: _ptr(weights.get(n)) for n, _ in
                                         abi.MoeWeights._fields_})
        self.ws = _ws(self.p["forward_ws_bytes"], device)
        self.y = torch.empty((cfg.T, cfg.d_model), dtype=_tdt(cfg), device=device)
        self.counts = torch.empty(3, dtype=torch.int64, device=device)
        self.taps = None
        self.tap_t = {}
        if taps:
            T, k, E, W, P, L = cfg.T, cfg.top_k, cfg.n_experts, cfg.n_waves, cfg.n_pools, cfg.d_latent
            dt = _tdt(cfg)
            i32 = dict(dtype=torch.int32, device=device)
            self.tap_t = dict(
                logits=torch.empty((T, E), dtype=torch.float32, device=device),
                topk_idx=torch.empty((T, k), **i32),
                gates=torch.empty((T, k), dtype=torch.float32, device=device),
                pool_slot=torch.empty((T, k), **i32),
                recv_slot=torch.empty((T, k), **i32),
                pool_count=torch.empty((W, P), **i32),
                expert_count=torch.empty((W, E), **i32),
                bank_rows=torch.full((W, E, self.p["cap_recv"]), -1, **i32),
                z=torch.empty((T, L), dtype=dt, device=device),
                pools=torch.empty(self.p["pools_bytes"], dtype=torch.uint8, device=device),
                expert_out=torch.empty(self.p["expert_out_bytes"], dtype=torch.uint8, device=device),
                y_latent=torch.empty((T, L), dtype=dt, device=device),
            )
            self.taps = abi.MoeTaps(**{n: _ptr(t) for n, t in self.tap_t.items()})

    def __call__(self, x: torch.Tensor):
        lib = library()
        abi.check("moe_forward", lib.moe_forward(
            C.byref(self.cfg), C.byref(self.wstruct), _ptr(x), _ptr(self.y),
            C.byref(self.taps) if self.taps is not None else None, _ptr(self.counts),
            _ptr(self.ws), self.ws.numel(), _stream(x.device)))
        return self.y

    def profiled(self, x: torch.Tensor, events):
        """As __call__, recording torch.cuda.Event objects (enable_timing) at
        the stage boundaries on the current stream: len(events) ==
        stage count + 1."""
        lib = library()
        arr = (C.c_void_p * len(events))(*[C.c_void_p(e.cuda_event) for e in events])
        abi.check("moe_forward_profiled", lib.moe_forward_profiled(
            C.byref(self.cfg), C.byref(self.wstruct), _ptr(x), _ptr(self.y),
            C.byref(self.taps) if self.taps is not None else None, _ptr(self.counts),
            _ptr(self.ws), self.ws.numel(), _stream(x.device), arr, len(events)))
        return self.y


def stage_count() -> int:
    return library().moe_forward_stage_count()


def forward(cfg, weights: Dict[str, torch.Tensor], x: torch.Tensor, taps=False):
    """One forward call; returns (y, counts, taps-dict)."""
    f = Forward(cfg, weights, x.device, taps=taps)
    y = f(x)
    return y, f.counts, f.tap_t


# ---------------------------------------------------------------- dropless


def dispatch_dropless(cfg, topk_idx: torch.Tensor, z: torch.Tensor) -> Dict[str, torch.Tensor]:
    """Rows ordered by expert: xs [T*k, L], row_of [T, k], expert_offsets [E+1]."""
    p = plan(cfg)
    dev = z.device
    T, k, E = cfg.T, cfg.top_k, cfg.n_experts
    out = dict(
        xs=torch.empty((p["dropless_rows"], cfg.d_latent), dtype=_tdt(cfg), device=dev),
        row_of=torch.empty((T, k), dtype=torch.int32, device=dev),
        expert_offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
        counts=torch.empty(3, dtype=torch.int64, device=dev),
    )
    ws = _ws(p["dropless_dispatch_ws_bytes"], dev)
    abi.check("moe_dispatch_dropless", library().moe_dispatch_dropless(
        C.byref(cfg), _ptr(topk_idx), _ptr(z), _ptr(out["xs"]), _ptr(out["row_of"]),
        _ptr(out["expert_offsets"]), _ptr(out["counts"]), _ptr(ws), ws.numel(), _stream(dev)))
    out["plan"] = p
    return out


def experts_dropless(cfg, xs, expert_offsets, w_gate, w_up, w_down, expert_out=None):
    p = plan(cfg)
    dev = xs.device
    if expert_out is None:
        expert_out = torch.empty((p["dropless_rows"], cfg.d_latent), dtype=_tdt(cfg), device=dev)
    ws = _ws(p["dropless_experts_ws_bytes"], dev)
    abi.check("moe_experts_dropless", library().moe_experts_dropless(
        C.byref(cfg), _ptr(xs), _ptr(expert_offsets), _ptr(w_gate), _ptr(w_up), _ptr(w_down),
        _ptr(expert_out), _ptr(ws), ws.numel(), _stream(dev)))
    return expert_out


def combine_dropless(cfg, expert_out, row_of, gates, y_latent=None):
    dev = expert_out.device
    if y_latent is None:
        y_latent = torch.empty((cfg.T, cfg.d_latent), dtype=_tdt(cfg), device=dev)
    abi.check("moe_combine_dropless", library().moe_combine_dropless(
        C.byref(cfg), _ptr(expert_out), _ptr(row_of), _ptr(gates), _ptr(y_latent), _stream(dev)))
    return y_latent


class ForwardDropless:
    """Reusable dropless forward call (weights, workspace and outputs bound once)."""

    def __init__(self, cfg, weights: Dict[str, torch.Tensor], device, taps=False):
        self.cfg = cfg
        self.p = plan(cfg)
        self.w = weights
        self.wstruct = abi.MoeWeights(**{n: _ptr(weights.get(n)) for n, _ in
                                         abi.MoeWeights._fields_})
        self.ws = _ws(self.p["dropless_forward_ws_bytes"], device)
        self.y = torch.empty((cfg.T, cfg.d_model), dtype=_tdt(cfg), device=device)
        self.counts = torch.empty(3, dtype=torch.int64, device=device)
        self.taps = None
        self.tap_t = {}
        if taps:
            T, k, E, L = cfg.T, cfg.top_k, cfg.n_experts, cfg.d_latent
            n = self.p["dropless_rows"]
            dt = _tdt(cfg)
            i32 = dict(dtype=torch.int32, device=device)
            self.tap_t = dict(
                logits=torch.empty((T, E), dtype=torch.float32, device=device),
                topk_idx=torch.empty((T, k), **i32),
                gates=torch.empty((T, k), dtype=torch.float32, device=device),
                row_of=torch.empty((T, k), **i32),
                expert_offsets=torch.empty(E + 1, **i32),
                z=torch.empty((T, L), dtype=dt, device=device),
                xs=torch.empty((n, L), dtype=dt, device=device),
                expert_out=torch.empty((n, L), dtype=dt, device=device),
                y_latent=torch.empty((T, L), dtype=dt, device=device),
            )
            self.taps = abi.MoeDroplessTaps(**{n_: _ptr(t) for n_, t in self.tap_t.items()})

    def _taps_arg(self):
        return C.byref(self.taps) if self.taps is not None else None

    def __call__(self, x: torch.Tensor):
        abi.check("moe_forward_dropless", library().moe_forward_dropless(
            C.byref(self.cfg), C.byref(self.wstruct), _ptr(x), _ptr(self.y), self._taps_arg(),
            _ptr(self.counts), _ptr(self.ws), self.ws.numel(), _stream(x.device)))
        return self.y

    def profiled(self, x: torch.Tensor, events):
        arr = (C.c_void_p * len(events))(*[C.c_void_p(e.cuda_event) for e in events])
        abi.check("moe_forward_dropless_profiled", library().moe_forward_dropless_profiled(
            C.byref(self.cfg), C.byref(self.wstruct), _ptr(x), _ptr(self.y), self._taps_arg(),
            _ptr(self.counts), _ptr(self.ws), self.ws.numel(), _stream(x.device), arr,
            len(events)))
        return self.y


def dropless_stage_count() -> int:
    return library().moe_forward_dropless_stage_count()


def forward_dropless(cfg, weights: Dict[str, torch.Tensor], x: torch.Tensor, taps=False):
    """One dropless forward call; returns (y, counts, taps-dict)."""
    f = ForwardDropless(cfg, weights, x.device, taps=taps)
    y = f(x)
    return y, f.counts, f.tap_t


# ---------------------------------------------------------------- backward
def combine_backward(cfg, expert_out, topk_idx, pool_slot, recv_slot, gates, dy_latent,
                     d_gates=None, d_expert_out=None):
    """(d_gates [T, k] fp32, d_expert_out bytes) = transpose of combine."""
    p = plan(cfg)
    dev = dy_latent.device
    if d_gates is None:
        d_gates = torch.empty((cfg.T, cfg.top_k), dtype=torch.float32, device=dev)
    if d_expert_out is None:
        d_expert_out = torch.empty(p["expert_out_bytes"], dtype=torch.uint8, device=dev)
    abi.check("moe_combine_backward", library().moe_combine_backward(
        C.byref(cfg), _ptr(expert_out), _ptr(topk_idx), _ptr(pool_slot), _ptr(recv_slot),
        _ptr(gates), _ptr(dy_latent), _ptr(d_gates), _ptr(d_expert_out), _stream(dev)))
    return d_gates, d_expert_out


def experts_backward(cfg, pools, bank_rows, expert_count, w_gate, w_up, w_down, d_expert_out,
                     d_pool_rows=None, dw=None):
    """(d_pool_rows bytes, (dw_gate, dw_up, dw_down)) = transpose of experts."""
    p = plan(cfg)
    dev = pools.device
    if d_pool_rows is None:
        d_pool_rows = torch.empty(p["expert_out_bytes"], dtype=torch.uint8, device=dev)
    if dw is None:
        dw = (torch.empty_like(w_gate), torch.empty_like(w_up), torch.empty_like(w_down))
    ws = _ws(p["experts_bwd_ws_bytes"], dev)
    abi.check("moe_experts_backward", library().moe_experts_backward(
        C.byref(cfg), _ptr(pools), _ptr(bank_rows), _ptr(expert_count), _ptr(w_gate), _ptr(w_up),
        _ptr(w_down), _ptr(d_expert_out), _ptr(d_pool_rows), _ptr(dw[0]), _ptr(dw[1]),
        _ptr(dw[2]), _ptr(ws), ws.numel(), _stream(dev)))
    return d_pool_rows, dw


def dispatch_backward(cfg, topk_idx, pool_slot, recv_slot, d_pool_rows, dz=None):
    """dz [T, L] = transpose of dispatch (sum over a token's kept rows)."""
    dev = d_pool_rows.device
    if dz is None:
        dz = torch.empty((cfg.T, cfg.d_latent), dtype=_tdt(cfg), device=dev)
    abi.check("moe_dispatch_backward", library().moe_dispatch_backward(
        C.byref(cfg), _ptr(topk_idx), _ptr(pool_slot), _ptr(recv_slot), _ptr(d_pool_rows),
        _ptr(dz), _stream(dev)))
    return dz


def route_backward(cfg, topk_idx, gates, d_gates, d_logits=None):
    """d_logits [T, E] fp32 = transpose of the gate softmax."""
    dev = gates.device
    if d_logits is None:
        d_logits = torch.empty((cfg.T, cfg.n_experts), dtype=torch.float32, device=dev)
    abi.check("moe_route_backward", library().moe_route_backward(
        C.byref(cfg), _ptr(topk_idx), _ptr(gates), _ptr(d_gates), _ptr(d_logits), _stream(dev)))
    return d_logits


class BackwardRouted:
    """Reusable routed-path backward bound to a Forward (or ForwardDropless)
    built with taps=True: its saved routing, rows and expert outputs feed the
    gradient (moe_backward_routed, or moe_backward_dropless)."""

    def __init__(self, fwd):
        if fwd.taps is None:
            raise ValueError("the forward must keep its taps (taps=True)")
        cfg, dev = fwd.cfg, fwd.y.device
        self.cfg, self.fwd = cfg, fwd
        self.p = fwd.p
        self.dropless = isinstance(fwd, ForwardDropless)
        self.ws = _ws(self.p["dropless_backward_ws_bytes" if self.dropless else "backward_ws_bytes"], dev)
        self.dz = torch.empty((cfg.T, cfg.d_latent), dtype=_tdt(cfg), device=dev)
        self.d_logits = torch.empty((cfg.T, cfg.n_experts), dtype=torch.float32, device=dev)
        w = fwd.w
        self.dw = (torch.empty_like(w["w_gate"]), torch.empty_like(w["w_up"]),
                   torch.empty_like(w["w_down"]))

    def _args(self, dy_latent):
        return (C.byref(self.cfg), C.byref(self.fwd.wstruct), C.byref(self.fwd.taps),
                _ptr(dy_latent), _ptr(self.dz), _ptr(self.d_logits), _ptr(self.dw[0]),
                _ptr(self.dw[1]), _ptr(self.dw[2]), _ptr(self.ws), self.ws.numel(),
                _stream(dy_latent.device))

    def __call__(self, dy_latent: torch.Tensor):
        name = "moe_backward_dropless" if self.dropless else "moe_backward_routed"
        abi.check(name, getattr(library(), name)(*self._args(dy_latent)))
        return self.dz, self.d_logits, self.dw

    def profiled(self, dy_latent: torch.Tensor, events):
        arr = (C.c_void_p * len(events))(*[C.c_void_p(e.cuda_event) for e in events])
        name = "moe_backward_dropless_profiled" if self.dropless else "moe_backward_routed_profiled"
        abi.check(name, getattr(library(), name)(*self._args(dy_latent), arr, len(events)))
        return self.dz, self.d_logits, self.dw


def backward_stage_count() -> int:
    return library().moe_backward_routed_stage_count()


def combine_backward_dropless(cfg, expert_out, row_of, gates, dy_latent, d_gates=None,
                              d_expert_out=None):
    """(d_gates [T, k] fp32, d_expert_out [T*k, L]) = transpose of combine_dropless."""
    dev = dy_latent.device
    if d_gates is None:
        d_gates = torch.empty((cfg.T, cfg.top_k), dtype=torch.float32, device=dev)
    if d_expert_out is None:
        d_expert_out = torch.empty_like(expert_out)
    abi.check("moe_combine_backward_dropless", library().moe_combine_backward_dropless(
        C.byref(cfg), _ptr(expert_out), _ptr(row_of), _ptr(gates), _ptr(dy_latent), _ptr(d_gates),
        _ptr(d_expert_out), _stream(dev)))
    return d_gates, d_expert_out


def experts_backward_dropless(cfg, xs, expert_offsets, w_gate, w_up, w_down, d_expert_out,
                              d_xs=None, dw=None):
    """(d_xs [T*k, L], (dw_gate, dw_up, dw_down)) = transpose of experts_dropless."""
    p = plan(cfg)
    dev = xs.device
    if d_xs is None:
        d_xs = torch.empty_like(xs)
    if dw is None:
        dw = (torch.empty_like(w_gate), torch.empty_like(w_up), torch.empty_like(w_down))
    ws = _ws(p["dropless_experts_bwd_ws_bytes"], dev)
    abi.check("moe_experts_backward_dropless", library().moe_experts_backward_dropless(
        C.byref(cfg), _ptr(xs), _ptr(expert_offsets), _ptr(w_gate), _ptr(w_up), _ptr(w_down),
        _ptr(d_expert_out), _ptr(d_xs), _ptr(dw[0]), _ptr(dw[1]), _ptr(dw[2]), _ptr(ws),
        ws.numel(), _stream(dev)))
    return d_xs, dw


def dispatch_backward_dropless(cfg, row_of, d_xs, dz=None):
    """dz [T, L] = transpose of dispatch_dropless."""
    dev = d_xs.device
    if dz is None:
        dz = torch.empty((cfg.T, cfg.d_latent), dtype=_tdt(cfg), device=dev)
    abi.check("moe_dispatch_backward_dropless", library().moe_dispatch_backward_dropless(
        C.byref(cfg), _ptr(row_of), _ptr(d_xs), _ptr(dz), _stream(dev)))
    return dz

