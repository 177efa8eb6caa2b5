#!/usr/bin/env python3
"""Benchmark of the pooled-wave MoE branch forward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload marin_16k]

A step is one moe_forward call (latent projection, router, top-k, pooled
dispatch with both caps, receiver binning, grouped SwiGLU experts, combine,
up-projection and shared experts) over one batch of seeded synthetic inputs
already resident in HBM.  Prints one JSON line.  --dropless times the
dropless ragged variant; --backward times the routed path's backward
(moe_backward_routed, or moe_backward_dropless with --dropless: gate, row and
weight gradients for one forward call's routing, a seeded dL/dy_latent,
forward state resident); --bias-update times the router's next-step bias
update (moe_router_bias_update) on one forward call's logits; --recv-share
times one EP rank's receive share (moe_experts over the capacity-bounded
bank of 6 local experts, then moe_combine of 65,536 tokens x 8 rows).

Stage durations come from HIP events the library records between its kernel
launches on the stream it launches them on (moe_forward_profiled), averaged
over the timed steps.  The dominant kernel's roofline fraction uses
algorithmic flops or bytes per launch (kept rows only, never padded
capacity).  The CPU baseline times the fp64 oracle on a bounded token sample
of the same workload on the host cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer fwd tokens/sec on 1 MI355X; % bf16 MFMA peak; drop fraction"
METRIC_BWD = "MoE routed-path bwd tokens/sec on 1 MI355X; % bf16 MFMA peak"
METRIC_BIAS = "MoE router next-step bias update tokens/sec on 1 MI355X; % HBM peak"
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}   # dense MFMA, MI355X
PEAK_HBM_GBS = 8000.0

# rocprofv3 kernel names of the stages (substrings that all must match)
STAGE_KERNEL = {
    "latent": ("dense1_bf16_kernel",),
    "expert_gate_up": ("ragged_gemm_kernel", ">, 1>("),
    "expert_down": ("ragged_gemm_kernel", ">, 0>("),
    "shared_gate_up": ("swiglu_bf16_kernel",),
    "output": ("densecat_bf16_kernel",),
    "combine": ("combine_kernel",),
    "scatter": ("scatter_kernel",),
    "swiglu_bwd": ("ragged_gemm_kernel", ">, 2>("),
    "dh": ("dgrad_kernel", "<0>"),
    "du": ("dgrad_kernel", "<1>"),
    "dw_down": ("wgrad_kernel",),
    "bias_range": ("range_kernel",),
    "bias_hist": ("hist_kernel",),
    "bias_quantile": ("quantile_kernel",),
}
COPY_KERNEL = ("copyBuffer",)
# sources of the kernel whose traffic the forward, dropless and backward lines
# report (ragged_gemm_kernel: the routed gate/up GEMM, and the backward's
# recompute): a measured traffic figure is used only while they are unchanged
KERNEL_SOURCES = ["gemm_core.h", "gemm_bf16.hip", "common.h"]
BIAS_SOURCES = ["bias.hip", "common.h"]


def code_only(text):
    """C/C++ source without its comments and with whitespace runs collapsed
    (string and character literals kept): what the compiler reads, so that
    a comment edit leaves the source hash unchanged."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def source_hash(paths):
    import hashlib
    h = hashlib.sha256()
    for path in paths:
        with open(path, encoding="utf-8") as fh:
            h.update(code_only(fh.read()).encode())
            h.update(b"\0")
    return h.hexdigest()


def kernel_source_hash(run_name=""):
    csrc = os.path.join(ROOT, "routing_capacity_dispatch_amd", "csrc")
    return source_hash(os.path.join(csrc, f)
                       for f in (BIAS_SOURCES if run_name.endswith("_bias") else KERNEL_SOURCES))


def summarize_pmc(fetch_csv, write_csv, stage, workload, copy_bytes, out_path, command):
    """Per-launch HBM bytes of one stage's kernel from two rocprofv3 --pmc
    counter files (FETCH_SIZE and WRITE_SIZE, KiB per dispatch), each scaled
    by what the same counter reads for a device copy of copy_bytes bytes."""
    import csv

    def per_dispatch(path, counter, pats):
        vals = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter or not all(p in r["Kernel_Name"] for p in pats):
                continue
            vals[r["Dispatch_Id"]] = vals.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
        return list(vals.values())

    pats = STAGE_KERNEL[stage]
    f_k = per_dispatch(fetch_csv, "FETCH_SIZE", pats)
    w_k = per_dispatch(write_csv, "WRITE_SIZE", pats)
    f_c = per_dispatch(fetch_csv, "FETCH_SIZE", COPY_KERNEL)
    w_c = per_dispatch(write_csv, "WRITE_SIZE", COPY_KERNEL)
    if not (f_k and w_k and f_c and w_c):
        raise SystemExit("kernel or copy dispatches missing from the counter files")
    # the calibration copy is the largest copy dispatch
    fc, wc = max(f_c), max(w_c)
    f_scale = copy_bytes / (fc * 1024.0)
    w_scale = copy_bytes / (wc * 1024.0)
    fk, wk = sum(f_k) / len(f_k), sum(w_k) / len(w_k)
    rec = {"workload": workload, "stage": stage, "kernel_pattern": list(pats),
           "dispatches": [len(f_k), len(w_k)],
           "fetch_kib_per_dispatch": fk, "write_kib_per_dispatch": wk,
           "copy_bytes": copy_bytes, "copy_fetch_kib": fc, "copy_write_kib": wc,
           "fetch_scale": f_scale, "write_scale": w_scale,
           "bytes_per_launch": fk * 1024.0 * f_scale + wk * 1024.0 * w_scale,
           "source_sha256": kernel_source_hash(workload), "command": command}
    with open(out_path, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec))


def summarize_clock(csv_path, xcds, simds, min_us, nominal_ghz=2.4):
    """Per library kernel, from one rocprofv3 --pmc file with GRBM_GUI_ACTIVE
    and SQ_VALU_MFMA_BUSY_CYCLES (mean over its dispatches): the duration,
    the shader clock (GUI-active cycles, which the counter sums over the
    XCDs, per nanosecond) and the fraction of SIMD cycles the matrix cores
    were busy.  Prints a markdown table of the kernels of at least min_us
    (the counter window of a short dispatch holds more than its run, so its
    clock reads high)."""
    import csv
    per = {}
    for r in csv.DictReader(open(csv_path)):
        name = r["Kernel_Name"]
        if "at::" in name or "copyBuffer" in name or "amd_rocclr" in name:
            continue
        d = per.setdefault(r["Dispatch_Id"], {"name": name, "ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    kern = {}
    for d in per.values():
        if "GRBM_GUI_ACTIVE" not in d or "SQ_VALU_MFMA_BUSY_CYCLES" not in d or d["ns"] < min_us * 1e3:
            continue
        kern.setdefault(d["name"], []).append(d)
    print(f"| kernel | dispatches | avg µs | clock GHz | MFMA busy | clock-limited bf16 peak TFLOP/s |")
    print("|---|---:|---:|---:|---:|---:|")
    for name, ds in sorted(kern.items(), key=lambda kv: -sum(x["ns"] for x in kv[1])):
        ns = sum(x["ns"] for x in ds) / len(ds)
        gui = sum(x["GRBM_GUI_ACTIVE"] for x in ds) / len(ds) / xcds
        mfma = sum(x["SQ_VALU_MFMA_BUSY_CYCLES"] for x in ds) / len(ds)
        ghz = gui / ns
        busy = mfma / (gui * simds) if gui else 0.0
        short = name.replace("moe::(anonymous namespace)::", "")
        short = short if len(short) <= 80 else short[:77] + "..."
        print(f"| `{short}` | {len(ds)} | {ns / 1e3:.1f} | {ghz:.2f} | {busy:.3f} | "
              f"{2500.0 * ghz / nominal_ghz:.0f} |")


def stage_work(w, kept, sent, dropless=False, backward=False, bias_bins=0):
    """Algorithmic flops (MFMA stages) or bytes (HBM stages) per launch."""
    eb = 2 if w.dtype == "bf16" else 4
    T, D, L, E, k, F = w.T, w.d_model, w.d_latent, w.n_experts, w.top_k, w.d_ff
    S, Fs = w.n_shared, w.d_ff_shared
    if bias_bins:
        # each pass over the fp32 logits reads them once; the histogram and
        # the quantiles are read or written once
        return {
            "bias_range": ("hbm", T * E * 4),
            "bias_hist": ("hbm", T * E * 4),
            "bias_quantile": ("hbm", E * bias_bins * 4 + E * 8),
            "bias_mean": ("hbm", E * 12),
        }
    if backward:
        # kept rows only, never the 64-row padding of the expert layout
        return {
            "combine_bwd": ("hbm", T * L * eb + 2 * kept * L * eb + 4 * T * k * 4),
            "layout": ("hbm", 0.0),
            "gather": ("hbm", 4 * kept * L * eb),
            "dh": ("mfma", 2.0 * kept * L * F),
            "swiglu_bwd": ("mfma", 2.0 * kept * L * 2 * F),
            "du": ("mfma", 2.0 * kept * 2 * F * L),
            "dw_down": ("mfma", 2.0 * kept * L * F),
            "dw_gate": ("mfma", 2.0 * kept * F * L),
            "dw_up": ("mfma", 2.0 * kept * F * L),
            "dispatch_bwd": ("hbm", kept * L * eb + T * L * eb + 3 * T * k * 4),
            "route_bwd": ("hbm", 3 * T * k * 4 + T * E * 4),
        }
    if dropless:
        n = kept   # every valid assignment has a row
        return {
            "latent": ("mfma", 2.0 * T * D * L),
            "router": ("mfma", 2.0 * T * L * E),
            "topk": ("hbm", T * E * 4 + T * k * 8),
            "sort": ("hbm", 2 * T * k * 4 + T * k * 4),
            "scatter": ("hbm", T * L * eb + n * L * eb + T * k * 4),
            "tiles": ("hbm", 0.0),
            "expert_gate_up": ("mfma", 2.0 * n * L * 2 * F),
            "expert_down": ("mfma", 2.0 * n * F * L),
            "combine": ("hbm", n * L * eb + T * L * eb + 2 * T * k * 4),
            "shared_gate_up": ("mfma", 2.0 * T * D * 2 * S * Fs),
            "output": ("mfma", 2.0 * T * D * (L + S * Fs)),
        }
    return {
        "latent": ("mfma", 2.0 * T * D * L),
        "router": ("mfma", 2.0 * T * L * E),
        "topk": ("hbm", T * E * 4 + T * k * 8),
        "assign": ("hbm", T * k * 4 + 2 * T * k * 4 + sent * 4),
        "scatter": ("hbm", T * L * eb + sent * L * eb + 2 * T * k * 4),
        "recv_bin": ("hbm", 0.0),
        "expert_rows": ("hbm", 0.0),
        "expert_gate_up": ("mfma", 2.0 * kept * L * 2 * F),
        "expert_down": ("mfma", 2.0 * kept * F * L),
        "combine": ("hbm", kept * L * eb + T * L * eb + 4 * T * k * 4),
        "shared_gate_up": ("mfma", 2.0 * T * D * 2 * S * Fs),
        "output": ("mfma", 2.0 * T * D * (L + S * Fs)),
    }


def cpu_baseline_bias(logits, top_k, n_bins):
    """The oracle's bias update on the whole step's logits (numpy, one core)."""
    from oracle import router_bias

    l = logits.detach().cpu().numpy()
    t0 = time.perf_counter()
    n = 0
    while True:
        b = router_bias.bias_update(l, top_k, n_bins)[0]
        n += 1
        if time.perf_counter() - t0 > 5.0:
            break
    dt = (time.perf_counter() - t0) / n
    assert b.shape == (l.shape[1],)
    return {"value": l.shape[0] / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"the whole step's {l.shape[0]}x{l.shape[1]} fp32 logits, {n_bins} bins, "
                      f"{n} oracle calls of {dt:.2f} s (numpy, single-threaded)"}


def blas_info():
    """Threads and vendor of the BLAS numpy calls (threadpoolctl), or (0, None)."""
    try:
        from threadpoolctl import threadpool_info
        libs = [i for i in threadpool_info() if i.get("user_api") == "blas"]
    except Exception:  # threadpoolctl missing: report the affinity mask
        return 0, None
    if not libs:
        return 0, None
    best = max(libs, key=lambda i: i.get("num_threads", 0))
    return best.get("num_threads", 0), f"{best.get('internal_api')} {best.get('version')}"


def cpu_baseline(w, inp, n_tok, dropless=False, backward=False, dy_latent=None, min_seconds=0.0):
    """The fp64 oracle on the first n_tok tokens (its own batch: caps are
    derived for n_tok tokens), weights given as the run's bf16 values."""
    import numpy as np
    import torch

    import oracle
    blas_threads, blas = blas_info()
    cores = len(os.sched_getaffinity(0))

    def f64(t):
        return t.detach().to("cpu").to(torch.float64).numpy()
    x = f64(inp["x"][:n_tok])
    wt = {k: f64(inp[k]) for k in ("w_latent", "w_router", "w_up_proj", "ws_gate", "ws_up",
                                   "ws_down")}
    wt["router_bias"] = inp["router_bias"].cpu().numpy().astype(np.float32)
    host = {k: inp[k].cpu() for k in ("w_gate", "w_up", "w_down")}   # bf16 on the host
    wt["expert_weights"] = lambda e: (host["w_gate"][e].to(torch.float64).numpy(),
                                      host["w_up"][e].to(torch.float64).numpy(),
                                      host["w_down"][e].to(torch.float64).numpy())
    if backward:
        # the saved state of the sample's own forward is not timed
        if dropless:
            r = oracle.forward_dropless(x, wt, top_k=w.top_k)
            keep = np.zeros(r["topk_idx"].shape, dtype=np.int64)
        else:
            r = oracle.forward(x, wt, top_k=w.top_k, n_pools=w.n_pools, n_waves=w.n_waves,
                               send_cap=w.send_cap, recv_cap=w.recv_cap)
            keep = r["assignment"]["recv_slot"]
        dy = f64(dy_latent[:n_tok])
        t0 = time.perf_counter()
        g = oracle.routed_backward(r["z"], r["topk_idx"], r["gates"], keep,
                                   wt["expert_weights"], dy, w.n_experts, o=r["expert_out"],
                                   experts=())
        dt = time.perf_counter() - t0
        assert g["dz"].shape == (n_tok, w.d_latent)
        what = (f"routed-path backward (dz, d_logits and every present expert's weight "
                f"gradients, computed and discarded) of the first {n_tok} tokens of the {w.name} "
                f"inputs as their own batch ({'no caps' if dropless else f'caps for {n_tok} tokens'})")
    else:
        # calls repeated until min_seconds of work (one call by default)
        t0 = time.perf_counter()
        calls = 0
        while True:
            if dropless:
                r = oracle.forward_dropless(x, wt, top_k=w.top_k)
            else:
                r = oracle.forward(x, wt, top_k=w.top_k, n_pools=w.n_pools, n_waves=w.n_waves,
                                   send_cap=w.send_cap, recv_cap=w.recv_cap)
            calls += 1
            if time.perf_counter() - t0 >= min_seconds:
                break
        total = time.perf_counter() - t0
        dt = total / calls
        assert r["y"].shape == (n_tok, w.d_model)
        what = (f"first {n_tok} tokens of the {w.name} inputs as their own batch "
                f"({'no caps' if dropless else f'caps for {n_tok} tokens'})")
        wall = f"{total:.1f} s wall over {calls} calls" if calls > 1 else f"{dt:.1f} s wall"
        return {"value": n_tok / dt, "unit": "tokens/s", "cores": blas_threads or cores,
                "kind": "oracle", "blas": blas,
                "sample": f"{what}, fp64 numpy, {wall}, {cores} cores in the affinity mask"}
    return {"value": n_tok / dt, "unit": "tokens/s", "cores": blas_threads or cores,
            "kind": "oracle", "blas": blas,
            "sample": f"{what}, fp64 numpy, {dt:.1f} s wall, {cores} cores in the affinity mask"}


def cpu_baseline_recv_share(sh, n_tok, dev):
    """The fp64 oracle on the first n_tok tokens of a receive share: their k
    bank rows each through the owning expert's SwiGLU, then the combine."""
    import numpy as np
    import torch

    import oracle
    k = sh["k"]
    ex = sh["expert_of"][:n_tok].numpy()
    sl = sh["slot_of"][:n_tok].numpy()
    wv = np.repeat((np.arange(n_tok) // sh["Tw"])[:, None], k, axis=1)
    u = sh["rows"][torch.from_numpy(wv).to(dev).long(), torch.from_numpy(sl).to(dev).long()]
    u = u.to("cpu", torch.float32).numpy().astype(np.float64)          # [n_tok, k, L]
    ws = {int(e): tuple(sh[n][int(e)].to("cpu", torch.float32).numpy().astype(np.float64)
                        for n in ("w_gate", "w_up", "w_down")) for e in np.unique(ex)}
    g64 = sh["gates"][:n_tok].numpy().astype(np.float64)
    t_c = time.perf_counter()
    o = np.zeros((n_tok, k, u.shape[-1]))
    for e in np.unique(ex):
        m = ex == e
        o[m] = oracle.swiglu(u[m], *ws[int(e)])
    oracle.combine(g64, np.zeros((n_tok, k)), o)
    dt = time.perf_counter() - t_c
    cores = len(os.sched_getaffinity(0))
    threads, blas = blas_info()
    return {"value": n_tok / dt, "unit": "tokens/s", "cores": threads or cores, "kind": "oracle", "blas": blas,
            "sample": f"the first {n_tok} tokens' {k} rows each through their experts' SwiGLU "
                      f"and the combine, fp64 numpy, {dt:.1f} s wall, {cores} cores in the affinity mask"}


# the oracle timed once per workload (context for the GPU figures; bounded samples)
CPU_CONFIGS = [("tiny_fp32", 256), ("mid_bf16", 512), ("marin_16k", 256), ("recv_share", 16384),
               ("zipf_64k", 256)]


def cpu_baselines_by_config(main_name, main_result, seed, dev):
    """One oracle timing per workload on a bounded token sample of it (the
    headline workload's is main_result)."""
    import torch

    import synth
    out = []
    for name, n_tok in CPU_CONFIGS:
        print(f"# cpu baseline: {name}, {n_tok} tokens", file=sys.stderr, flush=True)
        if name == main_name and main_result is not None:
            r = main_result
        elif name == "recv_share":
            sh = synth.make_recv_share(seed=seed, device=dev)
            r = cpu_baseline_recv_share(sh, n_tok, dev)
            del sh
        else:
            w = synth.workload(name)
            inp = synth.make_inputs(w, seed, device=dev)
            r = cpu_baseline(w, inp, n_tok, min_seconds=2.0)
            del inp
        torch.cuda.empty_cache()
        out.append(dict(r, workload=name))
    return out


METRIC_SHARE = "MoE receive-share (6 local experts) SwiGLU + combine tokens/sec on 1 MI355X; % bf16 MFMA peak"


def bench_recv_share(args):
    """One EP rank's receive share: the bank of 6 local experts (per wave one
    block of 6 x 33,497 slots, multinomial loads, id column), moe_experts over
    all waves' rows, then moe_combine of the rank's 65,536 tokens x 8 rows.
    A step is both calls; the stages are timed with events on the stream the
    library launches on (torch's current stream)."""
    import numpy as np
    import torch

    import routing_capacity_dispatch_amd as rcd
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    print("# generating the receive-share inputs", file=sys.stderr, flush=True)
    sh = synth.make_recv_share(seed=args.seed, device=dev)
    W, n_local, cw, L, F, T, k = (sh[x] for x in ("W", "n_local", "cap_wave", "L", "F", "T", "k"))
    cfg = rcd.make_config(T, 64, L, n_local, 1, k, F, n_waves=W, dtype="bf16",
                          cap_send_rows=n_local * cw, cap_recv_rows=cw)
    p = rcd.plan(cfg)
    pools = torch.empty(p["pools_bytes"], dtype=torch.uint8, device=dev)
    rows, ids = rcd.pool_views(cfg, pools)
    rows[:, 0].copy_(sh["rows"])
    counts = sh["counts"]
    slot = torch.arange(n_local * cw, dtype=torch.int32)
    ids[:, 0].copy_(torch.where((slot % cw)[None, :] < counts.repeat_interleave(cw, dim=1),
                                (slot // cw)[None, :].expand(W, -1), torch.full_like(slot, -1)[None, :]).to(dev))
    bank_rows = (torch.arange(n_local, dtype=torch.int32)[:, None] * cw
                 + torch.arange(cw, dtype=torch.int32)[None, :]).expand(W, -1, -1).contiguous().to(dev)
    cnt_d = counts.to(dev)
    expert_of = sh["expert_of"].to(dev)
    slot_of = sh["slot_of"].to(dev)
    recv = (sh["slot_of"] % cw).to(torch.int32).to(dev)
    gates = sh["gates"].to(dev)
    eo = torch.empty(p["expert_out_bytes"], dtype=torch.uint8, device=dev)
    y = torch.empty((T, L), dtype=torch.bfloat16, device=dev)

    def step(ev=None):
        if ev:
            ev[0].record()
        rcd.experts(cfg, pools, bank_rows, cnt_d, sh["w_gate"], sh["w_up"], sh["w_down"], expert_out=eo)
        if ev:
            ev[1].record()
        rcd.combine(cfg, eo, expert_of, slot_of, recv, gates, y_latent=y)
        if ev:
            ev[2].record()

    print(f"# warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    for row in ev:
        for e in row:
            e.record()
    torch.cuda.synchronize()
    print(f"# timing {K} steps", file=sys.stderr, flush=True)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t0.record()
    for i in range(K):
        step(ev[i])
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t0.elapsed_time(t1) / K
    ms_exp = sum(ev[i][0].elapsed_time(ev[i][1]) for i in range(K)) / K
    ms_cmb = sum(ev[i][1].elapsed_time(ev[i][2]) for i in range(K)) / K
    n_rows = int(counts.sum())
    flops = 6.0 * n_rows * L * F           # gate, up and down over the valid rows
    cbytes = n_rows * L * 2 + T * L * 2 + T * k * 16
    tf = flops / (ms_exp * 1e-3) / 1e12
    out = {
        "metric": METRIC_SHARE, "value": round(T / (ms_step * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": K, "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "recv_share", "pass": "experts+combine", "T": T, "n_local_experts": n_local,
                   "d_latent": L, "d_ff": F, "top_k": k, "n_waves": W, "cap_wave_rows": cw,
                   "valid_rows": n_rows, "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_TFLOPS["bf16"], "unit": "TFLOP/s",
                     "frac": round(tf / PEAK_TFLOPS["bf16"], 4), "kernel": "experts (gate/up and down GEMMs)",
                     "traffic": None},
        "stages": {"experts": {"ms": round(ms_exp, 4), "tflops": round(tf, 1),
                               "frac_peak": round(tf / PEAK_TFLOPS["bf16"], 4)},
                   "combine": {"ms": round(ms_cmb, 4), "gbs": round(cbytes / (ms_cmb * 1e-3) / 1e9, 1),
                               "frac_peak": round(cbytes / (ms_cmb * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}},
        "wall_s_timed": round(wall, 3),
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        n_tok = args.cpu_tokens or 32768
        print(f"# cpu baseline: oracle on the first {n_tok} tokens", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline_recv_share(sh, n_tok, dev)
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="marin_16k")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--dropless", action="store_true",
                    help="time the dropless ragged variant (moe_forward_dropless) instead")
    ap.add_argument("--backward", action="store_true",
                    help="time the routed path's backward (moe_backward_routed) instead")
    ap.add_argument("--bias-update", action="store_true",
                    help="time the router's next-step bias update (moe_router_bias_update) on one "
                         "forward call's logits instead")
    ap.add_argument("--recv-share", action="store_true",
                    help="time one EP rank's receive share instead: moe_experts over 6 local experts "
                         "(3 wave slabs of 33,497 rows each) then moe_combine of 65,536 tokens x 8")
    ap.add_argument("--bins", type=int, default=256, help="histogram bins of --bias-update")
    ap.add_argument("--cpu-tokens", type=int, default=None,
                    help="oracle sample for the CPU baseline (default 256; 64 with --backward)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-cpu-configs", action="store_true",
                    help="time the oracle on the headline workload only, not once per workload")
    ap.add_argument("--traffic", default=None,
                    help="measured HBM bytes per launch of the dominant kernel (JSON; default "
                         "profiles/traffic_<workload>.json)")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="run one device copy of this many MiB before the warmup (the "
                         "known-size kernel that scales the PMC byte counters)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the dominant kernel's measured traffic from two rocprofv3 "
                         "--pmc counter files and exit")
    ap.add_argument("--stage", default="expert_gate_up", help="stage for --summarize-pmc")
    ap.add_argument("--pmc-command", default="", help="command recorded by --summarize-pmc")
    ap.add_argument("--summarize-clock", metavar="COUNTER_CSV",
                    help="print each kernel's clock and matrix-core busy fraction from a rocprofv3 "
                         "--pmc file of GRBM_GUI_ACTIVE and SQ_VALU_MFMA_BUSY_CYCLES, and exit")
    ap.add_argument("--xcds", type=int, default=8, help="XCDs the GUI-active counter sums over")
    ap.add_argument("--simds", type=int, default=1024, help="SIMDs of the device (4 per CU)")
    ap.add_argument("--min-us", type=float, default=400.0, help="shortest kernel --summarize-clock lists")
    args = ap.parse_args()
    if args.summarize_clock:
        summarize_clock(args.summarize_clock, args.xcds, args.simds, args.min_us)
        return
    run_name = (args.workload + ("_dropless" if args.dropless else "") + ("_backward" if args.backward else "")
                + ("_bias" if args.bias_update else ""))
    if args.cpu_tokens is None and not args.recv_share:
        args.cpu_tokens = 64 if args.backward else 256
    if args.traffic is None:
        args.traffic = os.path.join(ROOT, "profiles", f"traffic_{run_name}.json")
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.stage, run_name,
                      args.calib_copy_mb * 1024 * 1024, args.traffic, args.pmc_command)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.recv_share:
        bench_recv_share(args)
        return

    import torch

    import routing_capacity_dispatch_amd as rcd
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    w = synth.workload(args.workload)
    cfg = rcd.config_of(w)
    print(f"# generating {w.name} inputs", file=sys.stderr, flush=True)
    inp = synth.make_inputs(w, args.seed, device=dev)
    x = inp["x"]
    weights = {k: v for k, v in inp.items() if k != "x"}
    dy = None
    if args.bias_update:
        fwd = rcd.Forward(cfg, weights, dev, taps=True)
        fwd(x)           # the step whose router logits feed the update
        step = rcd.RouterBias(cfg, args.bins, dev)
        nst = rcd.router_bias_stage_count()
        stages = rcd.abi.BIAS_STAGES
    elif args.backward:
        fwd = (rcd.ForwardDropless if args.dropless else rcd.Forward)(cfg, weights, dev, taps=True)
        fwd(x)           # the forward call whose gradient is taken: state saved
        dy = synth.grad_latent(w, args.seed, device=dev)
        step = rcd.BackwardRouted(fwd)
        nst = rcd.backward_stage_count()
        stages = rcd.abi.BACKWARD_STAGES
    elif args.dropless:
        fwd = rcd.ForwardDropless(cfg, weights, dev)
        nst = rcd.dropless_stage_count()
        stages = rcd.abi.DROPLESS_STAGES
        step = fwd
    else:
        fwd = rcd.Forward(cfg, weights, dev)
        nst = rcd.stage_count()
        stages = rcd.abi.STAGES
        step = fwd
    arg = dy if args.backward else (fwd.tap_t["logits"] if args.bias_update else x)
    if args.calib_copy_mb:
        n = args.calib_copy_mb * 1024 * 1024
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    assert len(stages) == nst

    print(f"# warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step(arg)
    torch.cuda.synchronize()

    K = args.steps
    # headline: the plain call, one event per step boundary (events on the
    # stream the library launches on: torch's current stream)
    tev = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(nst + 1)] for _ in range(K)]
    for e in tev + [e for row in ev for e in row]:   # torch creates its events lazily
        e.record()
    print(f"# timing {K} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    tev[0].record()
    for i in range(K):
        step(arg)
        tev[i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = tev[0].elapsed_time(tev[K]) / K
    per_step = [tev[i].elapsed_time(tev[i + 1]) for i in range(K)]
    # the median of steps 2 .. K-1 (1-based; 2-19 of 20), as the pages
    # quote a run's step time
    mid = sorted(per_step[1:K - 1] if K >= 4 else per_step)
    ms_median = (mid[(len(mid) - 1) // 2] + mid[len(mid) // 2]) / 2

    # stage breakdown: a second pass through the instrumented entry point
    print(f"# stage pass, {K} steps", file=sys.stderr, flush=True)
    for i in range(K):
        step.profiled(arg, ev[i])
    torch.cuda.synchronize()

    per = {s: 0.0 for s in stages}
    for i in range(K):
        for j, s in enumerate(stages):
            per[s] += ev[i][j].elapsed_time(ev[i][j + 1]) / K
    kept, sd, rd = [int(v) for v in fwd.counts.cpu().tolist()]
    sent = kept + rd
    work = stage_work(w, kept, sent, dropless=args.dropless and not args.backward, backward=args.backward,
                      bias_bins=args.bins if args.bias_update else 0)
    peak_f = PEAK_TFLOPS[w.dtype]
    st_out = {}
    for s in stages:
        kind, amount = work[s]
        ms = per[s]
        if kind == "mfma":
            ach = amount / (ms * 1e-3) / 1e12 if ms > 0 else 0.0
            st_out[s] = {"ms": round(ms, 4), "tflops": round(ach, 1),
                         "frac_peak": round(ach / peak_f, 4)}
        else:
            ach = amount / (ms * 1e-3) / 1e9 if ms > 0 else 0.0
            st_out[s] = {"ms": round(ms, 4), "gbs": round(ach, 1),
                         "frac_peak": round(ach / PEAK_HBM_GBS, 4)}
    dom = max(stages, key=lambda s: per[s])
    kind, amount = work[dom]
    if kind == "mfma":
        ach = amount / (per[dom] * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": peak_f, "unit": "TFLOP/s",
                "frac": round(ach / peak_f, 4)}
    else:
        ach = amount / (per[dom] * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBS, 4)}
    roof["kernel"] = dom
    roof["traffic"] = None
    if args.traffic and os.path.exists(args.traffic):
        try:
            tr = json.load(open(args.traffic))
            if (tr.get("stage") == dom and tr.get("workload") == run_name
                    and tr.get("source_sha256") == kernel_source_hash(run_name)):
                roof["traffic"] = round(tr["bytes_per_launch"])
        except (OSError, ValueError, KeyError):
            pass
    gemm_flops = sum(work[s][1] for s in stages if work[s][0] == "mfma")
    gemm_ms = sum(per[s] for s in stages if work[s][0] == "mfma")
    pass_name = "router_bias" if args.bias_update else ("backward" if args.backward else "forward")
    tokens_s = w.T / (ms_step * 1e-3)
    out = {
        "metric": METRIC_BIAS if args.bias_update else (METRIC_BWD if args.backward else METRIC),
        "value": round(tokens_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "median_ms_steps_2_19" if K == 20 else f"median_ms_steps_2_{K - 1}": round(ms_median, 4),
        "median_tokens_per_s": round(w.T / (ms_median * 1e-3), 1),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if args.bias_update else w.dtype,
        "data": "synthetic",
        "config": {"workload": run_name, "pass": pass_name, "T": w.T, "d_model": w.d_model, "d_latent": w.d_latent,
                   "n_experts": w.n_experts, "n_pools": w.n_pools, "top_k": w.top_k,
                   "d_ff": w.d_ff, "n_shared": w.n_shared, "d_ff_shared": w.d_ff_shared,
                   "n_waves": w.n_waves, "caps": [list(w.send_cap), list(w.recv_cap)],
                   "global_batch": w.T, "parallelism": "single GPU"},
        "roofline": roof,
        "gemm_mfma_frac": round(gemm_flops / (gemm_ms * 1e-3) / 1e12 / peak_f, 4) if gemm_ms > 0 else None,
        "drop_fraction": {"sender": sd / (w.T * w.top_k), "receiver": rd / (w.T * w.top_k),
                          "total": (sd + rd) / (w.T * w.top_k)},
        "stages": st_out,
        "wall_s_timed": round(wall, 3),
    }
    if args.bias_update:
        out["config"]["bins"] = args.bins
    if not args.no_cpu_baseline and args.bias_update:
        print("# cpu baseline: oracle bias update", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline_bias(arg, w.top_k, args.bins)
    elif not args.no_cpu_baseline:
        print(f"# cpu baseline: oracle on {args.cpu_tokens} tokens", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_tokens, dropless=args.dropless,
                                           backward=args.backward, dy_latent=dy)
        if pass_name == "forward" and not args.dropless and not args.no_cpu_configs:
            del fwd, step, inp, weights, x
            out["cpu_baseline_configs"] = cpu_baselines_by_config(w.name, out["cpu_baseline"], args.seed, dev)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
