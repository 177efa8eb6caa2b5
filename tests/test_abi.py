"""The C-ABI library loads, exports what include/moe.h declares, and its
host-side plan and validation behave (no GPU work: every call here returns
before anything is enqueued)."""
import ctypes as C
import os
import re
import subprocess

import pytest

import oracle
import synth
import routing_capacity_dispatch_amd as rcd
from routing_capacity_dispatch_amd import abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(abi.LIB_PATH):
        pytest.fail("libmoe.so is not built (python -m routing_capacity_dispatch_amd.build)")
    return abi.load()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ["moe_make_plan", "moe_route", "moe_dispatch", "moe_experts", "moe_combine",
              "moe_forward", "moe_status_string"]:
        assert n in names


def test_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", abi.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(l.split()[-1] for l in out.splitlines() if l.strip())
    for n in declared_functions():
        assert n in exported, n
        assert hasattr(lib, n)
    # the binding's signature table covers exactly the declared functions
    assert sorted(abi.SIGNATURES) == declared_functions()


def test_struct_layouts_match_header():
    # sizes implied by the header's field lists (natural alignment, no packing)
    assert C.sizeof(abi.MoeConfig) == 8 + 13 * 4 + 4 + 2 * 8 + 2 * 4
    assert C.sizeof(abi.MoePlan) == 24 * 8
    assert C.sizeof(abi.MoeWeights) == 10 * 8
    assert C.sizeof(abi.MoeTaps) == 12 * 8


def test_status_strings(lib):
    for s in range(5):
        assert lib.moe_status_string(s).decode().startswith(abi.STATUS_NAMES[s])
    assert lib.moe_version() >= 100


@pytest.mark.parametrize("name", ["tiny_fp32", "mid_bf16", "marin_16k", "zipf_64k"])
def test_plan_matches_oracle_capacity(lib, name):
    w = synth.workload(name)
    p = rcd.plan(rcd.config_of(w))
    o = oracle.capacity_plan(w.T, w.top_k, w.n_experts, w.n_pools, w.n_waves)
    assert (p["tokens_per_wave"], p["cap_send"], p["cap_recv"]) == (o["Tw"], o["cap_send"], o["cap_recv"])
    eb = 2 if w.dtype == "bf16" else 4
    assert p["row_bytes"] == w.d_latent * eb
    assert p["pool_block_bytes"] % 256 == 0
    assert p["pool_block_bytes"] >= p["cap_send"] * (w.d_latent * eb + 4)
    assert p["pools_bytes"] == w.n_waves * w.n_pools * p["pool_block_bytes"]
    assert p["max_expert_rows"] == w.n_waves * p["cap_recv"]
    for k in ("dispatch_ws_bytes", "experts_ws_bytes", "forward_ws_bytes"):
        assert p[k] % 256 == 0 and p[k] > 0


@pytest.mark.parametrize("T", [0, 1, 2, 5, 86, 100, 4095, 65536])
@pytest.mark.parametrize("k,E,P,W", [(1, 4, 1, 1), (2, 16, 4, 3), (8, 384, 64, 3), (8, 384, 384, 2),
                                     (3, 12, 3, 5)])
def test_plan_capacity_sweep(lib, T, k, E, P, W):
    cfg = rcd.make_config(T, 64, 64, E, P, k, 64, n_waves=W, dtype="bf16")
    p = rcd.plan(cfg)
    o = oracle.capacity_plan(T, k, E, P, W)
    assert (p["tokens_per_wave"], p["cap_send"], p["cap_recv"]) == (o["Tw"], o["cap_send"], o["cap_recv"])


def test_recv_share_plan(lib):
    sh = synth.RECV_SHARE
    cfg = rcd.make_config(sh["T"], 64, sh["d_latent"], sh["n_local"], 1, sh["top_k"], sh["d_ff"],
                          n_waves=3, cap_send_rows=sh["n_local"] * sh["cap_wave"],
                          cap_recv_rows=sh["cap_wave"])
    p = rcd.plan(cfg)
    assert p["cap_recv"] == 33497 and p["cap_send"] == 6 * 33497
    assert p["max_expert_rows"] == 3 * 33497


def _status(fn):
    try:
        fn()
    except abi.MoeError as e:
        return e.status
    return abi.MOE_OK


@pytest.mark.parametrize("field,value,status", [
    ("n_pools", 5, abi.MOE_ERR_INVALID_ARG),        # 16 % 5 != 0
    ("top_k", 65, abi.MOE_ERR_UNSUPPORTED),         # k > 64
    ("top_k", 0, abi.MOE_ERR_INVALID_ARG),
    ("n_waves", 0, abi.MOE_ERR_INVALID_ARG),
    ("T", -1, abi.MOE_ERR_INVALID_ARG),
    ("d_model", 0, abi.MOE_ERR_INVALID_ARG),
    ("send_cap_den", 0, abi.MOE_ERR_INVALID_ARG),
    ("recv_cap_num", -1, abi.MOE_ERR_INVALID_ARG),
    ("dtype", 7, abi.MOE_ERR_INVALID_ARG),
    ("reserved", 1, abi.MOE_ERR_INVALID_ARG),
    ("d_latent", 100, abi.MOE_ERR_UNSUPPORTED),     # not a multiple of 64
    ("d_ff", 96, abi.MOE_ERR_UNSUPPORTED),
    ("n_shared", 4, abi.MOE_ERR_UNSUPPORTED),
    ("n_waves", 65536, abi.MOE_ERR_UNSUPPORTED),
    # widths above 2^20 (multiples of 64): workspace sizes stay far inside int64
    ("d_model", (1 << 20) + 64, abi.MOE_ERR_UNSUPPORTED),
    ("d_latent", (1 << 20) + 64, abi.MOE_ERR_UNSUPPORTED),
    ("d_ff", (1 << 30), abi.MOE_ERR_UNSUPPORTED),
    ("d_ff_shared", (1 << 31) - 64, abi.MOE_ERR_UNSUPPORTED),
])
def test_plan_rejects(lib, field, value, status):
    cfg = rcd.config_of(synth.workload("tiny_fp32"))
    setattr(cfg, field, value)
    assert _status(lambda: rcd.plan(cfg)) == status


def test_widest_supported_fp32_plan_sizes(lib):
    # the widest fp32 widths: every size positive and exact (no wrap-around),
    # the shared hidden rows T * S * Fs * 4 bytes among them
    T, wide = 1 << 14, 1 << 20
    cfg = rcd.make_config(T, wide, wide, 64, 16, 8, wide, n_shared=3, d_ff_shared=wide, dtype="f32")
    p = rcd.plan(cfg)
    # z, y_latent and the shared hidden rows alone
    assert p["forward_ws_bytes"] > 2 * T * wide * 4 + T * 3 * wide * 4
    assert p["backward_ws_bytes"] > 0 and p["dropless_backward_ws_bytes"] > 0


def test_tile_lists_past_the_grid_limit_unsupported(lib):
    # one 512-thread workgroup per tile of a grouped GEMM: a grid must stay
    # below 2^32 work-items, so at most 2^23 - 8 tiles per list
    wide = 1 << 20
    ok = rcd.make_config(1 << 14, 64, 64, 64, 16, 8, wide, dtype="f32")
    rcd.plan(ok)
    big = rcd.make_config(1 << 16, 64, 64, 64, 16, 8, wide, dtype="f32")
    assert _status(lambda: rcd.plan(big)) == abi.MOE_ERR_UNSUPPORTED


def test_too_many_experts_unsupported(lib):
    cfg = rcd.make_config(16, 64, 64, 2048, 1, 2, 64)
    assert _status(lambda: rcd.plan(cfg)) == abi.MOE_ERR_UNSUPPORTED


def test_calls_validate_before_enqueue(lib):
    cfg = rcd.config_of(synth.workload("tiny_fp32"))
    nul = None
    # null data pointers
    assert lib.moe_route(C.byref(cfg), nul, nul, nul, nul, nul) == abi.MOE_ERR_INVALID_ARG
    assert lib.moe_dispatch(C.byref(cfg), nul, nul, nul, nul, nul, nul, nul, nul, nul, nul, 0,
                            nul) == abi.MOE_ERR_INVALID_ARG
    assert lib.moe_combine(C.byref(cfg), nul, nul, nul, nul, nul, nul, nul) == abi.MOE_ERR_INVALID_ARG
    assert lib.moe_experts(C.byref(cfg), nul, nul, nul, nul, nul, nul, nul, nul, 0,
                           nul) == abi.MOE_ERR_INVALID_ARG
    w = abi.MoeWeights()
    assert lib.moe_forward(C.byref(cfg), C.byref(w), nul, nul, nul, nul, nul, 0,
                           nul) == abi.MOE_ERR_INVALID_ARG
    assert lib.moe_forward(C.byref(cfg), nul, nul, nul, nul, nul, nul, 0,
                           nul) == abi.MOE_ERR_INVALID_ARG
    assert lib.moe_make_plan(nul, nul) == abi.MOE_ERR_INVALID_ARG
    # short or misaligned workspace (fake, never dereferenced: rejected first)
    fake = C.c_void_p(0x100000)
    p = rcd.plan(cfg)
    assert lib.moe_dispatch(C.byref(cfg), fake, fake, fake, fake, fake, fake, fake, fake, fake,
                            fake, p["dispatch_ws_bytes"] - 1, nul) == abi.MOE_ERR_WORKSPACE
    assert lib.moe_dispatch(C.byref(cfg), fake, fake, fake, fake, fake, fake, fake, fake, fake,
                            C.c_void_p(0x100010), p["dispatch_ws_bytes"], nul) == abi.MOE_ERR_WORKSPACE
    assert lib.moe_experts(C.byref(cfg), fake, fake, fake, fake, fake, fake, fake, fake,
                           p["experts_ws_bytes"] - 256, nul) == abi.MOE_ERR_WORKSPACE
    ww = abi.MoeWeights(*([0x100000] * 10))
    assert lib.moe_forward(C.byref(cfg), C.byref(ww), fake, fake, nul, nul, fake,
                           p["forward_ws_bytes"] - 1, nul) == abi.MOE_ERR_WORKSPACE
    # bad shapes on the route call
    bad = rcd.config_of(synth.workload("tiny_fp32"))
    bad.top_k = 20   # > E = 16
    assert lib.moe_route(C.byref(bad), fake, nul, fake, fake, nul) == abi.MOE_ERR_INVALID_ARG
    bad.top_k = 2
    bad.n_experts = 4096
    assert lib.moe_route(C.byref(bad), fake, nul, fake, fake, nul) == abi.MOE_ERR_UNSUPPORTED


def test_dropless_plan_and_validation(lib):
    w = synth.workload("marin_16k")
    p = rcd.plan(rcd.config_of(w))
    n = w.T * w.top_k
    assert p["dropless_rows"] == n
    # xs and expert_out rows plus the hidden rows are the bulk of the forward workspace
    assert p["dropless_forward_ws_bytes"] >= 2 * n * w.d_latent * 2 + n * w.d_ff * 2
    for k in ("dropless_dispatch_ws_bytes", "dropless_experts_ws_bytes",
              "dropless_forward_ws_bytes"):
        assert p[k] % 256 == 0 and p[k] > 0
    nul = None
    fake = C.c_void_p(0x100000)
    f32 = rcd.config_of(synth.workload("tiny_fp32"))
    assert lib.moe_dispatch_dropless(C.byref(f32), fake, fake, fake, fake, fake, nul, fake,
                                     1 << 30, nul) == abi.MOE_ERR_UNSUPPORTED
    bf = rcd.config_of(synth.workload("mid_bf16"))
    pb = rcd.plan(bf)
    assert lib.moe_dispatch_dropless(C.byref(bf), nul, fake, fake, fake, fake, nul, fake,
                                     1 << 30, nul) == abi.MOE_ERR_INVALID_ARG
    assert lib.moe_dispatch_dropless(C.byref(bf), fake, fake, fake, fake, fake, nul, fake,
                                     pb["dropless_dispatch_ws_bytes"] - 1, nul) == abi.MOE_ERR_WORKSPACE
    assert lib.moe_experts_dropless(C.byref(bf), fake, fake, fake, fake, fake, fake, fake,
                                    pb["dropless_experts_ws_bytes"] - 256, nul) == abi.MOE_ERR_WORKSPACE
    assert lib.moe_experts_dropless(C.byref(bf), fake, nul, fake, fake, fake, fake, fake,
                                    1 << 30, nul) == abi.MOE_ERR_INVALID_ARG
    assert lib.moe_combine_dropless(C.byref(bf), nul, fake, fake, fake, nul) == abi.MOE_ERR_INVALID_ARG
    ww = abi.MoeWeights(*([0x100000] * 10))
    assert lib.moe_forward_dropless(C.byref(bf), C.byref(ww), fake, fake, nul, nul, fake,
                                    pb["dropless_forward_ws_bytes"] - 1, nul) == abi.MOE_ERR_WORKSPACE
    assert lib.moe_forward_dropless(C.byref(bf), nul, fake, fake, nul, nul, fake,
                                    pb["dropless_forward_ws_bytes"], nul) == abi.MOE_ERR_INVALID_ARG
    assert lib.moe_forward_dropless_stage_count() == len(abi.DROPLESS_STAGES)
    assert lib.moe_forward_stage_count() == len(abi.STAGES)


def test_bf16_operands_above_4gib_unsupported(lib):
    # x of 350,000 tokens x 6144 bf16 is 4.3 GB: past the GEMMs' 32-bit lane offsets
    cfg = rcd.make_config(350_000, 6144, 3072, 384, 64, 8, 3072, n_shared=2, d_ff_shared=3072,
                          dtype="bf16")
    assert _status(lambda: rcd.plan(cfg)) == abi.MOE_ERR_UNSUPPORTED
    ok = rcd.make_config(65536, 6144, 3072, 384, 64, 8, 3072, n_shared=2, d_ff_shared=3072,
                         dtype="bf16")
    assert rcd.plan(ok)["pools_bytes"] < 2 ** 32


def test_backward_plan_and_validation(lib):
    w = synth.workload("marin_16k")
    p = rcd.plan(rcd.config_of(w))
    kept_max = min(w.T * w.top_k, w.n_experts * w.n_waves * p["cap_recv"])
    assert p["backward_rows"] == kept_max + 63 * w.n_experts
    # u, do, dh, da|db and h rows dominate the experts' backward workspace
    R, L, F = p["backward_rows"], w.d_latent, w.d_ff
    assert p["experts_bwd_ws_bytes"] >= R * (2 * L + 4 * F) * 2
    assert p["backward_ws_bytes"] >= p["experts_bwd_ws_bytes"] + 2 * p["expert_out_bytes"]
    for k in ("experts_bwd_ws_bytes", "backward_ws_bytes"):
        assert p[k] % 256 == 0
    nul = None
    fake = C.c_void_p(0x100000)
    # fp32, or widths not multiples of 256: unsupported
    f32 = rcd.config_of(synth.workload("tiny_fp32"))
    assert lib.moe_combine_backward(C.byref(f32), *([fake] * 8), nul) == abi.MOE_ERR_UNSUPPORTED
    odd = rcd.make_config(64, 256, 192, 16, 4, 2, 256, dtype="bf16")
    assert lib.moe_dispatch_backward(C.byref(odd), *([fake] * 5), nul) == abi.MOE_ERR_UNSUPPORTED
    bf = rcd.config_of(synth.workload("mid_bf16"))
    pb = rcd.plan(bf)
    assert lib.moe_combine_backward(C.byref(bf), *([fake] * 7), nul, nul) == abi.MOE_ERR_INVALID_ARG
    assert lib.moe_dispatch_backward(C.byref(bf), fake, fake, fake, nul, fake, nul) == abi.MOE_ERR_INVALID_ARG
    assert lib.moe_route_backward(C.byref(bf), fake, fake, nul, fake, nul) == abi.MOE_ERR_INVALID_ARG
    args = [fake] * 11
    assert lib.moe_experts_backward(C.byref(bf), *args, fake, pb["experts_bwd_ws_bytes"] - 256,
                                    nul) == abi.MOE_ERR_WORKSPACE
    assert lib.moe_experts_backward(C.byref(bf), *args, C.c_void_p(0x100010), pb["experts_bwd_ws_bytes"],
                                    nul) == abi.MOE_ERR_WORKSPACE
    assert lib.moe_experts_backward(C.byref(bf), nul, *args[1:], fake, 1 << 40, nul) == abi.MOE_ERR_INVALID_ARG
    ww = abi.MoeWeights(*([0x100000] * 10))
    taps = abi.MoeTaps(*([0x100000] * 12))
    assert lib.moe_backward_routed(C.byref(bf), C.byref(ww), C.byref(taps), *([fake] * 6), fake,
                                   pb["backward_ws_bytes"] - 1, nul) == abi.MOE_ERR_WORKSPACE
    taps.expert_out = None
    assert lib.moe_backward_routed(C.byref(bf), C.byref(ww), C.byref(taps), *([fake] * 6), fake,
                                   pb["backward_ws_bytes"], nul) == abi.MOE_ERR_INVALID_ARG
    assert lib.moe_backward_routed(C.byref(bf), C.byref(ww), nul, *([fake] * 6), fake,
                                   pb["backward_ws_bytes"], nul) == abi.MOE_ERR_INVALID_ARG
    assert lib.moe_backward_routed_stage_count() == len(abi.BACKWARD_STAGES)


def test_dropless_backward_plan_and_validation(lib):
    w = synth.workload("marin_16k")
    p = rcd.plan(rcd.config_of(w))
    n = w.T * w.top_k
    assert p["dropless_backward_rows"] == n + 63 * w.n_experts
    assert p["dropless_backward_ws_bytes"] >= p["dropless_experts_bwd_ws_bytes"] + 2 * n * w.d_latent * 2
    nul = None
    fake = C.c_void_p(0x100000)
    bf = rcd.config_of(synth.workload("mid_bf16"))
    pb = rcd.plan(bf)
    assert lib.moe_combine_backward_dropless(C.byref(bf), fake, nul, *([fake] * 4), nul) == abi.MOE_ERR_INVALID_ARG
    assert lib.moe_dispatch_backward_dropless(C.byref(bf), fake, fake, nul, nul) == abi.MOE_ERR_INVALID_ARG
    assert lib.moe_experts_backward_dropless(C.byref(bf), *([fake] * 10), fake,
                                             pb["dropless_experts_bwd_ws_bytes"] - 256, nul) == abi.MOE_ERR_WORKSPACE
    f32 = rcd.config_of(synth.workload("tiny_fp32"))
    assert lib.moe_dispatch_backward_dropless(C.byref(f32), fake, fake, fake, nul) == abi.MOE_ERR_UNSUPPORTED
    ww = abi.MoeWeights(*([0x100000] * 10))
    taps = abi.MoeDroplessTaps(*([0x100000] * 9))
    assert lib.moe_backward_dropless(C.byref(bf), C.byref(ww), C.byref(taps), *([fake] * 6), fake,
                                     pb["dropless_backward_ws_bytes"] - 1, nul) == abi.MOE_ERR_WORKSPACE
    taps.row_of = None
    assert lib.moe_backward_dropless(C.byref(bf), C.byref(ww), C.byref(taps), *([fake] * 6), fake,
                                     pb["dropless_backward_ws_bytes"], nul) == abi.MOE_ERR_INVALID_ARG



def test_router_bias_update_validation(lib):
    cfg = rcd.make_config(1000, 64, 64, 48, 8, 4, 64)
    n = C.c_size_t(0)
    assert lib.moe_router_bias_ws_bytes(C.byref(cfg), 256, C.byref(n)) == abi.MOE_OK
    # range partials, per-chunk histograms, ranges and quantiles, each 256-aligned
    c1, c2 = 1, 1
    expect = sum((b + 255) // 256 * 256 for b in (c1 * 48 * 8, c2 * 48 * 256 * 4, 48 * 8, 48 * 8))
    assert n.value == expect
    for nb in (0, -1, 1025):
        assert lib.moe_router_bias_ws_bytes(C.byref(cfg), nb, C.byref(n)) == abi.MOE_ERR_INVALID_ARG
    assert lib.moe_router_bias_ws_bytes(C.byref(cfg), 1024, C.byref(n)) == abi.MOE_OK
    assert lib.moe_router_bias_ws_bytes(C.byref(cfg), 8, None) == abi.MOE_ERR_INVALID_ARG
    fake, nul = C.c_void_p(0x100000), None
    lib.moe_router_bias_ws_bytes(C.byref(cfg), 64, C.byref(n))
    upd = lib.moe_router_bias_update
    assert upd(C.byref(cfg), nul, 64, fake, nul, nul, fake, n.value, nul) == abi.MOE_ERR_INVALID_ARG
    assert upd(C.byref(cfg), fake, 64, nul, nul, nul, fake, n.value, nul) == abi.MOE_ERR_INVALID_ARG
    assert upd(C.byref(cfg), fake, 64, fake, nul, nul, nul, n.value, nul) == abi.MOE_ERR_WORKSPACE
    assert upd(C.byref(cfg), fake, 64, fake, nul, nul, fake, n.value - 1, nul) == abi.MOE_ERR_WORKSPACE
    assert upd(C.byref(cfg), fake, 64, fake, nul, nul, C.c_void_p(0x100080), n.value,
               nul) == abi.MOE_ERR_WORKSPACE
    bad = rcd.make_config(0, 64, 64, 48, 8, 4, 64)      # T = 0: no logits to take quantiles of
    assert upd(C.byref(bad), fake, 64, fake, nul, nul, fake, n.value, nul) == abi.MOE_ERR_INVALID_ARG
    bad = rcd.make_config(1000, 64, 64, 48, 8, 49, 64)  # k > E
    assert upd(C.byref(bad), fake, 64, fake, nul, nul, fake, n.value, nul) == abi.MOE_ERR_INVALID_ARG
    bad = rcd.make_config(1000, 64, 64, 2048, 8, 4, 64)
    assert upd(C.byref(bad), fake, 64, fake, nul, nul, fake, n.value, nul) == abi.MOE_ERR_UNSUPPORTED
    assert lib.moe_router_bias_stage_count() == 4 == len(abi.BIAS_STAGES)
    prof = lib.moe_router_bias_update_profiled
    cfg_ok = rcd.make_config(1000, 64, 64, 48, 8, 4, 64)
    lib.moe_router_bias_ws_bytes(C.byref(cfg_ok), 64, C.byref(n))
    assert prof(C.byref(cfg_ok), fake, 64, fake, nul, nul, fake, n.value, nul, nul, 5) == abi.MOE_ERR_INVALID_ARG
    ev = (C.c_void_p * 4)()
    assert prof(C.byref(cfg_ok), fake, 64, fake, nul, nul, fake, n.value, nul, ev, 4) == abi.MOE_ERR_INVALID_ARG


def test_huge_explicit_caps_unsupported(lib):
    # an explicit capacity beyond int32 is rejected before any product with
    # W, P or E is formed (no int64 overflow on the way)
    for field in ("cap_send_rows", "cap_recv_rows"):
        cfg = rcd.config_of(synth.workload("mid_bf16"))
        setattr(cfg, field, 1 << 60)
        assert _status(lambda: rcd.plan(cfg)) == abi.MOE_ERR_UNSUPPORTED
        setattr(cfg, field, (1 << 31))
        assert _status(lambda: rcd.plan(cfg)) == abi.MOE_ERR_UNSUPPORTED



def test_dispatch_noalloc_validation(lib):
    # host checks come before the scratch's device address is looked up
    nul = None
    fake = C.c_void_p(0x100000)
    assert lib.moe_dispatch_noalloc_scratch_bytes() == 4 << 20
    cfg = rcd.config_of(synth.workload("mid_bf16"))
    assert lib.moe_dispatch_noalloc(C.byref(cfg), fake, fake, fake, fake, fake, fake, fake, fake,
                                    nul, nul) == abi.MOE_ERR_INVALID_ARG
    assert lib.moe_dispatch_noalloc(C.byref(cfg), nul, fake, fake, fake, fake, fake, fake, fake,
                                    fake, nul) == abi.MOE_ERR_INVALID_ARG
    # a shape whose scratch exceeds the array: 1M tokens x 8 over 1024 experts
    big = rcd.make_config(1 << 20, 64, 64, 1024, 1024, 8, 64, n_waves=1, dtype="bf16")
    assert rcd.plan(big)["dispatch_ws_bytes"] > lib.moe_dispatch_noalloc_scratch_bytes()
    assert lib.moe_dispatch_noalloc(C.byref(big), fake, fake, fake, fake, fake, fake, fake, fake,
                                    fake, nul) == abi.MOE_ERR_WORKSPACE
