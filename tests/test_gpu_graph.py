"""The forward and backward entry points under HIP graph capture.

The library allocates nothing, synchronises nothing and enqueues only kernel
launches on the caller's stream, so a caller may capture a whole forward or
backward call in a graph and replay it.  Each test captures one call, then replays it
several times with other inputs copied into the captured input buffer
between replays (eager work and synchronisations in between), and checks
every replay bit for bit against an eager call on the same input: the path
is deterministic, so the two must agree exactly.  Nothing but the library
call is recorded in the graph."""
import pytest
import torch

import routing_capacity_dispatch_amd as rcd
import synth
from gpu_common import dev, say

pytestmark = pytest.mark.gpu


def _capture(call, x):
    """A graph of one call(x), after a warm-up call on a side stream."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(x)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(x)
    torch.cuda.synchronize()
    return g


def _check_replays(call, make_call, xs, outputs):
    """Replay a graph of call on xs[0] with each of xs copied in turn into
    its input buffer, the outputs cleared before each replay; compare each
    replay with an eager call of a separate instance (make_call()) on the
    same input."""
    x = xs[0].clone()
    g = _capture(call, x)
    ref = make_call()
    for i, xi in enumerate(xs + xs[:1]):
        x.copy_(xi)
        for t in outputs(call):
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref(xi)
        torch.cuda.synchronize()
        for got, want in zip(outputs(call), outputs(ref)):
            assert torch.equal(got, want), f"replay {i} differs from the eager call"


@pytest.mark.parametrize("seeds", [(0, 1, 2)])
def test_forward_graph_replays_match_eager(seeds):
    d = dev()
    w = synth.workload("mid_bf16")
    say("forward under graph capture", w.name)
    cfg = rcd.config_of(w)
    inp = synth.make_inputs(w, seeds[0], device=d)
    weights = {k: v for k, v in inp.items() if k != "x"}
    xs = [synth.make_inputs(w, s, device=d)["x"] for s in seeds]
    fwd = rcd.Forward(cfg, weights, d)
    _check_replays(fwd, lambda: rcd.Forward(cfg, weights, d), xs, lambda f: (f.y, f.counts))


def test_forward_dropless_graph_replays_match_eager():
    d = dev()
    w = synth.workload("mid_bf16")
    say("dropless forward under graph capture", w.name)
    cfg = rcd.config_of(w)
    inp = synth.make_inputs(w, 3, device=d)
    weights = {k: v for k, v in inp.items() if k != "x"}
    xs = [synth.make_inputs(w, s, device=d)["x"] for s in (3, 4)]
    fwd = rcd.ForwardDropless(cfg, weights, d)
    _check_replays(fwd, lambda: rcd.ForwardDropless(cfg, weights, d), xs, lambda f: (f.y, f.counts))


@pytest.mark.parametrize("dropless", [False, True])
def test_backward_graph_replays_match_eager(dropless):
    d = dev()
    w = synth.workload("mid_bf16")
    say("backward under graph capture", w.name, "dropless" if dropless else "capped")
    cfg = rcd.config_of(w)
    inp = synth.make_inputs(w, 5, device=d)
    weights = {k: v for k, v in inp.items() if k != "x"}
    fwd = (rcd.ForwardDropless if dropless else rcd.Forward)(cfg, weights, d, taps=True)
    fwd(inp["x"])
    torch.cuda.synchronize()
    g_gen = torch.Generator(device="cpu").manual_seed(6)
    dys = [torch.randn((w.T, w.d_latent), generator=g_gen).to(device=d, dtype=torch.bfloat16)
           for _ in range(2)]
    bwd = rcd.BackwardRouted(fwd)
    _check_replays(bwd, lambda: rcd.BackwardRouted(fwd), dys,
                   lambda b: (b.dz, b.d_logits) + tuple(b.dw))
