"""The head step as a HIP graph and on concurrent streams: the library allocates nothing, launches
only kernels on the caller's stream and keeps no per-call state outside its arguments, so a captured
step replays to the eager result bit for bit, and two steps on two streams at once give what they
give one after the other."""
import numpy as np
import pytest
import torch

from lm_head_cross_amd import head as H
from lm_head_cross_amd import synth
from tests.gpu_helpers import dev, say

pytestmark = pytest.mark.gpu

OUTS = ("logp", "lse", "out", "g", "dh", "dW")


def _step(cfg, seed):
    d = dev()
    inp = synth.make_inputs(cfg, seed=seed, label_device="cuda")
    args = (inp.h.to(d), inp.w.to(d), torch.from_numpy(inp.labels).to(d),
            torch.from_numpy(inp.seg_offsets).to(d))
    return H.HeadStep(*args, cfg.V, cfg.softcap, cfg.lam)


def _snap(step):
    return {k: getattr(step, k).clone() for k in OUTS}


def test_head_step_replays_as_a_hip_graph():
    cfg = synth.reduced(synth.workload("e4b-bf16-softcap30"), 2).replace(V=20000, name="e4b-like-graph")
    say(f"[case] graph replay {cfg.name} M={cfg.M} V={cfg.V}")
    step = _step(cfg, 0)
    step.step()
    torch.cuda.synchronize()
    ref = _snap(step)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm-up on a side stream before capture
        step.step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step.step()
    for rep in range(3):
        for k in OUTS:                     # eager work between replays: clobber every output
            getattr(step, k).fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k in OUTS:
            assert torch.equal(getattr(step, k), ref[k]), (rep, k)
    say("[graph] 3 replays equal the eager step bit for bit")


def test_two_steps_on_two_streams_match_sequential():
    cfg = synth.reduced(synth.workload("minicpm-like-bf16"), 2).replace(name="minicpm-like-streams")
    say(f"[case] two streams {cfg.name} M={cfg.M} V={cfg.V}")
    a, b = _step(cfg, 1), _step(cfg, 2)
    a.step()
    b.step()
    torch.cuda.synchronize()
    ra, rb = _snap(a), _snap(b)
    for s in (a, b):
        for k in OUTS:
            getattr(s, k).fill_(float("nan"))
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    with torch.cuda.stream(sa):
        a.step()
    with torch.cuda.stream(sb):
        b.step()
    torch.cuda.synchronize()
    for k in OUTS:
        assert torch.equal(getattr(a, k), ra[k]) and torch.equal(getattr(b, k), rb[k]), k
    assert not torch.equal(ra["dh"], rb["dh"])       # the two problems differ
