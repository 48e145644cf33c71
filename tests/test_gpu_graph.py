"""The step calls under HIP graph capture: they enqueue kernels only (no
allocation, no synchronization, no memset), so a captured
fold_adamw_fp8_step_unpack replays to the same bits as the eager call.

The graph is replayed three times; before each replay the state, codes
and row-major outputs are reset to the pre-step values by ordinary eager
copies, and after it every output is compared with the eager step's,
bit for bit."""
import sys

import numpy as np
import pytest
import torch

import blockwise_fp8_zero_amd as bfz
from bench_workload import GpuWorkload, hp_for
from synth import workloads as WL

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[gpu-graph]", *a, flush=True)
    sys.stdout.flush()


def _snapshot(g):
    out = [g.state.clone(), g.codes.clone(), g.scale_inv.clone()]
    out += [x.clone() for x in g.out_fp8 + g.out_scale if x is not None]
    return out


def _restore(g, snap):
    dst = [g.state, g.codes, g.scale_inv] + [x for x in g.out_fp8 + g.out_scale if x is not None]
    for d, s in zip(dst, snap):
        d.copy_(s)


def _same(a, b):
    return all(torch.equal(x.view(torch.uint8), y.view(torch.uint8)) for x, y in zip(a, b))


@pytest.mark.parametrize("name", ["ragged", "moe_experts"])
def test_captured_step_replays_bit_identical(name):
    w = WL.BY_NAME[name]()
    if name == "ragged":
        w.dims = w.dims[:12]
    _say(name, "one-kernel step captured in a graph, 3 replays against the eager step")
    g = GpuWorkload(w, mode="fused_unpack", layout="interleaved")
    g.load_state()
    t = w.measured_step
    g.draw_grads(t)
    torch.cuda.synchronize()
    before = _snapshot(g)
    hp = hp_for(t)

    def step():
        bfz.fold_adamw_fp8_step_unpack(g.plan, g.grad_rm, g.master, g.m, g.v, g.codes,
                                       g.scale_inv, g.out_fp8, g.out_scale, hp)

    step()  # eager (also sets the kernel's LDS attribute before capture)
    torch.cuda.synchronize()
    want = _snapshot(g)
    assert not _same(want[:1], before[:1])  # the step changed the state

    _restore(g, before)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for k in range(3):
        _restore(g, before)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = _snapshot(g)
        assert _same(got, want), ("replay", k)
        _say(name, "replay", k, "bit-identical to the eager step")
    del graph, g
    torch.cuda.empty_cache()
