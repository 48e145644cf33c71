"""Every slot of the dense-LLM rank shard (49,408 tiles, 809.5M elements,
t = 11 after ten warm-up steps) and of the 2.01B-element shard (122,880
tiles, t = 1000) against the oracle, in the launch configuration and state
layout the benchmark times: master, m, v, tile-major codes and scale_inv
of every slot, and the row-major FP8 weights and scale grids of every
owned tile against the oracle's own unfold of its codes.

The oracle regenerates and steps every tile on the host: about one
minute for the dense shard and two for the 2.01B-element one on 16 threads
(progress is printed every 8 chunks of 2048 slots)."""
import gc
import sys

import numpy as np
import pytest
import torch

import oracle
from bench_workload import GpuWorkload
from synth import workloads as WL
from tests.compare import compare
from tests.oracle_run import oracle_slots

pytestmark = pytest.mark.gpu

CHUNK = 2048


def _say(*a):
    print("[gpu-full]", *a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("name", ["dense_llm", "large"])
def test_every_slot_full_size(name):
    w = WL.BY_NAME[name]()
    _say(name, "every slot, mode fused_unpack, layout interleaved, seed", w.seed, "steps", w.steps)
    g = GpuWorkload(w, mode="fused_unpack", layout="interleaved")
    g.load_state()
    g.run_steps()
    q, owned, table = oracle.plan(w.dims, w.D, w.rank)
    assert q == g.q
    ora_codes = np.empty((q, 16384), dtype=np.uint8)
    ora_scale = np.empty(q, dtype=np.float32)
    totals = {"codes_mismatch": 0, "codes_mismatch_near_midpoint": 0, "near_midpoint_elems": 0}
    exact = True
    for s0 in range(0, q, CHUNK):
        slots = list(range(s0, min(q, s0 + CHUNK)))
        ora = oracle_slots(w, slots)
        rep = compare(g.tiles(slots), ora)
        assert rep["ok"], (name, s0, rep["fail"])
        exact &= rep["exact"]
        for k in totals:
            totals[k] += rep[k]
        ora_codes[s0:s0 + len(slots)] = ora["codes"]
        ora_scale[s0:s0 + len(slots)] = ora["scale_inv"]
        if (s0 // CHUNK) % 8 == 0:
            _say(f"{name} slots {s0}..{s0 + len(slots) - 1}: exact={rep['exact']}")
        del ora
    _say(name, "every slot:", q, "slots, bit-exact", exact, totals)
    assert exact
    o8 = [None] * len(w.dims)
    osc = [None] * len(w.dims)
    for p in g.touched:
        E, H, W = w.dims[p]
        o8[p] = np.zeros((E, H, W), dtype=np.uint8)
        osc[p] = np.zeros((E, -(-H // 128), -(-W // 128)), dtype=np.float32)
    oracle.unpack(w.dims, ora_codes.reshape(-1), ora_scale, table, o8, osc)
    fp8, sc = g.rowmajor()
    torch.cuda.synchronize()
    # tiles other ranks own stay zero on both sides (the outputs start zeroed)
    for p in g.touched:
        assert np.array_equal(fp8[p].cpu().numpy().reshape(o8[p].shape), o8[p]), p
        assert np.array_equal(sc[p].cpu().numpy().reshape(osc[p].shape), osc[p]), p
    _say(name, "row-major FP8 and scale grids of", len(g.touched), "weights equal the oracle's unfold")
    del g, fp8, sc, o8, osc, ora_codes
    gc.collect()
    torch.cuda.empty_cache()
