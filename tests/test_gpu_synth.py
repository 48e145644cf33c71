"""The seeded input generator on the GPU: the device fill and the host fill
draw the same float32 values, bit for bit, for every kind of draw and at
element indices past 2^32 (the full-size workloads' device state and the
oracle's host regeneration of any slot rest on this)."""
import sys

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

KINDS = {
    "normal": dict(kind=synth.NORMAL, scale=0.02),
    "t3": dict(kind=synth.T3, scale=1e-3),
    "t3_squared": dict(kind=synth.T3_SQUARED, scale=1e-3),
    "expert_logu": dict(kind=synth.EXPERT_LOGU, scale=1.0, logu=(-5.0, -2.0)),
    "zero": dict(kind=synth.ZERO, scale=0.0),
    "normal_zero_tiles": dict(kind=synth.NORMAL, scale=1.0, zero_tile_prob=0.3),
}


@pytest.mark.parametrize("name", sorted(KINDS))
@pytest.mark.parametrize("lo", [0, 3 * 2 ** 31 + 12345])
def test_device_fill_equals_host_fill(name, lo):
    spec = dict(KINDS[name])
    kind = spec.pop("kind")
    H, W = 4096, 2048
    r = synth.recipe(kind, synth.key(11, 12, 13, 14), H, W, expert_key=synth.key(11, 12, 99, 0),
                     zero_key=synth.key(11, 12, 98, 0), **spec)
    n = 1 << 18
    print("[gpu-synth]", name, "lo", lo, "n", n, flush=True)
    sys.stdout.flush()
    dev = torch.empty(n, dtype=torch.float32, device="cuda")
    synth.fill_device(r, dev, lo, lo + n)
    torch.cuda.synchronize()
    host = synth.fill_host(r, lo, lo + n)
    assert np.array_equal(dev.cpu().numpy().view(np.uint32), host.view(np.uint32))
