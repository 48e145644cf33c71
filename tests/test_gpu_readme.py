"""The README's usage example, run as written on the GPU (seeded), then
checked against the oracle on the same inputs: the shard's master, moments,
codes and scales, and the rank's row-major FP8 weights and scale grids
(needs an MI355X)."""
import os
import re
import sys

import numpy as np
import pytest
import torch

import oracle
from tests.compare import compare

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _example():
    with open(os.path.join(ROOT, "README.md")) as f:
        blocks = re.findall(r"```python\n(.*?)```", f.read(), re.S)
    assert len(blocks) == 1, "README.md should hold one python example"
    return blocks[0]


def test_readme_example():
    print("[gpu-readme] running the README example", flush=True)
    sys.stdout.flush()
    torch.manual_seed(0)
    ns = {}
    exec(compile(_example(), "README.md", "exec"), ns)
    torch.cuda.synchronize()
    dims, plan, hp = ns["dims"], ns["plan"], ns["hp"]
    q, owned, table = oracle.plan(dims, plan.D, plan.rank)
    assert q == plan.shard_tiles and owned == plan.owned_tiles
    p = oracle.pack(dims, [w.cpu().numpy() for w in ns["weights"]], table)
    g = oracle.pack(dims, [x.cpu().numpy() for x in ns["grads"]], table)
    m = np.zeros_like(p)
    v = np.zeros_like(p)
    codes, scale, near = oracle.step(
        p, g, m, v, oracle.hparams(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay, hp.step))
    rep = compare(dict(master=ns["master"].cpu().numpy(), m=ns["m"].cpu().numpy(),
                       v=ns["v"].cpu().numpy(), codes=ns["codes"].cpu().numpy(),
                       scale_inv=ns["scale_inv"].cpu().numpy()),
                  dict(master=p, m=m, v=v, codes=codes, scale_inv=scale, near=near))
    print("[gpu-readme]", {k: v for k, v in rep.items() if k != "fail"}, flush=True)
    assert rep["ok"] and rep["exact"], rep["fail"]
    o8 = [np.zeros((E, H, W), dtype=np.uint8) for E, H, W in dims]
    osc = [np.zeros((E, -(-H // 128), -(-W // 128)), dtype=np.float32) for E, H, W in dims]
    oracle.unpack(dims, codes, scale, table, o8, osc)
    for k in range(len(dims)):
        assert np.array_equal(ns["fp8"][k].cpu().numpy(), o8[k]), k
        assert np.array_equal(ns["grid"][k].cpu().numpy(), osc[k]), k
