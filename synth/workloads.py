"""The five synthetic workloads: shapes, ranks, seeds and value recipes.

Shared by the tests, the smoke check and the benchmark.  Holds no optimizer
or quantizer arithmetic -- only which weights exist, which rank runs, and
how each input tensor is drawn (see synth.hip for the draws).

Common to all: AdamW lr 1e-4, betas (0.9, 0.95), eps 1e-8, weight decay 0.1;
128x128 tiles; master weights ~ N(0, 0.02) unless stated.
"""
from dataclasses import dataclass, field
from typing import Callable, List, Tuple

import synth

HP = dict(lr=1e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)

# stream ids of the tensors of one weight
MASTER, GRAD, MOM1, MOM2, EXPERT_SCALE, ZERO_TILES, DIMS = range(7)


@dataclass
class Workload:
    name: str
    config: int                 # stream id of the workload
    seed: int
    dims: List[Tuple[int, int, int]]
    D: int
    rank: int
    steps: List[int]            # step counters t, in order; the last is the measured one
    description: str
    kinds: dict = field(default_factory=dict)   # tensor -> (kind, scale)
    expert_logu: Tuple[float, float] = (0.0, 0.0)
    zero_tile_prob: float = 0.0
    emit_rowmajor: bool = True

    def _zero_key(self, p):
        return synth.key(self.seed, self.config, ZERO_TILES, p)

    def recipe(self, tensor: int, p: int, step: int = 0) -> synth.Recipe:
        """Recipe of tensor (MASTER, GRAD, MOM1, MOM2) of weight p; grads are
        drawn afresh for every step t, the others once (step 0)."""
        E, H, W = self.dims[p]
        kind, scale = self.kinds[tensor]
        k = synth.key(self.seed, self.config, tensor, p, step if tensor == GRAD else 0)
        return synth.recipe(kind, k, H, W, scale=scale, logu=self.expert_logu,
                            expert_key=synth.key(self.seed, self.config, EXPERT_SCALE, 0),
                            zero_tile_prob=self.zero_tile_prob, zero_key=self._zero_key(p))

    def numel(self, p):
        E, H, W = self.dims[p]
        return E * H * W

    @property
    def measured_step(self):
        return self.steps[-1]


def _kinds(master=(synth.NORMAL, 0.02), grad=(synth.NORMAL, 1e-3), m=(synth.ZERO, 0.0),
           v=(synth.ZERO, 0.0)):
    return {MASTER: master, GRAD: grad, MOM1: m, MOM2: v}


def tiny() -> Workload:
    return Workload(
        name="tiny", config=1, seed=0, dims=[(1, 256, 384)], D=1, rank=0, steps=[1, 2, 3],
        description="one 256x384 fp32 weight (2x3 tiles), grads N(0,1e-3) fresh each step, "
                    "m=v=0, 3 steps",
        kinds=_kinds())


def dense_llm() -> Workload:
    layer = [(1, 4096, 4096)] * 4 + [(1, 4096, 11008)] * 2 + [(1, 11008, 4096)]
    return Workload(
        name="dense_llm", config=2, seed=2, dims=layer * 32, D=8, rank=0,
        steps=list(range(1, 12)),
        description="32 layers x {4 of 4096x4096, 2 of 4096x11008, 1 of 11008x4096}, "
                    "D=8, rank 0 (49408 tiles, 809.5M elements); m/v warm from 10 prior "
                    "steps with fresh N(0,1e-3) grads, measured step t=11",
        kinds=_kinds())


def ragged_dims(seed=3, config=3, n=40):
    dims = []
    for p in range(n):
        k = synth.key(seed, config, DIMS, p)
        h = 129 + int(synth.lib().synth_uniform(k, 0) * 7040)
        w = 129 + int(synth.lib().synth_uniform(k, 1) * 7040)
        dims.append((1, h, w))
    return dims


def ragged() -> Workload:
    return Workload(
        name="ragged", config=3, seed=3, dims=ragged_dims(), D=8, rank=3, steps=[1],
        description="40 matrices, H and W uniform in [129, 7168], D=8, rank 3; "
                    "m=v=0, t=1",
        kinds=_kinds())


def moe() -> Workload:
    return Workload(
        name="moe_experts", config=4, seed=4,
        dims=[(256, 7168, 2048), (256, 7168, 2048), (256, 2048, 7168)], D=32, rank=0, steps=[1],
        description="256 experts x (gate 7168x2048, up 7168x2048, down 2048x7168), D=32, "
                    "rank 0 (21504 tiles); grads 10^U(-5,-2) x N(0,1) per expert; m=v=0, t=1",
        kinds=_kinds(grad=(synth.EXPERT_LOGU, 1.0)), expert_logu=(-5.0, -2.0))


def large() -> Workload:
    return Workload(
        name="large", config=5, seed=5, dims=[(1, 4096, 4096)] * 120, D=1, rank=0,
        steps=[1000],
        description="120 matrices of 4096x4096 (2.01B elements), D=1; grads, m 1e-3 t(3), "
                    "v (1e-3 t(3))^2; 1% of tiles all zero; t=1000; also row-major FP8 out",
        kinds=_kinds(grad=(synth.T3, 1e-3), m=(synth.T3, 1e-3), v=(synth.T3_SQUARED, 1e-3)),
        zero_tile_prob=0.01)


ALL: List[Callable[[], Workload]] = [tiny, dense_llm, ragged, moe, large]
BY_NAME = {f().name if f is not ragged else "ragged": f for f in (tiny, dense_llm, moe, large)}
BY_NAME["ragged"] = ragged


def rows_touched(table, p, dims):
    """Flat element range [lo, hi) of weight p covered by the table's slots of p
    (the rows of its first to its last owned tile row, whole width)."""
    E, H, W = dims[p]
    rows = [r for r in table if r[0] == p]
    if not rows:
        return 0, 0
    e0, i0 = int(rows[0][1]), int(rows[0][2])
    e1, i1 = int(rows[-1][1]), int(rows[-1][2])
    lo = (e0 * H + 128 * i0) * W
    hi = (e1 * H + min(H, 128 * (i1 + 1))) * W
    return lo, hi
