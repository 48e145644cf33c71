"""Device state of one rank's shard of a synthetic workload, driven through
the library's calls only (no oracle): used by bench.py, the smoke check and
the GPU tests.

Inputs are row-major FP32 weights drawn on the device by the seeded
generator; the path then folds them (pack_shard), steps (adamw_fp8_step)
and unfolds (unpack_fp8), exactly as a rank would.
"""
import numpy as np
import torch

import blockwise_fp8_zero_amd as bfz
import synth
from synth import workloads as WL

TILE_ELEMS = bfz.TILE_ELEMS


def hp_for(t):
    """The workloads' AdamW hyper-parameters at step counter t."""
    return bfz.AdamW(step=t, **WL.HP)


class GpuWorkload:
    """Device state of one rank's shard of workload w."""

    MODES = ("unfused", "fused", "fused_unpack")

    LAYOUTS = ("separate", "interleaved")

    def __init__(self, w: WL.Workload, device="cuda", mode="unfused", pow2=False, transposed=False,
                 layout="separate"):
        """mode: how a step is taken --
        "unfused": pack_shard + adamw_fp8_step (then unpack_fp8 on demand);
        "fused": fold_adamw_fp8_step (gradients read row-major);
        "fused_unpack": fold_adamw_fp8_step_unpack, which also writes the
        row-major FP8 weights and scale grids (self.out_fp8 / self.out_scale).
        transposed (fused_unpack with pow2 only): fold_adamw_fp8_step_unpack_t,
        which also writes W^T and its group scales (self.out_t / self.out_t_scale).
        layout: the FP32 state -- "separate": master, m, v are three
        tile-major arrays; "interleaved": one (q, bfz.STATE_STRIDE) tensor,
        each tile's [master | m | v] contiguous, passed as its three
        (q, 16384) column views."""
        assert mode in self.MODES, mode
        assert layout in self.LAYOUTS, layout
        self.layout = layout
        assert not transposed or (mode == "fused_unpack" and pow2), "transposed: fused_unpack + pow2"
        self.transposed = transposed
        self.w = w
        self.mode = mode
        self.pow2 = pow2  # power-of-two tile scales
        self.device = torch.device(device)
        with torch.cuda.device(self.device):
            self.plan = bfz.Plan(w.dims, w.D, w.rank)
        self.q = self.plan.shard_tiles
        self.owned = self.plan.owned_tiles
        self.table = self.plan.table()
        owned_rows = self.table[:self.owned]
        self.touched = sorted({int(p) for p in owned_rows[:, 0]})
        self.ranges = {p: WL.rows_touched(owned_rows, p, w.dims) for p in self.touched}
        n = self.q * TILE_ELEMS
        kw = dict(device=self.device)
        if layout == "interleaved":
            self.state = torch.empty((self.q, bfz.STATE_STRIDE), dtype=torch.float32, **kw)
            self.master, self.m, self.v = (self.state[:, k * TILE_ELEMS:(k + 1) * TILE_ELEMS]
                                           for k in range(3))
        else:
            self.master = torch.empty(n, dtype=torch.float32, **kw)
            self.m = torch.empty(n, dtype=torch.float32, **kw)
            self.v = torch.empty(n, dtype=torch.float32, **kw)
        self.grad = torch.empty(n, dtype=torch.float32, **kw)
        self.codes = torch.empty(n, dtype=torch.uint8, **kw)
        self.scale_inv = torch.empty(self.q, dtype=torch.float32, **kw)
        self.grad_rm = None
        # fused_unpack only: False = row-major output alone (a lone rank has
        # nothing to all-gather, so no tile-major codes or scales)
        self.tile_codes = True
        self.t_done = 0
        self.out_fp8 = self.out_scale = None
        self.out_t = self.out_t_scale = None
        if mode == "fused_unpack":
            self.out_fp8, self.out_scale = self.alloc_rowmajor_out()
        if transposed:
            self.out_t, self.out_t_scale = self.alloc_transposed_out()

    # ---- inputs ------------------------------------------------------------
    def _rowmajor(self, tensor, step=0):
        """Row-major device buffers of every touched weight, drawn over the
        rows the rank's tiles cover (other rows are never read)."""
        bufs = [None] * len(self.w.dims)
        for p in self.touched:
            lo, hi = self.ranges[p]
            b = torch.empty(self.w.numel(p), dtype=torch.float32, device=self.device)
            synth.fill_device(self.w.recipe(tensor, p, step), b[lo:hi], lo, hi)
            bufs[p] = b
        return bufs

    def load_state(self):
        """Fold the initial master, m and v into the shard."""
        for tensor, dst in ((WL.MASTER, self.master), (WL.MOM1, self.m), (WL.MOM2, self.v)):
            srcs = self._rowmajor(tensor)
            bfz.pack_shard(self.plan, srcs, dst)
            del srcs
        torch.cuda.synchronize(self.device)

    def draw_grads(self, t):
        self.grad_rm = self._rowmajor(WL.GRAD, t)

    # ---- the path ------------------------------------------------------------
    def pack_grads(self):
        bfz.pack_shard(self.plan, self.grad_rm, self.grad)

    def step(self, t):
        bfz.adamw_fp8_step(self.master, self.grad, self.m, self.v, self.codes, self.scale_inv,
                           hp_for(t), scale_pow2=self.pow2)

    def fold_step(self, t):
        bfz.fold_adamw_fp8_step(self.plan, self.grad_rm, self.master, self.m, self.v, self.codes,
                                self.scale_inv, hp_for(t), scale_pow2=self.pow2)

    def fold_step_unpack(self, t):
        codes, scale = (self.codes, self.scale_inv) if self.tile_codes else (None, None)
        if self.transposed:
            bfz.fold_adamw_fp8_step_unpack_t(self.plan, self.grad_rm, self.master, self.m, self.v,
                                             codes, scale, self.out_fp8, self.out_scale,
                                             self.out_t, self.out_t_scale, hp_for(t))
            return
        bfz.fold_adamw_fp8_step_unpack(self.plan, self.grad_rm, self.master, self.m, self.v,
                                       codes, scale, self.out_fp8, self.out_scale, hp_for(t),
                                       scale_pow2=self.pow2)

    def apply(self, t):
        """One step on the current row-major gradients."""
        if self.mode == "fused":
            self.fold_step(t)
        elif self.mode == "fused_unpack":
            self.fold_step_unpack(t)
        else:
            self.pack_grads()
            self.step(t)

    def rowmajor(self):
        """Row-major FP8 weights and scale grids of the owned tiles: those the
        last step wrote (fused_unpack), else a fresh unpack_fp8."""
        if self.mode == "fused_unpack":
            return self.out_fp8, self.out_scale
        fp8, sc = self.alloc_rowmajor_out()
        self.unpack(fp8, sc)
        return fp8, sc

    def run_steps(self, steps=None):
        """Draw, fold and apply the grads of each step counter in `steps`."""
        for t in (steps if steps is not None else self.w.steps):
            self.draw_grads(t)
            self.apply(t)
            self.t_done = t
        torch.cuda.synchronize(self.device)

    def alloc_rowmajor_out(self):
        fp8 = [None] * len(self.w.dims)
        sc = [None] * len(self.w.dims)
        for p in self.touched:
            E, H, W = self.w.dims[p]
            fp8[p] = torch.zeros(E * H * W, dtype=torch.uint8, device=self.device)
            sc[p] = torch.zeros(E * (-(-H // 128)) * (-(-W // 128)), dtype=torch.float32,
                                device=self.device)
        return fp8, sc

    def alloc_transposed_out(self):
        wt = [None] * len(self.w.dims)
        wts = [None] * len(self.w.dims)
        for p in self.touched:
            E, H, W = self.w.dims[p]
            wt[p] = torch.zeros(E * W * H, dtype=torch.uint8, device=self.device)
            wts[p] = torch.zeros(E * W * (-(-H // 128)), dtype=torch.float32, device=self.device)
        return wt, wts

    def unpack(self, fp8, sc):
        bfz.unpack_fp8(self.plan, self.codes, self.scale_inv, fp8, sc)

    # ---- read back ---------------------------------------------------------
    def tiles(self, slots):
        idx = torch.as_tensor(np.asarray(slots, dtype=np.int64), device=self.device)

        def take(x):
            return x.view(-1, TILE_ELEMS).index_select(0, idx).cpu().numpy()

        return dict(master=take(self.master), m=take(self.m), v=take(self.v),
                    codes=take(self.codes), scale_inv=self.scale_inv[idx].cpu().numpy())


def sample_slots(w, table, q, owned, n_random=24, seed=0):
    """A sample of a shard's slots for spot checks: first, last owned and
    last, the two slots at each weight boundary (up to 60), the first and
    last 8 edge slots, up to 8 all-zero tiles where the workload has them,
    and n_random seeded random slots.  table: the plan's [q, 6] table."""
    pick = {0, max(0, owned - 1), q - 1}
    for s in range(1, owned):
        if table[s][0] != table[s - 1][0]:
            pick.update((s - 1, s))
        if len(pick) > 60:
            break
    edge = [s for s in range(owned) if table[s][4] < 128 or table[s][5] < 128]
    pick.update(edge[:8] + edge[-8:])
    if w.zero_tile_prob > 0:
        zeros = []
        for s in range(owned):
            p, e, i, j = (int(x) for x in table[s][:4])
            E, H, W = w.dims[p]
            hb, wb = -(-H // 128), -(-W // 128)
            if synth.lib().synth_uniform(w._zero_key(p), (e * hb + i) * wb + j) < w.zero_tile_prob:
                zeros.append(s)
            if len(zeros) >= 8:
                break
        pick.update(zeros)
    rng = np.random.default_rng(seed)
    pick.update(int(x) for x in rng.integers(0, q, size=min(n_random, q)))
    return sorted(pick)


def launch_segments(table, owned, q, per_launch=64):
    """Launches one call of a plan-driven entry point makes: runs of owned
    slots whose weights span fewer than per_launch weight indices, plus one
    for the padding slots."""
    n, first = 0, None
    for s in range(owned):
        p = int(table[s][0])
        if first is None or p - first >= per_launch:
            n, first = n + 1, p
    return n + (1 if owned < q else 0)
