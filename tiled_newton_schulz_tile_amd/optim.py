"""torch.optim integration of the HiMuon step.

"Hierarchical Muon: Tiled Newton-Schulz Updates for Efficient Muon Optimization"
(Abstract) applies the tiled Newton-Schulz map to the momentum-gradient matrices of
dense weights and names runtime tile-size schedules among what the tiling allows.
Which parameters count as such matrices, and what updates the rest, is not on the
pages; the convention here: every 2-D parameter goes through HiMuon (all of them in one
plan, so one launch per kernel covers every layer), every other parameter through a
plain torch optimizer (AdamW unless one is given).  A parameter group can opt out with
``use_himuon=False``.

The HiMuon state lives on the device: fp32 weights are the parameters themselves, the
momentum is a tensor of the state dtype per matrix, and the gradient is copied into a
persistent buffer of that dtype each step (torch may hand out a new .grad tensor every
backward pass, while the plan holds device pointers).
"""
from __future__ import annotations

import bisect

import torch

from . import HiMuon, PREC_BF16X3, QUINTIC


class TileSchedule:
    """Tile size as a function of the optimizer step: a list of (first_step, T) pairs in
    increasing first_step, the first at step 0; T = 0 is FULL.  A plain int is a constant
    schedule."""

    def __init__(self, spec):
        if isinstance(spec, int):
            spec = [(0, spec)]
        spec = [(int(s), int(t)) for s, t in spec]
        if not spec or spec[0][0] != 0:
            raise ValueError("the schedule must start at step 0")
        if any(b[0] <= a[0] for a, b in zip(spec, spec[1:])):
            raise ValueError("schedule steps must increase")
        if any(t < 0 for _, t in spec):
            raise ValueError("tile sizes must be >= 0 (0 = FULL)")
        self.starts = [s for s, _ in spec]
        self.tiles = [t for _, t in spec]

    def __call__(self, step: int) -> int:
        return self.tiles[bisect.bisect_right(self.starts, step) - 1]

    @classmethod
    def every(cls, tiles, period: int):
        """Each T of `tiles` for `period` steps, in order (the last one stays)."""
        return cls([(i * period, t) for i, t in enumerate(tiles)])


def split_params(params):
    """(himuon_params, other_params) under the convention above; `params` is an iterable
    of tensors or of parameter-group dicts."""
    groups = list(params)
    if groups and not isinstance(groups[0], dict):
        groups = [{"params": groups}]
    hm_p, other = [], []
    for g in groups:
        use = g.get("use_himuon", True)
        for p in g["params"]:
            if not p.requires_grad:
                continue
            (hm_p if use and p.dim() == 2 else other).append(p)
    return hm_p, other


class HiMuonOptimizer(torch.optim.Optimizer):
    """HiMuon on the 2-D parameters, a plain optimizer on the others.

    lr, beta (momentum), steps (K), coeffs, eps and tile (an int or a TileSchedule) set
    the HiMuon step; state_dtype (torch.bfloat16 or torch.float32) is the dtype of the
    momentum and of the gradient copy; precision defaults to bf16x3.  `fallback` is a
    factory taking the list of other parameters (default: AdamW with lr fallback_lr)."""

    def __init__(self, params, lr: float = 0.02, beta: float = 0.95, tile=128, steps: int = 5,
                 coeffs=QUINTIC, eps: float = 1e-7, state_dtype=torch.bfloat16, precision=PREC_BF16X3,
                 workspace_budget: int = 4 * 10 ** 9, fallback=None, fallback_lr: float = 3e-4):
        hm_p, other = split_params(params)
        if not hm_p:
            raise ValueError("no 2-D parameters for HiMuon")
        for p in hm_p:
            if p.dtype != torch.float32 or not p.is_cuda:
                raise ValueError("HiMuon parameters must be float32 CUDA tensors")
        super().__init__(hm_p, dict(lr=lr))
        self.schedule = tile if isinstance(tile, TileSchedule) else TileSchedule(tile)
        self.steps, self.coeffs, self.beta, self.eps = steps, coeffs, beta, eps
        self.state_dtype, self.precision, self.budget = state_dtype, precision, workspace_budget
        self.fallback = None
        if other:
            self.fallback = (fallback(other) if fallback is not None
                             else torch.optim.AdamW(other, lr=fallback_lr))
        self.step_count = 0
        self._engine = None
        self._bufs = None

    def _build(self):
        ps = self.param_groups[0]["params"]
        self._bufs = [(torch.zeros(p.shape, dtype=self.state_dtype, device=p.device),
                       torch.zeros(p.shape, dtype=self.state_dtype, device=p.device)) for p in ps]
        self._tile = self.schedule(0)
        self._engine = HiMuon([(p.data, m, g) for p, (m, g) in zip(ps, self._bufs)], self._tile,
                              self.steps, self.coeffs, self.beta, self.eps, self.budget,
                              precision=self.precision)

    @torch.no_grad()
    def step(self, closure=None):
        loss = None
        if closure is not None:
            with torch.enable_grad():
                loss = closure()
        if self._engine is None:
            self._build()
        T = self.schedule(self.step_count)
        if T != self._tile:
            self._engine.set_tile_schedule(T)
            self._tile = T
        ps = self.param_groups[0]["params"]
        for p, (_, g) in zip(ps, self._bufs):
            if p.grad is None:
                g.zero_()
            else:
                g.copy_(p.grad)
        self._engine.step(self.param_groups[0]["lr"])
        if self.fallback is not None:
            self.fallback.step()
        self.step_count += 1
        return loss

    def zero_grad(self, set_to_none: bool = True):
        super().zero_grad(set_to_none)
        if self.fallback is not None:
            self.fallback.zero_grad(set_to_none)

    def momentum(self, p):
        """The HiMuon momentum tensor of 2-D parameter p."""
        for q, (m, _) in zip(self.param_groups[0]["params"], self._bufs or []):
            if q is p:
                return m
        raise KeyError("not a HiMuon parameter of this optimizer (or no step taken yet)")

    def close(self):
        if self._engine is not None:
            self._engine.close()
            self._engine = None
