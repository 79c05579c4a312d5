"""torch.optim integration of the HiMuon step.

"Hierarchical Muon: Tiled Newton-Schulz Updates for Efficient Muon Optimization"
(Abstract) applies the tiled Newton-Schulz map to the momentum-gradient matrices of
dense weights and names runtime tile-size schedules among what the tiling allows.
Which parameters count as such matrices, and what updates the rest, is not on the
pages; the convention here: every 2-D parameter goes through HiMuon, every other
parameter through a plain torch optimizer (AdamW unless one is given).  A parameter
group can opt out with ``use_himuon=False``.  HiMuon parameters that share a learning
rate share one plan (one launch per kernel covers all of their layers); groups with
their own ``lr`` get a plan each, and the step reads every group's current ``lr``, so
learning-rate schedulers work as usual.

The HiMuon state lives on the device: fp32 weights are the parameters themselves, the
momentum is ``state[p]["momentum_buffer"]`` (the state dtype, saved and restored by
``state_dict`` / ``load_state_dict``), and the gradient is copied into a persistent
buffer of that dtype each step (torch may hand out a new .grad tensor every backward
pass, while the plan holds device pointers).
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


def split_params(params, lr: float):
    """(himuon_groups, other_params) under the convention above.  `params` is an iterable
    of tensors or of parameter-group dicts; himuon_groups is a list of (lr, [params]),
    one per distinct learning rate, in order of first appearance."""
    groups = list(params)
    if groups and not isinstance(groups[0], dict):
        groups = [{"params": groups}]
    by_lr, other = {}, []
    for g in groups:
        use = g.get("use_himuon", True)
        glr = float(g.get("lr", lr))
        for p in g["params"]:
            if not p.requires_grad:
                continue
            if use and p.dim() == 2:
                by_lr.setdefault(glr, []).append(p)
            else:
                other.append(p)
    return list(by_lr.items()), other


class HiMuonOptimizer(torch.optim.Optimizer):
    """HiMuon on the 2-D parameters, a plain optimizer on the others.

    lr, beta (momentum), steps (K), coeffs, eps and tile (an int or a TileSchedule) set
    the HiMuon step; state_dtype (torch.bfloat16 or torch.float32) is the dtype of the
    momentum and of the gradient copy; precision defaults to bf16x3.  `fallback` is a
    factory taking the list of other parameters (default: AdamW with lr fallback_lr).
    The optimizer step count is saved with the state, so a restored optimizer resumes
    the tile schedule where it stopped."""

    def __init__(self, params, lr: float = 0.02, beta: float = 0.95, tile=128, steps: int = 5,
                 coeffs=QUINTIC, eps: float = 1e-7, state_dtype=torch.bfloat16, precision=PREC_BF16X3,
                 workspace_budget: int = 4 * 10 ** 9, fallback=None, fallback_lr: float = 3e-4):
        hm_groups, other = split_params(params, lr)
        if not hm_groups:
            raise ValueError("no 2-D parameters for HiMuon")
        for _, ps in hm_groups:
            for p in ps:
                if p.dtype != torch.float32 or not p.is_cuda:
                    raise ValueError("HiMuon parameters must be float32 CUDA tensors")
        super().__init__([{"params": ps, "lr": glr} for glr, ps in hm_groups], dict(lr=lr, step_count=0))
        self.schedule = tile if isinstance(tile, TileSchedule) else TileSchedule(tile)
        self.steps, self.coeffs, self.beta, self.eps = steps, coeffs, beta, eps
        self.state_dtype, self.precision, self.budget = state_dtype, precision, workspace_budget
        self.fallback = None
        if other:
            self.fallback = (fallback(other) if fallback is not None
                             else torch.optim.AdamW(other, lr=fallback_lr))
        self._engines = None
        self._grads = None
        self._tile = None

    @property
    def step_count(self) -> int:
        return int(self.param_groups[0]["step_count"])

    def _build(self):
        """One plan per parameter group over the group's weights, momentum buffers (made
        here on first use, or restored by load_state_dict) and gradient buffers."""
        self._tile = self.schedule(self.step_count)
        self._engines, self._grads = [], []
        for grp in self.param_groups:
            layers, grads = [], []
            for p in grp["params"]:
                st = self.state[p]
                if "momentum_buffer" not in st:
                    st["momentum_buffer"] = torch.zeros(p.shape, dtype=self.state_dtype, device=p.device)
                m = st["momentum_buffer"]
                if m.dtype != self.state_dtype or m.shape != p.shape or not m.is_contiguous():
                    raise ValueError("momentum_buffer must be a contiguous tensor of the state dtype")
                g = torch.zeros(p.shape, dtype=self.state_dtype, device=p.device)
                layers.append((p.data, m, g))
                grads.append(g)
            self._engines.append(HiMuon(layers, self._tile, self.steps, self.coeffs, self.beta, self.eps,
                                        self.budget, precision=self.precision))
            self._grads.append(grads)

    @torch.no_grad()
    def step(self, closure=None):
        loss = None
        if closure is not None:
            with torch.enable_grad():
                loss = closure()
        if self._engines is None:
            self._build()
        T = self.schedule(self.step_count)
        if T != self._tile:
            for eng in self._engines:
                eng.set_tile_schedule(T)
            self._tile = T
        for grp, eng, grads in zip(self.param_groups, self._engines, self._grads):
            for p, g in zip(grp["params"], grads):
                if p.grad is None:
                    g.zero_()
                else:
                    g.copy_(p.grad)
            eng.step(float(grp["lr"]))
        if self.fallback is not None:
            self.fallback.step()
        for grp in self.param_groups:
            grp["step_count"] = self.step_count + 1
        return loss

    def zero_grad(self, set_to_none: bool = True):
        super().zero_grad(set_to_none)
        if self.fallback is not None:
            self.fallback.zero_grad(set_to_none)

    def state_dict(self):
        sd = super().state_dict()
        if self.fallback is not None:
            sd["fallback"] = self.fallback.state_dict()
        return sd

    def load_state_dict(self, state_dict):
        """Restores momentum, step count and the fallback's state; the plans are rebuilt
        on the next step over the restored momentum tensors."""
        state_dict = dict(state_dict)
        fb = state_dict.pop("fallback", None)
        self.close()
        super().load_state_dict(state_dict)
        for st in self.state.values():
            m = st.get("momentum_buffer")
            if m is not None and (m.dtype != self.state_dtype or not m.is_contiguous()):
                st["momentum_buffer"] = m.to(self.state_dtype).contiguous()
        if fb is not None and self.fallback is not None:
            self.fallback.load_state_dict(fb)

    def momentum(self, p):
        """The HiMuon momentum tensor of 2-D parameter p."""
        st = self.state.get(p)
        if not st or "momentum_buffer" not in st:
            raise KeyError("not a HiMuon parameter of this optimizer (or no step taken yet)")
        return st["momentum_buffer"]

    def close(self):
        if self._engines is not None:
            for eng in self._engines:
                eng.close()
            self._engines = None
            self._grads = None
