"""One optimizer step over an hpo set, ordered as the pages order it.

"02 · Optimizer：算法与 infra" §10.2 / §11.1: zero found_inf, unscale + check,
global norm, clip, inner step, write-back; a found_inf step returns early,
with no clip, no inner step and no advance of the step counter, and the
caller gets (success, grad_norm, num_zeros) back, (False, None, None) on a
skipped step.  num_zeros is reported when log_num_zeros_in_grad is set
(§17's config field, off by default), else None.

Host logic only.  The computation is the library's: one norm pass that also
checks for inf/NaN and counts zeros, one finalize, one fused update launched
with the device flag so it skips itself, then a single 16-byte read of
{found_inf, norm, num_zeros}.
"""
from __future__ import annotations

from typing import Optional, Sequence, Tuple

import numpy as np
import torch

from . import hpo


class MixedPrecisionAdamW:
    def __init__(self, hset: hpo.HpoSet, groups: Sequence[Tuple[float, float]], *, beta1: float = 0.9,
                 beta2: float = 0.999, eps: float = 1e-8, mode: int = hpo.HPO_ADAMW,
                 max_norm: float = 1.0, loss_scale: Optional[float] = None,
                 log_num_zeros_in_grad: bool = False, device=None):
        self.set = hset
        self.cfg = hpo.make_cfg(beta1, beta2, eps, mode)
        self.groups, self.n_groups = hpo.make_groups(list(groups))
        self.max_norm = float(max_norm)
        self.loss_scale = loss_scale
        self.log_num_zeros_in_grad = bool(log_num_zeros_in_grad)
        self.t = 0  # applied steps so far
        dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
        # two step buffers, used in turn: [0] found_inf (int32), [1] norm (fp32
        # bits), [2:4] num_zeros (int64).  A step clears the other one for the
        # next step while the host waits, and its own keeps its results.
        self._bufs = torch.zeros(2, 4, dtype=torch.int32, device=dev)
        self._host = torch.zeros(4, dtype=torch.int32, pin_memory=True)
        self._cur = 0      # buffer of the last step (the attributes below)
        self._next = 0     # buffer the next step writes
        self._cleared = False   # the zeros above may still be in flight on the constructing stream

    @property
    def found_inf(self) -> torch.Tensor:
        return self._bufs[self._cur, 0:1]

    @property
    def norm(self) -> torch.Tensor:
        return self._bufs[self._cur, 1:2].view(torch.float32)

    @property
    def num_zeros(self) -> torch.Tensor:
        return self._bufs[self._cur, 2:4].view(torch.int64)

    def inv_scale(self) -> float:
        return 1.0 if self.loss_scale is None else float(np.float32(1.0 / self.loss_scale))

    def step(self, stream=None, inplace_unscale: bool = False):
        """Returns (applied, grad_norm, num_zeros): (False, None, None) on a
        skipped step; num_zeros is None unless log_num_zeros_in_grad is set.

        inplace_unscale=True runs the pages' literal sequence (grads are
        unscaled in place first, then norm and step take inv_scale = 1)."""
        inv = self.inv_scale()
        s = torch.cuda.current_stream() if stream is None else stream
        buf = self._bufs[self._next]
        found_inf, norm = buf[0:1], buf[1:2].view(torch.float32)
        zeros = buf[2:4].view(torch.int64) if self.log_num_zeros_in_grad else None
        with torch.cuda.stream(s):
            if not self._cleared:
                buf.zero_()
            if inplace_unscale:
                hpo.hpo_unscale_check_inf(self.set, inv, found_inf, s)
                inv = 1.0
                hpo.hpo_grad_global_norm(self.set, inv, norm, None, zeros, stream=s)
            else:
                hpo.hpo_grad_global_norm(self.set, inv, norm, found_inf, zeros, stream=s)
            hpo.hpo_adamw_step(self.set, self.cfg, self.groups, self.n_groups, self.t + 1, inv,
                               self.max_norm, norm, found_inf, s)
            self._host.copy_(buf, non_blocking=True)
            # the next step's buffer starts at 0; enqueued here, the clear runs
            # while the host waits, and the synchronisation below completes it
            # for every stream
            self._bufs[self._next ^ 1].zero_()
        s.synchronize()
        self._cleared = True
        self._cur, self._next = self._next, self._next ^ 1
        found = int(self._host[0]) != 0
        if found:
            return False, None, None
        self.t += 1
        n_zeros = int(self._host[2:4].view(torch.int64)[0]) if self.log_num_zeros_in_grad else None
        return True, float(self._host[1:2].view(torch.float32)[0]), n_zeros


class DeviceAdamW:
    """Steps enqueued with no host synchronisation: the loss scaler, the skip
    decision and the applied-step counter live in device memory
    (hpo_step_device).  The host only tracks which t values the unsynchronised
    steps can have; it reads the state back when that window (EAGER_WINDOW
    steps) is full, or when asked (sync / state).  graph() captures one step
    for replay over a window of HPO_MAX_WINDOW steps."""

    EAGER_WINDOW = 32   # steps between state reads in step(); each call forms this many bias corrections

    def __init__(self, hset: hpo.HpoSet, groups: Sequence[Tuple[float, float]], *, beta1: float = 0.9,
                 beta2: float = 0.999, eps: float = 1e-8, mode: int = hpo.HPO_ADAMW, max_norm: float = 1.0,
                 loss_scale: float = 2.0 ** 32, dynamic: bool = True, growth_interval: int = 1000,
                 hysteresis: int = 2, growth_factor: float = 2.0, backoff_factor: float = 0.5,
                 min_scale: float = 1.0, grad_norm_skip_threshold: float = float("inf"),
                 applied_steps: int = 0, device=None, stream=None):
        self.set = hset
        self.cfg = hpo.make_cfg(beta1, beta2, eps, mode)
        self.groups, self.n_groups = hpo.make_groups(list(groups))
        self.max_norm = float(max_norm)
        self.scfg = hpo.make_scaler_cfg(dynamic, growth_interval, hysteresis, growth_factor, backoff_factor,
                                        min_scale, grad_norm_skip_threshold)
        self.stream = torch.cuda.current_stream() if stream is None else stream
        self.d_state = hpo.new_scaler_state(device)
        hpo.hpo_scaler_state_init(self.d_state, loss_scale, hysteresis, applied_steps, self.stream)
        self.t_first = applied_steps + 1   # smallest t the next step can have
        self.pending = 0                   # steps enqueued since the last read of the state

    @property
    def loss_scale_tensor(self) -> torch.Tensor:
        """The current loss scale as a device fp32 scalar (no sync needed)."""
        return self.d_state.view(torch.float32)[0:1]

    def step(self) -> None:
        if self.pending == self.EAGER_WINDOW:
            self.sync()
        self.pending += 1
        hpo.hpo_step_device(self.set, self.cfg, self.groups, self.n_groups, self.max_norm, self.scfg, self.d_state,
                            self.t_first, self.pending, self.stream)

    def graph(self) -> "torch.cuda.CUDAGraph":
        """One step captured in a HIP graph (torch.cuda.CUDAGraph), to be
        replayed with g.replay() on this optimizer's stream at no launch cost.
        Nothing of the step lives on the host except the bias-correction table
        of the next HPO_MAX_WINDOW values of t, which the graph holds: replay it
        at most that many times, then call sync() and capture again (a replay
        past the window is not applied and sets the state's error flag, which
        sync() reports)."""
        self.sync()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            hpo.hpo_step_device(self.set, self.cfg, self.groups, self.n_groups, self.max_norm, self.scfg,
                                self.d_state, self.t_first, hpo.HPO_MAX_WINDOW)
        return g

    def sync(self) -> hpo.hpo_scaler_state:
        self.stream.synchronize()
        st = hpo.read_scaler_state(self.d_state)
        if st.error:
            raise RuntimeError("a device step fell outside its bias-correction window")
        self.t_first = st.applied_steps + 1
        self.pending = 0
        return st
