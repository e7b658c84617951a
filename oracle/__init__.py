"""CPU oracle for the mixed-precision AdamW step (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP library
and imports nothing from the product package; the product never imports it.

The arithmetic lives in ``hpo_oracle.c`` (plain C loops, fp32-literal "O32"
and binary64 "O64" variants).  This module loads it through ctypes and
orders the steps of one optimizer step the way the pages order them:

  [OPT-INFRA] "02 · Optimizer：算法与 infra"
    §10.2  the unscale pass sets found_inf; a step with found_inf set returns
           early: no clip, no inner step, the step counter does not advance;
    §11.1  total norm = sqrt(sum of squared grad norms); clip coefficient
           max_norm / (total + 1e-6), applied when below 1; clip_grad <= 0
           turns clipping off;
    §2,§3  the Adam/AdamW update of the fp32 master, m and v;
    §9.2   the master is then written back to the 16-bit model params.
  [FP32-RFC] "支持FP32优化器" §7.2: fp32 params are their own master.
  [OPT-INFRA] §16: the precision-aware optimizer may keep exp_avg /
           exp_avg_sq, the main grads and the master below fp32: bf16 or fp16
           moments and bf16 grads are widened exactly on read; an fp16 master
           under bf16 params is widened, updated in fp32 and stored with the
           fp16 RNE, and the param is the bf16 RNE of the stored master.

``muon.py`` adds the Muon step (momentum, Newton-Schulz, scaled update)
and the AdamW + Muon chain in numpy, with its own pins.

Parity pinning: every function here is checked in ``tests/test_oracle_pins.py``
against values the pages print, closed forms, ``math.fsum``, torch's CPU cast
and torch's CPU Adam/AdamW (a different op order).  NaN bit patterns of the
bf16 write-back are not fixed by the pages ("parity unpinned": NaN is compared
by class only).
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hpo_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

ADAMW = 0
ADAM_L2 = 1

GCC_FLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
             "-fno-fast-math", "-fno-finite-math-only"]


def build(verbose: bool = False) -> str:
    """Compile hpo_oracle.c into liboracle.so with gcc (always recompiles)."""
    cmd = ["gcc", *GCC_FLAGS, _SRC, "-o", _LIB_PATH + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


class _UpdateArgs(ctypes.Structure):
    _fields_ = [
        ("lr", ctypes.c_double),
        ("wd", ctypes.c_double),
        ("beta1", ctypes.c_double),
        ("beta2", ctypes.c_double),
        ("eps", ctypes.c_double),
        ("t", ctypes.c_int64),
        ("mode", ctypes.c_int32),
        ("do_clip", ctypes.c_int32),
        ("inv_scale", ctypes.c_float),
        ("clip_C", ctypes.c_float),
        ("clip_c64", ctypes.c_double),
        ("state_bf16", ctypes.c_int32),
        ("param_fp16", ctypes.c_int32),
    ]


_lib = None


def lib():
    """Load liboracle.so, building it first only when it does not exist."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        L.orc_version.restype = ctypes.c_int32
        L.orc_bf16_rne.argtypes = [ctypes.c_float]
        L.orc_bf16_rne.restype = ctypes.c_uint16
        L.orc_bf16_rne_array.argtypes = [P, P, I64]
        L.orc_bf16_rne_patterns.argtypes = [ctypes.c_uint32, I64, P]
        L.orc_fp16_rne.argtypes = [ctypes.c_float]
        L.orc_fp16_rne.restype = ctypes.c_uint16
        L.orc_fp16_rne_patterns.argtypes = [ctypes.c_uint32, I64, P]
        L.orc_fp16_rne_array.argtypes = [P, P, I64]
        L.orc_any_nonfinite.argtypes = [P, I64]
        L.orc_any_nonfinite.restype = ctypes.c_int32
        L.orc_unscale_inplace.argtypes = [P, I64, ctypes.c_float]
        L.orc_sumsq.argtypes = [P, I64, ctypes.c_float]
        L.orc_sumsq.restype = ctypes.c_double
        L.orc_count_zeros.argtypes = [P, I64, ctypes.c_float]
        L.orc_count_zeros.restype = ctypes.c_int64
        L.orc_clip_coeff.argtypes = [ctypes.c_double, ctypes.c_float,
                                     ctypes.POINTER(ctypes.c_float),
                                     ctypes.POINTER(ctypes.c_double)]
        L.orc_clip_coeff.restype = ctypes.c_int32
        for name in ("orc_update_f32", "orc_update_f64"):
            fn = getattr(L, name)
            fn.argtypes = [I64, P, P, P, P, P, ctypes.POINTER(_UpdateArgs)]
            fn.restype = None
        _lib = L
    return _lib


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be contiguous"
    return ctypes.c_void_p(a.ctypes.data)


def _f32(a: np.ndarray) -> np.ndarray:
    assert a.dtype == np.float32 and a.flags["C_CONTIGUOUS"]
    return a


# --------------------------------------------------------------------------
# elementary pieces
# --------------------------------------------------------------------------
def bf16_rne(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), IEEE RNE (oracle definition)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().orc_bf16_rne_array(_ptr(x), _ptr(out), x.size)
    return out


def bf16_rne_patterns(first: int, count: int) -> np.ndarray:
    out = np.empty(count, dtype=np.uint16)
    lib().orc_bf16_rne_patterns(ctypes.c_uint32(first), count, _ptr(out))
    return out


def fp16_rne_patterns(first: int, count: int) -> np.ndarray:
    out = np.empty(count, dtype=np.uint16)
    lib().orc_fp16_rne_patterns(ctypes.c_uint32(first), count, _ptr(out))
    return out


def fp16_rne(x: np.ndarray) -> np.ndarray:
    """fp32 -> fp16 bit patterns (uint16), IEEE RNE (oracle definition)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().orc_fp16_rne_array(_ptr(x), _ptr(out), x.size)
    return out


def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> fp32, exact: a bf16 value is the fp32
    value whose upper 16 bits are the pattern and whose lower 16 are zero."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def widen_fp16(bits: np.ndarray) -> np.ndarray:
    """fp16 bit patterns (uint16) -> fp32, exact (every binary16 value,
    subnormals and infinities included, is a binary32 value); numpy's half
    conversion does the widening."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return b.view(np.float16).astype(np.float32)


def grad_f32(G: np.ndarray) -> np.ndarray:
    """A main grad as the step reads it: fp32 as stored, or bf16 bit patterns
    (uint16 arrays: the lower-precision main grads of the precision-aware
    optimizer, [OPT-INFRA] §16) widened exactly."""
    if G.dtype == np.uint16:
        return widen_bf16(G)
    return np.ascontiguousarray(G, dtype=np.float32)


def any_nonfinite(G: np.ndarray) -> bool:
    G = _f32(G)
    return bool(lib().orc_any_nonfinite(_ptr(G), G.size))


def unscale_inplace(G: np.ndarray, inv_scale: float) -> None:
    G = _f32(G)
    lib().orc_unscale_inplace(_ptr(G), G.size, ctypes.c_float(inv_scale))


def unscale_inplace_bf16(G: np.ndarray, inv_scale: float) -> None:
    """The in-place unscale of bf16 main grads: each element is widened, taken
    through the fp32 unscale above, and stored back with the bf16 RNE (the
    rounding a bf16 tensor's in-place multiply stores)."""
    assert G.dtype == np.uint16 and G.flags["C_CONTIGUOUS"]
    x = widen_bf16(G).copy()
    unscale_inplace(x, inv_scale)
    G[...] = bf16_rne(x)


def sumsq(G: np.ndarray, inv_scale: float = 1.0) -> float:
    """sum over elements of (double)(fp32(G * inv))^2, sequential binary64."""
    G = _f32(G)
    return float(lib().orc_sumsq(_ptr(G), G.size, ctypes.c_float(inv_scale)))


def count_zeros(G: np.ndarray, inv_scale: float = 1.0) -> int:
    """Number of elements whose unscaled value fp32(G * inv) is zero (either
    sign); the step's num_zeros ([OPT-INFRA] §10.2 return value, §17
    log_num_zeros_in_grad), counted over the same grads as the norm."""
    G = _f32(G)
    return int(lib().orc_count_zeros(_ptr(G), G.size, ctypes.c_float(inv_scale)))


def clip_coeff(max_norm: float, norm32: float):
    """Returns (applies, C as fp32 value, c64)."""
    C = ctypes.c_float(1.0)
    c64 = ctypes.c_double(1.0)
    applies = lib().orc_clip_coeff(ctypes.c_double(max_norm), ctypes.c_float(norm32),
                                   ctypes.byref(C), ctypes.byref(c64))
    return bool(applies), float(np.float32(C.value)), float(c64.value)


def norm_from_sumsq(n2: float):
    """(binary64 norm, fp32 norm): sqrt in binary64, rounded once to fp32."""
    n64 = math.sqrt(n2) if n2 >= 0 else float("nan")
    return n64, float(np.float32(n64))


# --------------------------------------------------------------------------
# one whole optimizer step over a list of tensors
# --------------------------------------------------------------------------
@dataclass
class Hyper:
    """Adam hyperparameters ([OPT-INFRA] §2 defaults; §17 config fields)."""
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    mode: int = ADAMW


@dataclass
class OTensor:
    """One parameter's optimizer-side state, all host numpy arrays."""
    theta: np.ndarray                 # fp32 master (is the param for fp32 params)
    m: np.ndarray                     # exp_avg: fp32, or uint16 bf16 bits (bf16 state)
    v: np.ndarray                     # exp_avg_sq: same dtype as m
    p: Optional[np.ndarray] = None    # uint16 bits of the 16-bit model param, or None (fp32 param)
    group: int = 0
    param_fp16: bool = False          # p holds fp16 bits instead of bf16
    master_fp16: bool = False         # theta holds fp16 bits (uint16) under bf16 params
    moments_fp16: bool = False        # m and v hold fp16 bits (uint16) instead of bf16

    @property
    def state_bf16(self) -> bool:
        return self.m.dtype == np.uint16 and not self.moments_fp16

    @staticmethod
    def fresh(theta: np.ndarray, bf16_param: bool = True, group: int = 0, fp16_param: bool = False,
              state_bf16: bool = False, fp16_master: bool = False, fp16_moments: bool = False) -> "OTensor":
        theta = np.ascontiguousarray(theta, dtype=np.float32).copy()
        sdt = np.uint16 if (state_bf16 or fp16_moments) else np.float32
        if fp16_master:
            # the master is the fp16 image of the draw; the bf16 param that of the master
            assert bf16_param and not fp16_param
            t16 = fp16_rne(theta)
            return OTensor(t16, np.zeros(theta.shape, sdt), np.zeros(theta.shape, sdt),
                           bf16_rne(widen_fp16(t16)), group, False, True, fp16_moments)
        if fp16_param:
            p = fp16_rne(theta)
        else:
            p = bf16_rne(theta) if bf16_param else None
        return OTensor(theta, np.zeros(theta.shape, sdt), np.zeros(theta.shape, sdt), p, group, fp16_param,
                       False, fp16_moments)

    def copy(self) -> "OTensor":
        return OTensor(self.theta.copy(), self.m.copy(), self.v.copy(),
                       None if self.p is None else self.p.copy(), self.group, self.param_fp16,
                       self.master_fp16, self.moments_fp16)


@dataclass
class StepResult:
    applied: bool
    found_inf: bool
    norm32: Optional[float]
    norm64: Optional[float]
    clip_applied: bool = False
    clip_C: float = 1.0
    extra: dict = field(default_factory=dict)
    num_zeros: Optional[int] = None   # zeros of the unscaled grads; None on a non-finite step


def oracle_step(tensors: Sequence[OTensor], grads: Sequence[np.ndarray], hyper: Hyper,
                groups: Sequence[tuple], t: int, inv_scale: float = 1.0,
                max_norm: float = 0.0, variant: str = "f32") -> StepResult:
    """One full mixed-precision step, in place on ``tensors``.

    ``groups[k] = (lr, weight_decay)``; ``t`` is the 1-based count of applied
    steps including this one.  Returns the step's flags and norm; a skipped
    step leaves every tensor bit-identical.
    """
    assert len(tensors) == len(grads)
    grads = [grad_f32(G) for G in grads]
    inv32 = float(np.float32(inv_scale))
    # a1: found_inf over the stored grads
    found = False
    for G in grads:
        if G.size and any_nonfinite(G):
            found = True
    if found:
        return StepResult(False, True, None, None)
    # a2: global norm of the unscaled grads, binary64, tensors in list order
    n2 = 0.0
    for G in grads:
        if G.size:
            n2 = n2 + sumsq(G, inv32)
    norm64, norm32 = norm_from_sumsq(n2)
    # the step's zero count, over the same unscaled grads as the norm
    zeros = 0
    for G in grads:
        if G.size:
            zeros = zeros + count_zeros(G, inv32)
    # a3: clip coefficient from the fp32 norm
    do_clip, C, c64 = clip_coeff(max_norm, norm32)
    # a4 + a5: the update, one call per tensor with its group's lr / wd
    apply_update(tensors, grads, hyper, groups, t, inv32, do_clip, C, c64, variant)
    return StepResult(True, False, norm32, norm64, do_clip, C, num_zeros=zeros)


def apply_update(tensors: Sequence[OTensor], grads: Sequence[np.ndarray], hyper: Hyper,
                 groups: Sequence[tuple], t: int, inv_scale: float, do_clip: bool, C: float,
                 c64: float, variant: str = "f32") -> None:
    """The update + write-back of one applied step, with the clip decision
    already taken from the global norm (used directly when only a sample of a
    very large set is stepped on the host).

    Lower-precision storage ([OPT-INFRA] §16: main grads and main params may
    be kept below fp32): bf16 grads are widened exactly; an fp16 master is
    widened exactly, updated in fp32 like an fp32 master, stored back with the
    fp16 RNE, and the bf16 param is the bf16 RNE of that stored master (the
    param is a copy of the master, [OPT-INFRA] §9.2).  fp16 moments likewise:
    widened exactly, updated in fp32, stored with the fp16 RNE (subnormals
    kept; a v below half the smallest subnormal becomes 0)."""
    L = lib()
    fn = L.orc_update_f32 if variant == "f32" else L.orc_update_f64
    for T, G in zip(tensors, grads):
        if T.theta.size == 0:
            continue
        G = grad_f32(G)
        lr, wd = groups[T.group]
        args = _UpdateArgs(lr=lr, wd=wd, beta1=hyper.beta1, beta2=hyper.beta2,
                           eps=hyper.eps, t=t, mode=hyper.mode, do_clip=int(do_clip),
                           inv_scale=float(np.float32(inv_scale)), clip_C=C, clip_c64=c64,
                           state_bf16=int(T.state_bf16), param_fp16=int(T.param_fp16))
        if T.state_bf16:
            assert variant == "f32", "bf16 moments are defined for the fp32-literal reading only"
            assert T.m.flags["C_CONTIGUOUS"] and T.v.flags["C_CONTIGUOUS"]
            mp, vp = _ptr(T.m), _ptr(T.v)
        elif not T.moments_fp16:
            mp, vp = _ptr(_f32(T.m)), _ptr(_f32(T.v))
        if T.master_fp16 or T.moments_fp16:
            assert variant == "f32", "fp16 storage is defined for the fp32-literal reading only"
            if T.moments_fp16:
                assert T.m.dtype == np.uint16 and T.v.dtype == np.uint16
                m32, v32 = widen_fp16(T.m).copy(), widen_fp16(T.v).copy()
                args.state_bf16 = 0
                mp, vp = _ptr(m32), _ptr(v32)
            if T.master_fp16:
                assert T.p is not None and not T.param_fp16 and T.theta.dtype == np.uint16
                th = widen_fp16(T.theta).copy()
            else:
                th = _f32(T.theta)
            fn(th.size, _ptr(th), mp, vp, _ptr(_f32(G)), None if T.master_fp16 else _ptr(T.p), ctypes.byref(args))
            if T.moments_fp16:
                T.m[...] = fp16_rne(m32)
                T.v[...] = fp16_rne(v32)
            if T.master_fp16:
                T.theta[...] = fp16_rne(th)
                T.p[...] = bf16_rne(widen_fp16(T.theta))
            continue
        fn(T.theta.size, _ptr(_f32(T.theta)), mp, vp,
           _ptr(_f32(np.ascontiguousarray(G))), _ptr(T.p), ctypes.byref(args))


class LossScaler:
    """Loss scale and its update rule, [OPT-INFRA] §10.1.

    Constant scaler (dynamic=False): the scale never changes.  Dynamic
    scaler: a step with non-finite grads resets the growth tracker and takes
    one off the hysteresis tracker; once that tracker is at or below zero the
    scale is backed off to max(scale * backoff, min_scale).  After
    growth_interval clean steps in a row the scale grows by growth_factor and
    both trackers reset.  Defaults are the page's: initial 2^32, growth 2.0,
    backoff 0.5, interval 1000, hysteresis 2, min scale 1.0.  The scale is
    held in fp32."""

    def __init__(self, scale: float = 2.0 ** 32, dynamic: bool = True, growth_factor: float = 2.0,
                 backoff_factor: float = 0.5, growth_interval: int = 1000, hysteresis: int = 2,
                 min_scale: float = 1.0):
        self.scale = np.float32(scale)
        self.dynamic = dynamic
        self.growth_factor = np.float32(growth_factor)
        self.backoff_factor = np.float32(backoff_factor)
        self.growth_interval = growth_interval
        self.hysteresis = hysteresis
        self.min_scale = np.float32(min_scale)
        self.growth_tracker = 0
        self.hysteresis_tracker = hysteresis

    def inv_scale(self) -> float:
        """fp32(1 / scale), the division in binary64."""
        return float(np.float32(1.0 / float(self.scale)))

    def update(self, found_inf: bool) -> None:
        if not self.dynamic:
            return
        if found_inf:
            self.growth_tracker = 0
            self.hysteresis_tracker -= 1
            if self.hysteresis_tracker <= 0:
                self.scale = max(np.float32(self.scale * self.backoff_factor), self.min_scale)
        else:
            self.growth_tracker += 1
            if self.growth_tracker == self.growth_interval:
                self.growth_tracker = 0
                self.hysteresis_tracker = self.hysteresis
                self.scale = np.float32(self.scale * self.growth_factor)


class OracleOptimizer:
    """Keeps the applied-step counter the way the pages do: a skipped step
    does not advance it ([OPT-INFRA] §10.2)."""

    def __init__(self, tensors: List[OTensor], hyper: Hyper, groups: Sequence[tuple],
                 max_norm: float = 0.0, variant: str = "f32"):
        self.tensors = tensors
        self.hyper = hyper
        self.groups = list(groups)
        self.max_norm = max_norm
        self.variant = variant
        self.t = 0  # applied steps so far

    def step(self, grads: Sequence[np.ndarray], inv_scale: float = 1.0) -> StepResult:
        r = oracle_step(self.tensors, grads, self.hyper, self.groups, self.t + 1,
                        inv_scale, self.max_norm, self.variant)
        if r.applied:
            self.t += 1
        return r

    def step_scaled(self, grads: Sequence[np.ndarray], scaler: LossScaler,
                    skip_threshold: float = math.inf) -> StepResult:
        """One step with the loss scaler in the loop, in the pages' order
        ([OPT-INFRA] §10.2, §11.4): unscale with the current scale and check;
        update the scaler with found_inf; a non-finite step returns; otherwise
        take the norm, skip when it exceeds grad_norm_skip_threshold, else
        clip and update."""
        inv = scaler.inv_scale()
        grads = [grad_f32(G) for G in grads]
        found = any(G.size and any_nonfinite(G) for G in grads)
        scaler.update(found)
        if found:
            return StepResult(False, True, None, None)
        n2 = 0.0
        for G in grads:
            if G.size:
                n2 = n2 + sumsq(G, inv)
        norm64, norm32 = norm_from_sumsq(n2)
        zeros = 0
        for G in grads:
            if G.size:
                zeros = zeros + count_zeros(G, inv)
        if norm32 > skip_threshold:
            return StepResult(False, False, norm32, norm64, extra={"threshold_skip": True}, num_zeros=zeros)
        do_clip, C, c64 = clip_coeff(self.max_norm, norm32)
        apply_update(self.tensors, grads, self.hyper, self.groups, self.t + 1, inv, do_clip, C, c64,
                     self.variant)
        self.t += 1
        return StepResult(True, False, norm32, norm64, do_clip, C, num_zeros=zeros)
