"""CPU oracle for the Muon step chained with AdamW (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  It shares no code with the HIP library;
the product never imports it.

What it computes, and where the pages define it:

  [HANDBOOK] "优化器：AdamW、Muon 与分布式优化器", section on Muon (its three
      numbered steps and the Newton-Schulz listing):
        momentum   M <- mu*M + g
        Nesterov   g~ = g + mu*M          (the listing feeds this to NS)
        NS         X = g~ / (||g~||_F + 1e-7); work on the wide orientation
                   (transpose when rows > cols); repeat: A = X X^T,
                   X <- a X + (b A + c A A) X, with (a, b, c) =
                   (3.4445, -4.7750, 2.0315); transpose back
        update     W <- W (1 - lr*wd);  W <- W - lr * 0.2*sqrt(max(rows, cols)) * O
  [OPT-INFRA] "02 · Optimizer：算法与 infra":
      §1    the EMA (lerp) form of the momentum and of the Nesterov gradient:
            M <- mu*M + (1-mu)*g,  g~ = (1-mu)*g + mu*M  (selectable here);
      §5.2  the same NS iteration, its per-singular-value polynomial
            phi(s) = a s + b s^3 + c s^5, and that it runs in bf16;
      §5.4  Moonlight: decoupled weight decay and the 0.2*sqrt(max(A, B))
            update scale; NS in bf16 on the GPU;
      §5.5  only hidden 2-D matrices use Muon; embeddings, the output head and
            every 1-D parameter stay on AdamW;
      §11.4 a chain of AdamW and Muon shares one found_inf (any one skips
            the whole step), one global norm over both groups of grads and
            one clip coefficient;
      §14.2 routing: 2-D non-embedding params to Muon, the rest to AdamW;
      §14.3 fp16 params with Muon are an error (bf16 and fp32 only);
      §14.6 the alternative update scales (shape_scaling sqrt(max(1, m/n)),
            unit_rms_norm sqrt(m/n)) times an extra factor.
  [FP32-RFC] "AutoModels Trainer 支持 FP32 main_param 优化器" §7.1: the
      mixed-precision wrapper sits outside the AdamW + Muon chain.

Two readings of NS are implemented:
  ``newton_schulz_f64``  the method in binary64 (no rounding anywhere that
                         matters): the exact definition.
  ``newton_schulz_bf16`` the pages' bf16 NS: every matmul operand is a bf16
                         value (X, A and B are rounded to bf16, nearest even),
                         each product sum is formed exactly (binary64 over
                         bf16 operands) and rounded to fp32 once, and the
                         elementwise combinations (a X + ..., b A + c ...) are
                         fp32 with one rounding per operation.  The last step's
                         X is kept in fp32 (it feeds the fp32 master update).
The momentum, the Nesterov gradient and the master update are fp32-literal
(one rounding per written operation, no fused multiply-add): the momentum is
bit-comparable with the GPU, the NS output and the master are not (they go
through bf16 matmuls whose fp32 accumulation order is the hardware's).

Pins (``tests/test_oracle_muon.py``): the closed form U phi^k(S/(|S|+eps)) V^T
for matrices built from a known SVD; every number the handbook prints for its
256 x 1024 worked example; the exactly convergent quintic (15/8, -10/8, 3/8)
against the polar factor U V^T from numpy's SVD; the invariance of NS to a
positive scale of its input (so the two momentum forms give the same update);
decay-only steps on zero grads against closed forms; the bf16 reading within
its error of the binary64 one.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

from . import (ADAMW, Hyper, OTensor, StepResult, any_nonfinite, apply_update, bf16_rne, clip_coeff, count_zeros,
               grad_f32, norm_from_sumsq, sumsq)

# (a, b, c) of the quintic the pages print (the original single set)
NS_SIMPLE = (3.4445, -4.7750, 2.0315)
NS_EPS = 1e-7

MOMENTUM_SUM = 0   # [HANDBOOK]: M <- mu M + g,          g~ = g + mu M
MOMENTUM_EMA = 1   # [OPT-INFRA] §1: M <- mu M + (1-mu) g, g~ = (1-mu) g + mu M

SCALE_SPECTRAL = 0  # sqrt(max(rows, cols)) * extra   (extra 0.2: Moonlight)
SCALE_SHAPE = 1     # sqrt(max(1, rows / cols)) * extra
SCALE_UNIT_RMS = 2  # sqrt(rows / cols) * extra

F32 = np.float32


def _coeffs(steps: int, coeffs) -> List[tuple]:
    if coeffs is None:
        return [NS_SIMPLE] * steps
    coeffs = [tuple(float(x) for x in c) for c in coeffs]
    assert len(coeffs) == steps and all(len(c) == 3 for c in coeffs)
    return coeffs


# --------------------------------------------------------------------------
# Newton-Schulz
# --------------------------------------------------------------------------
def newton_schulz_f64(G: np.ndarray, steps: int = 5, coeffs=None, eps: float = NS_EPS) -> np.ndarray:
    """The NS map in binary64, in the order the pages give it."""
    G = np.asarray(G, dtype=np.float64)
    X = G / (np.linalg.norm(G) + eps)           # Frobenius norm
    transposed = G.shape[0] > G.shape[1]
    if transposed:
        X = X.T
    for a, b, c in _coeffs(steps, coeffs):
        A = X @ X.T
        B = b * A + c * (A @ A)
        X = a * X + B @ X
    return X.T if transposed else X


def _bf16_values(x32: np.ndarray) -> np.ndarray:
    """fp32 array -> the fp32 values of its bf16 (nearest even) roundings."""
    bits = bf16_rne(np.ascontiguousarray(x32, dtype=F32))
    return (bits.astype(np.uint32) << 16).view(F32).reshape(x32.shape)


def _exact_matmul_f32(P: np.ndarray, Q: np.ndarray) -> np.ndarray:
    """Product of two bf16-valued matrices: every product of two bf16 values is
    exact in binary64 and the sums are binary64, then one rounding to fp32."""
    return (P.astype(np.float64) @ Q.astype(np.float64)).astype(F32)


def _f32_matmul(P: np.ndarray, Q: np.ndarray) -> np.ndarray:
    """The same product with fp32 accumulation in the BLAS's own order: a
    second valid evaluation of the bf16 reading, for sizing how much the
    accumulation order alone moves the result."""
    return np.asarray(P, dtype=F32) @ np.asarray(Q, dtype=F32)


def frobenius_norm32(x32: np.ndarray) -> float:
    """fp32(sqrt(sum of squares in binary64)), the squares exact."""
    x = np.asarray(x32, dtype=np.float64).ravel()
    return float(F32(math.sqrt(float(np.dot(x, x)))))


def ns_input_bf16(Gt32: np.ndarray, eps: float = NS_EPS) -> np.ndarray:
    """X0 of the bf16 reading: bf16(fp32(g~ / fp32(norm32 + eps))) in the
    wide orientation (transposed when rows > cols)."""
    Gt32 = np.asarray(Gt32, dtype=F32)
    d = F32(F32(frobenius_norm32(Gt32)) + F32(eps))
    X = (Gt32 / d).astype(F32)
    if Gt32.shape[0] > Gt32.shape[1]:
        X = X.T
    return _bf16_values(np.ascontiguousarray(X))


def newton_schulz_bf16(Gt32: np.ndarray, steps: int = 5, coeffs=None, eps: float = NS_EPS,
                       acc: str = "exact") -> np.ndarray:
    """The pages' bf16 NS (module docstring); returns fp32 O in the input's
    orientation.  acc="exact": each product sum formed exactly and rounded
    once (the reference); acc="f32": summed in fp32 by the BLAS instead."""
    Gt32 = np.asarray(Gt32, dtype=F32)
    transposed = Gt32.shape[0] > Gt32.shape[1]
    X = ns_input_bf16(Gt32, eps)
    cs = _coeffs(steps, coeffs)
    mm = _exact_matmul_f32 if acc == "exact" else _f32_matmul
    for k, (a, b, c) in enumerate(cs):
        a32, b32, c32 = F32(a), F32(b), F32(c)
        A = _bf16_values(mm(X, X.T))
        AA = mm(A, A)
        B = _bf16_values((b32 * A).astype(F32) + (c32 * AA).astype(F32))
        BX = mm(B, X)
        Xn = ((a32 * X).astype(F32) + BX).astype(F32)
        X = Xn if k == len(cs) - 1 else _bf16_values(Xn)
    if steps == 0:
        X = X.astype(F32)
    return np.ascontiguousarray(X.T if transposed else X)


# --------------------------------------------------------------------------
# momentum, scale, master update (fp32-literal)
# --------------------------------------------------------------------------
def momentum_update(M: np.ndarray, g: np.ndarray, mu: float, form: int = MOMENTUM_SUM,
                    nesterov: bool = True) -> np.ndarray:
    """Updates M (fp32) in place and returns g~ (fp32).  mu and 1-mu are formed
    in binary64 and rounded to fp32 once."""
    mu32 = F32(mu)
    if form == MOMENTUM_SUM:
        M[...] = (mu32 * M).astype(F32) + g
        if not nesterov:
            return M.copy()
        return (g + (mu32 * M).astype(F32)).astype(F32)
    omu32 = F32(1.0 - mu)
    M[...] = (mu32 * M).astype(F32) + (omu32 * g).astype(F32)
    if not nesterov:
        return M.copy()
    return ((omu32 * g).astype(F32) + (mu32 * M).astype(F32)).astype(F32)


def update_scale(rows: int, cols: int, mode: int = SCALE_SPECTRAL, extra: float = 0.2) -> float:
    """Binary64 scale of the orthogonalized update ([OPT-INFRA] §5.4, §14.6)."""
    if mode == SCALE_SPECTRAL:
        base = math.sqrt(max(rows, cols))
    elif mode == SCALE_SHAPE:
        base = math.sqrt(max(1.0, rows / cols))
    elif mode == SCALE_UNIT_RMS:
        base = math.sqrt(rows / cols)
    else:
        raise ValueError(mode)
    return base * extra


def master_update(W: np.ndarray, O: np.ndarray, lr: float, wd: float, scale: float) -> None:
    """W <- fp32(W * fp32(1 - lr*wd)); W <- fp32(W - fp32(fp32(lr*scale) * O)),
    the handbook listing's order (decay first, then the scaled update).  The
    two scalars are formed in binary64 and rounded to fp32 once."""
    k1 = F32(1.0 - lr * wd)
    k2 = F32(lr * scale)
    W[...] = (W * k1).astype(F32)
    W[...] = (W - (k2 * O).astype(F32)).astype(F32)


# --------------------------------------------------------------------------
# state and the chained step
# --------------------------------------------------------------------------
@dataclass
class MuonCfg:
    mu: float = 0.95
    nesterov: bool = True
    form: int = MOMENTUM_SUM
    steps: int = 5
    coeffs: Optional[list] = None
    eps: float = NS_EPS
    scale_mode: int = SCALE_SPECTRAL
    extra_scale: float = 0.2


@dataclass
class OMatrix:
    """One Muon matrix: fp32 master W [rows, cols], fp32 momentum, 16-bit param bits."""
    W: np.ndarray
    M: np.ndarray
    p: Optional[np.ndarray] = None
    group: int = 0

    @staticmethod
    def fresh(W: np.ndarray, bf16_param: bool = True, group: int = 0) -> "OMatrix":
        W = np.ascontiguousarray(W, dtype=F32).copy()
        return OMatrix(W, np.zeros_like(W), bf16_rne(W).reshape(W.shape) if bf16_param else None, group)

    def copy(self) -> "OMatrix":
        return OMatrix(self.W.copy(), self.M.copy(), None if self.p is None else self.p.copy(), self.group)


def muon_matrix_step(T: OMatrix, G: np.ndarray, cfg: MuonCfg, lr: float, wd: float, inv_scale: float,
                     do_clip: bool, C: float, ns: str = "bf16") -> dict:
    """One applied Muon step on one matrix: g = fp32(G * inv) (* C when
    clipping), momentum, NS, decay + scaled update, bf16 write-back."""
    g = (np.asarray(G, dtype=F32) * F32(inv_scale)).astype(F32)
    if do_clip:
        g = (g * F32(C)).astype(F32)
    gt = momentum_update(T.M, g, cfg.mu, cfg.form, cfg.nesterov)
    if ns == "bf16":
        O = newton_schulz_bf16(gt, cfg.steps, cfg.coeffs, cfg.eps)
    else:
        O = newton_schulz_f64(gt, cfg.steps, cfg.coeffs, cfg.eps)
    rows, cols = T.W.shape
    scale = update_scale(rows, cols, cfg.scale_mode, cfg.extra_scale)
    master_update(T.W, np.asarray(O, dtype=F32) if ns == "bf16" else O.astype(F32), lr, wd, scale)
    if T.p is not None:
        T.p[...] = bf16_rne(T.W).reshape(T.W.shape)
    return {"g_tilde": gt, "O": O, "scale": scale}


class ChainedOracle:
    """AdamW on the list tensors and Muon on the matrices, under one
    mixed-precision wrapper: one found_inf and one global norm over every
    grad (AdamW tensors first, then the matrices), one clip coefficient, and
    one applied-step counter that a skipped step does not advance."""

    def __init__(self, adam: List[OTensor], hyper: Hyper, adam_groups: Sequence[tuple],
                 muon: List[OMatrix], cfg: MuonCfg, muon_groups: Sequence[tuple], max_norm: float = 0.0,
                 ns: str = "bf16"):
        self.adam, self.hyper, self.adam_groups = adam, hyper, list(adam_groups)
        self.muon, self.cfg, self.muon_groups = muon, cfg, list(muon_groups)
        self.max_norm, self.ns = max_norm, ns
        self.t = 0
        self.last = []

    def step(self, adam_grads: Sequence[np.ndarray], muon_grads: Sequence[np.ndarray],
             inv_scale: float = 1.0) -> StepResult:
        inv32 = float(F32(inv_scale))
        adam_grads = [grad_f32(G) for G in adam_grads]   # bf16 AdamW grads are read as their fp32 values
        allg = list(adam_grads) + list(muon_grads)
        if any(G.size and any_nonfinite(np.ascontiguousarray(G, dtype=F32).ravel()) for G in allg):
            return StepResult(False, True, None, None)
        n2 = 0.0
        for G in allg:
            if G.size:
                n2 = n2 + sumsq(np.ascontiguousarray(G, dtype=F32).ravel(), inv32)
        norm64, norm32 = norm_from_sumsq(n2)
        zeros = 0
        for G in allg:
            if G.size:
                zeros = zeros + count_zeros(np.ascontiguousarray(G, dtype=F32).ravel(), inv32)
        do_clip, C, c64 = clip_coeff(self.max_norm, norm32)
        t = self.t + 1
        if self.adam:
            apply_update(self.adam, [np.ascontiguousarray(G, dtype=F32).ravel() for G in adam_grads],
                         self.hyper, self.adam_groups, t, inv32, do_clip, C, c64, "f32")
        self.last = []
        for T, G in zip(self.muon, muon_grads):
            lr, wd = self.muon_groups[T.group]
            if T.W.size == 0:
                self.last.append(None)
                continue
            self.last.append(muon_matrix_step(T, G, self.cfg, lr, wd, inv32, do_clip, C, self.ns))
        self.t = t
        return StepResult(True, False, norm32, norm64, do_clip, C, num_zeros=zeros)


__all__ = ["NS_SIMPLE", "NS_EPS", "MOMENTUM_SUM", "MOMENTUM_EMA", "SCALE_SPECTRAL", "SCALE_SHAPE",
           "SCALE_UNIT_RMS", "newton_schulz_f64", "newton_schulz_bf16", "ns_input_bf16", "momentum_update",
           "update_scale", "master_update", "MuonCfg", "OMatrix", "muon_matrix_step", "ChainedOracle",
           "frobenius_norm32", "ADAMW"]
