"""Tolerances for the Muon GPU parity tests, derived from the oracle's own
arithmetic.

The GPU computes the bf16 Newton-Schulz reading with the same roundings as
oracle.muon.newton_schulz_bf16 (bf16 operands, fp32 elementwise steps); the
only freedom left is the order in which the matrix cores accumulate each
product sum in fp32.  The yardstick is therefore the spread between two valid
evaluations of the same reading that differ only there: exact sums rounded
once (the reference) and the BLAS's fp32 sums.  The GPU must sit within
4x that spread elementwise and 2x in Frobenius norm, plus a floor of one
bf16 rounding of the largest element (2^-8 of max|O|; 2^-9 relative in
norm) for cases whose sums are exact in fp32 either way.
"""
from __future__ import annotations

import numpy as np

K_MAX = 4.0
K_FRO = 2.0


def ns_reference(mu, G32, steps=5, coeffs=None):
    """(reference O, elementwise spread, relative Frobenius spread)."""
    O = mu.newton_schulz_bf16(G32, steps, coeffs)
    O2 = mu.newton_schulz_bf16(G32, steps, coeffs, acc="f32")
    spread = np.abs(O.astype(np.float64) - O2)
    nO = float(np.linalg.norm(O))
    rel = float(np.linalg.norm(spread)) / nO if nO > 0 else 0.0
    return O, spread, rel


def ns_tolerance(O, spread, rel):
    amax = float(np.abs(O).max()) if O.size else 0.0
    return K_MAX * float(spread.max(initial=0.0)) + 2.0 ** -8 * amax, K_FRO * rel + 2.0 ** -9


def check_ns(tag, got, O, spread, rel):
    """Asserts GPU O against the reference; returns the observed figures."""
    tol_max, tol_rel = ns_tolerance(O, spread, rel)
    d = np.abs(got.astype(np.float64) - O)
    nO = float(np.linalg.norm(O))
    grel = float(np.linalg.norm(d)) / nO if nO > 0 else float(np.linalg.norm(d))
    print(f"[ns] {tag}: max|d| {d.max(initial=0.0):.3e} (tol {tol_max:.3e}), rel {grel:.3e} "
          f"(tol {tol_rel:.3e}; spread {rel:.3e})", flush=True)
    assert np.all(np.isfinite(got)), f"{tag}: non-finite output"
    assert d.max(initial=0.0) <= tol_max, f"{tag}: max deviation {d.max():.3e} > {tol_max:.3e}"
    assert grel <= tol_rel, f"{tag}: relative deviation {grel:.3e} > {tol_rel:.3e}"
    return float(d.max(initial=0.0)), grel
