"""Per-element error bounds for one optimizer step (test helper).

The acceptance bar is "within rel 1e-6 per step".  A plain |x - x_ref|/|x_ref|
is meaningless where the state is a sum of terms that cancel (any fp32
implementation then errs by a large fraction of a tiny result), so each state
value is bounded by r = 1e-6 times the magnitudes of the terms that produce
it, and that error is carried forward through the later steps of the same
update (bias correction, square root, division, master update):

  a    = |g_unscaled * C|  (+ wd |theta| in the L2 mode)   magnitude of g's terms
  S_m  = b1 |m0| + (1-b1) a            E_m  = r S_m
  S_v  = b2 v0 + (1-b2) a^2            E_v  = r S_v
  E_mh = E_m / bc1 + r |m_hat|         E_vh = E_v / bc2 + r v_hat
  E_sq = min(E_vh / (2 sqrt(v_hat)), sqrt(E_vh)) + r sqrt(v_hat)
  E_d  = E_sq + r d,   d = sqrt(v_hat) + eps
  E_u  = (E_mh + |u| E_d) / max(d - E_d, d/2) + r |u|
  E_th = r (|theta0| + lr (|u| + wd |theta0|)) + lr E_u          (AdamW)
  E_th = r (|theta0| + lr |u|) + lr E_u                            (Adam + L2)

The exact intermediate values are evaluated in binary64 here only to size the
tolerance; the value compared against is always the oracle's.
"""
import numpy as np


def step_error_bounds(th0, m0, v0, G, *, inv, C, do_clip, lr, wd, t, mode,
                      b1=0.9, b2=0.999, eps=1e-8, r=1e-6):
    th0 = th0.astype(np.float64)
    m0 = m0.astype(np.float64)
    v0 = v0.astype(np.float64)
    g = G.astype(np.float64) * float(inv)
    if do_clip:
        g = g * float(C)
    a = np.abs(g)
    if mode == 1:
        a = a + wd * np.abs(th0)
        g = g + wd * th0
    bc1 = 1.0 - b1 ** t
    bc2 = 1.0 - b2 ** t
    m1 = b1 * m0 + (1 - b1) * g
    v1 = b2 * v0 + (1 - b2) * g * g
    mh = m1 / bc1
    vh = v1 / bc2
    sq = np.sqrt(vh)
    d = sq + eps
    u = mh / d
    E_m = r * (b1 * np.abs(m0) + (1 - b1) * a)
    E_v = r * (b2 * v0 + (1 - b2) * a * a)
    E_mh = E_m / bc1 + r * np.abs(mh)
    E_vh = E_v / bc2 + r * vh
    with np.errstate(divide="ignore", invalid="ignore"):
        lin = np.where(sq > 0, E_vh / (2 * np.where(sq > 0, sq, 1.0)), np.inf)
    E_sq = np.minimum(lin, np.sqrt(E_vh)) + r * sq
    E_d = E_sq + r * d
    E_u = (E_mh + np.abs(u) * E_d) / np.maximum(d - E_d, d / 2) + r * np.abs(u)
    if mode == 0:
        S_th = np.abs(th0) + lr * (np.abs(u) + wd * np.abs(th0))
    else:
        S_th = np.abs(th0) + lr * np.abs(u)
    E_th = r * S_th + lr * E_u
    return E_m, E_v, E_th


def check_within(name, got, ref, bound):
    """Assert |got - ref| <= bound elementwise; report the worst offender."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(got - ref)
    ok = err <= bound
    if not np.all(ok):
        i = int(np.argmax(err - bound))
        raise AssertionError(f"{name}: {int((~ok).sum())} of {ok.size} outside the bound; "
                             f"worst i={i} got={got[i]!r} ref={ref[i]!r} err={err[i]:.3e} "
                             f"bound={bound[i]:.3e}")
