"""Pins of the Muon oracle (CPU only).

Each test checks oracle/muon.py against something other than itself: the
numbers the handbook prints for its Newton-Schulz demonstration, the
singular-value closed form of NS, the polar factor from numpy's SVD, scale
invariance, closed forms of the momentum recursion and of decay-only steps,
and the chained step's shared skip / norm semantics.
"""
import math

import numpy as np
import pytest

from conftest import read_golden

F32 = np.float32


@pytest.fixture(scope="module")
def mu():
    import oracle
    import oracle.muon as m
    oracle.lib()
    return m


def _orthonormal(rng, n, r):
    Q, R = np.linalg.qr(rng.standard_normal((n, r)))
    return Q * np.sign(np.diag(R))  # any orthonormal columns will do


def _svd_matrix(rng, rows, cols, S):
    r = len(S)
    U, V = _orthonormal(rng, rows, r), _orthonormal(rng, cols, r)
    return U, V, (U * S) @ V.T


def _phi_iterate(s, coeffs):
    """Scalar iteration on the singular values ([OPT-INFRA] §5.2): each NS
    step maps sigma to a*sigma + b*sigma^3 + c*sigma^5."""
    s = np.array(s, dtype=np.float64)
    for a, b, c in coeffs:
        s = a * s + b * s ** 3 + c * s ** 5
    return s


# ---------------------------------------------------------------------------
# NS: closed form on singular values
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("rows,cols,rank", [(24, 80, 24), (80, 24, 24), (64, 64, 64), (40, 100, 10),
                                            (100, 40, 7), (1, 33, 1), (33, 1, 1)])
@pytest.mark.parametrize("steps", [0, 1, 3, 5])
def test_ns_equals_polynomial_of_singular_values(mu, rows, cols, rank, steps):
    rng = np.random.default_rng(rows * 1000 + cols + steps)
    S = np.sort(rng.uniform(0.01, 3.0, rank))[::-1]
    U, V, G = _svd_matrix(rng, rows, cols, S)
    sn = S / (math.sqrt(float(np.sum(S ** 2))) + mu.NS_EPS)   # ||G||_F = ||S||_2
    want = (U * _phi_iterate(sn, [mu.NS_SIMPLE] * steps)) @ V.T
    got = mu.newton_schulz_f64(G, steps)
    assert got.shape == (rows, cols)
    assert np.max(np.abs(got - want)) < 1e-11


def test_ns_coefficient_schedule_follows_step_order(mu):
    """A per-step (a, b, c) list is applied in order (the closed form with the
    same list, and a reversed list gives a different result)."""
    rng = np.random.default_rng(3)
    S = np.linspace(1.0, 0.05, 20)
    U, V, G = _svd_matrix(rng, 20, 50, S)
    sched = [(3.4445, -4.7750, 2.0315), (1.875, -1.25, 0.375), (2.0, -1.5, 0.5)]
    sn = S / (math.sqrt(float(np.sum(S ** 2))) + mu.NS_EPS)
    want = (U * _phi_iterate(sn, sched)) @ V.T
    assert np.max(np.abs(mu.newton_schulz_f64(G, 3, sched) - want)) < 1e-12
    other = (U * _phi_iterate(sn, sched[::-1])) @ V.T
    assert np.max(np.abs(other - want)) > 1e-3


def test_convergent_quintic_gives_polar_factor(mu):
    """With (15/8, -10/8, 3/8) the iteration converges to the polar factor
    U V^T, which numpy's SVD gives directly (a library routine)."""
    rng = np.random.default_rng(11)
    for rows, cols in ((30, 70), (70, 30), (40, 40)):
        r = min(rows, cols)
        _, _, G = _svd_matrix(rng, rows, cols, rng.uniform(0.3, 1.0, r))
        U, s, Vt = np.linalg.svd(G, full_matrices=False)
        got = mu.newton_schulz_f64(G, 40, [(15 / 8, -10 / 8, 3 / 8)] * 40)
        assert np.max(np.abs(got - U @ Vt)) < 1e-10


def test_orthogonal_update_rms(mu):
    """[OPT-INFRA] §5.4 (Moonlight Lemma 1): a full-rank semi-orthogonal [A, B]
    matrix has RMS sqrt(1/max(A, B)); times 0.2*sqrt(max(A, B)) it is 0.2."""
    rng = np.random.default_rng(5)
    for rows, cols in ((48, 160), (160, 48), (64, 64)):
        U, _, Vt = np.linalg.svd(rng.standard_normal((rows, cols)), full_matrices=False)
        O = U @ Vt
        rms = math.sqrt(float(np.mean(O ** 2)))
        assert abs(rms - 1 / math.sqrt(max(rows, cols))) < 1e-12
        scale = mu.update_scale(rows, cols)
        assert abs(scale * rms - 0.2) < 1e-12
    # the other two scales of [OPT-INFRA] §14.6 (fan_out = rows, fan_in = cols)
    assert mu.update_scale(4096, 1024, mu.SCALE_SHAPE, 1.0) == 2.0
    assert mu.update_scale(1024, 4096, mu.SCALE_SHAPE, 1.0) == 1.0
    assert mu.update_scale(1024, 4096, mu.SCALE_UNIT_RMS, 1.0) == 0.5


# ---------------------------------------------------------------------------
# NS: the handbook's printed demonstration
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("reading", ["f64", "bf16"])
def test_handbook_newton_schulz_printout(mu, reading):
    """The binary64 method reproduces every printed figure to the printed
    digits.  The page ran NS in fp32; the bf16 reading carries 8-bit-mantissa
    operand rounding on top, so for it each figure may also sit one unit of
    its last printed digit away."""
    gold = read_golden("handbook_muon_newton_schulz.txt")
    rng = np.random.default_rng(2024)
    S = np.logspace(0, -2, 256)
    U, V, G = _svd_matrix(rng, 256, 1024, S)
    exact = reading == "f64"
    ns = mu.newton_schulz_f64 if exact else mu.newton_schulz_bf16
    G_in = G if exact else G.astype(F32)

    def same(x, printed):
        pct = printed.endswith("%")
        txt = printed.rstrip("%")
        digits = len(txt.split(".")[1]) if "." in txt else 0
        val = 100 * x if pct else x
        if exact:
            return f"{val:.{digits}f}" == txt
        return abs(val - float(txt)) <= 1.5 * 10.0 ** -digits

    for steps in (1, 3, 5):
        s = np.linalg.svd(np.asarray(ns(G_in, steps), dtype=np.float64), compute_uv=False)
        share = float(np.mean((s > 0.7) & (s < 1.2)))
        lo, hi, pct = gold[f"ns_steps_{steps}"]
        assert same(s.min(), lo) and same(s.max(), hi) and same(share, pct), (steps, s.min(), s.max(), share)
    X = np.asarray(ns(G_in, 5), dtype=np.float64)
    e0 = float(np.sum(S[:8] ** 2) / np.sum(S ** 2))
    e5 = float(np.linalg.norm(X @ V[:, :8]) ** 2 / np.linalg.norm(X) ** 2)
    p0, p5 = gold["top8_energy"]
    assert same(e0, p0) and same(e5, p5), (e0, e5)
    rms = math.sqrt(float(np.mean(X ** 2)))
    r, inv, scaled = gold["rms"]
    assert same(rms, r) and same(1024 ** -0.5, inv) and same(rms * 0.2 * 1024 ** 0.5, scaled)


def test_ns_scale_invariance(mu):
    """NS divides by the Frobenius norm first, so a positive scale of its
    input changes the output only through the 1e-7 guard: the two momentum
    forms ((1-mu) apart) feed NS the same direction."""
    rng = np.random.default_rng(9)
    G = rng.standard_normal((50, 90))
    for alpha in (0.05, 1.0, 37.0):
        d = np.max(np.abs(mu.newton_schulz_f64(alpha * G, 5) - mu.newton_schulz_f64(G, 5)))
        assert d < 1e-6
    # and the guard matters for a tiny input (it is not dropped)
    tiny = 1e-9 * G / np.linalg.norm(G)
    assert np.max(np.abs(mu.newton_schulz_f64(tiny, 1))) < 0.1
    assert np.all(mu.newton_schulz_f64(np.zeros((5, 7)), 5) == 0)
    assert np.all(mu.newton_schulz_bf16(np.zeros((7, 5), F32), 5) == 0)


def test_bf16_reading_stays_near_the_method(mu):
    """The bf16 reading (8-bit mantissa operands) stays within a few percent
    of the binary64 method on Gaussian gradients; the pages state NS is
    stable in bf16.  Its singular values track the method's."""
    rng = np.random.default_rng(21)
    for rows, cols in ((64, 256), (256, 64), (128, 128), (1, 40)):
        G = rng.standard_normal((rows, cols)).astype(F32)
        O16 = mu.newton_schulz_bf16(G, 5)
        O64 = mu.newton_schulz_f64(G.astype(np.float64), 5)
        rel = np.linalg.norm(O16 - O64) / np.linalg.norm(O64)
        assert rel < 0.03, (rows, cols, rel)
        s16 = np.linalg.svd(O16.astype(np.float64), compute_uv=False)
        s64 = np.linalg.svd(O64, compute_uv=False)
        assert np.max(np.abs(s16 - s64)) < 0.05, (rows, cols)


def test_bf16_input_rounding(mu):
    """X0 of the bf16 reading: fp32 quotient by fp32(norm + eps), rounded to
    bf16, in the wide orientation."""
    rng = np.random.default_rng(4)
    G = rng.standard_normal((30, 10)).astype(F32)
    X0 = mu.ns_input_bf16(G)
    assert X0.shape == (10, 30)
    q = G.astype(np.float64) / (np.linalg.norm(G.astype(np.float64)))
    # within one bf16 ulp (2^-8 relative) plus the fp32 steps
    assert np.all(np.abs(X0.T - q) <= np.abs(q) * 2.0 ** -8 * 1.001 + 1e-30)
    # exactly bf16 values
    bits = X0.view(np.uint32)
    assert np.all(bits & 0xFFFF == 0)


# ---------------------------------------------------------------------------
# momentum and the master update
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("form", [0, 1])
def test_momentum_constant_gradient_closed_form(mu, form):
    """Constant g: the sum form gives M_t = g (1 - mu^t)/(1 - mu); the EMA form
    M_t = g (1 - mu^t)."""
    rng = np.random.default_rng(1)
    g = rng.standard_normal(1000).astype(F32)
    M = np.zeros_like(g)
    m_ = 0.95
    for t in range(1, 41):
        mu.momentum_update(M, g, m_, form, nesterov=False)
        k = (1 - m_ ** t) / (1 - m_) if form == mu.MOMENTUM_SUM else (1 - m_ ** t)
        want = g.astype(np.float64) * k
        assert np.all(np.abs(M - want) <= np.abs(want) * (4 * t) * 2.0 ** -24 + 1e-30), t


def test_nesterov_gradients(mu):
    """Sum form: g~ = g + mu M_new; EMA form: g~ = (1-mu) g + mu M_new; without
    Nesterov g~ is the new buffer.  The EMA form's g~ and M are (1-mu) times
    the sum form's (up to fp32 rounding)."""
    rng = np.random.default_rng(2)
    gs = [rng.standard_normal(500).astype(F32) for _ in range(6)]
    Ms, Me = np.zeros(500, F32), np.zeros(500, F32)
    m_ = 0.9
    for g in gs:
        gts = mu.momentum_update(Ms, g, m_, mu.MOMENTUM_SUM, True)
        gte = mu.momentum_update(Me, g, m_, mu.MOMENTUM_EMA, True)
        assert np.allclose(gte, (1 - m_) * gts.astype(np.float64), rtol=1e-5, atol=1e-6)
        assert np.allclose(Me, (1 - m_) * Ms.astype(np.float64), rtol=1e-5, atol=1e-6)
        assert np.allclose(gts, g + m_ * Ms.astype(np.float64), rtol=1e-6, atol=1e-7)
    M = np.zeros(500, F32)
    assert np.array_equal(mu.momentum_update(M, gs[0], m_, mu.MOMENTUM_SUM, False), M)


def test_two_momentum_forms_give_the_same_update(mu):
    rng = np.random.default_rng(12)
    W0 = rng.standard_normal((48, 96)).astype(F32)
    A = mu.OMatrix.fresh(W0)
    B = mu.OMatrix.fresh(W0)
    for k in range(4):
        G = (1e-3 * rng.standard_normal(W0.shape)).astype(F32)
        cs = mu.MuonCfg(form=mu.MOMENTUM_SUM)
        ce = mu.MuonCfg(form=mu.MOMENTUM_EMA)
        ra = mu.muon_matrix_step(A, G, cs, 0.02, 0.1, 1.0, False, 1.0, "f64")
        rb = mu.muon_matrix_step(B, G, ce, 0.02, 0.1, 1.0, False, 1.0, "f64")
        assert np.max(np.abs(ra["O"] - rb["O"])) < 1e-4
        assert np.max(np.abs(A.W - B.W)) <= 2e-6


def test_zero_grads_only_decay(mu):
    """Zero grads: the momentum stays 0, NS of 0 is 0, and each step multiplies
    the master by fp32(1 - lr*wd) -- k steps give (1 - lr*wd)^k within the
    rounding of k fp32 multiplies, and torch's CPU mul_ gives the same bits."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(6)
    W0 = rng.standard_normal((20, 36)).astype(F32)
    T = mu.OMatrix.fresh(W0)
    ref = torch.from_numpy(W0.copy())
    lr, wd = 0.02, 0.1
    for k in range(1, 26):
        mu.muon_matrix_step(T, np.zeros_like(W0), mu.MuonCfg(), lr, wd, 1.0, False, 1.0, "bf16")
        ref.mul_(1 - lr * wd)
        assert np.all(T.M == 0)
        assert np.array_equal(T.W, ref.numpy())
        want = W0.astype(np.float64) * (1 - lr * wd) ** k
        assert np.all(np.abs(T.W - want) <= np.abs(want) * (k + 1) * 2.0 ** -24)
    # the write-back is the bf16 of the master
    import oracle
    assert np.array_equal(T.p, oracle.bf16_rne(T.W).reshape(T.W.shape))


def test_wd_zero_update_is_scaled_ns(mu):
    """wd = 0, first step from a zero buffer: W1 = W0 - fp32(lr*scale) * O with
    O = NS((1+mu) g) = NS(g) up to the guard, scale 0.2 sqrt(max(A, B))."""
    rng = np.random.default_rng(8)
    W0 = rng.standard_normal((32, 80)).astype(F32)
    G = rng.standard_normal((32, 80)).astype(F32)
    T = mu.OMatrix.fresh(W0)
    mu.muon_matrix_step(T, G, mu.MuonCfg(), 0.01, 0.0, 1.0, False, 1.0, "f64")
    O = mu.newton_schulz_f64(G.astype(np.float64), 5)
    want = W0.astype(np.float64) - 0.01 * 0.2 * math.sqrt(80) * O
    assert np.max(np.abs(T.W - want)) < 1e-6
    assert np.array_equal(T.M, G)


# ---------------------------------------------------------------------------
# the chain: one skip, one norm, one clip
# ---------------------------------------------------------------------------
def _chain(mu, rng, max_norm=1.0):
    import oracle
    adam = [oracle.OTensor.fresh(rng.standard_normal(n).astype(F32), group=g)
            for n, g in ((300, 0), (17, 1))]
    mats = [mu.OMatrix.fresh(rng.standard_normal(s).astype(F32)) for s in ((24, 40), (40, 24))]
    ch = mu.ChainedOracle(adam, oracle.Hyper(), [(1e-3, 0.1), (1e-3, 0.0)], mats, mu.MuonCfg(),
                          [(0.02, 0.1)], max_norm=max_norm)
    return ch


def test_chained_norm_covers_both_groups(mu):
    rng = np.random.default_rng(31)
    ch = _chain(mu, rng, max_norm=0.5)
    ga = [rng.standard_normal(t.theta.size).astype(F32) * F32(0.1) for t in ch.adam]
    gm = [rng.standard_normal(m.W.shape).astype(F32) * F32(0.1) for m in ch.muon]
    r = ch.step(ga, gm)
    want = math.sqrt(math.fsum(float(x) ** 2 for g in ga + gm for x in np.ravel(g)))
    assert r.applied and abs(r.norm64 - want) <= 1e-12 * want
    assert r.clip_applied and abs(r.clip_C - 0.5 / (float(F32(want)) + 1e-6)) < 1e-7
    assert ch.t == 1


def test_chained_inf_in_either_group_skips_everything(mu):
    rng = np.random.default_rng(32)
    for where in ("adam", "muon"):
        ch = _chain(mu, rng)
        ga = [rng.standard_normal(t.theta.size).astype(F32) for t in ch.adam]
        gm = [rng.standard_normal(m.W.shape).astype(F32) for m in ch.muon]
        ch.step(ga, gm)
        before = ([t.copy() for t in ch.adam], [m.copy() for m in ch.muon])
        if where == "adam":
            ga[1][3] = np.inf
        else:
            gm[0][2, 5] = np.nan
        r = ch.step(ga, gm)
        assert not r.applied and r.found_inf and ch.t == 1
        for a, b in zip(before[0], ch.adam):
            assert np.array_equal(a.theta, b.theta) and np.array_equal(a.m, b.m) and np.array_equal(a.p, b.p)
        for a, b in zip(before[1], ch.muon):
            assert np.array_equal(a.W, b.W) and np.array_equal(a.M, b.M) and np.array_equal(a.p, b.p)
