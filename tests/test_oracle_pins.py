"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test names the passage it pins.  None of them re-types the oracle's
formula: they use printed values, closed forms, exact summation
(math.fsum), torch's CPU bf16 cast and torch's CPU Adam/AdamW (a different
op order), brute force and invariants.
"""
import math

import numpy as np
import pytest
import torch

from bounds import check_within, step_error_bounds
from conftest import read_golden

ADAMW, ADAM_L2 = 0, 1


def _rand_state(n, seed, t_prev=3):
    """A plausible mid-training state: theta ~ N(0,1), m ~ N(0,1e-3), v ~ (1e-3 N)^2."""
    rng = np.random.default_rng(seed)
    th = rng.standard_normal(n).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    v = ((rng.standard_normal(n) * 1e-3) ** 2).astype(np.float32)
    G = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    return th, m, v, G


def _one_step(orc, th, m, v, G, *, lr, wd, t, mode, variant, inv=1.0, do_clip=False, C=1.0, c64=1.0,
              b1=0.9, b2=0.999, eps=1e-8, bf16=True):
    T = orc.OTensor(th.copy(), m.copy(), v.copy(), orc.bf16_rne(th) if bf16 else None)
    args = orc._UpdateArgs(lr=lr, wd=wd, beta1=b1, beta2=b2, eps=eps, t=t, mode=mode,
                           do_clip=int(do_clip), inv_scale=np.float32(inv), clip_C=C, clip_c64=c64)
    fn = orc.lib().orc_update_f32 if variant == "f32" else orc.lib().orc_update_f64
    import ctypes
    fn(th.size, orc._ptr(T.theta), orc._ptr(T.m), orc._ptr(T.v), orc._ptr(np.ascontiguousarray(G)),
       orc._ptr(T.p), ctypes.byref(args))
    return T


# ---------------------------------------------------------------------------
# a4: the page's two-parameter decay experiment (printed values)
# ---------------------------------------------------------------------------
def _toy_run(orc, mode, steps=1000, variant="f32"):
    T = orc.OTensor.fresh(np.ones(2, np.float32), bf16_param=False)
    opt = orc.OracleOptimizer([T], orc.Hyper(mode=mode), [(1e-2, 0.1)], variant=variant)
    scale = np.array([0.01, 10.0], np.float32)
    for t in range(steps):
        r = opt.step([np.ascontiguousarray(scale * np.float32((-1.0) ** t))])
        assert r.applied
    return T.theta.copy()


@pytest.mark.parametrize("variant", ["f32", "f64"])
def test_toy_matches_printed_values(orc, variant):
    """Page "优化器：AdamW、Muon 与分布式优化器", AdamW section: printed results of the
    decoupled vs L2 experiment, three decimals each."""
    gold = read_golden("handbook_adamw_decay_toy.txt")
    l2 = _toy_run(orc, ADAM_L2, variant=variant)
    aw = _toy_run(orc, ADAMW, variant=variant)
    assert [f"{x:.3f}" for x in l2] == gold["adam_l2"]
    assert [f"{x:.3f}" for x in aw] == gold["adamw"]
    assert f"{(1 - 1e-2 * 0.1) ** 1000:.3f}" == gold["closed_form"][0]
    # the L2 mode's small-grad parameter is driven to (near) zero but stays positive
    assert 0.0 < l2[0] < 5e-4
    # decoupled decay treats both parameters alike
    assert abs(aw[0] - aw[1]) < 1e-5


def test_toy_o32_close_to_o64(orc):
    """Drift between the fp32-literal and binary64 readings after 1000 steps is tiny
    compared to the printed precision."""
    for mode in (ADAMW, ADAM_L2):
        a = _toy_run(orc, mode, variant="f32").astype(np.float64)
        b = _toy_run(orc, mode, variant="f64").astype(np.float64)
        assert np.all(np.abs(a - b) <= 1e-4 * np.maximum(np.abs(b), 1e-3))


# ---------------------------------------------------------------------------
# a4: closed forms
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("variant", ["f32", "f64"])
def test_zero_grad_pure_decay_closed_form(orc, variant):
    """Zero grads, wd > 0: the update term is 0/(0+eps) = 0, so AdamW reduces to
    theta_T = theta_0 (1 - lr wd)^T ("02 · Optimizer：算法与 infra" §3 with g = 0;
    the handbook's 0.368 closed form)."""
    rng = np.random.default_rng(7)
    th0 = rng.standard_normal(1000).astype(np.float32)
    T = orc.OTensor.fresh(th0, bf16_param=True)
    opt = orc.OracleOptimizer([T], orc.Hyper(mode=ADAMW), [(1e-2, 0.1)], variant=variant)
    z = np.zeros(1000, np.float32)
    for _ in range(1000):
        opt.step([z])
    exact = th0.astype(np.float64) * (1 - 1e-3) ** 1000
    # 1000 steps of 3 fp32 roundings each
    assert np.all(np.abs(T.theta - exact) <= 3000 * 2.0 ** -24 * np.abs(exact) + 1e-30)
    assert np.all(T.m == 0) and np.all(T.v == 0)
    ones = orc.OTensor.fresh(np.ones(1, np.float32), bf16_param=False)
    opt1 = orc.OracleOptimizer([ones], orc.Hyper(), [(1e-2, 0.1)], variant=variant)
    for _ in range(1000):
        opt1.step([np.zeros(1, np.float32)])
    assert f"{ones.theta[0]:.3f}" == read_golden("handbook_adamw_decay_toy.txt")["closed_form"][0]


@pytest.mark.parametrize("mode", [ADAMW, ADAM_L2])
def test_zero_grad_no_decay_is_identity(orc, mode):
    """Zero grads with wd = 0 from a fresh state leave master, m, v and the bf16
    param bit-unchanged (every term of the update is exactly zero)."""
    rng = np.random.default_rng(8)
    th0 = rng.standard_normal(4099).astype(np.float32)
    T = orc.OTensor.fresh(th0)
    p0 = T.p.copy()
    opt = orc.OracleOptimizer([T], orc.Hyper(mode=mode), [(1e-3, 0.0)], max_norm=1.0)
    for _ in range(5):
        opt.step([np.zeros(4099, np.float32)])
    assert np.array_equal(T.theta.view(np.uint32), th0.view(np.uint32))
    assert np.array_equal(T.p, p0)
    assert not T.m.any() and not T.v.any()


def test_first_step_closed_form(orc):
    """Step 1 from m = v = 0: m_hat = g and v_hat = g^2 exactly, so
    theta_1 = theta_0 - lr (g / (|g| + eps) + wd theta_0) ("02 · Optimizer：算法与 infra"
    §2 bias correction + §3)."""
    th, m, v, G = _rand_state(5000, 9)
    m[:] = 0
    v[:] = 0
    lr, wd = 1e-3, 0.1
    g = G.astype(np.float64)
    exact = th.astype(np.float64) - lr * (g / (np.abs(g) + 1e-8) + wd * th.astype(np.float64))
    T64 = _one_step(orc, th, m, v, G, lr=lr, wd=wd, t=1, mode=ADAMW, variant="f64")
    T32 = _one_step(orc, th, m, v, G, lr=lr, wd=wd, t=1, mode=ADAMW, variant="f32")
    # O64 rounds only the stored result
    assert np.all(np.abs(T64.theta - exact) <= 2.0 ** -24 * np.abs(exact) * 1.0001)
    S = np.abs(th) + lr * (1 + wd * np.abs(th))
    assert np.all(np.abs(T32.theta - exact) <= 1e-6 * S)
    assert np.allclose(T64.m, (0.1 * g).astype(np.float32), rtol=2 ** -23, atol=0)


def test_constant_grad_closed_form(orc):
    """Constant grad g: m_hat_t = g and v_hat_t = g^2 at every t, so the update is
    s = g/(|g|+eps) and theta_T = (theta_0 + s/wd)(1 - lr wd)^T - s/wd."""
    rng = np.random.default_rng(10)
    th0 = rng.standard_normal(256).astype(np.float32)
    G = (rng.standard_normal(256) * 1e-2).astype(np.float32)
    lr, wd, steps = 1e-3, 0.1, 50
    s = G.astype(np.float64) / (np.abs(G.astype(np.float64)) + 1e-8)
    exact = (th0 + s / wd) * (1 - lr * wd) ** steps - s / wd
    for variant in ("f32", "f64"):
        T = orc.OTensor.fresh(th0)
        opt = orc.OracleOptimizer([T], orc.Hyper(), [(lr, wd)], variant=variant)
        for _ in range(steps):
            opt.step([G])
        scale = np.abs(th0) + lr * steps * (1 + wd * np.abs(th0))
        assert np.all(np.abs(T.theta - exact) <= steps * 8 * 2.0 ** -24 * scale)


def test_betas_zero_reduce_to_sign_like_update(orc):
    """beta1 = beta2 = 0: m = g, v = g^2, both bias corrections are 1 at any t, so
    the update is g/(|g| + eps) regardless of the old state."""
    th, m, v, G = _rand_state(3000, 11)
    lr, wd = 1e-3, 0.1
    g = G.astype(np.float64)
    exact = th - lr * (g / (np.abs(g) + 1e-8) + wd * th.astype(np.float64))
    T = _one_step(orc, th, m, v, G, lr=lr, wd=wd, t=7, mode=ADAMW, variant="f64", b1=0.0, b2=0.0)
    assert np.all(np.abs(T.theta - exact) <= 2.0 ** -24 * np.abs(exact) * 1.0001)
    assert np.array_equal(T.m, G)


def test_l2_with_zero_decay_equals_adamw(orc):
    """Adam+L2 and AdamW differ only in where wd enters; with wd = 0 the two
    modes give bit-identical state ("02 · Optimizer：算法与 infra" §3)."""
    th, m, v, G = _rand_state(10000, 12)
    a = _one_step(orc, th, m, v, G, lr=1e-3, wd=0.0, t=4, mode=ADAMW, variant="f32")
    b = _one_step(orc, th, m, v, G, lr=1e-3, wd=0.0, t=4, mode=ADAM_L2, variant="f32")
    for x, y in ((a.theta, b.theta), (a.m, b.m), (a.v, b.v), (a.p, b.p)):
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8))


def test_fp32_master_is_needed(orc):
    """"02 · Optimizer：算法与 infra" §9.1: an update far below the weight's 16-bit
    spacing is lost when added in 16 bits, so the update runs on an fp32 master.
    theta_0 = 1, update lr*u = 1e-4 per step (u = 1): a bf16-only update never
    moves 1.0 (spacing 2^-8 below 1), while the master drifts and the written-back
    bf16 param flips to 0.99609375 exactly when the master drops below 1 - 2^-9."""
    T = orc.OTensor.fresh(np.ones(1, np.float32))
    opt = orc.OracleOptimizer([T], orc.Hyper(), [(1e-4, 0.0)])
    ps = []
    for _ in range(25):
        opt.step([np.ones(1, np.float32)])
        ps.append(int(T.p[0]))
    assert ps[18] == 0x3F80  # after 19 steps: 0.9981 still rounds to 1.0
    assert ps[19] == 0x3F7F  # after 20 steps: 0.998 < 0.998046875 -> 0.99609375
    # the same update applied to the bf16 value itself is lost every time
    p = torch.tensor([1.0], dtype=torch.bfloat16)
    for _ in range(25):
        p = (p.float() - 1e-4).to(torch.bfloat16)
    assert p.item() == 1.0


# ---------------------------------------------------------------------------
# a4: O32 against the exact shadow and against torch's own AdamW / Adam
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("mode", [ADAMW, ADAM_L2])
@pytest.mark.parametrize("t", [1, 2, 10, 1000])
def test_o32_within_error_bound_of_o64(orc, mode, t):
    """The fp32-literal reading stays within the rel-1e-6 propagated bound of the
    binary64 evaluation of the same formulas, one step from the same state."""
    th, m, v, G = _rand_state(200_000, 13 + t)
    if t == 1:
        m[:] = 0
        v[:] = 0
    lr, wd, inv, C = 1e-3, 0.1, 2.0 ** -16, 0.345
    Gs = (G * np.float32(65536.0)).astype(np.float32)
    kw = dict(lr=lr, wd=wd, t=t, mode=mode, inv=inv, do_clip=True, C=float(np.float32(C)), c64=C)
    a = _one_step(orc, th, m, v, Gs, variant="f32", **kw)
    b = _one_step(orc, th, m, v, Gs, variant="f64", **kw)
    E_m, E_v, E_th = step_error_bounds(th, m, v, Gs, inv=inv, C=C, do_clip=True, lr=lr, wd=wd,
                                       t=t, mode=mode)
    check_within("m", a.m, b.m, E_m)
    check_within("v", a.v, b.v, E_v)
    check_within("theta", a.theta, b.theta, E_th)
    # bf16 params within one bf16 ulp of each other
    assert np.all(np.abs(a.p.astype(np.int32) - b.p.astype(np.int32)) <= 1)


@pytest.mark.parametrize("mode", [ADAMW, ADAM_L2])
def test_o32_matches_torch_cpu_optimizer_per_step(orc, mode):
    """torch.optim.AdamW / Adam on CPU fp32 (prior art with its own op order:
    decay first, lerp for m, addcdiv) agree with O32 per step from the same
    state within the rel-1e-6 propagated bound."""
    n, lr, wd = 50_000, 1e-3, 0.1
    th, m, v, G = _rand_state(n, 21)
    for t in (1, 2, 5, 50):
        if t == 1:
            m0, v0 = np.zeros_like(m), np.zeros_like(v)
        else:
            m0, v0 = m, v
        a = _one_step(orc, th, m0, v0, G, lr=lr, wd=wd, t=t, mode=mode, variant="f32")
        p = torch.nn.Parameter(torch.from_numpy(th.copy()))
        cls = torch.optim.AdamW if mode == ADAMW else torch.optim.Adam
        opt = cls([p], lr=lr, weight_decay=wd, betas=(0.9, 0.999), eps=1e-8, foreach=False)
        p.grad = torch.from_numpy(G.copy())
        opt.state[p] = {"step": torch.tensor(float(t - 1)),
                        "exp_avg": torch.from_numpy(m0.copy()),
                        "exp_avg_sq": torch.from_numpy(v0.copy())}
        opt.step()
        st = opt.state[p]
        # both sides err, so the allowance is twice the single-implementation bound
        E_m, E_v, E_th = step_error_bounds(th, m0, v0, G, inv=1.0, C=1.0, do_clip=False, lr=lr,
                                           wd=wd, t=t, mode=mode)
        check_within("m", a.m, st["exp_avg"].numpy(), 2 * E_m)
        check_within("v", a.v, st["exp_avg_sq"].numpy(), 2 * E_v)
        check_within("theta", a.theta, p.detach().numpy(), 2 * E_th)


# ---------------------------------------------------------------------------
# a1 / a6: non-finite check and the whole-step skip
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("bad", [np.inf, -np.inf, np.nan])
@pytest.mark.parametrize("where", ["head", "middle", "tail"])
def test_nonfinite_check_brute_force(orc, bad, where):
    rng = np.random.default_rng(30)
    G = (rng.standard_normal(10_007) * 1e-3).astype(np.float32)
    G[:4] = [0.0, -0.0, np.float32(1e-45), np.finfo(np.float32).max]  # finite edge values
    assert orc.any_nonfinite(G) is False
    idx = {"head": 0, "middle": 5003, "tail": 10_006}[where]
    G[idx] = bad
    assert orc.any_nonfinite(G) is True
    assert orc.any_nonfinite(G) == (not np.all(np.isfinite(G)))


def test_skip_leaves_state_and_counter_alone(orc):
    """"02 · Optimizer：算法与 infra" §10.2: with found_inf the step returns early,
    runs no clip and no inner step, and the scheduler/step count does not move.
    Sequence [g1, g_bad, g2] must equal [g1, g2]."""
    rng = np.random.default_rng(31)
    th0 = rng.standard_normal(777).astype(np.float32)
    g1 = (rng.standard_normal(777) * 1e-3).astype(np.float32)
    g2 = (rng.standard_normal(777) * 1e-3).astype(np.float32)
    bad = g2.copy()
    bad[776] = np.inf
    A = orc.OTensor.fresh(th0)
    B = orc.OTensor.fresh(th0)
    oa = orc.OracleOptimizer([A], orc.Hyper(), [(1e-3, 0.1)], max_norm=1.0)
    ob = orc.OracleOptimizer([B], orc.Hyper(), [(1e-3, 0.1)], max_norm=1.0)
    oa.step([g1])
    snap = A.copy()
    r = oa.step([bad])
    assert not r.applied and r.found_inf and r.norm32 is None
    for x, y in ((A.theta, snap.theta), (A.m, snap.m), (A.v, snap.v), (A.p, snap.p)):
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8))
    assert oa.t == 1
    oa.step([g2])
    ob.step([g1])
    ob.step([g2])
    assert oa.t == ob.t == 2
    for x, y in ((A.theta, B.theta), (A.m, B.m), (A.v, B.v), (A.p, B.p)):
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8))


# ---------------------------------------------------------------------------
# the step's zero count ("02 · Optimizer：算法与 infra" §10.2 return value,
# §17 log_num_zeros_in_grad): zeros of the unscaled grads
# ---------------------------------------------------------------------------
def _bits(u):
    return np.array([u], dtype=np.uint32).view(np.float32)[0]


# Stored grads around fp32's underflow threshold under an unscale by 2^-16,
# each with whether fp32(G * 2^-16) is zero.  Round to nearest even: a product
# below 2^-150 (half the smallest subnormal 2^-149) rounds to zero, exactly
# 2^-150 is a tie that goes to the even neighbour 0, anything above rounds to
# 2^-149.  Decided by hand from IEEE 754, not computed.
_UNDERFLOW_CASES = [
    (0.0, True),                                   # +0
    (-0.0, True),                                  # -0 compares equal to 0
    (_bits(0x00000001), True),                     # 2^-149 -> 2^-165
    (-_bits(0x00000001), True),
    (_bits(0x00000200), True),                     # 2^-140 -> 2^-156
    (_bits(0x00008000), True),                     # 2^-134 -> 2^-150, the tie: even -> 0
    (-_bits(0x00008000), True),
    (_bits(0x00008001), False),                    # 2^-134 + 2^-149 -> just above 2^-150 -> 2^-149
    (_bits(0x0000C000), False),                    # 1.5 * 2^-134 -> 0.75 * 2^-149 -> 2^-149
    (_bits(0x00010000), False),                    # 2^-133 -> 2^-149 exactly
    (_bits(0x00800000), False),                    # 2^-126 (smallest normal) -> 2^-142, subnormal
    (np.float32(1e-3), False),
    (np.float32(-65536.0), False),
    (np.float32(np.nan), False),                   # NaN is not zero
    (np.float32(np.inf), False),
]


def test_zero_count_known_underflow_cases(orc):
    """Each case alone and all together: the count under 2^-16 is the number
    of cases marked zero; under no scale only the two signed zeros count.
    A count taken on the stored (scaled) grads, one that counts only +0's bit
    pattern, or one that treats NaN as zero fails here."""
    G = np.array([g for g, _ in _UNDERFLOW_CASES], dtype=np.float32)
    want = sum(1 for _, z in _UNDERFLOW_CASES if z)
    assert want == 7
    assert orc.count_zeros(G, 2.0 ** -16) == want
    assert orc.count_zeros(G, 1.0) == 2
    for g, z in _UNDERFLOW_CASES:
        assert orc.count_zeros(np.array([g], dtype=np.float32), 2.0 ** -16) == int(z), hex(
            int(np.array([g], dtype=np.float32).view(np.uint32)[0]))


def test_zero_count_against_numpy_products(orc):
    """Brute force with numpy's own fp32 multiply and compare, on grads with
    planted zeros of both signs and subnormals, at several scales; also
    permutation invariance and additivity over a split."""
    rng = np.random.default_rng(35)
    n = 200_003
    G = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    idx = rng.choice(n, 5000, replace=False)
    G[idx[:1000]] = 0.0
    G[idx[1000:2000]] = -0.0
    G[idx[2000:5000]] = (rng.integers(1, 1 << 20, 3000).astype(np.uint32)).view(np.float32)  # subnormals
    for inv in (1.0, 2.0 ** -16, 2.0 ** -24, 1.0 / 3.0):
        inv32 = np.float32(inv)
        prod = G * inv32
        assert prod.dtype == np.float32
        want = int(n - np.count_nonzero(prod))
        got = orc.count_zeros(G, inv)
        assert got == want, (inv, got, want)
        assert orc.count_zeros(G[rng.permutation(n)], inv) == got
        assert orc.count_zeros(G[:77_777], inv) + orc.count_zeros(G[77_777:], inv) == got
    assert orc.count_zeros(G, 1.0) == 2000


def test_step_returns_zero_count_and_none_on_skip(orc):
    """The applied step returns (success, grad_norm, num_zeros) and a skipped
    one (False, None, None) ("02 · Optimizer：算法与 infra" §10.2): the oracle's
    result carries the count over all tensors, and None on a non-finite step."""
    rng = np.random.default_rng(36)
    th = [rng.standard_normal(n).astype(np.float32) for n in (1000, 37, 4096)]
    G = [(rng.standard_normal(x.size) * 1e-3 + 1e-2).astype(np.float32) for x in th]  # no accidental zeros
    G[0][[3, 500, 999]] = [0.0, -0.0, 0.0]
    G[2][:40] = 0.0
    G[1][5] = _bits(0x00000003)   # 3 * 2^-149: not zero at S = 1, zero after * 2^-16
    O = orc.OracleOptimizer([orc.OTensor.fresh(x) for x in th], orc.Hyper(), [(1e-3, 0.1)], max_norm=1.0)
    assert all(np.all(g != 0) for g in (np.delete(G[0], [3, 500, 999]), np.delete(G[1], 5), G[2][40:]))
    r = O.step(G)
    assert r.applied and r.num_zeros == 43
    scaled = [g * np.float32(65536.0) for g in G]
    scaled[1][5] = _bits(0x00000003)   # stored 3 * 2^-149 underflows under the unscale
    r = O.step(scaled, inv_scale=2.0 ** -16)
    assert r.applied and r.num_zeros == 44
    bad = [g.copy() for g in G]
    bad[1][0] = np.nan
    r = O.step(bad)
    assert not r.applied and r.num_zeros is None and r.norm32 is None


def test_zero_count_is_taken_before_the_clip(orc):
    """R40: the count is of the unscaled grads whose norm is taken, before the
    clip.  One grad of 1e15 makes the clip coefficient about 1e-15, which
    would round the ten stored subnormals (2^-130) to zero if they were
    counted after it; only the three true zeros count."""
    th = np.linspace(-1, 1, 14).astype(np.float32)
    G = np.full(14, _bits(0x00010000), dtype=np.float32)   # 2^-133 each
    G[0] = np.float32(1e15)
    G[[5, 9, 13]] = [0.0, -0.0, 0.0]
    assert orc.count_zeros(G, 1.0) == 3
    _, C, _ = orc.clip_coeff(1.0, np.float32(1e15))
    assert np.count_nonzero(G[1:] * np.float32(C)) == 0   # after the clip they would all be zero
    O = orc.OracleOptimizer([orc.OTensor.fresh(th)], orc.Hyper(), [(1e-3, 0.1)], max_norm=1.0)
    r = O.step([G])
    assert r.applied and r.clip_applied and r.num_zeros == 3


def test_unscale_power_of_two_is_exact(orc):
    """Multiplying by 2^-16 is exact for normal fp32 values, so the in-place
    unscale recovers the unscaled grads bit for bit."""
    rng = np.random.default_rng(32)
    g = (rng.standard_normal(100_000) * 1e-3).astype(np.float32)
    G = (g * np.float32(65536.0)).astype(np.float32)
    orc.unscale_inplace(G, 2.0 ** -16)
    assert np.array_equal(G.view(np.uint32), g.view(np.uint32))


# ---------------------------------------------------------------------------
# a2 / a3: global norm and clip
# ---------------------------------------------------------------------------
def test_sumsq_against_fsum(orc):
    """"02 · Optimizer：算法与 infra" §11.1 total norm; math.fsum gives the correctly
    rounded exact sum of the (exact) binary64 squares."""
    rng = np.random.default_rng(40)
    for n, std in ((1, 1.0), (1000, 1e-3), (1_000_003, 1e-2)):
        g = (rng.standard_normal(n) * std).astype(np.float32)
        exact = math.fsum(float(x) * float(x) for x in g.astype(np.float64))
        got = orc.sumsq(g)
        assert abs(got - exact) <= n * 2.0 ** -53 * exact


def test_norm_closed_forms_and_permutation(orc):
    c = np.float32(2.0 ** -7)
    g = np.full(4 ** 8, c, np.float32)  # N = 65536 -> norm = c * 256 exactly
    assert orc.norm_from_sumsq(orc.sumsq(g))[0] == float(c) * 256
    one = np.zeros(12345, np.float32)
    one[4321] = np.float32(-3.25)
    assert orc.norm_from_sumsq(orc.sumsq(one))[0] == 3.25
    rng = np.random.default_rng(41)
    x = (rng.standard_normal(500_000) * 1e-3).astype(np.float32)
    a, b = orc.sumsq(x), orc.sumsq(x[rng.permutation(x.size)].copy())
    assert abs(a - b) <= x.size * 2.0 ** -53 * a
    # unscale by 2^-16 inside the sum equals summing the unscaled copy, exactly
    xs = (x * np.float32(65536.0)).astype(np.float32)
    assert orc.sumsq(xs, 2.0 ** -16) == orc.sumsq(x)


def test_clip_coefficient(orc):
    """c = max_norm / (norm + 1e-6), applied iff c < 1; max_norm <= 0 disables."""
    applies, C, c64 = orc.clip_coeff(1.0, 2.9)
    assert applies and c64 == 1.0 / (float(np.float32(2.9)) + 1e-6) and C == float(np.float32(c64))
    # post-clip norm: C * norm == max_norm * norm / (norm + 1e-6) up to fp32 rounding
    assert abs(C * float(np.float32(2.9)) - 2.9 / (2.9 + 1e-6)) < 1e-6
    assert orc.clip_coeff(1.0, 0.5)[0] is False            # below max_norm: untouched
    # norm == max_norm: c = 1 / (1 + 1e-6) < 1, so the (tiny) clip applies
    applies, C1, _ = orc.clip_coeff(1.0, 1.0)
    assert applies and C1 == float(np.float32(1.0 / (1.0 + 1e-6)))
    assert orc.clip_coeff(0.0, 100.0)[0] is False
    assert orc.clip_coeff(-1.0, 100.0)[0] is False


def test_clip_boundary_strict(orc):
    """No clip exactly when norm + 1e-6 <= max_norm (strict '< 1' comparison)."""
    for norm in (0.999, 0.999998, 0.999999, 1.0, 1.5):
        n32 = float(np.float32(norm))
        applies = orc.clip_coeff(1.0, n32)[0]
        assert applies == (1.0 / (n32 + 1e-6) < 1.0)


def test_full_step_clips_to_max_norm(orc):
    """After clipping, the norm of the grads that enter the update is max_norm up
    to the 1e-6 guard (checked through m_1 = (1 - b1) g on step 1)."""
    rng = np.random.default_rng(42)
    G = (rng.standard_normal(300_000) * 1e-2).astype(np.float32)
    T = orc.OTensor.fresh(rng.standard_normal(300_000).astype(np.float32))
    r = orc.oracle_step([T], [G], orc.Hyper(), [(1e-3, 0.1)], 1, 1.0, 1.0, "f64")
    assert r.clip_applied and r.norm64 > 1
    g_used = T.m.astype(np.float64) / 0.1
    assert abs(np.sqrt(np.sum(g_used ** 2)) - r.norm64 / (r.norm64 + 1e-6)) < 1e-5


# ---------------------------------------------------------------------------
# a5: bf16 write-back
# ---------------------------------------------------------------------------
def test_bf16_rne_known_values(orc):
    """IEEE RNE cases: ties to even, subnormals kept, overflow to inf, NaN quiet."""
    cases = {0x3F808000: 0x3F80, 0x3F818000: 0x3F82, 0x3F808001: 0x3F81, 0x00018000: 0x0002,
             0x7F7FFFFF: 0x7F80, 0xFF7FFFFF: 0xFF80, 0x7F800000: 0x7F80, 0x80000000: 0x8000,
             0x00000001: 0x0000, 0x00008000: 0x0000, 0x00008001: 0x0001, 0x7F7F7FFF: 0x7F7F}
    for bits, want in cases.items():
        x = np.array([bits], np.uint32).view(np.float32)[0]
        assert int(orc.bf16_rne(np.array([x]))[0]) == want, hex(bits)
    nan = np.array([0x7FA00001, 0xFFC00000], np.uint32).view(np.float32)
    assert [int(b) for b in orc.bf16_rne(nan)] == [0x7FC0, 0xFFC0]


def test_bf16_rne_exhaustive_against_torch_cast(orc):
    """All 2^32 fp32 bit patterns against torch's CPU fp32->bf16 cast (a library
    routine).  Non-NaN results must be bit-equal; NaNs are compared by class
    (the pages do not fix NaN encodings)."""
    step = 1 << 28
    base = np.arange(step, dtype=np.uint32)
    for first in range(0, 1 << 32, step):
        bits = base + np.uint32(first)
        ours = orc.bf16_rne_patterns(first, step)
        ref = torch.from_numpy(bits.view(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        isnan = ((bits & 0x7FFFFFFF) > 0x7F800000)
        assert np.array_equal(ours[~isnan], ref[~isnan]), hex(first)
        on = ours[isnan]
        assert np.all(((on & 0x7FFF) > 0x7F80))


# ---------------------------------------------------------------------------
# ledgers
# ---------------------------------------------------------------------------
def test_state_bytes_per_param(orc):
    """Page "优化器：AdamW、Muon 与分布式优化器", state-size output: AdamW holds 8 bytes of
    optimizer state per parameter at 8.4M parameters (two fp32 moments)."""
    gold = read_golden("handbook_optimizer_state_bytes.txt")
    n = 4096 * 1024 + 1024 * 4096
    Ts = [orc.OTensor.fresh(np.zeros(4096 * 1024, np.float32)), orc.OTensor.fresh(np.zeros(1024 * 4096, np.float32))]
    state = sum(T.m.nbytes + T.v.nbytes for T in Ts)
    assert f"{n / 1e6:.1f}" == gold["params_millions"][0]
    assert state / n == int(gold["adamw_state_bytes_per_param"][0])


def test_memory_ledgers():
    gold = read_golden("memory_ledgers.txt")
    bf16_w, bf16_g, fp32 = 2, 2, 4
    assert bf16_w + bf16_g + 3 * fp32 == int(gold["handbook_adamw_bytes_per_param"][0])
    assert f"{70e9 * 16 / 1e12:.1f}" == gold["handbook_70b_total_tb"][0]
    # the layout this library steps: bf16 param + fp32 grad + fp32 master/m/v
    assert bf16_w + fp32 + 3 * fp32 == int(gold["megatron_fp32_grad_bytes_per_param"][0])


# ---------------------------------------------------------------------------
# loss scaler ("02 · Optimizer：算法与 infra" §10.1)
# ---------------------------------------------------------------------------
def test_scaler_defaults_and_single_spike_tolerance(orc):
    """The page's defaults (initial 2^32, growth x2, backoff x0.5, window 1000,
    hysteresis 2) and its point that a single inf does not lower the scale."""
    sc = orc.LossScaler()
    assert float(sc.scale) == 2.0 ** 32 and sc.growth_interval == 1000 and sc.hysteresis == 2
    sc.update(True)
    assert float(sc.scale) == 2.0 ** 32           # one spike is tolerated
    sc.update(False)
    sc.update(True)
    assert float(sc.scale) == 2.0 ** 31           # the second one (no growth in between) backs off
    sc.update(True)
    assert float(sc.scale) == 2.0 ** 30           # and every further one, until a growth resets
    for _ in range(999):
        sc.update(False)
    assert float(sc.scale) == 2.0 ** 30
    sc.update(False)                               # 1000 clean steps in a row: grow
    assert float(sc.scale) == 2.0 ** 31 and sc.hysteresis_tracker == 2 and sc.growth_tracker == 0
    sc.update(True)
    assert float(sc.scale) == 2.0 ** 31           # hysteresis restored by the growth


def test_scaler_floor_and_constant(orc):
    sc = orc.LossScaler(scale=4.0, hysteresis=1, min_scale=1.0)
    for _ in range(5):
        sc.update(True)
    assert float(sc.scale) == 1.0
    c = orc.LossScaler(scale=65536.0, dynamic=False)
    for f in (True, True, False) * 400:
        c.update(f)
    assert float(c.scale) == 65536.0 and c.inv_scale() == 2.0 ** -16


def test_scaler_matches_torch_amp_update_at_hysteresis_one(orc):
    """With hysteresis 1 and no floor the rule is torch's own GradScaler
    update (torch._amp_update_scale_, a library routine) step for step."""
    rng = np.random.default_rng(50)
    flags = rng.random(5000) < 0.03
    sc = orc.LossScaler(scale=2.0 ** 20, hysteresis=1, growth_interval=37, min_scale=2.0 ** -126)
    s_t = torch.tensor([2.0 ** 20])
    g_t = torch.tensor([0], dtype=torch.int32)
    for f in flags:
        sc.update(bool(f))
        torch._amp_update_scale_(s_t, g_t, torch.tensor([1.0 if f else 0.0]), 2.0, 0.5, 37)
        assert float(sc.scale) == float(s_t[0]) and sc.growth_tracker == int(g_t[0])


def test_scaled_step_skips_and_counts(orc):
    """With the scaler in the loop: a non-finite step is skipped and backs off
    (after hysteresis), a step over grad_norm_skip_threshold is skipped but
    counts as clean, and t only counts applied steps."""
    rng = np.random.default_rng(51)
    th0 = rng.standard_normal(1000).astype(np.float32)
    T = orc.OTensor.fresh(th0)
    O = orc.OracleOptimizer([T], orc.Hyper(), [(1e-3, 0.1)], max_norm=1.0)
    sc = orc.LossScaler(scale=1024.0, hysteresis=1, growth_interval=2)
    g = (rng.standard_normal(1000) * 1e-3).astype(np.float32)
    r = O.step_scaled([g * np.float32(1024.0)], sc)
    assert r.applied and O.t == 1
    bad = g * np.float32(1024.0)
    bad[5] = np.nan
    r = O.step_scaled([bad], sc, 10.0)
    assert not r.applied and r.found_inf and O.t == 1 and float(sc.scale) == 512.0
    big = (g * np.float32(1e5) * np.float32(512.0)).astype(np.float32)   # unscaled norm ~3, over 1.0
    r = O.step_scaled([big], sc, skip_threshold=1.0)
    assert not r.applied and not r.found_inf and O.t == 1 and r.extra["threshold_skip"]
    r = O.step_scaled([g * np.float32(512.0)], sc, skip_threshold=1.0)
    assert r.applied and O.t == 2 and float(sc.scale) == 1024.0  # two clean steps: grown


# ---------------------------------------------------------------------------
# reduced-precision variants ("02 · Optimizer：算法与 infra" §9.2 fp16/bf16 model
# params, §16 lower-precision exp_avg / exp_avg_sq)
# ---------------------------------------------------------------------------
def test_fp16_rne_exhaustive_against_torch_cast(orc):
    """All 2^32 fp32 patterns against torch's CPU float32 -> float16 cast (a
    library routine, IEEE round to nearest even with subnormals).  NaNs by
    class."""
    step = 1 << 28
    base = np.arange(step, dtype=np.uint32)
    for first in range(0, 1 << 32, step):
        bits = base + np.uint32(first)
        ours = orc.fp16_rne_patterns(first, step)
        ref = torch.from_numpy(bits.view(np.float32)).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
        isnan = (bits & 0x7FFFFFFF) > 0x7F800000
        assert np.array_equal(ours[~isnan], ref[~isnan]), hex(first)
        assert np.all((ours[isnan] & 0x7FFF) > 0x7C00)


def test_fp16_rne_against_numpy_cast_stratified(orc):
    """A second library (numpy's float32 -> float16) on every exponent and sign
    with random mantissas plus every tie pattern of the dropped bits."""
    rng = np.random.default_rng(61)
    se = np.repeat(np.arange(512, dtype=np.uint32) << 23, 16384)
    mant = rng.integers(0, 1 << 23, size=se.size, dtype=np.uint32)
    ties = []
    for drop in range(13, 24):  # a dropped-bits field of width `drop` exactly at half, +-1
        for d in (-1, 0, 1):
            ties.append(((1 << (drop - 1)) + d) & 0x7FFFFF)
    tie_bits = (np.arange(512, dtype=np.uint32)[:, None] << 23 | np.array(ties, np.uint32)[None, :]).ravel()
    odd = (tie_bits | (1 << 13)) & 0xFFFFFFFF  # same, with an odd kept bit
    bits = np.concatenate([se | mant, tie_bits, odd.astype(np.uint32)])
    x = bits.view(np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    ours = orc.fp16_rne(x)
    isnan = (bits & 0x7FFFFFFF) > 0x7F800000
    assert np.array_equal(ours[~isnan], ref[~isnan])


@pytest.mark.parametrize("mode", [ADAMW, ADAM_L2])
def test_bf16_moments_are_the_fp32_update_rounded(orc, mode):
    """With moments held in bf16, one step equals the fp32-moment step run from
    the same (bf16-representable) moments, followed by the bf16 rounding of the
    new moments (torch's CPU cast), with the master untouched by that
    rounding; the fp16 param is the fp16 rounding of the master (numpy cast)."""
    th, m, v, G = _rand_state(100_003, 60)
    m16 = torch.from_numpy(m).to(torch.bfloat16)
    v16 = torch.from_numpy(v).to(torch.bfloat16)
    m_b = m16.view(torch.int16).numpy().view(np.uint16).copy()
    v_b = v16.view(torch.int16).numpy().view(np.uint16).copy()
    m_f = m16.float().numpy().copy()
    v_f = v16.float().numpy().copy()
    import ctypes
    for t in (1, 7):
        a = orc.OTensor(th.copy(), m_b.copy(), v_b.copy(), np.zeros(th.size, np.uint16), 0, param_fp16=True)
        b = orc.OTensor(th.copy(), m_f.copy(), v_f.copy(), np.zeros(th.size, np.uint16), 0, param_fp16=False)
        for T in (a, b):
            orc.apply_update([T], [G], orc.Hyper(mode=mode), [(1e-3, 0.1)], t, 1.0, True, 0.5, 0.5)
        assert np.array_equal(a.theta.view(np.uint32), b.theta.view(np.uint32))
        assert np.array_equal(a.m, torch.from_numpy(b.m).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
        assert np.array_equal(a.v, torch.from_numpy(b.v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
        with np.errstate(over="ignore"):
            assert np.array_equal(a.p, a.theta.astype(np.float16).view(np.uint16))


# ---------------------------------------------------------------------------
# lower-precision main grads and master ([OPT-INFRA] §16: main_grads /
# main_params may be stored below fp32)
# ---------------------------------------------------------------------------
def _torch_bits(t):
    return t.view(torch.int16).numpy().view(np.uint16)


def test_widening_is_exact_for_every_pattern(orc):
    """bf16 and fp16 -> fp32 over all 65536 patterns equal torch's CPU casts,
    and the RNE store of a widened value gives the pattern back (NaN by class)."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    tb = torch.from_numpy(bits.view(np.int16))
    for widen, tdt, rne in ((orc.widen_bf16, torch.bfloat16, orc.bf16_rne),
                            (orc.widen_fp16, torch.float16, orc.fp16_rne)):
        ours = widen(bits)
        ref = tb.view(tdt).float().numpy()
        isnan = np.isnan(ref)
        assert np.array_equal(np.isnan(ours), isnan)
        assert np.array_equal(ours[~isnan].view(np.uint32), ref[~isnan].view(np.uint32))
        assert np.array_equal(rne(ours)[~isnan], bits[~isnan])


# (lr, sign of g) -> (fp16 master bits, bf16 param bits) after one step from
# a master of 1.0: the first AdamW step with eps = 0 and wd = 0 moves the
# master by -lr * sign(g) (m_hat = g, v_hat = g^2), so the fp32 result is
# 1 -+ lr up to a few fp32 ulps, and the stores round that:
#   1 - 2^-9   is an fp16 value (ulp 2^-11 below 1); in bf16 (ulp 2^-8 below
#              1) it is the midpoint of 1 - 2^-8 and 1, and the tie goes to
#              the even pattern, 1.0;
#   1 - 3*2^-13 is 2^-13 from 1 - 2^-11 and 3*2^-13 from 1: fp16 1 - 2^-11;
#   1 -+ 2^-13 is below half an fp16 ulp on either side of 1: the update is
#              lost and the master stays 1.0;
#   1 + 2^-9   is an fp16 value (ulp 2^-10 above 1); bf16 rounds it to 1.0;
#   1 + 3*2^-13 is 3*2^-13 from 1 and 5*2^-13 from 1 + 2^-10: fp16 1.0.
_FP16_MASTER_CASES = [
    (2.0 ** -9, +1, 1.0 - 2.0 ** -9),
    (3 * 2.0 ** -13, +1, 1.0 - 2.0 ** -11),
    (2.0 ** -13, +1, 1.0),
    (2.0 ** -9, -1, 1.0 + 2.0 ** -9),
    (3 * 2.0 ** -13, -1, 1.0),
    (2.0 ** -13, -1, 1.0),
]


@pytest.mark.parametrize("lr,sign,master", _FP16_MASTER_CASES)
def test_fp16_master_first_step_closed_form(orc, lr, sign, master):
    g = np.full(257, sign * 3.0e-3, np.float32)
    T = orc.OTensor.fresh(np.ones(257, np.float32), fp16_master=True)
    assert np.all(T.theta == 0x3C00) and np.all(T.p == 0x3F80)
    opt = orc.OracleOptimizer([T], orc.Hyper(eps=0.0), [(lr, 0.0)])
    assert opt.step([g]).applied
    # every expected master is an fp16 value, so its cast is exact
    want = np.float16(master).view(np.uint16)
    assert float(np.float16(master)) == master
    assert np.all(T.theta == want), hex(int(T.theta[0]))
    assert np.all(T.p == 0x3F80)


@pytest.mark.parametrize("mode", [ADAMW, ADAM_L2])
def test_fp16_master_is_the_fp32_update_rounded(orc, mode):
    """An fp16 master steps exactly as an fp32 master holding the same
    (widened) value, followed by the fp16 rounding of the new master (torch's
    CPU cast); the bf16 param is torch's bf16 cast of the stored fp16 master."""
    th, m, v, G = _rand_state(100_003, 61)
    th16 = torch.from_numpy(th).to(torch.float16)
    t_b = _torch_bits(th16).copy()
    t_f = th16.float().numpy().copy()
    for t in (1, 9):
        a = orc.OTensor(t_b.copy(), m.copy(), v.copy(), np.zeros(th.size, np.uint16), 0, master_fp16=True)
        b = orc.OTensor(t_f.copy(), m.copy(), v.copy(), None, 0)
        for T in (a, b):
            orc.apply_update([T], [G], orc.Hyper(mode=mode), [(1e-3, 0.1)], t, 1.0, True, 0.5, 0.5)
        assert np.array_equal(a.m.view(np.uint32), b.m.view(np.uint32))
        assert np.array_equal(a.v.view(np.uint32), b.v.view(np.uint32))
        want16 = torch.from_numpy(b.theta).to(torch.float16)
        assert np.array_equal(a.theta, _torch_bits(want16))
        assert np.array_equal(a.p, _torch_bits(want16.to(torch.bfloat16)))


def test_bf16_grads_step_as_their_exact_fp32_values(orc):
    """bf16 main grads (uint16 patterns) give the step of their fp32 values
    (torch's widening cast): same norm, same state; a bf16 inf or NaN
    pattern skips the step and leaves every array unchanged."""
    th, m, v, G = _rand_state(40_000, 62)
    g16 = torch.from_numpy(G * np.float32(2.0 ** 10)).to(torch.bfloat16)
    gb = _torch_bits(g16).copy()
    gf = g16.float().numpy().copy()
    a = orc.OTensor.fresh(th)
    b = orc.OTensor.fresh(th)
    ra = orc.oracle_step([a], [gb], orc.Hyper(), [(1e-3, 0.1)], 1, 2.0 ** -10, max_norm=0.1)
    rb = orc.oracle_step([b], [gf], orc.Hyper(), [(1e-3, 0.1)], 1, 2.0 ** -10, max_norm=0.1)
    assert ra.applied and rb.applied and ra.clip_applied
    assert ra.norm64 == rb.norm64
    assert math.isclose(ra.norm64, math.sqrt(math.fsum((gf.astype(np.float64) * 2.0 ** -10) ** 2)),
                        rel_tol=1e-12)
    for x, y in ((a.theta, b.theta), (a.m, b.m), (a.v, b.v), (a.p, b.p)):
        assert np.array_equal(x.view(np.uint32) if x.dtype == np.float32 else x,
                              y.view(np.uint32) if y.dtype == np.float32 else y)
    for bad in (0x7F80, 0xFF80, 0x7FC1):
        gbad = gb.copy()
        gbad[12345] = bad
        c = orc.OTensor.fresh(th)
        before = c.copy()
        r = orc.oracle_step([c], [gbad], orc.Hyper(), [(1e-3, 0.1)], 1)
        assert r.found_inf and not r.applied
        assert np.array_equal(c.theta, before.theta) and np.array_equal(c.p, before.p)


def test_bf16_unscale_inplace_matches_torch(orc):
    """The in-place unscale of bf16 grads stores what torch's CPU bf16
    in-place multiply stores."""
    rng = np.random.default_rng(63)
    x = torch.from_numpy((rng.standard_normal(70_000) * 1e4).astype(np.float32)).to(torch.bfloat16)
    for inv in (2.0 ** -13, 1.0 / 3.0, 1.0):
        bits = _torch_bits(x).copy()
        orc.unscale_inplace_bf16(bits, float(np.float32(inv)))
        ref = x.clone().mul_(float(np.float32(inv)))
        assert np.array_equal(bits, _torch_bits(ref))


@pytest.mark.parametrize("mode", [ADAMW, ADAM_L2])
def test_fp16_moments_are_the_fp32_update_rounded(orc, mode):
    """fp16 exp_avg / exp_avg_sq: one step equals the fp32-moment step from
    the same (fp16-representable) moments, followed by torch's fp16 cast of
    the new moments; the master and its bf16 param are those of that fp32
    step.  Grads of unit scale keep v in fp16's normal range."""
    th, m, v, G = _rand_state(100_003, 64)
    m16 = torch.from_numpy(m * np.float32(300)).to(torch.float16)
    v16 = torch.from_numpy(v * np.float32(1e4)).to(torch.float16)
    G = G * np.float32(300)
    for t in (1, 5):
        a = orc.OTensor(th.copy(), _torch_bits(m16).copy(), _torch_bits(v16).copy(), orc.bf16_rne(th), 0,
                        moments_fp16=True)
        b = orc.OTensor(th.copy(), m16.float().numpy().copy(), v16.float().numpy().copy(), orc.bf16_rne(th), 0)
        for T in (a, b):
            orc.apply_update([T], [G], orc.Hyper(mode=mode), [(1e-3, 0.1)], t, 1.0, True, 0.5, 0.5)
        assert np.array_equal(a.theta.view(np.uint32), b.theta.view(np.uint32))
        assert np.array_equal(a.p, b.p)
        assert np.array_equal(a.m, _torch_bits(torch.from_numpy(b.m).to(torch.float16)))
        assert np.array_equal(a.v, _torch_bits(torch.from_numpy(b.v).to(torch.float16)))


def test_fp16_second_moment_underflows_at_small_grads(orc):
    """The format's limit, reproduced and not corrected: at t = 1 from zero
    moments v = (1 - beta2) g^2.  For |g| = 2^-10 that is about 9.5e-10, below
    half fp16's smallest subnormal (2^-25), so the stored v is +0; the update
    that step used the fp32 v before the store (u = 1, the first-step closed
    form), and the next step starts from v = 0."""
    g = np.full(64, 2.0 ** -10, np.float32)
    T = orc.OTensor.fresh(np.ones(64, np.float32), fp16_moments=True)
    opt = orc.OracleOptimizer([T], orc.Hyper(eps=0.0), [(2.0 ** -9, 0.0)])
    assert opt.step([g]).applied
    assert np.all(T.v == 0)
    # m = 0.1 g is an fp16 normal (about 9.8e-5 > 2^-14): stored with the RNE, not lost
    assert np.all(T.m == _torch_bits(torch.tensor([0.1 * 2.0 ** -10], dtype=torch.float32).to(torch.float16)))
    assert np.all(T.theta == np.float32(1.0 - 2.0 ** -9))


@pytest.mark.parametrize("sigma", [1e-3, 1e-4])
def test_16bit_moments_track_fp32_only_in_bf16(orc, sigma):
    """Why the library refuses fp16 moments ("02 · Optimizer：算法与 infra" §16
    allows lower-precision exp_avg / exp_avg_sq without fixing a format or a
    scale): over 200 steps at the grad scales of the two-matrix set (1e-3)
    and the 70B/8 shard (1e-4), the total update with bf16 moments stays
    within 2% of the fp32-moment update, while unscaled fp16 moments lose
    exp_avg_sq to underflow and move the weights tens of times further."""
    rng = np.random.default_rng(5)
    n = 20000
    th0 = rng.standard_normal(n).astype(np.float32)
    kinds = {"fp32": {}, "bf16": dict(state_bf16=True), "fp16": dict(fp16_moments=True)}
    Ts = {k: orc.OTensor.fresh(th0, **kw) for k, kw in kinds.items()}
    Os = {k: orc.OracleOptimizer([T], orc.Hyper(), [(1e-3, 0.0)]) for k, T in Ts.items()}
    for _ in range(200):
        G = (rng.standard_normal(n) * sigma).astype(np.float32)
        for O in Os.values():
            O.step([G])
    d = {k: T.theta.astype(np.float64) - th0 for k, T in Ts.items()}
    ref = np.mean(np.abs(d["fp32"]))
    assert np.mean(np.abs(d["bf16"] - d["fp32"])) <= 0.02 * ref
    assert np.mean(np.abs(d["fp16"])) >= 20 * ref
