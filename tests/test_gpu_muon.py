"""GPU parity of the Muon path (bf16 MFMA Newton-Schulz, momentum, scaled
update, AdamW chain) against oracle/muon.py, through the C ABI.

What is exact and what is not:
  * the momentum buffer, the 16-bit write-back of the GPU's own master, the
    skip decision and the counters are compared bit for bit;
  * NS output (and hence the master) differs from the oracle's bf16 reading
    only through the fp32 accumulation order of the matrix cores; the bound
    is derived in muon_util.py from the oracle's own spread between two
    accumulation orders;
  * the master's bound adds up, step by step, fp32(lr*scale) times the NS
    bound of that step plus two fp32 roundings.
"""
import math

import numpy as np
import pytest
import torch

from gpu_util import banner, bf16_of, require_gpu, to_np
from muon_util import check_ns, ns_reference, ns_tolerance

pytestmark = pytest.mark.gpu

F32 = np.float32


@pytest.fixture(scope="module")
def H():
    return require_gpu()


@pytest.fixture(scope="module")
def mu():
    import oracle
    import oracle.muon as m
    oracle.lib()
    return m


@pytest.fixture(scope="module")
def I():
    from mixed_precision_optimizer_amd import inputs
    return inputs


def gpu_ns(H, G: np.ndarray, cfg) -> np.ndarray:
    dev = torch.device("cuda")
    g = torch.from_numpy(np.ascontiguousarray(G, dtype=F32)).to(dev)
    out = torch.full(G.shape, float("nan"), dtype=torch.float32, device=dev)
    ws = torch.empty(max(1, H.hpo_newton_schulz_workspace(*G.shape)), dtype=torch.uint8, device=dev)
    H.hpo_newton_schulz(g, out, cfg, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy()


# ---------------------------------------------------------------------------
# Newton-Schulz alone
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("shape", [(96, 200), (200, 96), (256, 256), (300, 1000), (1000, 300), (1, 40), (40, 1),
                                   (513, 257), (1024, 4096), (4096, 1024)])
def test_newton_schulz_matches_bf16_reading(H, mu, I, shape):
    banner(f"NS {shape}")
    G = I.seeded_matrix(shape, seed=shape[0] * 7 + shape[1])
    O, spread, rel = ns_reference(mu, G)
    got = gpu_ns(H, G, H.make_muon_cfg())
    check_ns(f"{shape}", got, O, spread, rel)


@pytest.mark.parametrize("steps,coeffs", [(1, None), (3, [(3.4445, -4.7750, 2.0315), (1.875, -1.25, 0.375),
                                                          (2.0, -1.5, 0.5)]), (12, None)])
def test_newton_schulz_steps_and_schedules(H, mu, I, steps, coeffs):
    banner(f"NS steps {steps} schedule {coeffs is not None}")
    G = I.seeded_matrix((160, 416), seed=31)
    O, spread, rel = ns_reference(mu, G, steps, coeffs)
    got = gpu_ns(H, G, H.make_muon_cfg(ns_steps=steps, ns_coeffs=coeffs))
    check_ns(f"steps={steps}", got, O, spread, rel)


def test_newton_schulz_degenerate_inputs(H, mu, I):
    banner("NS zero / rank-one / tiny")
    zero = np.zeros((64, 130), F32)
    assert np.all(gpu_ns(H, zero, H.make_muon_cfg()) == 0)
    u = I.seeded_matrix((100, 1), 5)
    v = I.seeded_matrix((1, 300), 6)
    rank1 = (u @ v).astype(F32)
    O, spread, rel = ns_reference(mu, rank1)
    check_ns("rank one", gpu_ns(H, rank1, H.make_muon_cfg()), O, spread, rel)
    tiny = (I.seeded_matrix((50, 70), 8) * F32(1e-30)).astype(F32)
    O, spread, rel = ns_reference(mu, tiny)
    check_ns("tiny (below the guard)", gpu_ns(H, tiny, H.make_muon_cfg()), O, spread, rel)


@pytest.mark.parametrize("shape", [(96, 200), (200, 96)])
def test_newton_schulz_unaligned_buffers(H, mu, I, shape):
    """G and out one float past a 16-byte boundary (the boundary asks for
    4-byte alignment only): the output leaves through the element-wise path
    and must equal, bit for bit, the aligned call's float4 stores."""
    banner(f"NS unaligned {shape}")
    dev = torch.device("cuda")
    G = I.seeded_matrix(shape, seed=77 + shape[0])
    n = G.size
    gbuf = torch.zeros(n + 4, dtype=torch.float32, device=dev)
    obuf = torch.full((n + 4,), float("nan"), dtype=torch.float32, device=dev)
    g = gbuf[1:n + 1].view(shape)
    out = obuf[1:n + 1].view(shape)
    assert g.data_ptr() % 16 == 4 and out.data_ptr() % 16 == 4
    g.copy_(torch.from_numpy(G))
    ws = torch.empty(H.hpo_newton_schulz_workspace(*shape), dtype=torch.uint8, device=dev)
    H.hpo_newton_schulz(g, out, H.make_muon_cfg(), ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert torch.isnan(obuf[0]) and torch.all(torch.isnan(obuf[n + 1:])), "wrote outside the output view"
    aligned = gpu_ns(H, G, H.make_muon_cfg())
    assert np.array_equal(got.view(np.uint32), aligned.view(np.uint32))
    O, spread, rel = ns_reference(mu, G)
    check_ns(f"unaligned {shape}", got, O, spread, rel)


def test_newton_schulz_handbook_printout(H, I):
    """The GPU's NS output reproduces the figures the handbook prints for its
    256 x 1024 demonstration, within one unit of each printed last digit."""
    banner("NS handbook demonstration")
    from conftest import read_golden
    gold = read_golden("handbook_muon_newton_schulz.txt")
    G, V = I.handbook_ns_matrix()
    for steps in (1, 3, 5):
        s = np.linalg.svd(gpu_ns(H, G, H.make_muon_cfg(ns_steps=steps)).astype(np.float64), compute_uv=False)
        lo, hi, pct = gold[f"ns_steps_{steps}"]
        share = 100.0 * float(np.mean((s > 0.7) & (s < 1.2)))
        assert abs(s.min() - float(lo)) <= 0.015 and abs(s.max() - float(hi)) <= 0.015, (steps, s.min(), s.max())
        assert abs(share - float(pct.rstrip("%"))) <= 1.5, (steps, share)
    X = gpu_ns(H, G, H.make_muon_cfg()).astype(np.float64)
    e5 = 100.0 * float(np.linalg.norm(X @ V[:, :8]) ** 2 / np.linalg.norm(X) ** 2)
    assert abs(e5 - float(gold["top8_energy"][1].rstrip("%"))) <= 0.15
    rms = math.sqrt(float(np.mean(X ** 2)))
    assert abs(rms - float(gold["rms"][0])) <= 1.5e-4
    assert abs(rms * 0.2 * 32 - float(gold["rms"][2])) <= 0.015


# ---------------------------------------------------------------------------
# Muon sets: momentum + NS + update, host-driven
# ---------------------------------------------------------------------------
class MuonCase:
    """Device tensors of a Muon set and the oracle's copy of the same start."""

    def __init__(self, H, mu, I, shapes, pdt="bf16", seed=100, groups=None):
        dev = torch.device("cuda")
        self.shapes = shapes
        self.group_index = groups or [i % 2 for i in range(len(shapes))]
        W0 = [I.seeded_matrix(s, seed + i, 0.02) for i, s in enumerate(shapes)]
        self.master = [torch.from_numpy(w.copy()).to(dev) for w in W0]
        self.grad = [torch.zeros(s, dtype=torch.float32, device=dev) for s in shapes]
        self.mom = [torch.zeros(s, dtype=torch.float32, device=dev) for s in shapes]
        if pdt == "bf16":
            self.param = [m.to(torch.bfloat16) for m in self.master]
        else:
            self.param = None
        self.set = H.hpo_muon_set_create(self.param, self.master, self.grad, self.mom, self.group_index)
        self.orc = [mu.OMatrix.fresh(w, bf16_param=(pdt == "bf16"), group=g) for w, g in zip(W0, self.group_index)]
        self.bound = [np.zeros(s, np.float64) for s in shapes]

    def set_grads(self, grads):
        for t, g in zip(self.grad, grads):
            t.copy_(torch.from_numpy(g))


def _compare_case(case, mu, cfg_o, last, groups, tag):
    """Momentum bit-exact; master within the accumulated bound; param is
    bf16 of the GPU master."""
    for i, s in enumerate(case.shapes):
        o = case.orc[i]
        M = to_np(case.mom[i])
        W = to_np(case.master[i])
        assert np.array_equal(M.view(np.uint32), o.M.view(np.uint32)), f"{tag} matrix {i}: momentum not bit-equal"
        if case.param is not None:
            p = to_np(case.param[i])
            assert np.array_equal(p, bf16_of(W.ravel()).reshape(s)), f"{tag} matrix {i}: param != bf16(master)"
        if W.size == 0:
            continue
        d = np.abs(W.astype(np.float64) - o.W)
        assert np.all(d <= case.bound[i]), (f"{tag} matrix {i} {s}: master off by {d.max():.3e}, "
                                            f"bound {case.bound[i].max():.3e}")


def _grow_bounds(case, mu, cfg, groups, rec):
    """Adds this applied step's NS bound (times fp32(lr*scale)) and two fp32
    roundings of the master to every matrix's bound."""
    for i, s in enumerate(case.shapes):
        r = rec[i]
        if r is None:
            continue
        O, spread, rel = ns_reference(mu, r["g_tilde"], cfg.steps, cfg.coeffs)
        tol_max, _ = ns_tolerance(O, spread, rel)
        lr, wd = groups[case.orc[i].group]
        k2 = float(F32(lr * r["scale"]))
        W = np.abs(case.orc[i].W.astype(np.float64))
        case.bound[i] = case.bound[i] * float(F32(1.0 - lr * wd)) + k2 * tol_max * (1 + 2 ** -20) + \
            2 * np.spacing(W.astype(F32)).astype(np.float64)


@pytest.mark.parametrize("variant", ["bf16_sum_nesterov", "fp32_ema", "bf16_ema_plain", "bf16_plain_shape_scale",
                                     "bf16_unit_rms_scale"])
def test_muon_set_steps(H, mu, I, variant):
    banner(f"Muon set {variant}")
    dev = torch.device("cuda")
    shapes = I.MUON_PARITY_SHAPES
    pdt = "fp32" if variant == "fp32_ema" else "bf16"
    case = MuonCase(H, mu, I, shapes, pdt=pdt)
    if variant == "fp32_ema":
        cfg_o = mu.MuonCfg(mu=0.9, form=mu.MOMENTUM_EMA)
        cfg = H.make_muon_cfg(momentum=0.9, momentum_form=H.HPO_MUON_MOMENTUM_EMA)
    elif variant == "bf16_ema_plain":
        cfg_o = mu.MuonCfg(mu=0.8, form=mu.MOMENTUM_EMA, nesterov=False)
        cfg = H.make_muon_cfg(momentum=0.8, momentum_form=H.HPO_MUON_MOMENTUM_EMA, nesterov=False)
    elif variant == "bf16_plain_shape_scale":
        cfg_o = mu.MuonCfg(nesterov=False, scale_mode=mu.SCALE_SHAPE, extra_scale=1.0)
        cfg = H.make_muon_cfg(nesterov=False, scale_mode=H.HPO_MUON_SCALE_SHAPE, extra_scale=1.0)
    elif variant == "bf16_unit_rms_scale":
        cfg_o = mu.MuonCfg(scale_mode=mu.SCALE_UNIT_RMS, extra_scale=0.5)
        cfg = H.make_muon_cfg(scale_mode=H.HPO_MUON_SCALE_UNIT_RMS, extra_scale=0.5)
    else:
        cfg_o = mu.MuonCfg()
        cfg = H.make_muon_cfg()
    groups = [(0.02, 0.1), (0.01, 0.0)]
    chain = mu.ChainedOracle([], None, [], case.orc, cfg_o, groups, max_norm=1.0)
    d_norm = torch.zeros(1, dtype=torch.float32, device=dev)
    d_found = torch.zeros(1, dtype=torch.int32, device=dev)
    loss_scale = 1024.0
    inv = 1.0 / loss_scale
    for k in range(1, 5):
        # stored grads: N(0, 1e-2) * loss scale; step 3 carries an inf in one matrix
        grads = [(I.seeded_matrix(s, 1000 * k + i, 1e-2) * F32(loss_scale)).astype(F32)
                 for i, s in enumerate(shapes)]
        if k == 3:
            grads[2][5, 7] = np.inf
        case.set_grads(grads)
        d_found.zero_()
        H.hpo_grad_global_norm(case.set, inv, d_norm, d_found)
        H.hpo_muon_step(case.set, cfg, groups, None, inv, 1.0, d_norm, d_found)
        torch.cuda.synchronize()
        r = chain.step([], grads, inv)
        found = bool(d_found.item())
        assert found == r.found_inf, f"step {k}: found_inf {found} vs oracle {r.found_inf}"
        if r.applied:
            assert float(d_norm.item()) == r.norm32, f"step {k}: norm {d_norm.item()} vs {r.norm32}"
            _grow_bounds(case, mu, cfg_o, groups, chain.last)
        _compare_case(case, mu, cfg_o, chain.last, groups, f"{variant} step {k}")


def test_muon_set_batches_under_a_small_workspace(H, mu, I):
    """A workspace cap that fits one matrix per batch gives the same bits as
    the default plan (batching changes no arithmetic)."""
    banner("Muon batching invariance")
    shapes = [(300, 700)] * 3 + [(128, 384)] * 2
    a = MuonCase(H, mu, I, shapes, seed=7)
    dev = torch.device("cuda")
    W0 = [I.seeded_matrix(s, 7 + i, 0.02) for i, s in enumerate(shapes)]
    master = [torch.from_numpy(w.copy()).to(dev) for w in W0]
    grad = [torch.zeros(s, dtype=torch.float32, device=dev) for s in shapes]
    mom = [torch.zeros(s, dtype=torch.float32, device=dev) for s in shapes]
    param = [m.to(torch.bfloat16) for m in master]
    small = H.hpo_muon_set_create(param, master, grad, mom, a.group_index, workspace_bytes=1)
    info_a, info_b = a.set.info(), small.info()
    assert info_b.device_bytes < info_a.device_bytes
    cfg = H.make_muon_cfg()
    groups = [(0.02, 0.1), (0.01, 0.0)]
    for k in range(1, 3):
        grads = [I.seeded_matrix(s, 50 * k + i, 1e-2) for i, s in enumerate(shapes)]
        a.set_grads(grads)
        for t, g in zip(grad, grads):
            t.copy_(torch.from_numpy(g))
        H.hpo_muon_step(a.set, cfg, groups, None)
        H.hpo_muon_step(small, cfg, groups, None)
    torch.cuda.synchronize()
    for i in range(len(shapes)):
        assert torch.equal(a.master[i], master[i]) and torch.equal(a.mom[i], mom[i])
        assert torch.equal(a.param[i].view(torch.int16), param[i].view(torch.int16))


def test_muon_rejects_adam_calls_and_vice_versa(H, mu, I):
    case = MuonCase(H, mu, I, [(64, 96)])
    cfg = H.make_cfg()
    with pytest.raises(H.HpoError):
        H.hpo_adamw_step(case.set, cfg, [(1e-3, 0.1), (1e-3, 0.0)], None, 1, 1.0, 0.0, None, None)
    dev = torch.device("cuda")
    t = [torch.zeros(64, dtype=torch.float32, device=dev) for _ in range(4)]
    adam = H.hpo_set_create_list(None, [t[0]], [t[1]], [t[2]], [t[3]])
    with pytest.raises(H.HpoError):
        H.hpo_muon_step(adam, H.make_muon_cfg(), [(1e-3, 0.1)], None)
    with pytest.raises(H.HpoError):
        H.hpo_muon_set_create([torch.zeros((4, 4), dtype=torch.float16, device=dev)],
                              [torch.zeros((4, 4), device=dev)], [torch.zeros((4, 4), device=dev)],
                              [torch.zeros((4, 4), device=dev)])


# ---------------------------------------------------------------------------
# The chain: AdamW + Muon, device-resident, with the loss scaler
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("lowp", [False, True])
def test_chained_device_step(H, mu, I, lowp):
    """AdamW tensors (an embedding-like matrix and norm gains) and Muon
    matrices stepped by hpo_step_device_chain with a dynamic loss scaler:
    one norm over both, one skip, one counter.  AdamW state is bit-exact; the
    Muon momentum is bit-exact; masters within the NS bound.  lowp: the AdamW
    set keeps bf16 main grads and an fp16 master."""
    banner(f"chained AdamW + Muon device step, AdamW bf16 grads + fp16 master {lowp}")
    import oracle
    dev = torch.device("cuda")
    adam_shapes = [(3000,), (256,), (64 * 50,)]
    groups = [(1e-3, 0.0), (1e-3, 0.1)]   # no-decay group (norm gains), decaying group
    aidx = [0, 0, 1]
    A0 = [I.seeded_matrix(s, 500 + i, 0.02).ravel() for i, s in enumerate(adam_shapes)]
    am = [torch.from_numpy(a.copy()).to(dev) for a in A0]
    if lowp:
        am = [t.half() for t in am]
    ap = [t.to(torch.bfloat16) for t in am]
    ag = [torch.zeros(t.numel(), dtype=torch.bfloat16 if lowp else torch.float32, device=dev) for t in am]
    a1 = [torch.zeros(t.numel(), device=dev) for t in am]
    a2 = [torch.zeros(t.numel(), device=dev) for t in am]
    aset = H.hpo_set_create_list(ap, am, ag, a1, a2, aidx)
    shapes = [(128, 384), (384, 128), (300, 700), (37, 129)]
    case = MuonCase(H, mu, I, shapes, groups=[0, 1, 0, 1])
    mgroups = [(0.02, 0.1), (0.01, 0.0)]
    cfg_o = mu.MuonCfg()
    chain = mu.ChainedOracle([oracle.OTensor.fresh(a, group=g, fp16_master=lowp) for a, g in zip(A0, aidx)], oracle.Hyper(),
                             groups, case.orc, cfg_o, mgroups, max_norm=1.0)
    scaler = oracle.LossScaler(scale=2.0 ** 16, growth_interval=3, hysteresis=1)
    d_state = H.new_scaler_state(dev)
    H.hpo_scaler_state_init(d_state, 2.0 ** 16, 1, 0)
    scfg = H.make_scaler_cfg(dynamic=True, growth_interval=3, hysteresis=1)
    acfg = H.make_cfg()
    mcfg = H.make_muon_cfg()
    for k in range(1, 8):
        S = float(scaler.scale)
        ga = [(I.seeded_matrix(s, 900 * k + i, 1e-2).ravel() * F32(S)).astype(F32)
              for i, s in enumerate(adam_shapes)]
        gm = [(I.seeded_matrix(s, 700 * k + i, 1e-2) * F32(S)).astype(F32) for i, s in enumerate(shapes)]
        if k == 4:
            gm[1][3, 3] = np.inf
        for t, g in zip(ag, ga):
            t.copy_(torch.from_numpy(g))
        if lowp:     # the oracle reads the bf16 patterns the set holds
            ga = [to_np(t) for t in ag]
        case.set_grads(gm)
        st_before = H.read_scaler_state(d_state)
        H.hpo_step_device_chain(aset, acfg, groups, case.set, mcfg, mgroups, 1.0, scfg, d_state,
                                st_before.applied_steps + 1, 1)
        torch.cuda.synchronize()
        inv = scaler.inv_scale()
        found = any(not np.all(np.isfinite(g)) for g in gm) or any(
            not np.all(np.isfinite(oracle.grad_f32(g))) for g in ga)
        scaler.update(found)
        r = chain.step(ga, gm, inv)
        assert r.found_inf == found
        st = H.read_scaler_state(d_state)
        assert st.error == 0
        assert bool(st.found_inf) == found and bool(st.applied) == (not found), k
        assert st.loss_scale == float(scaler.scale), (k, st.loss_scale, scaler.scale)
        assert st.applied_steps == chain.t
        if r.applied:
            assert st.grad_norm == r.norm32, (k, st.grad_norm, r.norm32)
            _grow_bounds(case, mu, cfg_o, mgroups, chain.last)
        for i, T in enumerate(chain.adam):
            assert np.array_equal(to_np(am[i]).view(np.uint8), T.theta.view(np.uint8)), f"step {k} adam {i}"
            assert np.array_equal(to_np(a1[i]).view(np.uint32), T.m.view(np.uint32))
            assert np.array_equal(to_np(a2[i]).view(np.uint32), T.v.view(np.uint32))
            assert np.array_equal(to_np(ap[i]), T.p)
        _compare_case(case, mu, cfg_o, chain.last, mgroups, f"chain step {k}")


def test_chain_with_one_set_matches_the_separate_calls(H, mu, I):
    """hpo_step_device_chain with only a Muon set, or only an AdamW set, does
    what the separate calls do: the same bits as hpo_grad_global_norm_sets +
    hpo_muon_step, and as hpo_step_device, on identical twins of the sets."""
    banner("chain with one set")
    dev = torch.device("cuda")
    shapes = [(128, 384), (384, 128), (37, 129)]
    mgroups = [(0.02, 0.1), (0.01, 0.0)]

    def muon_twin():
        W0 = [I.seeded_matrix(s, 40 + i, 0.02) for i, s in enumerate(shapes)]
        m = [torch.from_numpy(w.copy()).to(dev) for w in W0]
        g = [torch.zeros(s, dtype=torch.float32, device=dev) for s in shapes]
        o = [torch.zeros(s, dtype=torch.float32, device=dev) for s in shapes]
        p = [t.to(torch.bfloat16) for t in m]
        return H.hpo_muon_set_create(p, m, g, o, [0, 1, 0]), m, g, o, p

    a, b = muon_twin(), muon_twin()
    d_state = H.new_scaler_state(dev)
    H.hpo_scaler_state_init(d_state, 1.0, 1, 0)
    d_norm = torch.zeros(1, dtype=torch.float32, device=dev)
    d_found = torch.zeros(1, dtype=torch.int32, device=dev)
    scfg = H.make_scaler_cfg(dynamic=False)
    for k in range(1, 4):
        grads = [I.seeded_matrix(s, 60 * k + i, 1e-1) for i, s in enumerate(shapes)]
        for twin in (a, b):
            for t, g in zip(twin[2], grads):
                t.copy_(torch.from_numpy(g))
        H.hpo_step_device_chain(None, None, None, a[0], H.make_muon_cfg(), mgroups, 1.0, scfg, d_state, k, 1)
        d_found.zero_()
        H.hpo_grad_global_norm_sets([b[0]], 1.0, d_norm, d_found)
        H.hpo_muon_step(b[0], H.make_muon_cfg(), mgroups, None, 1.0, 1.0, d_norm, d_found)
        torch.cuda.synchronize()
        st = H.read_scaler_state(d_state)
        assert st.applied_steps == k and st.grad_norm == float(d_norm.item()), k
        for x, y in zip(a[1] + a[3] + a[4], b[1] + b[3] + b[4]):
            assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x,
                               y.view(torch.int16) if y.dtype == torch.bfloat16 else y), f"muon-only chain step {k}"

    # AdamW only: the chain against hpo_step_device
    sizes = [3000, 256, 1000]

    def adam_twin():
        m = [torch.from_numpy(I.seeded_matrix((n,), 80 + i, 0.02)).to(dev) for i, n in enumerate(sizes)]
        p = [t.to(torch.bfloat16) for t in m]
        g = [torch.zeros_like(t) for t in m]
        m1 = [torch.zeros_like(t) for t in m]
        m2 = [torch.zeros_like(t) for t in m]
        return H.hpo_set_create_list(p, m, g, m1, m2, [0, 1, 0]), m, g, m1, m2, p

    a, b = adam_twin(), adam_twin()
    sa, sb = H.new_scaler_state(dev), H.new_scaler_state(dev)
    for st_ in (sa, sb):
        H.hpo_scaler_state_init(st_, 256.0, 2, 0)
    groups = [(1e-3, 0.1), (1e-3, 0.0)]
    scfg = H.make_scaler_cfg(dynamic=True, growth_interval=2)
    for k in range(1, 5):
        scale = H.read_scaler_state(sa).loss_scale
        grads = [(I.seeded_matrix((n,), 90 * k + i, 1e-2) * F32(scale)).astype(F32) for i, n in enumerate(sizes)]
        if k == 2:
            grads[1][7] = np.nan
        for twin in (a, b):
            for t, g in zip(twin[2], grads):
                t.copy_(torch.from_numpy(g))
        ta = H.read_scaler_state(sa).applied_steps + 1
        tb = H.read_scaler_state(sb).applied_steps + 1
        H.hpo_step_device_chain(a[0], H.make_cfg(), groups, None, None, None, 1.0, scfg, sa, ta, 1)
        H.hpo_step_device(b[0], H.make_cfg(), groups, None, 1.0, scfg, sb, tb, 1)
        torch.cuda.synchronize()
        assert sa.cpu().numpy().tobytes() == sb.cpu().numpy().tobytes(), f"scaler state step {k}"
        for x, y in zip(a[1] + a[3] + a[4] + a[5], b[1] + b[3] + b[4] + b[5]):
            assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x,
                               y.view(torch.int16) if y.dtype == torch.bfloat16 else y), f"adam-only chain step {k}"


def test_muon_profile_counts(H, mu, I):
    """The opt-in timing records one momentum and one input launch per batch,
    ns_steps Gram / polynomial launches per batch, ns_steps - 1 plain steps
    and one fused update; flops follow m(m+1)n, m^2(m+1) and 2 m^2 n."""
    banner("Muon profile")
    shapes = [(300, 700), (300, 700), (128, 384)]
    case = MuonCase(H, mu, I, shapes, seed=3)
    H.hpo_muon_profile_enable(case.set, True)
    H.hpo_muon_step(case.set, H.make_muon_cfg(), [(0.02, 0.1), (0.01, 0.0)], None)
    p = H.hpo_muon_profile_read(case.set)
    H.hpo_muon_profile_enable(case.set, False)
    n_batches = 2
    assert p["momentum"]["launches"] == n_batches and p["input"]["launches"] == n_batches
    assert p["gram"]["launches"] == 5 * n_batches and p["poly"]["launches"] == 5 * n_batches
    assert p["step"]["launches"] == 4 * n_batches and p["update"]["launches"] == n_batches
    want_gram = 5 * (2 * 300 * 301 * 700 + 128 * 129 * 384)
    want_step = 4 * (2 * 2 * 300 ** 2 * 700 + 2 * 128 ** 2 * 384)
    assert p["gram"]["flops"] == want_gram and p["step"]["flops"] == want_step
    assert p["momentum"]["bytes"] == 16 * (2 * 300 * 700 + 128 * 384)
    assert all(v["ms"] > 0 for v in p.values())
    with pytest.raises(H.HpoError):
        H.hpo_muon_profile_read(case.set)
