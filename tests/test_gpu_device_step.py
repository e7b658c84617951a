"""GPU parity of the device-resident step (hpo_step_device): the loss scaler,
the skip decisions and the applied-step counter live on the device and steps
are enqueued without host synchronisation.  Compared with the oracle's
scaled trajectory (oracle.LossScaler + OracleOptimizer.step_scaled)."""
import math

import numpy as np
import pytest
import torch

from gpu_util import banner, require_gpu, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def H():
    return require_gpu()


@pytest.fixture(scope="module")
def orc():
    import oracle
    oracle.lib()
    return oracle


SIZES = [70_001, 4096, 131_072, 3]
GROUPS = [0, 1, 0, 1]
INF_STEPS = {3, 4, 10, 25}
BIG_STEP = 15          # finite grads whose norm exceeds the skip threshold
SYNC_AFTER = {2, 9, 16, 17, 40}


def _true_grads(k, rng_seed=500):
    rng = np.random.default_rng(rng_seed + k)
    gs = [(rng.standard_normal(n) * 1e-3).astype(np.float32) for n in SIZES]
    if k == BIG_STEP:
        gs = [(g * np.float32(1e4)).astype(np.float32) for g in gs]
    return gs


@pytest.mark.parametrize("mode,pdt,lowp", [(0, "bf16", False), (1, "bf16", False), (0, "fp16", False),
                                           (1, "bf16", True)])
def test_device_step_sequence_matches_oracle(H, orc, mode, pdt, lowp):
    """lowp: bf16 main grads and an fp16 master under the bf16 params."""
    banner(f"device-resident step sequence, mode {mode}, {pdt} params, bf16 grads + fp16 master {lowp}")
    from mixed_precision_optimizer_amd import DeviceAdamW
    rng = np.random.default_rng(400)
    th0 = [rng.standard_normal(n).astype(np.float32) for n in SIZES]
    ths = [torch.from_numpy(a.copy()).to(DEV).to(torch.float16 if lowp else torch.float32) for a in th0]
    tdt = torch.float16 if pdt == "fp16" else torch.bfloat16
    ps = [t.to(tdt) for t in ths]
    gs = [torch.zeros(n, device=DEV, dtype=torch.bfloat16 if lowp else torch.float32) for n in SIZES]
    ms = [torch.zeros(n, device=DEV) for n in SIZES]
    vs = [torch.zeros(n, device=DEV) for n in SIZES]
    hset = H.hpo_set_create_list(ps, ths, gs, ms, vs, GROUPS)
    groups = [(1e-3, 0.1), (1e-3, 0.0)]
    kw = dict(loss_scale=2.0 ** 16, dynamic=True, growth_interval=5, hysteresis=2, min_scale=1.0,
              grad_norm_skip_threshold=50.0)
    opt = DeviceAdamW(hset, groups, mode=mode, max_norm=1.0, **kw)
    T = [orc.OTensor(to_np(t), np.zeros_like(a), np.zeros_like(a), to_np(p), g, pdt == "fp16", lowp)
         for a, t, p, g in zip(th0, ths, ps, GROUPS)]
    O = orc.OracleOptimizer(T, orc.Hyper(mode=mode), groups, max_norm=1.0)
    sc = orc.LossScaler(scale=2.0 ** 16, dynamic=True, growth_interval=5, hysteresis=2, min_scale=1.0)
    applied = skipped = 0
    for k in range(1, 41):
        true = _true_grads(k)
        # the caller's backward: stored grads = true grads * current loss scale,
        # taken from the device state without a sync
        for g, t in zip(gs, true):
            g.copy_(torch.from_numpy(t))
            g.mul_(opt.loss_scale_tensor)
        if k in INF_STEPS:
            gs[2][-1] = float("inf")
        if lowp:   # the bf16 image of the true grads, times the power-of-two scale (exact)
            stored = [to_np(torch.from_numpy(t).to(torch.bfloat16).mul_(sc.scale)) for t in true]
            if k in INF_STEPS:
                stored[2][-1] = 0x7F80
        else:
            stored = [(t * sc.scale).astype(np.float32) for t in true]
            if k in INF_STEPS:
                stored[2][-1] = np.inf
        r = O.step_scaled(stored, sc, skip_threshold=50.0)
        applied += int(r.applied)
        skipped += int(not r.applied)
        opt.step()
        if k in SYNC_AFTER:
            st = opt.sync()
            assert st.error == 0
            assert st.applied_steps == O.t == applied and st.skipped_steps == skipped, k
            assert st.loss_scale == float(sc.scale) and st.inv_scale == sc.inv_scale(), k
            assert st.growth_tracker == sc.growth_tracker and st.hysteresis_tracker == sc.hysteresis_tracker, k
            assert bool(st.found_inf) == bool(r.found_inf) and bool(st.applied) == r.applied, k
            if r.norm32 is not None:
                assert st.grad_norm == r.norm32 or abs(st.grad_norm - r.norm64) <= 1e-5 * r.norm64
            for i in range(len(SIZES)):
                assert np.array_equal(to_np(ths[i]).view(np.uint8), T[i].theta.view(np.uint8)), (k, i)
                assert np.array_equal(to_np(ms[i]).view(np.uint32), T[i].m.view(np.uint32)), (k, i)
                assert np.array_equal(to_np(vs[i]).view(np.uint32), T[i].v.view(np.uint32)), (k, i)
                assert np.array_equal(to_np(ps[i]), T[i].p), (k, i)
    # the script exercised every branch: skips by inf and by threshold, a back-off and a growth
    assert skipped == len(INF_STEPS) + 1 and applied == 40 - skipped
    hset.close()


def test_long_unsynchronised_run_uses_full_window(H, orc):
    """More steps than one window without any explicit sync: the optimizer
    re-reads the state every 32 steps; the result equals the oracle's."""
    banner("device-resident step, 70 steps without explicit sync")
    from mixed_precision_optimizer_amd import DeviceAdamW
    n = 50_000
    rng = np.random.default_rng(410)
    th0 = rng.standard_normal(n).astype(np.float32)
    th = torch.from_numpy(th0.copy()).to(DEV)
    p = th.to(torch.bfloat16)
    g = torch.zeros(n, device=DEV)
    m = torch.zeros(n, device=DEV)
    v = torch.zeros(n, device=DEV)
    hset = H.hpo_set_create_flat(p, th, g, m, v)
    opt = DeviceAdamW(hset, [(1e-3, 0.1)], max_norm=1.0, loss_scale=1.0, dynamic=False)
    T = orc.OTensor.fresh(th0)
    O = orc.OracleOptimizer([T], orc.Hyper(), [(1e-3, 0.1)], max_norm=1.0)
    sc = orc.LossScaler(scale=1.0, dynamic=False)
    grads = [(np.random.default_rng(420 + k).standard_normal(n) * 1e-2).astype(np.float32) for k in range(70)]
    dev_grads = [torch.from_numpy(x).to(DEV) for x in grads]
    for k in range(70):
        g.copy_(dev_grads[k])
        opt.step()
        O.step_scaled([grads[k]], sc)
    st = opt.sync()
    assert st.applied_steps == 70 and st.error == 0
    assert np.array_equal(to_np(th).view(np.uint32), T.theta.view(np.uint32))
    assert np.array_equal(to_np(p), T.p)
    hset.close()


def test_window_error_is_reported_not_applied(H):
    """A step whose device t falls outside the window the host gave is not
    applied and sets the sticky error flag (condition forced from the host;
    every kernel runs to completion)."""
    banner("window error")
    n = 4096
    th = torch.randn(n, device=DEV)
    p = th.to(torch.bfloat16)
    g = torch.randn(n, device=DEV) * 1e-3
    m = torch.zeros(n, device=DEV)
    v = torch.zeros(n, device=DEV)
    th0 = th.clone()
    hset = H.hpo_set_create_flat(p, th, g, m, v)
    d_state = H.new_scaler_state()
    H.hpo_scaler_state_init(d_state, 1.0, 1, 0)
    scfg = H.make_scaler_cfg(dynamic=False)
    H.hpo_step_device(hset, H.make_cfg(), [(1e-3, 0.1)], None, 1.0, scfg, d_state, 5, 1)  # device t = 1, window {5}
    torch.cuda.synchronize()
    st = H.read_scaler_state(d_state)
    assert st.error == 1 and st.applied == 0 and st.applied_steps == 0 and st.skipped_steps == 1
    assert torch.equal(th, th0) and not m.any()
    with pytest.raises(H.HpoError):
        H.hpo_step_device(hset, H.make_cfg(), [(1e-3, 0.1)], None, 1.0, scfg, d_state, 1, H.HPO_MAX_WINDOW + 1)
    hset.close()


def test_graph_replays_match_eager_steps(H):
    """The device-resident step keeps no host state between calls, so one
    step captured in a HIP graph (DeviceAdamW.graph) replays as the step
    itself.  Twin sets from one seeded state, a dynamic scaler and an inf at
    step 5: 12 graph replays against 12 eager steps, with fresh grads copied
    in, other eager work and a synchronisation before every replay; each
    replay leaves the same bits (params, masters, moments, scaler state) as its
    eager twin.  Replays past the graph's window of t values are refused on
    the device (error flag), not applied."""
    banner("device-resident step replayed from a HIP graph")
    from mixed_precision_optimizer_amd import DeviceAdamW
    sizes = [70_001, 4096, 3]
    rng = np.random.default_rng(430)
    th0 = [rng.standard_normal(n).astype(np.float32) for n in sizes]

    def make():
        ths = [torch.from_numpy(a.copy()).to(DEV) for a in th0]
        ps = [t.to(torch.bfloat16) for t in ths]
        gs, ms, vs = ([torch.zeros(n, device=DEV) for n in sizes] for _ in range(3))
        hset = H.hpo_set_create_list(ps, ths, gs, ms, vs, [0, 1, 0])
        opt = DeviceAdamW(hset, [(1e-3, 0.1), (1e-3, 0.0)], max_norm=1.0, loss_scale=2.0 ** 10, dynamic=True,
                          growth_interval=3, hysteresis=1)
        return hset, opt, (ths, ps, gs, ms, vs)

    set_a, opt_a, bufs_a = make()
    set_b, opt_b, bufs_b = make()
    graph = opt_a.graph()
    other = torch.zeros(1 << 20, device=DEV)
    for k in range(1, 13):
        scale = H.read_scaler_state(opt_b.d_state).loss_scale
        G = [(np.random.default_rng(440 + k).standard_normal(n) * 1e-2 * scale).astype(np.float32) for n in sizes]
        if k == 5:
            G[0][123] = np.inf
        for ga, gb, x in zip(bufs_a[2], bufs_b[2], G):
            ga.copy_(torch.from_numpy(x))
            gb.copy_(torch.from_numpy(x))
        other.add_(1.0)
        torch.cuda.synchronize()
        graph.replay()
        opt_b.step()
        torch.cuda.synchronize()
        for i in range(len(sizes)):
            for j in (0, 3, 4):
                assert torch.equal(bufs_a[j][i].view(torch.int32), bufs_b[j][i].view(torch.int32)), (k, i, j)
            assert torch.equal(bufs_a[1][i].view(torch.int16), bufs_b[1][i].view(torch.int16)), (k, i)
        assert torch.equal(opt_a.d_state, opt_b.d_state), f"step {k}: scaler state differs"
    st = H.read_scaler_state(opt_a.d_state)
    assert st.applied_steps == 11 and st.skipped_steps == 1 and st.error == 0
    # the graph holds t = 1 .. HPO_MAX_WINDOW: that many applied steps in all, then refusals
    for _ in range(H.HPO_MAX_WINDOW - 11 + 4):
        graph.replay()
    torch.cuda.synchronize()
    st = H.read_scaler_state(opt_a.d_state)
    assert st.applied_steps == H.HPO_MAX_WINDOW and st.skipped_steps == 5 and st.error == 1
    set_a.close()
    set_b.close()


def test_long_run_eager_then_graph_replays(H, orc):
    """2000 device-resident steps on a small set against the oracle's scaled
    trajectory: steps 1..1000 eager (DeviceAdamW.step, the state read every 32
    steps), steps 1001..2000 replayed from a captured step (captured again
    every 256 replays).  A dynamic scaler (growth after 40 clean steps,
    hysteresis 2), infs in pairs (k = 0, 1 mod 97: the second one backs the
    scale off) and a spike every 151st step that the norm threshold skips.  At every capture and at the end, the scaler
    state, the counters and every element equal the oracle's, bit for bit."""
    banner("device-resident step, 2000 steps, eager then graph replays")
    from mixed_precision_optimizer_amd import DeviceAdamW
    sizes, gidx = [20_011, 4096, 7], [0, 1, 0]
    groups = [(1e-3, 0.1), (1e-3, 0.0)]
    rng = np.random.default_rng(450)
    th0 = [rng.standard_normal(n).astype(np.float32) for n in sizes]
    ths = [torch.from_numpy(a.copy()).to(DEV) for a in th0]
    ps = [t.to(torch.bfloat16) for t in ths]
    gs, ms, vs = ([torch.zeros(n, device=DEV) for n in sizes] for _ in range(3))
    hset = H.hpo_set_create_list(ps, ths, gs, ms, vs, gidx)
    scaler = dict(dynamic=True, growth_interval=40, hysteresis=2, min_scale=1.0)
    opt = DeviceAdamW(hset, groups, max_norm=1.0, loss_scale=2.0 ** 12, grad_norm_skip_threshold=50.0, **scaler)
    T = [orc.OTensor.fresh(a, group=g) for a, g in zip(th0, gidx)]
    O = orc.OracleOptimizer(T, orc.Hyper(), groups, max_norm=1.0)
    sc = orc.LossScaler(scale=2.0 ** 12, **scaler)

    def check(k):
        st = opt.sync()
        assert st.error == 0 and st.applied_steps == O.t, (k, st.applied_steps, O.t)
        assert st.loss_scale == float(sc.scale) and st.growth_tracker == sc.growth_tracker, k
        assert st.hysteresis_tracker == sc.hysteresis_tracker, k
        for i in range(len(sizes)):
            for got, want in ((ths[i], T[i].theta), (ms[i], T[i].m), (vs[i], T[i].v)):
                assert np.array_equal(to_np(got).view(np.uint32), want.view(np.uint32)), (k, i)
            assert np.array_equal(to_np(ps[i]), T[i].p), (k, i)

    graph, replays = None, 0
    skipped = 0
    for k in range(1, 2001):
        if k > 1000 and (graph is None or replays == H.HPO_MAX_WINDOW):
            check(k - 1)   # both sides have taken steps 1 .. k - 1
            graph, replays = opt.graph(), 0
        true = [(np.random.default_rng(460 + k).standard_normal(n) * 1e-3).astype(np.float32) for n in sizes]
        if k % 151 == 0:
            true = [(t * np.float32(1e4)).astype(np.float32) for t in true]
        for g, t in zip(gs, true):
            g.copy_(torch.from_numpy(t))
            g.mul_(opt.loss_scale_tensor)   # the caller's backward, scaled on the device, no sync
        stored = [(t * sc.scale).astype(np.float32) for t in true]
        if k % 97 in (0, 1):
            gs[0][5] = float("inf")
            stored[0][5] = np.inf
        r = O.step_scaled(stored, sc, skip_threshold=50.0)
        skipped += int(not r.applied)
        if k <= 1000:
            opt.step()
        else:
            graph.replay()
            replays += 1
    check(2000)
    assert skipped == sum(1 for k in range(1, 2001) if k % 97 in (0, 1) or k % 151 == 0)
    hset.close()


def test_binding_refuses_wrong_or_short_device_buffers(H):
    """Device buffers of the wrong dtype, too short or strided are refused by
    the binding with a clear error, before any kernel could read or write past
    them; the well-formed call right after still runs."""
    banner("binding: device buffer checks")
    n = 4096
    t = [torch.zeros(n, device=DEV) for _ in range(4)]
    hset = H.hpo_set_create_list([x.to(torch.bfloat16) for x in t[:1]], t[:1], t[1:2], t[2:3], t[3:4])
    with pytest.raises(TypeError, match="d_norm must be torch.float32"):
        H.hpo_grad_global_norm(hset, 1.0, torch.zeros(1, dtype=torch.float64, device=DEV))
    with pytest.raises(ValueError, match="d_norm spans 0 bytes"):
        H.hpo_grad_global_norm(hset, 1.0, torch.zeros(0, device=DEV))
    with pytest.raises(TypeError, match="d_found_inf must be torch.int32"):
        H.hpo_unscale_check_inf(hset, 1.0, torch.zeros(1, device=DEV))
    with pytest.raises(ValueError, match="d_state spans 40 bytes"):
        H.hpo_scaler_state_init(torch.zeros(5, dtype=torch.int64, device=DEV), 1.0, 1)
    g = torch.zeros(64, 64, device=DEV)
    ws = torch.zeros(2 * H.hpo_newton_schulz_workspace(64, 64), dtype=torch.uint8, device=DEV)
    with pytest.raises(ValueError, match="workspace must be contiguous"):
        H.hpo_newton_schulz(g, torch.empty_like(g), H.make_muon_cfg(), ws[::2])
    norm = torch.zeros(1, device=DEV)
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    H.hpo_grad_global_norm(hset, 1.0, norm, flag)
    torch.cuda.synchronize()
    assert norm.item() == 0.0 and flag.item() == 0
    hset.close()
