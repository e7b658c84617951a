"""GPU parity of the chained AdamW + Muon step at the full Llama-8B-shaped
size (8.03e9 parameters, 116.6 GB of state), in the configuration bench.py
times (hpo_step_device_chain, the default Muon workspace and batch plan).

The oracle cannot step the whole model, so after one device step it checks:
  * the global norm: every stored grad of both sets streamed to the host and
    summed by the oracle (binary64), against the device state's norm;
  * AdamW: sampled elements (whole norm gains, head / tail / seeded windows
    of the embedding and output head) stepped by the oracle with its own
    clip decision -- bit-exact;
  * Muon: one whole matrix of every shape class (4096 x 4096, 1024 x 4096,
    14336 x 4096 -- transposed by NS -- and 4096 x 14336), stepped by the
    oracle's bf16 NS: momentum bit-exact, master within the NS bound of
    muon_util.py (times fp32(lr * scale)), param == bf16(GPU master).
"""
import numpy as np
import pytest
import torch

from gpu_util import banner, bf16_of, oracle_sumsq_streamed, require_gpu, to_np
from muon_util import ns_tolerance

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

DEV = "cuda:0"
F32 = np.float32


@pytest.fixture(scope="module")
def H():
    return require_gpu()


def test_llama8b_chain_full_size(H):
    import oracle
    import oracle.muon as mu
    from mixed_precision_optimizer_amd import inputs
    oracle.lib()
    dev = torch.device(DEV)
    wa, mats = inputs.llama8b_chain()
    banner(f"llama8b chain: {wa.numel} AdamW + {sum(r * c for _, (r, c), _ in mats)} Muon params")
    bufs = inputs.allocate(wa, dev)
    inputs.fill_grads_(bufs, 1)
    ps, ms, gs, m1, m2 = bufs.lists()
    aset = H.hpo_set_create_list(ps, ms, gs, m1, m2, [wa.group_of(i) for i in range(wa.n_tensors)])
    mb = inputs.allocate_muon(mats, dev)
    mset = H.hpo_muon_set_create(mb.views(mb.param), mb.views(mb.master), mb.views(mb.grad), mb.views(mb.momentum))
    torch.cuda.synchronize()

    # host copies of what the oracle needs, taken before the step
    names = [n for n, _, _ in mats]
    pick = [names.index(n) for n in ("l0.q", "l0.k", "l0.gate", "l31.down")]
    W0 = {i: to_np(mb.views(mb.master)[i]) for i in pick}
    G0 = {i: to_np(mb.views(mb.grad)[i]) for i in pick}
    a_pick = [i for i in range(wa.n_tensors) if wa.ndims[i] == 1][:8] + [0, wa.n_tensors - 1]
    A0 = {}
    for i in a_pick:
        n = wa.numels[i]
        rng = [(0, min(n, 4096))] if n <= 8192 else [(0, 4096), (n // 2, n // 2 + 65536), (n - 4096, n)]
        for lo, hi in rng:
            o = bufs.offs[i]
            A0[(i, lo, hi)] = (to_np(bufs.master[o + lo:o + hi]), to_np(bufs.grad[o + lo:o + hi]))

    banner("oracle norm over all grads (streamed)")
    ranges = [(bufs.offs[i], n) for i, n in enumerate(wa.numels)] + \
        [(o, r * c) for o, (r, c) in zip(mb.offs, mb.shapes)]
    n2 = oracle_sumsq_streamed(oracle, bufs.grad, ranges[:wa.n_tensors], 1.0) + \
        oracle_sumsq_streamed(oracle, mb.grad, ranges[wa.n_tensors:], 1.0)
    norm64, norm32 = oracle.norm_from_sumsq(n2)
    do_clip, C, c64 = oracle.clip_coeff(wa.max_norm, norm32)
    assert do_clip

    banner("device chain step")
    d_state = H.new_scaler_state(dev)
    H.hpo_scaler_state_init(d_state, 1.0, 1, 0)
    H.hpo_step_device_chain(aset, H.make_cfg(), wa.groups(), mset, H.make_muon_cfg(), [(wa.lr, wa.weight_decay)],
                            wa.max_norm, H.make_scaler_cfg(dynamic=False), d_state, 1, 1)
    torch.cuda.synchronize()
    st = H.read_scaler_state(d_state)
    assert st.applied == 1 and st.applied_steps == 1 and st.error == 0
    assert abs(st.grad_norm - norm32) <= 1e-5 * norm32, (st.grad_norm, norm32)
    assert st.grad_norm == norm32

    banner("AdamW samples")
    hyper = oracle.Hyper()
    for (i, lo, hi), (th, g) in A0.items():
        T = oracle.OTensor.fresh(th, group=wa.group_of(i))
        oracle.apply_update([T], [g], hyper, wa.groups(), 1, 1.0, do_clip, C, c64)
        o = bufs.offs[i]
        assert np.array_equal(to_np(bufs.master[o + lo:o + hi]).view(np.uint32), T.theta.view(np.uint32)), (i, lo)
        assert np.array_equal(to_np(bufs.exp_avg[o + lo:o + hi]).view(np.uint32), T.m.view(np.uint32))
        assert np.array_equal(to_np(bufs.exp_avg_sq[o + lo:o + hi]).view(np.uint32), T.v.view(np.uint32))
        assert np.array_equal(to_np(bufs.param[o + lo:o + hi]), T.p)

    cfg = mu.MuonCfg()
    for i in pick:
        name, (r, c), _ = mats[i]
        banner(f"Muon {name} {r}x{c}")
        T = mu.OMatrix.fresh(W0[i])
        rec = mu.muon_matrix_step(T, G0[i], cfg, wa.lr, wa.weight_decay, 1.0, do_clip, C, "bf16")
        M = to_np(mb.views(mb.momentum)[i])
        W = to_np(mb.views(mb.master)[i])
        P = to_np(mb.views(mb.param)[i])
        assert np.array_equal(M.view(np.uint32), T.M.view(np.uint32)), f"{name}: momentum"
        assert np.array_equal(P, bf16_of(W.ravel()).reshape(r, c)), f"{name}: param != bf16(master)"
        O = rec["O"]  # the exact-sum bf16 reading; the spread needs only the fp32-sum one
        spread = np.abs(O.astype(np.float64) - mu.newton_schulz_bf16(rec["g_tilde"], acc="f32"))
        tol_max, _ = ns_tolerance(O, spread, float(np.linalg.norm(spread) / np.linalg.norm(O)))
        k2 = float(F32(wa.lr * rec["scale"]))
        bound = k2 * tol_max * (1 + 2 ** -20) + 2 * np.spacing(np.abs(T.W)).astype(np.float64)
        d = np.abs(W.astype(np.float64) - T.W)
        print(f"[muon-full] {name}: max |dW| {d.max():.3e}, bound {bound.max():.3e}", flush=True)
        assert np.all(d <= bound), f"{name}: master off by {d.max():.3e}"
    aset.close()
    mset.close()
