"""GPU parity: the HIP path through the C ABI against the CPU oracle, element
by element, on seeded inputs at sizes the oracle finishes in seconds (several
chunks plus ragged tails), plus the edge cases of the method.

The oracle runs its own trajectory from the same seeded initial state and the
same seeded grads; the GPU state is never fed back into it.
"""
import math

import numpy as np
import pytest
import torch

from gpu_util import (banner, bf16_of, compare_tensor, make_opt, make_set, read_state, require_gpu,
                      to_np)

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


def _oracle_tensors(orc, bufs):
    """Oracle copies of the seeded initial state (taken before any GPU step)."""
    w = bufs.workload
    out = []
    for i in range(w.n_tensors):
        st = read_state(bufs, i)
        T = orc.OTensor(st["theta"], st["m"], st["v"], st.get("p"), w.group_of(i), w.param_dtype == "fp16",
                        w.master_dtype == "fp16", w.state_dtype == "fp16")
        out.append(T)
    return out


def _grads_np(bufs):
    w = bufs.workload
    return [to_np(bufs.view(bufs.grad, i)) for i in range(w.n_tensors)]


def _run_parity(H, orc, w, steps=None, stats=None, inplace=False):
    from mixed_precision_optimizer_amd import inputs
    stats = {} if stats is None else stats
    bufs = inputs.allocate(w, DEV)
    hset = make_set(bufs)
    opt = make_opt(hset, w)
    Ts = _oracle_tensors(orc, bufs)
    O = orc.OracleOptimizer(Ts, orc.Hyper(w.beta1, w.beta2, w.eps, w.mode), w.groups(), max_norm=w.max_norm)
    steps = w.steps if steps is None else steps
    for k in range(1, steps + 1):
        inputs.fill_grads_(bufs, k)
        torch.cuda.synchronize()
        G = _grads_np(bufs)
        prev = [T.copy() for T in Ts]
        r = O.step(G, inv_scale=w.inv_scale())
        applied, norm, zeros = opt.step(inplace_unscale=inplace)
        assert applied == r.applied, f"step {k}: skip decision differs"
        assert opt.t == O.t
        assert zeros == r.num_zeros, f"step {k}: zero count {zeros} vs {r.num_zeros}"
        if r.num_zeros:
            stats.setdefault("zeros", []).append(r.num_zeros)
        if not r.applied:
            for i, T in enumerate(Ts):
                st = read_state(bufs, i)
                for key in ("theta", "m", "v"):
                    assert np.array_equal(st[key].view(np.uint8), getattr(T, key).view(np.uint8))
                if T.p is not None:
                    assert np.array_equal(st["p"], T.p)
            stats.setdefault("skipped", []).append(k)
            continue
        assert abs(norm - r.norm64) <= 1e-5 * r.norm64, f"step {k}: norm {norm} vs {r.norm64}"
        stats.setdefault("norm_rel", []).append(abs(norm - r.norm64) / max(r.norm64, 1e-300))
        c64 = w.max_norm / (float(np.float32(r.norm32)) + 1e-6) if r.clip_applied else 1.0
        for i, T in enumerate(Ts):
            st = read_state(bufs, i)
            lr, wd = w.groups()[T.group]
            compare_tensor(f"{w.name} step {k} tensor {i}", st, T, prev[i], G[i], inv=w.inv_scale(),
                           clip=r.clip_applied, C=r.clip_C, c64=c64, lr=lr, wd=wd, t=O.t, mode=w.mode,
                           bf16=w.param_dtype == "bf16", fp16=w.param_dtype == "fp16", stats=stats)
    hset.close()
    return stats, Ts, bufs


# ---------------------------------------------------------------------------
@pytest.mark.parametrize("mode", [0, 1])
def test_toy_two_params_both_modes(H, orc, mode):
    """The handbook's decay experiment on the GPU (fp32 params are their own
    master), every step against the oracle; final values as printed."""
    from mixed_precision_optimizer_amd import inputs
    banner(f"toy mode={mode}")
    w = inputs.toy(mode)
    stats, Ts, bufs = _run_parity(H, orc, w)
    th = to_np(bufs.master[:2])
    want = {0: ["0.361", "0.361"], 1: ["0.000", "0.889"]}[mode]
    assert [f"{x:.3f}" for x in th] == want
    print(f"bit-equal {stats['bit_equal']}/{stats['compared']}")
    assert stats["bit_equal"] == stats["compared"]


def test_two_matrices_ten_steps(H, orc):
    """8.4M params in two bf16 matrices, clip 1.0, 10 steps: every element,
    every step."""
    from mixed_precision_optimizer_amd import inputs
    banner("two matrices 4096x1024 + 1024x4096, 10 steps")
    w = inputs.two_matrices()
    stats, Ts, bufs = _run_parity(H, orc, w)
    print(f"bit-equal {stats['bit_equal']}/{stats['compared']}  norm rel {max(stats['norm_rel']):.2e}")
    assert stats["bit_equal"] >= 0.999999 * stats["compared"]


def _edge_workload(mode, loss_scale, inf_step=None, max_norm=1.0, steps=4, param_dtype="bf16",
                   state_dtype="fp32", grad_dtype="fp32", master_dtype="fp32", grad_std_scale=1.0):
    from mixed_precision_optimizer_amd.inputs import Workload
    sizes = [1, 3, 4, 5, 63, 64, 65, 255, 1023, 4095, 4096, 4097, 0, 12345, 70001, 131072, 300000, 2]
    ndims = [1 if n in (4095, 5, 63) else 2 for n in sizes]
    return Workload(f"edge_mode{mode}", sizes, ndims, lr=1e-3, weight_decay=0.1, mode=mode, max_norm=max_norm,
                    loss_scale=loss_scale, steps=steps,
                    grad_std=[1e-3 * grad_std_scale * (1 + (i % 5)) for i in range(len(sizes))],
                    inf_step=inf_step, param_dtype=param_dtype, state_dtype=state_dtype, grad_dtype=grad_dtype,
                    master_dtype=master_dtype, zero_every=97)


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("inplace", [False, True])
def test_ragged_tails_groups_scale_and_skip(H, orc, mode, inplace):
    """Ragged sizes (1 .. 300000, empty tensors, scalar tails), a no-decay
    group, loss scale 1024, clipping, and a +inf at step 2 that skips the step
    without moving t; both the fused and the pages' in-place unscale."""
    banner(f"edge mode={mode} inplace={inplace}")
    w = _edge_workload(mode, 1024.0, inf_step=2, steps=5)
    stats, Ts, bufs = _run_parity(H, orc, w, inplace=inplace)
    assert stats["skipped"] == [2]
    assert stats["bit_equal"] == stats["compared"]
    assert len(stats["zeros"]) == 4   # planted zeros in every applied step, counted bit-exactly


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("pdt,sdt", [("fp16", "fp32"), ("bf16", "bf16"), ("fp16", "bf16"), ("fp32", "bf16")])
def test_reduced_precision_variants(H, orc, mode, pdt, sdt):
    """fp16 model params (fp16 RNE write-back) and bf16 moments, on the ragged
    edge sets with loss scale 1024, clipping, a no-decay group and a skipped
    step, against the oracle's own trajectory."""
    banner(f"reduced precision: params {pdt}, moments {sdt}, mode {mode}")
    w = _edge_workload(mode, 1024.0, inf_step=3, steps=6, param_dtype=pdt, state_dtype=sdt)
    stats, Ts, bufs = _run_parity(H, orc, w)
    assert stats["skipped"] == [3]
    assert stats["bit_equal"] == stats["compared"]


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("gdt,tdt,sdt", [("bf16", "fp32", "fp32"), ("fp32", "fp16", "fp32"), ("bf16", "fp16", "fp32"),
                                         ("bf16", "fp16", "bf16"), ("fp32", "fp32", "bf16")])
@pytest.mark.parametrize("inplace", [False, True])
def test_lower_precision_grads_and_master(H, orc, mode, gdt, tdt, sdt, inplace):
    """bf16 main grads and an fp16 master under bf16 params, alone and
    together with bf16 moments, on the ragged edge sets (loss scale 1024,
    clipping, a no-decay group, a skipped step), with the fused and the
    in-place unscale, against the oracle's own trajectory."""
    banner(f"lower precision: grads {gdt}, master {tdt}, moments {sdt}, mode {mode}, inplace {inplace}")
    w = _edge_workload(mode, 1024.0, inf_step=3, steps=6, state_dtype=sdt, grad_dtype=gdt, master_dtype=tdt)
    stats, Ts, bufs = _run_parity(H, orc, w, inplace=inplace)
    assert stats["skipped"] == [3]
    assert stats["bit_equal"] == stats["compared"]


@pytest.mark.parametrize("grads", ["fp32", "bf16"])
def test_inplace_unscale_against_oracle(H, orc, grads):
    """hpo_unscale_check_inf over a ragged list (vector bodies, scalar tails,
    a misaligned view) stores the oracle's unscaled grads bit for bit, for
    inv_scale values that round (1/3) and that are exact (2^-13, 1), with
    fp32 or bf16 grads; an inf anywhere sets the flag and is kept."""
    banner(f"in-place unscale, {grads} grads")
    gdt = torch.bfloat16 if grads == "bf16" else torch.float32
    sizes = [1, 5, 4096, 70001, 3, 131075]
    rng = np.random.default_rng(17)
    for inv in (float(np.float32(1.0 / 3.0)), 2.0 ** -13, 1.0):
        buf = torch.zeros(sum(sizes) + 8, dtype=gdt, device=DEV)
        views, o = [], 1     # the first view starts one element in
        for n in sizes:
            views.append(buf[o:o + n])
            o += n + 1
        for k, v in enumerate(views):
            v.copy_(torch.from_numpy((rng.standard_normal(v.numel()) * 3e4).astype(np.float32)))
        views[3][777] = float("inf")
        before = [to_np(v) for v in views]
        ths = [torch.zeros(v.numel(), device=DEV) for v in views]
        ms = [torch.zeros(v.numel(), device=DEV) for v in views]
        vs = [torch.zeros(v.numel(), device=DEV) for v in views]
        hset = H.hpo_set_create_list(None, ths, views, ms, vs)
        flag = torch.zeros(1, dtype=torch.int32, device=DEV)
        H.hpo_unscale_check_inf(hset, inv, flag)
        torch.cuda.synchronize()
        assert int(flag.item()) == 1
        for G0, v in zip(before, views):
            want = G0.copy()
            if grads == "bf16":
                orc.unscale_inplace_bf16(want, inv)
            else:
                orc.unscale_inplace(want, inv)
            assert np.array_equal(to_np(v).view(np.uint8), want.view(np.uint8))
        hset.close()


def test_fp16_writeback_exhaustive(H, orc):
    """hpo_copy_main_to_model on an fp16 set over all 2^32 fp32 patterns against
    the oracle's fp16 RNE: bit-equal for every non-NaN input, NaN stays NaN."""
    banner("exhaustive fp16 write-back")
    step = 1 << 30
    master = torch.empty(step, dtype=torch.float32, device=DEV)
    extra = [torch.zeros(step, dtype=torch.float32, device=DEV) for _ in range(3)]
    param = torch.empty(step, dtype=torch.float16, device=DEV)
    hset = H.hpo_set_create_flat(param, master, *extra)
    base = torch.arange(step, dtype=torch.int64, device=DEV)
    for first in range(0, 1 << 32, step):
        bits = base + first
        master.view(torch.int32).copy_(torch.where(bits >= 2 ** 31, bits - 2 ** 32, bits).to(torch.int32))
        H.hpo_copy_main_to_model(hset)
        torch.cuda.synchronize()
        got = to_np(param)
        want = orc.fp16_rne_patterns(first, step)
        u = np.arange(step, dtype=np.uint32) + np.uint32(first)
        nan = (u & 0x7FFFFFFF) > 0x7F800000
        assert np.array_equal(got[~nan], want[~nan]), hex(first)
        assert np.all((got[nan] & 0x7FFF) > 0x7C00)
        print(f"  patterns {first:#x}.. ok", flush=True)
    hset.close()


def test_fp16_master_copy_exhaustive(H, orc):
    """hpo_copy_main_to_model on a set with an fp16 master and bf16 params,
    over all 65536 fp16 master patterns, with aligned arrays (vector path)
    and with views one element in (three elements on the element path, the
    rest vectorized): each param is the oracle's bf16 RNE of the widened
    master, NaN staying NaN."""
    banner("exhaustive fp16-master copy")
    n = 1 << 16
    pats = torch.arange(n, dtype=torch.int32).to(torch.int16)
    want = orc.bf16_rne(orc.widen_fp16(pats.numpy().view(np.uint16)))
    nan = (pats.numpy().view(np.uint16) & 0x7FFF) > 0x7C00
    for shift in (0, 1):
        master = torch.zeros(n + 4, dtype=torch.float16, device=DEV)
        grad = torch.zeros(n + 4, dtype=torch.float32, device=DEV)
        m, v = (torch.zeros(n + 4, dtype=torch.float32, device=DEV) for _ in range(2))
        param = torch.zeros(n + 4, dtype=torch.bfloat16, device=DEV)
        t, g, mm, vv, p = (b[shift:shift + n] for b in (master, grad, m, v, param))
        t.view(torch.int16).copy_(pats.to(DEV))
        hset = H.hpo_set_create_list([p], [t], [g], [mm], [vv])
        assert hset.info().n_vector == 1   # every array shares the shift: peeled head + vector body
        H.hpo_copy_main_to_model(hset)
        torch.cuda.synchronize()
        got = to_np(p)
        assert np.array_equal(got[~nan], want[~nan]), shift
        assert np.all((got[nan] & 0x7FFF) > 0x7F80)
        hset.close()


@pytest.mark.parametrize("bad", [float("inf"), float("-inf"), float("nan")])
@pytest.mark.parametrize("where", ["head", "middle", "tail"])
def test_nonfinite_anywhere_skips(H, orc, bad, where):
    from mixed_precision_optimizer_amd import inputs
    banner(f"nonfinite {bad} at {where}")
    w = _edge_workload(0, None, steps=1)
    bufs = inputs.allocate(w, DEV)
    inputs.fill_grads_(bufs, 1)
    i = {"head": 0, "middle": 13, "tail": len(w.numels) - 2}[where]
    e = {"head": 0, "middle": w.numels[i] // 2, "tail": w.numels[i] - 1}[where]
    bufs.grad[bufs.offs[i] + e] = bad
    before = {k: v.clone() for k, v in (("m", bufs.master), ("a", bufs.exp_avg), ("b", bufs.exp_avg_sq),
                                       ("p", bufs.param))}
    hset = make_set(bufs)
    opt = make_opt(hset, w)
    applied, norm, zeros = opt.step()
    assert applied is False and opt.t == 0 and norm is None and zeros is None
    assert int(opt.found_inf.item()) == 1
    for k, t in (("m", bufs.master), ("a", bufs.exp_avg), ("b", bufs.exp_avg_sq), ("p", bufs.param)):
        assert torch.equal(before[k].view(torch.int16) if k == "p" else before[k].view(torch.int32),
                           t.view(torch.int16) if k == "p" else t.view(torch.int32))
    hset.close()


def test_norm_matches_oracle_and_is_deterministic(H, orc):
    from mixed_precision_optimizer_amd import inputs
    banner("norm")
    w = _edge_workload(0, 65536.0, steps=1)
    bufs = inputs.allocate(w, DEV)
    inputs.fill_grads_(bufs, 1)
    hset = make_set(bufs)
    norm = torch.zeros(1, dtype=torch.float32, device=DEV)
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    H.hpo_grad_global_norm(hset, float(np.float32(1 / 65536)), norm, flag)
    torch.cuda.synchronize()
    G = [to_np(bufs.view(bufs.grad, i)) for i in range(w.n_tensors)]
    n2 = sum(orc.sumsq(g, float(np.float32(1 / 65536))) for g in G if g.size)
    assert abs(norm.item() - math.sqrt(n2)) <= 1e-5 * math.sqrt(n2)
    assert norm.item() == float(np.float32(math.sqrt(n2)))  # same fp32 rounding of the same sum
    assert flag.item() == 0
    vals = set()
    for _ in range(5):
        H.hpo_grad_global_norm(hset, float(np.float32(1 / 65536)), norm, None)
        vals.add(norm.item())
    assert len(vals) == 1
    hset.close()


def test_norm_over_several_sets(H, orc):
    """hpo_grad_global_norm_sets over four sets of the four kinds (list, flat,
    flat with param ranges, Muon): one norm over every stored grad of all of
    them, unscaled ([OPT-INFRA] §11.4), equal to the fp32 rounding of the
    oracle's binary64 sum; repeated calls give the same bits, the sets in
    reverse order differ at most by the order of four binary64 partials; a
    non-finite grad in any one set raises the flag; a set given twice and a
    fifth set are refused."""
    banner("norm over several sets")
    rng = np.random.default_rng(11)
    inv = float(np.float32(1 / 1024))
    draw = lambda shape: torch.from_numpy((rng.standard_normal(shape) * 1024 * 1e-2).astype(np.float32)).to(DEV)
    zeros = lambda t: torch.zeros_like(t)
    lsizes = [5000, 1, 70_001]
    lg = [draw(n) for n in lsizes]
    lt = [torch.zeros(n, device=DEV) for n in lsizes]
    s_list = H.hpo_set_create_list([t.to(torch.bfloat16) for t in lt], lt, lg, [zeros(t) for t in lt],
                                   [zeros(t) for t in lt], [0, 1, 0])
    fg = draw(300_007)
    ft = zeros(fg)
    s_flat = H.hpo_set_create_flat(ft.to(torch.bfloat16), ft, fg, zeros(ft), zeros(ft))
    rg = draw(100_000)
    rt = zeros(rg)
    s_rng = H.hpo_set_create_flat_ranges(rt.to(torch.bfloat16), rt, rg, zeros(rt), zeros(rt), [0, 4096, 50_000],
                                         [0, 1, 0])
    mshapes = [(64, 300), (300, 64)]
    mg = [draw(s) for s in mshapes]
    mm = [torch.zeros(s, device=DEV) for s in mshapes]
    s_mu = H.hpo_muon_set_create([m.to(torch.bfloat16) for m in mm], mm, mg, [zeros(m) for m in mm])
    sets = [s_list, s_flat, s_rng, s_mu]
    grads = lg + [fg, rg] + mg
    n2 = sum(orc.sumsq(to_np(g).ravel(), inv) for g in grads)
    norm = torch.zeros(1, device=DEV)
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    H.hpo_grad_global_norm_sets(sets, inv, norm, flag)
    torch.cuda.synchronize()
    assert flag.item() == 0
    first = norm.item()
    assert first == float(np.float32(math.sqrt(n2))), (first, math.sqrt(n2))
    for _ in range(3):
        H.hpo_grad_global_norm_sets(sets, inv, norm, None)
    torch.cuda.synchronize()
    assert norm.item() == first
    H.hpo_grad_global_norm_sets(sets[::-1], inv, norm, None)
    torch.cuda.synchronize()
    assert abs(norm.item() - first) <= float(np.spacing(np.float32(first)))
    for k, g in enumerate([lg[2], fg, rg, mg[1]]):
        flat = g.view(-1)
        keep = flat[7].item()
        flat[7] = float("nan") if k % 2 else float("inf")
        flag.zero_()
        H.hpo_grad_global_norm_sets(sets, inv, norm, flag)
        torch.cuda.synchronize()
        assert flag.item() == 1, f"set {k}: non-finite grad not flagged"
        flat[7] = keep
    with pytest.raises(H.HpoError, match="twice"):
        H.hpo_grad_global_norm_sets([s_list, s_flat, s_list], inv, norm, None)
    with pytest.raises(H.HpoError):
        H.hpo_grad_global_norm_sets(sets + [s_list], inv, norm, None)
    for s in sets:
        s.close()


def test_norm_paths_agree_across_the_two_stage_boundary(H, orc):
    """The single-set norm call, the multi-set call on that one set and the
    device step's finalize give the same norm, zero count and flag bits,
    call after call, on both sides of the 8192-workgroup boundary where the
    finalize takes a second stage; the count equals torch's own count of
    zero grads."""
    banner("norm paths across the two-stage boundary")
    rng = np.random.default_rng(19)
    inv = float(np.float32(1 / 1024))
    for n in (1, 4097, 3_000_001, 8192 * 65536, 8192 * 65536 + 3 * 65536):
        g = torch.randn(n, device=DEV).mul_(1e-2 * 1024)
        g[::97] = 0.0
        t = torch.zeros(n, device=DEV)
        hset = H.hpo_set_create_flat(None, t, g, torch.zeros_like(t), torch.zeros_like(t))
        parts = hset.info().n_grad_parts
        out = torch.zeros(4, dtype=torch.int32, device=DEV)
        ref = torch.zeros(4, dtype=torch.int32, device=DEV)
        norm, flag, zeros = out[0:1].view(torch.float32), out[1:2], out[2:4].view(torch.int64)
        rnorm, rflag, rzeros = ref[0:1].view(torch.float32), ref[1:2], ref[2:4].view(torch.int64)
        H.hpo_grad_global_norm_sets([hset], inv, rnorm, rflag, rzeros)
        for rep in range(3):
            out.zero_()
            H.hpo_grad_global_norm(hset, inv, norm, flag, zeros)
            torch.cuda.synchronize()
            assert torch.equal(out, ref), (n, parts, rep, out.tolist(), ref.tolist())
        assert int(zeros.item()) == int((g == 0).sum().item()), (n, zeros.item())   # torch's own count
        if n < 10_000:
            want = orc.sumsq(to_np(g), inv)
            assert norm.item() == float(np.float32(math.sqrt(want)))
        # a non-finite grad: the folded flag, the norm of the check pass
        g[n // 2] = float("inf")
        out.zero_()
        H.hpo_grad_global_norm(hset, inv, norm, flag, zeros)
        f2 = torch.zeros(1, dtype=torch.int32, device=DEV)
        H.hpo_unscale_check_inf(hset, 1.0, f2)
        torch.cuda.synchronize()
        assert flag.item() == 1 and f2.item() == 1 and not math.isfinite(norm.item()), n
        g[n // 2] = 0.0
        # the device step's folded finalize writes the same norm and count into the state
        d_state = H.new_scaler_state()
        H.hpo_scaler_state_init(d_state, 1024.0, 1)
        H.hpo_step_device(hset, H.make_cfg(), [(1e-3, 0.1)], None, 1.0, H.make_scaler_cfg(dynamic=False), d_state,
                          1, 1)
        st = H.read_scaler_state(d_state)
        assert st.applied == 1 and st.applied_steps == 1 and st.error == 0
        d_norm = torch.zeros(1, device=DEV)
        d_zeros = torch.zeros(1, dtype=torch.int64, device=DEV)
        H.hpo_grad_global_norm_sets([hset], inv, d_norm, None, d_zeros)   # the grads as the step saw them
        torch.cuda.synchronize()
        assert st.grad_norm == d_norm.item() and st.num_zeros == int(d_zeros.item())
        assert st.step_inv_scale == inv and st.inv_scale == inv
        print(f"[norm paths] n={n} workgroups={parts} norm={rnorm.item()} zeros={int(rzeros.item())}", flush=True)
        hset.close()
        del g, t
        torch.cuda.empty_cache()


def test_norm_calls_agree_call_after_call(H):
    """The single-set norm call and the multi-set call on that set, 300 times
    each, with the grads rescaled, given an inf or a zero in between on the
    same stream and no host synchronisation: norm, zero count and flag are
    bit-identical every time, and the flag is set exactly on the calls that
    saw an inf (a partial left over from an earlier call would show as a
    difference).  List and flat sets, fp32 and bf16 grads, and 1 to 8192
    grad-pass workgroups (the most that one finalize stage folds)."""
    banner("norm calls, 300 per set")
    inv = float(np.float32(1 / 512))
    cases = [("list two 4096x1024", [4096 * 1024, 1024 * 4096], torch.float32),
             ("flat 8192 workgroups", [8192 * 65536], torch.float32),
             ("flat one workgroup", [3000], torch.float32),
             ("list ragged bf16 grads", [1_000_003, 77, 65536 * 5 + 1], torch.bfloat16)]
    for name, sizes, gdt in cases:
        gen = torch.Generator(device=DEV).manual_seed(23)
        grads = [torch.randn(n, device=DEV, generator=gen).mul_(1e-2).to(gdt) for n in sizes]
        for g in grads:
            g[::89] = 0
        masters = [torch.zeros(n, device=DEV) for n in sizes]
        m1 = [torch.zeros(n, device=DEV) for n in sizes]
        m2 = [torch.zeros(n, device=DEV) for n in sizes]
        if len(sizes) == 1 and gdt == torch.float32:
            hset = H.hpo_set_create_flat(None, masters[0], grads[0], m1[0], m2[0])
        else:   # the grads' dtype selects bf16 grads
            hset = H.hpo_set_create_list([None] * len(sizes), masters, grads, m1, m2, [0] * len(sizes),
                                         param_dtype=H.HPO_PARAM_FP32)
        parts = hset.info().n_grad_parts
        calls = 300
        got = torch.zeros(calls, 4, dtype=torch.int32, device=DEV)
        ref = torch.zeros(calls, 4, dtype=torch.int32, device=DEV)
        for k in range(calls):
            if k % 7 == 3:
                grads[k % len(grads)][(k * 131) % sizes[k % len(grads)]] = float("inf")
            elif k % 7 == 4:
                grads[(k - 1) % len(grads)][((k - 1) * 131) % sizes[(k - 1) % len(grads)]] = 0.0
            else:
                for g in grads:
                    g.mul_(1.0 + (k % 5) / 64.0)
            for out, call in ((got[k], "one"), (ref[k], "sets")):
                norm, flag, zeros = out[0:1].view(torch.float32), out[1:2], out[2:4].view(torch.int64)
                if call == "one":
                    H.hpo_grad_global_norm(hset, inv, norm, flag, zeros)
                else:
                    H.hpo_grad_global_norm_sets([hset], inv, norm, flag, zeros)
        torch.cuda.synchronize()
        bad = (got != ref).any(dim=1).nonzero().flatten().tolist()
        print(f"[norm calls] {name}: {parts} workgroups, {calls} calls, mismatches {len(bad)}", flush=True)
        assert not bad, (name, bad[:5], got[bad[0]].tolist(), ref[bad[0]].tolist())
        assert int(got[:, 1].sum().item()) == sum(1 for k in range(calls) if k % 7 == 3)
        hset.close()
        del grads, masters, m1, m2
        torch.cuda.empty_cache()


def test_cached_and_streaming_updates_agree(H):
    """A set whose arrays take at most 192 MiB takes cached loads and stores in
    the update; a larger one takes streaming ones.  The same 12M elements
    stepped as one flat set (216 MB: streaming) and as two flat sets of half
    the size over the same storage (108 MB each: cached) end bit-identical
    over three steps (no clip, so that the two norm folds do not enter)."""
    banner("cached vs streaming update accesses")
    n = 12 * 1024 * 1024
    gen = torch.Generator(device=DEV).manual_seed(31)
    th0 = torch.randn(n, device=DEV, generator=gen)
    grads = [torch.randn(n, device=DEV, generator=gen).mul_(1e-3) for _ in range(3)]
    cfg = H.make_cfg()
    groups, ng = H.make_groups([(1e-3, 0.1)])
    out = {}
    for kind in ("one", "halves"):
        th = th0.clone()
        p = th.to(torch.bfloat16)
        g = torch.zeros(n, device=DEV)
        m = torch.zeros(n, device=DEV)
        v = torch.zeros(n, device=DEV)
        if kind == "one":
            sets = [H.hpo_set_create_flat(p, th, g, m, v)]
        else:
            h = n // 2
            sets = [H.hpo_set_create_flat(p[a:a + h], th[a:a + h], g[a:a + h], m[a:a + h], v[a:a + h])
                    for a in (0, h)]
        for k in range(3):
            g.copy_(grads[k])
            for hs in sets:
                H.hpo_adamw_step(hs, cfg, groups, ng, k + 1, 1.0, 0.0, None, None)
        torch.cuda.synchronize()
        out[kind] = (th.clone(), m.clone(), v.clone(), p.clone())
        for hs in sets:
            hs.close()
    a, b = out["one"], out["halves"]
    assert not torch.equal(a[0], th0)   # the steps moved the master
    for x, y, name in zip(a, b, ("master", "exp_avg", "exp_avg_sq", "param")):
        assert torch.equal(x.view(torch.int16 if x.dtype == torch.bfloat16 else torch.int32),
                           y.view(torch.int16 if y.dtype == torch.bfloat16 else torch.int32)), name


def test_zero_count_is_taken_before_the_clip(H, orc):
    """R40 on the GPU: one grad of 1e15 sets the clip coefficient near 1e-15,
    which would round the stored subnormals to zero; the host-driven and the
    device-resident steps both count only the true zeros, as the oracle."""
    banner("zero count before the clip")
    n = 5000
    g = torch.full((n,), 2.0 ** -133, device=DEV)
    g[0] = 1e15
    g[1234::1000] = 0.0
    want = int((g == 0).sum().item())
    assert want == 4 and orc.count_zeros(to_np(g), 1.0) == want
    for kind in ("host", "device"):
        th = torch.linspace(-1, 1, n, device=DEV)
        p = th.to(torch.bfloat16)
        m, v = torch.zeros(n, device=DEV), torch.zeros(n, device=DEV)
        hset = H.hpo_set_create_flat(p, th, g.clone(), m, v)
        if kind == "host":
            from mixed_precision_optimizer_amd import MixedPrecisionAdamW
            opt = MixedPrecisionAdamW(hset, [(1e-3, 0.1)], max_norm=1.0, log_num_zeros_in_grad=True)
            applied, norm, zeros = opt.step()
            assert applied and zeros == want, (applied, zeros)
        else:
            d_state = H.new_scaler_state()
            H.hpo_scaler_state_init(d_state, 1.0, 1)
            H.hpo_step_device(hset, H.make_cfg(), [(1e-3, 0.1)], None, 1.0, H.make_scaler_cfg(dynamic=False),
                              d_state, 1, 1)
            st = H.read_scaler_state(d_state)
            assert st.applied == 1 and st.num_zeros == want, (st.applied, st.num_zeros)
        hset.close()


def test_empty_set_and_zero_sizes(H):
    banner("empty set")
    hset = H.hpo_set_create_list([], [], [], [], [], param_dtype=H.HPO_PARAM_BF16)
    norm = torch.full((1,), 7.0, device=DEV)
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    H.hpo_grad_global_norm(hset, 1.0, norm, flag)
    H.hpo_adamw_step(hset, H.make_cfg(), [(1e-3, 0.1)], None, 1, 1.0, 1.0, norm, flag)
    H.hpo_unscale_check_inf(hset, 0.5, flag)
    torch.cuda.synchronize()
    assert norm.item() == 0.0 and flag.item() == 0
    info = hset.info()
    assert info.n_tensors == 0 and info.numel == 0 and info.n_chunks == 0
    hset.close()


def test_device_flag_skips_the_update(H):
    banner("device-side skip")
    n = 100_003
    th = torch.randn(n, device=DEV)
    p = th.to(torch.bfloat16)
    g = torch.randn(n, device=DEV) * 1e-3
    m = torch.zeros(n, device=DEV)
    v = torch.zeros(n, device=DEV)
    th0, p0 = th.clone(), p.clone()
    hset = H.hpo_set_create_flat(p, th, g, m, v)
    flag = torch.ones(1, dtype=torch.int32, device=DEV)
    H.hpo_adamw_step(hset, H.make_cfg(), [(1e-3, 0.1)], None, 1, 1.0, 0.0, None, flag)
    torch.cuda.synchronize()
    assert torch.equal(th, th0) and torch.equal(p, p0) and not m.any() and not v.any()
    flag.zero_()
    H.hpo_adamw_step(hset, H.make_cfg(), [(1e-3, 0.1)], None, 1, 1.0, 0.0, None, flag)
    torch.cuda.synchronize()
    assert not torch.equal(th, th0)
    hset.close()


def test_flat_and_list_sets_agree_bitwise(H):
    banner("flat vs list")
    n = 1_000_001
    gen = torch.Generator(device=DEV).manual_seed(5)
    base = torch.randn(n, device=DEV, generator=gen)
    g = torch.randn(n, device=DEV, generator=gen) * 1e-2
    outs = []
    for kind in ("flat", "list"):
        th = base.clone()
        p = th.to(torch.bfloat16)
        m = torch.zeros(n, device=DEV)
        v = torch.zeros(n, device=DEV)
        if kind == "flat":
            hset = H.hpo_set_create_flat(p, th, g, m, v)
        else:
            hset = H.hpo_set_create_list([p], [th], [g], [m], [v])
        norm = torch.zeros(1, device=DEV)
        for t in (1, 2, 3):
            H.hpo_grad_global_norm(hset, 1.0, norm, None)
            H.hpo_adamw_step(hset, H.make_cfg(), [(1e-3, 0.1)], None, t, 1.0, 1.0, norm, None)
        torch.cuda.synchronize()
        outs.append((th.clone(), m.clone(), v.clone(), p.clone(), norm.item()))
        hset.close()
    for a, b in zip(outs[0], outs[1]):
        if isinstance(a, float):
            assert a == b
        else:
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))


@pytest.mark.parametrize("moments,param,grads,master", [("fp32", "bf16", "fp32", "fp32"), ("bf16", "bf16", "fp32", "fp32"),
                                                        ("bf16", "fp16", "fp32", "fp32"), ("fp32", "bf16", "bf16", "fp32"),
                                                        ("fp32", "bf16", "fp32", "fp16"), ("bf16", "bf16", "bf16", "fp16")])
def test_misaligned_tensors_peel_or_go_scalar(H, orc, moments, param, grads, master):
    """Views that start 1..3 elements into their buffers, as a list set and
    as a flat set: when all five pointers share the element offset (for
    16-bit moments and params, the offset within their own 4-element lines),
    the head is peeled and the body vectorized; when they do not, the whole
    tensor runs element by element.  Every layout and kind gives the same
    bits, and the oracle's, for fp32 or bf16 moments, bf16 or fp16 params,
    fp32 or bf16 grads and an fp32 or fp16 master."""
    banner(f"misaligned, {moments} moments, {param} params, {grads} grads, {master} master")
    n = 50_001
    rng = np.random.default_rng(6)
    th0 = rng.standard_normal(n).astype(np.float32)
    G = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    mdt = {"fp32": torch.float32, "bf16": torch.bfloat16}[moments]
    pdt = torch.float16 if param == "fp16" else torch.bfloat16
    tdt = torch.float16 if master == "fp16" else torch.float32
    gdt = torch.bfloat16 if grads == "bf16" else torch.float32
    res = []
    layouts = [(0, 0), (1, 1), (2, 2), (3, 3), (1, 2), (0, 3)]  # (shift of master/m/v/param, shift of grad)
    for (shift, gshift), kind in [(lay, kind) for lay in layouts for kind in ("list", "flat")]:
        tb = torch.zeros(n + 4, dtype=tdt, device=DEV)
        gb = torch.zeros(n + 4, dtype=gdt, device=DEV)
        mb, vb = (torch.zeros(n + 4, dtype=mdt, device=DEV) for _ in range(2))
        pb = torch.zeros(n + 4, dtype=pdt, device=DEV)
        th, m, v, p = (b[shift:shift + n] for b in (tb, mb, vb, pb))
        g = gb[gshift:gshift + n]
        th.copy_(torch.from_numpy(th0))
        g.copy_(torch.from_numpy(G))
        if kind == "list":
            hset = H.hpo_set_create_list([p], [th], [g], [m], [v])
        else:   # a flat range off the vector lines is planned as table pieces, still a flat set
            hset = H.hpo_set_create_flat(p, th, g, m, v)
            assert hset.info().is_flat == 1
        assert hset.info().n_vector == (1 if shift == gshift else 0), (shift, gshift, kind)
        norm = torch.zeros(1, device=DEV)
        H.hpo_grad_global_norm(hset, 1.0, norm, None)
        H.hpo_adamw_step(hset, H.make_cfg(mode=1), [(1e-3, 0.1)], None, 1, 1.0, 1.0, norm, None)
        torch.cuda.synchronize()
        res.append((to_np(th), to_np(m), to_np(v), to_np(p)))
        G_stored = to_np(g)     # bf16 grads: the patterns the set read
        hset.close()
    for r in res[1:]:
        for a, b in zip(res[0], r):
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
    T = orc.OTensor.fresh(th0, fp16_param=param == "fp16", state_bf16=moments == "bf16",
                          fp16_master=master == "fp16")
    orc.OracleOptimizer([T], orc.Hyper(mode=1), [(1e-3, 0.1)], max_norm=1.0).step([G_stored])
    for got, want in zip(res[0], (T.theta, T.m, T.v, T.p)):
        assert np.array_equal(got.view(np.uint8), want.view(np.uint8))


def _mini_model_layout():
    """(sizes, ndims) of a small Llama-like model and the 64-element-aligned
    start of each param in one flat buffer (the DDP buffer layout)."""
    h, f, vocab, layers = 512, 1792, 3000, 3
    shapes = [(vocab, h)]
    for _ in range(layers):
        shapes += [(h, h), (128, h), (128, h), (h, h), (f, h), (f, h), (h, f), (h,), (h,)]
    shapes += [(h,), (vocab, h)]
    sizes = [int(np.prod(s)) for s in shapes]
    ndims = [len(s) for s in shapes]
    from mixed_precision_optimizer_amd.inputs import offsets
    offs, total = offsets(sizes)
    return sizes, ndims, offs, total


def _cuts():
    sizes, ndims, offs, total = _mini_model_layout()
    first_norm = next(o for o, d in zip(offs, ndims) if d == 1)
    return [0, 1_530_001, first_norm - 1001]


@pytest.mark.parametrize("cut", _cuts())
def test_flat_shard_with_param_ranges(H, orc, cut):
    """One data-parallel rank's slice of a flat param buffer, cut at an
    arbitrary element: the ranges of 1-D params take no weight decay.  Checked
    against the oracle (range by range, with its group) and bit for bit
    against the same ranges given as a list set."""
    banner(f"flat shard with ranges, cut at {cut}")
    sizes, ndims, offs, total = _mini_model_layout()
    shard_len = min(6_000_000, total - cut)
    lo, hi = cut, cut + shard_len
    starts, groups = [], []
    for n, d, o in zip(sizes, ndims, offs):
        a, b = max(o, lo), min(o + n, hi)
        if a < b:
            starts.append(a - lo)
            groups.append(1 if d == 1 else 0)
        # the 64-element padding after a param belongs to no param: give it the
        # preceding param's group (its grads are zero, it is stepped harmlessly)
    merged_s, merged_g = [], []
    for s_, g_ in zip(starts, groups):
        if merged_g and merged_g[-1] == g_:
            continue
        merged_s.append(s_)
        merged_g.append(g_)
    if merged_s[0] != 0:
        merged_s[0] = 0
    rng = np.random.default_rng(80 + cut)
    th0 = rng.standard_normal(shard_len).astype(np.float32)
    groups_lrwd = [(1e-3, 0.1), (1e-3, 0.0)]
    bounds = merged_s[1:] + [shard_len]
    results = {}
    for kind in ("ranges", "list"):
        th = torch.from_numpy(th0.copy()).to(DEV)
        p = th.to(torch.bfloat16)
        g = torch.zeros(shard_len, device=DEV)
        m = torch.zeros(shard_len, device=DEV)
        v = torch.zeros(shard_len, device=DEV)
        if kind == "ranges":
            hset = H.hpo_set_create_flat_ranges(p, th, g, m, v, merged_s, merged_g)
        else:
            views = lambda t: [t[a:b] for a, b in zip(merged_s, bounds)]
            hset = H.hpo_set_create_list(views(p), views(th), views(g), views(m), views(v), merged_g)
        from mixed_precision_optimizer_amd import MixedPrecisionAdamW
        opt = MixedPrecisionAdamW(hset, groups_lrwd, max_norm=1.0, loss_scale=1024.0)
        grng = np.random.default_rng(90 + cut)
        states = []
        for k in range(3):
            G = (grng.standard_normal(shard_len) * 1e-3 * 1024).astype(np.float32)
            g.copy_(torch.from_numpy(G))
            applied, norm, _ = opt.step()
            assert applied
            states.append((to_np(th), to_np(m), to_np(v), to_np(p), norm))
        results[kind] = states
        hset.close()
    for a, b in zip(results["ranges"], results["list"]):
        for x, y in zip(a[:4], b[:4]):
            assert np.array_equal(x.view(np.uint8), y.view(np.uint8))
        assert a[4] == b[4]
    # oracle: one OTensor per range with its group, the same grads, every step
    Ts = [orc.OTensor.fresh(th0[a:b], group=gid) for a, b, gid in zip(merged_s, bounds, merged_g)]
    O = orc.OracleOptimizer(Ts, orc.Hyper(), groups_lrwd, max_norm=1.0)
    grng = np.random.default_rng(90 + cut)
    for k in range(3):
        G = (grng.standard_normal(shard_len) * 1e-3 * 1024).astype(np.float32)
        r = O.step([np.ascontiguousarray(G[a:b]) for a, b in zip(merged_s, bounds)],
                   inv_scale=float(np.float32(1 / 1024)))
        th_g, m_g, v_g, p_g, norm = results["ranges"][k]
        assert abs(norm - r.norm64) <= 1e-5 * r.norm64
        for got, key in ((th_g, "theta"), (m_g, "m"), (v_g, "v")):
            want = np.concatenate([getattr(T, key) for T in Ts])
            assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), (k, key)
        assert np.array_equal(p_g, np.concatenate([T.p for T in Ts]))
    # the no-decay ranges really took no decay: with wd = 0 they differ from a decayed step
    assert len(set(merged_g)) == 2


def test_fp32_param_set_has_no_writeback(H, orc):
    banner("fp32 params")
    n = 77_777
    rng = np.random.default_rng(7)
    th0 = rng.standard_normal(n).astype(np.float32)
    G = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    th = torch.from_numpy(th0).to(DEV)
    g = torch.from_numpy(G).to(DEV)
    m = torch.zeros(n, device=DEV)
    v = torch.zeros(n, device=DEV)
    hset = H.hpo_set_create_list([th], [th], [g], [m], [v])  # the param is its own master
    assert hset.info().param_dtype == H.HPO_PARAM_FP32
    norm = torch.zeros(1, device=DEV)
    H.hpo_grad_global_norm(hset, 1.0, norm, None)
    H.hpo_adamw_step(hset, H.make_cfg(), [(1e-3, 0.1)], None, 1, 1.0, 1.0, norm, None)
    H.hpo_copy_main_to_model(hset)  # no-op for fp32 sets
    torch.cuda.synchronize()
    T = orc.OTensor.fresh(th0, bf16_param=False)
    orc.OracleOptimizer([T], orc.Hyper(), [(1e-3, 0.1)], max_norm=1.0).step([G])
    assert np.array_equal(to_np(th).view(np.uint32), T.theta.view(np.uint32))
    with pytest.raises(H.HpoError) as e:
        H.hpo_set_create_list([th.clone()], [th], [g], [m], [v], param_dtype=H.HPO_PARAM_FP32)
    assert e.value.status == H.HPO_EINVAL
    hset.close()


def test_unsupported_param_dtype_is_rejected(H):
    n = 64
    th = torch.zeros(n, device=DEV)
    with pytest.raises(H.HpoError) as e:
        H.hpo_set_create_flat(th.double(), th, th.clone(), th.clone(), th.clone())
    assert e.value.status == H.HPO_EDTYPE
    with pytest.raises(TypeError):  # mixed moment dtypes are refused before the call
        H.hpo_set_create_flat(th.to(torch.bfloat16), th, th.clone(), th.to(torch.bfloat16), th.clone())


def test_bf16_writeback_exhaustive(H, orc):
    """hpo_copy_main_to_model over all 2^32 fp32 bit patterns against the
    oracle's RNE: bit-equal for every non-NaN input, NaN stays NaN."""
    banner("exhaustive bf16 write-back")
    step = 1 << 30
    hset = None
    master = torch.empty(step, dtype=torch.float32, device=DEV)
    extra = [torch.zeros(step, dtype=torch.float32, device=DEV) for _ in range(3)]
    param = torch.empty(step, dtype=torch.bfloat16, device=DEV)
    hset = H.hpo_set_create_flat(param, master, *extra)
    base = torch.arange(step, dtype=torch.int64, device=DEV)
    for first in range(0, 1 << 32, step):
        bits = (base + first).to(torch.int64)
        master.view(torch.int32).copy_(torch.where(bits >= 2 ** 31, bits - 2 ** 32, bits).to(torch.int32))
        H.hpo_copy_main_to_model(hset)
        torch.cuda.synchronize()
        got = to_np(param)
        want = orc.bf16_rne_patterns(first, step)
        u = np.arange(step, dtype=np.uint32) + np.uint32(first)
        nan = (u & 0x7FFFFFFF) > 0x7F800000
        assert np.array_equal(got[~nan], want[~nan]), hex(first)
        assert np.all((got[nan] & 0x7FFF) > 0x7F80)
        print(f"  patterns {first:#x}.. ok", flush=True)
    hset.close()


# ---------------------------------------------------------------------------
# degenerate cases of the method, each against the oracle element by element
# ---------------------------------------------------------------------------
def _one_shot(H, orc, th0, G, *, mode=0, lr=1e-3, wd=0.1, b1=0.9, b2=0.999, eps=1e-8, t=1, inv=1.0,
              max_norm=0.0, m0=None, v0=None):
    """One step on the GPU (list set of one tensor) and in the oracle from the
    same state; returns both states."""
    n = th0.size
    m0 = np.zeros(n, np.float32) if m0 is None else m0
    v0 = np.zeros(n, np.float32) if v0 is None else v0
    th = torch.from_numpy(th0.copy()).to(DEV)
    p = torch.from_numpy(orc.bf16_rne(th0).view(np.int16)).to(DEV).view(torch.bfloat16)
    g = torch.from_numpy(G.copy()).to(DEV)
    m = torch.from_numpy(m0.copy()).to(DEV)
    v = torch.from_numpy(v0.copy()).to(DEV)
    hset = H.hpo_set_create_list([p], [th], [g], [m], [v])
    norm = torch.zeros(1, device=DEV)
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    H.hpo_grad_global_norm(hset, inv, norm, flag)
    H.hpo_adamw_step(hset, H.make_cfg(b1, b2, eps, mode), [(lr, wd)], None, t, inv, max_norm, norm, None)
    torch.cuda.synchronize()
    gpu = {"theta": to_np(th), "m": to_np(m), "v": to_np(v), "p": to_np(p), "norm": norm.item(),
           "flag": flag.item()}
    hset.close()
    T = orc.OTensor(th0.copy(), m0.copy(), v0.copy(), orc.bf16_rne(th0))
    r = orc.oracle_step([T], [G], orc.Hyper(b1, b2, eps, mode), [(lr, wd)], t, inv, max_norm)
    return gpu, T, r


def _same_bits(a, b):
    """Bit-equal, except that NaNs only need to agree as NaNs (their payload
    is not fixed by the pages)."""
    a = np.asarray(a)
    b = np.asarray(b)
    if a.dtype == np.uint16:
        an = (a & 0x7FFF) > 0x7F80
        bn = (b & 0x7FFF) > 0x7F80
    else:
        an, bn = np.isnan(a), np.isnan(b)
    assert np.array_equal(an, bn)
    assert np.array_equal(a[~an].view(np.uint8) if a.dtype != np.uint16 else a[~an],
                          b[~bn].view(np.uint8) if b.dtype != np.uint16 else b[~bn])


def _check_same(gpu, T):
    for key in ("theta", "m", "v", "p"):
        _same_bits(gpu[key], getattr(T, key))


@pytest.mark.parametrize("mode", [0, 1])
def test_degenerate_hyperparameters(H, orc, mode):
    banner(f"degenerate hyperparameters mode={mode}")
    rng = np.random.default_rng(70)
    n = 40_000
    th0 = rng.standard_normal(n).astype(np.float32)
    G = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    G[:100] = 0.0
    m0 = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    v0 = ((rng.standard_normal(n) * 1e-3) ** 2).astype(np.float32)
    cases = [dict(b1=0.0, b2=0.0, t=3), dict(eps=0.0, t=1), dict(t=1_000_000, m0=m0, v0=v0),
             dict(lr=0.0, t=2, m0=m0, v0=v0), dict(wd=0.0, t=5, m0=m0, v0=v0), dict(b1=0.5, b2=0.5, t=2, m0=m0, v0=v0)]
    for kw in cases:
        gpu, T, r = _one_shot(H, orc, th0, G, mode=mode, **kw)
        _check_same(gpu, T)
        if kw.get("eps") == 0.0 and mode == 0:
            # zero grad, eps = 0: 0 / (sqrt(0) + 0) -- the method itself yields NaN
            # (in the L2 mode the grad is wd * theta, not zero)
            assert np.isnan(T.theta[:100]).all()


def test_extreme_values(H, orc):
    """Huge grads (g^2 overflows fp32 in v), subnormal grads and masters,
    masters near the bf16 overflow boundary, zeros of both signs."""
    banner("extreme values")
    fmax = np.finfo(np.float32).max
    th0 = np.array([1.0, -1.0, 1e-40, -1e-40, 0.0, -0.0, fmax, -fmax, 3.3e38, 1e30, 2.0 ** -126, 5.0], np.float32)
    G = np.array([1e30, -1e30, 1e-40, -1e-44, 0.0, -0.0, 1.0, -1.0, 1e-3, 1e20, 2.0 ** -130, 3e38], np.float32)
    for mode in (0, 1):
        for max_norm in (0.0, 1.0):
            gpu, T, r = _one_shot(H, orc, th0, G, mode=mode, max_norm=max_norm)
            _check_same(gpu, T)


def test_clip_boundary_and_disabled(H, orc):
    """The norm sits exactly at max_norm (the strict '< 1' test with the 1e-6
    guard still clips by 1/(1+1e-6)); max_norm <= 0 disables clipping."""
    banner("clip boundary")
    G = np.zeros(4096, np.float32)
    G[0], G[1] = 0.6, 0.8  # norm 1.0 (up to fp32 rounding of the operands)
    th0 = np.linspace(-1, 1, 4096, dtype=np.float32)
    for max_norm in (1.0, float(np.float32(np.sqrt(np.float32(0.6) ** 2 + np.float32(0.8) ** 2))), 0.0, -5.0, 1e9):
        gpu, T, r = _one_shot(H, orc, th0, G, max_norm=max_norm)
        _check_same(gpu, T)
        assert gpu["norm"] == r.norm32


def test_zero_grads_leave_state_alone(H, orc):
    """Zero grads with wd = 0 from a fresh state: master, m, v and param
    unchanged bit for bit, over several steps, both modes."""
    banner("zero grads")
    rng = np.random.default_rng(71)
    n = 12_345
    th0 = rng.standard_normal(n).astype(np.float32)
    for mode in (0, 1):
        th = torch.from_numpy(th0.copy()).to(DEV)
        p = th.to(torch.bfloat16)
        p0 = p.clone()
        g = torch.zeros(n, device=DEV)
        m = torch.zeros(n, device=DEV)
        v = torch.zeros(n, device=DEV)
        hset = H.hpo_set_create_list([p], [th], [g], [m], [v])
        from mixed_precision_optimizer_amd import MixedPrecisionAdamW
        opt = MixedPrecisionAdamW(hset, [(1e-3, 0.0)], mode=mode, max_norm=1.0)
        for _ in range(4):
            applied, norm, _ = opt.step()
            assert applied and norm == 0.0
        assert np.array_equal(to_np(th).view(np.uint32), th0.view(np.uint32))
        assert torch.equal(p.view(torch.int16), p0.view(torch.int16))
        assert not m.any() and not v.any()
        hset.close()
