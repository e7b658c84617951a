"""GPU parity at the full workload sizes, in the launch configuration the
bench times (the library plans the same chunk table for the same sizes).

The oracle cannot step 8e9 elements, so it steps a deterministic sample of
elements (each tensor's first and last elements, whole small tensors, and
seeded windows inside large ones) from the seeded initial state, with the
seeded grads and its OWN global norm and zero count: every step the stored
grads are streamed to the host and summed and counted there by the oracle.
The skip decision, the norm (rel 1e-5), the zero count (exact) and every
sampled master / m / v / bf16 param are compared after each step.  The
write-back invariant param == 16-bit(master) is checked on every element of
the whole buffers after every step, on the device, with torch's own cast.

The Llama-8B-shaped list and the 70B/8 shard take the full sampling
protocol: each tensor's first and last 4096 elements plus 256 seeded windows
of 2^20 elements over the set (about 2.7e8 elements per step).

Device memory: 99..158 GB per test.
"""
import concurrent.futures as cf
import math

import numpy as np
import pytest
import torch

from gpu_util import banner, compare_tensor, make_opt, make_set, oracle_grad_stats_streamed, require_gpu, to_np

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

DEV = "cuda:0"


@pytest.fixture(scope="module")
def H():
    return require_gpu()


@pytest.fixture(scope="module")
def orc():
    import oracle
    oracle.lib()
    return oracle


def _picks(w, seed, head=4096, windows_big=2, window=65536, whole_below=8192, max_whole=None, windows_total=0):
    """(tensor, lo, hi) element ranges of the sample, per tensor in order:
    heads and tails, `windows_big` seeded windows in every large tensor, and
    `windows_total` seeded windows over the whole set, each in a tensor drawn
    with probability proportional to its size."""
    rng = np.random.default_rng(seed)
    sizes = np.array(w.numels, dtype=np.float64)
    extra = {}
    if windows_total:
        fits = np.where(sizes > 2 * head + window, sizes, 0.0)
        for i in rng.choice(len(sizes), size=windows_total, p=fits / fits.sum()):
            extra[int(i)] = extra.get(int(i), 0) + 1
    picks = []
    n_whole = 0
    for i, n in enumerate(w.numels):
        if n == 0:
            continue
        if n <= whole_below and (max_whole is None or n_whole < max_whole):
            picks.append((i, 0, n))
            n_whole += 1
            continue
        h = min(head, n // 2)
        rs = [(0, h)]
        for _ in range((windows_big if n > 4 * window else 0) + extra.get(i, 0)):
            lo = int(rng.integers(h, n - h - window))
            lo -= lo % 4 if rng.random() < 0.5 else 0  # mix aligned and unaligned window starts
            rs.append((lo, lo + window))
        rs.append((n - h, n))
        rs.sort()
        merged = []
        for lo, hi in rs:
            if merged and lo <= merged[-1][1]:
                merged[-1] = (merged[-1][0], max(merged[-1][1], hi))
            else:
                merged.append((lo, hi))
        picks += [(i, lo, hi) for lo, hi in merged]
    return picks


class Sample:
    """Gathers the sampled elements of every state array with one device
    gather + one host copy per array."""

    def __init__(self, bufs, picks):
        self.bufs = bufs
        self.picks = picks
        w = bufs.workload
        offs = bufs.offs
        idx = np.concatenate([np.arange(offs[i] + lo, offs[i] + hi, dtype=np.int64) for i, lo, hi in picks])
        self.idx = torch.from_numpy(idx).to(DEV)
        self.seg = []
        pos = 0
        for i, lo, hi in picks:
            self.seg.append((i, pos, hi - lo))
            pos += hi - lo
        self.n = pos

    def gather(self, buf):
        return to_np(buf[self.idx])

    def state(self):
        b = self.bufs
        out = {"theta": self.gather(b.master), "m": self.gather(b.exp_avg), "v": self.gather(b.exp_avg_sq)}
        if b.workload.param_dtype in ("bf16", "fp16"):
            out["p"] = self.gather(b.param)
        return out


def _check_writeback_everywhere(bufs, chunk=1 << 28):
    """param == 16-bit(master) on every element of the buffers (padding gaps
    included, where both keep their initial values), with torch's device cast."""
    w = bufs.workload
    if w.param_dtype == "fp32":
        return
    pdt = torch.float16 if w.param_dtype == "fp16" else torch.bfloat16
    for a in range(0, bufs.total, chunk):
        b = min(bufs.total, a + chunk)
        want = bufs.master[a:b].to(pdt)
        assert torch.equal(bufs.param[a:b].view(torch.int16), want.view(torch.int16)), \
            f"param != {pdt}(master) in [{a}, {b})"
        del want


def _apply_update_threaded(orc, Ts, Gs, hyper, groups, t, inv, do_clip, C, c64, threads=16):
    """The oracle's update of the sampled tensors, the segments split over
    threads (each segment is stepped by the oracle's own loop, unchanged)."""
    k = max(1, len(Ts) // (4 * threads))
    parts = [(Ts[a:a + k], Gs[a:a + k]) for a in range(0, len(Ts), k)]
    with cf.ThreadPoolExecutor(max_workers=threads) as pool:
        for f in [pool.submit(orc.apply_update, T, G, hyper, groups, t, inv, do_clip, C, c64) for T, G in parts]:
            f.result()


def _ranges(bufs):
    w = bufs.workload
    if w.flat:
        return [(0, w.numel)]  # a flat shard has no gaps: stream it as one range
    return [(bufs.offs[i], n) for i, n in enumerate(w.numels) if n > 0]


class _DeviceStep:
    """The device-resident step (hpo_step_device: scaler state, skip decision and
    t on the device) behind the host-driven optimizer's interface: each step
    is enqueued, then the state is read back for the comparison."""

    def __init__(self, hset, w):
        from mixed_precision_optimizer_amd import DeviceAdamW
        self.opt = DeviceAdamW(hset, w.groups(), beta1=w.beta1, beta2=w.beta2, eps=w.eps, mode=w.mode,
                               max_norm=w.max_norm, loss_scale=1.0 if w.loss_scale is None else w.loss_scale,
                               dynamic=False)
        self.t = 0

    def step(self):
        self.opt.step()
        st = self.opt.sync()
        assert st.error == 0
        self.t = st.applied_steps
        return bool(st.applied), (float(st.grad_norm) if st.applied else None), int(st.num_zeros)


def _run_fullsize(H, orc, w, picks_kw, steps=None, device_step=False):
    from mixed_precision_optimizer_amd import inputs
    banner(f"{w.name}: {w.numel} elements in {w.n_tensors} tensors, allocating {w.numel * 18 / 1e9:.1f} GB")
    bufs = inputs.allocate(w, DEV)
    picks = _picks(w, seed=99, **picks_kw)
    S = Sample(bufs, picks)
    banner(f"sample: {S.n} elements in {len(S.seg)} segments")
    # the oracle's sampled state: one array per field, one view per segment
    big = S.state()
    bf16 = w.param_dtype == "bf16"
    fp16 = w.param_dtype == "fp16"
    has_p = bf16 or fp16
    t16 = w.master_dtype == "fp16"
    s16 = w.state_dtype == "fp16"
    Ts = []
    lr_e = np.empty(S.n)
    wd_e = np.empty(S.n)
    for i, pos, n in S.seg:
        sl = slice(pos, pos + n)
        g = w.group_of(i)
        Ts.append(orc.OTensor(big["theta"][sl], big["m"][sl], big["v"][sl], big["p"][sl] if has_p else None, g, fp16,
                              t16, s16))
        lr_e[sl], wd_e[sl] = w.groups()[g]
    hset = make_set(bufs)
    opt = _DeviceStep(hset, w) if device_step else make_opt(hset, w)
    hyper = orc.Hyper(w.beta1, w.beta2, w.eps, w.mode)
    inv = w.inv_scale()
    t_orc = 0
    stats = {}
    steps = w.steps if steps is None else steps
    for k in range(1, steps + 1):
        inputs.fill_grads_(bufs, k)
        torch.cuda.synchronize()
        Gs = S.gather(bufs.grad)
        # the oracle's own global norm, zero count and non-finite decision over ALL grads
        n2, n_zeros = oracle_grad_stats_streamed(orc, bufs.grad, _ranges(bufs), inv)
        found = not math.isfinite(n2)  # |G * inv| <= |G| here, so the sum is finite iff every G is
        applied, norm, zeros = opt.step()
        banner(f"step {k}: gpu applied={applied} norm={norm} zeros={zeros}  oracle found_inf={found} "
               f"norm={math.sqrt(n2) if not found else None} zeros={n_zeros}")
        assert applied == (not found)
        if applied:
            assert zeros == n_zeros, (zeros, n_zeros)
            stats.setdefault("zeros", []).append(zeros)
        st = S.state()
        if found:
            for key in ("theta", "m", "v"):
                assert np.array_equal(st[key].view(np.uint8), big[key].view(np.uint8))
            if has_p:
                assert np.array_equal(st["p"], big["p"])
            stats.setdefault("skipped", []).append(k)
            continue
        t_orc += 1
        norm64, norm32 = orc.norm_from_sumsq(n2)
        assert abs(norm - norm64) <= 1e-5 * norm64
        do_clip, C, c64 = orc.clip_coeff(w.max_norm, norm32)
        prev = orc.OTensor(big["theta"].copy(), big["m"].copy(), big["v"].copy(),
                           big["p"].copy() if has_p else None, 0, fp16, t16, s16)
        _apply_update_threaded(orc, Ts, [Gs[pos:pos + n] for _, pos, n in S.seg], hyper, w.groups(), t_orc, inv,
                               do_clip, C, c64)
        assert opt.t == t_orc
        _check_writeback_everywhere(bufs)
        for a in range(0, S.n, 1 << 25):   # elementwise bounds, compared a slice at a time
            b = min(S.n, a + (1 << 25))
            cut = lambda x: None if x is None else x[a:b]
            now = orc.OTensor(big["theta"][a:b], big["m"][a:b], big["v"][a:b], cut(big["p"] if has_p else None),
                              0, fp16, t16, s16)
            was = orc.OTensor(prev.theta[a:b], prev.m[a:b], prev.v[a:b], cut(prev.p), 0, fp16, t16, s16)
            compare_tensor(f"{w.name} step {k} [{a}:{b}]", {key: x[a:b] for key, x in st.items()}, now, was,
                           Gs[a:b], inv=inv, clip=do_clip, C=C, c64=c64, lr=lr_e[a:b], wd=wd_e[a:b], t=t_orc,
                           mode=w.mode, bf16=bf16, fp16=fp16, stats=stats)
    banner(f"bit-equal {stats.get('bit_equal', 0)}/{stats.get('compared', 0)}; skipped {stats.get('skipped', [])}")
    hset.close()
    del bufs
    torch.cuda.empty_cache()
    return stats


@pytest.mark.timeout(900)
def test_zero_shard_70b_over_8(H, orc):
    """8.75e9-element flat shard (> 2^32: 64-bit indexing), grads N(0, 1e-4),
    norm ~9.35 so the clip fires, 3 steps."""
    from mixed_precision_optimizer_amd import inputs
    w = inputs.zero_shard()
    stats = _run_fullsize(H, orc, w, dict(head=4096, windows_big=0, window=1 << 20, windows_total=256))
    assert stats["bit_equal"] == stats["compared"]
    assert len(stats["zeros"]) == 3 and min(stats["zeros"]) > 0


@pytest.mark.timeout(900)
def test_zero_shard_70b_over_8_device_resident(H, orc):
    """The same 8.75e9-element shard through the device-resident step, the
    configuration of the bench's device-resident leg: the two-stage finalize
    (133,515 partials) writes the norm, the zero count and the apply decision
    into the device state, and the update (streaming accesses) takes t and
    the unscale factor from it; the sampled elements match the oracle bit for
    bit and every param equals bf16(master)."""
    from mixed_precision_optimizer_amd import inputs
    w = inputs.zero_shard()
    stats = _run_fullsize(H, orc, w, dict(head=4096, windows_big=0, window=1 << 20, windows_total=256),
                          device_step=True)
    assert stats["bit_equal"] == stats["compared"]
    assert len(stats["zeros"]) == 3 and min(stats["zeros"]) > 0


@pytest.mark.timeout(900)
def test_llama8b_shaped_list(H, orc):
    """291 tensors (65 1-D in the no-decay group), per-tensor grad scales
    log-uniform in [1e-5, 1e-2], clip 1.0, 5 steps."""
    from mixed_precision_optimizer_amd import inputs
    w = inputs.llama8b()
    stats = _run_fullsize(H, orc, w, dict(head=4096, windows_big=0, window=1 << 20, whole_below=8192,
                                          windows_total=256))
    assert stats["bit_equal"] == stats["compared"]


@pytest.mark.timeout(900)
def test_ragged_20000_tensors_with_skip(H, orc):
    """20000 tensors of log-uniform size in [1, 4M], loss scale 65536, +inf in
    the stored grads at step 3 (skipped, t not advanced), 8 steps."""
    from mixed_precision_optimizer_amd import inputs
    w = inputs.ragged()
    stats = _run_fullsize(H, orc, w, dict(head=256, windows_big=1, window=4096, whole_below=1024))
    assert stats["skipped"] == [3]
    assert stats["bit_equal"] == stats["compared"]
    # planted +0 / -0 and stored subnormals that the 2^-16 unscale rounds to zero, counted exactly
    assert len(stats["zeros"]) == 7 and min(stats["zeros"]) > 0


@pytest.mark.timeout(900)
def test_ragged_20000_tensors_device_resident(H, orc):
    """The same ragged set through the device-resident step: the loss scale
    (65536) lives in the device state, the norm and skip decision are written
    there by the two-stage finalize (83K partials), the update takes t from
    it.  The +inf at step 3 is skipped on the device; every sampled element
    matches the oracle bit for bit."""
    from mixed_precision_optimizer_amd import inputs
    w = inputs.ragged()
    stats = _run_fullsize(H, orc, w, dict(head=256, windows_big=1, window=4096, whole_below=1024), device_step=True)
    assert stats["skipped"] == [3]
    assert stats["bit_equal"] == stats["compared"]
    assert len(stats["zeros"]) == 7 and min(stats["zeros"]) > 0


@pytest.mark.timeout(900)
def test_zero_shard_with_param_ranges_llama70b(H, orc):
    """Rank 3 of 8 of a Llama-70B-shaped flat buffer (8.82e9 elements): 95
    ranges, the 1-D norm gains in the no-decay group, clip 1.0, 3 steps."""
    from mixed_precision_optimizer_amd import inputs
    w = inputs.zero_shard_ranges()
    stats = _run_fullsize(H, orc, w, dict(head=2048, windows_big=2, window=16384, whole_below=8192))
    assert stats["bit_equal"] == stats["compared"]


@pytest.mark.timeout(900)
def test_zero_shard_bf16_moments(H, orc):
    """The 70B/8 flat shard with exp_avg / exp_avg_sq held in bf16 (22 bytes per
    element per update instead of 30), 3 steps."""
    from mixed_precision_optimizer_amd import inputs
    w = inputs.zero_shard(state_dtype="bf16")
    stats = _run_fullsize(H, orc, w, dict(head=4096, windows_big=64, window=65536))
    assert stats["bit_equal"] == stats["compared"]


@pytest.mark.timeout(900)
def test_zero_shard_bf16_grads_fp16_master(H, orc):
    """The 70B/8 flat shard with bf16 main grads and an fp16 master under the
    bf16 params (the update moves 24 bytes per element instead of 30), 3
    steps: the norm over all 8.75e9 widened grads, the sampled state within
    one fp16 ulp (bit-equal in practice), every param the bf16 rounding of
    its stored master."""
    from mixed_precision_optimizer_amd import inputs
    w = inputs.zero_shard(grad_dtype="bf16", master_dtype="fp16")
    stats = _run_fullsize(H, orc, w, dict(head=4096, windows_big=64, window=65536))
    assert stats["bit_equal"] == stats["compared"]


@pytest.mark.timeout(900)
def test_zero_shard_fp16_params_bf16_moments(H, orc):
    """The 70B/8 flat shard with fp16 model params and bf16 moments (the
    reduced-precision variants together: 22 bytes per element per update),
    3 steps; the fp16 write-back of every sampled master is checked."""
    from mixed_precision_optimizer_amd import inputs
    w = inputs.zero_shard(state_dtype="bf16", param_dtype="fp16")
    stats = _run_fullsize(H, orc, w, dict(head=4096, windows_big=64, window=65536))
    assert stats["bit_equal"] == stats["compared"]
