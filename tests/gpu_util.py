"""Helpers for the GPU parity tests: build hpo sets over the seeded inputs,
read state back, and compare it with the oracle's own trajectory.

Nothing here feeds GPU results into the oracle: the oracle starts from the
seeded initial state and the seeded grads only (both produced by
mixed_precision_optimizer_amd.inputs), and runs its own steps.
"""
from __future__ import annotations

import concurrent.futures as cf

import numpy as np
import pytest
import torch

from bounds import check_within, step_error_bounds


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from mixed_precision_optimizer_amd import hpo
    hpo.load()  # raises if libhpo.so is missing: no fallback exists
    return hpo


def banner(msg: str) -> None:
    print(f"\n[gpu-test] {msg}", flush=True)


def to_np(t: torch.Tensor) -> np.ndarray:
    """Host copy; 16-bit float tensors come back as their uint16 bit patterns."""
    t = t.detach()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).cpu().numpy().view(np.uint16).copy()
    return t.cpu().numpy().copy()


def bf16_of(theta: np.ndarray) -> np.ndarray:
    """torch's CPU fp32 -> bf16 cast (a library routine, not the oracle)."""
    return torch.from_numpy(theta).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def fp16_of(theta: np.ndarray) -> np.ndarray:
    """torch's CPU fp32 -> fp16 cast (a library routine, not the oracle)."""
    return torch.from_numpy(theta).to(torch.float16).view(torch.int16).numpy().view(np.uint16)


def widen_bf16(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def widen_fp16(bits: np.ndarray) -> np.ndarray:
    """torch's CPU fp16 -> fp32 cast of fp16 bit patterns."""
    return torch.from_numpy(bits.view(np.int16)).view(torch.float16).float().numpy()


def ordered16(bits: np.ndarray) -> np.ndarray:
    """Sign-magnitude 16-bit float patterns mapped to integers in value order,
    so that adjacent values differ by one."""
    b = bits.astype(np.int32)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def make_set(bufs, stream=None):
    from mixed_precision_optimizer_amd import hpo
    w = bufs.workload
    pdt = {"fp32": hpo.HPO_PARAM_FP32, "bf16": hpo.HPO_PARAM_BF16, "fp16": hpo.HPO_PARAM_FP16}[w.param_dtype]
    if w.flat and w.n_tensors > 1:
        return hpo.hpo_set_create_flat_ranges(None if w.param_dtype == "fp32" else bufs.param, bufs.master, bufs.grad,
                                              bufs.exp_avg, bufs.exp_avg_sq, bufs.offs,
                                              [w.group_of(i) for i in range(w.n_tensors)], param_dtype=pdt,
                                              stream=stream)
    if w.flat:
        return hpo.hpo_set_create_flat(None if w.param_dtype == "fp32" else bufs.param, bufs.master, bufs.grad,
                                       bufs.exp_avg, bufs.exp_avg_sq, stream=stream, param_dtype=pdt)
    ps, ms, gs, m1, m2 = bufs.lists()
    if w.param_dtype == "fp32":
        ps = None
    return hpo.hpo_set_create_list(ps, ms, gs, m1, m2, [w.group_of(i) for i in range(w.n_tensors)],
                                   param_dtype=pdt, stream=stream)


def make_opt(hset, w, device=None):
    from mixed_precision_optimizer_amd import MixedPrecisionAdamW
    return MixedPrecisionAdamW(hset, w.groups(), beta1=w.beta1, beta2=w.beta2, eps=w.eps, mode=w.mode,
                               max_norm=w.max_norm, loss_scale=w.loss_scale, log_num_zeros_in_grad=True,
                               device=device)


def compare_tensor(tag, gpu, orc_new, orc_prev, G, *, inv, clip, C, c64, lr, wd, t, mode, bf16, stats,
                   fp16=False):
    """gpu: dict theta/m/v[/p] numpy; orc_new / orc_prev: oracle OTensor after / before the step.
    fp32 moments: the rel-1e-6 propagated bound; bf16 moments: within one bf16
    ulp (the master's bound then uses the widened moments)."""
    s16 = orc_new.m.dtype == np.uint16
    wid = widen_fp16 if getattr(orc_new, "moments_fp16", False) else widen_bf16
    t16 = getattr(orc_new, "master_fp16", False)
    m_prev = wid(orc_prev.m) if s16 else orc_prev.m
    v_prev = wid(orc_prev.v) if s16 else orc_prev.v
    th_prev = widen_fp16(orc_prev.theta) if t16 else orc_prev.theta
    if G.dtype == np.uint16:
        G = widen_bf16(G)
    E_m, E_v, E_th = step_error_bounds(th_prev, m_prev, v_prev, G, inv=inv, C=c64, do_clip=clip,
                                       lr=lr, wd=wd, t=t, mode=mode)
    if s16:
        for key in ("m", "v"):
            d = np.abs(ordered16(gpu[key]) - ordered16(getattr(orc_new, key)))
            assert np.all(d <= 1), f"{tag} {key}: 16-bit moment more than 1 ulp from the oracle"
        eq_mv = int(np.sum(gpu["m"] == orc_new.m)) + int(np.sum(gpu["v"] == orc_new.v))
    else:
        check_within(f"{tag} m", gpu["m"], orc_new.m, E_m)
        check_within(f"{tag} v", gpu["v"], orc_new.v, E_v)
        eq_mv = int(np.sum(gpu["m"].view(np.uint32) == orc_new.m.view(np.uint32)))
        eq_mv += int(np.sum(gpu["v"].view(np.uint32) == orc_new.v.view(np.uint32)))
    n = gpu["theta"].size
    if t16:
        # fp16 master: within one fp16 ulp of the oracle's stored master
        d = np.abs(ordered16(gpu["theta"]) - ordered16(orc_new.theta))
        assert np.all(d <= 1), f"{tag} theta: fp16 master more than 1 ulp from the oracle"
        eq = int(np.sum(gpu["theta"] == orc_new.theta)) + eq_mv
    else:
        check_within(f"{tag} theta", gpu["theta"], orc_new.theta, E_th)
        eq = int(np.sum(gpu["theta"].view(np.uint32) == orc_new.theta.view(np.uint32))) + eq_mv
    stats["bit_equal"] = stats.get("bit_equal", 0) + eq
    stats["compared"] = stats.get("compared", 0) + 3 * n
    if bf16 or fp16:
        p = gpu["p"]
        # the write-back of the GPU's own master is bit-exact (the pages' invariant)
        th = widen_fp16(gpu["theta"]) if t16 else gpu["theta"]
        want = fp16_of(th) if fp16 else bf16_of(th)
        isnan = np.isnan(th)
        assert np.array_equal(p[~isnan], want[~isnan]), f"{tag}: param != 16-bit(master)"
        # and within one ulp of the oracle's param
        d = np.abs(p.astype(np.int32) - orc_new.p.astype(np.int32))
        assert np.all(d <= 1), f"{tag}: 16-bit param more than 1 ulp from the oracle"


def read_state(bufs, i=None, lo=0, hi=None):
    """GPU state of tensor (or range) i, or of the whole flat set when i is
    None, in element range [lo, hi)."""
    w = bufs.workload
    off = 0 if i is None else bufs.offs[i]
    n = w.numel if i is None else w.numels[i]
    hi = n if hi is None else hi
    a, b = off + lo, off + hi
    out = {"theta": to_np(bufs.master[a:b]), "m": to_np(bufs.exp_avg[a:b]), "v": to_np(bufs.exp_avg_sq[a:b])}
    if w.param_dtype in ("bf16", "fp16"):
        out["p"] = to_np(bufs.param[a:b])
    return out


# ---------------------------------------------------------------------------
# full-size norms: stream the stored grads to the host and sum there
# ---------------------------------------------------------------------------
def oracle_sumsq_streamed(orc, grad: torch.Tensor, ranges, inv: float, chunk: int = 1 << 27,
                          threads: int = 8) -> float:
    """Oracle sum of squares over the given (offset, length) ranges of a flat
    device grad buffer: each range is copied to pinned host memory in slices,
    each slice is summed by the oracle's plain loop (up to `threads` slices at
    once), and the slice sums are added in range order."""
    return oracle_grad_stats_streamed(orc, grad, ranges, inv, chunk, threads)[0]


def oracle_grad_stats_streamed(orc, grad: torch.Tensor, ranges, inv: float, chunk: int = 1 << 27,
                               threads: int = 8):
    """(sum of squares, zero count) of the unscaled grads over the given
    ranges, both by the oracle's plain loops over pinned host slices; the
    slice sums are added in range order, the counts are integers."""
    host = [torch.empty(chunk, dtype=torch.float32, pin_memory=True) for _ in range(threads)]
    pieces = []
    for off, n in ranges:
        for a in range(0, n, chunk):
            pieces.append((off + a, min(chunk, n - a)))
    sums = [0.0] * len(pieces)
    zeros = [0] * len(pieces)
    busy = [None] * threads
    with cf.ThreadPoolExecutor(max_workers=threads) as pool:
        for k, (off, n) in enumerate(pieces):
            slot = k % threads
            if busy[slot] is not None:
                busy[slot].result()
            host[slot][:n].copy_(grad[off:off + n])
            arr = host[slot][:n].numpy()

            def work(arr=arr, k=k):
                sums[k] = orc.sumsq(arr, inv)
                zeros[k] = orc.count_zeros(arr, inv)
            busy[slot] = pool.submit(work)
        for f in busy:
            if f is not None:
                f.result()
    total = 0.0
    for x in sums:
        total = total + x
    return total, sum(zeros)


def oracle_any_nonfinite_streamed(orc, grad: torch.Tensor, ranges, chunk: int = 1 << 28) -> bool:
    host = torch.empty(chunk, dtype=torch.float32, pin_memory=True)
    for off, n in ranges:
        for a in range(0, n, chunk):
            m = min(chunk, n - a)
            host[:m].copy_(grad[off + a:off + a + m])
            if orc.any_nonfinite(host[:m].numpy()):
                return True
    return False
