"""Seeded synthetic inputs for the optimizer-step workloads.

This module only draws random numbers and lays out buffers; it holds none of
the optimizer's arithmetic.  Both the HIP path's callers (tests, bench) and
the CPU oracle's callers take their inputs from here, so the two sides see the
same bits.

Workload shapes come from the pages:
  * toy: the two-parameter decay experiment of the page
    "优化器：AdamW、Muon 与分布式优化器" (section "AdamW：解耦的权重衰减");
  * two matrices 4096x1024 and 1024x4096 drawn with torch.manual_seed(0), as in
    that page's state-size measurement (section "优化器的显存账本");
  * a Llama-8B-shaped parameter list, a ragged 20000-tensor list and a flat
    ZeRO-1 shard of a 70B model over 8 data-parallel ranks (the flat shard
    layout follows "02 · Optimizer：算法与 infra" §12.1: each rank owns one
    contiguous slice of the flat buffer, param boundaries ignored).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np
import torch

# Param starts inside a flat buffer are aligned to 64 elements, the alignment
# the DDP buffer layout uses ("02 · Optimizer：算法与 infra" §16, param_layout).
ALIGN_ELEMS = 64
FILL_CHUNK = 1 << 30  # elements per in-place RNG fill (bounds temporaries)


@dataclass
class Workload:
    name: str
    numels: List[int]
    ndims: List[int]
    param_dtype: str = "bf16"          # "bf16", "fp16" or "fp32" (fp32 params are their own master)
    state_dtype: str = "fp32"          # exp_avg / exp_avg_sq storage: "fp32", "bf16" or "fp16"
    grad_dtype: str = "fp32"           # main grad storage: "fp32" or "bf16" (the bf16 image of the fp32 draw)
    master_dtype: str = "fp32"         # master storage: "fp32" or "fp16" (the fp16 image of the fp32 draw)
    lr: float = 1e-3
    weight_decay: float = 0.1
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    mode: int = 0                      # 0 AdamW, 1 Adam + L2
    max_norm: float = 0.0              # <= 0: no clipping
    loss_scale: Optional[float] = None
    steps: int = 1
    grad_std: List[float] = field(default_factory=list)
    master_seed: int = 0
    grad_seed_base: int = 1000
    inf_step: Optional[int] = None     # 1-based call index whose grads carry one +inf
    flat: bool = False                 # one flat shard instead of a tensor list
    no_decay_1d: bool = True           # 1-D tensors go to the weight_decay = 0 group
    zero_every: int = 0                # > 0: plant exact zeros and tiny subnormals every this many elements

    @property
    def numel(self) -> int:
        return int(sum(self.numels))

    @property
    def n_tensors(self) -> int:
        return len(self.numels)

    def group_of(self, i: int) -> int:
        """Group 0 decays, group 1 (1-D tensors: norm gains, biases) does not."""
        return 1 if (self.no_decay_1d and self.ndims[i] == 1) else 0

    def groups(self):
        return [(self.lr, self.weight_decay), (self.lr, 0.0)]

    def inv_scale(self) -> float:
        return 1.0 if self.loss_scale is None else float(np.float32(1.0 / self.loss_scale))


# --------------------------------------------------------------------------
# workload definitions
# --------------------------------------------------------------------------
def toy(mode: int) -> Workload:
    return Workload("toy_2param", [2], [1], param_dtype="fp32", lr=1e-2, weight_decay=0.1,
                    mode=mode, steps=1000, grad_std=[0.0], no_decay_1d=False)


def toy_grad(k: int) -> np.ndarray:
    """Gradient of 1-based call k: [0.01, 10] * (-1)^(k-1)."""
    return np.ascontiguousarray(np.array([0.01, 10.0], np.float32) * np.float32((-1.0) ** (k - 1)))


def two_matrices() -> Workload:
    return Workload("two_matrices_8.4M", [4096 * 1024, 1024 * 4096], [2, 2], lr=1e-3,
                    weight_decay=0.1, max_norm=1.0, steps=10, grad_std=[1e-3, 1e-3])


def llama8b_shapes():
    """(name, shape) of a Llama-8B-shaped parameter list: 32 layers, hidden 4096,
    FFN 14336, 8 KV heads of 128, vocab 128256, untied embedding/head."""
    h, f, kv, vocab, layers = 4096, 14336, 8 * 128, 128256, 32
    out = [("embed", (vocab, h))]
    for l in range(layers):
        out += [(f"l{l}.q", (h, h)), (f"l{l}.k", (kv, h)), (f"l{l}.v", (kv, h)),
                (f"l{l}.o", (h, h)), (f"l{l}.gate", (f, h)), (f"l{l}.up", (f, h)),
                (f"l{l}.down", (h, f)), (f"l{l}.attn_norm", (h,)), (f"l{l}.mlp_norm", (h,))]
    out += [("final_norm", (h,)), ("lm_head", (vocab, h))]
    return out


def llama8b() -> Workload:
    shapes = llama8b_shapes()
    rng = np.random.default_rng(3)
    sig = np.exp(rng.uniform(math.log(1e-5), math.log(1e-2), size=len(shapes)))
    return Workload("llama8b_shaped", [int(np.prod(s)) for _, s in shapes], [len(s) for _, s in shapes],
                    lr=1e-3, weight_decay=0.1, max_norm=1.0, steps=5, grad_std=[float(x) for x in sig])


def ragged_sizes(n: int = 20000, max_elems: int = 4 * 2 ** 20, seed: int = 4) -> List[int]:
    rng = np.random.default_rng(seed)
    return [max(1, int(round(math.exp(x)))) for x in rng.uniform(0.0, math.log(max_elems), size=n)]


def ragged(n: int = 20000, max_elems: int = 4 * 2 ** 20, steps: int = 8, inf_step: int = 3) -> Workload:
    sizes = ragged_sizes(n, max_elems)
    return Workload(f"ragged_{n}", sizes, [2] * n, lr=1e-3, weight_decay=0.1, max_norm=1.0,
                    loss_scale=65536.0, steps=steps, grad_std=[1e-3] * n, inf_step=inf_step, zero_every=1009)


def zero_shard(numel: int = 8_750_000_000, state_dtype: str = "fp32", param_dtype: str = "bf16",
               grad_dtype: str = "fp32", master_dtype: str = "fp32") -> Workload:
    # a flat shard mixes every kind of param; it is stepped as one decaying group
    tag = "" if (state_dtype, param_dtype) == ("fp32", "bf16") else f"_{param_dtype}_params_{state_dtype}_moments"
    if grad_dtype != "fp32":
        tag += f"_{grad_dtype}_grads"
    if master_dtype != "fp32":
        tag += f"_{master_dtype}_master"
    return Workload(f"zero1_shard_70b_over_8{tag}", [numel], [1], lr=1e-3, weight_decay=0.1, max_norm=1.0,
                    steps=3, grad_std=[1e-4], flat=True, no_decay_1d=False, state_dtype=state_dtype,
                    param_dtype=param_dtype, grad_dtype=grad_dtype, master_dtype=master_dtype, zero_every=4099)


def llama70b_shapes():
    """(name, shape) of a Llama-70B-shaped parameter list: 80 layers, hidden
    8192, FFN 28672, 8 KV heads of 128, vocab 128256, untied embedding/head."""
    h, f, kv, vocab, layers = 8192, 28672, 8 * 128, 128256, 80
    out = [("embed", (vocab, h))]
    for l in range(layers):
        out += [(f"l{l}.q", (h, h)), (f"l{l}.k", (kv, h)), (f"l{l}.v", (kv, h)),
                (f"l{l}.o", (h, h)), (f"l{l}.gate", (f, h)), (f"l{l}.up", (f, h)),
                (f"l{l}.down", (h, f)), (f"l{l}.attn_norm", (h,)), (f"l{l}.mlp_norm", (h,))]
    out += [("final_norm", (h,)), ("lm_head", (vocab, h))]
    return out


def zero_shard_ranges(rank: int = 3, dp: int = 8) -> Workload:
    """Rank `rank`'s contiguous 1/dp slice of the flat param buffer of a
    Llama-70B-shaped model ("02 · Optimizer：算法与 infra" §12.1: the buffer is
    split evenly by data-parallel rank without regard to param boundaries).
    Params start on 64-element boundaries; the buffer is padded to a multiple
    of 64 * dp.  Each range of the slice carries the group of the param it
    belongs to (the padding after a param, that of the param before it); the
    1-D norm gains take no weight decay."""
    shapes = llama70b_shapes()
    sizes = [int(np.prod(sh)) for _, sh in shapes]
    offs, total = offsets(sizes)
    total = (total + 64 * dp - 1) // (64 * dp) * (64 * dp)
    shard = total // dp
    lo, hi = rank * shard, (rank + 1) * shard
    starts, dims = [], []
    for (name, sh), o, n in zip(shapes, offs, sizes):
        end = o + (n + ALIGN_ELEMS - 1) // ALIGN_ELEMS * ALIGN_ELEMS  # param + its padding
        a, b = max(o, lo), min(end, hi)
        if a < b:
            starts.append(a - lo)
            dims.append(len(sh))
    lens = [b - a for a, b in zip(starts, starts[1:] + [shard])]
    return Workload(f"zero1_shard_ranges_llama70b_rank{rank}_of_{dp}", lens, dims, lr=1e-3, weight_decay=0.1,
                    max_norm=1.0, steps=3, grad_std=[1e-4] * len(lens), flat=True, no_decay_1d=True)


def inf_position(w: Workload) -> tuple:
    """(tensor index, element) of the injected +inf: the last element of the
    highest-index tensor whose size is not a multiple of 4 (so it sits on the
    scalar tail), else the last element of the last tensor."""
    for i in range(w.n_tensors - 1, -1, -1):
        if w.numels[i] % 4 != 0:
            return i, w.numels[i] - 1
    return w.n_tensors - 1, w.numels[-1] - 1


# --------------------------------------------------------------------------
# buffers
# --------------------------------------------------------------------------
def offsets(numels: List[int], align: int = ALIGN_ELEMS):
    """Start offset of every tensor inside one flat buffer, each aligned to
    ``align`` elements; returns (offsets, total length)."""
    offs, cur = [], 0
    for n in numels:
        offs.append(cur)
        cur += (n + align - 1) // align * align
    return offs, max(cur, 1)


def fill_normal_(buf: torch.Tensor, seed: int, std: float = 1.0) -> None:
    """In-place N(0, std) fill of a flat tensor in FILL_CHUNK slices from one
    seeded generator on buf's device."""
    gen = torch.Generator(device=buf.device)
    gen.manual_seed(seed)
    n = buf.numel()
    for a in range(0, n, FILL_CHUNK):
        b = min(n, a + FILL_CHUNK)
        buf[a:b].normal_(0.0, 1.0, generator=gen)
        if std != 1.0:
            buf[a:b].mul_(std)


@dataclass
class Buffers:
    """Flat device buffers for one workload, and the per-tensor views."""
    workload: Workload
    offs: List[int]
    total: int
    master: torch.Tensor
    grad: torch.Tensor
    exp_avg: torch.Tensor
    exp_avg_sq: torch.Tensor
    param: torch.Tensor        # 16-bit buffer, or the master itself for fp32 params

    def view(self, buf: torch.Tensor, i: int) -> torch.Tensor:
        o = self.offs[i]
        return buf[o:o + self.workload.numels[i]]

    def lists(self):
        w = self.workload
        return ([self.view(self.param, i) for i in range(w.n_tensors)],
                [self.view(self.master, i) for i in range(w.n_tensors)],
                [self.view(self.grad, i) for i in range(w.n_tensors)],
                [self.view(self.exp_avg, i) for i in range(w.n_tensors)],
                [self.view(self.exp_avg_sq, i) for i in range(w.n_tensors)])


def _narrowed(x: torch.Tensor, dtype) -> torch.Tensor:
    """A 16-bit copy of x made in FILL_CHUNK slices (torch's cast)."""
    out = torch.empty(x.numel(), dtype=dtype, device=x.device)
    for a in range(0, x.numel(), FILL_CHUNK):
        b = min(x.numel(), a + FILL_CHUNK)
        out[a:b].copy_(x[a:b])
    return out


def allocate(w: Workload, device) -> Buffers:
    """Allocate flat master/grad/m/v (+bf16 param) buffers and initialise the
    state: master N(0,1) from ``master_seed``, m = v = 0, param = bf16 cast of
    the master (torch's cast; the param's initial value is an input).  An
    fp16 master holds the fp16 image of the same draw, and the param is then
    the cast of that fp16 master; bf16 grads are the bf16 image of the fp32
    grads fill_grads_ draws."""
    if w.flat:
        # a flat shard, possibly cut into ranges of different groups: the
        # ranges are consecutive, with no gaps
        offs = [int(x) for x in np.cumsum([0] + w.numels[:-1])]
        total = w.numel
    else:
        offs, total = offsets(w.numels)
    f32 = dict(dtype=torch.float32, device=device)
    master = torch.empty(total, **f32)
    if w.name.startswith("toy"):
        master.fill_(1.0)
    elif w.name.startswith("two_matrices"):
        m = two_matrix_masters()
        master[offs[0]:offs[0] + m[0].numel()].copy_(m[0].reshape(-1))
        master[offs[1]:offs[1] + m[1].numel()].copy_(m[1].reshape(-1))
    else:
        fill_normal_(master, w.master_seed)
    if w.master_dtype == "fp16":
        master = _narrowed(master, torch.float16)
    grad = torch.zeros(total, dtype=torch.bfloat16 if w.grad_dtype == "bf16" else torch.float32, device=device)
    sdt = {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}[w.state_dtype]
    exp_avg = torch.zeros(total, dtype=sdt, device=device)
    exp_avg_sq = torch.zeros(total, dtype=sdt, device=device)
    if w.param_dtype == "fp32":
        param = master
    else:
        pdt = torch.float16 if w.param_dtype == "fp16" else torch.bfloat16
        param = torch.empty(total, dtype=pdt, device=device)
        for a in range(0, total, FILL_CHUNK):
            b = min(total, a + FILL_CHUNK)
            param[a:b].copy_(master[a:b])
    return Buffers(w, offs, total, master, grad, exp_avg, exp_avg_sq, param)


def two_matrix_masters():
    """w1 = randn(4096,1024), w2 = randn(1024,4096) after torch.manual_seed(0),
    drawn on the CPU as the page's state-size script does."""
    g = torch.Generator().manual_seed(0)
    w1 = torch.randn(4096, 1024, generator=g)
    w2 = torch.randn(1024, 4096, generator=g)
    return w1, w2


def fill_grads_(bufs: Buffers, k: int) -> None:
    """Stored grads of 1-based call k, written into bufs.grad in place.

    toy: the page's alternating grads.  Otherwise N(0, 1) from seed
    grad_seed_base + k over the whole flat buffer, each tensor's slice then
    multiplied by its std, then by the loss scale (exact for powers of two);
    at ``inf_step`` one element becomes +inf (see inf_position)."""
    w = bufs.workload
    if bufs.grad.dtype != torch.float32:
        # the 16-bit image of the fp32 grads below (torch's cast)
        full = Buffers(w, bufs.offs, bufs.total, bufs.master, torch.empty(bufs.total, dtype=torch.float32,
                       device=bufs.grad.device), bufs.exp_avg, bufs.exp_avg_sq, bufs.param)
        fill_grads_(full, k)
        for a in range(0, bufs.total, FILL_CHUNK):
            b = min(bufs.total, a + FILL_CHUNK)
            bufs.grad[a:b].copy_(full.grad[a:b])
        return
    if w.name.startswith("toy"):
        bufs.grad[:2].copy_(torch.from_numpy(toy_grad(k)))
        return
    if w.name.startswith("two_matrices"):
        g = torch.Generator().manual_seed(w.grad_seed_base + k)
        for i in range(w.n_tensors):
            cpu = torch.randn(w.numels[i], generator=g).mul_(w.grad_std[i])
            bufs.view(bufs.grad, i).copy_(cpu)
    else:
        fill_normal_(bufs.grad, w.grad_seed_base + k)
        stds = w.grad_std
        if len(set(stds)) == 1:
            bufs.grad.mul_(stds[0])
        else:
            for i in range(w.n_tensors):
                bufs.view(bufs.grad, i).mul_(stds[i])
    if w.loss_scale is not None:
        bufs.grad.mul_(w.loss_scale)
    if w.zero_every > 0:
        plant_zeros_(bufs.grad, w.zero_every, k)
    if w.inf_step is not None and k == w.inf_step:
        ti, e = inf_position(w)
        bufs.grad[bufs.offs[ti] + e] = float("inf")


# The stored value 3 * 2^-149, an fp32 subnormal: not zero as stored, zero
# after an unscale by 2^-16 (3 * 2^-165 is below half the smallest subnormal).
TINY_SUBNORMAL = float(np.array([3], dtype=np.uint32).view(np.float32)[0])


def plant_zeros_(grad: torch.Tensor, every: int, k: int) -> None:
    """Stored grads that are exactly zero, as real grads are where a weight
    got no signal (embedding rows of unseen tokens, dead units): in call k,
    elements o, o + every, o + 2 every, ... with o = (7919 k) mod every
    become +0 and -0 alternately, and elements o + every/2 + j every become
    TINY_SUBNORMAL, which is zero only after a 2^-16 unscale.  Written after
    the loss-scale multiply, so these are the stored values."""
    o = (7919 * k) % every
    grad[o::2 * every] = 0.0
    grad[o + every::2 * every] = -0.0
    grad[o + every // 2::every] = TINY_SUBNORMAL


# ---------------------------------------------------------------------------
# Muon workloads
# ---------------------------------------------------------------------------
# Shapes of the small Muon parity set: tall and wide matrices (transposed and
# not), square, a shape class of two (one batch of two), vectors as 1 x n and
# n x 1 matrices, an empty matrix, sizes that are not multiples of the 256
# padding, and one wider than a single GEMM tile in both directions.
MUON_PARITY_SHAPES = [(128, 384), (384, 128), (200, 200), (1, 64), (64, 1), (0, 5), (300, 700), (300, 700),
                      (37, 129), (520, 260)]


def seeded_matrix(shape, seed: int, std: float = 1.0) -> np.ndarray:
    """fp32 N(0, std) matrix from torch's CPU generator seeded with seed."""
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(int(np.prod(shape)) if len(shape) else 1, generator=g, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.numpy().reshape(shape)


def handbook_ns_matrix(seed: int = 2024) -> np.ndarray:
    """256 x 1024 fp32 G = U diag(S) V^T with orthonormal U, V (QR of seeded
    Gaussians) and S = 256 values log-spaced from 1 to 0.01: the input of the
    Newton-Schulz demonstration on "优化器：AdamW、Muon 与分布式优化器" (Muon
    section).  Returns (G, V) -- V's first columns are the largest directions."""
    rng = np.random.default_rng(seed)
    U, R = np.linalg.qr(rng.standard_normal((256, 256)))
    U = U * np.sign(np.diag(R))
    V, R = np.linalg.qr(rng.standard_normal((1024, 256)))
    V = V * np.sign(np.diag(R))
    S = np.logspace(0, -2, 256)
    return ((U * S) @ V.T).astype(np.float32), V


def llama8b_muon_split():
    """Route the Llama-8B-shaped parameters the way the pages do
    ("02 · Optimizer：算法与 infra" §5.5, §14.2): hidden 2-D matrices to
    Muon; embedding, output head and every 1-D parameter to AdamW.
    Returns (adam [(name, shape)], muon [(name, shape)])."""
    adam, muon = [], []
    for name, shape in llama8b_shapes():
        if len(shape) == 2 and name not in ("embed", "lm_head"):
            muon.append((name, shape))
        else:
            adam.append((name, shape))
    return adam, muon


def llama8b_chain():
    """The Llama-8B-shaped parameters split between the two optimizers of a
    chain: (AdamW Workload over the embedding, output head and 1-D gains, and
    the Muon matrices as (name, (rows, cols), grad std)).  Grad stds are the
    per-tensor ones of llama8b()."""
    full = llama8b_shapes()
    stds = dict(zip([n for n, _ in full], llama8b().grad_std))
    adam, muon = llama8b_muon_split()
    w = Workload("llama8b_chain_adamw_part", [int(np.prod(s)) for _, s in adam], [len(s) for _, s in adam],
                 lr=1e-3, weight_decay=0.1, max_norm=1.0, steps=5, grad_std=[stds[n] for n, _ in adam])
    return w, [(n, s, stds[n]) for n, s in muon]


@dataclass
class MuonBuffers:
    """Flat buffers of a Muon matrix list (64-element aligned starts) and the
    per-matrix 2-D views."""
    shapes: list
    offs: list
    master: torch.Tensor
    grad: torch.Tensor
    momentum: torch.Tensor
    param: torch.Tensor

    def views(self, buf):
        return [buf[o:o + r * c].view(r, c) for o, (r, c) in zip(self.offs, self.shapes)]


def fill_muon_grads_(mb: MuonBuffers, matrices, k: int, grad_seed: int = 2001) -> None:
    """fp32 grads of call k of a Muon matrix list: N(0, 1) from seed
    grad_seed + 1000 (k - 1) over the flat buffer, then matrix i's slice
    times its std (call 1 repeats the draw allocate_muon makes)."""
    fill_normal_(mb.grad, grad_seed + 1000 * (k - 1))
    for (_, (r, c), std), o in zip(matrices, mb.offs):
        mb.grad[o:o + r * c].mul_(std)


def allocate_muon(matrices, device, master_seed: int = 7, grad_seed: int = 2001) -> MuonBuffers:
    """fp32 master N(0, 1), fp32 momentum 0, bf16 param = cast of the master,
    fp32 grads N(0, std_i) for matrix i (one seeded fill, then per-matrix
    scaling)."""
    shapes = [tuple(s) for _, s, _ in matrices]
    offs, total = offsets([r * c for r, c in shapes])
    f32 = dict(dtype=torch.float32, device=device)
    master = torch.empty(total, **f32)
    fill_normal_(master, master_seed)
    grad = torch.empty(total, **f32)
    fill_normal_(grad, grad_seed)
    for (_, (r, c), std), o in zip(matrices, offs):
        grad[o:o + r * c].mul_(std)
    momentum = torch.zeros(total, **f32)
    param = torch.empty(total, dtype=torch.bfloat16, device=device)
    for a in range(0, total, FILL_CHUNK):
        b = min(total, a + FILL_CHUNK)
        param[a:b].copy_(master[a:b])
    return MuonBuffers(shapes, offs, master, grad, momentum, param)
