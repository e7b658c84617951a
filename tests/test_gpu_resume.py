"""Resume equivalence of the chained AdamW + Muon device step.

[FP32-RFC] section 2 ("core guard cases"), case 2.2: train, save the model
weights, the Muon and AdamW states and the fp32 main params, build a new
trainer from the saved files, continue on the same next batch, and compare
with a run that never stopped.  Here everything a step depends on lives in
caller-owned buffers plus the 64-byte device scaler state (which holds the
applied-step counter), so "save" is a host copy of those buffers, "load"
builds fresh device buffers and fresh sets from the copies, and the
continued run must match the uninterrupted one bit for bit: AdamW master, m,
v and bf16 params; Muon master, momentum and bf16 params; the scaler state.
The restored masters are the fp32 copies: rebuilding them from the bf16
params would lose the tail bits the check below shows they carry.
"""
import numpy as np
import pytest
import torch

from gpu_util import banner, require_gpu

pytestmark = pytest.mark.gpu

F32 = np.float32
ADAM_SHAPES = [(3000,), (256,), (64 * 50,)]
ADAM_GROUP = [0, 0, 1]
GROUPS = [(1e-3, 0.0), (1e-3, 0.1)]            # no-decay (norm gains), decaying
MUON_SHAPES = [(128, 384), (384, 128), (300, 700), (37, 129)]
MUON_GROUP = [0, 1, 0, 1]
MUON_GROUPS = [(0.02, 0.1), (0.01, 0.0)]
STEPS, SAVE_AFTER, INF_STEP = 6, 2, 4


@pytest.fixture(scope="module")
def H():
    return require_gpu()


def _grads(I, k, scale):
    ga = [(I.seeded_matrix(s, 900 * k + i, 1e-2).ravel() * F32(scale)).astype(F32)
          for i, s in enumerate(ADAM_SHAPES)]
    gm = [(I.seeded_matrix(s, 700 * k + i, 1e-2) * F32(scale)).astype(F32) for i, s in enumerate(MUON_SHAPES)]
    if k == INF_STEP:
        gm[1][3, 3] = np.inf
    return ga, gm


class Run:
    """Device buffers, sets and scaler state of one training run."""

    def __init__(self, H, dev, host=None):
        from mixed_precision_optimizer_amd import inputs as I
        if host is None:   # fresh start, seeded
            am = [I.seeded_matrix(s, 500 + i, 0.02).ravel() for i, s in enumerate(ADAM_SHAPES)]
            mm = [I.seeded_matrix(s, 600 + i, 0.02) for i, s in enumerate(MUON_SHAPES)]
            host = {"am": am, "a1": [np.zeros_like(a) for a in am], "a2": [np.zeros_like(a) for a in am],
                    "ap": [torch.from_numpy(a).to(torch.bfloat16) for a in am],
                    "mm": mm, "mo": [np.zeros_like(m) for m in mm],
                    "mp": [torch.from_numpy(m).to(torch.bfloat16) for m in mm], "state": None}
        up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
        self.am = [up(a) for a in host["am"]]
        self.a1 = [up(a) for a in host["a1"]]
        self.a2 = [up(a) for a in host["a2"]]
        self.ap = [p.to(dev) for p in host["ap"]]
        self.ag = [torch.zeros_like(t) for t in self.am]
        self.mm = [up(m) for m in host["mm"]]
        self.mo = [up(m) for m in host["mo"]]
        self.mp = [p.to(dev) for p in host["mp"]]
        self.mg = [torch.zeros_like(t) for t in self.mm]
        self.aset = H.hpo_set_create_list(self.ap, self.am, self.ag, self.a1, self.a2, ADAM_GROUP)
        self.mset = H.hpo_muon_set_create(self.mp, self.mm, self.mg, self.mo, MUON_GROUP)
        self.state = H.new_scaler_state(dev)
        if host["state"] is None:
            H.hpo_scaler_state_init(self.state, 2.0 ** 16, 1, 0)
        else:
            self.state.copy_(host["state"].to(dev))
        torch.cuda.synchronize()

    def step(self, H, I, k):
        st = H.read_scaler_state(self.state)
        ga, gm = _grads(I, k, st.loss_scale)
        for t, g in zip(self.ag + self.mg, ga + gm):
            t.copy_(torch.from_numpy(g))
        H.hpo_step_device_chain(self.aset, H.make_cfg(), GROUPS, self.mset, H.make_muon_cfg(), MUON_GROUPS, 1.0,
                                H.make_scaler_cfg(dynamic=True, growth_interval=2, hysteresis=1), self.state,
                                st.applied_steps + 1, 1)
        torch.cuda.synchronize()

    def save(self):
        """Host copies of every caller-owned buffer the next step reads."""
        host = lambda ts: [t.cpu().numpy().copy() for t in ts]
        out = {"am": host(self.am), "a1": host(self.a1), "a2": host(self.a2), "ap": [p.cpu() for p in self.ap],
               "mm": host(self.mm), "mo": host(self.mo), "mp": [p.cpu() for p in self.mp],
               "state": self.state.cpu()}
        self.aset.close()
        self.mset.close()
        return out

    def bits(self):
        u32 = lambda ts: [t.cpu().numpy().view(np.uint32) for t in ts]
        u16 = lambda ts: [t.view(torch.int16).cpu().numpy() for t in ts]
        return {"am": u32(self.am), "a1": u32(self.a1), "a2": u32(self.a2), "ap": u16(self.ap),
                "mm": u32(self.mm), "mo": u32(self.mo), "mp": u16(self.mp),
                "state": [self.state.cpu().numpy()]}


def test_save_restore_continue_matches_continuous(H):
    banner("resume: save, rebuild, continue vs continuous")
    from mixed_precision_optimizer_amd import inputs as I
    dev = torch.device("cuda")
    ref = Run(H, dev)
    for k in range(1, STEPS + 1):
        ref.step(H, I, k)
    want = ref.bits()
    st_ref = H.read_scaler_state(ref.state)
    assert st_ref.applied_steps == STEPS - 1 and st_ref.error == 0   # the inf step was skipped
    ref.aset.close()
    ref.mset.close()

    first = Run(H, dev)
    for k in range(1, SAVE_AFTER + 1):
        first.step(H, I, k)
    saved = first.save()
    del first
    torch.cuda.synchronize()
    # the fp32 masters carry bits that their bf16 params do not
    tail = [m.view(np.uint32) & 0xFFFF for m in saved["am"] + saved["mm"]]
    assert any(np.any(t != 0) for t in tail)

    resumed = Run(H, dev, host=saved)
    for k in range(SAVE_AFTER + 1, STEPS + 1):
        resumed.step(H, I, k)
    got = resumed.bits()
    for key in want:
        for i, (a, b) in enumerate(zip(want[key], got[key])):
            assert np.array_equal(a, b), f"{key}[{i}] differs after resume"
    resumed.aset.close()
    resumed.mset.close()
