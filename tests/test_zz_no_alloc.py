"""The device step with no allocation (hpo_step_device_flat_static, through
the C ABI) against the set-based device step (hpo_set_create_flat +
hpo_step_device) over copies of the same arrays: every state array and the
56-byte scaler state must match bit for bit after every step.

Two calls in a row share the library's static partials: first a shard large
enough for the two-stage finalize (9156 grad-pass partials), then a smaller
one that reads fewer partials than the first left behind; then a shard off
its vector lines (element-by-element path).  Each runs three steps with a
dynamic loss scale, planted zeros and an inf at step 2.
"""
import pytest
import torch

from gpu_util import banner, require_gpu

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def H():
    return require_gpu()


def _state_bytes(d_state):
    return d_state.cpu().numpy().tobytes()


def _same(a, b):
    if a.dtype in (torch.bfloat16, torch.float16):
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


def _pair(H, n, seed, shift=0, steps=3):
    from mixed_precision_optimizer_amd import inputs
    banner(f"no-alloc step vs set step: {n} elements, shift {shift}, {steps} steps")
    gen = torch.Generator(device=DEV)
    gen.manual_seed(seed)
    th = torch.randn(n + shift, generator=gen, device=DEV)[shift:]
    arrays = {}
    for side in ("set", "static"):
        a = {"theta": torch.empty(n + shift, device=DEV)[shift:], "grad": torch.empty(n + shift, device=DEV)[shift:],
             "m": torch.zeros(n + shift, device=DEV)[shift:], "v": torch.zeros(n + shift, device=DEV)[shift:],
             "p": torch.empty(n + shift, dtype=torch.bfloat16, device=DEV)[shift:]}
        a["theta"].copy_(th)
        a["p"].copy_(th)
        arrays[side] = a
    cfg = H.make_cfg()
    scfg = H.make_scaler_cfg(dynamic=True, growth_interval=2, hysteresis=1)
    states = {k: H.new_scaler_state() for k in arrays}
    for d in states.values():
        H.hpo_scaler_state_init(d, 1024.0, 1)
    A = arrays["set"]
    hset = H.hpo_set_create_flat(A["p"], A["theta"], A["grad"], A["m"], A["v"])
    B = arrays["static"]
    for k in range(1, steps + 1):
        g = torch.randn(n, generator=gen, device=DEV).mul_(1e-3 * 1024.0)
        inputs.plant_zeros_(g, 997, k)
        if k == 2:
            g[n // 3] = float("inf")
        A["grad"].copy_(g)
        B["grad"].copy_(g)
        H.hpo_step_device(hset, cfg, [(1e-3, 0.1)], None, 1.0, scfg, states["set"], 1, k)
        H.hpo_step_device_flat_static(B["p"], B["theta"], B["grad"], B["m"], B["v"], cfg, (1e-3, 0.1), 1.0, scfg,
                                      states["static"], 1, k)
        torch.cuda.synchronize()
        for key in A:
            assert _same(A[key], B[key]), f"step {k}: {key} differs"
        sa, sb = _state_bytes(states["set"]), _state_bytes(states["static"])
        assert sa == sb, f"step {k}: scaler state differs"
        st = H.hpo_scaler_state.from_buffer_copy(sb)
        assert st.error == 0
        assert bool(st.applied) == (k != 2), k
        if k != 2:
            assert st.num_zeros >= n // 997 - 2, st.num_zeros
    st = H.hpo_scaler_state.from_buffer_copy(_state_bytes(states["static"]))
    assert st.applied_steps == steps - 1 and st.skipped_steps == 1
    hset.close()
    del arrays
    torch.cuda.empty_cache()


def test_static_step_matches_the_set_step_twice_smaller_second(H):
    _pair(H, 600_000_001, seed=11)
    _pair(H, 1_000_003, seed=12)
    _pair(H, 250_001, seed=13, shift=1)

