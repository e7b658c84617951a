"""ctypes binding of libhpo (include/hpo.h): argument marshalling only.

Every entry point keeps its C name and argument order; torch tensors are
accepted where the C call takes a device pointer, and `stream=None` means
torch's current stream on the current device.  Every step of the optimizer
runs in the HIP library; nothing here computes on the data.  If libhpo.so is
missing the first call raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhpo.so")

HPO_OK, HPO_EINVAL, HPO_EDTYPE, HPO_ENOMEM, HPO_EHIP, HPO_EDEVICE = 0, -1, -2, -3, -4, -5
HPO_PARAM_BF16, HPO_PARAM_FP32, HPO_PARAM_FP16 = 0, 1, 2
HPO_STATE_BF16 = 0x100
HPO_STATE_FP16 = 0x800
HPO_GRAD_BF16 = 0x200
HPO_MASTER_FP16 = 0x400
HPO_ADAMW, HPO_ADAM_L2 = 0, 1
HPO_MAX_GROUPS = 16


class HpoError(RuntimeError):
    def __init__(self, status: int, call: str, message: str):
        super().__init__(f"{call} failed with {status}: {message}")
        self.status = status


class hpo_adam_cfg(ctypes.Structure):
    _fields_ = [("beta1", ctypes.c_double), ("beta2", ctypes.c_double),
                ("eps", ctypes.c_double), ("mode", ctypes.c_int32)]


class hpo_group(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("weight_decay", ctypes.c_double)]


class hpo_set_info_t(ctypes.Structure):
    _fields_ = [("n_tensors", ctypes.c_int32), ("param_dtype", ctypes.c_int32),
                ("is_flat", ctypes.c_int32), ("chunk_elems", ctypes.c_int32),
                ("numel", ctypes.c_int64), ("n_chunks", ctypes.c_int64),
                ("device_bytes", ctypes.c_int64), ("device", ctypes.c_int32),
                ("n_vector", ctypes.c_int32), ("grad_group", ctypes.c_int32),
                ("kind", ctypes.c_int32), ("n_grad_parts", ctypes.c_int64)]


HPO_SET_ADAM = 0
HPO_SET_MUON = 1
HPO_MUON_MOMENTUM_SUM = 0
HPO_MUON_MOMENTUM_EMA = 1
HPO_MUON_SCALE_SPECTRAL = 0
HPO_MUON_SCALE_SHAPE = 1
HPO_MUON_SCALE_UNIT_RMS = 2
HPO_NS_MAX_STEPS = 16
HPO_MUON_DEFAULT_WORKSPACE = 16 << 30
HPO_MUON_MAX_DIM = 1 << 21


HPO_MUON_PROF_N = 6
MUON_PROF_KINDS = ("momentum", "input", "gram", "poly", "step", "update")


class hpo_muon_profile(ctypes.Structure):
    _fields_ = [("ms", ctypes.c_double * HPO_MUON_PROF_N), ("launches", ctypes.c_int64 * HPO_MUON_PROF_N),
                ("flops", ctypes.c_double * HPO_MUON_PROF_N), ("bytes", ctypes.c_double * HPO_MUON_PROF_N)]


class hpo_muon_cfg(ctypes.Structure):
    _fields_ = [("momentum", ctypes.c_double), ("nesterov", ctypes.c_int32), ("momentum_form", ctypes.c_int32),
                ("ns_steps", ctypes.c_int32), ("scale_mode", ctypes.c_int32), ("extra_scale", ctypes.c_double),
                ("ns_eps", ctypes.c_double), ("ns_coeffs", ctypes.POINTER(ctypes.c_double))]


class hpo_scaler_state(ctypes.Structure):
    _fields_ = [("loss_scale", ctypes.c_float), ("inv_scale", ctypes.c_float),
                ("growth_tracker", ctypes.c_int32), ("hysteresis_tracker", ctypes.c_int32),
                ("applied_steps", ctypes.c_int64), ("skipped_steps", ctypes.c_int64),
                ("grad_norm", ctypes.c_float), ("found_inf", ctypes.c_int32),
                ("applied", ctypes.c_int32), ("error", ctypes.c_int32), ("num_zeros", ctypes.c_int64),
                ("step_inv_scale", ctypes.c_float), ("reserved", ctypes.c_int32)]


class hpo_scaler_cfg(ctypes.Structure):
    _fields_ = [("dynamic", ctypes.c_int32), ("growth_interval", ctypes.c_int32),
                ("hysteresis", ctypes.c_int32), ("growth_factor", ctypes.c_float),
                ("backoff_factor", ctypes.c_float), ("min_scale", ctypes.c_float),
                ("grad_norm_skip_threshold", ctypes.c_double)]


HPO_MAX_WINDOW = 256
SCALER_STATE_BYTES = ctypes.sizeof(hpo_scaler_state)

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_PP = ctypes.POINTER(ctypes.c_void_p)

# name -> (restype, argtypes), exactly as declared in include/hpo.h
SIGNATURES = {
    "hpo_set_create_list": (_I32, [ctypes.POINTER(_P), _I32, _I32, _PP, _PP, _PP, _PP, _PP,
                                   ctypes.POINTER(_I64), ctypes.POINTER(_I32), _P]),
    "hpo_set_create_flat": (_I32, [ctypes.POINTER(_P), _I64, _I32, _P, _P, _P, _P, _P, _P]),
    "hpo_set_create_flat_ranges": (_I32, [ctypes.POINTER(_P), _I64, _I32, _P, _P, _P, _P, _P, _I32,
                                          ctypes.POINTER(_I64), ctypes.POINTER(_I32), _P]),
    "hpo_set_destroy": (_I32, [_P]),
    "hpo_set_info": (_I32, [_P, ctypes.POINTER(hpo_set_info_t)]),
    "hpo_unscale_check_inf": (_I32, [_P, ctypes.c_float, _P, _P]),
    "hpo_grad_global_norm": (_I32, [_P, ctypes.c_float, _P, _P, _P, _P]),
    "hpo_adamw_step": (_I32, [_P, ctypes.POINTER(hpo_adam_cfg), ctypes.POINTER(hpo_group), _I32,
                              _I64, ctypes.c_float, ctypes.c_double, _P, _P, _P]),
    "hpo_copy_main_to_model": (_I32, [_P, _P]),
    "hpo_stream_probe": (_I32, [_P, _P]),
    "hpo_step_device_flat_static": (_I32, [_I64, _I32, _P, _P, _P, _P, _P, ctypes.POINTER(hpo_adam_cfg),
                                           ctypes.POINTER(hpo_group), ctypes.c_double, ctypes.POINTER(hpo_scaler_cfg),
                                           _P, _I64, _I32, _P]),
    "hpo_scaler_state_init": (_I32, [_P, ctypes.c_float, _I32, _I64, _P]),
    "hpo_step_device": (_I32, [_P, ctypes.POINTER(hpo_adam_cfg), ctypes.POINTER(hpo_group), _I32, ctypes.c_double,
                               ctypes.POINTER(hpo_scaler_cfg), _P, _I64, _I32, _P]),
    "hpo_muon_set_create": (_I32, [ctypes.POINTER(_P), _I32, _I32, _PP, _PP, _PP, _PP, ctypes.POINTER(_I64),
                                   ctypes.POINTER(_I64), ctypes.POINTER(_I32), _I64, _P]),
    "hpo_muon_step": (_I32, [_P, ctypes.POINTER(hpo_muon_cfg), ctypes.POINTER(hpo_group), _I32, ctypes.c_float,
                             ctypes.c_double, _P, _P, _P]),
    "hpo_grad_global_norm_sets": (_I32, [ctypes.POINTER(_P), _I32, ctypes.c_float, _P, _P, _P, _P]),
    "hpo_step_device_chain": (_I32, [_P, ctypes.POINTER(hpo_adam_cfg), ctypes.POINTER(hpo_group), _I32, _P,
                                     ctypes.POINTER(hpo_muon_cfg), ctypes.POINTER(hpo_group), _I32, ctypes.c_double,
                                     ctypes.POINTER(hpo_scaler_cfg), _P, _I64, _I32, _P]),
    "hpo_newton_schulz": (_I32, [_P, _I64, _I64, ctypes.POINTER(hpo_muon_cfg), _P, _P, _I64, _P]),
    "hpo_newton_schulz_workspace": (_I32, [_I64, _I64, ctypes.POINTER(_I64)]),
    "hpo_muon_profile_enable": (_I32, [_P, _I32]),
    "hpo_muon_profile_read": (_I32, [_P, ctypes.POINTER(hpo_muon_profile)]),
    "hpo_plan": (_I32, [_I32, ctypes.POINTER(_I64), ctypes.POINTER(_I32), ctypes.POINTER(_I64),
                        ctypes.POINTER(_I64)]),
    "hpo_plan_chunks": (_I32, [_I32, ctypes.POINTER(_I64), _I64, ctypes.POINTER(_I32),
                               ctypes.POINTER(_I64), ctypes.POINTER(_I32)]),
    "hpo_last_error": (ctypes.c_char_p, []),
    "hpo_status_string": (ctypes.c_char_p, [_I32]),
    "hpo_abi_version": (_I32, []),
}

_lib = None


def load(path: str = LIB_PATH):
    """Load libhpo.so (after torch, so that both share torch's HIP runtime)."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run `python -m mixed_precision_optimizer_amd.build` "
                               "(or __graft_entry__.build()). There is no non-HIP fallback.")
        L = ctypes.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(status: int, call: str) -> None:
    if status != HPO_OK:
        msg = load().hpo_last_error().decode(errors="replace")
        raise HpoError(status, call, msg)


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _ptr(t: Optional[torch.Tensor]) -> ctypes.c_void_p:
    if t is None:
        return ctypes.c_void_p(0)
    if isinstance(t, int):
        return ctypes.c_void_p(t)
    return ctypes.c_void_p(t.data_ptr())


def _on_current_device(t: torch.Tensor, what: str) -> None:
    d = t.get_device()   # -1 for a host tensor
    if d < 0:
        raise ValueError(f"{what} must be a device tensor")
    cur = torch.cuda.current_device()
    if d != cur:
        raise ValueError(f"{what} is on {t.device} but the current device is cuda:{cur}")


def _dptr(t, what: str, dtype=None, min_bytes: int = 0) -> ctypes.c_void_p:
    """Device pointer of a buffer argument the kernels read or write.  None is
    NULL and an int is taken as a raw device address; a tensor must live on
    the current device, be contiguous, hold `dtype` and span `min_bytes`, so
    that a host tensor or a short buffer is refused here rather than reaching
    a kernel."""
    if t is None or isinstance(t, int):
        return _ptr(t)
    _on_current_device(t, what)
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{what} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    nbytes = t.numel() * t.element_size()
    if nbytes < min_bytes:
        raise ValueError(f"{what} spans {nbytes} bytes, the call needs {min_bytes}")
    return ctypes.c_void_p(t.data_ptr())


def _flag_ptr(t, what: str = "d_found_inf") -> ctypes.c_void_p:
    return _dptr(t, what, torch.int32, 4)


def _norm_ptr(t, what: str = "d_norm") -> ctypes.c_void_p:
    return _dptr(t, what, torch.float32, 4)


def _zeros_ptr(t, what: str = "d_num_zeros") -> ctypes.c_void_p:
    return _dptr(t, what, torch.int64, 8)


def _state_ptr(t) -> ctypes.c_void_p:
    return _dptr(t, "d_state", None, SCALER_STATE_BYTES)


def _require(t: torch.Tensor, dtype, what: str, i: int) -> None:
    if t.dtype != dtype:
        raise TypeError(f"{what}[{i}] must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{what}[{i}] must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{what}[{i}] must be contiguous")


def _check_params(params: Sequence[Optional[torch.Tensor]], tensors: Sequence[torch.Tensor]) -> None:
    """The 16-bit params of one set share one dtype (the set writes them all
    in one encoding), and every tensor of the set lives on one device: the
    current one, which the library records as the set's device."""
    given = [p for p in params if p is not None]
    dts = {p.dtype for p in given}
    if len(dts) > 1:
        raise TypeError(f"params mix dtypes {sorted(str(d) for d in dts)}; a set writes one encoding")
    everything = list(tensors) + given
    devs = {t.device for t in everything}
    if len(devs) > 1:
        raise ValueError(f"the tensors of a set must share one device, got {sorted(str(d) for d in devs)}")
    if everything and everything[0].is_cuda:   # host tensors are refused tensor by tensor
        _on_current_device(everything[0], "the set's tensors")
    for i, p in enumerate(params):
        if p is not None and not p.is_cuda:
            raise ValueError(f"params[{i}] must be a device tensor")


def param_dtype_code(dtype) -> int:
    """bf16 / fp32 / fp16 -> the library's code; any other dtype goes to the
    library as an unsupported code, which it rejects."""
    if dtype == torch.bfloat16:
        return HPO_PARAM_BF16
    if dtype == torch.float32:
        return HPO_PARAM_FP32
    if dtype == torch.float16:
        return HPO_PARAM_FP16
    return 100 + {torch.float64: 1}.get(dtype, 9)


def _moments_flag(exp_avgs, exp_avg_sqs) -> int:
    """HPO_STATE_BF16 when the moments are bf16 tensors, 0 for fp32; fp16
    moments map to HPO_STATE_FP16, which the library refuses (HPO_EDTYPE).
    Both moments of every tensor must share one of these dtypes."""
    dts = {t.dtype for t in list(exp_avgs) + list(exp_avg_sqs)}
    if not dts or dts == {torch.float32}:
        return 0
    if dts == {torch.bfloat16}:
        return HPO_STATE_BF16
    if dts == {torch.float16}:
        return HPO_STATE_FP16
    raise TypeError(f"exp_avg / exp_avg_sq must all be float32, all bfloat16 or all float16, "
                    f"got {sorted(map(str, dts))}")


def _storage_flags(main_params, main_grads, exp_avgs, exp_avg_sqs):
    """(flags, master dtype, grad dtype, moment dtype) of a set's arrays: the
    master fp32 or fp16 (HPO_MASTER_FP16), the grads fp32 or bf16
    (HPO_GRAD_BF16), the moments fp32 or bf16 (HPO_STATE_BF16); each kind
    shares one dtype over the whole set."""
    flags = _moments_flag(exp_avgs, exp_avg_sqs)
    mdt = {0: torch.float32, HPO_STATE_BF16: torch.bfloat16, HPO_STATE_FP16: torch.float16}[flags]
    out = [flags, torch.float32, torch.float32, mdt]
    for k, what, ts, low, flag in ((1, "main_param", main_params, torch.float16, HPO_MASTER_FP16),
                                   (2, "main_grad", main_grads, torch.bfloat16, HPO_GRAD_BF16)):
        dts = {t.dtype for t in ts}
        if dts == {low}:
            out[0] |= flag
            out[k] = low
        elif dts and dts != {torch.float32}:
            raise TypeError(f"{what} tensors must all be float32 or all {low}, got {sorted(map(str, dts))}")
    return tuple(out)


# --------------------------------------------------------------------------
# entry points (same names as the C ABI)
# --------------------------------------------------------------------------
class HpoSet:
    """Owner of one hpo_set handle; keeps the tensors it points at alive."""

    def __init__(self, handle: ctypes.c_void_p, keepalive):
        self.handle = handle
        self._keep = keepalive

    def info(self) -> hpo_set_info_t:
        return hpo_set_info(self)

    def close(self) -> None:
        if self.handle:
            _check(load().hpo_set_destroy(self.handle), "hpo_set_destroy")
            self.handle = None

    def __del__(self):
        try:
            if self.handle:
                load().hpo_set_destroy(self.handle)
        except Exception:
            pass


def hpo_set_create_list(params: Sequence[Optional[torch.Tensor]], main_params: Sequence[torch.Tensor],
                        main_grads: Sequence[torch.Tensor], exp_avgs: Sequence[torch.Tensor],
                        exp_avg_sqs: Sequence[torch.Tensor], group_index: Optional[Sequence[int]] = None,
                        param_dtype: Optional[int] = None, stream=None) -> HpoSet:
    n = len(main_params)
    if not (len(main_grads) == len(exp_avgs) == len(exp_avg_sqs) == n):
        raise ValueError("all per-tensor lists must have the same length")
    if params is None:
        params = [None] * n
    if len(params) != n:
        raise ValueError("params has the wrong length")
    if param_dtype is None:
        first = next((p for p in params if p is not None), None)
        param_dtype = HPO_PARAM_FP32 if first is None else param_dtype_code(first.dtype)
    mflag, tdt, gdt, mdt = _storage_flags(main_params, main_grads, exp_avgs, exp_avg_sqs)
    _check_params(params, list(main_params) + list(main_grads) + list(exp_avgs) + list(exp_avg_sqs))
    numel = []
    for i in range(n):
        for what, lst, dt in (("main_params", main_params, tdt), ("main_grads", main_grads, gdt),
                              ("exp_avgs", exp_avgs, mdt), ("exp_avg_sqs", exp_avg_sqs, mdt)):
            _require(lst[i], dt, what, i)
            if lst[i].numel() != main_params[i].numel():
                raise ValueError(f"{what}[{i}] has {lst[i].numel()} elements, main_params[{i}] has "
                                 f"{main_params[i].numel()}")
        if params[i] is not None:
            if not params[i].is_contiguous() or params[i].numel() != main_params[i].numel():
                raise ValueError(f"params[{i}] must be contiguous with main_params[{i}]'s size")
        numel.append(main_params[i].numel())
    arr = lambda ts: (ctypes.c_void_p * max(n, 1))(*[(t.data_ptr() if t is not None else 0) for t in ts])
    c_numel = (ctypes.c_int64 * max(n, 1))(*numel)
    c_groups = None
    if group_index is not None:
        if len(group_index) != n:
            raise ValueError("group_index has the wrong length")
        c_groups = (ctypes.c_int32 * max(n, 1))(*group_index)
    out = ctypes.c_void_p()
    st = load().hpo_set_create_list(ctypes.byref(out), n, param_dtype | mflag, arr(params), arr(main_params),
                                    arr(main_grads), arr(exp_avgs), arr(exp_avg_sqs), c_numel, c_groups,
                                    _stream(stream))
    _check(st, "hpo_set_create_list")
    return HpoSet(out, (list(params), list(main_params), list(main_grads), list(exp_avgs), list(exp_avg_sqs)))


def hpo_set_create_flat(param: Optional[torch.Tensor], main_param: torch.Tensor, main_grad: torch.Tensor,
                        exp_avg: torch.Tensor, exp_avg_sq: torch.Tensor, param_dtype: Optional[int] = None,
                        stream=None) -> HpoSet:
    mflag, tdt, gdt, mdt = _storage_flags([main_param], [main_grad], [exp_avg], [exp_avg_sq])
    for what, t, dt in (("main_param", main_param, tdt), ("main_grad", main_grad, gdt),
                        ("exp_avg", exp_avg, mdt), ("exp_avg_sq", exp_avg_sq, mdt)):
        _require(t, dt, what, 0)
        if t.numel() != main_param.numel():
            raise ValueError(f"{what} has the wrong number of elements")
    _check_params([param], [main_param, main_grad, exp_avg, exp_avg_sq])
    if param_dtype is None:
        param_dtype = HPO_PARAM_FP32 if param is None else param_dtype_code(param.dtype)
    if param is not None and (not param.is_contiguous() or param.numel() != main_param.numel()):
        raise ValueError("param must be contiguous with main_param's size")
    out = ctypes.c_void_p()
    st = load().hpo_set_create_flat(ctypes.byref(out), main_param.numel(), param_dtype | mflag, _ptr(param),
                                    _ptr(main_param), _ptr(main_grad), _ptr(exp_avg), _ptr(exp_avg_sq),
                                    _stream(stream))
    _check(st, "hpo_set_create_flat")
    return HpoSet(out, (param, main_param, main_grad, exp_avg, exp_avg_sq))


def hpo_set_create_flat_ranges(param: Optional[torch.Tensor], main_param: torch.Tensor, main_grad: torch.Tensor,
                               exp_avg: torch.Tensor, exp_avg_sq: torch.Tensor, range_start: Sequence[int],
                               range_group: Sequence[int], param_dtype: Optional[int] = None, stream=None) -> HpoSet:
    mflag, tdt, gdt, mdt = _storage_flags([main_param], [main_grad], [exp_avg], [exp_avg_sq])
    for what, t, dt in (("main_param", main_param, tdt), ("main_grad", main_grad, gdt),
                        ("exp_avg", exp_avg, mdt), ("exp_avg_sq", exp_avg_sq, mdt)):
        _require(t, dt, what, 0)
        if t.numel() != main_param.numel():
            raise ValueError(f"{what} has the wrong number of elements")
    _check_params([param], [main_param, main_grad, exp_avg, exp_avg_sq])
    if param_dtype is None:
        param_dtype = HPO_PARAM_FP32 if param is None else param_dtype_code(param.dtype)
    if param is not None and (not param.is_contiguous() or param.numel() != main_param.numel()):
        raise ValueError("param must be contiguous with main_param's size")
    if len(range_start) != len(range_group):
        raise ValueError("range_start and range_group must have the same length")
    k = len(range_start)
    c_start = (ctypes.c_int64 * max(k, 1))(*range_start)
    c_group = (ctypes.c_int32 * max(k, 1))(*range_group)
    out = ctypes.c_void_p()
    st = load().hpo_set_create_flat_ranges(ctypes.byref(out), main_param.numel(), param_dtype | mflag, _ptr(param),
                                           _ptr(main_param), _ptr(main_grad), _ptr(exp_avg), _ptr(exp_avg_sq),
                                           k, c_start, c_group, _stream(stream))
    _check(st, "hpo_set_create_flat_ranges")
    return HpoSet(out, (param, main_param, main_grad, exp_avg, exp_avg_sq))


def hpo_set_destroy(s: HpoSet) -> None:
    s.close()


def hpo_set_info(s: HpoSet) -> hpo_set_info_t:
    info = hpo_set_info_t()
    _check(load().hpo_set_info(s.handle, ctypes.byref(info)), "hpo_set_info")
    return info


def hpo_unscale_check_inf(s: HpoSet, inv_scale: float, d_found_inf, stream=None) -> None:
    flag = _flag_ptr(d_found_inf)
    _check(load().hpo_unscale_check_inf(s.handle, inv_scale, flag, _stream(stream)), "hpo_unscale_check_inf")


def hpo_grad_global_norm(s: HpoSet, inv_scale: float, d_norm, d_found_inf=None, d_num_zeros=None,
                         stream=None) -> None:
    norm, flag, zeros = _norm_ptr(d_norm), _flag_ptr(d_found_inf), _zeros_ptr(d_num_zeros)
    _check(load().hpo_grad_global_norm(s.handle, inv_scale, norm, flag, zeros, _stream(stream)),
           "hpo_grad_global_norm")


def make_cfg(beta1=0.9, beta2=0.999, eps=1e-8, mode=HPO_ADAMW) -> hpo_adam_cfg:
    return hpo_adam_cfg(beta1, beta2, eps, mode)


def make_groups(groups: Sequence[tuple]):
    arr = (hpo_group * max(len(groups), 1))()
    for k, (lr, wd) in enumerate(groups):
        arr[k] = hpo_group(lr, wd)
    return arr, len(groups)


def hpo_adamw_step(s: HpoSet, cfg: hpo_adam_cfg, groups, n_groups: Optional[int], t: int,
                   inv_scale: float, max_norm: float, d_norm=None, d_found_inf=None, stream=None) -> None:
    """`groups` is either a ctypes hpo_group array (with n_groups) or a list of
    (lr, weight_decay) tuples (n_groups may then be None)."""
    if not isinstance(groups, ctypes.Array):
        groups, n_groups = make_groups(groups)
    norm, flag = _norm_ptr(d_norm), _flag_ptr(d_found_inf)
    _check(load().hpo_adamw_step(s.handle, ctypes.byref(cfg), groups, n_groups, t, inv_scale, max_norm,
                                 norm, flag, _stream(stream)), "hpo_adamw_step")


def new_scaler_state(device=None) -> torch.Tensor:
    """Device buffer for one hpo_scaler_state (64 bytes, 8-byte aligned)."""
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    return torch.zeros(SCALER_STATE_BYTES // 8, dtype=torch.int64, device=dev)


def read_scaler_state(d_state: torch.Tensor) -> hpo_scaler_state:
    """Copies the state to the host (synchronises d_state's stream)."""
    raw = d_state.cpu().numpy().tobytes()
    return hpo_scaler_state.from_buffer_copy(raw)


def make_scaler_cfg(dynamic=True, growth_interval=1000, hysteresis=2, growth_factor=2.0, backoff_factor=0.5,
                    min_scale=1.0, grad_norm_skip_threshold=float("inf")) -> hpo_scaler_cfg:
    return hpo_scaler_cfg(int(dynamic), growth_interval, hysteresis, growth_factor, backoff_factor, min_scale,
                          grad_norm_skip_threshold)


def hpo_scaler_state_init(d_state, loss_scale: float, hysteresis: int, applied_steps: int = 0, stream=None) -> None:
    state = _state_ptr(d_state)
    _check(load().hpo_scaler_state_init(state, loss_scale, hysteresis, applied_steps, _stream(stream)),
           "hpo_scaler_state_init")


def hpo_step_device(s: HpoSet, cfg: hpo_adam_cfg, groups, n_groups: Optional[int], max_norm: float,
                    scfg: hpo_scaler_cfg, d_state, t_first: int, window: int, stream=None) -> None:
    if not isinstance(groups, ctypes.Array):
        groups, n_groups = make_groups(groups)
    state = _state_ptr(d_state)
    _check(load().hpo_step_device(s.handle, ctypes.byref(cfg), groups, n_groups, max_norm, ctypes.byref(scfg),
                                  state, t_first, window, _stream(stream)), "hpo_step_device")


HPO_STATIC_MAX_PARTS = 1 << 18


def hpo_step_device_flat_static(param: Optional[torch.Tensor], main_param: torch.Tensor, main_grad: torch.Tensor,
                                exp_avg: torch.Tensor, exp_avg_sq: torch.Tensor, cfg: hpo_adam_cfg, group: tuple,
                                max_norm: float, scfg: hpo_scaler_cfg, d_state, t_first: int, window: int,
                                param_dtype: Optional[int] = None, stream=None) -> None:
    """hpo_set_create_flat + hpo_step_device over one group, with no set and
    no device allocation (the library keeps the reduction partials in a
    static device array); `group` is (lr, weight_decay)."""
    mflag, tdt, gdt, mdt = _storage_flags([main_param], [main_grad], [exp_avg], [exp_avg_sq])
    n = main_param.numel()
    ptrs = []
    for what, t, dt in (("main_param", main_param, tdt), ("main_grad", main_grad, gdt),
                        ("exp_avg", exp_avg, mdt), ("exp_avg_sq", exp_avg_sq, mdt)):
        if t.numel() != n:
            raise ValueError(f"{what} has {t.numel()} elements, main_param {n}")
        ptrs.append(_dptr(t, what, dt))
    if param_dtype is None:
        param_dtype = HPO_PARAM_FP32 if param is None else param_dtype_code(param.dtype)
    if param is not None and param.numel() != n:
        raise ValueError("param must have main_param's size")
    p_ptr = _dptr(param, "param")
    g = hpo_group(*group)
    _check(load().hpo_step_device_flat_static(n, param_dtype | mflag, p_ptr, *ptrs, ctypes.byref(cfg), ctypes.byref(g),
                                              max_norm, ctypes.byref(scfg), _state_ptr(d_state), t_first, window,
                                              _stream(stream)), "hpo_step_device_flat_static")


def hpo_stream_probe(s: HpoSet, stream=None) -> None:
    _check(load().hpo_stream_probe(s.handle, _stream(stream)), "hpo_stream_probe")


def hpo_copy_main_to_model(s: HpoSet, stream=None) -> None:
    _check(load().hpo_copy_main_to_model(s.handle, _stream(stream)), "hpo_copy_main_to_model")


# ---------------------------------------------------------------------------
# Muon
# ---------------------------------------------------------------------------
def make_muon_cfg(momentum=0.95, nesterov=True, momentum_form=HPO_MUON_MOMENTUM_SUM, ns_steps=5,
                  scale_mode=HPO_MUON_SCALE_SPECTRAL, extra_scale=0.2, ns_eps=1e-7, ns_coeffs=None) -> hpo_muon_cfg:
    """Defaults: the handbook's Muon (Nesterov, sum form, 5 steps of the
    original quintic) with Moonlight's 0.2 * sqrt(max(A, B)) update scale."""
    cfg = hpo_muon_cfg(momentum=momentum, nesterov=int(bool(nesterov)), momentum_form=momentum_form,
                       ns_steps=ns_steps, scale_mode=scale_mode, extra_scale=extra_scale, ns_eps=ns_eps)
    if ns_coeffs is not None:
        flat = [float(x) for c in ns_coeffs for x in c]
        if len(flat) != 3 * ns_steps:
            raise ValueError("ns_coeffs needs one (a, b, c) per step")
        cfg._coeffs = (ctypes.c_double * len(flat))(*flat)  # kept alive with the struct
        cfg.ns_coeffs = ctypes.cast(cfg._coeffs, ctypes.POINTER(ctypes.c_double))
    return cfg


def hpo_muon_set_create(params: Sequence[Optional[torch.Tensor]], main_params: Sequence[torch.Tensor],
                        main_grads: Sequence[torch.Tensor], momenta: Sequence[torch.Tensor],
                        group_index: Optional[Sequence[int]] = None, workspace_bytes: int = 0,
                        stream=None) -> HpoSet:
    """A Muon set over 2-D matrices (each tensor's shape gives rows x cols)."""
    n = len(main_params)
    if not (len(main_grads) == len(momenta) == n):
        raise ValueError("all per-matrix lists must have the same length")
    if params is None:
        params = [None] * n
    if len(params) != n:
        raise ValueError("params has the wrong length")
    first = next((p for p in params if p is not None), None)
    param_dtype = HPO_PARAM_FP32 if first is None else param_dtype_code(first.dtype)
    _check_params(params, list(main_params) + list(main_grads) + list(momenta))
    rows, cols = [], []
    for i in range(n):
        if main_params[i].dim() != 2:
            raise ValueError(f"main_params[{i}] is not a matrix")
        for what, lst in (("main_params", main_params), ("main_grads", main_grads), ("momenta", momenta)):
            _require(lst[i], torch.float32, what, i)
            if tuple(lst[i].shape) != tuple(main_params[i].shape):
                raise ValueError(f"{what}[{i}] has shape {tuple(lst[i].shape)}, main_params[{i}] "
                                 f"{tuple(main_params[i].shape)}")
        if params[i] is not None and (not params[i].is_contiguous()
                                      or tuple(params[i].shape) != tuple(main_params[i].shape)):
            raise ValueError(f"params[{i}] must be contiguous with main_params[{i}]'s shape")
        rows.append(main_params[i].shape[0])
        cols.append(main_params[i].shape[1])
    arr = lambda ts: (ctypes.c_void_p * max(n, 1))(*[(t.data_ptr() if t is not None else 0) for t in ts])
    c_rows = (ctypes.c_int64 * max(n, 1))(*rows)
    c_cols = (ctypes.c_int64 * max(n, 1))(*cols)
    c_groups = None
    if group_index is not None:
        if len(group_index) != n:
            raise ValueError("group_index has the wrong length")
        c_groups = (ctypes.c_int32 * max(n, 1))(*group_index)
    out = ctypes.c_void_p()
    st = load().hpo_muon_set_create(ctypes.byref(out), n, param_dtype, arr(params), arr(main_params),
                                    arr(main_grads), arr(momenta), c_rows, c_cols, c_groups, workspace_bytes,
                                    _stream(stream))
    _check(st, "hpo_muon_set_create")
    return HpoSet(out, (list(params), list(main_params), list(main_grads), list(momenta)))


def hpo_muon_step(s: HpoSet, cfg: hpo_muon_cfg, groups, n_groups: Optional[int], inv_scale: float = 1.0,
                  max_norm: float = 0.0, d_norm=None, d_found_inf=None, stream=None) -> None:
    if not isinstance(groups, ctypes.Array):
        groups, n_groups = make_groups(groups)
    norm, flag = _norm_ptr(d_norm), _flag_ptr(d_found_inf)
    _check(load().hpo_muon_step(s.handle, ctypes.byref(cfg), groups, n_groups, inv_scale, max_norm, norm, flag,
                                _stream(stream)), "hpo_muon_step")


def hpo_grad_global_norm_sets(sets: Sequence[HpoSet], inv_scale: float, d_norm, d_found_inf=None,
                              d_num_zeros=None, stream=None) -> None:
    handles = (ctypes.c_void_p * max(len(sets), 1))(*[x.handle for x in sets])
    norm, flag, zeros = _norm_ptr(d_norm), _flag_ptr(d_found_inf), _zeros_ptr(d_num_zeros)
    _check(load().hpo_grad_global_norm_sets(handles, len(sets), inv_scale, norm, flag, zeros, _stream(stream)),
           "hpo_grad_global_norm_sets")


def hpo_step_device_chain(adam_set: Optional[HpoSet], cfg: Optional[hpo_adam_cfg], groups,
                          muon_set: Optional[HpoSet], mcfg: Optional[hpo_muon_cfg], muon_groups, max_norm: float,
                          scfg: hpo_scaler_cfg, d_state, t_first: int, window: int, stream=None) -> None:
    g, ng = make_groups(groups) if groups else (None, 0)
    mg, nmg = make_groups(muon_groups) if muon_groups else (None, 0)
    state = _state_ptr(d_state)
    _check(load().hpo_step_device_chain(adam_set.handle if adam_set else None,
                                        ctypes.byref(cfg) if cfg is not None else None, g, ng,
                                        muon_set.handle if muon_set else None,
                                        ctypes.byref(mcfg) if mcfg is not None else None, mg, nmg, max_norm,
                                        ctypes.byref(scfg), state, t_first, window, _stream(stream)),
           "hpo_step_device_chain")


def hpo_newton_schulz_workspace(rows: int, cols: int) -> int:
    out = ctypes.c_int64()
    _check(load().hpo_newton_schulz_workspace(rows, cols, ctypes.byref(out)), "hpo_newton_schulz_workspace")
    return out.value


def hpo_newton_schulz(G: torch.Tensor, out: torch.Tensor, cfg: hpo_muon_cfg, workspace: torch.Tensor,
                      stream=None) -> None:
    """O = NS(G) on the device: G and out fp32 (rows, cols) contiguous; the
    workspace a uint8 device tensor of at least hpo_newton_schulz_workspace bytes."""
    for what, t in (("G", G), ("out", out)):
        if t.dtype != torch.float32 or not t.is_contiguous() or t.dim() != 2:
            raise ValueError(f"{what} must be a contiguous fp32 matrix")
    if tuple(out.shape) != tuple(G.shape):
        raise ValueError("out must have G's shape")
    g_ptr, o_ptr = _dptr(G, "G"), _dptr(out, "out")
    ws_ptr = _dptr(workspace, "workspace")
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(load().hpo_newton_schulz(g_ptr, G.shape[0], G.shape[1], ctypes.byref(cfg), o_ptr, ws_ptr, ws_bytes,
                                    _stream(stream)), "hpo_newton_schulz")


def hpo_muon_profile_enable(s: HpoSet, enable: bool = True) -> None:
    _check(load().hpo_muon_profile_enable(s.handle, int(bool(enable))), "hpo_muon_profile_enable")


def hpo_muon_profile_read(s: HpoSet) -> dict:
    """{kind: {"ms", "launches", "flops", "bytes"}} since the last read."""
    out = hpo_muon_profile()
    _check(load().hpo_muon_profile_read(s.handle, ctypes.byref(out)), "hpo_muon_profile_read")
    return {k: {"ms": out.ms[i], "launches": out.launches[i], "flops": out.flops[i], "bytes": out.bytes[i]}
            for i, k in enumerate(MUON_PROF_KINDS)}


def hpo_plan(numel: Sequence[int]):
    """(chunk_elems, n_chunks, device_bytes) of a list set over these sizes."""
    n = len(numel)
    c_numel = (ctypes.c_int64 * max(n, 1))(*numel)
    ch, nc, nb = ctypes.c_int32(), ctypes.c_int64(), ctypes.c_int64()
    _check(load().hpo_plan(n, c_numel, ctypes.byref(ch), ctypes.byref(nc), ctypes.byref(nb)), "hpo_plan")
    return ch.value, nc.value, nb.value


def hpo_plan_chunks(numel: Sequence[int]):
    """Chunk table of a list set over these sizes: (tensor, start, len) arrays."""
    import numpy as np
    _, nc, _ = hpo_plan(numel)
    n = len(numel)
    c_numel = (ctypes.c_int64 * max(n, 1))(*numel)
    ten = np.empty(max(nc, 1), np.int32)
    start = np.empty(max(nc, 1), np.int64)
    ln = np.empty(max(nc, 1), np.int32)
    _check(load().hpo_plan_chunks(n, c_numel, nc, ten.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                  start.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                  ln.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))), "hpo_plan_chunks")
    return ten[:nc], start[:nc], ln[:nc]


def hpo_last_error() -> str:
    return load().hpo_last_error().decode(errors="replace")


def hpo_status_string(status: int) -> str:
    return load().hpo_status_string(status).decode()


def hpo_abi_version() -> int:
    return load().hpo_abi_version()
