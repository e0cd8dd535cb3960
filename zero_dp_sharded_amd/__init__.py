"""zero_dp_sharded_amd -- the owner-rank step of ZeRO-DP (P_os / P_os+g) on gfx950.

A thin ctypes binding of libzeroshard.so (include/zero_shard.h).  Functions
carry the C names and do argument marshalling only: torch tensors become
device pointers and a torch stream becomes its hipStream_t.  Every step of the
path runs in the library's HIP kernels; there is no CPU fallback, and calling
anything without the built library raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
# ZERO_SHARD_LIB: another build of the library (a tuning variant, see build.py)
LIB_PATH = os.environ.get("ZERO_SHARD_LIB") or os.path.join(HERE, "libzeroshard.so")

ZERO_OK = 0
ZERO_ERR_INVALID_ARG = 1
ZERO_ERR_STATE = 2
ZERO_ERR_HIP = 3
ZERO_ERR_OOM = 4
ZERO_ERR_UNSUPPORTED = 5

ZERO_FP16 = 1
ZERO_BF16 = 2
ZERO_FP32 = 3
ZERO_WD_DECOUPLED = 0
ZERO_WD_L2 = 1
ZERO_MAX_CONTRIB = 64

ABI_SYMBOLS = (
    "zero_state_bytes", "zero_state_bytes_ex", "zero_shard_init", "zero_shard_init_sgd",
    "zero_bucket_reduce", "zero_overflow_check", "zero_overflow_merge", "zero_adam_step",
    "zero_adam_step_gated", "zero_sgd_step", "zero_sgd_step_gated", "zero_step_resolve",
    "zero_shard_set_clip", "zero_device_begin", "zero_step_device", "zero_device_end",
    "zero_shard_inline_folds", "zero_adam_step_noalloc", "zero_shard_get_counters",
    "zero_shard_set_counters", "zero_shard_destroy", "zero_status_str", "zero_last_error",
    "zero_abi_version",
)

_i32, _i64, _f64, _vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p


class ZeroShardDesc(ctypes.Structure):
    _fields_ = [("psi", _i64), ("nd", _i32), ("rank", _i32), ("bucket_elems", _i64),
                ("lp", ctypes.c_int), ("master", _vp), ("exp_avg", _vp), ("exp_avg_sq", _vp),
                ("grad_shard", _vp), ("param_shard", _vp)]


class ZeroAdamHParams(ctypes.Structure):
    _fields_ = [("lr", _f64), ("beta1", _f64), ("beta2", _f64), ("eps", _f64),
                ("weight_decay", _f64), ("bias_correction", _i32), ("wd_mode", ctypes.c_int),
                ("initial_step", _i64)]


class ZeroSgdHParams(ctypes.Structure):
    _fields_ = [("lr", _f64), ("momentum", _f64), ("weight_decay", _f64), ("initial_step", _i64)]


class ZeroLossScaleCfg(ctypes.Structure):
    _fields_ = [("init_scale", _f64), ("dynamic", _i32), ("growth_interval", _i32),
                ("min_scale", _f64)]


class ZeroStepInfo(ctypes.Structure):
    _fields_ = [("overflow", _i32), ("skipped", _i32), ("step_t", _i64), ("grad_norm", _f64),
                ("scale_used", _f64), ("scale_next", _f64)]


class ZeroStateBytes(ctypes.Structure):
    _fields_ = [("shard_elems", _i64), ("bytes_master", _i64), ("bytes_m", _i64),
                ("bytes_v", _i64), ("bytes_grad", _i64), ("bytes_param", _i64),
                ("bytes_shard_total", _i64), ("bytes_staging", _i64),
                ("per_rank_stage", _f64 * 4), ("comm_bytes_stage", _f64 * 4),
                ("comm_bytes_stage1_with_gather", _f64), ("comp_params", _f64 * 4),
                ("comp_grads", _f64 * 4), ("comp_optim", _f64 * 4)]


class ZeroError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: {_status_name(status)}: {detail}")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library.  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m zero_dp_sharded_amd.build` "
                "(or __graft_entry__.build()); there is no fallback path")
        L = ctypes.CDLL(LIB_PATH)
        L.zero_state_bytes.argtypes = [_i64, _i32, _i32, _i64, ctypes.c_int,
                                       ctypes.POINTER(ZeroStateBytes)]
        L.zero_state_bytes_ex.argtypes = [_i64, _i32, _i32, _i64, ctypes.c_int, _i32, _i32,
                                          ctypes.POINTER(ZeroStateBytes)]
        L.zero_shard_init.argtypes = [ctypes.POINTER(ZeroShardDesc),
                                      ctypes.POINTER(ZeroAdamHParams),
                                      ctypes.POINTER(ZeroLossScaleCfg), ctypes.POINTER(_vp)]
        L.zero_shard_init_sgd.argtypes = [ctypes.POINTER(ZeroShardDesc),
                                          ctypes.POINTER(ZeroSgdHParams),
                                          ctypes.POINTER(ZeroLossScaleCfg), ctypes.POINTER(_vp)]
        L.zero_sgd_step.argtypes = [_vp, ctypes.POINTER(ZeroSgdHParams), _vp,
                                    ctypes.POINTER(ZeroStepInfo)]
        L.zero_sgd_step_gated.argtypes = [_vp, ctypes.POINTER(ZeroSgdHParams), _vp]
        L.zero_bucket_reduce.argtypes = [_vp, ctypes.POINTER(_vp), _i32, _i64, _i64, _vp]
        L.zero_overflow_check.argtypes = [_vp, _vp, ctypes.POINTER(ZeroStepInfo)]
        L.zero_adam_step.argtypes = [_vp, ctypes.POINTER(ZeroAdamHParams), _vp,
                                     ctypes.POINTER(ZeroStepInfo)]
        L.zero_overflow_merge.argtypes = [_vp, _i32, _f64, ctypes.POINTER(ZeroStepInfo)]
        L.zero_adam_step_gated.argtypes = [_vp, ctypes.POINTER(ZeroAdamHParams), _vp]
        L.zero_step_resolve.argtypes = [_vp, ctypes.POINTER(ZeroStepInfo)]
        L.zero_shard_set_clip.argtypes = [_vp, _f64]
        L.zero_device_begin.argtypes = [_vp, _vp]
        L.zero_step_device.argtypes = [_vp, ctypes.POINTER(_vp), _i32, _vp]
        L.zero_device_end.argtypes = [_vp, _vp, ctypes.POINTER(ZeroStepInfo)]
        L.zero_shard_inline_folds.argtypes = [_vp, ctypes.POINTER(_i64)]
        L.zero_adam_step_noalloc.argtypes = [
            ctypes.POINTER(ZeroShardDesc), ctypes.POINTER(ZeroAdamHParams),
            ctypes.POINTER(ZeroLossScaleCfg), _f64, ctypes.POINTER(_vp), _i32,
            ctypes.POINTER(_i64), ctypes.POINTER(_f64), ctypes.POINTER(_i64), _vp,
            ctypes.POINTER(ZeroStepInfo)]
        L.zero_shard_get_counters.argtypes = [_vp, ctypes.POINTER(_i64), ctypes.POINTER(_f64),
                                              ctypes.POINTER(_i64)]
        L.zero_shard_set_counters.argtypes = [_vp, _i64, _f64, _i64]
        L.zero_shard_destroy.argtypes = [_vp]
        L.zero_status_str.argtypes = [ctypes.c_int]
        L.zero_status_str.restype = ctypes.c_char_p
        L.zero_last_error.restype = ctypes.c_char_p
        L.zero_last_error.argtypes = []
        L.zero_abi_version.restype = ctypes.c_int
        L.zero_abi_version.argtypes = []
        for name in ABI_SYMBOLS:
            if name not in ("zero_status_str", "zero_last_error", "zero_abi_version"):
                getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _status_name(s: int) -> str:
    return lib().zero_status_str(s).decode()


def _check(status: int, where: str) -> None:
    if status != ZERO_OK:
        raise ZeroError(status, where, lib().zero_last_error().decode())


def zero_abi_version() -> int:
    return int(lib().zero_abi_version())


def zero_status_str(status: int) -> str:
    return _status_name(status)


def zero_last_error() -> str:
    return lib().zero_last_error().decode()


# ------------------------------------------------------------------ parameters

@dataclass
class AdamHParams:
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.0
    bias_correction: int = 1
    wd_mode: int = ZERO_WD_DECOUPLED
    initial_step: int = 0

    def to_c(self) -> ZeroAdamHParams:
        return ZeroAdamHParams(self.lr, self.beta1, self.beta2, self.eps, self.weight_decay,
                               self.bias_correction, self.wd_mode, self.initial_step)


@dataclass
class SGDHParams:
    lr: float = 1e-2
    momentum: float = 0.0
    weight_decay: float = 0.0
    initial_step: int = 0

    def to_c(self) -> ZeroSgdHParams:
        return ZeroSgdHParams(self.lr, self.momentum, self.weight_decay, self.initial_step)


@dataclass
class LossScaleCfg:
    init_scale: float = 1.0
    dynamic: int = 1
    growth_interval: int = 1000
    min_scale: float = 1.0

    def to_c(self) -> ZeroLossScaleCfg:
        return ZeroLossScaleCfg(self.init_scale, self.dynamic, self.growth_interval,
                                self.min_scale)


@dataclass
class StepInfo:
    overflow: int
    skipped: int
    step_t: int
    grad_norm: float
    scale_used: float
    scale_next: float

    @staticmethod
    def from_c(c: ZeroStepInfo) -> "StepInfo":
        return StepInfo(c.overflow, c.skipped, c.step_t, c.grad_norm, c.scale_used, c.scale_next)


# ------------------------------------------------------------------ marshalling

def _stream_ptr(stream) -> Optional[int]:
    """hipStream_t of a torch stream, or of torch's current stream if None."""
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _dptr(x) -> int:
    """Device address of a GPU tensor (or an int address, passed through)."""
    if isinstance(x, int):
        return x
    if x.device.type != "cuda":
        raise ValueError(f"expected a GPU tensor, got one on {x.device}")
    return x.data_ptr()


# Storage dtype and shard size of each live handle made through this binding,
# so contribution tensors can be checked before their addresses cross the ABI
# (the library sees only allocations, not the tensors inside them).
_handles = {}


def _contrib_ptrs(h: int, contribs: Sequence, n_elems: int, who: str) -> list:
    """Addresses of contribution tensors (ints pass through unchecked); each
    tensor must be a contiguous GPU tensor of the handle's storage dtype with
    at least n_elems elements."""
    meta = _handles.get(h)
    out = []
    for r, c in enumerate(contribs):
        if isinstance(c, int):
            out.append(c)
            continue
        if meta is not None:
            _check_tensor(f"{who}: contribution {r}", c, meta[0], n_elems)
        out.append(_dptr(c))
    return out


def _ledger(out: ZeroStateBytes) -> dict:
    d = {}
    for name, _ in ZeroStateBytes._fields_:
        v = getattr(out, name)
        d[name] = list(v) if hasattr(v, "__len__") else v
    return d


def zero_state_bytes(psi: int, nd: int, n_contrib: int, bucket_elems: int,
                     lp: int = ZERO_FP16) -> dict:
    out = ZeroStateBytes()
    _check(lib().zero_state_bytes(psi, nd, n_contrib, bucket_elems, lp, ctypes.byref(out)),
           "zero_state_bytes")
    return _ledger(out)


def zero_state_bytes_ex(psi: int, nd: int, n_contrib: int, bucket_elems: int, lp: int,
                        param_bytes: int, k_optim: int) -> dict:
    out = ZeroStateBytes()
    _check(lib().zero_state_bytes_ex(psi, nd, n_contrib, bucket_elems, lp, param_bytes,
                                     k_optim, ctypes.byref(out)), "zero_state_bytes_ex")
    return _ledger(out)


def _check_tensor(name, t, dtype, n):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_contiguous() or t.numel() < n:
        raise ValueError(f"{name}: must be contiguous with at least {n} elements")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must live on the GPU, got {t.device}")


def _lp_of(grad_shard):
    import torch
    lp = {torch.float16: ZERO_FP16, torch.bfloat16: ZERO_BF16,
          torch.float32: ZERO_FP32}.get(grad_shard.dtype)
    if lp is None:
        raise TypeError(f"grad_shard must be float16, bfloat16 or float32, got {grad_shard.dtype}")
    return lp


def _desc_of(master, exp_avg, exp_avg_sq, grad_shard, param_shard, psi, nd, rank,
             bucket_elems) -> ZeroShardDesc:
    """Descriptor over torch tensors (None for an absent array).  fp32
    grad_shard selects 4-byte storage, which takes no param_shard."""
    import torch
    lp = _lp_of(grad_shard)
    S = -(-psi // nd)
    for name, t, dt in (("master", master, torch.float32), ("exp_avg", exp_avg, torch.float32),
                        ("exp_avg_sq", exp_avg_sq, torch.float32),
                        ("grad_shard", grad_shard, grad_shard.dtype),
                        ("param_shard", param_shard, grad_shard.dtype)):
        if t is not None:
            _check_tensor(name, t, dt, S)
    ptr = lambda t: None if t is None else t.data_ptr()
    return ZeroShardDesc(psi, nd, rank, bucket_elems, lp, ptr(master), ptr(exp_avg),
                         ptr(exp_avg_sq), ptr(grad_shard), ptr(param_shard))


def zero_shard_init(master, exp_avg, exp_avg_sq, grad_shard, param_shard, *, psi: int,
                    nd: int, rank: int, bucket_elems: int, hp: AdamHParams,
                    ls: LossScaleCfg) -> int:
    """Create an Adam handle over caller-owned torch tensors; returns the handle.
    fp32 grad_shard: 4-byte storage, param_shard None."""
    desc = _desc_of(master, exp_avg, exp_avg_sq, grad_shard, param_shard, psi, nd, rank,
                    bucket_elems)
    h = _vp()
    _check(lib().zero_shard_init(ctypes.byref(desc), ctypes.byref(hp.to_c()),
                                 ctypes.byref(ls.to_c()), ctypes.byref(h)), "zero_shard_init")
    _handles[h.value] = (grad_shard.dtype, -(-psi // nd))
    return h.value


def zero_shard_init_sgd(master, momentum_buf, grad_shard, param_shard, *, psi: int, nd: int,
                        rank: int, bucket_elems: int, hp: SGDHParams, ls: LossScaleCfg) -> int:
    """Create an SGD handle; momentum_buf None for plain SGD."""
    desc = _desc_of(master, momentum_buf, None, grad_shard, param_shard, psi, nd, rank,
                    bucket_elems)
    h = _vp()
    _check(lib().zero_shard_init_sgd(ctypes.byref(desc), ctypes.byref(hp.to_c()),
                                     ctypes.byref(ls.to_c()), ctypes.byref(h)),
           "zero_shard_init_sgd")
    _handles[h.value] = (grad_shard.dtype, -(-psi // nd))
    return h.value


def zero_bucket_reduce(h: int, contribs: Sequence, bucket_off: int, bucket_len: int,
                       stream=None) -> None:
    """contribs: R tensors (or device addresses), each holding this bucket's
    bucket_len gradients of one contribution in the storage format."""
    ptrs = _contrib_ptrs(h, contribs, bucket_len, "zero_bucket_reduce")
    arr = (_vp * len(ptrs))(*ptrs)
    _check(lib().zero_bucket_reduce(h, arr, len(contribs), bucket_off, bucket_len,
                                    _stream_ptr(stream)), "zero_bucket_reduce")


def zero_overflow_check(h: int, stream=None) -> StepInfo:
    out = ZeroStepInfo()
    _check(lib().zero_overflow_check(h, _stream_ptr(stream), ctypes.byref(out)),
           "zero_overflow_check")
    return StepInfo.from_c(out)


def zero_adam_step(h: int, hp: Optional[AdamHParams] = None, stream=None) -> StepInfo:
    out = ZeroStepInfo()
    hpc = ctypes.byref(hp.to_c()) if hp is not None else None
    _check(lib().zero_adam_step(h, hpc, _stream_ptr(stream), ctypes.byref(out)),
           "zero_adam_step")
    return StepInfo.from_c(out)


def zero_overflow_merge(h: int, global_overflow: int, global_grad_norm: float) -> StepInfo:
    out = ZeroStepInfo()
    _check(lib().zero_overflow_merge(h, global_overflow, global_grad_norm, ctypes.byref(out)),
           "zero_overflow_merge")
    return StepInfo.from_c(out)


def zero_adam_step_gated(h: int, hp: Optional[AdamHParams] = None, stream=None) -> None:
    hpc = ctypes.byref(hp.to_c()) if hp is not None else None
    _check(lib().zero_adam_step_gated(h, hpc, _stream_ptr(stream)), "zero_adam_step_gated")


def zero_sgd_step(h: int, hp: Optional[SGDHParams] = None, stream=None) -> StepInfo:
    out = ZeroStepInfo()
    hpc = ctypes.byref(hp.to_c()) if hp is not None else None
    _check(lib().zero_sgd_step(h, hpc, _stream_ptr(stream), ctypes.byref(out)), "zero_sgd_step")
    return StepInfo.from_c(out)


def zero_sgd_step_gated(h: int, hp: Optional[SGDHParams] = None, stream=None) -> None:
    hpc = ctypes.byref(hp.to_c()) if hp is not None else None
    _check(lib().zero_sgd_step_gated(h, hpc, _stream_ptr(stream)), "zero_sgd_step_gated")


def zero_step_resolve(h: int) -> StepInfo:
    out = ZeroStepInfo()
    _check(lib().zero_step_resolve(h, ctypes.byref(out)), "zero_step_resolve")
    return StepInfo.from_c(out)


def zero_shard_set_clip(h: int, max_grad_norm: float) -> None:
    _check(lib().zero_shard_set_clip(h, max_grad_norm), "zero_shard_set_clip")


def zero_device_begin(h: int, stream=None) -> None:
    _check(lib().zero_device_begin(h, _stream_ptr(stream)), "zero_device_begin")


def zero_step_device(h: int, contribs: Optional[Sequence] = None, stream=None) -> None:
    """Enqueue one whole device-resident step; contribs are R shard-sized
    tensors (or device addresses), None to scan a caller-filled grad_shard.
    Capturable in a graph."""
    if contribs is None:
        arr, n = None, 0
    else:
        meta = _handles.get(h)
        ptrs = _contrib_ptrs(h, contribs, meta[1] if meta else 0, "zero_step_device")
        arr, n = (_vp * len(ptrs))(*ptrs), len(ptrs)
    _check(lib().zero_step_device(h, arr, n, _stream_ptr(stream)), "zero_step_device")


def zero_shard_inline_folds(h: int) -> int:
    """Device-resident steps of this handle whose update folded the partials
    itself (no fold launch)."""
    n = _i64()
    _check(lib().zero_shard_inline_folds(h, ctypes.byref(n)), "zero_shard_inline_folds")
    return n.value


def zero_device_end(h: int, stream=None) -> StepInfo:
    out = ZeroStepInfo()
    _check(lib().zero_device_end(h, _stream_ptr(stream), ctypes.byref(out)), "zero_device_end")
    return StepInfo.from_c(out)


def zero_adam_step_noalloc(master, exp_avg, exp_avg_sq, grad_shard, param_shard, *, psi: int,
                           nd: int, rank: int, bucket_elems: int, hp: AdamHParams,
                           ls: LossScaleCfg, counters, contribs: Optional[Sequence] = None,
                           max_grad_norm: float = 0.0, stream=None):
    """One whole synchronous Adam step with no handle and no device allocation
    (the check's scratch is the library's static array).  counters = (step_t,
    scale, good_steps) before the step; returns (StepInfo, counters after)."""
    desc = _desc_of(master, exp_avg, exp_avg_sq, grad_shard, param_shard, psi, nd, rank,
                    bucket_elems)
    S = -(-psi // nd)
    if contribs is None:
        arr, n = None, 0
    else:
        ptrs = []
        for r, c in enumerate(contribs):
            if not isinstance(c, int):
                _check_tensor(f"zero_adam_step_noalloc: contribution {r}", c, grad_shard.dtype, S)
            ptrs.append(_dptr(c))
        arr, n = (_vp * len(ptrs))(*ptrs), len(ptrs)
    t, sc, g = _i64(counters[0]), _f64(counters[1]), _i64(counters[2])
    out = ZeroStepInfo()
    _check(lib().zero_adam_step_noalloc(ctypes.byref(desc), ctypes.byref(hp.to_c()),
                                        ctypes.byref(ls.to_c()), max_grad_norm, arr, n,
                                        ctypes.byref(t), ctypes.byref(sc), ctypes.byref(g),
                                        _stream_ptr(stream), ctypes.byref(out)),
           "zero_adam_step_noalloc")
    return StepInfo.from_c(out), (t.value, sc.value, g.value)


def zero_shard_get_counters(h: int):
    t, s, g = _i64(), _f64(), _i64()
    _check(lib().zero_shard_get_counters(h, ctypes.byref(t), ctypes.byref(s), ctypes.byref(g)),
           "zero_shard_get_counters")
    return t.value, s.value, g.value


def zero_shard_set_counters(h: int, step_t: int, scale: float, good_steps: int) -> None:
    _check(lib().zero_shard_set_counters(h, step_t, scale, good_steps),
           "zero_shard_set_counters")


def zero_shard_destroy(h: int) -> None:
    _check(lib().zero_shard_destroy(h), "zero_shard_destroy")
    _handles.pop(h, None)


def reduce_buckets(h: int, contribs: Sequence, shard_elems: int, bucket_elems: int,
                   stream=None, esz: Optional[int] = None) -> None:
    """Submit every C_B bucket of a step in ascending order.  contribs are R
    shard-sized tensors (or addresses); bucket b passes the views
    [off, off + len).  esz, the bytes per element, defaults to the handle's
    storage format (2 for an address whose handle this binding did not make)."""
    meta = _handles.get(h)
    if esz is None:
        esz = meta[0].itemsize if meta is not None else 2
    ptrs = _contrib_ptrs(h, contribs, shard_elems, "reduce_buckets")
    for off in range(0, shard_elems, bucket_elems):
        ln = min(bucket_elems, shard_elems - off)
        zero_bucket_reduce(h, [p + off * esz for p in ptrs], off, ln, stream)
