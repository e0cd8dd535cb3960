"""Scalar CPU oracle for the ZeRO-DP owner-rank step -- TEST INFRASTRUCTURE.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product library never loads it, and it imports
nothing from the product package: the two share no code.

The arithmetic lives in ``zero_oracle.c`` (plain scalar C, one element at a
time, in the order the method defines).  This module marshals numpy arrays to
it and composes whole steps, in the order the pages describe:

  reduce each C_B bucket of the owner's shard   ("ZeRO：大模型训练的内存优化革命",
                                                  3.1.2 and 3.2.2)
  -> overflow flag and gradient norm            (pages silent; reading below)
  -> Adam on the fp32 shard, cast to 2 bytes     (same page, 3.1.1; "SC-2020 ZeRO"
                                                  notes, "Where Did All the Memory Go?")

It also holds the per-rank byte ledger of the blog.vllbc.top ZeRO/DeepSpeed
page (stage formulas, Table 1, worked examples) and that page's GB display
rule, so the ledger can be compared with the printed tables.

Parity status: every function here is pinned by tests/test_oracle*.py against
the pages' printed tables, closed forms of Adam, library conversions (numpy
float16, torch bfloat16) or brute force; none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field
from fractions import Fraction
from typing import Callable, List, Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# ZERO_ORACLE_LIB points the pin tests at a deliberately broken copy of the
# oracle (tests/test_oracle_mutations.py); normally unset.
LIB_PATH = os.environ.get("ZERO_ORACLE_LIB") or os.path.join(HERE, "liboracle.so")

FP16 = 1
BF16 = 2
FP32 = 3      # 4-byte storage of grads, contributions and params (b = 4)

_lib = None

_u16p = ctypes.POINTER(ctypes.c_uint16)
_f32p = ctypes.POINTER(ctypes.c_float)
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_vp = ctypes.c_void_p


class _Bytes(ctypes.Structure):
    _fields_ = [
        ("shard_elems", ctypes.c_int64),
        ("bytes_master", ctypes.c_int64), ("bytes_m", ctypes.c_int64),
        ("bytes_v", ctypes.c_int64), ("bytes_grad", ctypes.c_int64),
        ("bytes_param", ctypes.c_int64), ("bytes_shard_total", ctypes.c_int64),
        ("bytes_staging", ctypes.c_int64),
        ("per_rank_stage", ctypes.c_double * 4),
        ("comm_bytes_stage", ctypes.c_double * 4),
        ("comm_bytes_stage1_with_gather", ctypes.c_double),
        ("comp_params", ctypes.c_double * 4),
        ("comp_grads", ctypes.c_double * 4),
        ("comp_optim", ctypes.c_double * 4),
    ]


def lib():
    """Load liboracle.so, building it with gcc if it is not there yet."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from . import build as _b
            _b.build()
        L = ctypes.CDLL(LIB_PATH)
        L.oracle_f16_to_f32.restype = ctypes.c_float
        L.oracle_f16_to_f32.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_to_f32.restype = ctypes.c_float
        L.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.oracle_f32_to_f16.restype = ctypes.c_uint16
        L.oracle_f32_to_f16.argtypes = [ctypes.c_float]
        L.oracle_f32_to_bf16.restype = ctypes.c_uint16
        L.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
        L.oracle_lp_to_f32_array.argtypes = [_i32, _u16p, _i64, _f32p]
        L.oracle_f32_to_lp_array.argtypes = [_i32, _f32p, _i64, _u16p]
        L.oracle_partition.argtypes = [_i64, _i32, _i32, ctypes.POINTER(_i64),
                                       ctypes.POINTER(_i64), ctypes.POINTER(_i64)]
        L.oracle_take_shard_u16.argtypes = [_u16p, _i64, _i32, _i32, _u16p]
        L.oracle_take_shard_f32.argtypes = [_f32p, _i64, _i32, _i32, _f32p]
        L.oracle_bucket_reduce.argtypes = [_i32, _i32, ctypes.POINTER(_vp), _i64, _vp]
        L.oracle_flag_sumsq.argtypes = [_i32, _vp, _i64, ctypes.c_float,
                                        ctypes.POINTER(_i32), ctypes.POINTER(ctypes.c_double)]
        L.oracle_adam_scalars.argtypes = [ctypes.c_double] * 5 + [_i32, _i64, ctypes.c_double, _f32p]
        L.oracle_adam_update.argtypes = [_i32, _i64, _vp, _f32p, _f32p, _f32p, _vp, _f32p, _i32]
        L.oracle_sgd_update.argtypes = [_i32, _i64, _vp, _f32p, _f32p, _vp, _f32p]
        L.oracle_clip_coef.argtypes = [ctypes.c_double, ctypes.c_double]
        L.oracle_clip_coef.restype = ctypes.c_float
        L.oracle_loss_scale_next.argtypes = [_i32, _i32, _i32, ctypes.c_double,
                                             ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_i64)]
        L.oracle_state_bytes.argtypes = [_i64, _i32, _i32, _i64, _i32, _i32, _i32,
                                         ctypes.POINTER(_Bytes)]
        _lib = L
    return _lib


def _p16(a: np.ndarray):
    assert a.dtype == np.uint16 and a.flags.c_contiguous
    return a.ctypes.data_as(_u16p)


def _p32(a: np.ndarray):
    assert a.dtype == np.float32 and a.flags.c_contiguous
    return a.ctypes.data_as(_f32p)


def _store_dtype(lp: int):
    return np.float32 if lp == FP32 else np.uint16


def _pg(lp: int, a: Optional[np.ndarray]):
    """Pointer to gradient-like storage: uint16 bits, or fp32 values for FP32."""
    if a is None:
        return None
    assert a.dtype == _store_dtype(lp) and a.flags.c_contiguous, (a.dtype, lp)
    return a.ctypes.data_as(_vp)


# ---------------------------------------------------------------- 2-byte formats

def lp_to_f32(lp: int, bits: np.ndarray) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.shape, np.float32)
    lib().oracle_lp_to_f32_array(lp, _p16(bits), bits.size, _p32(out))
    return out


def f32_to_lp(lp: int, x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().oracle_f32_to_lp_array(lp, _p32(x), x.size, _p16(out))
    return out


# ---------------------------------------------------------------- partition (a1)

def partition(psi: int, nd: int, rank: int):
    """(S, begin, valid) of rank's shard of a flat Psi-element buffer."""
    s, b, v = _i64(), _i64(), _i64()
    lib().oracle_partition(psi, nd, rank, ctypes.byref(s), ctypes.byref(b), ctypes.byref(v))
    return s.value, b.value, v.value


def take_shard(flat: np.ndarray, nd: int, rank: int) -> np.ndarray:
    flat = np.ascontiguousarray(flat)
    s, _, _ = partition(flat.size, nd, rank)
    if flat.dtype == np.uint16:
        out = np.empty(s, np.uint16)
        lib().oracle_take_shard_u16(_p16(flat), flat.size, nd, rank, _p16(out))
    else:
        flat = flat.astype(np.float32, copy=False)
        out = np.empty(s, np.float32)
        lib().oracle_take_shard_f32(_p32(flat), flat.size, nd, rank, _p32(out))
    return out


# ---------------------------------------------------------------- reduce (a2)

def bucket_reduce(lp: int, contribs: Sequence[np.ndarray]) -> np.ndarray:
    """Mean of R contributions, fp32 accumulate in ascending order."""
    dt = _store_dtype(lp)
    cs = [np.ascontiguousarray(c, dtype=dt) for c in contribs]
    n = cs[0].size
    assert all(c.size == n for c in cs)
    arr = (_vp * len(cs))(*[c.ctypes.data for c in cs])
    out = np.empty(n, dt)
    lib().oracle_bucket_reduce(lp, len(cs), arr, n, _pg(lp, out))
    return out


def reduce_shard(lp: int, contribs: Sequence[np.ndarray], bucket_elems: int) -> np.ndarray:
    """Reduce a whole shard one C_B bucket at a time, buckets in ascending order."""
    n = contribs[0].size
    out = np.empty(n, _store_dtype(lp))
    for off in range(0, n, bucket_elems):
        end = min(n, off + bucket_elems)
        out[off:end] = bucket_reduce(lp, [c[off:end] for c in contribs])
    return out


# ---------------------------------------------------------------- flag / norm (a3)

def flag_sumsq(lp: int, g: np.ndarray, scale: float, flag: int = 0, sumsq: float = 0.0):
    g = np.ascontiguousarray(g, dtype=_store_dtype(lp))
    f = _i32(flag)
    s = ctypes.c_double(sumsq)
    inv = float(np.float32(1.0 / scale))
    lib().oracle_flag_sumsq(lp, _pg(lp, g), g.size, inv, ctypes.byref(f), ctypes.byref(s))
    return f.value, s.value


# ---------------------------------------------------------------- Adam (a4, a5)

@dataclass
class AdamHP:
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.0
    bias_correction: int = 1
    wd_mode: int = 0          # 0 decoupled (AdamW form), 1 L2
    initial_step: int = 0


@dataclass
class LossScale:
    init_scale: float = 1.0
    dynamic: int = 1
    growth_interval: int = 1000
    min_scale: float = 1.0


def clip_coef(sumsq: float, max_norm: float) -> float:
    """Global-norm clipping coefficient min(1, max_norm / (sqrt(sumsq) + 1e-6))
    in fp64, rounded to fp32; 1 when max_norm <= 0 (textbook clipping; the
    pages are silent)."""
    return float(lib().oracle_clip_coef(sumsq, max_norm))


def adam_scalars(hp: AdamHP, t: int, scale: float, coef: float = 1.0) -> np.ndarray:
    # the update uses the fp32 roundings of the betas; one that rounds to 1
    # leaves a zero bias correction (Adam needs beta < 1)
    if not (np.float32(hp.beta1) < 1 and np.float32(hp.beta2) < 1):
        raise ValueError("betas must stay below 1 after rounding to fp32")
    out = np.empty(11, np.float32)
    lib().oracle_adam_scalars(hp.beta1, hp.beta2, hp.lr, hp.eps, hp.weight_decay,
                              hp.bias_correction, t, scale, _p32(out))
    out[10] = np.float32(coef)
    return out


def adam_update(lp: int, grad: np.ndarray, master: np.ndarray, m: np.ndarray,
                v: np.ndarray, param: Optional[np.ndarray], sc: np.ndarray,
                wd_mode: int = 0) -> None:
    """In place: master, m, v (fp32) and param (2-byte bits; None with FP32
    storage, where master is the parameter)."""
    n = master.size
    assert grad.size == n and (param is None or param.size == n)
    for a in (master, m, v):
        assert a.size == n and a.dtype == np.float32
    lib().oracle_adam_update(lp, n, _pg(lp, grad), _p32(master), _p32(m), _p32(v),
                             _pg(lp, param), _p32(np.ascontiguousarray(sc, np.float32)), wd_mode)


@dataclass
class SGDHP:
    """Heavy-ball SGD with L2 weight decay; momentum 0 with no buffer = plain SGD."""
    lr: float = 1e-2
    momentum: float = 0.9
    weight_decay: float = 0.0
    initial_step: int = 0


def sgd_scalars(hp: SGDHP, scale: float, coef: float = 1.0) -> np.ndarray:
    return np.array([hp.lr, hp.momentum, hp.weight_decay, 1.0 / scale, coef],
                    dtype=np.float64).astype(np.float32)


def sgd_update(lp: int, grad: np.ndarray, master: np.ndarray, momentum: Optional[np.ndarray],
               param: Optional[np.ndarray], sc: np.ndarray) -> None:
    """In place: master (and the momentum buffer, and 2-byte param bits)."""
    n = master.size
    assert grad.size == n and master.dtype == np.float32
    if momentum is not None:
        assert momentum.size == n and momentum.dtype == np.float32
    lib().oracle_sgd_update(lp, n, _pg(lp, grad), _p32(master),
                            None if momentum is None else _p32(momentum), _pg(lp, param),
                            _p32(np.ascontiguousarray(sc, np.float32)))


def loss_scale_next(overflow: int, ls: LossScale, scale: float, good_steps: int):
    s = ctypes.c_double(scale)
    g = _i64(good_steps)
    lib().oracle_loss_scale_next(overflow, ls.dynamic, ls.growth_interval, ls.min_scale,
                                 ctypes.byref(s), ctypes.byref(g))
    return s.value, g.value


# ---------------------------------------------------------------- whole steps

@dataclass
class StepInfo:
    overflow: int
    skipped: int
    step_t: int
    grad_norm: float
    scale_used: float
    scale_next: float


@dataclass
class ShardState:
    """The owner's shard: fp32 master / m / v and the gradient / param storage
    (2-byte bits, or fp32 values with FP32 storage, where param is None and
    master is the parameter).  For SGD, m is the momentum buffer (None for
    plain SGD) and v is None."""
    lp: int
    master: np.ndarray
    m: Optional[np.ndarray]
    v: Optional[np.ndarray]
    grad: np.ndarray
    param: Optional[np.ndarray]
    t: int = 0
    scale: float = 1.0
    good_steps: int = 0

    def copy(self) -> "ShardState":
        c = lambda a: None if a is None else a.copy()
        return ShardState(self.lp, self.master.copy(), c(self.m), c(self.v), self.grad.copy(),
                          c(self.param), self.t, self.scale, self.good_steps)


def new_state(lp: int, master: np.ndarray, m, v, hp, ls: LossScale) -> ShardState:
    n = master.size
    st = ShardState(lp, np.array(master, np.float32),
                    None if m is None else np.array(m, np.float32),
                    None if v is None else np.array(v, np.float32),
                    np.zeros(n, _store_dtype(lp)), None,
                    t=hp.initial_step, scale=float(ls.init_scale), good_steps=0)
    if lp != FP32:
        st.param = f32_to_lp(lp, st.master)
    return st


def bucket_flag_sumsq(lp: int, g: np.ndarray, scale: float, bucket_elems: int):
    """Overflow flag and squared unscaled norm of a shard's stored gradient:
    one fp64 sum per C_B bucket (its squares added in element order), the
    bucket sums added in bucket order.  (The pages fix no order; this one lets
    a chunked evaluation, one bucket per chunk, reproduce it bitwise.)"""
    flag, sumsq = 0, 0.0
    for off in range(0, g.size, bucket_elems):
        f, s = flag_sumsq(lp, g[off:off + bucket_elems], scale)
        flag |= f
        sumsq += s
    return flag, sumsq


def step(st: ShardState, contribs: Sequence[np.ndarray], bucket_elems: int,
         hp, ls: LossScale, max_norm: float = 0.0,
         clip_sumsq: Optional[float] = None) -> StepInfo:
    """One owner-rank step on the whole shard held in memory; hp is an AdamHP
    or an SGDHP.  clip_sumsq is the squared norm the clipping coefficient is
    taken from (default: this shard's; a global norm over several shards
    otherwise).  max_norm > 0 clips the unscaled gradient to that global
    norm."""
    st.grad = reduce_shard(st.lp, contribs, bucket_elems)
    flag, sumsq = bucket_flag_sumsq(st.lp, st.grad, st.scale, bucket_elems)
    coef = 1.0
    if not flag:
        coef = clip_coef(sumsq if clip_sumsq is None else clip_sumsq, max_norm)
    scale_used = st.scale
    if flag:
        skipped = 1
    else:
        skipped = 0
        st.t += 1
        if isinstance(hp, SGDHP):
            sgd_update(st.lp, st.grad, st.master, st.m, st.param,
                       sgd_scalars(hp, st.scale, coef))
        else:
            sc = adam_scalars(hp, st.t, st.scale, coef)
            adam_update(st.lp, st.grad, st.master, st.m, st.v, st.param, sc, hp.wd_mode)
    st.scale, st.good_steps = loss_scale_next(flag, ls, st.scale, st.good_steps)
    return StepInfo(flag, skipped, st.t, float(np.sqrt(sumsq)), scale_used, st.scale)


# ---------------------------------------------------------------- chunked evaluation

@dataclass
class ChunkStep:
    """The decision of one step of a chunked run: its overflow flag, squared
    norm, the loss scale its gradients carried, the applied-step count t the
    update uses (unchanged by a skip) and the clipping coefficient."""
    overflow: int
    sumsq: float
    scale: float
    t: int
    coef: float


class ChunkedRun:
    """k steps over a shard too large to hold whole, one C_B bucket (chunk) at
    a time, with the results of the whole-shard steps, bitwise.  Everything
    but the overflow decision and the norm is per element, so:

      pass 1 (scan_step, once per step, in step order): reduce every chunk of
        the step's contributions, take the flag and the squared norm over all
        chunks, decide the step (skip, t, clipping coefficient) and the next
        loss scale;
      pass 2 (evolve, once per chunk, any chunk order): apply the recorded
        steps to the chunk's state, given its reduced gradient of each step.

    A step's contributions depend on the loss scale, which depends on the
    flags of the steps before it, so pass 1 must see the steps in order.
    hp: an AdamHP or an SGDHP."""

    def __init__(self, lp: int, n: int, bucket_elems: int, hp, ls: LossScale,
                 max_norm: float = 0.0, threads: int = 1):
        self.lp, self.n, self.bucket_elems = lp, n, bucket_elems
        self.hp, self.ls, self.max_norm, self.threads = hp, ls, max_norm, max(1, threads)
        self.t = hp.initial_step
        self.scale = float(ls.init_scale)
        self.good_steps = 0
        self.steps: List[ChunkStep] = []

    def chunks(self):
        cb = self.bucket_elems
        return [(off, min(cb, self.n - off)) for off in range(0, self.n, cb)]

    def scan_step(self, contribs_of: Callable[[int, int], Sequence[np.ndarray]],
                  grads_out: Optional[np.ndarray] = None) -> StepInfo:
        """Pass 1 of the next step.  contribs_of(off, n) returns the R
        contributions of shard elements [off, off + n) (stored values, drawn
        with the current self.scale); it is called in chunk order from this
        thread.  Chunks are reduced on worker threads; their flags and sums
        combine in chunk order.  grads_out (n elements) receives the reduced
        gradient."""
        from collections import deque
        from concurrent.futures import ThreadPoolExecutor

        def work(cs):
            g = bucket_reduce(self.lp, cs)
            return g, flag_sumsq(self.lp, g, self.scale)

        flag, sumsq = 0, 0.0

        def finish(off, n, fut):
            nonlocal flag, sumsq
            g, (f, s) = fut.result()
            flag |= f
            sumsq += s
            if grads_out is not None:
                grads_out[off:off + n] = g

        with ThreadPoolExecutor(self.threads) as ex:
            pending = deque()
            for off, n in self.chunks():
                pending.append((off, n, ex.submit(work, contribs_of(off, n))))
                while len(pending) > self.threads:
                    finish(*pending.popleft())
            while pending:
                finish(*pending.popleft())
        return self._decide(flag, sumsq)

    def check_step(self, stored_of: Callable[[int, int], np.ndarray]) -> StepInfo:
        """Pass 1 of the next step when the gradient is already stored (the P_os
        case: the owner's slice of an all-reduced gradient, no reduce).
        stored_of(off, n) returns the stored gradient of shard elements
        [off, off + n); flags and sums combine in chunk order as in
        scan_step."""
        from collections import deque
        from concurrent.futures import ThreadPoolExecutor

        flag, sumsq = 0, 0.0
        with ThreadPoolExecutor(self.threads) as ex:
            pending = deque()
            for off, n in self.chunks():
                pending.append(ex.submit(flag_sumsq, self.lp, stored_of(off, n), self.scale))
                while len(pending) > self.threads:
                    f, s = pending.popleft().result()
                    flag |= f
                    sumsq += s
            while pending:
                f, s = pending.popleft().result()
                flag |= f
                sumsq += s
        return self._decide(flag, sumsq)

    def _decide(self, flag: int, sumsq: float) -> StepInfo:
        scale_used = self.scale
        coef = 1.0
        if not flag:
            self.t += 1
            coef = clip_coef(sumsq, self.max_norm)
        self.steps.append(ChunkStep(flag, sumsq, scale_used, self.t, coef))
        self.scale, self.good_steps = loss_scale_next(flag, self.ls, self.scale, self.good_steps)
        return StepInfo(flag, flag, self.t, float(np.sqrt(sumsq)), scale_used, self.scale)

    def evolve(self, master: np.ndarray, m: Optional[np.ndarray], v: Optional[np.ndarray],
               param: Optional[np.ndarray], grad_of: Callable[[int], np.ndarray]) -> None:
        """Pass 2 for one chunk: apply every recorded step, in order, to the
        chunk's state (in place; m / v / param None where absent).
        grad_of(s) returns the chunk's reduced gradient of step s."""
        for s, rec in enumerate(self.steps):
            if rec.overflow:
                continue
            g = grad_of(s)
            if isinstance(self.hp, SGDHP):
                sgd_update(self.lp, g, master, m, param, sgd_scalars(self.hp, rec.scale, rec.coef))
            else:
                adam_update(self.lp, g, master, m, v, param,
                            adam_scalars(self.hp, rec.t, rec.scale, rec.coef), self.hp.wd_mode)


def run_steps(st: ShardState, contribs_for_step: Callable[[int, float], Sequence[np.ndarray]],
              nsteps: int, bucket_elems: int, hp: AdamHP, ls: LossScale) -> List[StepInfo]:
    """contribs_for_step(step_index, loss_scale) -> the R contributions of that step."""
    infos = []
    for s in range(nsteps):
        infos.append(step(st, contribs_for_step(s, st.scale), bucket_elems, hp, ls))
    return infos


# ---------------------------------------------------------------- ledger (a6)

def state_bytes(psi: int, nd: int, n_contrib: int = 1, bucket_elems: int = 1,
                lp_bytes: int = 2, param_bytes: int = 2, k_optim: int = 12) -> dict:
    out = _Bytes()
    lib().oracle_state_bytes(psi, nd, n_contrib, bucket_elems, lp_bytes, param_bytes,
                             k_optim, ctypes.byref(out))
    d = {}
    for name, _ in _Bytes._fields_:
        val = getattr(out, name)
        d[name] = list(val) if hasattr(val, "__len__") else val
    return d


def display_gb(x) -> str:
    """GB display rule of the blog.vllbc.top ZeRO/DeepSpeed page (calculator
    rules under the stage formulas): GB = 1e9 bytes; at or above 100 GB the
    integer part is shown; from 10 to 100 GB at most one decimal; below 10 GB
    at most two decimals; trailing zeros are dropped.  Table 1 shows that the
    >= 100 case truncates (4187.5 -> 4187) and that smaller values round half
    up (41.25 -> 41.3).  x is an exact byte count (int or Fraction)."""
    g = Fraction(x) / Fraction(10 ** 9)
    if g >= 100:
        q = int(g)                       # floor for non-negative values
        return str(q)
    digits = 1 if g >= 10 else 2
    scale = 10 ** digits
    q = (g * scale + Fraction(1, 2)).__floor__()
    s = f"{q // scale}.{q % scale:0{digits}d}".rstrip("0").rstrip(".")
    return s
