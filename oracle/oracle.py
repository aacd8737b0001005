"""ctypes wrapper of the CPU oracle (oracle.cpp) plus the per-step composition.

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the
benchmark's CPU-baseline leg, never by the product package.  Arrays are numpy;
fp16 and bf16 values travel as uint16 bit patterns.

The step composition (`shard_step`) follows the order in which the
pages describe one rank's optimizer step over its FlatParameter shard:
  Reduce-Scatter's reduce ("DeepSpeed 与 FSDP", ZeRO-2; "PyTorch FSDP 源码级深度解析" §3.3)
  -> unscale + overflow test + global norm (ZeRO reading at 2kiu.com, §5.1/§5.3)
  -> skip on overflow, else clip + AdamW on the fp32 master ("DeepSpeed 与 FSDP",
     ZeRO-Offload Adam equations; 2kiu.com §5.1 AdamW hyper-parameters)
  -> fp16/bf16 write-back into the All-Gather slot ("PyTorch FSDP 源码级深度解析" §7.2)
  -> optional blockwise INT8 of that slot ("DeepSpeed 与 FSDP", ZeRO++)
  -> loss-scaler update (2kiu.com §5.1/§5.3).
"""
import ctypes as C
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")

F32, F16, BF16 = 0, 1, 2
SUM, AVG = 0, 1

class Hparams(C.Structure):
    _fields_ = [("lr", C.c_double), ("beta1", C.c_double), ("beta2", C.c_double),
                ("eps", C.c_double), ("weight_decay", C.c_double),
                ("max_grad_norm", C.c_double)]


class Scaler(C.Structure):
    _fields_ = [("loss_scale", C.c_float), ("min_scale", C.c_float),
                ("dynamic", C.c_int32), ("window", C.c_int32),
                ("good_steps", C.c_int32), ("step", C.c_int32)]

    def as_tuple(self):
        return (self.loss_scale, self.min_scale, self.dynamic, self.window,
                self.good_steps, self.step)


_lib = None


def lib():
    """The oracle library.  ORACLE_LIB may name another build of oracle.cpp
    (the mutation tests load planted-mistake copies this way)."""
    global _lib
    if _lib is None:
        path = os.environ.get("ORACLE_LIB", LIB_PATH)
        if path == LIB_PATH and not os.path.exists(LIB_PATH):
            from . import build as _b
            _b.build()
        L = C.CDLL(path)
        L.oracle_f32_to_f16.restype = C.c_uint16
        L.oracle_f32_to_f16.argtypes = [C.c_float]
        L.oracle_f32_to_bf16.restype = C.c_uint16
        L.oracle_f32_to_bf16.argtypes = [C.c_float]
        L.oracle_f16_to_f32.restype = C.c_float
        L.oracle_f16_to_f32.argtypes = [C.c_uint16]
        L.oracle_bf16_to_f32.restype = C.c_float
        L.oracle_bf16_to_f32.argtypes = [C.c_uint16]
        for name in ("oracle_f32_to_f16_n", "oracle_f32_to_bf16_n"):
            getattr(L, name).restype = None
            getattr(L, name).argtypes = [C.c_void_p, C.c_int64, C.c_void_p]
        for name in ("oracle_f16_to_f32_n", "oracle_bf16_to_f32_n"):
            getattr(L, name).restype = None
            getattr(L, name).argtypes = [C.c_void_p, C.c_int64, C.c_void_p]
        L.oracle_layout.restype = C.c_int64
        L.oracle_layout.argtypes = [C.c_void_p, C.c_int32, C.c_int32, C.c_int64, C.c_void_p,
                                    C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p,
                                    C.c_void_p, C.c_void_p, C.c_int64]
        L.oracle_accounting.restype = None
        L.oracle_accounting.argtypes = [C.c_int64, C.c_int64, C.c_int32, C.c_int32, C.c_int32,
                                        C.c_void_p]
        L.oracle_reduce.restype = None
        L.oracle_reduce.argtypes = [C.c_void_p, C.c_int32, C.c_int32, C.c_int64, C.c_int64,
                                    C.c_int32, C.c_void_p]
        L.oracle_unscale_stats.restype = None
        L.oracle_unscale_stats.argtypes = [C.c_void_p, C.c_int32, C.c_int64, C.c_float,
                                           C.POINTER(C.c_double), C.POINTER(C.c_int32)]
        L.oracle_clip_coef.restype = C.c_float
        L.oracle_clip_coef.argtypes = [C.c_double, C.c_double]
        L.oracle_adamw.restype = None
        L.oracle_adamw.argtypes = [C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p,
                                   C.c_int64, C.c_float, C.c_float, C.c_int64,
                                   C.POINTER(Hparams), C.c_void_p, C.c_int32]
        L.oracle_quant_int8.restype = None
        L.oracle_quant_int8.argtypes = [C.c_void_p, C.c_int32, C.c_int64, C.c_int32,
                                        C.c_void_p, C.c_void_p]
        L.oracle_reduce_accumulate.restype = None
        L.oracle_reduce_accumulate.argtypes = [C.c_void_p, C.c_int32, C.c_int32, C.c_int64,
                                               C.c_int64, C.c_int32, C.c_void_p]
        L.oracle_dequant_int8.restype = None
        L.oracle_dequant_int8.argtypes = [C.c_void_p, C.c_void_p, C.c_int32, C.c_int64,
                                          C.c_int32, C.c_int32, C.c_void_p]
        L.oracle_reduce_q8.restype = None
        L.oracle_reduce_q8.argtypes = [C.c_void_p, C.c_void_p, C.c_int32, C.c_int64, C.c_int32,
                                       C.c_int32, C.c_void_p]
        L.oracle_scaler_update.restype = None
        L.oracle_scaler_update.argtypes = [C.POINTER(Scaler), C.c_int32]
        _lib = L
    return _lib


def _ptr(a):
    return a.ctypes.data_as(C.c_void_p)


def _check(a, dt):
    assert isinstance(a, np.ndarray) and a.dtype == dt and a.flags.c_contiguous, (a.dtype, dt)


def dtype_np(code):
    return np.float32 if code == F32 else np.uint16


# ---------------------------------------------------------------- formats
def f32_to_f16(x):
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().oracle_f32_to_f16_n(_ptr(x), x.size, _ptr(out))
    return out


def f32_to_bf16(x):
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().oracle_f32_to_bf16_n(_ptr(x), x.size, _ptr(out))
    return out


def f16_to_f32(h):
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, np.float32)
    lib().oracle_f16_to_f32_n(_ptr(h), h.size, _ptr(out))
    return out


def bf16_to_f32(h):
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, np.float32)
    lib().oracle_bf16_to_f32_n(_ptr(h), h.size, _ptr(out))
    return out


def to_f32(a, code):
    if code == F32:
        return np.asarray(a, np.float32)
    return f16_to_f32(a) if code == F16 else bf16_to_f32(a)


def from_f32(x, code):
    if code == F32:
        return np.asarray(x, np.float32).copy()
    return f32_to_f16(x) if code == F16 else f32_to_bf16(x)


# ---------------------------------------------------------------- layout
def layout(numels, n_ranks, align=1, rank=0):
    numels = np.ascontiguousarray(numels, dtype=np.int64)
    n = len(numels)
    out = np.zeros(4, np.int64)
    starts = np.zeros(max(n, 1), np.int64)
    ends = np.zeros(max(n, 1), np.int64)
    cap = n + 1
    sp, so, ss, sl = (np.zeros(cap, np.int64) for _ in range(4))
    r = lib().oracle_layout(_ptr(numels), n, n_ranks, align, _ptr(out), _ptr(starts),
                            _ptr(ends), rank, _ptr(sp), _ptr(so), _ptr(ss), _ptr(sl), cap)
    if r < 0:
        raise ValueError("oracle_layout rejected the input (%d)" % r)
    segs = [(int(sp[i]), int(so[i]), int(ss[i]), int(sl[i])) for i in range(r)]
    return dict(total=int(out[0]), shard=int(out[1]), padded=int(out[2]), pad=int(out[3]),
                starts=[int(x) for x in starts[:n]], ends=[int(x) for x in ends[:n]],
                segments=segs)


def accounting(total, shard, param_bytes, grad_bytes, optim_bytes):
    out = np.zeros(4, np.int64)
    lib().oracle_accounting(total, shard, param_bytes, grad_bytes, optim_bytes, _ptr(out))
    return dict(dp=int(out[0]), z1=int(out[1]), z2=int(out[2]), z3=int(out[3]))


# ---------------------------------------------------------------- step parts
def reduce(bufs, dtype, offset, n, op):
    """red[i] = sum_k f32(bufs[k][offset+i]) (rank order); AVG divides by N."""
    for b in bufs:
        _check(b, dtype_np(dtype))
        assert offset + n <= b.size
    arr = (C.c_void_p * len(bufs))(*[b.ctypes.data for b in bufs])
    red = np.empty(n, np.float32)
    lib().oracle_reduce(arr, len(bufs), dtype, offset, n, op, _ptr(red))
    return red


def reduce_accumulate(bufs, dtype, offset, n, op, acc):
    """acc[i] += red_i (one micro-step of sharded gradient accumulation), in place."""
    for b in bufs:
        _check(b, dtype_np(dtype))
        assert offset + n <= b.size
    _check(acc, np.float32)
    assert acc.size >= n
    arr = (C.c_void_p * len(bufs))(*[b.ctypes.data for b in bufs])
    lib().oracle_reduce_accumulate(arr, len(bufs), dtype, offset, n, op, _ptr(acc))
    return acc


def reduce_q8(qs, scales, n, block, op):
    """red[i] = sum_k f32(qs[k][i]) * scales[k][i // block] (rank order); AVG / N."""
    assert len(qs) == len(scales)
    for q, sc in zip(qs, scales):
        _check(q, np.int8)
        _check(sc, np.float32)
        assert q.size >= n and sc.size >= (n + block - 1) // block
    qa = (C.c_void_p * len(qs))(*[q.ctypes.data for q in qs])
    sa = (C.c_void_p * len(qs))(*[sc.ctypes.data for sc in scales])
    red = np.empty(n, np.float32)
    lib().oracle_reduce_q8(qa, sa, len(qs), n, block, op, _ptr(red))
    return red


def unscale_stats(g, dtype, loss_scale, sumsq=0.0, overflow=0):
    _check(g, dtype_np(dtype))
    s = C.c_double(sumsq)
    o = C.c_int32(overflow)
    lib().oracle_unscale_stats(_ptr(g), dtype, g.size, loss_scale, C.byref(s), C.byref(o))
    return s.value, o.value


def clip_coef(sumsq_total, max_norm):
    return lib().oracle_clip_coef(sumsq_total, max_norm)


def adamw(g, gdtype, p, m, v, loss_scale, coef, t, hp, lp_dtype=None):
    """Updates p, m, v (float32 arrays) in place; returns the fp16/bf16 copy."""
    _check(g, dtype_np(gdtype))
    for a in (p, m, v):
        _check(a, np.float32)
        assert a.size == g.size
    lp = None
    if lp_dtype is not None:
        lp = np.empty(g.size, np.uint16)
    h = hp if isinstance(hp, Hparams) else Hparams(**hp)
    lib().oracle_adamw(_ptr(g), gdtype, _ptr(p), _ptr(m), _ptr(v), g.size, loss_scale, coef, t,
                       C.byref(h), _ptr(lp) if lp is not None else None,
                       lp_dtype if lp_dtype is not None else F16)
    return lp


def quant_int8(x, dtype, block=256):
    _check(x, np.uint16)
    nb = (x.size + block - 1) // block
    q = np.empty(x.size, np.int8)
    s = np.empty(nb, np.float32)
    lib().oracle_quant_int8(_ptr(x), dtype, x.size, block, _ptr(q), _ptr(s))
    return q, s


def dequant_int8(q, scales, n_slots, slot_numel, block, dtype):
    """Full flat buffer out[s*S+i] = round_dtype(f32(q) * scale) over n_slots slots;
    uint16 bit patterns for fp16/bf16, float32 for F32."""
    _check(q, np.int8)
    _check(scales, np.float32)
    nb = (slot_numel + block - 1) // block
    assert q.size >= n_slots * slot_numel and scales.size >= n_slots * nb
    out = np.empty(n_slots * slot_numel, np.float32 if dtype == F32 else np.uint16)
    lib().oracle_dequant_int8(_ptr(q), _ptr(scales), n_slots, slot_numel, block, dtype, _ptr(out))
    return out


def scaler_update(sc, overflow):
    lib().oracle_scaler_update(C.byref(sc), int(overflow))


def make_scaler(loss_scale, dynamic, window=1000, min_scale=1.0):
    return Scaler(loss_scale=loss_scale, min_scale=min_scale, dynamic=int(dynamic),
                  window=window, good_steps=0, step=0)


# ---------------------------------------------------------------- one step
def shard_step(*, grad, grad_dtype, master, exp_avg, exp_avg_sq, scaler, hp,
               param_dtype, remote_sumsq=0.0, remote_overflow=0, quant_block=None,
               sumsq_local=None, overflow_local=None):
    """One rank's optimizer step over its shard, in the pages' order.

    `grad` is the reduced gradient shard (fp32 from `reduce`, or an fp16/bf16
    pre-reduced shard).  `sumsq_local`/`overflow_local` may be supplied when
    `grad` is a subset of the shard (sampled checks of a large shard); they
    must then be the oracle's own statistics over the whole shard.
    Returns a dict with the written slot (lp), INT8 payload, norm, coef and
    whether the step was skipped.  master/exp_avg/exp_avg_sq change in place.
    """
    if sumsq_local is None:
        sumsq_local, overflow_local = unscale_stats(grad, grad_dtype, scaler.loss_scale)
    total = sumsq_local + remote_sumsq
    ovf = int(bool(overflow_local) or bool(remote_overflow))
    res = dict(sumsq=total, norm=float(np.sqrt(total)), overflow=ovf, skipped=ovf,
               lp=None, q=None, scales=None, coef=None)
    if ovf:
        scaler_update(scaler, 1)
        return res
    coef = clip_coef(total, hp.max_grad_norm if isinstance(hp, Hparams) else hp["max_grad_norm"])
    t = scaler.step + 1
    lp = adamw(grad, grad_dtype, master, exp_avg, exp_avg_sq, scaler.loss_scale, coef, t, hp,
               param_dtype)
    res["coef"] = coef
    res["lp"] = lp
    if quant_block:
        res["q"], res["scales"] = quant_int8(lp, param_dtype, quant_block)
    scaler_update(scaler, 0)
    return res
