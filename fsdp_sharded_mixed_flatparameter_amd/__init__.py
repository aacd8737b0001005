"""Python binding of libzeroflat: one rank's sharded mixed-precision AdamW step
over a FlatParameter on MI355X (gfx950).

The functions mirror the C ABI in include/zeroflat.h one to one and only
marshal arguments: torch tensors supply device pointers, the stream is torch's
current HIP stream unless given, and every step runs in the library's
kernels.  There is no fallback: importing this package fails if the library
has not been built (``__graft_entry__.build()`` or ``python -m
fsdp_sharded_mixed_flatparameter_amd._build``).
"""
import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libzeroflat.so")

ZERO_F32, ZERO_F16, ZERO_BF16 = 0, 1, 2
ZERO_SUM, ZERO_AVG = 0, 1
ZERO_STEP_FINALIZE = 1
ZERO_MAX_RANKS = 256
ZERO_MAX_PARTIALS = 65536

EXPORTS = ("zero_last_error", "zero_flat_layout", "zero_step_state_init",
           "zero_grad_reduce_shard", "zero_unscale_norm", "zero_adamw_shard_step",
           "zero_quant_allgather_slot", "zero_dequant_allgather", "zero_grad_accumulate_shard",
           "zero_grad_reduce_shard_int8", "zero_offload_adamw_host", "zero_offload_step",
           "zero_grad_reduce_shard_noalloc")


class zero_span_t(C.Structure):
    _fields_ = [("start", C.c_int64), ("end", C.c_int64)]


class zero_segment_t(C.Structure):
    _fields_ = [("param", C.c_int32), ("reserved", C.c_int32), ("off_in_param", C.c_int64),
                ("off_in_shard", C.c_int64), ("len", C.c_int64)]


class zero_layout_t(C.Structure):
    _fields_ = [("total", C.c_int64), ("shard", C.c_int64), ("padded", C.c_int64),
                ("pad", C.c_int64), ("n_ranks", C.c_int32), ("reserved", C.c_int32),
                ("align", C.c_int64), ("bytes_dp", C.c_int64), ("bytes_z1", C.c_int64),
                ("bytes_z2", C.c_int64), ("bytes_z3", C.c_int64)]


class zero_step_state_t(C.Structure):
    _fields_ = [("sumsq", C.c_double), ("overflow", C.c_int32),
                ("remote_overflow", C.c_int32), ("remote_sumsq", C.c_double),
                ("loss_scale", C.c_float), ("min_scale", C.c_float), ("dynamic", C.c_int32),
                ("window", C.c_int32), ("good_steps", C.c_int32), ("step", C.c_int32),
                ("beta1_pow", C.c_double), ("beta2_pow", C.c_double),
                ("last_norm", C.c_double), ("last_coef", C.c_float),
                ("last_skipped", C.c_int32), ("n_partials", C.c_int32),
                ("tile_counter", C.c_int32), ("partials", C.c_double * ZERO_MAX_PARTIALS)]


class zero_adamw_hparams_t(C.Structure):
    _fields_ = [("lr", C.c_double), ("beta1", C.c_double), ("beta2", C.c_double),
                ("eps", C.c_double), ("weight_decay", C.c_double),
                ("max_grad_norm", C.c_double)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError("libzeroflat.so is not built (%s); run __graft_entry__.build()" % LIB_PATH)
    L = C.CDLL(LIB_PATH)
    vp, i32, i64, u32 = C.c_void_p, C.c_int32, C.c_int64, C.c_uint32
    L.zero_last_error.restype = C.c_char_p
    L.zero_last_error.argtypes = []
    L.zero_flat_layout.restype = C.c_int
    L.zero_flat_layout.argtypes = [vp, i32, i32, i64, i32, i32, i32, i32, vp, vp, vp, i32, vp]
    L.zero_step_state_init.restype = C.c_int
    L.zero_step_state_init.argtypes = [vp, C.c_float, i32, i32, C.c_float]
    L.zero_grad_reduce_shard.restype = C.c_int
    L.zero_grad_reduce_shard.argtypes = [vp, i32, i32, i64, i64, i32, vp, vp, vp]
    L.zero_grad_reduce_shard_noalloc.restype = C.c_int
    L.zero_grad_reduce_shard_noalloc.argtypes = [vp, i32, i32, i64, i64, i32, vp, vp, vp]
    L.zero_unscale_norm.restype = C.c_int
    L.zero_unscale_norm.argtypes = [vp, i32, i64, vp, vp]
    L.zero_adamw_shard_step.restype = C.c_int
    L.zero_adamw_shard_step.argtypes = [vp, i32, vp, vp, vp, i64, vp, i32, i64, vp, vp, i64,
                                        i64, i32, vp, u32, vp, vp]
    L.zero_quant_allgather_slot.restype = C.c_int
    L.zero_quant_allgather_slot.argtypes = [vp, i32, i64, i32, vp, i64, vp, i64, vp]
    L.zero_dequant_allgather.restype = C.c_int
    L.zero_dequant_allgather.argtypes = [vp, vp, i32, i64, i32, vp, i32, vp]
    L.zero_grad_accumulate_shard.restype = C.c_int
    L.zero_grad_accumulate_shard.argtypes = [vp, i32, i32, i64, i64, i32, vp, vp, vp]
    L.zero_grad_reduce_shard_int8.restype = C.c_int
    L.zero_grad_reduce_shard_int8.argtypes = [vp, vp, i32, i64, i32, i32, vp, vp, vp]
    L.zero_offload_adamw_host.restype = C.c_int
    L.zero_offload_adamw_host.argtypes = [vp, i32, vp, vp, vp, i64, vp, i32, vp, vp, i32, vp]
    L.zero_offload_step.restype = C.c_int
    L.zero_offload_step.argtypes = [vp, i32, i64, vp, vp, vp, vp, vp, vp, i32, i64, vp, vp, i64,
                                    i32, vp]
    return L


_lib = _load()


class ZeroError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__("libzeroflat error %d: %s" % (code, msg))
        self.code = code


def _check(rc):
    if rc != 0:
        raise ZeroError(rc, _lib.zero_last_error().decode())


def lib():
    return _lib


_DTYPE_CODES = {"float32": ZERO_F32, "float16": ZERO_F16, "bfloat16": ZERO_BF16}


def _dtype_code(t):
    try:
        return _DTYPE_CODES[_dtype_name(t.dtype)]
    except KeyError:
        raise ValueError("unsupported dtype %s" % t.dtype) from None


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _current_raw_stream():
    """torch's current HIP stream on the current device, as an integer handle
    (the raw-stream query torch's own generated code uses; the public
    torch.cuda.current_stream() costs several microseconds per call)."""
    import torch
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is None:
        return torch.cuda.current_stream().cuda_stream
    return raw(torch._C._cuda_getDevice())


def _stream(stream):
    if stream is None:
        return C.c_void_p(_current_raw_stream())
    if hasattr(stream, "cuda_stream"):
        return C.c_void_p(stream.cuda_stream)
    return C.c_void_p(int(stream))


def _contig(t, name):
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


_F16_BF16 = ("float16", "bfloat16")
_FLOATS = ("float32", "float16", "bfloat16")


_DTYPE_NAMES = {}


def _dtype_name(dt):
    name = _DTYPE_NAMES.get(dt)
    if name is None:
        name = _DTYPE_NAMES[dt] = str(dt).replace("torch.", "")
    return name


def _dev(t, name, dtypes=None):
    """A device argument: a contiguous CUDA tensor of one of `dtypes` (names)."""
    _contig(t, name)
    if not t.is_cuda:
        raise ValueError("%s must be a device (CUDA) tensor" % name)
    if dtypes is not None and _dtype_name(t.dtype) not in dtypes:
        raise ValueError("%s must be %s, not %s" % (name, " or ".join(dtypes), t.dtype))
    return t


# ------------------------------------------------------------------ layout
def zero_flat_layout(numels, n_ranks, align=1, param_bytes=2, grad_bytes=2, optim_bytes=12,
                     rank=0):
    """FlatParameter layout and per-rank accounting (host only)."""
    n = len(numels)
    arr = (C.c_int64 * max(n, 1))(*[int(x) for x in numels])
    out = zero_layout_t()
    spans = (zero_span_t * max(n, 1))()
    cap = n + 1
    segs = (zero_segment_t * cap)()
    nseg = C.c_int32(0)
    _check(_lib.zero_flat_layout(arr, n, n_ranks, align, param_bytes, grad_bytes, optim_bytes,
                                 rank, C.byref(out), spans, segs, cap, C.byref(nseg)))
    return dict(total=out.total, shard=out.shard, padded=out.padded, pad=out.pad,
                n_ranks=out.n_ranks, align=out.align,
                bytes=dict(dp=out.bytes_dp, z1=out.bytes_z1, z2=out.bytes_z2, z3=out.bytes_z3),
                spans=[(spans[j].start, spans[j].end) for j in range(n)],
                segments=[(segs[i].param, segs[i].off_in_param, segs[i].off_in_shard, segs[i].len)
                          for i in range(nseg.value)])


# ------------------------------------------------------------------ state
STATE_BYTES = C.sizeof(zero_step_state_t)
STATE_HEADER_BYTES = zero_step_state_t.partials.offset   # all zero_grad_reduce_shard_noalloc uses


def zero_step_state_init(loss_scale, dynamic, window=1000, min_scale=1.0):
    """Host zero_step_state_t for step 0 (ctypes struct)."""
    st = zero_step_state_t()
    _check(_lib.zero_step_state_init(C.byref(st), loss_scale, int(bool(dynamic)), window,
                                     min_scale))
    return st


class StepState:
    """Device-resident zero_step_state_t (a torch uint8 buffer) plus host views."""

    def __init__(self, loss_scale, dynamic, window=1000, min_scale=1.0, device="cuda"):
        import torch
        self.buf = torch.empty(STATE_BYTES, dtype=torch.uint8, device=device)
        self.upload(zero_step_state_init(loss_scale, dynamic, window, min_scale))

    def upload(self, host_state):
        import torch
        raw = bytes(bytearray(host_state))
        self.buf.copy_(torch.frombuffer(bytearray(raw), dtype=torch.uint8))

    def read(self):
        """Host copy of the state (synchronizes with the current stream)."""
        raw = self.buf.cpu().numpy().tobytes()
        return zero_step_state_t.from_buffer_copy(raw)

    def set_remote(self, sumsq=0.0, overflow=0):
        st = self.read()
        st.remote_sumsq = float(sumsq)
        st.remote_overflow = int(overflow)
        self.upload(st)

    def ptr(self):
        return C.c_void_p(self.buf.data_ptr())


def _state_ptr(state, need=STATE_BYTES):
    if state is None:
        return None
    if isinstance(state, StepState):
        return state.ptr()
    _dev(state, "state", ("uint8",))
    if state.numel() < need:
        raise ValueError("state must hold %d bytes" % need)
    return C.c_void_p(state.data_ptr())


# ------------------------------------------------------------------ the step
def _rank_buffers(grad_bufs, elem_offset, shard_numel, out):
    if not grad_bufs:
        raise ValueError("grad_bufs is empty")
    dt = _dtype_code(grad_bufs[0])
    for k, b in enumerate(grad_bufs):
        _dev(b, "grad_bufs[%d]" % k, _FLOATS)
        if _dtype_code(b) != dt:
            raise ValueError("grad_bufs dtypes differ")
        if elem_offset + shard_numel > b.numel():
            raise ValueError("grad_bufs[%d] is shorter than elem_offset + shard_numel" % k)
    _dev(out, "output shard", ("float32",))
    if out.numel() < shard_numel:
        raise ValueError("the output shard must be float32 with >= shard_numel elements")
    return dt, (C.c_void_p * len(grad_bufs))(*[b.data_ptr() for b in grad_bufs])


def zero_grad_reduce_shard(grad_bufs, elem_offset, shard_numel, op, red_out, state=None,
                           stream=None):
    """red_out[i] = sum_k grad_bufs[k][elem_offset + i] (rank order), AVG -> / N;
    accumulates the step statistics into `state` when given."""
    dt, arr = _rank_buffers(grad_bufs, elem_offset, shard_numel, red_out)
    _check(_lib.zero_grad_reduce_shard(arr, len(grad_bufs), dt, elem_offset, shard_numel, op,
                                       _ptr(red_out), _state_ptr(state), _stream(stream)))


def zero_grad_reduce_shard_noalloc(grad_bufs, elem_offset, shard_numel, op, red_out, state=None,
                                   stream=None):
    """zero_grad_reduce_shard for callers that cannot allocate: the statistics'
    partial sums live in the library's per-device scratch, so `state` may be a
    uint8 device tensor of only STATE_HEADER_BYTES bytes.  Calls that overlap
    in time on one device race on that scratch."""
    dt, arr = _rank_buffers(grad_bufs, elem_offset, shard_numel, red_out)
    _check(_lib.zero_grad_reduce_shard_noalloc(arr, len(grad_bufs), dt, elem_offset, shard_numel,
                                               op, _ptr(red_out),
                                               _state_ptr(state, STATE_HEADER_BYTES),
                                               _stream(stream)))


def zero_grad_accumulate_shard(grad_bufs, elem_offset, shard_numel, op, acc, state=None,
                               stream=None):
    """One micro-step of sharded gradient accumulation: acc[i] += the reduce of
    grad_bufs over [elem_offset, +shard_numel); pass `state` on the last
    micro-step to take the step statistics over the accumulated shard."""
    dt, arr = _rank_buffers(grad_bufs, elem_offset, shard_numel, acc)
    _check(_lib.zero_grad_accumulate_shard(arr, len(grad_bufs), dt, elem_offset, shard_numel,
                                           op, _ptr(acc), _state_ptr(state), _stream(stream)))


def zero_unscale_norm(grad_shard, state, n=None, stream=None):
    _dev(grad_shard, "grad_shard", _FLOATS)
    n = grad_shard.numel() if n is None else n
    if not 0 <= n <= grad_shard.numel():
        raise ValueError("n exceeds grad_shard")
    _check(_lib.zero_unscale_norm(_ptr(grad_shard), _dtype_code(grad_shard), n,
                                  _state_ptr(state), _stream(stream)))


def zero_adamw_shard_step(grad_shard, master, exp_avg, exp_avg_sq, allgather_buf, slot_offset,
                          hp, state, q_buf=None, q_scales=None, q_slot_offset=0,
                          q_scale_offset=0, q_block=256, finalize=True, stream=None):
    """Skip-on-overflow, clip, AdamW on master/m/v, write-back into
    allgather_buf[slot_offset:], optional INT8 payload, scaler update."""
    n = master.numel()
    _dev(grad_shard, "grad_shard", _FLOATS)
    for name, t in (("master", master), ("exp_avg", exp_avg), ("exp_avg_sq", exp_avg_sq)):
        _dev(t, name, ("float32",))
    _dev(allgather_buf, "allgather_buf", _F16_BF16)
    if q_buf is not None:
        if q_scales is None:
            raise ValueError("q_buf needs q_scales")
        _dev(q_buf, "q_buf", ("int8",))
        _dev(q_scales, "q_scales", ("float32",))
    if grad_shard.numel() < n or exp_avg.numel() != n or exp_avg_sq.numel() != n:
        raise ValueError("shard tensors disagree in size")
    if slot_offset + n > allgather_buf.numel():
        raise ValueError("slot exceeds the all-gather buffer")
    if q_buf is not None:
        if q_slot_offset + n > q_buf.numel() or \
                q_scale_offset + (n + q_block - 1) // q_block > q_scales.numel():
            raise ValueError("INT8 slot exceeds its buffers")
    h = hp if isinstance(hp, zero_adamw_hparams_t) else zero_adamw_hparams_t(**hp)
    _check(_lib.zero_adamw_shard_step(
        _ptr(grad_shard), _dtype_code(grad_shard), _ptr(master), _ptr(exp_avg), _ptr(exp_avg_sq),
        n, _ptr(allgather_buf), _dtype_code(allgather_buf), slot_offset, _ptr(q_buf),
        _ptr(q_scales), q_slot_offset, q_scale_offset, q_block, C.byref(h),
        ZERO_STEP_FINALIZE if finalize else 0, _state_ptr(state), _stream(stream)))


def zero_quant_allgather_slot(slot, q_buf, q_scales, q_slot_offset=0, q_scale_offset=0,
                              block=256, n=None, stream=None):
    _dev(slot, "slot", _F16_BF16)
    _dev(q_buf, "q_buf", ("int8",))
    _dev(q_scales, "q_scales", ("float32",))
    n = slot.numel() if n is None else n
    if not 0 <= n <= slot.numel():
        raise ValueError("n exceeds the slot")
    if q_slot_offset + n > q_buf.numel() or q_scale_offset + (n + block - 1) // block > q_scales.numel():
        raise ValueError("INT8 slot exceeds its buffers")
    _check(_lib.zero_quant_allgather_slot(_ptr(slot), _dtype_code(slot), n, block, _ptr(q_buf),
                                          q_slot_offset, _ptr(q_scales), q_scale_offset,
                                          _stream(stream)))


def zero_grad_reduce_shard_int8(q_slices, scale_slices, shard_numel, op, red_out, state=None,
                                block=256, stream=None):
    """red_out[i] = sum_k f32(q_slices[k][i]) * scale_slices[k][i // block] (rank
    order), AVG -> / N: the reduce over the N ranks' INT8-quantised gradient
    slices for this rank; statistics into `state` when given."""
    import torch
    if not q_slices or len(q_slices) != len(scale_slices):
        raise ValueError("need one codes and one scales tensor per rank")
    nb = (shard_numel + block - 1) // block
    for k, (q, sc) in enumerate(zip(q_slices, scale_slices)):
        _dev(q, "q_slices[%d]" % k, ("int8",))
        _dev(sc, "scale_slices[%d]" % k, ("float32",))
        if q.numel() < shard_numel or sc.numel() < nb:
            raise ValueError("rank %d's payload is shorter than the shard" % k)
    _dev(red_out, "red_out", ("float32",))
    if red_out.numel() < shard_numel:
        raise ValueError("red_out must hold >= shard_numel elements")
    n = len(q_slices)
    qa = (C.c_void_p * n)(*[q.data_ptr() for q in q_slices])
    sa = (C.c_void_p * n)(*[sc.data_ptr() for sc in scale_slices])
    _check(_lib.zero_grad_reduce_shard_int8(qa, sa, n, shard_numel, block, op, _ptr(red_out),
                                            _state_ptr(state), _stream(stream)))


# ------------------------------------------------------------------ ZeRO-Offload
def _host(t, name):
    _contig(t, name)
    if t.is_cuda:
        raise ValueError("%s must be a host tensor" % name)
    return t


def zero_offload_adamw_host(grad, master, exp_avg, exp_avg_sq, lp_out, hp, host_state,
                            n_threads=0):
    """The AdamW step of one shard on host cores, over host tensors, with the
    step scalars of `host_state` (a zero_step_state_t); returns 1 if the state
    records an overflow (then nothing is written)."""
    n = master.numel()
    for name, t in (("grad", grad), ("master", master), ("exp_avg", exp_avg),
                    ("exp_avg_sq", exp_avg_sq), ("lp_out", lp_out)):
        _host(t, name)
    for name, t in (("master", master), ("exp_avg", exp_avg), ("exp_avg_sq", exp_avg_sq)):
        if t.dtype.itemsize != 4 or not t.is_floating_point():
            raise ValueError("%s must be float32" % name)
    if grad.numel() < n or exp_avg.numel() != n or exp_avg_sq.numel() != n or lp_out.numel() < n:
        raise ValueError("host tensors disagree in size")
    h = hp if isinstance(hp, zero_adamw_hparams_t) else zero_adamw_hparams_t(**hp)
    sk = C.c_int32(0)
    _check(_lib.zero_offload_adamw_host(_ptr(grad), _dtype_code(grad), _ptr(master), _ptr(exp_avg),
                                        _ptr(exp_avg_sq), n, _ptr(lp_out), _dtype_code(lp_out),
                                        C.byref(h), C.byref(host_state), n_threads, C.byref(sk)))
    return sk.value


def zero_offload_step(grad_shard, master, exp_avg, exp_avg_sq, grad_stage, lp_stage,
                      allgather_buf, slot_offset, hp, state, chunk=0, n_threads=0, stream=None):
    """ZeRO-Offload step: the device gradient shard to pinned host staging in
    chunks, the update on host cores over host master/m/v, the 16-bit
    parameters back into allgather_buf[slot_offset:], then the device
    loss-scaler update.  Blocks until done."""
    n = master.numel()
    _dev(grad_shard, "grad_shard", _FLOATS)
    _dev(allgather_buf, "allgather_buf", _F16_BF16)
    for name, t in (("master", master), ("exp_avg", exp_avg), ("exp_avg_sq", exp_avg_sq),
                    ("grad_stage", grad_stage), ("lp_stage", lp_stage)):
        _host(t, name)
    if not grad_stage.is_pinned() or not lp_stage.is_pinned():
        raise ValueError("the staging buffers must be pinned host memory")
    if grad_shard.numel() < n or grad_stage.numel() < n or lp_stage.numel() < n or \
            exp_avg.numel() != n or exp_avg_sq.numel() != n:
        raise ValueError("tensors disagree in size")
    if grad_stage.dtype != grad_shard.dtype or lp_stage.dtype != allgather_buf.dtype:
        raise ValueError("staging dtypes must match the device tensors")
    if slot_offset + n > allgather_buf.numel():
        raise ValueError("slot exceeds the all-gather buffer")
    h = hp if isinstance(hp, zero_adamw_hparams_t) else zero_adamw_hparams_t(**hp)
    _check(_lib.zero_offload_step(_ptr(grad_shard), _dtype_code(grad_shard), n, _ptr(master),
                                  _ptr(exp_avg), _ptr(exp_avg_sq), _ptr(grad_stage),
                                  _ptr(lp_stage), _ptr(allgather_buf), _dtype_code(allgather_buf),
                                  slot_offset, C.byref(h), _state_ptr(state), chunk, n_threads,
                                  _stream(stream)))


# ------------------------------------------------------------------ All-Gather consumer
def zero_dequant_allgather(q_buf, q_scales, n_slots, slot_numel, out, block=256, stream=None):
    """out[s*S + i] = round(f32(q) * scale) over the n_slots gathered INT8 slots
    (the full flat parameter, fp16/bf16 or fp32)."""
    _dev(q_buf, "q_buf", ("int8",))
    _dev(q_scales, "q_scales", ("float32",))
    _dev(out, "out", _FLOATS)
    nb = (slot_numel + block - 1) // block
    if q_buf.numel() < n_slots * slot_numel or q_scales.numel() < n_slots * nb or \
            out.numel() < n_slots * slot_numel:
        raise ValueError("buffers are shorter than n_slots slots")
    _check(_lib.zero_dequant_allgather(_ptr(q_buf), _ptr(q_scales), n_slots, slot_numel, block,
                                       _ptr(out), _dtype_code(out), _stream(stream)))


def unflatten(flat, shapes, n_ranks=1, align=1):
    """Views of the parameters inside a gathered flat buffer, at the [start, end)
    ranges zero_flat_layout gives for these shapes (no copy)."""
    import math
    numels = [int(math.prod(sh)) for sh in shapes]
    lay = zero_flat_layout(numels, n_ranks, align)
    if flat.numel() < lay["total"]:
        raise ValueError("flat buffer is shorter than the parameters")
    return [flat[a:b].view(tuple(sh)) for (a, b), sh in zip(lay["spans"], shapes)]


from . import shard  # noqa: E402
from .shard import MultiShardOptimizer, OffloadShardOptimizer, ShardOptimizer  # noqa: E402,F401
