"""Seeded synthetic inputs for tests and the benchmark.

One generator definition (SplitMix64 outputs -> Irwin-Hall(12) variate, see
synth_cpu.c), implemented twice: in C for the host (the oracle's inputs) and in
HIP for the device (bulk fills of multi-GB shards).  The stream key is derived
here once, on the host, and handed to either side; values depend only on
(key, global element index), so any slice or sample of a tensor can be
regenerated on its own.  Nothing here computes any part of the optimizer step.
"""
import ctypes as C
import os
import zlib
from concurrent.futures import ThreadPoolExecutor

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
CPU_LIB = os.path.join(HERE, "libsynth_cpu.so")
GPU_LIB = os.path.join(HERE, "libsynth_gpu.so")

BASE_SEED = 42
_M64 = (1 << 64) - 1
_GAMMA = 0x9E3779B97F4A7C15


def _mix64(z):
    z &= _M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
    return z ^ (z >> 31)


def stream_key(*parts):
    """64-bit stream key from a path of labels/ints, e.g. ("grad", cfg, step, rank)."""
    k = BASE_SEED
    for p in parts:
        v = zlib.crc32(p.encode()) if isinstance(p, str) else int(p)
        k = _mix64(k ^ _mix64((v + 1) * _GAMMA))
    return k


_cpu = None
_gpu = None


def _cpu_lib():
    global _cpu
    if _cpu is None:
        if not os.path.exists(CPU_LIB):
            from . import build as _b
            _b.build()
        L = C.CDLL(CPU_LIB)
        L.synth_normal_f32.restype = None
        L.synth_normal_f32.argtypes = [C.c_uint64, C.c_int64, C.c_int64, C.c_float, C.c_void_p]
        L.synth_normal_f32_at.restype = None
        L.synth_normal_f32_at.argtypes = [C.c_uint64, C.c_void_p, C.c_int64, C.c_float,
                                          C.c_void_p]
        L.synth_codes_i8.restype = None
        L.synth_codes_i8.argtypes = [C.c_uint64, C.c_int64, C.c_int64, C.c_void_p]
        L.synth_codes_i8_at.restype = None
        L.synth_codes_i8_at.argtypes = [C.c_uint64, C.c_void_p, C.c_int64, C.c_void_p]
        L.synth_mix64.restype = C.c_uint64
        L.synth_mix64.argtypes = [C.c_uint64]
        _cpu = L
    return _cpu


def _gpu_lib():
    global _gpu
    if _gpu is None:
        if not os.path.exists(GPU_LIB):
            raise RuntimeError("synth GPU library not built: run __graft_entry__.build()")
        L = C.CDLL(GPU_LIB)
        L.synth_fill_normal.restype = C.c_int
        L.synth_fill_normal.argtypes = [C.c_uint64, C.c_int64, C.c_int64, C.c_float,
                                        C.c_void_p, C.c_int32, C.c_void_p]
        L.synth_fill_codes.restype = C.c_int
        L.synth_fill_codes.argtypes = [C.c_uint64, C.c_int64, C.c_int64, C.c_void_p, C.c_void_p]
        L.synth_copy.restype = C.c_int
        L.synth_copy.argtypes = [C.c_void_p, C.c_void_p, C.c_int64, C.c_int32, C.c_void_p]
        L.synth_read.restype = C.c_int
        L.synth_read.argtypes = [C.c_void_p, C.c_int64, C.c_void_p, C.c_void_p]
        L.synth_read_streams.restype = C.c_int
        L.synth_read_streams.argtypes = [C.c_void_p, C.c_int32, C.c_int64, C.c_void_p,
                                         C.c_void_p]
        L.synth_write.restype = C.c_int
        L.synth_write.argtypes = [C.c_void_p, C.c_int64, C.c_uint32, C.c_void_p]
        L.synth_mix28.restype = C.c_int
        L.synth_mix28.argtypes = [C.c_void_p] * 5 + [C.c_int64, C.c_void_p]
        L.synth_set_launch_form.restype = C.c_int
        L.synth_set_launch_form.argtypes = [C.c_int64, C.c_uint32]
        _gpu = L
    return _gpu


# ------------------------------------------------------------------ host side
F32, F16, BF16 = 0, 1, 2
_CHUNK = 1 << 22


def normal_f32(key, start, n, sigma, threads=1):
    """sigma * z(key, j) for j in [start, start+n) as float32."""
    out = np.empty(n, np.float32)
    L = _cpu_lib()
    if threads <= 1 or n <= _CHUNK:
        L.synth_normal_f32(key, start, n, sigma, out.ctypes.data_as(C.c_void_p))
        return out

    def job(lo):
        hi = min(lo + _CHUNK, n)
        L.synth_normal_f32(key, start + lo, hi - lo, sigma,
                           C.c_void_p(out.ctypes.data + 4 * lo))

    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(job, range(0, n, _CHUNK)))
    return out


def normal_f32_at(key, idx, sigma):
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    out = np.empty(idx.size, np.float32)
    _cpu_lib().synth_normal_f32_at(key, idx.ctypes.data_as(C.c_void_p), idx.size, sigma,
                                   out.ctypes.data_as(C.c_void_p))
    return out


def codes(key, start, n):
    """Integer codes in [-127, 127] for elements [start, start+n) (int8)."""
    out = np.empty(n, np.int8)
    _cpu_lib().synth_codes_i8(key, start, n, out.ctypes.data_as(C.c_void_p))
    return out


def codes_at(key, idx):
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    out = np.empty(idx.size, np.int8)
    _cpu_lib().synth_codes_i8_at(key, idx.ctypes.data_as(C.c_void_p), idx.size,
                                 out.ctypes.data_as(C.c_void_p))
    return out


def to_storage(x, dtype):
    """Round float32 values to the storage format (nearest-even): float32
    array, or uint16 bit patterns for fp16 (numpy) / bf16 (torch CPU)."""
    if dtype == F32:
        return np.asarray(x, np.float32)
    if dtype == F16:
        return np.asarray(x, np.float32).astype(np.float16).view(np.uint16)
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def normal(key, start, n, sigma, dtype, threads=1):
    return to_storage(normal_f32(key, start, n, sigma, threads), dtype)


def normal_at(key, idx, sigma, dtype):
    return to_storage(normal_f32_at(key, idx, sigma), dtype)


# ------------------------------------------------------------------ device side
def _torch_code(t):
    import torch
    return {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}[t.dtype]


def fill_normal(t, key, start, sigma, stream=None):
    """Fill contiguous CUDA tensor `t` with sigma*z(key, start+i) in t's dtype."""
    import torch
    assert t.is_cuda and t.is_contiguous()
    s = stream if stream is not None else torch.cuda.current_stream().cuda_stream
    rc = _gpu_lib().synth_fill_normal(key, start, t.numel(), sigma, C.c_void_p(t.data_ptr()),
                                      _torch_code(t), C.c_void_p(s))
    if rc != 0:
        raise RuntimeError("synth_fill_normal failed: hip error %d" % rc)
    return t


def fill_codes(t, key, start=0, stream=None):
    """Fill a contiguous int8 CUDA tensor with the codes of (key, start+i)."""
    import torch
    assert t.is_cuda and t.is_contiguous() and t.dtype == torch.int8
    s = stream if stream is not None else torch.cuda.current_stream().cuda_stream
    rc = _gpu_lib().synth_fill_codes(key, start, t.numel(), C.c_void_p(t.data_ptr()),
                                     C.c_void_p(s))
    if rc != 0:
        raise RuntimeError("synth_fill_codes failed: hip error %d" % rc)
    return t


def copy(src, dst, grid=0, stream=None):
    import torch
    nbytes = src.numel() * src.element_size()
    assert dst.numel() * dst.element_size() == nbytes
    s = stream if stream is not None else torch.cuda.current_stream().cuda_stream
    rc = _gpu_lib().synth_copy(C.c_void_p(src.data_ptr()), C.c_void_p(dst.data_ptr()), nbytes,
                               grid, C.c_void_p(s))
    if rc != 0:
        raise RuntimeError("synth_copy failed: hip error %d" % rc)


def _stream(stream):
    import torch
    return C.c_void_p(stream if stream is not None else torch.cuda.current_stream().cuda_stream)


def read_stream(src, sink, stream=None):
    """Read every byte of `src` once (calibration); `sink` is a 1-element int32 tensor."""
    rc = _gpu_lib().synth_read(C.c_void_p(src.data_ptr()), src.numel() * src.element_size(),
                               C.c_void_p(sink.data_ptr()), _stream(stream))
    if rc != 0:
        raise RuntimeError("synth_read failed: hip error %d" % rc)


def read_streams(bufs, nbytes, sink, stream=None):
    """Read the first `nbytes` of every tensor in `bufs` (at most 128, 8-byte
    aligned) at once, as many concurrent streams (calibration); `sink` is a
    1-element int32 tensor."""
    ptrs = (C.c_void_p * len(bufs))(*[b.data_ptr() for b in bufs])
    for b in bufs:
        assert b.is_cuda and b.numel() * b.element_size() >= nbytes
    rc = _gpu_lib().synth_read_streams(ptrs, len(bufs), nbytes, C.c_void_p(sink.data_ptr()),
                                       _stream(stream))
    if rc != 0:
        raise RuntimeError("synth_read_streams failed: hip error %d" % rc)


def write_stream(dst, val=0x3f800000, stream=None):
    """Write every byte of `dst` once (calibration)."""
    rc = _gpu_lib().synth_write(C.c_void_p(dst.data_ptr()), dst.numel() * dst.element_size(), val,
                                _stream(stream))
    if rc != 0:
        raise RuntimeError("synth_write failed: hip error %d" % rc)


def mix28(g, p, m, v, lp, stream=None):
    """The fused update's byte mix with trivial arithmetic (calibration): g and
    lp 16-bit, p, m, v fp32, all of n elements, n a multiple of 1024."""
    n = p.numel()
    assert g.numel() == m.numel() == v.numel() == lp.numel() == n
    rc = _gpu_lib().synth_mix28(*[C.c_void_p(t.data_ptr()) for t in (g, p, m, v, lp)], n,
                                _stream(stream))
    if rc != 0:
        raise RuntimeError("synth_mix28 failed: hip error %d" % rc)

class launch_form:
    """Context manager: issue the calibration streams (read, write, copy without
    a grid, mix28) as consecutive launches of at most `slice_blocks` blocks, each
    with `lds_bytes` of dynamic LDS reserved (caps the resident blocks per
    compute unit); the library's streaming kernels use such launch forms."""

    def __init__(self, slice_blocks=0, lds_bytes=0):
        self.form = (slice_blocks, lds_bytes)

    def __enter__(self):
        rc = _gpu_lib().synth_set_launch_form(*self.form)
        if rc != 0:
            raise RuntimeError("synth_set_launch_form failed: hip error %d" % rc)
        return self

    def __exit__(self, *exc):
        _gpu_lib().synth_set_launch_form(0, 0)
        return False
