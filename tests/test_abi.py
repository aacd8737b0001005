"""Host-side tests of libzeroflat (no GPU needed): the library loads and
exports every entry point declared in include/zeroflat.h, the FlatParameter
layout and accounting agree with the oracle and the pages' figures, the step
state has the layout the binding assumes, and bad arguments are rejected
before anything is launched."""
import ctypes as C
import json
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "zeroflat.h")
GOLDEN = os.path.join(ROOT, "tests", "golden", "memory_accounting.json")


@pytest.fixture(scope="module")
def zf():
    import fsdp_sharded_mixed_flatparameter_amd as m
    return m


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(zero_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_function(zf):
    decl = declared_functions()
    assert set(decl) == set(zf.EXPORTS), decl
    for name in decl:
        assert hasattr(zf.lib(), name), name


def test_layout_matches_oracle(zf, orc):
    rng = np.random.default_rng(21)
    cases = [([512 * 1024, 1024, 1024 * 512, 512], 4, 1), ([10], 4, 1), ([7], 8, 1),
             ([3, 5], 3, 1), ([0, 0], 2, 1), ([], 3, 1), ([10 ** 10], 8, 1),
             ([7 * 10 ** 10], 64, 1), ([1000, 3], 6, 64)]
    for _ in range(100):
        cases.append(([int(x) for x in rng.integers(0, 50, size=int(rng.integers(1, 6)))],
                      int(rng.integers(1, 9)), int(rng.choice([1, 2, 8]))))
    for numels, n_ranks, align in cases:
        for rank in range(n_ranks):
            a = zf.zero_flat_layout(numels, n_ranks, align=align, rank=rank)
            b = orc.layout(numels, n_ranks, align, rank)
            assert (a["total"], a["shard"], a["padded"], a["pad"]) == \
                (b["total"], b["shard"], b["padded"], b["pad"])
            assert a["segments"] == b["segments"], (numels, n_ranks, align, rank)
            assert [s for s, _ in a["spans"]] == b["starts"]
            assert [e for _, e in a["spans"]] == b["ends"]


def test_accounting_printed_values(zf):
    g = json.load(open(GOLDEN))
    for case in g["cases"]:
        lay = zf.zero_flat_layout([case["total"]], case["n_ranks"], param_bytes=case["P"],
                                  grad_bytes=case["G"], optim_bytes=case["K"])
        assert lay["bytes"][case["field"]] == case["bytes"], case["cite"]


def test_layout_errors(zf):
    with pytest.raises(zf.ZeroError):
        zf.zero_flat_layout([4], 0)
    with pytest.raises(zf.ZeroError):
        zf.zero_flat_layout([4], 2, rank=2)
    with pytest.raises(zf.ZeroError):
        zf.zero_flat_layout([-1], 2)
    with pytest.raises(zf.ZeroError):
        zf.zero_flat_layout([4], 2, align=0)
    with pytest.raises(zf.ZeroError):
        zf.zero_flat_layout([2 ** 62, 2 ** 62], 1)          # total overflows int64
    # too small a segment buffer: ZERO_ERANGE with the count needed
    arr = (C.c_int64 * 3)(5, 5, 5)
    out = zf.zero_layout_t()
    segs = (zf.zero_segment_t * 1)()
    n = C.c_int32(0)
    rc = zf.lib().zero_flat_layout(arr, 3, 1, 1, 2, 2, 12, 0, C.byref(out), None, segs, 1,
                                   C.byref(n))
    assert rc == -3 and n.value == 3


def test_state_struct_size_and_init(zf):
    size = zf.STATE_BYTES
    buf = (C.c_uint8 * (size + 64))()
    C.memset(buf, 0xAB, size + 64)
    rc = zf.lib().zero_step_state_init(buf, 1024.0, 1, 7, 2.0)
    assert rc == 0
    raw = bytes(buf)
    assert raw[size - 1] == 0                  # the C struct reaches the last byte
    assert raw[size:] == b"\xab" * 64          # ... and not one byte further
    st = zf.zero_step_state_t.from_buffer_copy(raw[:size])
    assert (st.loss_scale, st.min_scale, st.dynamic, st.window) == (1024.0, 2.0, 1, 7)
    assert (st.step, st.good_steps, st.sumsq, st.overflow) == (0, 0, 0.0, 0)
    assert st.beta1_pow == 1.0 and st.beta2_pow == 1.0
    assert st.n_partials == 0 and st.tile_counter == 0   # the launch counter starts at zero


@pytest.mark.parametrize("scale,dyn,window,floor", [
    (1000.0, 0, 1, 1.0), (0.5, 0, 1, 1.0), (65536.0, 1, 0, 1.0), (4.0, 0, 1, 8.0),
    (float("inf"), 0, 1, 1.0), (float("nan"), 0, 1, 1.0), (4.0, 0, 1, 0.5)])
def test_state_init_rejects(zf, scale, dyn, window, floor):
    with pytest.raises(zf.ZeroError):
        zf.zero_step_state_init(scale, dyn, window, floor)


def test_step_calls_validate_before_launch(zf):
    """Invalid arguments return an error without touching a device."""
    L = zf.lib()
    st = C.c_void_p(0x1000)                     # never dereferenced: validation fails first
    hp = zf.zero_adamw_hparams_t(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0,
                                 max_grad_norm=1.0)
    bufs = (C.c_void_p * 1)(0x1000)
    assert L.zero_grad_reduce_shard(bufs, 0, 1, 0, 8, 0, C.c_void_p(0x1000), None, None) == -3
    assert L.zero_grad_reduce_shard(bufs, 1, 7, 0, 8, 0, C.c_void_p(0x1000), None, None) == -1
    assert L.zero_grad_reduce_shard(bufs, 1, 1, 0, 8, 5, C.c_void_p(0x1000), None, None) == -1
    assert L.zero_grad_reduce_shard(bufs, 1, 1, 0, 8, 0, None, None, None) == -1
    assert L.zero_grad_reduce_shard(bufs, 1, 1, 0, 8, 0, C.c_void_p(0x1002), None, None) == -2
    assert L.zero_grad_reduce_shard(bufs, 257, 1, 0, 8, 0, C.c_void_p(0x1000), None, None) == -3
    odd = (C.c_void_p * 1)(0x1001)
    assert L.zero_grad_reduce_shard(odd, 1, 1, 0, 8, 0, C.c_void_p(0x1000), None, None) == -2
    assert L.zero_unscale_norm(None, 1, 8, st, None) == -1
    assert L.zero_unscale_norm(C.c_void_p(0x1000), 1, -1, st, None) == -1
    p = C.c_void_p(0x1000)
    args = [p, 1, p, p, p, 16, p, 1, 0, None, None, 0, 0, 256]
    assert L.zero_adamw_shard_step(*args, C.byref(hp), 1, None, None) == -1      # no state
    assert L.zero_adamw_shard_step(*args[:7], 0, *args[8:], C.byref(hp), 1, st, None) == -1
    assert L.zero_adamw_shard_step(*args, C.byref(hp), 4, st, None) == -1         # bad flag
    bad = zf.zero_adamw_hparams_t(lr=1e-3, beta1=1.0, beta2=0.999, eps=1e-8, weight_decay=0.0,
                                  max_grad_norm=1.0)
    assert L.zero_adamw_shard_step(*args, C.byref(bad), 1, st, None) == -1
    qargs = [p, 1, p, p, p, 16, p, 1, 0, p, p, 0, 0, 128]
    assert L.zero_adamw_shard_step(*qargs, C.byref(hp), 1, st, None) == -1        # block != 256
    assert L.zero_adamw_shard_step(p, 1, C.c_void_p(0x1002), p, p, 16, p, 1, 0, None, None,
                                   0, 0, 256, C.byref(hp), 1, st, None) == -2
    assert L.zero_quant_allgather_slot(p, 0, 16, 256, p, 0, p, 0, None) == -1      # fp32 slot
    assert L.zero_quant_allgather_slot(p, 1, 16, 64, p, 0, p, 0, None) == -1
    assert L.zero_quant_allgather_slot(C.c_void_p(0x1001), 1, 16, 256, p, 0, p, 0, None) == -2
    assert b"block" in L.zero_last_error() or L.zero_last_error()


def test_consumer_and_accumulate_validate_before_launch(zf):
    L = zf.lib()
    p = C.c_void_p(0x1000)
    assert L.zero_dequant_allgather(p, p, 4, 256, 256, p, 7, None) == -1          # bad dtype
    assert L.zero_dequant_allgather(p, p, 0, 256, 256, p, 2, None) == -3          # no slots
    assert L.zero_dequant_allgather(p, p, 65537, 256, 256, p, 2, None) == -3
    assert L.zero_dequant_allgather(p, p, 4, -1, 256, p, 2, None) == -1
    assert L.zero_dequant_allgather(p, p, 4, 256, 6, p, 2, None) == -1            # block % 4
    assert L.zero_dequant_allgather(p, p, 4, 256, 0, p, 2, None) == -1
    assert L.zero_dequant_allgather(None, p, 4, 256, 256, p, 2, None) == -1
    assert L.zero_dequant_allgather(p, C.c_void_p(0x1002), 4, 256, 256, p, 2, None) == -2
    assert L.zero_dequant_allgather(p, p, 4, 256, 256, C.c_void_p(0x1001), 2, None) == -2
    assert L.zero_dequant_allgather(p, p, 4, 256, 256, C.c_void_p(0x1002), 0, None) == -2
    assert L.zero_dequant_allgather(p, p, 2, 1 << 62, 256, p, 2, None) == -3      # overflow
    assert L.zero_dequant_allgather(None, None, 4, 0, 256, None, 2, None) == 0   # empty: no-op
    bufs = (C.c_void_p * 1)(0x1000)
    assert L.zero_grad_accumulate_shard(bufs, 0, 1, 0, 8, 0, p, None, None) == -3
    assert L.zero_grad_accumulate_shard(bufs, 1, 1, 0, 8, 3, p, None, None) == -1
    assert L.zero_grad_accumulate_shard(bufs, 1, 1, 0, 8, 0, None, None, None) == -1
    assert L.zero_grad_accumulate_shard(bufs, 1, 1, 0, 8, 0, C.c_void_p(0x1002), None, None) == -2
    assert b"zero_grad_accumulate_shard" in L.zero_last_error()
    assert L.zero_grad_accumulate_shard(bufs, 1, 1, 0, 0, 0, p, None, None) == 0  # empty: no-op


def test_unflatten_views_follow_the_layout(zf):
    """Views at the spans zero_flat_layout gives: the flat buffer is the
    parameters back to back, each view a reshape of its range (no copy)."""
    import torch
    shapes = [(512, 1024), (1024,), (1024, 512), (512,)]
    flat = torch.arange(1_050_112 + 3, dtype=torch.float32)       # + tail padding
    views = zf.unflatten(flat, shapes, n_ranks=4)
    off = 0
    for v, sh in zip(views, shapes):
        assert tuple(v.shape) == sh and v.data_ptr() == flat.data_ptr() + 4 * off
        assert v.flatten()[0].item() == off
        off += v.numel()
    with pytest.raises(ValueError):
        zf.unflatten(torch.zeros(10), shapes)


def test_int8_gradient_reduce_validates_before_launch(zf):
    L = zf.lib()
    p = C.c_void_p(0x1000)
    q = (C.c_void_p * 2)(0x1000, 0x2000)
    s = (C.c_void_p * 2)(0x3000, 0x4000)
    assert L.zero_grad_reduce_shard_int8(None, s, 2, 8, 256, 1, p, None, None) == -1
    assert L.zero_grad_reduce_shard_int8(q, s, 0, 8, 256, 1, p, None, None) == -3
    assert L.zero_grad_reduce_shard_int8(q, s, 129, 8, 256, 1, p, None, None) == -3
    assert L.zero_grad_reduce_shard_int8(q, s, 2, 8, 256, 4, p, None, None) == -1
    assert L.zero_grad_reduce_shard_int8(q, s, 2, 8, 250, 1, p, None, None) == -1
    assert L.zero_grad_reduce_shard_int8(q, s, 2, -1, 256, 1, p, None, None) == -1
    assert L.zero_grad_reduce_shard_int8(q, s, 2, 8, 256, 1, None, None, None) == -1
    assert L.zero_grad_reduce_shard_int8(q, s, 2, 8, 256, 1, C.c_void_p(0x1002), None, None) == -2
    bad = (C.c_void_p * 2)(0x3000, 0x4002)
    assert L.zero_grad_reduce_shard_int8(q, bad, 2, 8, 256, 1, p, None, None) == -2
    nul = (C.c_void_p * 2)(0x1000, 0)
    assert L.zero_grad_reduce_shard_int8(nul, s, 2, 8, 256, 1, p, None, None) == -1
    assert L.zero_grad_reduce_shard_int8(q, s, 2, 0, 256, 1, p, None, None) == 0


def test_offload_step_validates_before_launch(zf):
    """zero_offload_step rejects bad arguments before any copy or launch,
    among them staging buffers that overlap other than as one 16-bit buffer
    used in place."""
    L = zf.lib()
    p = C.c_void_p(0x1000)
    st = C.c_void_p(0x8000)
    hp = zf.zero_adamw_hparams_t(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0,
                                 max_grad_norm=1.0)

    def call(grad_stage=0x20000, lp_stage=0x40000, n=1024, gdt=1, pdt=1, state=st, chunk=0):
        return L.zero_offload_step(p, gdt, n, p, p, p, C.c_void_p(grad_stage),
                                   C.c_void_p(lp_stage), p, pdt, 0, C.byref(hp), state, chunk, 0,
                                   None)

    assert call(state=None) == -1
    assert call(state=C.c_void_p(0x8004)) == -2
    assert call(gdt=5) == -1
    assert call(pdt=0) == -1                                   # fp32 parameters
    assert call(n=-1) == -1
    assert call(chunk=-5) == -1
    assert call(grad_stage=0x20001) == -2
    assert call(gdt=0, lp_stage=0x20000) == -1                 # one buffer, fp32 gradient
    assert b"overlap" in L.zero_last_error()
    assert call(lp_stage=0x20002) == -1                        # 16-bit, shifted by one element
    assert call(grad_stage=0x20000, lp_stage=0x20000 + 2 * 1024 - 2) == -1   # last element shared
    assert call(gdt=0, grad_stage=0x20000, lp_stage=0x20000 + 2 * 1024) == -1  # fp32 grads: 4 B each
