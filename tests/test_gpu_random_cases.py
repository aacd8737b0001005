"""Seeded random cases through the launch-shape choices of every GPU entry
point, each compared with the oracle to the same bar as the hand-picked cases
(bit-exact outputs and flags; the sum of squares within n * 2^-53 relative).

A case draws, from its own seed: the rank count (which picks the tile shape,
one buffer group or several, and the run length), the format, SUM or AVG, the
shard length (tails of every size), the element offset and the start of each
buffer inside its allocation (so pointers are 2-, 4-, 8- or 16-byte aligned
and the vector and element-wise paths both run), accumulation into an fp32
shard or a plain reduce, and whether the statistics are taken.  The
quantiser, the INT8 consumer and the AdamW step get random lengths, offsets,
formats, blocks and clipping the same way.  ZF_RANDOM_SCALE=k in the
environment draws k times as many seeds of every kind."""
import os

import numpy as np
import pytest
import torch

from harness import assert_bitwise, assert_bitwise_nan_class, to_dev, to_host
from oracle import oracle as orc
from synth import synth

pytestmark = pytest.mark.gpu

# ZF_RANDOM_SCALE=k draws k times as many seeds of every kind (default 1)
SCALE = max(1, int(os.environ.get("ZF_RANDOM_SCALE", "1")))

TORCH_DT = {0: torch.float32, 1: torch.float16, 2: torch.bfloat16}


@pytest.fixture(scope="module")
def zf():
    import fsdp_sharded_mixed_flatparameter_amd as m
    assert torch.cuda.is_available()
    return m


def say(*a):
    print(*a, flush=True)


def rel(a, b):
    return abs(a - b) / max(abs(b), 1e-300)


def view_at(h, code, start):
    """Device copy of host array h (float32 or 16-bit patterns) that begins
    `start` elements into its allocation."""
    pad = np.zeros(start, h.dtype)
    return to_dev(np.concatenate([pad, h]), code)[start:]


def reduce_case(i):
    """The drawn parameters of random reduce case i.  Offsets favour alignment,
    so that about half the cases take the vector path (every buffer at
    start + off a multiple of 4 elements and the output 16-byte aligned)."""
    r = np.random.default_rng(7100 + i)
    N = int(r.choice([1, 1, 2, 3, 4, 4, 5, 8, 8, 8, 12, 16, 16, 17, 24, 32, 48, 64, 64, 70]))
    dt = int(r.integers(0, 3))
    op = int(r.integers(0, 2))
    S = int(r.choice([1, 3, 255, 256, 257, 511, 512, 1023, 4097, 30_001, 123_457, 262_144,
                      300_001, 1_000_003]))
    S = max(1, min(S, 4_000_000 // N))
    aligned = bool(r.integers(0, 2))
    off = int(r.choice([0, 4, 8, 12])) if aligned else int(r.integers(0, 9))
    start = int(r.choice([0, 4])) if aligned else int(r.integers(0, 5))
    out_start = 0 if aligned else int(r.integers(0, 4))
    acc = bool(r.integers(0, 2))
    stats = bool(r.integers(0, 2))
    scale = float(r.choice([1.0, 1024.0, 65536.0]))
    return N, dt, op, S, off, start, out_start, acc, stats, scale


@pytest.mark.parametrize("i", range(60 * SCALE))
def test_random_reduce(zf, i):
    N, dt, op, S, off, start, out_start, acc, stats, scale = reduce_case(i)
    say("random reduce", i, dict(N=N, dt=dt, op=op, S=S, off=off, start=start, out_start=out_start,
                                 acc=acc, stats=stats, scale=scale))
    total = off + S + 2
    bufs = [synth.normal(synth.stream_key("rnd-red", i, k), 0, total, 1e-3 * (1 + k % 5), dt)
            for k in range(N)]
    dbufs = [view_at(b, dt, start) for b in bufs]
    state = zf.StepState(scale, False) if stats else None
    if acc:
        acc0 = synth.normal_f32(synth.stream_key("rnd-acc", i), 0, S, 1e-3)
        out = view_at(acc0, 0, out_start)
        zf.zero_grad_accumulate_shard(dbufs, off, S, op, out, state)
        ref = acc0.copy()
        orc.reduce_accumulate(bufs, dt, off, S, op, ref)
    else:
        out = torch.full((out_start + S,), float("nan"), device="cuda")[out_start:]
        zf.zero_grad_reduce_shard(dbufs, off, S, op, out, state)
        ref = orc.reduce(bufs, dt, off, S, op)
    assert_bitwise(to_host(out), ref, "reduced shard")
    if stats:
        s_ref, o_ref = orc.unscale_stats(ref, orc.F32, scale)
        st = state.read()
        assert st.overflow == o_ref == 0
        assert rel(st.sumsq, s_ref) <= max(1e-12, S * 2.0 ** -53)


@pytest.mark.parametrize("i", range(12 * SCALE))
def test_random_int8_reduce(zf, i):
    r = np.random.default_rng(7300 + i)
    N = int(r.choice([1, 2, 3, 8, 16, 24, 64]))
    S = int(r.choice([1, 100, 256, 1000, 4097, 77_777, 200_003]))
    block = int(r.choice([4, 12, 64, 256, 1000]))
    op = int(r.integers(0, 2))
    mis = int(r.integers(0, 4))
    say("random int8 reduce", i, dict(N=N, S=S, block=block, op=op, mis=mis))
    nb = -(-S // block)
    qs = [synth.codes(synth.stream_key("rnd-q", i, k), 0, S) for k in range(N)]
    scs = [np.abs(synth.normal_f32(synth.stream_key("rnd-s", i, k), 0, nb, 4.7e-6))
           .astype(np.float32) for k in range(N)]
    qd = [torch.from_numpy(np.concatenate([np.zeros(mis, np.int8), q])).cuda()[mis:] for q in qs]
    red = torch.full((S,), float("nan"), device="cuda")
    state = zf.StepState(65536.0, False)
    zf.zero_grad_reduce_shard_int8(qd, [to_dev(sc, 0) for sc in scs], S, op, red, state,
                                   block=block)
    ref = orc.reduce_q8(qs, scs, S, block, op)
    assert_bitwise_nan_class(to_host(red), ref, 0, "reduced shard")
    s_ref, o_ref = orc.unscale_stats(ref, orc.F32, 65536.0)
    st = state.read()
    assert st.overflow == o_ref == 0
    assert rel(st.sumsq, s_ref) <= max(1e-12, S * 2.0 ** -53)


@pytest.mark.parametrize("i", range(16 * SCALE))
def test_random_quantiser(zf, i):
    r = np.random.default_rng(7500 + i)
    pdt = int(r.integers(1, 3))
    n = int(r.choice([1, 255, 256, 257, 2047, 2048, 2049, 10_000, 65_537, 300_000]))
    path = int(r.integers(0, 3))   # the kernel the alignment picks: 8 per lane, quad, element-wise
    start, q_off = ((int(r.choice([0, 8])), int(r.choice([0, 8]))) if path == 0 else
                    (4, 4) if path == 1 else (int(r.integers(0, 9)), int(r.integers(0, 9))))
    say("random quantiser", i, dict(pdt=pdt, n=n, start=start, q_off=q_off))
    x = synth.normal(synth.stream_key("rnd-x", i), 0, n, float(r.choice([1e-3, 0.02, 3.0])), pdt)
    nb = -(-n // 256)
    q = torch.zeros(q_off + n + 8, dtype=torch.int8, device="cuda")
    s = torch.zeros(nb, device="cuda")
    zf.zero_quant_allgather_slot(view_at(x, pdt, start), q, s, q_slot_offset=q_off)
    rq, rs = orc.quant_int8(x, pdt, 256)
    qh = to_host(q)
    assert_bitwise(qh[q_off:q_off + n].view(np.uint8), rq.view(np.uint8), "codes")
    assert not qh[:q_off].any() and not qh[q_off + n:].any()
    assert_bitwise(to_host(s), rs, "scales")


@pytest.mark.parametrize("i", range(12 * SCALE))
def test_random_consumer(zf, i):
    r = np.random.default_rng(7700 + i)
    n_slots = int(r.integers(1, 10))
    S = int(r.choice([1, 100, 256, 2048, 2049, 30_001, 100_000]))
    block = int(r.choice([4, 12, 64, 256, 1000]))
    out_dt = int(r.integers(0, 3))
    start = 0 if r.integers(0, 2) else int(r.integers(0, 4))
    say("random consumer", i, dict(n_slots=n_slots, S=S, block=block, out_dt=out_dt, start=start))
    nb = -(-S // block)
    q = synth.codes(synth.stream_key("rnd-dq", i), 0, n_slots * S)
    sc = np.abs(synth.normal_f32(synth.stream_key("rnd-dqs", i), 0, n_slots * nb, 4.7e-4)) \
        .astype(np.float32)
    out = torch.empty(start + n_slots * S, dtype=TORCH_DT[out_dt], device="cuda")[start:]
    zf.zero_dequant_allgather(torch.from_numpy(q).cuda(), to_dev(sc, 0), n_slots, S, out,
                              block=block)
    ref = orc.dequant_int8(q, sc, n_slots, S, block, out_dt)
    assert_bitwise(to_host(out), ref, "dequantised flat parameter")


@pytest.mark.parametrize("i", range(10 * SCALE))
def test_random_adamw_steps(zf, i):
    import test_gpu_parity as parity
    r = np.random.default_rng(7900 + i)
    gdt = int(r.integers(0, 3))
    pdt = int(r.integers(1, 3))
    n = int(r.choice([1, 255, 1000, 1024, 4097, 65_537, 262_528]))
    slot = int(r.integers(0, 10))
    quant = bool(r.integers(0, 2))
    max_norm = float(r.choice([0.0, 1e-4, 1.0]))
    scale = float(r.choice([1.0, 1024.0, 65536.0])) if gdt != 2 else 1.0
    say("random adamw", i, dict(gdt=gdt, pdt=pdt, n=n, slot=slot, quant=quant, max_norm=max_norm,
                                scale=scale))
    parity.test_adamw_step_parity(zf, gdt, pdt, n, slot, quant, max_norm, scale)


@pytest.mark.parametrize("i", range(12 * SCALE))
def test_random_offload(zf, i):
    """The offloaded step (statistics on the GPU, the update on host threads,
    chunked copies both ways) over a random size, chunk, thread count, pair of
    formats and staging (in place or two buffers), two steps, the second
    sometimes overflowing; master, m, v and the slot bit for bit."""
    from harness import OracleRank
    r = np.random.default_rng(8100 + i)
    gdt = int(r.integers(0, 3))
    pdt = int(r.integers(1, 3))
    n = int(r.choice([1, 100, 4097, 65_536, 100_003, 300_001]))
    chunk = max(int(r.choice([1, 1000, 4096, 65_536, 1 << 24])), -(-n // 64))   # <= 64 chunks
    threads = int(r.integers(1, 17))
    in_place = bool(r.integers(0, 2))
    slot = int(r.integers(0, 9))
    scale = 1024.0 if gdt != 2 else 1.0
    overflow_step = int(r.integers(0, 3))          # 2: no overflow
    say("random offload", i, dict(gdt=gdt, pdt=pdt, n=n, chunk=chunk, threads=threads,
                                  in_place=in_place, slot=slot, overflow_step=overflow_step))
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, max_grad_norm=1.0)
    p0 = synth.normal_f32(synth.stream_key("rnd-off-p", i), 0, n, 0.02)
    opt = zf.OffloadShardOptimizer(torch.from_numpy(p0.copy()), hp, loss_scale=scale, dynamic=True,
                                   window=1, n_threads=threads, chunk=chunk,
                                   in_place_staging=in_place)
    ref = OracleRank(p0, scale, True, window=1)
    ag = torch.zeros(slot + n + 3, dtype=TORCH_DT[pdt], device="cuda")
    for step in range(2):
        g = synth.normal(synth.stream_key("rnd-off-g", i, step), 0, n, 1e-3 * scale, gdt)
        if step == overflow_step:
            g[n // 2] = np.float32(np.inf) if gdt == 0 else 0x7F80 if gdt == 2 else 0x7C00
        opt.step_from_reduced(to_dev(g, gdt), ag, slot)
        res = ref.step(g, gdt, hp, pdt)
        st = opt.state.read()
        assert st.last_skipped == res["skipped"] == int(step == overflow_step)
        assert (st.loss_scale, st.good_steps, st.step) == \
            (ref.scaler.loss_scale, ref.scaler.good_steps, ref.scaler.step)
        assert_bitwise(opt.master.numpy(), ref.p, "master step %d" % step)
        assert_bitwise(opt.exp_avg.numpy(), ref.m, "exp_avg step %d" % step)
        assert_bitwise(opt.exp_avg_sq.numpy(), ref.v, "exp_avg_sq step %d" % step)
        if not res["skipped"]:
            assert st.last_coef == res["coef"]
            assert_bitwise(to_host(ag[slot:slot + n]), res["lp"], "slot step %d" % step)
    assert not to_host(ag[:slot]).any() and not to_host(ag[slot + n:]).any()
