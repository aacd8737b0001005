"""GPU parity of sharded gradient accumulation (zero_grad_accumulate_shard,
through its C ABI) against the oracle on the same seeded inputs: every
micro-step's accumulated shard bit for bit over both kernel paths, the step
statistics taken on the last micro-step, whole optimizer steps on accumulated
gradients (Tiny MLP, all 4 ranks), an overflow in an early micro-step, and the
10B / 8-rank shard at full size on samples.

Pages: "DeepSpeed 与 FSDP" 实践要点 (gradient accumulation, loss divided by
the step count); ZeRO reading at 2kiu.com §5.1 (two accumulation steps),
§5.3 (accumulated while sharded).
"""
import math

import numpy as np
import pytest
import torch

from harness import OracleRank, assert_bitwise, to_dev, to_host
from oracle import oracle as orc
from synth import synth
from synth.workloads import WORKLOADS, key_grad_micro, key_master

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def zf():
    import fsdp_sharded_mixed_flatparameter_amd as m
    assert torch.cuda.is_available()
    return m


def say(*a):
    print(*a, flush=True)


def rel(a, b):
    return abs(a - b) / max(abs(b), 1e-300)


ACC_CASES = [
    # (dtype, n_ranks, op, shard, elem_offset, micro_steps)
    (1, 4, 1, 262_528, 262_528, 2), (2, 8, 0, 100_003, 16, 3), (1, 64, 1, 20_000, 0, 2),
    (0, 2, 1, 3001, 1, 2), (1, 3, 1, 1000, 3, 2), (2, 8, 1, 1, 0, 2), (1, 1, 0, 4097, 0, 4),
    (2, 5, 1, 2048 * 4, 8, 2),
    (1, 256, 1, 2001, 0, 2), (2, 255, 0, 999, 4, 2),     # the most buffers per call, odd below
]


@pytest.mark.parametrize("dt,N,op,S,off,K", ACC_CASES)
def test_accumulate_parity(zf, dt, N, op, S, off, K):
    say("accumulate", dt, N, op, S, off, K)
    total = off + S + 3
    acc_d = torch.zeros(S, device="cuda")
    acc = np.zeros(S, np.float32)
    state = zf.StepState(1024.0, False)
    for k in range(K):
        bufs = [synth.normal(synth.stream_key("acc", dt, N, S, k, r), 0, total, 1e-3 * (r + 1), dt)
                for r in range(N)]
        last = k == K - 1
        zf.zero_grad_accumulate_shard([to_dev(b, dt) for b in bufs], off, S, op, acc_d,
                                      state if last else None)
        orc.reduce_accumulate(bufs, dt, off, S, op, acc)
        assert_bitwise(to_host(acc_d), acc, "accumulated shard after micro-step %d" % k)
    s_ref, o_ref = orc.unscale_stats(acc, orc.F32, 1024.0)
    st = state.read()
    assert st.overflow == o_ref == 0
    assert rel(st.sumsq, s_ref) <= 1e-12


def test_first_micro_step_by_reduce_equals_accumulating_into_zeros(zf):
    dt, N, S = 2, 8, 50_000
    bufs = [to_dev(synth.normal(synth.stream_key("acc0", r), 0, S, 1e-3, dt), dt) for r in range(N)]
    a = torch.zeros(S, device="cuda")
    b = torch.full((S,), float("nan"), device="cuda")
    zf.zero_grad_accumulate_shard(bufs, 0, S, 1, a)
    zf.zero_grad_reduce_shard(bufs, 0, S, 1, b)
    assert_bitwise(to_host(a), to_host(b), "reduce vs accumulate into zeros")


def test_overflow_in_an_early_micro_step_skips_the_step(zf):
    """+inf in micro-step 0 stays non-finite in the shard: the statistics of
    the last micro-step flag it and the step is skipped."""
    w = WORKLOADS["tiny_mlp_n4_accum2"]
    S, start = w.shard, w.start
    master = torch.zeros(S, device="cuda")
    opt = zf.ShardOptimizer(master, w.hp, loss_scale=w.loss_scale, dynamic=True)
    ag = torch.zeros(w.padded, dtype=torch.float16, device="cuda")
    for micro in range(2):
        bufs = [torch.zeros(w.padded, dtype=torch.float16, device="cuda") for _ in range(4)]
        if micro == 0:
            bufs[2][start + 17] = float("inf")
        opt.micro_step(bufs, start, first=micro == 0, last=micro == 1)
    opt.step_from_accumulated(ag, start)
    st = opt.state.read()
    assert st.last_skipped == 1 and st.step == 0 and st.loss_scale == w.loss_scale / 2
    assert not ag.any() and not opt.master.any()


def micro_bufs_host(w, step, micro, start, n):
    """Rank buffers of one micro-step over flat [start, start+n) (zero past T)."""
    out = []
    for k in range(w.n_ranks):
        x = synth.normal_f32(key_grad_micro(w, step, micro, k), start, n, w.grad_sigma)
        x[max(0, w.total - start):] = 0.0
        out.append(synth.to_storage(x, w.grad_dtype))
    return out


@pytest.mark.parametrize("rank", [0, 1, 2, 3])
def test_tiny_mlp_accumulated_steps(zf, rank):
    """3 optimizer steps of 2 micro-steps each on rank `rank` of the Tiny MLP
    (4 ranks), against the oracle's reduce + accumulate + step."""
    w0 = WORKLOADS["tiny_mlp_n4_accum2"]
    S, start = w0.shard, rank * w0.shard
    say("tiny accum2 rank", rank)
    master0 = synth.normal_f32(key_master(w0), start, S, w0.master_sigma)
    master0[max(0, w0.total - start):] = 0.0
    opt = zf.ShardOptimizer(to_dev(master0, 0), w0.hp, loss_scale=w0.loss_scale,
                            dynamic=w0.dynamic)
    ref = OracleRank(master0, w0.loss_scale, w0.dynamic)
    ag = torch.zeros(w0.padded, dtype=torch.float16, device="cuda")
    for step in range(w0.steps):
        acc = np.zeros(S, np.float32)
        for micro in range(w0.micro_steps):
            full = micro_bufs_host(w0, step, micro, 0, w0.padded)
            opt.micro_step([to_dev(b, w0.grad_dtype) for b in full], start, op=w0.op,
                           first=micro == 0, last=micro == w0.micro_steps - 1)
            orc.reduce_accumulate(full, w0.grad_dtype, start, S, w0.op, acc)
        assert_bitwise(to_host(opt.reduced_buffer()), acc, "accumulated gradient step %d" % step)
        opt.step_from_accumulated(ag, start)
        res = ref.step(acc, orc.F32, w0.hp, w0.param_dtype)
        st = opt.state.read()
        assert st.last_skipped == res["skipped"] == 0
        assert abs(st.last_norm - res["norm"]) <= 1e-12 * res["norm"]
        assert st.last_coef == res["coef"]
        assert_bitwise(to_host(opt.master), ref.p, "master step %d" % step)
        assert_bitwise(to_host(opt.exp_avg), ref.m, "exp_avg step %d" % step)
        assert_bitwise(to_host(opt.exp_avg_sq), ref.v, "exp_avg_sq step %d" % step)
        assert_bitwise(to_host(ag[start:start + S]), res["lp"], "slot step %d" % step)


# ------------------------------------------------------------------ full size
def test_10b_n8_accum2_full_size(zf):
    """10B over 8 ranks, rank 7: 2 micro-steps of 8 fp16 rank slices per step,
    accumulated in the fp32 shard, then the step; sampled elements followed by
    the oracle bit for bit, the norm of step 0 over the whole shard."""
    w = WORKLOADS["10b_n8_accum2"]
    S, start, N = w.shard, w.start, w.n_ranks
    steps = 2
    say("10b accum2: shard", S)
    dev = torch.device("cuda:0")
    master = torch.empty(S, device=dev)
    synth.fill_normal(master, key_master(w), start, w.master_sigma)
    opt = zf.ShardOptimizer(master, w.hp, loss_scale=w.loss_scale, dynamic=w.dynamic)
    ag = torch.zeros(w.padded, dtype=torch.float16, device=dev)
    slices = [torch.empty(S, dtype=torch.float16, device=dev) for _ in range(N)]
    rng = np.random.default_rng(11)
    idx = np.unique(np.concatenate([rng.integers(0, S, 30_000), np.arange(0, 1024),
                                    np.arange(S - 1024, S)])).astype(np.int64)
    x = synth.normal_f32_at(key_master(w), start + idx, w.master_sigma)
    ref = OracleRank(x, w.loss_scale, w.dynamic)
    for step in range(steps):
        acc = np.zeros(idx.size, np.float32)
        for micro in range(w.micro_steps):
            say("10b accum2 step", step, "micro", micro)
            for k in range(N):
                synth.fill_normal(slices[k], key_grad_micro(w, step, micro, k), start,
                                  w.grad_sigma)
            opt.micro_step(slices, 0, op=w.op, first=micro == 0,
                           last=micro == w.micro_steps - 1)
            hb = [synth.normal_at(key_grad_micro(w, step, micro, k), start + idx, w.grad_sigma,
                                  w.grad_dtype) for k in range(N)]
            orc.reduce_accumulate(hb, w.grad_dtype, 0, idx.size, w.op, acc)
        got = to_host(opt.reduced_buffer()[torch.from_numpy(idx).to(dev)])
        assert_bitwise(got, acc, "accumulated gradient samples step %d" % step)
        opt.step_from_accumulated(ag, start)
        st = opt.state.read()
        # the norm over the whole accumulated shard (checked bitwise on samples
        # above), summed independently in binary64 by torch, chunk by chunk
        red = opt.reduced_buffer()
        sumsq = sum(torch.sum(torch.square(red[i:i + (1 << 27)].double())).item()
                    for i in range(0, S, 1 << 27)) / (w.loss_scale ** 2)
        assert abs(st.last_norm - math.sqrt(sumsq)) <= 1e-5 * math.sqrt(sumsq)
        # |u| <= 2 micro-steps * 6 sigma (+ rounding) / scale bounds the norm far
        # below max_norm, so the clip coefficient is exactly 1 at any sum
        assert 2 * 6 * w.grad_sigma * 1.01 / w.loss_scale * math.sqrt(S) < 1.0 - 1e-6
        res = ref.step(acc, orc.F32, w.hp, w.param_dtype, sumsq_local=0.0, overflow_local=0)
        assert res["coef"] == 1.0 == st.last_coef and st.last_skipped == 0
        gi = torch.from_numpy(idx).to(dev)
        assert_bitwise(to_host(opt.master[gi]), ref.p, "master step %d" % step)
        assert_bitwise(to_host(opt.exp_avg[gi]), ref.m, "exp_avg step %d" % step)
        assert_bitwise(to_host(opt.exp_avg_sq[gi]), ref.v, "exp_avg_sq step %d" % step)
        assert_bitwise(to_host(ag[gi + start]), res["lp"], "slot step %d" % step)
    del opt, ag, slices, master
    torch.cuda.empty_cache()

