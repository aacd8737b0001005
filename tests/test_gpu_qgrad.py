"""GPU parity of the quantised gradient reduce (zero_grad_reduce_shard_int8,
through its C ABI) against the oracle on the same seeded inputs: the reduce
and its statistics over both kernel paths and the edge cases, whole steps on
INT8-quantised rank gradients (Tiny MLP, all ranks; the payload written by
the library's own quantiser and checked against the oracle's), and the 10B /
8-rank shard at full size on sampled blocks.  Bar: bit-exact (NaN results
compared as NaN).

Pages: "DeepSpeed 与 FSDP" -- ZeRO++：量化通信压缩 (gradients cross the
Reduce-Scatter quantised).
"""
import math

import numpy as np
import pytest
import torch

from harness import OracleRank, assert_bitwise, assert_bitwise_nan_class, to_dev, to_host
from oracle import oracle as orc
from synth import synth
from synth.workloads import WORKLOADS, key_grad, key_master

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


QG_CASES = [
    # (n_ranks, shard, block, op, extra byte offset of the codes, special scales)
    (4, 262_528, 256, 1, 0, False), (8, 100_003, 256, 0, 0, False), (64, 20_000, 256, 1, 0, False),
    (3, 1001, 64, 1, 0, False), (2, 4097, 12, 0, 0, False), (8, 2048 * 3, 256, 1, 1, False),
    (1, 5000, 256, 1, 0, False), (128, 3000, 256, 1, 0, False), (8, 9000, 256, 1, 0, True),
]


@pytest.mark.parametrize("N,S,block,op,mis,special", QG_CASES)
def test_reduce_int8_parity(zf, N, S, block, op, mis, special):
    say("qgrad reduce", N, S, block, op, mis, special)
    nb = -(-S // block)
    tag = "%d-%d-%d-%d" % (N, S, block, op)
    qs = [synth.codes(synth.stream_key("qg", tag, "q", k), 0, S) for k in range(N)]
    scs = [np.abs(synth.normal_f32(synth.stream_key("qg", tag, "s", k), 0, nb, 4.7e-6))
           .astype(np.float32) for k in range(N)]
    if special:                      # a zero-scale block and an infinite one (-> NaN/inf)
        scs[1][3] = 0.0
        scs[5][nb - 1] = np.inf
    qd = [torch.from_numpy(np.concatenate([np.zeros(mis, np.int8), q])).cuda()[mis:] for q in qs]
    sd = [to_dev(sc, 0) for sc in scs]
    red_d = torch.full((S,), float("nan"), device="cuda")
    state = zf.StepState(65536.0, False)
    zf.zero_grad_reduce_shard_int8(qd, sd, S, op, red_d, state, block=block)
    red = orc.reduce_q8(qs, scs, S, block, op)
    assert_bitwise_nan_class(to_host(red_d), red, 0, "reduced shard")
    s_ref, o_ref = orc.unscale_stats(red, orc.F32, 65536.0)
    st = state.read()
    assert st.overflow == o_ref == int(special)
    if not special:
        assert rel(st.sumsq, s_ref) <= 1e-12


def payload_gpu(zf, grad_slice, block=256):
    """The library's quantiser on one rank's gradient slice for this rank."""
    n = grad_slice.numel()
    q = torch.empty(n, dtype=torch.int8, device="cuda")
    sc = torch.empty(-(-n // block), device="cuda")
    zf.zero_quant_allgather_slot(grad_slice, q, sc, block=block)
    return q, sc


@pytest.mark.parametrize("rank", [0, 1, 2, 3])
def test_tiny_mlp_steps_on_int8_gradients(zf, rank):
    """3 steps on rank `rank` of the Tiny MLP: every rank's fp16 gradient
    slice is quantised (library; oracle on the same slice, codes compared),
    reduced from the INT8 payloads, then the step."""
    w = WORKLOADS["tiny_mlp_n4_qg"]
    S, start = w.shard, rank * w.shard
    say("tiny qg rank", rank)
    master0 = synth.normal_f32(key_master(w), start, S, w.master_sigma)
    master0[max(0, w.total - start):] = 0.0
    opt = zf.ShardOptimizer(to_dev(master0, 0), w.hp, loss_scale=w.loss_scale,
                            dynamic=w.dynamic)
    ref = OracleRank(master0, w.loss_scale, w.dynamic)
    ag = torch.zeros(w.padded, dtype=torch.float16, device="cuda")
    for step in range(w.steps):
        qd, sd, qh, sh = [], [], [], []
        for k in range(w.n_ranks):
            x = synth.normal_f32(key_grad(w, step, k), start, S, w.grad_sigma)
            x[max(0, w.total - start):] = 0.0
            g = synth.to_storage(x, w.grad_dtype)
            q, sc = payload_gpu(zf, to_dev(g, w.grad_dtype))
            rq, rs = orc.quant_int8(g, w.grad_dtype, 256)
            assert_bitwise(to_host(q).view(np.uint8), rq.view(np.uint8), "codes rank %d" % k)
            assert_bitwise(to_host(sc), rs, "scales rank %d" % k)
            qd.append(q)
            sd.append(sc)
            qh.append(rq)
            sh.append(rs)
        opt.step_from_int8_grads(qd, sd, ag, start, op=w.op)
        red = orc.reduce_q8(qh, sh, S, 256, w.op)
        assert_bitwise(to_host(opt.reduced_buffer()), red, "reduced gradient step %d" % step)
        res = ref.step(red, orc.F32, w.hp, w.param_dtype)
        st = opt.state.read()
        assert st.last_skipped == res["skipped"] == 0
        assert abs(st.last_norm - res["norm"]) <= 1e-12 * res["norm"]
        assert st.last_coef == res["coef"]
        assert_bitwise(to_host(opt.master), ref.p, "master step %d" % step)
        assert_bitwise(to_host(opt.exp_avg), ref.m, "exp_avg step %d" % step)
        assert_bitwise(to_host(opt.exp_avg_sq), ref.v, "exp_avg_sq step %d" % step)
        assert_bitwise(to_host(ag[start:start + S]), res["lp"], "slot step %d" % step)


def test_10b_n8_int8_gradients_full_size(zf):
    """10B over 8 ranks, rank 7: 8 fp16 rank slices quantised by the library,
    reduced from INT8, then the step; 120 whole 256-element blocks (plus the
    first and last) followed by the oracle bit for bit (payload, reduced
    gradient, master, m, v, slot); the norm over the whole reduced shard
    summed independently in binary64."""
    w = WORKLOADS["10b_n8_qg"]
    S, start, N = w.shard, w.start, w.n_ranks
    nb = -(-S // 256)
    steps = 2
    say("10b qg: shard", S)
    dev = torch.device("cuda:0")
    master = torch.empty(S, device=dev)
    synth.fill_normal(master, key_master(w), start, w.master_sigma)
    opt = zf.ShardOptimizer(master, w.hp, loss_scale=w.loss_scale, dynamic=w.dynamic)
    ag = torch.zeros(w.padded, dtype=torch.float16, device=dev)
    g = torch.empty(S, dtype=torch.float16, device=dev)
    qd = [torch.empty(S, dtype=torch.int8, device=dev) for _ in range(N)]
    sd = [torch.empty(nb, device=dev) for _ in range(N)]
    rng = np.random.default_rng(13)
    blocks = np.unique(np.concatenate([rng.integers(0, nb, 120), [0, nb - 1]]))
    idx = np.concatenate([np.arange(b * 256, min((b + 1) * 256, S)) for b in blocks]).astype(np.int64)
    ref = OracleRank(synth.normal_f32_at(key_master(w), start + idx, w.master_sigma),
                     w.loss_scale, w.dynamic)
    gi = torch.from_numpy(idx).to(dev)
    bound = 6 * w.grad_sigma * 1.01 / w.loss_scale * math.sqrt(S)
    assert bound < 1.0 - 1e-6          # the clip coefficient is exactly 1 at any sum
    for step in range(steps):
        say("10b qg step", step)
        qh, sh = [], []
        for k in range(N):
            synth.fill_normal(g, key_grad(w, step, k), start, w.grad_sigma)
            zf.zero_quant_allgather_slot(g, qd[k], sd[k])
            hq, hs = [], []
            for b in blocks:
                lo, hi = b * 256, min((b + 1) * 256, S)
                xb = synth.normal_at(key_grad(w, step, k), start + np.arange(lo, hi), w.grad_sigma,
                                     w.grad_dtype)
                q1, s1 = orc.quant_int8(xb, w.grad_dtype, 256)
                hq.append(q1)
                hs.append(np.repeat(s1, hi - lo))
            qh.append(np.concatenate(hq))
            sh.append(np.concatenate(hs).astype(np.float32))
            assert_bitwise(to_host(qd[k][gi]).view(np.uint8), qh[k].view(np.uint8),
                           "codes rank %d step %d" % (k, step))
        opt.step_from_int8_grads(qd, sd, ag, start, op=w.op)
        # the sampled elements, one scale per element (block size 1)
        red = orc.reduce_q8(qh, sh, idx.size, 1, w.op)
        assert_bitwise(to_host(opt.reduced_buffer()[gi]), red, "reduced gradient step %d" % step)
        st = opt.state.read()
        rb = opt.reduced_buffer()
        sumsq = sum(torch.sum(torch.square(rb[i:i + (1 << 27)].double())).item()
                    for i in range(0, S, 1 << 27)) / (w.loss_scale ** 2)
        assert abs(st.last_norm - math.sqrt(sumsq)) <= 1e-5 * math.sqrt(sumsq)
        res = ref.step(red, orc.F32, w.hp, w.param_dtype, sumsq_local=0.0, overflow_local=0)
        assert res["coef"] == 1.0 == st.last_coef and st.last_skipped == 0
        assert_bitwise(to_host(opt.master[gi]), ref.p, "master step %d" % step)
        assert_bitwise(to_host(opt.exp_avg[gi]), ref.m, "exp_avg step %d" % step)
        assert_bitwise(to_host(opt.exp_avg_sq[gi]), ref.v, "exp_avg_sq step %d" % step)
        assert_bitwise(to_host(ag[gi + start]), res["lp"], "slot step %d" % step)
    del opt, ag, g, qd, sd, master
    torch.cuda.empty_cache()
