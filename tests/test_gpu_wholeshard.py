"""Whole-shard parity at full size: every element of the shard, after the last
step, against the oracle -- the fp32 master, m and v, the 16-bit slot, and on
the 70B workload the INT8 codes and block scales.  ZeRO gives the same update
as an unsharded step (2kiu.com §5.2), so nothing short of the whole shard
shows that the sharded step computed it everywhere.

The oracle streams the shard in 2^24-element chunks on host threads: an
element's trajectory depends only on its own inputs and on the per-step
scalars (clip coefficient, skip), and those depend only on the gradients, so
pass 1 takes each step's global sum of squares over all chunks (compared with
the GPU's norm at every step) and pass 2 runs every chunk through all steps
and compares it with the GPU's state.

Inputs: the GPU fills its tensors with the device copy of the seeded
generator, and the oracle receives host copies of exactly those tensors (the
generator's values; copying 20 GB down beats regenerating it on the host).
That they are the generator's values is checked against its host
implementation at sampled indices in each test.
"""
import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

from harness import assert_bitwise, to_host
from oracle import oracle as orc
from synth import synth
from synth.workloads import WORKLOADS, key_grad_reduced, key_master

pytestmark = pytest.mark.gpu

THREADS = min(16, os.cpu_count() or 4)
CHUNK = 1 << 24          # a multiple of the INT8 block: blocks restart at chunk starts too


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def zf():
    import fsdp_sharded_mixed_flatparameter_amd as m
    assert torch.cuda.is_available()
    return m


def check_generator(host, key, start, sigma, dtype, S, seed):
    """The host copy holds the seeded generator's values (host implementation,
    sampled indices plus both ends)."""
    rng = np.random.default_rng(seed)
    idx = np.unique(np.concatenate([rng.integers(0, S, 20_000), [0, 1, S - 2, S - 1]]))
    want = (synth.normal_f32_at(key, start + idx, sigma) if dtype == orc.F32
            else synth.normal_at(key, start + idx, sigma, dtype))
    assert_bitwise(host[idx], want, "generator copy")


def chunk_sums(g_host, dtype, scale):
    """The oracle's sum of squares of u = f32(g) / scale over the whole shard:
    chunks on threads, chunk sums added in chunk order."""
    S = g_host.size

    def job(lo):
        return orc.unscale_stats(np.ascontiguousarray(g_host[lo:lo + CHUNK]), dtype, scale)

    with ThreadPoolExecutor(THREADS) as ex:
        parts = list(ex.map(job, range(0, S, CHUNK)))
    return sum(p[0] for p in parts), int(any(p[1] for p in parts))


def run_whole_shard(zf, w, steps, quant):
    S, start = w.shard, w.start
    gd, pd = w.grad_dtype, w.param_dtype
    tdt = {orc.F16: torch.float16, orc.BF16: torch.bfloat16}
    dev = torch.device("cuda:0")
    say(w.name, "whole shard:", S, "elements,", steps, "steps")
    master = torch.empty(S, device=dev)
    synth.fill_normal(master, key_master(w), start, w.master_sigma)
    master0 = to_host(master).copy()
    check_generator(master0, key_master(w), start, w.master_sigma, orc.F32, S, 1)
    opt = zf.ShardOptimizer(master, w.hp, loss_scale=w.loss_scale, dynamic=w.dynamic,
                            quant_block=256 if quant else 0)
    if w.full_allgather:
        ag, off = torch.zeros(w.padded, dtype=tdt[pd], device=dev), start
    else:
        ag, off = torch.zeros(S, dtype=tdt[pd], device=dev), 0
    nb = -(-S // 256)
    q = torch.zeros(S, dtype=torch.int8, device=dev) if quant else None
    qs = torch.zeros(nb, device=dev) if quant else None
    g = torch.empty(S, dtype=tdt[gd], device=dev)
    grads, coefs = [], []
    for step in range(steps):
        synth.fill_normal(g, key_grad_reduced(w, step), start, w.grad_sigma)
        gh = to_host(g).copy()
        check_generator(gh, key_grad_reduced(w, step), start, w.grad_sigma, gd, S, 2 + step)
        grads.append(gh)
        opt.step_from_reduced(g, ag, off, q_buf=q, q_scales=qs)
        st = opt.state.read()
        # pass 1: the step's global sum of squares, compared with the GPU's norm
        sumsq, ovf = chunk_sums(gh, gd, w.loss_scale)
        assert ovf == 0 and st.last_skipped == 0
        norm = math.sqrt(sumsq)
        assert abs(st.last_norm - norm) <= 1e-5 * norm, (step, st.last_norm, norm)
        coef = orc.clip_coef(sumsq, w.hp["max_grad_norm"])
        assert st.last_coef == coef, (step, st.last_coef, coef)
        coefs.append(coef)
        say("  step", step, "norm", st.last_norm, "oracle", norm, "coef", coef)
    torch.cuda.synchronize()
    del g
    slot = ag[off:off + S]
    hp = orc.Hparams(**w.hp)

    # pass 2: every chunk through every step, compared with the GPU's state
    def job(lo):
        n = min(CHUNK, S - lo)
        p = master0[lo:lo + n].copy()
        m = np.zeros(n, np.float32)
        v = np.zeros(n, np.float32)
        lp = None
        for step in range(steps):
            lp = orc.adamw(np.ascontiguousarray(grads[step][lo:lo + n]), gd, p, m, v,
                           w.loss_scale, coefs[step], step + 1, hp, pd)
        where = "chunk at %d" % lo
        assert_bitwise(to_host(opt.master[lo:lo + n]), p, "master, " + where)
        assert_bitwise(to_host(opt.exp_avg[lo:lo + n]), m, "exp_avg, " + where)
        assert_bitwise(to_host(opt.exp_avg_sq[lo:lo + n]), v, "exp_avg_sq, " + where)
        assert_bitwise(to_host(slot[lo:lo + n]), lp, "slot, " + where)
        if quant:
            rq, rs = orc.quant_int8(lp, pd, 256)
            b0 = lo // 256
            assert_bitwise(to_host(q[lo:lo + n]).view(np.uint8), rq.view(np.uint8),
                           "INT8 codes, " + where)
            assert_bitwise(to_host(qs[b0:b0 + rs.size]), rs, "INT8 scales, " + where)
        return n

    with ThreadPoolExecutor(THREADS) as ex:
        done = sum(ex.map(job, range(0, S, CHUNK)))
    assert done == S
    st = opt.state.read()
    assert st.step == steps
    if w.full_allgather:   # nothing outside the rank's slot was written
        assert not ag[:off].any() and not ag[off + S:].any()
    del opt, ag, q, qs, master
    torch.cuda.empty_cache()


def test_10b_n8_whole_shard(zf):
    """10B over 8 ranks, rank 7: 1.25e9 elements, pre-reduced fp16 gradients,
    fp16 write-back into the full All-Gather buffer at offset 8.75e9."""
    run_whole_shard(zf, WORKLOADS["10b_n8"], steps=2, quant=False)


def test_70b_n64_int8_whole_shard(zf):
    """70B over 64 ranks, rank 63: 1.09375e9 elements, bf16, clipping active,
    bf16 write-back and the INT8 payload (4,272,461 blocks, the last of 240)."""
    w = WORKLOADS["70b_n64_int8"]
    run_whole_shard(zf, w, steps=2, quant=True)
