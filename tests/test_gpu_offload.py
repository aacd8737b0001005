"""GPU parity of the ZeRO-Offload step (zero_offload_step through the C ABI:
device statistics, chunked device-to-host gradient copies, the update on host
cores, host-to-device parameter copies into the All-Gather slot, the device
loss-scaler update) against the oracle on the same seeded inputs: the Tiny
MLP on all ranks with ragged chunks and a skipped step, and the 10B / 8-rank
shard at full size on samples.  Bar: bit-exact.

Pages: "DeepSpeed 与 FSDP", ZeRO-Offload; ZeRO reading at 2kiu.com §4.1, §5.1.
"""
import math

import numpy as np
import pytest
import torch

from harness import OracleRank, assert_bitwise, to_dev, to_host
from oracle import oracle as orc
from synth import synth
from synth.workloads import WORKLOADS, key_grad_reduced, key_master

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def zf():
    import fsdp_sharded_mixed_flatparameter_amd as m
    assert torch.cuda.is_available()
    return m


def say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("rank,in_place,gdt", [(0, True, 1), (1, True, 1), (2, True, 1),
                                               (3, True, 1), (0, False, 1), (3, False, 1),
                                               (1, True, 0)])
def test_tiny_mlp_offloaded_steps(zf, rank, in_place, gdt):
    """4 steps of the Tiny MLP's rank `rank` with the update on 3 host threads
    in chunks of 10,000 elements (a ragged last chunk); step 2 carries an inf
    in the gradient: skipped on the host, scale halved on the device.  The
    pinned staging is one buffer used in place, or one per direction (always
    so for an fp32 gradient, gdt 0)."""
    w = WORKLOADS["tiny_mlp_n4"]
    S, start = w.shard, rank * w.shard
    say("tiny offload rank", rank, "in place" if in_place else "two staging buffers",
        "grad dtype", gdt)
    master0 = synth.normal_f32(key_master(w), start, S, w.master_sigma)
    master0[max(0, w.total - start):] = 0.0
    opt = zf.OffloadShardOptimizer(torch.from_numpy(master0.copy()), w.hp,
                                   loss_scale=w.loss_scale, dynamic=True, n_threads=3,
                                   chunk=10_000, in_place_staging=in_place)
    ref = OracleRank(master0, w.loss_scale, True)
    ag = torch.zeros(w.padded, dtype=torch.float16, device="cuda")
    for step in range(4):
        x = synth.normal_f32(key_grad_reduced(w, step), start, S, w.grad_sigma)
        x[max(0, w.total - start):] = 0.0
        g = synth.to_storage(x, gdt).copy()
        if step == 2:
            g[S // 2] = np.inf if gdt == 0 else 0x7C00
        before = opt.master.clone()
        opt.step_from_reduced(to_dev(g, gdt), ag, start)
        res = ref.step(g, gdt, w.hp, w.param_dtype)
        st = opt.state.read()
        assert st.last_skipped == res["skipped"] == int(step == 2)
        assert (st.loss_scale, st.good_steps, st.step) == \
            (ref.scaler.loss_scale, ref.scaler.good_steps, ref.scaler.step)
        if step == 2:
            assert torch.equal(opt.master, before)
            continue
        # the two sums of squares add S non-negative terms in different orders:
        # each within (S - 1) * 2^-53 relative of the exact sum
        assert abs(st.last_norm - res["norm"]) <= max(1e-12, S * 2.0 ** -53) * res["norm"]
        assert st.last_coef == res["coef"]
        assert_bitwise(opt.master.numpy(), ref.p, "master step %d" % step)
        assert_bitwise(opt.exp_avg.numpy(), ref.m, "exp_avg step %d" % step)
        assert_bitwise(opt.exp_avg_sq.numpy(), ref.v, "exp_avg_sq step %d" % step)
        assert_bitwise(to_host(ag[start:start + S]), res["lp"], "slot step %d" % step)
    assert not ag[:start].any() and not ag[start + S:].any()


def test_10b_n8_offload_full_size(zf):
    """10B over 8 ranks, rank 7, offloaded: 15 GB of fp32 state in host
    memory, 16 host threads; 40,000 sampled elements plus both ends followed
    by the oracle bit for bit, the norm over the whole shard in binary64."""
    w = WORKLOADS["10b_n8"]
    S, start = w.shard, w.start
    say("10b offload: shard", S)
    master = torch.empty(S, dtype=torch.float32)
    master.copy_(synth.fill_normal(torch.empty(S, device="cuda"), key_master(w), start,
                                   w.master_sigma).cpu())
    opt = zf.OffloadShardOptimizer(master, w.hp, loss_scale=w.loss_scale, dynamic=w.dynamic,
                                   n_threads=16)
    ag = torch.zeros(w.padded, dtype=torch.float16, device="cuda")
    g = torch.empty(S, dtype=torch.float16, device="cuda")
    rng = np.random.default_rng(17)
    idx = np.unique(np.concatenate([rng.integers(0, S, 40_000), np.arange(0, 1024),
                                    np.arange(S - 1024, S)])).astype(np.int64)
    ref = OracleRank(synth.normal_f32_at(key_master(w), start + idx, w.master_sigma),
                     w.loss_scale, w.dynamic)
    ti = torch.from_numpy(idx)
    for step in range(2):
        say("10b offload step", step)
        synth.fill_normal(g, key_grad_reduced(w, step), start, w.grad_sigma)
        opt.step_from_reduced(g, ag, start)
        st = opt.state.read()
        sumsq = sum(torch.sum(torch.square(g[i:i + (1 << 27)].double())).item()
                    for i in range(0, S, 1 << 27)) / (w.loss_scale ** 2)
        assert abs(st.last_norm - math.sqrt(sumsq)) <= 1e-5 * math.sqrt(sumsq)
        gs = synth.normal_at(key_grad_reduced(w, step), start + idx, w.grad_sigma, w.grad_dtype)
        res = ref.step(gs, w.grad_dtype, w.hp, w.param_dtype, sumsq_local=sumsq, overflow_local=0)
        assert res["coef"] == 1.0 == st.last_coef and st.last_skipped == 0
        assert_bitwise(opt.master[ti].numpy(), ref.p, "master step %d" % step)
        assert_bitwise(opt.exp_avg[ti].numpy(), ref.m, "exp_avg step %d" % step)
        assert_bitwise(opt.exp_avg_sq[ti].numpy(), ref.v, "exp_avg_sq step %d" % step)
        assert_bitwise(to_host(ag[torch.from_numpy(idx + start).cuda()]), res["lp"],
                       "slot step %d" % step)
    assert not ag[start - (1 << 20):start].any()
    del opt, ag, g, master
    torch.cuda.empty_cache()
