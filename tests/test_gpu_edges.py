"""Edge cases of every entry point on the GPU, through the C ABI: empty inputs
(nothing launched, nothing written, the counters still advance on a finalize)
and shards past 2^32 elements (64-bit indexing in every kernel), checked
against the oracle on samples around 2^31, 2^32 and the ragged end.
"""
import numpy as np
import pytest
import torch

from harness import OracleRank, assert_bitwise, to_host
from oracle import oracle as orc
from synth import synth

pytestmark = pytest.mark.gpu

HP = dict(lr=3e-5, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, max_grad_norm=1.0)


@pytest.fixture(scope="module")
def zf():
    import fsdp_sharded_mixed_flatparameter_amd as m
    assert torch.cuda.is_available()
    return m


def say(*a):
    print(*a, flush=True)


def test_empty_inputs_everywhere(zf):
    say("empty inputs")
    dev = "cuda"
    st = zf.StepState(1024.0, True, window=2)
    sentinel = torch.full((8,), 7.0, device=dev)
    g16 = torch.zeros(0, dtype=torch.float16, device=dev)
    zf.zero_grad_reduce_shard([g16, g16], 0, 0, zf.ZERO_AVG, sentinel, st)
    zf.zero_grad_accumulate_shard([g16, g16], 0, 0, zf.ZERO_AVG, sentinel, st)
    zf.zero_unscale_norm(g16, st)
    q = torch.zeros(0, dtype=torch.int8, device=dev)
    s = torch.zeros(0, device=dev)
    zf.zero_grad_reduce_shard_int8([q, q], [s, s], 0, zf.ZERO_SUM, sentinel, st)
    zf.zero_dequant_allgather(q, s, 4, 0, torch.zeros(0, dtype=torch.bfloat16, device=dev))
    empty = torch.zeros(0, device=dev)
    ag = torch.full((8,), 3.0, dtype=torch.float16, device=dev)
    zf.zero_adamw_shard_step(g16, empty, empty, empty, ag, 0, HP, st, finalize=True)
    zf.zero_quant_allgather_slot(torch.zeros(0, dtype=torch.float16, device=dev), q, s)
    torch.cuda.synchronize()
    assert torch.equal(sentinel, torch.full((8,), 7.0, device=dev))
    assert torch.equal(ag, torch.full((8,), 3.0, dtype=torch.float16, device=dev))
    r = st.read()
    # one finalize without overflow: one applied step, one good step, sums reset
    assert (r.step, r.good_steps, r.overflow, r.sumsq, r.last_skipped) == (1, 1, 0, 0.0, 0)
    assert r.loss_scale == 1024.0
    host = torch.zeros(0)
    stage = torch.zeros(8, dtype=torch.float16).pin_memory()
    zf.zero_offload_step(g16, host, host, host, stage, stage.clone().pin_memory(), ag, 0, HP, st)
    r = st.read()
    assert (r.step, r.good_steps, r.loss_scale) == (2, 0, 2048.0)   # window 2: doubled


def samples(S, extra=()):
    idx = []
    for c in (0, 1 << 31, 1 << 32) + tuple(extra):
        idx.append(np.arange(max(0, c - 600), min(S, c + 600)))
    idx.append(np.arange(S - 1200, S))
    idx.append(np.random.default_rng(3).integers(0, S, 5000))
    return np.unique(np.concatenate(idx)).astype(np.int64)


def test_shard_past_2_pow_32(zf):
    """S = 2^32 + 261 (a ragged tail): statistics, AdamW with bf16 write-back and
    INT8 blocks, then the 2-rank reduce and the dequantisation of the written
    slot, each sampled around 2^31, 2^32 and the end."""
    S = (1 << 32) + 261
    nb = -(-S // 256)
    dev = torch.device("cuda:0")
    say("shard", S)
    key_m, key_g = synth.stream_key("edge", "master"), synth.stream_key("edge", "grad")
    master = torch.empty(S, device=dev)
    synth.fill_normal(master, key_m, 0, 0.02)
    opt = zf.ShardOptimizer(master, HP, loss_scale=1.0, quant_block=256)
    g = torch.empty(S, dtype=torch.bfloat16, device=dev)
    synth.fill_normal(g, key_g, 0, 1e-3)
    slot = torch.zeros(S, dtype=torch.bfloat16, device=dev)
    q = torch.zeros(S, dtype=torch.int8, device=dev)
    qs = torch.zeros(nb, device=dev)
    opt.step_from_reduced(g, slot, 0, q_buf=q, q_scales=qs)
    st = opt.state.read()
    sumsq = sum(torch.sum(torch.square(g[i:i + (1 << 27)].double())).item()
                for i in range(0, S, 1 << 27))
    assert abs(st.last_norm - sumsq ** 0.5) <= 1e-5 * sumsq ** 0.5
    blocks = np.unique(np.concatenate([samples(S) // 256]))
    idx = np.concatenate([np.arange(b * 256, min((b + 1) * 256, S)) for b in blocks]).astype(np.int64)
    ref = OracleRank(synth.normal_f32_at(key_m, idx, 0.02), 1.0, False)
    gs = synth.normal_at(key_g, idx, 1e-3, orc.BF16)
    # the global norm enters through coef; take the device's sum (checked at full
    # size elsewhere) so that the sampled elements see the same coefficient
    res = ref.step(gs, orc.BF16, HP, orc.BF16, sumsq_local=st.last_norm ** 2, overflow_local=0)
    assert st.last_coef == res["coef"]
    gi = torch.from_numpy(idx).to(dev)
    assert_bitwise(to_host(opt.master[gi]), ref.p, "master")
    assert_bitwise(to_host(opt.exp_avg[gi]), ref.m, "exp_avg")
    assert_bitwise(to_host(opt.exp_avg_sq[gi]), ref.v, "exp_avg_sq")
    assert_bitwise(to_host(slot[gi]), res["lp"], "bf16 slot")
    pos = 0
    for b in blocks:
        n_b = min((b + 1) * 256, S) - b * 256
        rq, rsc = orc.quant_int8(np.ascontiguousarray(res["lp"][pos:pos + n_b]), orc.BF16, 256)
        assert_bitwise(to_host(q[b * 256:b * 256 + n_b]).view(np.uint8), rq.view(np.uint8),
                       "int8 block %d" % b)
        assert to_host(qs[int(b):int(b) + 1])[0] == rsc[0]
        pos += n_b
    del opt, g, master
    torch.cuda.empty_cache()
    # the consumer over the whole > 2^32 slot
    out = torch.empty(S, dtype=torch.bfloat16, device=dev)
    zf.zero_dequant_allgather(q, qs, 1, S, out)
    qh = to_host(q[gi])
    sh = to_host(qs[torch.from_numpy(idx // 256).to(dev)])
    assert_bitwise(to_host(out[gi]), orc.dequant_int8(qh, sh, idx.size, 1, 1, orc.BF16),
                   "dequantised slot")
    del out, q, qs, slot
    torch.cuda.empty_cache()
    # a 2-rank fp16 reduce over the same length
    key_r = [synth.stream_key("edge", "rank", k) for k in range(2)]
    bufs = []
    for k in range(2):
        b = torch.empty(S, dtype=torch.float16, device=dev)
        synth.fill_normal(b, key_r[k], 0, 1e-3)
        bufs.append(b)
    red = torch.empty(S, device=dev)
    zf.zero_grad_reduce_shard(bufs, 0, S, zf.ZERO_AVG, red)
    hb = [synth.normal_at(key_r[k], idx, 1e-3, orc.F16) for k in range(2)]
    assert_bitwise(to_host(red[gi]), orc.reduce(hb, orc.F16, 0, idx.size, orc.AVG), "reduce")
    del bufs, red
    torch.cuda.empty_cache()
