"""Several FlatParameters (FSDP units) under one optimizer, through
MultiShardOptimizer and the C ABI: the statistics of every unit go into one
step state, then each unit's AdamW runs with the finalize only on the last.
The oracle is one shard step over the concatenation of the units' reduced
shards: the update is elementwise given the step's scalars, so the two agree
exactly when the norm, the clip coefficient, the skip and the loss scale are
global over the units.

Pages: "DeepSpeed 与 FSDP", FlatParameter section (one FlatParameter per
wrapped unit); 2kiu.com §5.1 (gradient_clipping over the model) and §5.3
(overflow and clipping agree everywhere).
"""
import numpy as np
import pytest
import torch

from harness import OracleRank, assert_bitwise, to_dev, to_host
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


@pytest.mark.parametrize("rank", [1, 3])
def test_units_share_norm_skip_and_scaler(zf, rank):
    """The 2-layer MLP wrapped as two units, (W1, b1) and (W2, b2), plus a
    third one-element unit, over 4 ranks.  Four steps with a dynamic scale
    (window 2): step 1 doubles the scale; step 2 carries an inf in the second
    unit only, and every unit skips; step 3 adds a remote sum of squares so
    that the global clip coefficient is below 1 for every unit."""
    N = 4
    units = [512 * 1024 + 1024, 1024 * 512 + 512, 1]
    S = [zf.zero_flat_layout([t], N)["shard"] for t in units]
    say("multi-unit rank", rank, "shards", S)
    masters0 = [synth.normal_f32(synth.stream_key("mu-master", u), rank * s, s, 0.02)
                for u, s in enumerate(S)]
    opt = zf.MultiShardOptimizer([to_dev(m0, 0) for m0 in masters0], HP, loss_scale=65536.0,
                                 dynamic=True, window=2)
    ref = OracleRank(np.concatenate(masters0), 65536.0, True, window=2)
    ags = [torch.zeros(N * s, dtype=torch.float16, device="cuda") for s in S]
    cuts = np.cumsum(S)[:-1]
    for step in range(4):
        bufs = [[synth.normal(synth.stream_key("mu-grad", u, step, k), 0, N * s, 1e-3, orc.F16)
                 for k in range(N)] for u, s in enumerate(S)]
        if step == 2:
            bufs[1][2][rank * S[1] + 77] = 0x7C00             # +inf in unit 1 only
        remote = 4.0 if step == 3 else 0.0
        if step == 3:
            opt.state.set_remote(sumsq=remote)
        before = [m.clone() for m in opt.master]
        opt.step_from_rank_buffers([[to_dev(b, orc.F16) for b in bu] for bu in bufs],
                                   [rank * s for s in S], ags, [rank * s for s in S])
        reds = [orc.reduce(bufs[u], orc.F16, rank * s, s, orc.AVG) for u, s in enumerate(S)]
        res = ref.step(np.concatenate(reds), orc.F32, HP, orc.F16, remote_sumsq=remote)
        st = opt.state.read()
        assert st.last_skipped == res["skipped"] == int(step == 2)
        assert (st.loss_scale, st.good_steps, st.step) == \
            (ref.scaler.loss_scale, ref.scaler.good_steps, ref.scaler.step)
        if step == 2:                                         # the inf makes both norms inf
            assert not np.isfinite(st.last_norm) and not np.isfinite(res["norm"])
            for m, b in zip(opt.master, before):
                assert torch.equal(m, b)
            continue
        # the sums of squares of the units and the oracle's one sum: same terms,
        # different order, each within n * 2^-53 relative of the exact sum
        assert abs(st.last_norm - res["norm"]) <= sum(S) * 2.0 ** -53 * res["norm"]
        assert st.last_coef == res["coef"]
        if step == 3:
            assert res["coef"] < 1.0
        for u, (p, mm, vv, lp) in enumerate(zip(np.split(ref.p, cuts), np.split(ref.m, cuts),
                                                np.split(ref.v, cuts), np.split(res["lp"], cuts))):
            assert_bitwise(to_host(opt.master[u]), p, "unit %d master step %d" % (u, step))
            assert_bitwise(to_host(opt.exp_avg[u]), mm, "unit %d exp_avg step %d" % (u, step))
            assert_bitwise(to_host(opt.exp_avg_sq[u]), vv, "unit %d exp_avg_sq step %d" % (u, step))
            assert_bitwise(to_host(ags[u][rank * S[u]:(rank + 1) * S[u]]), lp,
                           "unit %d slot step %d" % (u, step))
    for u, s in enumerate(S):
        assert not ags[u][:rank * s].any() and not ags[u][(rank + 1) * s:].any()


def test_unit_lists_must_match(zf):
    opt = zf.MultiShardOptimizer([torch.zeros(8, device="cuda"), torch.zeros(4, device="cuda")],
                                 HP)
    with pytest.raises(ValueError):
        opt.step_from_reduced([torch.zeros(8, device="cuda")], [None], [0])


def test_units_accumulate_micro_steps(zf):
    """Two units, two optimizer steps of three micro-steps each (the first
    reduces, the others add into each unit's fp32 gradient shard, the last
    takes the statistics of both); against the oracle's reduce and
    accumulate per unit and one shard step over the concatenation."""
    N, rank = 8, 5
    units = [100_003, 40_000]
    S = [zf.zero_flat_layout([t], N)["shard"] for t in units]
    masters0 = [synth.normal_f32(synth.stream_key("mu-acc-master", u), rank * s, s, 0.02)
                for u, s in enumerate(S)]
    opt = zf.MultiShardOptimizer([to_dev(m0, 0) for m0 in masters0], HP, loss_scale=1024.0)
    ref = OracleRank(np.concatenate(masters0), 1024.0, False)
    ags = [torch.zeros(N * s, dtype=torch.bfloat16, device="cuda") for s in S]
    cuts = np.cumsum(S)[:-1]
    with pytest.raises(RuntimeError):
        opt.step_from_accumulated(ags, [rank * s for s in S])
    for step in range(2):
        accs = [np.zeros(s, np.float32) for s in S]
        for micro in range(3):
            bufs = [[synth.normal(synth.stream_key("mu-acc-grad", u, step, micro, k), 0, N * s,
                                  1e-3, orc.BF16) for k in range(N)] for u, s in enumerate(S)]
            opt.micro_step([[to_dev(b, orc.BF16) for b in bu] for bu in bufs],
                           [rank * s for s in S], first=micro == 0, last=micro == 2)
            for u, s in enumerate(S):
                if micro == 0:
                    accs[u] = orc.reduce(bufs[u], orc.BF16, rank * s, s, orc.AVG)
                else:
                    orc.reduce_accumulate(bufs[u], orc.BF16, rank * s, s, orc.AVG, accs[u])
        for u in range(len(S)):
            assert_bitwise(to_host(opt._red[u]), accs[u], "unit %d accumulated step %d" % (u, step))
        opt.step_from_accumulated(ags, [rank * s for s in S])
        res = ref.step(np.concatenate(accs), orc.F32, HP, orc.BF16)
        st = opt.state.read()
        assert st.last_skipped == 0 and st.step == step + 1
        assert abs(st.last_norm - res["norm"]) <= sum(S) * 2.0 ** -53 * res["norm"]
        assert st.last_coef == res["coef"]
        for u, (p, lp) in enumerate(zip(np.split(ref.p, cuts), np.split(res["lp"], cuts))):
            assert_bitwise(to_host(opt.master[u]), p, "unit %d master step %d" % (u, step))
            assert_bitwise(to_host(ags[u][rank * S[u]:(rank + 1) * S[u]]), lp,
                           "unit %d slot step %d" % (u, step))


def test_units_int8_payloads(zf):
    """Pre-reduced bf16 gradients of three units, two steps, the first two
    units also emitting their blockwise-INT8 All-Gather payload (blocks of 256
    restarting at each unit's slot), the third none: codes and scales equal
    the oracle's quantisation of each unit's written slot."""
    N, rank = 64, 63
    units = [1_000_003, 77_777, 4_096]
    S = [zf.zero_flat_layout([t], N)["shard"] for t in units]
    nb = [-(-s // 256) for s in S]
    masters0 = [synth.normal_f32(synth.stream_key("mu-q-master", u), rank * s, s, 0.02)
                for u, s in enumerate(S)]
    opt = zf.MultiShardOptimizer([to_dev(m0, 0) for m0 in masters0], HP, loss_scale=1.0)
    ref = OracleRank(np.concatenate(masters0), 1.0, False)
    ags = [torch.zeros(N * s, dtype=torch.bfloat16, device="cuda") for s in S]
    qs = [torch.zeros(N * s, dtype=torch.int8, device="cuda") for s in S[:2]]
    scs = [torch.zeros(N * b, device="cuda") for b in nb[:2]]
    quant = [(qs[0], scs[0], rank * S[0], rank * nb[0]), (qs[1], scs[1], rank * S[1], rank * nb[1]),
             None]
    cuts = np.cumsum(S)[:-1]
    for step in range(2):
        gs = [synth.normal(synth.stream_key("mu-q-grad", u, step), rank * s, s, 1e-3, orc.BF16)
              for u, s in enumerate(S)]
        opt.step_from_reduced([to_dev(g, orc.BF16) for g in gs], ags, [rank * s for s in S],
                              quant=quant)
        res = ref.step(np.concatenate([orc.bf16_to_f32(g) for g in gs]), orc.F32, HP, orc.BF16)
        st = opt.state.read()
        assert st.last_coef == res["coef"] and st.last_skipped == 0
        for u, lp in enumerate(np.split(res["lp"], cuts)):
            got = to_host(ags[u][rank * S[u]:(rank + 1) * S[u]])
            assert_bitwise(got, lp, "unit %d slot step %d" % (u, step))
            if u < 2:
                rq, rs = orc.quant_int8(lp, orc.BF16, 256)
                assert_bitwise(to_host(qs[u][rank * S[u]:]).view(np.uint8), rq.view(np.uint8),
                               "unit %d codes step %d" % (u, step))
                assert_bitwise(to_host(scs[u][rank * nb[u]:]), rs, "unit %d scales step %d" % (u, step))
                assert not qs[u][:rank * S[u]].any() and not scs[u][:rank * nb[u]].any()
