"""GPU parity when rank slices and slots do not start on a vector boundary
("PyTorch FSDP 源码级深度解析" §3.3: rank r's slice of the flat buffer starts
at r*S, and S need not be a multiple of anything): the reduce over slices
that all start 1, 2 or 3 elements past a quad boundary (its shifted vector
path: the head element-wise, aligned quads shifted across lanes onto the
aligned output, tile edges element-wise), the statistics pass over such a
shard, and the AdamW step writing a slot and INT8 codes at odd offsets.
Compared with the oracle on the same seeded inputs: bit-exact outputs and
flags, the sum of squares within n * 2^-53 relative."""
import numpy as np
import pytest
import torch

from harness import assert_bitwise, to_dev, to_host
from oracle import oracle as orc
from synth import synth

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


SHIFT_CASES = [
    # (dtype, n_ranks, op, shard, elem_offset (mod 4 != 0), accumulate)
    (1, 8, 1, 3 * 512 * 16 + 7, 1, False),   # several tiles per wave, ragged end
    (1, 8, 1, 1_000_003, 3, True),
    (1, 8, 0, 2_000_000, 2, False),
    (2, 8, 0, 777_777, 2, False),
    (2, 8, 1, 262_528, 7, True),
    (0, 4, 1, 100_003, 1, True),
    (0, 16, 1, 50_001, 3, False),
    (0, 2, 0, 4099, 2, False),
    (1, 64, 1, 20_001, 1, False),
    (1, 16, 1, 33_333, 5, True),
    (2, 3, 1, 4097, 1, False),                # odd rank count (one chunk, eight per tile)
    (2, 1, 1, 1025, 2, False),                # one buffer
    (1, 2, 0, 2, 1, False),                   # shorter than the head
    (1, 2, 0, 3, 1, False),                   # exactly the head
    (1, 8, 1, 5, 3, True),
    (1, 8, 1, 515, 1, False),                 # one tile plus the head
]


@pytest.mark.parametrize("dt,n_ranks,op,shard,off,acc", SHIFT_CASES)
def test_reduce_shifted_slices(zf, dt, n_ranks, op, shard, off, acc):
    say("shifted reduce", dt, n_ranks, op, shard, off, acc)
    total = off + shard + 3
    bufs = [synth.normal(synth.stream_key("shift", dt, k, shard, off), 0, total,
                         1e-3 * (1 + k % 3), dt) for k in range(n_ranks)]
    dbufs = [to_dev(b, dt) for b in bufs]
    state = zf.StepState(1024.0, False)
    if acc:
        acc0 = synth.normal_f32(synth.stream_key("shift-acc", shard), 0, shard, 1e-3)
        out = to_dev(acc0, 0)
        zf.zero_grad_accumulate_shard(dbufs, off, shard, op, out, state)
        ref = acc0.copy()
        orc.reduce_accumulate(bufs, dt, off, shard, op, ref)
    else:
        out = torch.full((shard,), float("nan"), device="cuda")
        zf.zero_grad_reduce_shard(dbufs, off, shard, op, out, state)
        ref = orc.reduce(bufs, dt, off, shard, op)
    assert_bitwise(to_host(out), ref, "reduced shard")
    s_ref, o_ref = orc.unscale_stats(ref, orc.F32, 1024.0)
    st = state.read()
    assert st.overflow == o_ref == 0
    assert rel(st.sumsq, s_ref) <= max(1e-12, shard * 2.0 ** -53)


@pytest.mark.parametrize("where", ["head", "body", "edge", "tail"])
def test_reduce_shifted_overflow(zf, where):
    """An inf in the head, the vector body, a tile edge or the tail of a
    shifted slice reaches the overflow flag."""
    dt, N, S, off = 1, 8, 3 * 512 * 8 + 11, 3
    bufs = [synth.normal(synth.stream_key("shift-ovf", k), 0, off + S, 1e-3, dt) for k in range(N)]
    pos = {"head": 0, "body": 1000, "edge": 512, "tail": S - 2}[where]
    bufs[5][off + pos] = np.float16(np.inf).view(np.uint16)
    state = zf.StepState(65536.0, True)
    out = torch.empty(S, device="cuda")
    zf.zero_grad_reduce_shard([to_dev(b, dt) for b in bufs], off, S, zf.ZERO_AVG, out, state)
    assert state.read().overflow == 1


@pytest.mark.parametrize("dt,n,start", [(1, 100_003, 1), (2, 65_537, 3), (0, 40_001, 2),
                                        (1, 2, 1), (0, 513, 3)])
def test_unscale_norm_shifted(zf, dt, n, start):
    g = synth.normal(synth.stream_key("shift-un", dt, n), 0, n, 1e-3, dt)
    gd = to_dev(np.concatenate([np.zeros(start, g.dtype), g]), dt)[start:]
    state = zf.StepState(256.0, False)
    zf.zero_unscale_norm(gd, state)
    s, o = orc.unscale_stats(g, dt, 256.0)
    st = state.read()
    assert st.overflow == o and rel(st.sumsq, s) <= max(1e-12, n * 2.0 ** -53)


@pytest.mark.parametrize("pdt,n,slot,q_off", [(1, 262_528, 1, 3), (2, 1_000_003, 3, 1),
                                              (1, 65_536, 2, 2), (2, 4097, 7, 5)])
def test_adamw_slot_at_odd_offsets(zf, pdt, n, slot, q_off):
    """The update's vector path writes a slot (and INT8 codes) that starts at
    any element: bit-exact against the oracle over two steps, the buffer
    around the slot untouched."""
    say("adamw odd slot", pdt, n, slot, q_off)
    hp = dict(lr=3e-5, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, max_grad_norm=1.0)
    p0 = synth.normal_f32(synth.stream_key("odd-p", n), 0, n, 0.02)
    opt = zf.ShardOptimizer(to_dev(p0, 0), hp, loss_scale=1.0, dynamic=False, quant_block=256)
    tdt = {1: torch.float16, 2: torch.bfloat16}[pdt]
    ag = torch.zeros(slot + n + 9, dtype=tdt, device="cuda")
    nb = -(-n // 256)
    q = torch.zeros(q_off + n + 9, dtype=torch.int8, device="cuda")
    qs = torch.zeros(nb, device="cuda")
    p, m, v = p0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    sc = orc.make_scaler(1.0, False)
    for step in range(2):
        g = synth.normal(synth.stream_key("odd-g", n, step), 0, n, 1e-3, pdt)
        opt.step_from_reduced(to_dev(g, pdt), ag, slot, q_buf=q, q_scales=qs, q_slot_offset=q_off)
        res = orc.shard_step(grad=g, grad_dtype=pdt, master=p, exp_avg=m, exp_avg_sq=v, scaler=sc,
                             hp=orc.Hparams(**hp), param_dtype=pdt, quant_block=256)
        assert_bitwise(to_host(opt.master), p, "master step %d" % step)
        assert_bitwise(to_host(opt.exp_avg), m, "exp_avg step %d" % step)
        assert_bitwise(to_host(opt.exp_avg_sq), v, "exp_avg_sq step %d" % step)
        agh = to_host(ag)
        assert_bitwise(agh[slot:slot + n], res["lp"], "slot step %d" % step)
        assert not agh[:slot].any() and not agh[slot + n:].any()
        qh = to_host(q)
        assert_bitwise(qh[q_off:q_off + n].view(np.uint8), res["q"].view(np.uint8),
                       "INT8 codes step %d" % step)
        assert not qh[:q_off].any() and not qh[q_off + n:].any()
        assert_bitwise(to_host(qs), res["scales"], "INT8 scales step %d" % step)
