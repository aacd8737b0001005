"""Reduce parity at sizes where every wave runs the pipelined loop, whole
outputs compared element by element with the oracle (not samples).  A
reduce of 16-bit or fp32 buffers gives each wave one tile, whose steps (one
buffer group each) the loop pipelines; INT8 payloads and the statistics
pass give each wave a run of R tiles (about 16 steps, fewer when the shard
is small).  Per case:

  8 fp16 buffers, 60,500,123 elements   one step of four chunks per wave
  32 bf16 buffers, 10,000,257           two groups of 16 (2 steps)
  12 fp16 buffers, 20,000,263, 2 micro-steps accumulated
                                        three groups of 4 (3 steps)
  8 INT8 payloads, 45,200,000           one group, R = 5
  4 fp16 buffers, 135,000,000           65,918 blocks: three launches,
                                        the later two adding onto the
                                        first's 32,768 partial sums
  2 fp32 buffers, 53,000,003            one group of two
  statistics pass, 80,000,001 fp16      one buffer, R = 9

and in each the last wave's work is cut short by the end of the full tiles,
followed by the ragged tail.  Bar: the reduced (or accumulated) shard bit for
bit; the overflow flag exact; the sum of squares within n * 2^-53 relative:
the oracle adds the n non-negative terms one after another in binary64, which
bounds its own relative error by (n - 1) * 2^-53, and the device adds them in
another order (the norm's tolerance, 1e-5, is far above either)."""
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


def inputs(tag, dt, N, total):
    return [synth.normal(synth.stream_key("runs", tag, k), 0, total, 1e-3 * (1 + k % 3), dt,
                         threads=8) for k in range(N)]


def sum_bound(n):
    return max(1e-12, n * 2.0 ** -53)


def check_stats(state, red, scale):
    s_ref, o_ref = orc.unscale_stats(red, orc.F32, scale)
    st = state.read()
    assert st.overflow == o_ref == 0
    assert rel(st.sumsq, s_ref) <= sum_bound(red.size)


@pytest.mark.parametrize("dt,N,op,S,off", [
    (1, 8, 1, 60_500_123, 8), (2, 32, 0, 10_000_257, 0), (1, 4, 1, 135_000_000, 0),
    (0, 2, 0, 53_000_003, 4)])
def test_reduce_runs_whole_output(zf, dt, N, op, S, off):
    say("reduce runs", dt, N, op, S, off)
    bufs = inputs("red-%d-%d" % (dt, N), dt, N, off + S + 3)
    red_d = torch.full((S,), float("nan"), device="cuda")
    state = zf.StepState(65536.0, False)
    zf.zero_grad_reduce_shard([to_dev(b, dt) for b in bufs], off, S, op, red_d, state)
    red = orc.reduce(bufs, dt, off, S, op)
    assert_bitwise(to_host(red_d), red, "reduced shard")
    check_stats(state, red, 65536.0)


def test_accumulate_runs_whole_output(zf):
    dt, N, op, S, off = 1, 12, 1, 20_000_263, 12
    say("accumulate runs", dt, N, op, S, off)
    acc_d = torch.zeros(S, device="cuda")
    acc = np.zeros(S, np.float32)
    state = zf.StepState(1024.0, False)
    for k in range(2):
        bufs = inputs("acc-%d" % k, dt, N, off + S + 1)
        zf.zero_grad_accumulate_shard([to_dev(b, dt) for b in bufs], off, S, op, acc_d,
                                      state if k == 1 else None)
        orc.reduce_accumulate(bufs, dt, off, S, op, acc)
        assert_bitwise(to_host(acc_d), acc, "accumulated shard after micro-step %d" % k)
    check_stats(state, acc, 1024.0)


def test_int8_reduce_runs_whole_output(zf):
    N, S, block, op = 8, 45_200_000, 256, 1
    say("int8 reduce runs", N, S)
    nb = -(-S // block)
    qs = [synth.codes(synth.stream_key("runs", "q", k), 0, S) for k in range(N)]
    scs = [np.abs(synth.normal_f32(synth.stream_key("runs", "s", k), 0, nb, 4.7e-6))
           .astype(np.float32) for k in range(N)]
    red_d = torch.full((S,), float("nan"), device="cuda")
    state = zf.StepState(65536.0, False)
    zf.zero_grad_reduce_shard_int8([torch.from_numpy(q).cuda() for q in qs],
                                   [to_dev(sc, 0) for sc in scs], S, op, red_d, state,
                                   block=block)
    red = orc.reduce_q8(qs, scs, S, block, op)
    assert_bitwise(to_host(red_d), red, "reduced shard")
    check_stats(state, red, 65536.0)


def test_statistics_pass_runs(zf):
    dt, S = 1, 80_000_001
    say("statistics runs", S)
    g = inputs("stats", dt, 1, S)[0]
    state = zf.StepState(65536.0, False)
    zf.zero_unscale_norm(to_dev(g, dt), state)
    s_ref, o_ref = orc.unscale_stats(g, dt, 65536.0)
    st = state.read()
    assert st.overflow == o_ref == 0
    assert rel(st.sumsq, s_ref) <= sum_bound(S)
