"""GPU parity of a reduce that takes several launches: a reduce of 16-bit
slices is issued as launches of at most 32,768 blocks (4 tiles of 1,024
elements each for eight slices) over consecutive tile ranges, and with the
step statistics each later launch adds its block sums onto the partials the
first one wrote.  Shards of 2^28 elements and more take three launches or
more.  The whole reduced shard is compared with the oracle bit for
bit (ZeRO's Reduce-Scatter, "PyTorch FSDP 源码级深度解析" §3.3: every element
of the rank's slice is the rank-order reduce), the sum of squares within
n * 2^-53 relative; the no-allocation entry point must give the same bits.

Inputs: the GPU fills the slices with the device copy of the seeded
generator; the oracle reduces host copies of exactly those slices, which are
checked against the host generator at sampled indices.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

from harness import assert_bitwise, to_host
from oracle import oracle as orc
from synth import synth

pytestmark = pytest.mark.gpu

THREADS = min(16, os.cpu_count() or 4)
CHUNK = 1 << 22
TDT = {orc.F16: torch.float16, orc.BF16: torch.bfloat16}


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def zf():
    import fsdp_sharded_mixed_flatparameter_amd as m
    assert torch.cuda.is_available()
    return m


def rel(a, b):
    return abs(a - b) / max(abs(b), 1e-300)


# (dtype, op, shard elements, slice offset, accumulate): more than twice
# 32768 blocks x 4 tiles x 1024 elements (2^27), so three launches or more
CASES = [
    (orc.F16, 1, (1 << 28) + 5_000, 0, False),
    (orc.F16, 1, (1 << 28) + 1_000_003, 1, False),    # slices one element into a line
    (orc.BF16, 0, 3 * (1 << 28) + 77, 3, False),       # six launches and the tail, SUM
    (orc.F16, 1, (1 << 28) + 4099, 2, True),           # accumulation with statistics
]


@pytest.mark.parametrize("dt,op,n,off,acc", CASES)
def test_reduce_over_several_launches(zf, dt, op, n, off, acc):
    N = 8
    say("multi-launch reduce", dt, op, n, off, acc)
    dev = torch.device("cuda:0")
    keys = [synth.stream_key("multi", dt, n, k) for k in range(N)]
    bufs = []
    for k in range(N):
        b = torch.empty(off + n, dtype=TDT[dt], device=dev)
        synth.fill_normal(b, keys[k], 0, 1e-3 * (1 + k % 3))
        bufs.append(b)
    acc0 = None
    if acc:
        acc0 = torch.empty(n, device=dev)
        synth.fill_normal(acc0, synth.stream_key("multi-acc", n), 0, 1e-3)
    scale = 1024.0

    def run(noalloc):
        out = acc0.clone() if acc else torch.full((n,), float("nan"), device=dev)
        if noalloc:   # a state of only the header
            H = zf.STATE_HEADER_BYTES
            raw = bytes(bytearray(zf.zero_step_state_init(scale, 0, 1000, 1.0)))[:H]
            st = torch.frombuffer(bytearray(raw), dtype=torch.uint8).to(dev)
            zf.zero_grad_reduce_shard_noalloc(bufs, off, n, op, out, st)
            back = st.cpu().numpy().tobytes()
            return out, zf.zero_step_state_t.from_buffer_copy(back + bytes(zf.STATE_BYTES - H))
        state = zf.StepState(scale, False)
        if acc:
            zf.zero_grad_accumulate_shard(bufs, off, n, op, out, state)
        else:
            zf.zero_grad_reduce_shard(bufs, off, n, op, out, state)
        return out, state.read()

    out, st = run(False)
    say("  reduced; host copies")
    host = []
    rng = np.random.default_rng(n)
    idx = np.unique(np.concatenate([rng.integers(0, off + n, 20_000), [0, off, off + n - 1]]))
    for k in range(N):
        h = to_host(bufs[k]).copy()
        want = synth.normal_at(keys[k], idx, 1e-3 * (1 + k % 3), dt)
        assert_bitwise(h[idx], want, "slice %d copy" % k)
        host.append(h)
    acc_h = to_host(acc0).copy() if acc else None
    got = to_host(out)

    def job(lo):
        m = min(CHUNK, n - lo)
        parts = [h[off + lo:off + lo + m] for h in host]
        if acc:
            ref = acc_h[lo:lo + m].copy()
            orc.reduce_accumulate(parts, dt, 0, m, op, ref)
        else:
            ref = orc.reduce(parts, dt, 0, m, op)
        assert_bitwise(got[lo:lo + m], ref, "reduced shard at %d" % lo)
        return orc.unscale_stats(ref, orc.F32, scale)

    with ThreadPoolExecutor(THREADS) as ex:
        parts = list(ex.map(job, range(0, n, CHUNK)))
    s_ref = sum(p[0] for p in parts)
    assert st.overflow == 0 and not any(p[1] for p in parts)
    assert rel(st.sumsq, s_ref) <= n * 2.0 ** -53, (st.sumsq, s_ref)
    say("  sumsq", st.sumsq, "oracle", s_ref, "partials", st.n_partials)
    assert st.n_partials == 32768          # the first launch's full grid
    if not acc:
        out2, st2 = run(True)
        assert_bitwise(to_host(out2), got, "no-allocation reduce")
        assert st2.sumsq == st.sumsq and st2.overflow == 0
        del out2
    del bufs, out, host, acc0
    torch.cuda.empty_cache()
