"""The no-allocation reduce entry point, zero_grad_reduce_shard_noalloc, for
callers that cannot allocate: called through the C ABI and compared with
zero_grad_reduce_shard on the same seeded inputs, bit for bit (the reduced
shard, the overflow flag, the fold's sum of squares and the partial count).

Two calls run back to back on one device, the second over a smaller shard,
so the second reuses the scratch the first left behind.  The caller's state
for the new entry point holds only the header of zero_step_state_t followed
by a canary region where the partials table would begin: the canary must
come back untouched."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

CANARY = 4096


@pytest.fixture(scope="module")
def env():
    import torch

    import fsdp_sharded_mixed_flatparameter_amd as zf
    from synth import synth
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    return zf, synth, torch


def _header_state(zf, torch, host_state):
    raw = bytes(bytearray(host_state))[:zf.STATE_HEADER_BYTES]
    buf = torch.full((zf.STATE_HEADER_BYTES + CANARY,), 0xA5, dtype=torch.uint8, device="cuda")
    buf[:zf.STATE_HEADER_BYTES].copy_(torch.frombuffer(bytearray(raw), dtype=torch.uint8))
    return buf


def _header_of(zf, raw):
    return zf.zero_step_state_t.from_buffer_copy(
        raw[:zf.STATE_HEADER_BYTES] + bytes(zf.STATE_BYTES - zf.STATE_HEADER_BYTES))


def _buffers(synth, torch, dtype, n_ranks, length, tag):
    bufs = []
    for k in range(n_ranks):
        b = torch.empty(length, dtype=dtype, device="cuda")
        synth.fill_normal(b, synth.stream_key("noalloc", *tag, k), 0, 1e-3)
        bufs.append(b)
    return bufs


# (format, ranks, op, first shard, offset of the first, second shard, inject inf)
CASES = [
    ("bfloat16", 8, "avg", 25_297_920, 3 * 25_297_920, 70_001, False),   # the 7B block's rank-3 slice
    ("float16", 3, "sum", 5_000_003, 12_345, 4_099, True),
    ("float32", 16, "avg", 1_048_577, 0, 257, False),
]


@pytest.mark.parametrize("dt,n_ranks,op,n1,off1,n2,inject", CASES)
def test_noalloc_reduce_matches_reduce(env, dt, n_ranks, op, n1, off1, n2, inject):
    zf, synth, torch = env
    dtype = getattr(torch, dt)
    opc = zf.ZERO_AVG if op == "avg" else zf.ZERO_SUM
    bufs = _buffers(synth, torch, dtype, n_ranks, off1 + n1, (dt, n_ranks, n1, op))
    if inject:
        bufs[n_ranks - 1][off1 + n1 // 2] = float("inf")
    host = zf.zero_step_state_init(65536.0, 1, 1000, 1.0)
    print("noalloc case", dt, n_ranks, op, n1, off1, n2, flush=True)
    for call, (n, off) in enumerate(((n1, off1), (n2, 0))):
        ref_state = zf.StepState(65536.0, True)
        ref_state.upload(host)
        new_state = _header_state(zf, torch, host)
        ref_out = torch.full((n,), float("nan"), device="cuda")
        new_out = torch.full((n,), float("nan"), device="cuda")
        zf.zero_grad_reduce_shard(bufs, off, n, opc, ref_out, ref_state)
        zf.zero_grad_reduce_shard_noalloc(bufs, off, n, opc, new_out, new_state)
        # without statistics the scratch is not used at all
        plain = torch.full((n,), float("nan"), device="cuda")
        zf.zero_grad_reduce_shard_noalloc(bufs, off, n, opc, plain, None)
        torch.cuda.synchronize()
        a = ref_out.cpu().numpy().view(np.uint32)
        assert np.array_equal(a, new_out.cpu().numpy().view(np.uint32)), ("reduced shard", call)
        assert np.array_equal(a, plain.cpu().numpy().view(np.uint32)), ("reduced shard", call)
        raw = new_state.cpu().numpy().tobytes()
        assert raw[zf.STATE_HEADER_BYTES:] == b"\xa5" * CANARY, "wrote past the state's header"
        got, want = _header_of(zf, raw), ref_state.read()
        assert got.n_partials == want.n_partials and got.n_partials > 0
        assert np.float64(got.sumsq).view(np.uint64) == np.float64(want.sumsq).view(np.uint64)
        assert got.overflow == want.overflow == int(inject and call == 0)
        for f in ("loss_scale", "step", "good_steps", "remote_sumsq", "remote_overflow"):
            assert getattr(got, f) == getattr(want, f), f
