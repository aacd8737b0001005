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


@pytest.mark.parametrize("vector", [True, False])
def test_adamw_over_several_launches(zf, vector):
    """The fused AdamW step over 2 x 131,072 tiles + 777 elements: launches of
    32,768 blocks (4 tiles of 1,024 elements each) over consecutive tile
    ranges, three here.  With `vector` False the master shard starts 4 bytes
    past a 16-byte boundary, which sends every tile down the element-wise
    path, in the same launch ranges.  Two steps, every element of master, m,
    v and the fp16 slot against the oracle; clipping active."""
    n = 2 * 131072 * 1024 + 777
    say("adamw over launches", n, "vector" if vector else "element-wise")
    dev = torch.device("cuda:0")
    hp = dict(lr=3e-5, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, max_grad_norm=0.5)
    scale = 1024.0
    kp = synth.stream_key("multi-adam-p", n)
    base = torch.empty(n + (0 if vector else 1), device=dev)
    master = base if vector else base[1:]
    synth.fill_normal(master, kp, 0, 0.02)
    p = to_host(master).copy()
    opt = zf.ShardOptimizer(master, hp, loss_scale=scale, dynamic=False)
    assert (master.data_ptr() % 16 == 0) == vector
    ag = torch.zeros(n, dtype=torch.float16, device=dev)
    g = torch.empty(n, dtype=torch.float16, device=dev)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    hpo = orc.Hparams(**hp)
    for step in range(2):
        kg = synth.stream_key("multi-adam-g", n, step)
        synth.fill_normal(g, kg, 0, 1e-3 * scale)
        gh = to_host(g).copy()
        idx = np.unique(np.random.default_rng(step).integers(0, n, 5_000))
        assert_bitwise(gh[idx], synth.normal_at(kg, idx, 1e-3 * scale, orc.F16), "grad copy")
        opt.step_from_reduced(g, ag, 0)
        st = opt.state.read()

        def stats(lo):
            return orc.unscale_stats(np.ascontiguousarray(gh[lo:lo + CHUNK]), orc.F16, scale)

        with ThreadPoolExecutor(THREADS) as ex:
            sumsq = sum(s for s, _ in ex.map(stats, range(0, n, CHUNK)))
        coef = orc.clip_coef(sumsq, hp["max_grad_norm"])
        assert coef < 1.0 and st.last_coef == coef, (st.last_coef, coef)

        def job(lo):
            k = min(CHUNK, n - lo)
            pc, mc, vc = p[lo:lo + k], m[lo:lo + k], v[lo:lo + k]   # views: updated in place
            return lo, orc.adamw(np.ascontiguousarray(gh[lo:lo + k]), orc.F16, pc, mc, vc, scale,
                                 coef, step + 1, hpo, orc.F16)

        with ThreadPoolExecutor(THREADS) as ex:
            lps = dict(ex.map(job, range(0, n, CHUNK)))
        got_p, got_m, got_v, got_lp = (to_host(t) for t in (opt.master, opt.exp_avg,
                                                             opt.exp_avg_sq, ag))
        for lo, lp in lps.items():
            k = lp.size
            w = "step %d, chunk at %d" % (step, lo)
            assert_bitwise(got_p[lo:lo + k], p[lo:lo + k], "master, " + w)
            assert_bitwise(got_m[lo:lo + k], m[lo:lo + k], "exp_avg, " + w)
            assert_bitwise(got_v[lo:lo + k], v[lo:lo + k], "exp_avg_sq, " + w)
            assert_bitwise(got_lp[lo:lo + k], lp, "slot, " + w)
    del opt, base, master, ag, g
    torch.cuda.empty_cache()


def test_adamw_group_counter_across_calls(zf):
    """The update of a large shard takes its tile groups from a counter in the
    step state, which every launch must return to zero.  Two FlatParameter
    units share one state (one global norm): two updates per step on the same
    state, a skipped step (an inf in unit 0) between two applied ones; unit 1
    also writes the INT8 codes and block scales of its slot.  Every element of
    both units (and unit 1's codes and scales) against the oracle at each
    step, the counter zero after each, nothing written by the skipped step."""
    dev = torch.device("cuda:0")
    sizes = (40_000_003, 34_000_001)        # at least 8,192 groups of four 1,024-element tiles
    hp = dict(lr=3e-5, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, max_grad_norm=0.5)
    hpo = orc.Hparams(**hp)
    scale = 256.0
    state = zf.StepState(scale, False)
    units = []
    for u, n in enumerate(sizes):
        master = torch.empty(n, device=dev)
        synth.fill_normal(master, synth.stream_key("ctr-p", u), 0, 0.02)
        units.append(dict(n=n, master=master, m=torch.zeros_like(master),
                          v=torch.zeros_like(master), ag=torch.zeros(n, dtype=torch.float16, device=dev),
                          g=torch.empty(n, dtype=torch.float16, device=dev),
                          p_ref=to_host(master).copy(), m_ref=np.zeros(n, np.float32),
                          v_ref=np.zeros(n, np.float32),
                          q=torch.zeros(n, dtype=torch.int8, device=dev) if u == 1 else None,
                          qs=torch.zeros(-(-n // 256), device=dev) if u == 1 else None))
    applied = 0
    for step, skip in enumerate((False, True, False)):
        say("group counter step", step, "skip" if skip else "")
        for u, U in enumerate(units):
            synth.fill_normal(U["g"], synth.stream_key("ctr-g", u, step), 0, 1e-3 * scale)
        if skip:
            units[0]["g"][12345] = float("inf")
        before = [to_host(U["master"]).copy() for U in units] if skip else None
        before_q = (to_host(units[1]["q"]).copy(), to_host(units[1]["qs"]).copy()) if skip else None
        for U in units:
            zf.zero_unscale_norm(U["g"], state)
        for u, U in enumerate(units):
            zf.zero_adamw_shard_step(U["g"], U["master"], U["m"], U["v"], U["ag"], 0, hp, state,
                                     q_buf=U["q"], q_scales=U["qs"],
                                     finalize=u == len(units) - 1)
        st = state.read()
        assert st.tile_counter == 0
        assert st.last_skipped == int(skip)
        if skip:
            for U, b in zip(units, before):
                assert_bitwise(to_host(U["master"]), b, "master after a skipped step")
            assert_bitwise(to_host(units[1]["q"]), before_q[0], "INT8 codes after a skipped step")
            assert_bitwise(to_host(units[1]["qs"]), before_q[1], "INT8 scales after a skipped step")
            continue
        applied += 1
        gh = [to_host(U["g"]).copy() for U in units]
        sumsq = sum(orc.unscale_stats(g, orc.F16, scale)[0] for g in gh)
        coef = orc.clip_coef(sumsq, hp["max_grad_norm"])
        assert coef < 1.0 and st.last_coef == coef
        for U, g in zip(units, gh):
            lp = orc.adamw(g, orc.F16, U["p_ref"], U["m_ref"], U["v_ref"], scale, coef, applied,
                           hpo, orc.F16)
            assert_bitwise(to_host(U["master"]), U["p_ref"], "master, step %d" % step)
            assert_bitwise(to_host(U["m"]), U["m_ref"], "exp_avg, step %d" % step)
            assert_bitwise(to_host(U["v"]), U["v_ref"], "exp_avg_sq, step %d" % step)
            assert_bitwise(to_host(U["ag"]), lp, "slot, step %d" % step)
            if U["q"] is not None:
                rq, rs = orc.quant_int8(lp, orc.F16, 256)
                assert_bitwise(to_host(U["q"]), rq, "INT8 codes, step %d" % step)
                assert_bitwise(to_host(U["qs"]), rs, "INT8 scales, step %d" % step)
    del units
    torch.cuda.empty_cache()
