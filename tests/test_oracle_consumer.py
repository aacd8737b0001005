"""Pins of the oracle's two steps next to the optimizer step: the INT8
All-Gather consumer (dequantise the gathered slots into the full flat
parameter) and sharded gradient accumulation over micro-steps.  Each pin is a
closed form, an exact case, a hand table, a round trip through the separately
pinned quantiser, or an error bound -- none re-types the oracle's arithmetic.

Pages: "DeepSpeed 与 FSDP" (docs.ifdog.com) -- "ZeRO++：量化通信压缩" (int8
parameter shards, dequantised by the receiver), "FSDP 的分片粒度与
FlatParameter" (one All-Gather of the flat buffer, then unflatten), "实践要点"
(gradient accumulation, loss divided by the step count); ZeRO reading at
2kiu.com §4.2 (INT8 weights restored before local compute), §5.1 (two
accumulation steps), §5.3 (gradients accumulate while sharded; the changed
summation order only moves results by rounding).
"""
from fractions import Fraction as Fr

import numpy as np
import pytest
import torch


def f16(x):
    return np.asarray(x, np.float32).astype(np.float16).view(np.uint16)


def bf16_of(xf32):
    """Library RNE binary32 -> bfloat16 (torch CPU), as uint16 bit patterns."""
    t = torch.from_numpy(np.ascontiguousarray(xf32, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


# ------------------------------------------------------------------ dequant
@pytest.mark.parametrize("dt", ["F32", "F16", "BF16"])
def test_dequant_power_of_two_scales_is_exact(orc, dt):
    """q * 2^k needs at most 7 significant bits: exact in every format."""
    rng = np.random.default_rng(21)
    S, blk = 256 * 5, 256
    q = rng.integers(-127, 128, S).astype(np.int8)
    ks = rng.integers(-10, 6, S // blk)
    scales = np.ldexp(np.ones(S // blk), ks).astype(np.float32)
    out = orc.dequant_int8(q, scales, 1, S, blk, getattr(orc, dt))
    exact = q.astype(np.float64) * np.repeat(np.ldexp(1.0, ks), blk)  # exact values
    if dt == "F32":
        assert np.array_equal(out, exact.astype(np.float32))
    elif dt == "F16":
        assert np.array_equal(out, exact.astype(np.float16).view(np.uint16))
    else:
        assert np.array_equal(out, bf16_of(exact.astype(np.float32)))


def test_dequant_slot_and_block_indexing(orc):
    """Hand table: 3 slots of 300 codes, blocks of 256 restart at each slot
    (2 scales per slot, the second block 44 long).  Code 1 everywhere and the
    scale of (slot s, block b) = 2^-(2s+b+1), so out shows which scale served
    every element."""
    n_slots, S, blk = 3, 300, 256
    nb = 2
    q = np.ones(n_slots * S, np.int8)
    scales = np.array([2.0 ** -(i + 1) for i in range(n_slots * nb)], np.float32)
    out = orc.dequant_int8(q, scales, n_slots, S, blk, orc.F32)
    want = []
    for s in range(n_slots):
        want += [2.0 ** -(2 * s + 1)] * 256 + [2.0 ** -(2 * s + 2)] * 44
    assert np.array_equal(out, np.array(want, np.float32))
    # the slot's codes land at s*S in the full flat buffer
    q2 = np.zeros(n_slots * S, np.int8)
    q2[S + 7] = 5
    out2 = orc.dequant_int8(q2, np.ones(n_slots * nb, np.float32), n_slots, S, blk, orc.F32)
    assert np.flatnonzero(out2).tolist() == [S + 7] and out2[S + 7] == 5.0


def test_dequant_zero_scale_and_zero_code(orc):
    """A block the producer saw as all-zero has scale 0: its values are zeros
    (IEEE sign of a product: negative code times +0 is -0)."""
    q = np.array([0, 3, -3, 127, -127] + [0] * 251, np.int8)
    out = orc.dequant_int8(q, np.zeros(1, np.float32), 1, 256, 256, orc.F32)
    assert not out.any()
    assert np.signbit(out[2]) and np.signbit(out[4]) and not np.signbit(out[1])
    outb = orc.dequant_int8(q, np.zeros(1, np.float32), 1, 256, 256, orc.BF16)
    assert outb[2] == 0x8000 and outb[1] == 0 and outb[0] == 0


@pytest.mark.parametrize("dt", ["F16", "BF16"])
def test_dequant_round_trip_through_the_quantiser(orc, dt):
    """quant (pinned separately) then dequant: every block's absmax element
    comes back bit-exact (127 * f32(amax/127) is within 2^-23 relative of amax,
    far inside half an ulp of the 16-bit format), and every element is within
    half a quantisation step plus half an ulp of the 16-bit result."""
    code = getattr(orc, dt)
    rng = np.random.default_rng(22)
    n_slots, S, blk = 4, 256 * 3 + 50, 256
    x = orc.from_f32((rng.standard_normal(n_slots * S) * 0.02).astype(np.float32), code)
    qs, ss = [], []
    for s in range(n_slots):
        q, sc = orc.quant_int8(x[s * S:(s + 1) * S], code, blk)
        qs.append(q)
        ss.append(sc)
    q, sc = np.concatenate(qs), np.concatenate(ss)
    out = orc.dequant_int8(q, sc, n_slots, S, blk, code)
    xv, ov = orc.to_f32(x, code), orc.to_f32(out, code)
    nb = -(-S // blk)
    half_ulp = 2.0 ** -11 if dt == "F16" else 2.0 ** -8   # relative, normal range
    for s in range(n_slots):
        for b in range(nb):
            lo, hi = s * S + b * blk, s * S + min((b + 1) * blk, S)
            j = lo + int(np.argmax(np.abs(xv[lo:hi])))
            assert out[j] == x[j]
            step = float(sc[s * nb + b])
            err = np.abs(ov[lo:hi].astype(np.float64) - xv[lo:hi])
            assert np.all(err <= step * (0.5 + 2.0 ** -15) + np.abs(ov[lo:hi]) * half_ulp + 1e-30)


def test_dequant_rounding_vs_exact_product(orc):
    """Random codes and fp32 scales: the binary64 product q*scale is exact
    (7 + 24 bits), so rounding it once to binary32, then once to the 16-bit
    format with the libraries' RNE, is the definition's value."""
    rng = np.random.default_rng(23)
    n_slots, S, blk = 2, 1000, 256
    nb = -(-S // blk)
    q = rng.integers(-127, 128, n_slots * S).astype(np.int8)
    sc = (np.abs(rng.standard_normal(n_slots * nb)) * 3e-4).astype(np.float32)
    per = np.concatenate([np.repeat(sc[s * nb:(s + 1) * nb], blk)[:S] for s in range(n_slots)])
    exact32 = (q.astype(np.float64) * per.astype(np.float64)).astype(np.float32)
    assert np.array_equal(orc.dequant_int8(q, sc, n_slots, S, blk, orc.F32), exact32)
    assert np.array_equal(orc.dequant_int8(q, sc, n_slots, S, blk, orc.F16),
                          exact32.astype(np.float16).view(np.uint16))
    assert np.array_equal(orc.dequant_int8(q, sc, n_slots, S, blk, orc.BF16), bf16_of(exact32))


# ------------------------------------------------------------------ accumulation
def test_accumulate_first_micro_step_is_the_reduce(orc):
    """Into a zeroed shard the first micro-step leaves exactly the reduce's
    result (0 + r == r, and the reduce never yields -0)."""
    rng = np.random.default_rng(31)
    for dt in (orc.F16, orc.BF16):
        bufs = [orc.from_f32((rng.standard_normal(999) * 1e-3).astype(np.float32), dt)
                for _ in range(4)]
        bufs[1][5] = 0x8000   # -0 in one rank buffer
        for op in (orc.SUM, orc.AVG):
            red = orc.reduce(bufs, dt, 0, 999, op)
            acc = orc.reduce_accumulate(bufs, dt, 0, 999, op, np.zeros(999, np.float32))
            assert np.array_equal(acc.view(np.uint32), red.view(np.uint32))


def test_accumulate_exact_sums(orc):
    """K micro-steps of dyadic values with few bits: every sum is exact, so
    acc = sum over micro-steps of (sum over ranks)/N as rationals."""
    rng = np.random.default_rng(32)
    n, N, K = 600, 8, 3
    off = 2 * n
    want = [Fr(0)] * n
    acc = np.zeros(n, np.float32)
    for k in range(K):
        ints = rng.integers(-64, 65, (N, 4 * n))
        bufs = [f16(ints[r] * 2.0 ** -10) for r in range(N)]
        orc.reduce_accumulate(bufs, orc.F16, off, n, orc.AVG, acc)
        for i in range(n):
            want[i] += Fr(int(ints[:, off + i].sum()), 1024 * N)
    assert [Fr(float(a)) for a in acc] == want


def test_accumulate_reduces_before_adding(orc):
    """acc = 1, two ranks each holding 2^-24 (an fp16 subnormal): the
    micro-step's reduce gives 2^-23 and 1 + 2^-23 is exact; adding the ranks
    one by one into the shard would round each 1 + 2^-24 back to 1."""
    tiny = np.array([1], np.uint16)                     # fp16 bits of 2^-24
    acc = np.ones(1, np.float32)
    orc.reduce_accumulate([tiny, tiny], orc.F16, 0, 1, orc.SUM, acc)
    assert float(acc[0]) == 1.0 + 2.0 ** -23


def test_accumulate_order_moves_results_only_by_rounding(orc):
    """Sharded accumulation (reduce each micro-step, then add) and local
    accumulation followed by one reduce sum the same terms in another order;
    both stay within the summation error bound of the exact sum."""
    rng = np.random.default_rng(33)
    n, N, K = 4096, 4, 2
    # bf16 values with magnitudes spread over 2^-30..1, so that partial sums round
    xs = [[orc.from_f32((rng.standard_normal(n) * 2.0 ** rng.integers(-30, 1, n))
                        .astype(np.float32), orc.BF16) for _ in range(N)] for _ in range(K)]
    acc = np.zeros(n, np.float32)
    for k in range(K):
        orc.reduce_accumulate(xs[k], orc.BF16, 0, n, orc.SUM, acc)
    vals = np.array([[orc.to_f32(xs[k][r], orc.BF16) for r in range(N)] for k in range(K)],
                    np.float64)
    exact = vals.sum(axis=(0, 1))
    bound = (N + K) * 2.0 ** -24 * np.abs(vals).sum(axis=(0, 1))
    assert np.all(np.abs(acc - exact) <= bound)
    # the other order (each rank accumulates locally in binary32, then one reduce)
    local = [np.zeros(n, np.float32) for _ in range(N)]
    for k in range(K):
        for r in range(N):
            local[r] = local[r] + vals[k, r].astype(np.float32)
    other = np.zeros(n, np.float32)
    for r in range(N):
        other = other + local[r]
    assert np.all(np.abs(other - exact) <= bound)
    assert np.count_nonzero(other != acc) > 0      # the order is visible in the last bits


def test_accumulated_overflow_persists(orc):
    """An inf in an early micro-step stays non-finite in the shard, so the
    overflow test on the accumulated gradient still fires."""
    n = 64
    a = f16(np.full(n, 1e-3))
    b = a.copy()
    b[9] = 0x7C00                                        # +inf
    acc = orc.reduce_accumulate([a, b], orc.F16, 0, n, orc.AVG, np.zeros(n, np.float32))
    orc.reduce_accumulate([a, a], orc.F16, 0, n, orc.AVG, acc)
    _, ovf = orc.unscale_stats(acc, orc.F32, 1.0)
    assert ovf == 1 and np.isinf(acc[9]) and np.isfinite(np.delete(acc, 9)).all()


# ------------------------------------------------------------------ quantised gradient reduce
# "DeepSpeed 与 FSDP", ZeRO++：量化通信压缩: gradients cross the Reduce-Scatter in a
# quantised form; the reading takes the parameter payload's INT8 block scheme.
def test_reduce_q8_exact_sums(orc):
    """Power-of-two scales: every product and sum is exact, so the reduce is
    the rational sum (AVG: divided by N)."""
    rng = np.random.default_rng(41)
    N, n, blk = 8, 700, 256
    nb = -(-n // blk)
    qs = [rng.integers(-127, 128, n).astype(np.int8) for _ in range(N)]
    ks = [rng.integers(-12, -3, nb) for _ in range(N)]
    scs = [np.ldexp(np.ones(nb), k).astype(np.float32) for k in ks]
    for op in (orc.SUM, orc.AVG):
        red = orc.reduce_q8(qs, scs, n, blk, op)
        for i in range(0, n, 37):
            want = sum(Fr(int(qs[k][i])) * Fr(2) ** int(ks[k][i // blk]) for k in range(N))
            if op == orc.AVG:
                want /= N
            assert Fr(float(red[i])) == want


def test_reduce_q8_block_indexing_hand_table(orc):
    """2 ranks, 300 codes of 1, blocks of 256: rank k's block b has scale
    2^-(2k+b+1); element i in block b reduces to 2^-(b+1) + 2^-(b+3)."""
    n = 300
    qs = [np.ones(n, np.int8), np.ones(n, np.int8)]
    scs = [np.array([0.5, 0.25], np.float32), np.array([0.125, 0.0625], np.float32)]
    red = orc.reduce_q8(qs, scs, n, 256, orc.SUM)
    want = np.array([0.5 + 0.125] * 256 + [0.25 + 0.0625] * 44, np.float32)
    assert np.array_equal(red, want)


def test_reduce_q8_is_rank_ordered(orc):
    """Codes 1 with scales 2^24, 1, 1: in rank order 2^24 + 1 rounds back to
    2^24 twice; summed the other way round it would give 2^24 + 2."""
    qs = [np.ones(1, np.int8)] * 3
    scs = [np.array([2.0 ** 24], np.float32), np.ones(1, np.float32), np.ones(1, np.float32)]
    assert float(orc.reduce_q8(qs, scs, 1, 256, orc.SUM)[0]) == 2.0 ** 24


def test_reduce_q8_equals_dequantise_then_reduce(orc):
    """Random codes and scales: the quantised reduce equals dequantising each
    rank's slice (pinned above) to fp32 and reducing those buffers (pinned in
    test_oracle_step) -- element by element, bitwise."""
    rng = np.random.default_rng(42)
    N, n, blk = 5, 1000, 64
    nb = -(-n // blk)
    qs = [rng.integers(-127, 128, n).astype(np.int8) for _ in range(N)]
    scs = [(np.abs(rng.standard_normal(nb)) * 1e-3).astype(np.float32) for _ in range(N)]
    deq = [orc.dequant_int8(q, sc, 1, n, blk, orc.F32) for q, sc in zip(qs, scs)]
    for op in (orc.SUM, orc.AVG):
        assert np.array_equal(orc.reduce_q8(qs, scs, n, blk, op).view(np.uint32),
                              orc.reduce(deq, orc.F32, 0, n, op).view(np.uint32))


def test_reduce_q8_error_bound_vs_the_fp16_reduce(orc):
    """Each rank quantises its fp16 slice (the pinned quantiser); the quantised
    reduce stays within the sum of the ranks' half quantisation steps (/N for
    AVG), plus binary32 rounding, of the plain fp16 reduce."""
    rng = np.random.default_rng(43)
    N, n, blk = 8, 256 * 6 + 77, 256
    xs = [orc.from_f32((rng.standard_normal(n) * 1e-3).astype(np.float32), orc.F16)
          for _ in range(N)]
    pay = [orc.quant_int8(x, orc.F16, blk) for x in xs]
    for op, div in ((orc.SUM, 1), (orc.AVG, N)):
        red_q = orc.reduce_q8([p[0] for p in pay], [p[1] for p in pay], n, blk, op)
        red = orc.reduce(xs, orc.F16, 0, n, op)
        step = sum(np.repeat(p[1].astype(np.float64), blk)[:n] for p in pay)
        bound = step * (0.5 + 2.0 ** -15) / div + np.abs(red.astype(np.float64)) * 2.0 ** -21
        assert np.all(np.abs(red_q.astype(np.float64) - red) <= bound)


def test_reduce_q8_overflow_reaches_the_flag(orc):
    """A rank whose slice held +inf sent scale inf (codes 0 for the finite
    values): its products are NaN, so the reduce is non-finite and the
    overflow test fires."""
    n = 256
    x = f16(np.full(n, 1e-3))
    x[5] = 0x7C00
    q, sc = orc.quant_int8(x, orc.F16, 256)
    assert np.isinf(sc[0])
    q2, sc2 = orc.quant_int8(f16(np.full(n, 2e-3)), orc.F16, 256)
    red = orc.reduce_q8([q2, q], [sc2, sc], n, 256, orc.AVG)
    assert not np.isfinite(red).any()
    assert orc.unscale_stats(red, orc.F32, 65536.0)[1] == 1
