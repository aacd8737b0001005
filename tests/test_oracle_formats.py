"""Pins of the oracle's fp16/bf16 converters against independent library
routines (numpy's binary16 cast, torch's CPU bfloat16 cast; both round to
nearest-even) and against hand-derived special values.  The write-back of the
fp32 master into the All-Gather slot is this rounding ("PyTorch FSDP 源码级深度解析"
§7.2: the fp16/bf16 copy is derived from the fp32 master)."""
import numpy as np
import pytest
import torch


def _f32_samples():
    rng = np.random.default_rng(7)
    # every fp32 pattern on a prime stride, plus random patterns
    a = np.arange(0, 1 << 32, 1021, dtype=np.uint64).astype(np.uint32)
    b = rng.integers(0, 1 << 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    return np.concatenate([a, b]).view(np.float32)


def _f16_ties_and_neighbours():
    """Midpoints between consecutive binary16 values (as fp32) and the fp32
    values one ulp either side of them: the cases where rounding decides."""
    h = np.arange(0, 0x7C00, dtype=np.uint16)  # non-negative finite halves
    lo = h[:-1].view(np.float16).astype(np.float64)
    hi = h[1:].view(np.float16).astype(np.float64)
    mid = ((lo + hi) / 2).astype(np.float32)   # exact in fp32
    mb = mid.view(np.uint32)
    cand = np.concatenate([mb, mb + 1, mb - 1]).view(np.float32)
    return np.concatenate([cand, -cand])


def test_f16_to_f32_exhaustive(orc):
    h = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    got = orc.f16_to_f32(h)
    ref = h.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


@pytest.mark.parametrize("which", ["samples", "ties"])
def test_f32_to_f16_vs_numpy(orc, which):
    x = _f32_samples() if which == "samples" else _f16_ties_and_neighbours()
    got = orc.f32_to_f16(x)
    with np.errstate(over="ignore", invalid="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], ref[~nan])
    # NaN -> quiet NaN, sign kept
    gn = got[nan]
    assert np.all((gn & 0x7C00) == 0x7C00) and np.all((gn & 0x3FF) != 0)
    assert np.array_equal(gn >> 15, (x[nan].view(np.uint32) >> 31).astype(np.uint16))


def test_bf16_to_f32_exhaustive(orc):
    h = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    got = orc.bf16_to_f32(h)
    ref = torch.from_numpy(h.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_f32_to_bf16_vs_torch(orc):
    x = _f32_samples()
    # bf16 ties: fp32 patterns whose low 16 bits are exactly 0x8000, and neighbours
    rng = np.random.default_rng(11)
    hi = rng.integers(0, 1 << 16, size=1 << 18, dtype=np.uint64).astype(np.uint32) << 16
    ties = np.concatenate([hi | 0x8000, hi | 0x7FFF, hi | 0x8001]).view(np.float32)
    x = np.concatenate([x, ties])
    got = orc.f32_to_bf16(x)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], ref[~nan])
    gn = got[nan]
    assert np.all((gn & 0x7F80) == 0x7F80) and np.all((gn & 0x7F) != 0)


def test_special_values(orc):
    cases16 = {
        65504.0: 0x7BFF,                 # largest finite
        65519.99609375: 0x7BFF,          # just below the overflow threshold
        65520.0: 0x7C00,                 # tie with 65536 rounds to even -> inf
        float("inf"): 0x7C00, float("-inf"): 0xFC00,
        2.0 ** -24: 0x0001,              # smallest subnormal
        2.0 ** -25: 0x0000,              # tie to even (0)
        3 * 2.0 ** -25: 0x0002,          # tie 1.5 -> 2
        2.0 ** -14: 0x0400,              # smallest normal
        1.0 + 2.0 ** -11: 0x3C00,        # tie, even is 1.0
        1.0 + 3 * 2.0 ** -11: 0x3C02,    # tie, even is 1+2^-9
        -0.0: 0x8000,
    }
    for v, bits in cases16.items():
        assert orc.lib().oracle_f32_to_f16(v) == bits, (v, hex(bits))
    cases_bf = {
        1.0 + 2.0 ** -8: 0x3F80,          # tie -> even
        1.0 + 3 * 2.0 ** -8: 0x3F82,
        float("inf"): 0x7F80,
        3.3895313892515355e38: 0x7F7F,    # largest finite bf16
        2.0 ** -149: 0x0000,              # fp32 min subnormal -> below half a bf16 quantum
        2.0 ** -133: 0x0001,              # smallest bf16 subnormal
    }
    for v, bits in cases_bf.items():
        assert orc.lib().oracle_f32_to_bf16(v) == bits, (v, hex(bits))
