"""ZeRO-Offload's host step (zero_offload_adamw_host, libzeroflat's C ABI;
host code, no GPU needed) against the oracle on the same seeded inputs:
bit-exact master, m, v and 16-bit parameters for every gradient/parameter
format, ragged sizes and thread counts, steps t = 1..5, clipping, and the
skip on overflow.

Pages: "DeepSpeed 与 FSDP", ZeRO-Offload (fp32 optimizer state and the Adam
update on the CPU); ZeRO reading at 2kiu.com §4.1, §5.1.
"""
import numpy as np
import pytest
import torch

from oracle import oracle as orc
from synth import synth

HP = dict(lr=3e-5, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, max_grad_norm=1.0)
TDT = {0: torch.float32, 1: torch.float16, 2: torch.bfloat16}


@pytest.fixture(scope="module")
def zf():
    import fsdp_sharded_mixed_flatparameter_amd as m
    return m


def host_tensor(a, code):
    if code == 0:
        return torch.from_numpy(np.ascontiguousarray(a, np.float32).copy())
    return torch.from_numpy(np.ascontiguousarray(a, np.uint16).view(np.int16).copy()).view(TDT[code])


def bits16(t):
    return t.view(torch.int16).numpy().view(np.uint16)


def state_for(zf, step, scale, sumsq=0.0, remote=0.0, overflow=0, hp=HP):
    """A host step state as the device holds it before step `step`+1: beta
    powers as `step` successive binary64 products."""
    st = zf.zero_step_state_init(scale, False)
    b1 = b2 = 1.0
    for _ in range(step):
        b1 *= hp["beta1"]
        b2 *= hp["beta2"]
    st.step, st.beta1_pow, st.beta2_pow = step, b1, b2
    st.sumsq, st.remote_sumsq, st.overflow = sumsq, remote, overflow
    return st


CASES = [  # (grad dtype, param dtype, n, threads, loss scale)
    (1, 1, 262_528, 4, 65536.0), (2, 2, 100_003, 3, 1.0), (0, 1, 4097, 1, 1024.0),
    (0, 2, 1, 2, 1.0), (1, 2, 70_000, 8, 65536.0), (2, 1, 777, 16, 1.0),
]


@pytest.mark.parametrize("gdt,pdt,n,threads,scale", CASES)
def test_host_step_matches_oracle(zf, orc, gdt, pdt, n, threads, scale):
    key = synth.stream_key("offload-host", gdt, pdt, n)
    p0 = synth.normal_f32(key, 0, n, 0.02)
    p_ref, m_ref, v_ref = p0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    p, m, v = host_tensor(p0, 0), torch.zeros(n), torch.zeros(n)
    lp = torch.empty(n, dtype=TDT[pdt])
    hp = orc.Hparams(**HP)
    for step in range(5):
        g = synth.normal(synth.stream_key("offload-host-g", gdt, n, step), 0, n,
                         1e-3 * (scale if gdt == 0 else 1.0), gdt)
        sumsq, ovf = orc.unscale_stats(g, gdt, scale)
        remote = 0.0 if step < 3 else 4.0 * max(sumsq, 1e-30)     # clipping on later steps
        st = state_for(zf, step, scale, sumsq, remote)
        assert zf.zero_offload_adamw_host(host_tensor(g, gdt), p, m, v, lp, HP, st, threads) == 0
        coef = orc.clip_coef(sumsq + remote, HP["max_grad_norm"])
        lp_ref = orc.adamw(g, gdt, p_ref, m_ref, v_ref, scale, coef, step + 1, hp, pdt)
        for name, got, ref in (("master", p, p_ref), ("exp_avg", m, m_ref), ("exp_avg_sq", v, v_ref)):
            assert np.array_equal(got.numpy().view(np.uint32), ref.view(np.uint32)), (name, step)
        assert np.array_equal(bits16(lp), lp_ref), step


@pytest.mark.parametrize("gdt,pdt,n,threads", [(1, 1, 262_528, 4), (2, 1, 70_001, 3),
                                              (1, 2, 4097, 16), (2, 2, 1, 1)])
def test_host_step_in_place(zf, orc, gdt, pdt, n, threads):
    """A 16-bit gradient and the 16-bit parameters in one array (in-place
    staging): the parameters that overwrite the gradient, and master, m, v,
    equal the oracle's bit for bit over three steps (the later ones clipped)."""
    scale = 1024.0
    p0 = synth.normal_f32(synth.stream_key("offload-inplace", gdt, pdt, n), 0, n, 0.02)
    p_ref, m_ref, v_ref = p0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    p, m, v = host_tensor(p0, 0), torch.zeros(n), torch.zeros(n)
    hp = orc.Hparams(**HP)
    for step in range(3):
        g = synth.normal(synth.stream_key("offload-inplace-g", gdt, n, step), 0, n, 1e-3, gdt)
        sumsq, _ = orc.unscale_stats(g, gdt, scale)
        remote = 0.0 if step == 0 else 4.0 * max(sumsq, 1e-30)
        st = state_for(zf, step, scale, sumsq, remote)
        buf = host_tensor(g, gdt)
        assert zf.zero_offload_adamw_host(buf, p, m, v, buf.view(TDT[pdt]), HP, st, threads) == 0
        coef = orc.clip_coef(sumsq + remote, HP["max_grad_norm"])
        lp_ref = orc.adamw(g, gdt, p_ref, m_ref, v_ref, scale, coef, step + 1, hp, pdt)
        for name, got, ref in (("master", p, p_ref), ("exp_avg", m, m_ref), ("exp_avg_sq", v, v_ref)):
            assert np.array_equal(got.numpy().view(np.uint32), ref.view(np.uint32)), (name, step)
        assert np.array_equal(bits16(buf), lp_ref), step


def test_host_step_refuses_partial_overlap(zf):
    n = 1000
    st = state_for(zf, 0, 1.0)
    p, m, v = torch.zeros(n), torch.zeros(n), torch.zeros(n)
    big = torch.zeros(n + 1, dtype=torch.float16)
    with pytest.raises(zf.ZeroError, match="overlaps"):
        zf.zero_offload_adamw_host(big[:n], p, m, v, big[1:], HP, st)    # shifted by one
    g32 = torch.zeros(n)
    with pytest.raises(zf.ZeroError, match="overlaps"):
        zf.zero_offload_adamw_host(g32, p, m, v, g32.view(torch.float16)[:n], HP, st)


def test_host_step_skips_on_overflow(zf):
    n = 1000
    p = torch.randn(n)
    m, v = torch.randn(n), torch.rand(n)
    lp = torch.zeros(n, dtype=torch.float16)
    before = [t.clone() for t in (p, m, v, lp)]
    g = torch.zeros(n, dtype=torch.float16)
    for local, remote in ((1, 0), (0, 1)):
        st = state_for(zf, 2, 65536.0, overflow=local)
        st.remote_overflow = remote
        assert zf.zero_offload_adamw_host(g, p, m, v, lp, HP, st, 4) == 1
        for t, b in zip((p, m, v, lp), before):
            assert torch.equal(t.view(torch.int16) if t.dtype == torch.float16 else t,
                               b.view(torch.int16) if b.dtype == torch.float16 else b)


def test_host_step_special_values(zf, orc):
    """Write-back rounding corner cases through the host path: values that
    round to fp16 infinity, subnormals and exact ties, against the oracle."""
    n = 64
    p0 = np.array([65504.0, 65519.99, 65520.0, 6.0e-8, 2.0 ** -24 * 1.5, 1.0 + 2.0 ** -11,
                   -0.0, 3.0e38] * 8, np.float32)
    g = np.zeros(n, np.uint16)
    hp0 = dict(HP, lr=0.0, weight_decay=0.0)                       # p' = p * 1 - 0
    p = host_tensor(p0, 0)
    lp = torch.empty(n, dtype=torch.float16)
    st = state_for(zf, 0, 1.0, hp=hp0)
    assert zf.zero_offload_adamw_host(host_tensor(g, 1), p, torch.zeros(n), torch.zeros(n), lp,
                                      hp0, st, 2) == 0
    assert np.array_equal(bits16(lp), orc.f32_to_f16(p0))


def test_host_step_rejects_bad_arguments(zf):
    n = 16
    t = torch.zeros(n)
    lp = torch.zeros(n, dtype=torch.float16)
    st = state_for(zf, 0, 1.0)
    with pytest.raises(zf.ZeroError):
        zf.zero_offload_adamw_host(t, t, t, t, lp, dict(HP, beta1=1.0), st)
    with pytest.raises(zf.ZeroError):
        zf.zero_offload_adamw_host(t, t, t, t, t, HP, st)          # fp32 parameters
    with pytest.raises(ValueError):
        zf.zero_offload_adamw_host(t, t, t[:8], t, lp, HP, st)
