"""Test helpers: host<->device array moves, and running the same step on the
GPU library and on the oracle from identical seeded inputs."""
import numpy as np
import torch

from oracle import oracle as orc

TORCH_DT = {0: torch.float32, 1: torch.float16, 2: torch.bfloat16}


def to_dev(a, code, dev="cuda"):
    """numpy (float32, or uint16 bit patterns) -> torch tensor of the format."""
    if code == 0:
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)
    t = torch.from_numpy(np.ascontiguousarray(a, np.uint16).view(np.int16))
    return t.view(TORCH_DT[code]).to(dev)


def to_host(t):
    """torch tensor -> numpy float32, or uint16 bit patterns for 16-bit formats."""
    t = t.detach().cpu()
    if t.dtype == torch.float32:
        return t.numpy()
    if t.dtype in (torch.float16, torch.bfloat16):
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def bits(a):
    a = np.asarray(a)
    return a.view(np.uint32) if a.dtype == np.float32 else a


def assert_bitwise(got, ref, what):
    g, r = bits(got), bits(ref)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    bad = np.nonzero(g != r)[0]
    if bad.size:
        i = int(bad[0])
        raise AssertionError("%s: %d of %d elements differ; first at %d: got %r want %r"
                             % (what, bad.size, g.size, i, got[i], ref[i]))


def is_nan(a, code):
    """NaN mask of float32 values (code 0) or 16-bit bit patterns (1 fp16, 2 bf16)."""
    a = np.asarray(a)
    if code == 0:
        return np.isnan(a)
    exp, man = (0x7C00, 0x03FF) if code == 1 else (0x7F80, 0x007F)
    return ((a & exp) == exp) & ((a & man) != 0)


def assert_bitwise_nan_class(got, ref, code, what):
    """Bit-exact, except that NaN results only have to be NaN: IEEE 754 leaves
    the sign of the NaN of an invalid operation (0 * inf) to the platform."""
    ng, nr = is_nan(got, code), is_nan(ref, code)
    bad = np.nonzero(ng != nr)[0]
    assert bad.size == 0, "%s: NaN at different places, first %d" % (what, int(bad[0]))
    g, r = bits(got).copy(), bits(ref).copy()
    g[ng] = 0
    r[nr] = 0
    assert_bitwise(g, r, what)


def ulp16_distance(a, b):
    """|ord(a) - ord(b)| for 16-bit float bit patterns (sign-magnitude order)."""
    def order(x):
        x = x.astype(np.int32)
        return np.where(x & 0x8000, -(x & 0x7FFF), x & 0x7FFF)
    return np.abs(order(a) - order(b))


def rel_err(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return np.abs(got - ref) / np.maximum(np.abs(ref), 2.0 ** -126)


def assert_within_tolerance(got_p, got_m, got_v, got_lp, p, m, v, lp):
    """The stated acceptance bar: rel 1e-6 on master/m/v, 1 ulp on the slot."""
    for name, g, r in (("master", got_p, p), ("exp_avg", got_m, m), ("exp_avg_sq", got_v, v)):
        e = rel_err(g, r).max() if g.size else 0.0
        assert e <= 1e-6, "%s max rel err %g" % (name, e)
    if lp is not None and got_lp.size:
        assert ulp16_distance(got_lp, lp).max() <= 1


class OracleRank:
    """The oracle's state for one rank's shard across steps."""

    def __init__(self, master0, loss_scale, dynamic, window=1000, min_scale=1.0):
        self.p = np.array(master0, np.float32, copy=True)
        self.m = np.zeros_like(self.p)
        self.v = np.zeros_like(self.p)
        self.scaler = orc.make_scaler(loss_scale, dynamic, window, min_scale)

    def step(self, grad, grad_dtype, hp, param_dtype, remote_sumsq=0.0, remote_overflow=0,
             quant_block=None, sumsq_local=None, overflow_local=None):
        return orc.shard_step(grad=grad, grad_dtype=grad_dtype, master=self.p, exp_avg=self.m,
                              exp_avg_sq=self.v, scaler=self.scaler, hp=orc.Hparams(**hp),
                              param_dtype=param_dtype, remote_sumsq=remote_sumsq,
                              remote_overflow=remote_overflow, quant_block=quant_block,
                              sumsq_local=sumsq_local, overflow_local=overflow_local)
