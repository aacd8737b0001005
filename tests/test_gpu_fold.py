"""The statistics' fold: the sum of squares is the per-block partial sums added
in one fixed order -- 1,024 lanes, lane t adding partials t, t + 1024, ...; a
butterfly over each 64-lane wave; the 16 wave sums in order.  A reduce of at
most 1,024 blocks in one launch folds inside its last block instead of in the
fold kernel, and must give the same bits.  Both paths are compared with that
order computed on the host from the partials the state holds, bit for bit,
and the in-kernel path's counter must be back at zero."""
import numpy as np
import pytest
import torch

from synth import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def zf():
    import fsdp_sharded_mixed_flatparameter_amd as m
    assert torch.cuda.is_available()
    return m


def host_fold(partials):
    """The fixed fold order, in binary64 on the host."""
    n = partials.size
    lanes = np.zeros(1024)
    for t in range(1024):
        s = 0.0
        for i in range(t, n, 1024):
            s = s + float(partials[i])
        lanes[t] = s
    total = 0.0
    for w in range(16):
        x = lanes[64 * w:64 * (w + 1)].copy()
        off = 32
        while off > 0:
            x = x + x[np.arange(64) ^ off]
            off >>= 1
        total = total + float(x[0])
    return total


@pytest.mark.parametrize("n,N,dt", [(262_528, 4, torch.float16),        # Tiny: 129 blocks, folded in the kernel
                                    (4096 * 1024, 8, torch.bfloat16),   # exactly 1,024 blocks: in the kernel
                                    (4096 * 1024 + 1, 8, torch.float16),  # 1,025: the fold kernel
                                    (1_000_001, 1, torch.float16),      # statistics pass, 489 blocks
                                    (3_000_001, 1, torch.float16)])     # statistics pass, 1,465 blocks
def test_fold_order(zf, n, N, dt):
    bufs = []
    for k in range(N):
        b = torch.empty(n, dtype=dt, device="cuda")
        synth.fill_normal(b, synth.stream_key("fold", n, k), 0, 1e-3)
        bufs.append(b)
    st = zf.StepState(1024.0, False)
    if N == 1:
        zf.zero_unscale_norm(bufs[0], st)
    else:
        out = torch.empty(n, device="cuda")
        zf.zero_grad_reduce_shard(bufs, 0, n, zf.ZERO_AVG, out, st)
    s = st.read()
    parts = np.frombuffer(bytes(s.partials), dtype=np.float64)[:s.n_partials]
    assert s.n_partials >= 1 and s.tile_counter == 0
    assert s.sumsq == host_fold(parts), (s.sumsq, host_fold(parts), s.n_partials)
