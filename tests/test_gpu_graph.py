"""The step inside a captured HIP graph: every library call only enqueues
kernels on the current stream (no allocation, no synchronisation, no memset),
so a whole step -- reduce with statistics, AdamW, write-back, finalize -- can
be captured once and replayed.  Each replay, with eager work and
synchronisations between replays, must equal the eager step bit for bit,
including a step skipped on overflow and the loss scaler it moves."""
import numpy as np
import pytest
import torch

from harness import assert_bitwise, to_dev, to_host
from synth import synth
from synth.workloads import WORKLOADS, key_grad, key_master

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def zf():
    import fsdp_sharded_mixed_flatparameter_amd as m
    assert torch.cuda.is_available()
    return m


def say(*a):
    print(*a, flush=True)


def test_captured_step_replays_equal_eager_steps(zf):
    w = WORKLOADS["tiny_mlp_n4"]
    S, r, N = w.shard, w.rank, w.n_ranks
    start = r * S
    master0 = synth.normal_f32(key_master(w), start, S, w.master_sigma)
    dev = torch.device("cuda:0")

    def make():
        opt = zf.ShardOptimizer(to_dev(master0, 0), w.hp, loss_scale=w.loss_scale, dynamic=True,
                                window=2)
        ag = torch.zeros(w.padded, dtype=torch.float16, device=dev)
        bufs = [torch.zeros(w.padded, dtype=torch.float16, device=dev) for _ in range(N)]
        return opt, ag, bufs

    eager, ag_e, bufs_e = make()
    graphed, ag_g, bufs_g = make()

    def load(bufs, step):
        for k in range(N):
            g = synth.normal(key_grad(w, step, k), 0, w.padded, w.grad_sigma, synth.F16)
            if step == 3 and k == 1:
                g[start + 5] = 0x7C00                         # +inf: this step is skipped
            bufs[k].copy_(to_dev(g, synth.F16))

    # one eager step on the graphed optimizer's twin buffers warms every code path
    # up (kernel loading, occupancy queries) before capture, then both restart
    load(bufs_g, 0)
    warm = zf.ShardOptimizer(to_dev(master0, 0), w.hp, loss_scale=w.loss_scale)
    warm.step_from_rank_buffers(bufs_g, start, ag_g.clone(), start)
    torch.cuda.synchronize()

    graphed.reduced_buffer()                                  # allocated before capture
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            graphed.step_from_rank_buffers(bufs_g, start, ag_g, start)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    # capture recorded the step without running it: the state is untouched
    assert graphed.state.read().step == 0

    for step in range(6):
        say("graph replay", step)
        load(bufs_e, step)
        eager.step_from_rank_buffers(bufs_e, start, ag_e, start)
        load(bufs_g, step)
        graph.replay()
        torch.cuda.synchronize()
        se, sg = eager.state.read(), graphed.state.read()
        assert (sg.step, sg.good_steps, sg.loss_scale, sg.last_skipped) == \
            (se.step, se.good_steps, se.loss_scale, se.last_skipped)
        assert sg.last_norm == se.last_norm and sg.last_coef == se.last_coef
        for a, b, name in ((graphed.master, eager.master, "master"),
                           (graphed.exp_avg, eager.exp_avg, "exp_avg"),
                           (graphed.exp_avg_sq, eager.exp_avg_sq, "exp_avg_sq"),
                           (ag_g, ag_e, "slot")):
            assert_bitwise(to_host(a), to_host(b), "%s after replay %d" % (name, step))
    assert se.last_skipped == 0 and se.step == 5       # step 3 was skipped
    assert np.isfinite(se.last_norm)


def test_captured_large_step_replays_equal_eager_steps(zf):
    """A shard large enough for the reduce's launch slices (two launches, the
    statistics added across them) and for the update's counter-scheduled
    kernel: the captured step replayed four times (one step skipped on an
    inf) equals the eager step bit for bit, and the tile counter is back at
    zero after every replay."""
    S, N = 140_000_001, 8
    dev = torch.device("cuda:0")
    hp = dict(lr=3e-5, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, max_grad_norm=1.0)
    master0 = torch.empty(S, device=dev)
    synth.fill_normal(master0, synth.stream_key("graph-large-p"), 0, 0.02)
    eager = zf.ShardOptimizer(master0.clone(), hp, loss_scale=1024.0, dynamic=True, window=2)
    graphed = zf.ShardOptimizer(master0.clone(), hp, loss_scale=1024.0, dynamic=True, window=2)
    del master0
    ag_e = torch.zeros(S, dtype=torch.float16, device=dev)
    ag_g = torch.zeros(S, dtype=torch.float16, device=dev)
    bufs = [torch.empty(S, dtype=torch.float16, device=dev) for _ in range(N)]

    def load(step):
        for k in range(N):
            synth.fill_normal(bufs[k], synth.stream_key("graph-large-g", step, k), 0, 1.0)
        if step == 2:
            bufs[3][S - 7] = float("inf")                     # this step is skipped

    load(0)
    warm = zf.ShardOptimizer(eager.master.clone(), hp, loss_scale=1024.0)
    warm.step_from_rank_buffers(bufs, 0, ag_g.clone(), 0)
    del warm
    graphed.reduced_buffer()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            graphed.step_from_rank_buffers(bufs, 0, ag_g, 0)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    assert graphed.state.read().step == 0

    for step in range(4):
        say("large graph replay", step)
        load(step)
        eager.step_from_rank_buffers(bufs, 0, ag_e, 0)
        graph.replay()
        torch.cuda.synchronize()
        se, sg = eager.state.read(), graphed.state.read()
        assert se.tile_counter == 0 and sg.tile_counter == 0
        assert (sg.step, sg.good_steps, sg.loss_scale, sg.last_skipped) == \
            (se.step, se.good_steps, se.loss_scale, se.last_skipped)
        assert sg.last_norm == se.last_norm and sg.last_coef == se.last_coef
        for a, b, name in ((graphed.master, eager.master, "master"),
                           (graphed.exp_avg, eager.exp_avg, "exp_avg"),
                           (graphed.exp_avg_sq, eager.exp_avg_sq, "exp_avg_sq"),
                           (ag_g, ag_e, "slot")):
            assert torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a.view(torch.int16),
                               b.view(torch.int32) if b.dtype == torch.float32 else b.view(torch.int16)), \
                "%s after replay %d" % (name, step)
    assert se.last_skipped == 0 and se.step == 3
    del eager, graphed, ag_e, ag_g, bufs
    torch.cuda.empty_cache()
