"""GPU parity of the INT8 All-Gather consumer (zero_dequant_allgather, through
its C ABI) against the oracle, on the same seeded inputs: small cases over
both kernel paths and the edge cases, a round trip through the library's own
producer, the unflattened parameter views, and the workloads' full sizes (the
7B block exhaustively, the 70B flat parameter on samples plus every slot
boundary).  Bar: bit-exact.

Pages: "DeepSpeed 与 FSDP" -- ZeRO++：量化通信压缩 (int8 shards dequantised on
receipt), FSDP 的分片粒度与 FlatParameter (one All-Gather, then unflatten);
ZeRO reading at 2kiu.com §4.2.
"""
import numpy as np
import pytest
import torch

from harness import assert_bitwise, assert_bitwise_nan_class, to_dev, to_host
from oracle import oracle as orc
from synth import synth
from synth.workloads import GATHERS, key_codes, key_scales

pytestmark = pytest.mark.gpu

TORCH_DT = {0: torch.float32, 1: torch.float16, 2: torch.bfloat16}


@pytest.fixture(scope="module")
def zf():
    import fsdp_sharded_mixed_flatparameter_amd as m
    assert torch.cuda.is_available()
    return m


def say(*a):
    print(*a, flush=True)


def host_payload(tag, n_slots, S, block, sigma=4.7e-4):
    nb = -(-S // block)
    q = synth.codes(synth.stream_key("dq", tag, "codes"), 0, n_slots * S)
    sc = np.abs(synth.normal_f32(synth.stream_key("dq", tag, "scales"), 0, n_slots * nb, sigma))
    return q, sc.astype(np.float32), nb


DEQ_CASES = [
    # (n_slots, slot_numel, block, out dtype, extra byte offset of the codes)
    (1, 1, 256, 2, 0), (1, 4, 256, 2, 0), (1, 2048, 256, 1, 0), (2, 2047, 256, 2, 0),
    (4, 262_528, 256, 1, 0), (8, 2048 * 3 + 100, 256, 2, 0), (3, 1001, 256, 2, 0),
    (5, 4096 + 12, 64, 0, 0), (2, 3000, 12, 2, 0), (2, 2048, 256, 2, 1), (2, 4096, 4, 1, 0),
    (64, 20_000, 256, 2, 0), (7, 513, 256, 0, 0),
    (65536, 4, 4, 2, 0), (65536, 7, 256, 1, 0),    # the most slots per call (tiny slots)
    # flat tiling (slot_numel >= 2048 and a multiple of 4): slot boundaries inside
    # tiles, at offsets that are not multiples of a cache line
    (3, 2052, 256, 2, 0), (5, 2196, 260, 1, 0), (3, 4100, 256, 0, 0), (2, 1_000_004, 256, 2, 0),
]


@pytest.mark.parametrize("n_slots,S,block,dt,mis", DEQ_CASES)
def test_dequant_parity(zf, n_slots, S, block, dt, mis):
    say("dequant", n_slots, S, block, dt, mis)
    q, sc, nb = host_payload("%d-%d-%d" % (n_slots, S, block), n_slots, S, block)
    # edge values: a zero scale, an infinite one, one whose products leave the
    # fp16 range, one whose products are binary32/bfloat16 subnormals
    specials = [0.0, np.inf, 1000.0, 1e-40]
    for i, v in enumerate(specials[:sc.size]):
        sc[(i * 7) % sc.size] = v
    qd = torch.from_numpy(np.concatenate([np.zeros(mis, np.int8), q])).to("cuda")[mis:]
    scd = to_dev(sc, 0)
    out = torch.full((n_slots * S,), float("nan"), dtype=TORCH_DT[dt], device="cuda")
    zf.zero_dequant_allgather(qd, scd, n_slots, S, out, block=block)
    ref = orc.dequant_int8(q, sc, n_slots, S, block, dt)
    assert_bitwise_nan_class(to_host(out), ref, dt, "dequantised flat buffer")


def test_dequant_round_trip_through_the_producer(zf):
    """Slots written by the library's own quantiser, gathered and dequantised,
    equal the oracle's quantise-then-dequantise of the same bf16 slots."""
    n_slots, S = 4, 10_003
    x = synth.normal(synth.stream_key("dq", "roundtrip"), 0, n_slots * S, 0.02, orc.BF16)
    xd = to_dev(x, orc.BF16)
    nb = -(-S // 256)
    qd = torch.zeros(n_slots * S, dtype=torch.int8, device="cuda")
    sd = torch.zeros(n_slots * nb, device="cuda")
    for s in range(n_slots):
        zf.zero_quant_allgather_slot(xd[s * S:(s + 1) * S], qd, sd, q_slot_offset=s * S,
                                     q_scale_offset=s * nb)
    out = torch.empty(n_slots * S, dtype=torch.bfloat16, device="cuda")
    zf.zero_dequant_allgather(qd, sd, n_slots, S, out)
    qs, ss = zip(*[orc.quant_int8(x[s * S:(s + 1) * S], orc.BF16, 256) for s in range(n_slots)])
    q, sc = np.concatenate(qs), np.concatenate(ss)
    assert_bitwise(to_host(qd).view(np.uint8), q.view(np.uint8), "codes")
    assert_bitwise(to_host(out), orc.dequant_int8(q, sc, n_slots, S, 256, orc.BF16), "round trip")


def test_gathered_views_unflatten_the_parameters(zf):
    """Tiny MLP over 4 ranks with tail padding ((1000, 37) + the MLP): the
    views of the dequantised flat buffer are the parameters, in order."""
    shapes = [(512, 1024), (1024,), (1024, 512), (512,), (37,)]
    numels = [int(np.prod(s)) for s in shapes]
    lay = zf.zero_flat_layout(numels, 4)
    S, n_slots = lay["shard"], 4
    assert lay["pad"] > 0
    q, sc, nb = host_payload("views", n_slots, S, 256)
    out = torch.empty(lay["padded"], dtype=torch.float16, device="cuda")
    zf.zero_dequant_allgather(torch.from_numpy(q).cuda(), to_dev(sc, 0), n_slots, S, out)
    ref = orc.dequant_int8(q, sc, n_slots, S, 256, orc.F16)
    views = zf.unflatten(out, shapes, n_ranks=4)
    for (a, b), v, sh in zip(lay["spans"], views, shapes):
        assert tuple(v.shape) == sh
        assert_bitwise(to_host(v.reshape(-1)), ref[a:b], "parameter view")


# ------------------------------------------------------------------ full sizes
def gather_payload_gpu(g, dev):
    q = torch.empty(g.padded, dtype=torch.int8, device=dev)
    synth.fill_codes(q, key_codes(g))
    sc = torch.empty(g.n_ranks * g.n_blocks, device=dev)
    synth.fill_normal(sc, key_scales(g), 0, g.scale_sigma)
    sc.abs_()
    return q, sc


def test_llama7b_block_gather_full_size(zf):
    """The 7B block's flat parameter from 8 INT8 slots, every element checked."""
    g = GATHERS["llama7b_block_n8_gather"]
    say("gather", g.name, g.shard, g.padded)
    q, sc = gather_payload_gpu(g, "cuda")
    out = torch.empty(g.padded, dtype=TORCH_DT[g.out_dtype], device="cuda")
    zf.zero_dequant_allgather(q, sc, g.n_ranks, g.shard, out, block=g.block)
    qh = synth.codes(key_codes(g), 0, g.padded)
    sh = np.abs(synth.normal_f32(key_scales(g), 0, g.n_ranks * g.n_blocks, g.scale_sigma))
    assert_bitwise(to_host(q).view(np.uint8), qh.view(np.uint8), "codes (generator)")
    ref = orc.dequant_int8(qh, sh.astype(np.float32), g.n_ranks, g.shard, g.block, g.out_dtype)
    assert_bitwise(to_host(out), ref, "7B block flat parameter")
    del q, sc, out
    torch.cuda.empty_cache()


def test_gather_over_several_launches(zf):
    """A flat output of 3 x 200,000,004 elements: the vector path issues it as
    launches of 32,768 blocks (268,435,456 elements each) over consecutive
    tile ranges, three here, with slot boundaries inside tiles.  Every element
    against the oracle (codes and scales generated on the GPU, host copies
    checked against the host generator at sampled indices)."""
    n_slots, S, block = 3, 200_000_004, 256
    nb = -(-S // block)
    say("gather over launches", n_slots, S)
    q = torch.empty(n_slots * S, dtype=torch.int8, device="cuda")
    kq, ks = synth.stream_key("dq-launch", "codes"), synth.stream_key("dq-launch", "scales")
    synth.fill_codes(q, kq)
    sc = torch.empty(n_slots * nb, device="cuda")
    synth.fill_normal(sc, ks, 0, 4.7e-6)
    sc.abs_()
    out = torch.empty(n_slots * S, dtype=torch.bfloat16, device="cuda")
    zf.zero_dequant_allgather(q, sc, n_slots, S, out, block=block)
    qh, sh = to_host(q), to_host(sc).copy()
    rng = np.random.default_rng(11)
    idx = np.unique(rng.integers(0, n_slots * S, 20_000))
    assert_bitwise(qh[idx].view(np.uint8), synth.codes_at(kq, idx).view(np.uint8), "codes copy")
    sidx = np.unique(rng.integers(0, sh.size, 2_000))
    assert_bitwise(sh[sidx], np.abs(synth.normal_f32_at(ks, sidx, 4.7e-6)), "scales copy")
    ref = orc.dequant_int8(qh, sh, n_slots, S, block, orc.BF16)
    assert_bitwise(to_host(out), ref, "flat buffer over three launches")
    del q, sc, out
    torch.cuda.empty_cache()


def test_70b_n64_gather_full_size(zf):
    """The whole 70B flat parameter (7e10 bf16) from 64 slots: 2^20 random
    elements plus 2,048 elements on each side of every slot boundary and of
    every launch slice (261 launches), and the last (short) block of every
    slot, each against the oracle."""
    g = GATHERS["70b_n64_gather"]
    torch.cuda.empty_cache()
    free, _ = torch.cuda.mem_get_info()
    need = g.padded * 3 + g.n_ranks * g.n_blocks * 4
    if free < need + (4 << 30):
        pytest.skip("needs %.0f GB of free device memory, %.0f free" % (need / 1e9, free / 1e9))
    say("gather", g.name, g.shard, g.padded)
    q, sc = gather_payload_gpu(g, "cuda")
    out = torch.empty(g.padded, dtype=TORCH_DT[g.out_dtype], device="cuda")
    zf.zero_dequant_allgather(q, sc, g.n_ranks, g.shard, out, block=g.block)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    S = g.shard
    parts = [rng.integers(0, g.padded, 1 << 20)]
    slice_elems = 32768 * 4 * 2048     # the elements of one launch slice
    for b in range(slice_elems, g.padded, slice_elems):
        parts.append(np.arange(b - 2048, min(g.padded, b + 2048)))
    for s in range(g.n_ranks):
        parts.append(np.arange(max(0, s * S - 2048), min(g.padded, s * S + 2048)))
        parts.append(np.arange((s + 1) * S - (S - (g.n_blocks - 1) * g.block), (s + 1) * S))
    idx = np.unique(np.concatenate(parts)).astype(np.int64)
    slot, within = idx // S, idx % S
    sidx = slot * g.n_blocks + within // g.block
    qh = synth.codes_at(key_codes(g), idx)
    sh = np.abs(synth.normal_f32_at(key_scales(g), sidx, g.scale_sigma)).astype(np.float32)
    # one (code, scale) pair per "slot" of one element: the oracle's definition per element
    ref = orc.dequant_int8(qh, sh, idx.size, 1, 1, g.out_dtype)
    got = to_host(out[torch.from_numpy(idx).cuda()])
    assert_bitwise(got, ref, "70B flat parameter samples")
    del q, sc, out
    torch.cuda.empty_cache()
