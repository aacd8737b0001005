"""Pins of the oracle's FlatParameter layout and memory accounting.

Layout: brute force (walk every flat element), hand-derived tables, and the
invariant of the numpy 4-rank simulation on "DeepSpeed 与 FSDP" ("用 numpy 模拟
ZeRO 分片过程"): concatenating the shards gives back the flat tensor.
Accounting: the per-GPU figures the pages print (tests/golden/memory_accounting.json).
"""
import json
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "memory_accounting.json")

TINY = [512 * 1024, 1024, 1024 * 512, 512]               # 2-layer MLP, 1,050,112 params
LLAMA_BLOCK = [4096 * 4096] * 4 + [11008 * 4096, 11008 * 4096, 4096 * 11008, 4096, 4096]


def brute_segments(numels, n_ranks, align, rank):
    """Element-by-element construction: label every flat element with
    (param, offset), pad the tail to N equal shards, cut rank's shard into
    maximal runs."""
    total = sum(numels)
    shard = -(-total // n_ranks) if total else 0
    shard = -(-shard // align) * align
    labels = []
    for j, n in enumerate(numels):
        labels += [(j, k) for k in range(n)]
    labels += [(-1, k) for k in range(shard * n_ranks - total)]
    mine = labels[rank * shard:(rank + 1) * shard]
    segs = []
    for pos, (j, k) in enumerate(mine):
        if segs and segs[-1][0] == j and segs[-1][1] + segs[-1][3] == k:
            segs[-1][3] += 1
        else:
            segs.append([j, k, pos, 1])
    return shard, [tuple(s) for s in segs]


def test_layout_brute_force(orc):
    rng = np.random.default_rng(3)
    for _ in range(300):
        n_params = int(rng.integers(0, 6))
        numels = [int(x) for x in rng.integers(0, 9, size=n_params)]
        n_ranks = int(rng.integers(1, 9))
        align = int(rng.choice([1, 1, 2, 4]))
        for rank in range(n_ranks):
            shard, segs = brute_segments(numels, n_ranks, align, rank)
            lay = orc.layout(numels, n_ranks, align, rank)
            assert lay["shard"] == shard
            assert lay["segments"] == segs, (numels, n_ranks, align, rank)


@pytest.mark.parametrize("numels,n_ranks,shard,rank,segs", [
    # 10 elements over 4 ranks: S=3, rank 3 holds 1 real element and 2 padding
    ([10], 4, 3, 3, [(0, 9, 0, 1), (-1, 0, 1, 2)]),
    # 7 over 8: S=1, rank 7 is all padding (torch.chunk would give only 7 chunks)
    ([7], 8, 1, 7, [(-1, 0, 0, 1)]),
    # [3, 5] over 3: S=3, rank 2 = p1[3:5] + 1 padding
    ([3, 5], 3, 3, 2, [(1, 3, 0, 2), (-1, 0, 2, 1)]),
    # the 2-layer MLP over 4 ranks (no padding): shards straddle parameters
    (TINY, 4, 262528, 0, [(0, 0, 0, 262528)]),
    (TINY, 4, 262528, 1, [(0, 262528, 0, 261760), (1, 0, 261760, 768)]),
    (TINY, 4, 262528, 2, [(1, 768, 0, 256), (2, 0, 256, 262272)]),
    (TINY, 4, 262528, 3, [(2, 262272, 0, 262016), (3, 0, 262016, 512)]),
    # one Llama-style 7B block (q,k,v,o, gate, up, down, 2 norms) over 8 ranks:
    # rank 3's shard [75,893,760, 101,191,680) lies inside `gate`
    (LLAMA_BLOCK, 8, 25297920, 3, [(4, 8784896, 0, 25297920)]),
])
def test_layout_hand_tables(orc, numels, n_ranks, shard, rank, segs):
    lay = orc.layout(numels, n_ranks, 1, rank)
    assert lay["shard"] == shard
    assert lay["segments"] == segs


def test_tiny_totals(orc):
    lay = orc.layout(TINY, 4, 1, 0)
    assert lay["total"] == 1050112 and lay["padded"] == 1050112 and lay["pad"] == 0
    assert lay["starts"] == [0, 524288, 525312, 1049600]
    assert lay["ends"] == [524288, 525312, 1049600, 1050112]
    blk = orc.layout(LLAMA_BLOCK, 8, 1, 3)
    assert blk["total"] == 202383360


def test_concat_of_shards_is_flat(orc):
    """numpy simulation invariant: np.concatenate(shards) equals the original."""
    rng = np.random.default_rng(5)
    numels = [37, 1, 0, 250, 13]
    flat = rng.standard_normal(sum(numels)).astype(np.float32)
    params = np.split(flat, np.cumsum(numels)[:-1])
    for n_ranks in (1, 2, 3, 4, 7, 8, 64):
        lay0 = orc.layout(numels, n_ranks, 1, 0)
        shards = []
        for r in range(n_ranks):
            lay = orc.layout(numels, n_ranks, 1, r)
            sh = np.full(lay["shard"], np.nan, np.float32)
            for j, off_p, off_s, ln in lay["segments"]:
                sh[off_s:off_s + ln] = 0.0 if j < 0 else params[j][off_p:off_p + ln]
            assert not np.isnan(sh).any()
            shards.append(sh)
        cat = np.concatenate(shards)
        assert cat.size == lay0["padded"]
        assert np.array_equal(cat[:flat.size], flat)
        assert np.all(cat[flat.size:] == 0)


def test_layout_rejects_bad_input(orc):
    with pytest.raises(ValueError):
        orc.layout([4], 0, 1, 0)
    with pytest.raises(ValueError):
        orc.layout([4], 2, 1, 2)
    with pytest.raises(ValueError):
        orc.layout([-1], 2, 1, 0)


def _acct(orc, case):
    lay = orc.layout([case["total"]], case["n_ranks"], 1, 0)
    return orc.accounting(lay["total"], lay["shard"], case["P"], case["G"], case["K"])


def test_accounting_printed_values(orc):
    g = json.load(open(GOLDEN))
    for case in g["cases"]:
        assert _acct(orc, case)[case["field"]] == case["bytes"], case["cite"]


def test_accounting_printed_ratios(orc):
    g = json.load(open(GOLDEN))
    for case in g["ratios"]:
        a = _acct(orc, case)
        if case.get("den"):
            red = 100.0 * (1.0 - a[case["num"]] / a[case["den"]])
            assert abs(red - case["reduction_pct"]) <= case["abs_tol_pct"], case["cite"]
        else:
            assert a[case["num"]] * case["n_ranks"] == case["times_ranks_bytes"], case["cite"]


def test_accounting_stage_formula_limits(orc):
    """'ZeRO-3 的数学总结': with N=1 every stage equals pure DP; ZeRO-3 is
    (P+G+K)*Psi/N exactly when N divides Psi."""
    for P, G, K in ((2, 2, 12), (2, 2, 8), (4, 4, 8)):
        a = orc.accounting(1000, 1000, P, G, K)
        assert a["dp"] == a["z1"] == a["z2"] == a["z3"] == (P + G + K) * 1000
        a = orc.accounting(1000, 125, P, G, K)
        assert a["z3"] * 8 == a["dp"]
