"""Pins for the fp64 oracle against facts fixed by the pages and by mathematics.

None of these tests re-types an oracle formula: each compares the oracle with a
hand-derived value, a closed form, a brute-force search over tiny inputs, or an
independent library routine (torch's CPU scaled_dot_product_attention and
logsumexp, scipy's softmax).
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _sdpa(q, k, v, scale):
    """Reference attention and natural-log LSE from torch (fp64, CPU)."""
    q = torch.as_tensor(q, dtype=torch.float64)
    k = torch.as_tensor(k, dtype=torch.float64)
    v = torch.as_tensor(v, dtype=torch.float64)
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=scale)
    lse = torch.logsumexp(scale * (q @ k.transpose(-1, -2)), dim=-1)
    return o.numpy(), lse.numpy()


# --------------------------------------------------------------------------
# pooling and similarity
# --------------------------------------------------------------------------

def test_pool_golden_cases():
    cases = json.load(open(os.path.join(GOLDEN, "pool_cases.json")))["cases"]
    for c in cases:
        x = np.array(c["tokens"], dtype=np.float64)
        means, sims, flags = oracle.pool_and_gate(x, x.shape[0], 0.001)
        assert np.allclose(means[0], c["mean"], atol=1e-15), c["name"]
        assert abs(sims[0] - c["sim"]) < 1e-15, c["name"]
        assert bool(flags[0]) == (c["sim"] > 0.001), c["name"]


def test_sim_equals_brute_force_mean_cosine():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((64, 32))
    x[7] = 0.0
    unit = np.array([r / np.linalg.norm(r) if np.linalg.norm(r) > 0 else r for r in x])
    brute = np.mean([[float(unit[i] @ unit[j]) for j in range(64)] for i in range(64)])
    assert abs(oracle.block_self_similarity(x) - brute) < 1e-12


def test_one_hot_block_similarity_is_one_over_n():
    x = np.eye(64)
    assert oracle.block_self_similarity(x) == pytest.approx(1.0 / 64, abs=1e-15)


def test_gate_is_strict_greater():
    x = np.eye(4)            # sim = 0.25 exactly
    _, _, flags = oracle.pool_and_gate(x, 4, 0.25)
    assert not flags[0]
    _, _, flags = oracle.pool_and_gate(x, 4, 0.2499)
    assert flags[0]


def test_random_tokens_similarity_near_one_over_n():
    rng = np.random.default_rng(0)
    vals = [oracle.block_self_similarity(rng.standard_normal((64, 128))) for _ in range(50)]
    assert 0.008 < min(vals) and max(vals) < 0.03


def test_pool_partial_block_pools_its_own_tokens():
    # 65 tokens: a full block of ones and a one-token block of twos (reading R1).
    x = np.ones((65, 4))
    x[64] = [2.0, -2.0, 0.0, 0.0]
    means, sims, flags = oracle.pool_and_gate(x, 64, 0.999)
    assert means.shape == (2, 4)
    assert np.array_equal(means[1], [2.0, -2.0, 0.0, 0.0])
    assert abs(sims[1] - 1.0) < 1e-15 and flags[1]


# --------------------------------------------------------------------------
# pooled scores and softmax
# --------------------------------------------------------------------------

def test_pooled_scores_exact_integers_and_mask():
    qbar = np.array([[1.0, 2.0, 0.0, -1.0], [0.0, 1.0, 1.0, 1.0]])
    kbar = np.array([[2.0, 0.0, 1.0, 1.0], [1.0, 1.0, 1.0, 1.0], [0.0, 0.0, 0.0, 4.0]])
    # d = 4 -> scale 1/2; hand products: row0: 1, 2, -4 ; row1: 2, 3, 4
    s = oracle.pooled_scores(qbar, kbar, np.array([True, True, True]), 0.5)
    assert np.array_equal(s, np.array([[0.5, 1.0, -2.0], [1.0, 1.5, 2.0]]))
    s = oracle.pooled_scores(qbar, kbar, np.array([True, False, True]), 0.5)
    assert s[0, 1] == -math.inf and s[1, 1] == -math.inf and s[1, 2] == 2.0


def test_softmax_matches_scipy_and_handles_all_masked():
    from scipy.special import softmax
    rng = np.random.default_rng(1)
    s = rng.standard_normal((3, 7)) * 5
    s[1, 2] = -math.inf
    p = oracle.row_softmax(s)
    ref = softmax(np.where(np.isinf(s), -1e300, s), axis=1)
    assert np.allclose(p, ref, rtol=1e-13, atol=1e-300)
    assert p[1, 2] == 0.0
    z = oracle.row_softmax(np.full((1, 5), -math.inf))
    assert np.array_equal(z, np.zeros((1, 5)))


# --------------------------------------------------------------------------
# selection
# --------------------------------------------------------------------------

def test_selection_golden_cases():
    cases = json.load(open(os.path.join(GOLDEN, "selection_cases.json")))["cases"]
    for c in cases:
        sel = oracle.select_row(np.array(c["prob"], dtype=np.float64), c["sim_q"],
                                np.array(c["sim_k"], dtype=bool), c["topk"], c["cdf"])
        assert list(sel) == c["expect"], c["name"]


@pytest.mark.parametrize("topk,nk,expect", [
    (0.1, 256, 25), (0.2, 256, 51), (0.4, 256, 102), (0.6, 256, 153), (0.8, 256, 204),
    (0.4, 64, 25), (1.0, 64, 64), (0.5, 8, 4), (0.001, 8, 1), (1.0, 1, 1)])
def test_topk_counts_at_workload_sizes(topk, nk, expect):
    # floor(float32(topk) * nk), clamped to [1, nk]: worked out by hand for each row
    assert oracle.topk_count(topk, nk) == expect


def _brute_force_topk(prob, n):
    """Among all n-subsets with the largest exact probability sum, the one whose
    sorted index tuple is lexicographically smallest (= lower index wins ties)."""
    fr = [Fraction(p) for p in prob]
    best = None
    for sub in itertools.combinations(range(len(prob)), n):
        key = (-sum(fr[i] for i in sub), sub)
        if best is None or key < best:
            best = key
    return list(best[1])


def test_topk_selection_against_brute_force_with_ties():
    rng = np.random.default_rng(2)
    for trial in range(300):
        nk = int(rng.integers(2, 9))
        levels = rng.integers(0, 4, size=nk).astype(np.float64)   # many ties
        prob = levels / 8.0
        n = int(rng.integers(1, nk + 1))
        topk = n / nk + 1e-6
        assert oracle.topk_count(topk, nk) == n
        sel = oracle.select_row(prob, True, np.ones(nk, bool), topk, None)
        assert list(sel) == _brute_force_topk(prob, n), (prob, n)


def test_rank_formula():
    rng = np.random.default_rng(3)
    for _ in range(200):
        nk = 12
        prob = rng.integers(0, 5, size=nk) / 16.0
        n = int(rng.integers(1, nk + 1))
        sel = set(oracle.select_row(prob, True, np.ones(nk, bool), n / nk + 1e-6, None))
        for kb in range(nk):
            rank = sum(1 for j in range(nk) if prob[j] > prob[kb] or (prob[j] == prob[kb] and j < kb))
            assert (kb in sel) == (rank < n)


def test_cdf_dyadic_boundaries():
    prob = np.array([2.0 ** -(i + 1) for i in range(10)])
    prob[-1] *= 2                                       # sums to exactly 1
    order = oracle.selection_order(prob)
    for n in range(1, 11):
        exact = float(sum(Fraction(p) for p in prob[:n]))
        assert oracle.cdf_count(prob, order, exact) == n
    assert oracle.cdf_count(prob, order, 0.0) == 1


def test_selection_rows_are_ascending_and_lut_encoding():
    rows = [np.array([1, 3]), np.array([], dtype=np.int64), np.array([0, 1, 2, 3])]
    lut, count, bm = oracle.lut_from_selection(rows, 4)
    assert lut.tolist() == [[1, 3, -1, -1], [-1, -1, -1, -1], [0, 1, 2, 3]]
    assert count.tolist() == [2, 0, 4]
    assert bm.tolist() == [[0, 1, 0, 1], [0, 0, 0, 0], [1, 1, 1, 1]]


def test_block_map_gate_on_hand_built_tiles():
    # d = 4, blocks of 4 tokens.  Q block 1 and K block 2 are +-v pairs (sim 0).
    d, blk = 4, 4
    same = np.tile(np.array([[1.0, 0.5, 0.0, 0.0]]), (blk, 1))
    pm = np.array([[1.0, 1.0, 0.0, 0.0], [-1.0, -1.0, 0.0, 0.0],
                   [0.0, 0.0, 1.0, 0.0], [0.0, 0.0, -1.0, 0.0]])
    q = np.concatenate([same, pm, same * 2.0])[None, None]
    k = np.concatenate([same, same * -1.0, pm, same * 3.0])[None, None]
    bm = oracle.block_map(q, k, topk=[0.25], simthreshd1=[0.001], blk_q=blk, blk_k=blk)
    assert bm["sim_q"][0, 0].tolist() == [True, False, True]
    assert bm["sim_k"][0, 0].tolist() == [True, True, False, True]
    assert bm["prob"][0, 0, 0, 2] == 0.0
    # topk 0.25 of 4 -> 1 block, plus the forced K block 2; Q block 1 takes all.
    assert bm["count"][0, 0].tolist() == [2, 4, 2]
    assert bm["lut"][0, 0, 1].tolist() == [0, 1, 2, 3]
    for qb in (0, 2):
        row = bm["lut"][0, 0, qb, :2].tolist()
        assert 2 in row
        # the largest pooled score among K blocks 0, 1, 3 is block 3 (3x the mean)
        assert row == [2, 3]


# --------------------------------------------------------------------------
# attention
# --------------------------------------------------------------------------

def test_attend_hand_example():
    q = np.array([[1.0, 0.0]])
    k = np.array([[1.0, 0.0], [0.0, 0.0]])
    v = np.array([[1.0, 0.0], [0.0, 1.0]])
    o, lse = oracle.attend(q, k, v, 1.0)
    e = math.e
    assert np.allclose(o, [[e / (1 + e), 1 / (1 + e)]], atol=1e-15)
    assert abs(lse[0] - math.log(1 + e)) < 1e-15


def test_full_lut_equals_sdpa():
    rng = np.random.default_rng(4)
    b, hq, hkv, s, d = 1, 4, 2, 256, 32
    q = rng.standard_normal((b, hq, s, d))
    k = rng.standard_normal((b, hkv, s, d))
    v = rng.standard_normal((b, hkv, s, d))
    nq = nk = s // 64
    lut = np.tile(np.arange(nk, dtype=np.int32), (b, hq, nq, 1))
    count = np.full((b, hq, nq), nk, dtype=np.int32)
    o, lse = oracle.block_sparse_attention(q, k, v, lut, count, 64, 64)
    kk = np.repeat(k, hq // hkv, axis=1)
    vv = np.repeat(v, hq // hkv, axis=1)
    ro, rl = _sdpa(q, kk, vv, 1 / math.sqrt(d))
    assert np.abs(o - ro).max() < 1e-12
    assert np.abs(lse - rl).max() < 1e-12
    o2, l2 = oracle.block_sparse_attention(q, k, v, None, None, 64, 64)
    assert np.abs(o2 - ro).max() < 1e-12 and np.abs(l2 - rl).max() < 1e-12


def test_topk_one_block_map_equals_dense():
    rng = np.random.default_rng(6)
    b, h, s, d = 1, 2, 256, 16
    q = rng.standard_normal((b, h, s, d))
    k = rng.standard_normal((b, h, s, d))
    v = rng.standard_normal((b, h, s, d))
    bm = oracle.block_map(q, k, topk=[1.0, 1.0], simthreshd1=[0.001, 0.001])
    assert (bm["count"] == s // 64).all()
    o, lse = oracle.block_sparse_attention(q, k, v, bm["lut"], bm["count"])
    ro, rl = _sdpa(q, k, v, 1 / math.sqrt(d))
    assert np.abs(o - ro).max() < 1e-12 and np.abs(lse - rl).max() < 1e-12


def test_sparse_rows_equal_sdpa_over_gathered_keys():
    rng = np.random.default_rng(7)
    b, h, s, d = 1, 1, 512, 16
    q = rng.standard_normal((b, h, s, d))
    k = rng.standard_normal((b, h, s, d))
    v = rng.standard_normal((b, h, s, d))
    lut = np.full((1, 1, 8, 8), -1, np.int32)
    count = np.zeros((1, 1, 8), np.int32)
    picks = [[0], [1, 5], [2, 3, 7], [6], [0, 4], [1, 2, 3, 4, 5], [7], [3]]
    for r, p in enumerate(picks):
        lut[0, 0, r, :len(p)] = p
        count[0, 0, r] = len(p)
    o, lse = oracle.block_sparse_attention(q, k, v, lut, count)
    for r, p in enumerate(picks):
        idx = np.concatenate([np.arange(64) + 64 * kb for kb in p])
        ro, rl = _sdpa(q[0, 0, 64 * r:64 * r + 64], k[0, 0, idx], v[0, 0, idx], 0.25)
        assert np.abs(o[0, 0, 64 * r:64 * r + 64] - ro).max() < 1e-12
        assert np.abs(lse[0, 0, 64 * r:64 * r + 64] - rl).max() < 1e-12


def test_zero_query_closed_form():
    rng = np.random.default_rng(8)
    b, h, s, d = 1, 1, 256, 8
    q = np.zeros((b, h, s, d))
    k = rng.standard_normal((b, h, s, d))
    v = rng.standard_normal((b, h, s, d))
    lut = np.array([[[[1, 3, -1, -1], [0, -1, -1, -1], [0, 1, 2, 3], [2, -1, -1, -1]]]], np.int32)
    count = np.array([[[2, 1, 4, 1]]], np.int32)
    o, lse = oracle.block_sparse_attention(q, k, v, lut, count)
    for r in range(4):
        blocks = lut[0, 0, r, :count[0, 0, r]]
        rows = np.concatenate([v[0, 0, 64 * kb:64 * kb + 64] for kb in blocks])
        assert np.abs(o[0, 0, 64 * r:64 * r + 64] - rows.mean(axis=0)).max() < 1e-13
        assert np.allclose(lse[0, 0, 64 * r:64 * r + 64], math.log(64 * len(blocks)), atol=1e-14)


def test_empty_row_gives_zero_and_minus_inf():
    rng = np.random.default_rng(9)
    q = rng.standard_normal((1, 1, 128, 8))
    k = rng.standard_normal((1, 1, 128, 8))
    v = rng.standard_normal((1, 1, 128, 8))
    lut = np.array([[[[-1, -1], [1, -1]]]], np.int32)
    count = np.array([[[0, 1]]], np.int32)
    o, lse = oracle.block_sparse_attention(q, k, v, lut, count)
    assert (o[0, 0, :64] == 0).all() and (lse[0, 0, :64] == -math.inf).all()
    assert np.isfinite(lse[0, 0, 64:]).all()


def test_lut_order_does_not_matter():
    rng = np.random.default_rng(10)
    q = rng.standard_normal((1, 1, 64, 16))
    k = rng.standard_normal((1, 1, 512, 16))
    v = rng.standard_normal((1, 1, 512, 16))
    a = np.array([[[[0, 2, 5, 7, -1, -1, -1, -1]]]], np.int32)
    bperm = np.array([[[[7, 0, 5, 2, -1, -1, -1, -1]]]], np.int32)
    c = np.array([[[4]]], np.int32)
    o1, l1 = oracle.block_sparse_attention(q, k, v, a, c)
    o2, l2 = oracle.block_sparse_attention(q, k, v, bperm, c)
    assert np.abs(o1 - o2).max() < 1e-12 and np.abs(l1 - l2).max() < 1e-12


def test_gqa_head_mapping():
    # KV head j holds V rows all equal to j; query head i must read KV head i // 4.
    b, hq, hkv, s, d = 1, 8, 2, 128, 4
    rng = np.random.default_rng(11)
    q = rng.standard_normal((b, hq, s, d))
    k = rng.standard_normal((b, hkv, s, d))
    v = np.stack([np.full((s, d), float(j)) for j in range(hkv)])[None]
    o, _ = oracle.block_sparse_attention(q, k, v, None, None)
    for i in range(hq):
        assert np.allclose(o[0, i], i // 4, atol=1e-13)
    lists = np.tile(np.arange(0, s, 3, dtype=np.int32), (b, hkv, 1))
    o2, _ = oracle.token_list_attention(q[:, :, :1], k, v, lists)
    for i in range(hq):
        assert np.allclose(o2[0, i], i // 4, atol=1e-13)


@pytest.mark.parametrize("ratio", [1, 2, 4])
def test_dense_attention_is_sdpa_on_expanded_kv_heads(ratio):
    # aiter 6841 page: query head j reads KV head j // ratio.  Every KV head
    # holds different keys and values, so a wrong head map (j % h_kv, or no
    # map) gives a different result; torch's SDPA over K/V with each head
    # repeated for its query heads is the independent routine.
    rng = np.random.default_rng(30 + ratio)
    b, hkv, s_q, s_k, d = 2, 3, 70, 130, 16
    q = rng.standard_normal((b, hkv * ratio, s_q, d))
    k = rng.standard_normal((b, hkv, s_k, d))
    v = rng.standard_normal((b, hkv, s_k, d))
    o, lse = oracle.dense_attention(q, k, v)
    kk = np.repeat(k, ratio, axis=1)
    vv = np.repeat(v, ratio, axis=1)
    ro, rl = _sdpa(q, kk, vv, 1 / math.sqrt(d))
    assert np.abs(o - ro).max() < 1e-12
    assert np.abs(lse - rl).max() < 1e-12
    o2, l2 = oracle.dense_attention(q, k, v, scale=0.3)
    ro2, rl2 = _sdpa(q, kk, vv, 0.3)
    assert np.abs(o2 - ro2).max() < 1e-12 and np.abs(l2 - rl2).max() < 1e-12


def test_token_lists_skip_minus_one_and_match_sdpa():
    rng = np.random.default_rng(12)
    b, hq, hkv, s, d = 2, 4, 2, 300, 16
    q = rng.standard_normal((b, hq, 1, d))
    k = rng.standard_normal((b, hkv, s, d))
    v = rng.standard_normal((b, hkv, s, d))
    lists = np.full((b, hkv, 40), -1, np.int32)
    for ib in range(b):
        for j in range(hkv):
            pos = np.sort(rng.choice(s, size=30, replace=False))
            lists[ib, j, :30] = pos
            lists[ib, j, 5] = -1                   # a hole inside the list
    lists[1, 1, :] = -1                             # an empty list
    o, lse = oracle.token_list_attention(q, k, v, lists)
    for ib in range(b):
        for i in range(hq):
            j = i // 2
            idx = lists[ib, j][lists[ib, j] >= 0]
            if len(idx) == 0:
                assert (o[ib, i] == 0).all() and lse[ib, i, 0] == -math.inf
                continue
            ro, rl = _sdpa(q[ib, i], k[ib, j, idx], v[ib, j, idx], 0.25)
            assert np.abs(o[ib, i] - ro).max() < 1e-12
            assert abs(lse[ib, i, 0] - rl[0]) < 1e-12


# --------------------------------------------------------------------------
# combine
# --------------------------------------------------------------------------

SPLITS = ["interleaved", "spec_heavy", "miss_heavy", "contiguous_miss"]


def _split(name, nblk, rng):
    blocks = np.arange(nblk)
    if name == "interleaved":
        a = blocks[::2]
    elif name == "spec_heavy":
        a = blocks[: (3 * nblk) // 4]
    elif name == "miss_heavy":
        a = blocks[: nblk // 4]
    else:
        a = np.concatenate([blocks[: nblk // 3], blocks[(2 * nblk) // 3:]])
    b = np.setdiff1d(blocks, a)
    return a, b


@pytest.mark.parametrize("seqlen_q", [1, 4, 16])
@pytest.mark.parametrize("block", [32, 64, 128])
@pytest.mark.parametrize("split", SPLITS)
def test_combine_identity(seqlen_q, block, split):
    rng = np.random.default_rng(seqlen_q * 1000 + block + len(split))
    d, nblk = 32, 8
    q = rng.standard_normal((seqlen_q, d))
    k = rng.standard_normal((nblk * block, d))
    v = rng.standard_normal((nblk * block, d))
    a, b = _split(split, nblk, rng)
    ia = np.concatenate([np.arange(block) + block * x for x in a])
    ib = np.concatenate([np.arange(block) + block * x for x in b])
    scale = 1 / math.sqrt(d)
    oa, la = oracle.attend(q, k[ia], v[ia], scale)
    ob, lb = oracle.attend(q, k[ib], v[ib], scale)
    o, l = oracle.combine([oa, ob], [la, lb])
    ro, rl = _sdpa(q, k, v, scale)
    assert np.abs(o - ro).max() < 1e-10 and np.abs(l - rl).max() < 1e-10
    o2, l2 = oracle.combine([ob, oa], [lb, la])
    assert np.abs(o2 - o).max() < 1e-12 and np.abs(l2 - l).max() < 1e-12


def test_combine_empty_partials():
    rng = np.random.default_rng(13)
    o1 = rng.standard_normal((5, 8))
    l1 = rng.standard_normal(5)
    oe = np.zeros((5, 8))
    le = np.full(5, -math.inf)
    o, l = oracle.combine([o1, oe], [l1, le])
    assert np.array_equal(o, o1) and np.array_equal(l, l1)
    o, l = oracle.combine([oe, o1], [le, l1])
    assert np.array_equal(o, o1) and np.array_equal(l, l1)
    o, l = oracle.combine([oe, oe], [le, le])
    assert (o == 0).all() and (l == -math.inf).all()


def test_combine_many_parts_matches_sdpa():
    rng = np.random.default_rng(14)
    q = rng.standard_normal((3, 16))
    k = rng.standard_normal((700, 16))
    v = rng.standard_normal((700, 16))
    cuts = [0, 13, 200, 201, 450, 700]
    parts = [oracle.attend(q, k[a:b], v[a:b], 0.25) for a, b in zip(cuts[:-1], cuts[1:])]
    parts.append(oracle.attend(q, k[:0], v[:0], 0.25))          # an empty split
    o, l = oracle.combine([p[0] for p in parts], [p[1] for p in parts])
    ro, rl = _sdpa(q, k, v, 0.25)
    assert np.abs(o - ro).max() < 1e-12 and np.abs(l - rl).max() < 1e-12
