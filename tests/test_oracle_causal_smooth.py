"""Pins for the oracle's causal mode, attention sink and K smoothing (CPU).

These options are the CK page's not-yet-ported items ("Sparge Attention
(Composable Kernel)" page, "Status vs Upstream"): the is_causal mask in the
pooled score, attention_sink (column 0 forced on) and K smoothing (the
pre-pool k -= km).  Each pin checks the oracle against something other than
its own formulas: torch's scaled_dot_product_attention with is_causal=True,
closed forms, hand-derived selections and invariances.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# ----------------------------------------------------------------------------
# causal attention
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("s,d,seed", [(128, 16, 0), (192, 32, 1)])
def test_causal_dense_attention_matches_sdpa(s, d, seed):
    q, k, v = _rand((1, 2, s, d), seed), _rand((1, 2, s, d), seed + 10), _rand((1, 2, s, d), seed + 20)
    o, lse = oracle.block_sparse_attention(q, k, v, None, None, causal=True)
    qt, kt, vt = (torch.from_numpy(x) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
    np.testing.assert_allclose(o, ref.numpy(), atol=1e-12, rtol=1e-12)
    # LSE of row i = logsumexp over keys 0..i, from torch's own logsumexp
    scale = 1.0 / math.sqrt(d)
    scores = torch.einsum("bhid,bhjd->bhij", qt, kt) * scale
    mask = torch.ones(s, s, dtype=torch.bool).tril()
    ref_lse = torch.logsumexp(scores.masked_fill(~mask, float("-inf")), dim=-1)
    np.testing.assert_allclose(lse, ref_lse.numpy(), atol=1e-12, rtol=1e-12)


def test_causal_full_selection_equals_causal_sdpa():
    s, d = 256, 16
    q, k, v = _rand((1, 2, s, d), 3), _rand((1, 2, s, d), 4), _rand((1, 2, s, d), 5)
    bm = oracle.block_map(q, k, [1.0, 1.0], [-1.0, -1.0], causal=True)
    nq = s // 64
    for qb in range(nq):
        assert list(bm["lut"][0, 0, qb, :bm["count"][0, 0, qb]]) == list(range(qb + 1))
    o, _ = oracle.block_sparse_attention(q, k, v, bm["lut"], bm["count"], causal=True)
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(x) for x in (q, k, v)), is_causal=True)
    np.testing.assert_allclose(o, ref.numpy(), atol=1e-12, rtol=1e-12)


def test_causal_block_past_the_tile_contributes_nothing():
    # A LUT row that lists a block in the tile's future: causal attention must
    # equal attention over the same row without that block.
    s, d = 192, 8
    q, k, v = _rand((1, 1, s, d), 6), _rand((1, 1, s, d), 7), _rand((1, 1, s, d), 8)
    lut = np.array([[[[0, 1, 2], [0, 1, 2], [0, 1, 2]]]], dtype=np.int32)
    cnt = np.array([[[3, 3, 3]]], dtype=np.int32)
    lut2 = np.array([[[[0, -1, -1], [0, 1, -1], [0, 1, 2]]]], dtype=np.int32)
    cnt2 = np.array([[[1, 2, 3]]], dtype=np.int32)
    o1, l1 = oracle.block_sparse_attention(q, k, v, lut, cnt, causal=True)
    o2, l2 = oracle.block_sparse_attention(q, k, v, lut2, cnt2, causal=True)
    # equal up to summation order (the masked keys are zero terms in one sum)
    np.testing.assert_allclose(o1, o2, atol=1e-14, rtol=0)
    np.testing.assert_allclose(l1, l2, atol=1e-14, rtol=0)


def test_row_with_no_allowed_key_is_empty():
    # Query rows whose only listed block lies in their future: O = 0, LSE = -inf.
    s, d = 128, 4
    q, k, v = _rand((1, 1, s, d), 9), _rand((1, 1, s, d), 10), _rand((1, 1, s, d), 11)
    lut = np.array([[[[1], [1]]]], dtype=np.int32)
    cnt = np.array([[[1, 1]]], dtype=np.int32)
    o, lse = oracle.block_sparse_attention(q, k, v, lut, cnt, causal=True)
    assert np.all(o[0, 0, :64] == 0.0) and np.all(lse[0, 0, :64] == -np.inf)
    assert np.all(np.isfinite(lse[0, 0, 64:]))


# ----------------------------------------------------------------------------
# causal selection and attention sink
# ----------------------------------------------------------------------------

def test_causal_pooled_scores_mask_future_blocks():
    qbar, kbar = _rand((4, 8), 12), _rand((4, 8), 13)
    s = oracle.pooled_scores(qbar, kbar, np.ones(4, bool), 0.5, causal=True)
    for qb in range(4):
        for kb in range(4):
            assert (s[qb, kb] == -np.inf) == (kb > qb)


@pytest.mark.parametrize("prob,valid,topk,expect", [
    # nk = 4, top-k 0.75 -> n = 3, clamped to the 2 valid blocks
    ([0.5, 0.5, 0.0, 0.0], [1, 1, 0, 0], 0.75, [0, 1]),
    # n = 2 of 3 valid blocks: the two largest
    ([0.25, 0.5, 0.25, 0.0], [1, 1, 1, 0], 0.5, [0, 1]),
    # a valid block with probability 0 is still taken before any invalid one
    ([1.0, 0.0, 0.0, 0.0], [1, 1, 0, 0], 0.75, [0, 1]),
])
def test_causal_select_row_hand_cases(prob, valid, topk, expect):
    row = oracle.select_row(np.array(prob), True, np.ones(4, bool), topk, None,
                            np.array(valid, bool))
    assert list(row) == expect


def test_causal_forced_blocks_respect_the_mask():
    # K block 3 fails the gate but lies in the future of tile 1: not forced.
    sim_k = np.array([True, True, True, False])
    row = oracle.select_row(np.array([0.75, 0.25, 0.0, 0.0]), True, sim_k, 0.25, None,
                            np.array([1, 1, 0, 0], bool))
    assert list(row) == [0]
    # a Q block that fails the gate selects every valid block
    row = oracle.select_row(np.array([0.75, 0.25, 0.0, 0.0]), False, sim_k, 0.25, None,
                            np.array([1, 1, 0, 0], bool))
    assert list(row) == [0, 1]


def test_attention_sink_forces_block_zero():
    row = oracle.select_row(np.array([0.0, 0.1, 0.9, 0.0]), True, np.ones(4, bool), 0.25, None,
                            None, attention_sink=True)
    assert list(row) == [0, 2]
    q, k = _rand((1, 2, 512, 16), 14), _rand((1, 2, 512, 16), 15)
    bm = oracle.block_map(q, k, [0.125, 0.125], [-1.0, -1.0], causal=True, attention_sink=True)
    for h in range(2):
        for qb in range(8):
            sel = bm["lut"][0, h, qb, :bm["count"][0, h, qb]]
            assert sel[0] == 0 and np.all(sel <= qb) and np.all(np.diff(sel) > 0)


def test_causal_block_map_properties():
    q, k = _rand((1, 2, 512, 16), 16), _rand((1, 2, 512, 16), 17)
    bm = oracle.block_map(q, k, [0.5, 0.25], [-1.0, -1.0], causal=True)
    nk = 8
    for h, topk in enumerate([0.5, 0.25]):
        n = oracle.topk_count(topk, nk)
        for qb in range(8):
            c = bm["count"][0, h, qb]
            assert c == min(n, qb + 1)
            assert np.all(bm["lut"][0, h, qb, :c] <= qb)
            assert np.all(bm["prob"][0, h, qb, qb + 1:] == 0.0)


# ----------------------------------------------------------------------------
# K smoothing
# ----------------------------------------------------------------------------

def test_smoothed_keys_have_zero_mean_and_shifted_block_means():
    k = _rand((2, 3, 256, 16), 18) + 5.0
    ks = oracle.smooth_keys(k)
    np.testing.assert_allclose(ks.mean(axis=2), 0.0, atol=1e-12)
    km = k.mean(axis=2)
    for b in range(2):
        for h in range(3):
            raw, _, _ = oracle.pool_and_gate(k[b, h], 64, 0.0)
            sm, _, _ = oracle.pool_and_gate(ks[b, h], 64, 0.0)
            np.testing.assert_allclose(sm, raw - km[b, h], atol=1e-12)


def test_smoothing_flips_the_gate_of_a_plus_minus_block():
    # Every block holds c + v and c - v in equal numbers (c the same for all
    # blocks, |c| >> |v|).  Raw tokens all point near c: sim close to 1.  After
    # smoothing the tokens are +v and -v: their unit vectors cancel, sim = 0.
    d, n = 8, 64
    c = np.zeros(d); c[0] = 100.0
    v = np.zeros(d); v[1] = 1.0
    blk = np.stack([c + v if i % 2 == 0 else c - v for i in range(n)])
    k = np.concatenate([blk, blk])[None, None]              # [1, 1, 128, d]
    q = np.ones((1, 1, 128, d))
    raw = oracle.block_map(q, k, [1.0], [0.5])
    sm = oracle.block_map(q, k, [1.0], [0.5], smooth_k=True)
    np.testing.assert_allclose(raw["sim_k_val"], 1.0 - 1e-4, atol=2e-4)
    np.testing.assert_allclose(sm["sim_k_val"], 0.0, atol=1e-15)
    assert raw["sim_k"].all() and not sm["sim_k"].any()


def test_smoothing_shift_leaves_pooled_softmax_unchanged():
    # With every gate open, smoothing shifts each pooled row by a constant
    # (scale * qbar . km), which the softmax removes.
    q, k = _rand((1, 2, 512, 16), 19), _rand((1, 2, 512, 16), 20) + 2.0
    raw = oracle.block_map(q, k, [0.25, 0.5], [-1.0, -1.0])
    sm = oracle.block_map(q, k, [0.25, 0.5], [-1.0, -1.0], smooth_k=True)
    np.testing.assert_allclose(sm["prob"], raw["prob"], atol=1e-12, rtol=1e-10)
    km = k.mean(axis=2)
    scale = 1.0 / math.sqrt(16)
    shift = scale * np.einsum("bhqd,bhd->bhq", raw["q_mean"], km)
    np.testing.assert_allclose(sm["scores"], raw["scores"] - shift[..., None], atol=1e-10)
