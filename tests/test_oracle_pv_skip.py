"""Pins for the oracle's pv_threshold skip (CPU).

CK page, "Status vs Upstream", not-yet-ported list: pv_threshold is a
per-Q-tile skip of work inside the attention kernel.  The oracle's test (reading
R25) is pinned here against closed forms on hand-built tiles whose scores are
constant per block or per key half (so every exponential is known exactly),
against torch's scaled_dot_product_attention when nothing can be skipped, and
against the error bound that the rule implies.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def _tile(scores_per_key, d=4, seed=0):
    """One 64-query tile and keys whose score against query row i is
    row_sign[i] * scores_per_key[key] with scale 1: q_i = (row_sign_i, 0, ...),
    k_j = (score_j, 0, ...)."""
    n_keys = len(scores_per_key)
    q = np.zeros((1, 1, 64, d))
    q[0, 0, :, 0] = 1.0
    k = np.zeros((1, 1, n_keys, d))
    k[0, 0, :, 0] = scores_per_key
    v = np.random.default_rng(seed).standard_normal((1, 1, n_keys, d))
    return q, k, v


def _run(q, k, v, blocks, tau, **kw):
    n = len(blocks)
    lut = np.array(blocks, dtype=np.int32).reshape(1, 1, 1, n)
    cnt = np.array([[[n]]], dtype=np.int32)
    return oracle.block_sparse_attention_pv_skip(q, k, v, lut, cnt, tau, scale=1.0,
                                                 return_skips=True, **kw)


def test_low_block_after_high_block_is_dropped_from_the_numerator_only():
    sc = np.r_[np.zeros(64), np.full(64, -5.0)]
    q, k, v = _tile(sc)
    vv = v[0, 0]
    den = 64.0 + 64.0 * math.exp(-5.0)
    o, lse, ns, nu = _run(q, k, v, [0, 1], 4.0)
    assert (ns, nu) == (1, 2)
    np.testing.assert_allclose(o[0, 0], np.broadcast_to(vv[:64].sum(0) / den, (64, 4)), rtol=1e-13)
    np.testing.assert_allclose(lse[0, 0], math.log(den), rtol=1e-14)
    # tau = 5 puts block 1 exactly on the boundary: the test is strict, so it stays
    o, lse, ns, _ = _run(q, k, v, [0, 1], 5.0)
    assert ns == 0
    exact = (vv[:64].sum(0) + math.exp(-5.0) * vv[64:].sum(0)) / den
    np.testing.assert_allclose(o[0, 0], np.broadcast_to(exact, (64, 4)), rtol=1e-13)


@pytest.mark.parametrize("tau,skipped", [(4.0, 0), (3.75, 1)])
def test_boundary_is_strict_on_dyadic_scores(tau, skipped):
    q, k, v = _tile(np.r_[np.zeros(64), np.full(64, -4.0)])
    _, _, ns, _ = _run(q, k, v, [0, 1], tau)
    assert ns == skipped


def test_running_maximum_covers_only_blocks_already_visited():
    # The low block comes first in LUT order: when it is visited it sets the
    # maximum itself, so nothing is skipped and the result is exact.
    sc = np.r_[np.full(64, -5.0), np.zeros(64)]
    q, k, v = _tile(sc)
    vv = v[0, 0]
    o, _, ns, _ = _run(q, k, v, [0, 1], 4.0)
    assert ns == 0
    exact = (math.exp(-5.0) * vv[:64].sum(0) + vv[64:].sum(0)) / (64.0 + 64.0 * math.exp(-5.0))
    np.testing.assert_allclose(o[0, 0], np.broadcast_to(exact, (64, 4)), rtol=1e-13)


def test_block_maximum_spans_all_of_the_blocks_keys():
    # Block 0: keys 0..31 score 0, keys 32..63 score -100.  Block 1: all -10.
    # The tile's running maximum after block 0 is 0 in every row, block 1's
    # maximum is -10, so block 1 is dropped at tau 4 -- whole, both key halves
    # (a rule that kept one maximum per 32-key half would keep keys 96..127,
    # whose half had only seen -100 before).
    sc = np.r_[np.zeros(32), np.full(32, -100.0), np.full(64, -10.0)]
    q, k, v = _tile(sc)
    vv = v[0, 0]
    den = 32.0 + 32.0 * math.exp(-100.0) + 64.0 * math.exp(-10.0)
    base = vv[:32].sum(0) + math.exp(-100.0) * vv[32:64].sum(0)
    o, lse, ns, nu = _run(q, k, v, [0, 1], 4.0)
    assert (ns, nu) == (1, 2)
    np.testing.assert_allclose(o[0, 0], np.broadcast_to(base / den, (64, 4)), rtol=1e-12)
    np.testing.assert_allclose(lse[0, 0], math.log(den), rtol=1e-14)


def test_every_row_of_the_tile_must_lie_below():
    # Rows 0..31 see block 1 at -5 (below the maximum 0 by more than 4); rows
    # 32..63 see it at +5, a new maximum.  The unit is the whole tile, so the
    # block stays for every row and the result is exact.
    q, k, v = _tile(np.r_[np.zeros(64), np.full(64, -5.0)])
    q[0, 0, 32:, 0] = -1.0
    vv = v[0, 0]
    o, lse, ns, nu = _run(q, k, v, [0, 1], 4.0)
    assert (ns, nu) == (0, 2)
    den = 64.0 + 64.0 * math.exp(-5.0)
    exact_lo = (vv[:64].sum(0) + math.exp(-5.0) * vv[64:].sum(0)) / den
    exact_hi = (math.exp(-5.0) * vv[:64].sum(0) + vv[64:].sum(0)) / den
    np.testing.assert_allclose(o[0, 0, :32], np.broadcast_to(exact_lo, (32, 4)), rtol=1e-13)
    np.testing.assert_allclose(o[0, 0, 32:], np.broadcast_to(exact_hi, (32, 4)), rtol=1e-13)
    np.testing.assert_allclose(lse[0, 0, 32:], 5.0 + math.log(den), rtol=1e-14)


@pytest.mark.parametrize("row", [0, 17, 63])
def test_one_row_near_its_maximum_keeps_the_block(row):
    # Every row but one sees block 1 at -5; that row sees it at -3 (its scores
    # are scaled by 0.6), within tau = 4 of its maximum 0.  The block stays.
    q, k, v = _tile(np.r_[np.zeros(64), np.full(64, -5.0)])
    _, _, ns, _ = _run(q, k, v, [0, 1], 4.0)
    assert ns == 1
    q[0, 0, row, 0] = 0.6
    _, _, ns, _ = _run(q, k, v, [0, 1], 4.0)
    assert ns == 0


def test_later_blocks_compare_with_every_block_before_them():
    # Scores per block 0, -6, -6, -3 at tau 4: blocks 1 and 2 lie 6 below the
    # maximum 0 and are dropped; block 3 lies 3 below and stays.  The running
    # maximum is over the blocks visited, not only the previous one.
    sc = np.r_[np.zeros(64), np.full(64, -6.0), np.full(64, -6.0), np.full(64, -3.0)]
    q, k, v = _tile(sc)
    vv = v[0, 0]
    o, _, ns, nu = _run(q, k, v, [0, 1, 2, 3], 4.0)
    assert (ns, nu) == (2, 4)
    den = 64.0 * (1.0 + 2.0 * math.exp(-6.0) + math.exp(-3.0))
    kept = (vv[:64].sum(0) + math.exp(-3.0) * vv[192:].sum(0)) / den
    np.testing.assert_allclose(o[0, 0], np.broadcast_to(kept, (64, 4)), rtol=1e-12)
    skip = oracle.pv_skip_blocks(np.broadcast_to(sc.reshape(1, 4, 64), (64, 4, 64)), 4.0)
    assert skip.tolist() == [False, True, True, False]


def test_masked_rows_follow_the_rule_with_minus_infinity():
    # A row with no key in a block (r = -inf) lies below any finite running
    # maximum; a row that has met no key yet (M = -inf) keeps the block.
    sc = np.zeros((64, 2, 64))
    sc[:, 1, :] = -math.inf
    assert oracle.pv_skip_blocks(sc, 1.0).tolist() == [False, True]
    sc[5, 0, :] = -math.inf
    sc[5, 1, :] = -math.inf
    assert oracle.pv_skip_blocks(sc, 1.0).tolist() == [False, False]


@pytest.mark.parametrize("causal", [False, True])
def test_infinite_threshold_is_sdpa(causal):
    rng = np.random.default_rng(3)
    q, k, v = (rng.standard_normal((1, 2, 256, 16)) for _ in range(3))
    o, lse = oracle.block_sparse_attention_pv_skip(q, k, v, None, None, math.inf, causal=causal)
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(x) for x in (q, k, v)), is_causal=causal)
    np.testing.assert_allclose(o, ref.numpy(), atol=1e-12, rtol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_skipping_keeps_the_lse_and_stays_within_its_bound(causal):
    # K block t is scaled by 2^-t, so later blocks score lower and many of
    # them are dropped at tau = 3.  Every dropped key scores more than tau
    # below its row's maximum, so it carries less than exp(-tau) of the row's
    # mass: |O - O_exact| <= that mass * max|v|.
    rng = np.random.default_rng(4)
    s, d = 512, 16
    q = 4.0 * rng.standard_normal((1, 1, s, d))
    k, v = rng.standard_normal((1, 1, s, d)), rng.standard_normal((1, 1, s, d))
    k *= np.repeat(2.0 ** -np.arange(s // 64), 64)[None, None, :, None]
    tau, scale = 3.0, 1.0 / math.sqrt(d)
    o, lse, ns, nu = oracle.block_sparse_attention_pv_skip(
        q, k, v, None, None, tau, causal=causal, return_skips=True)
    assert 0 < ns < nu
    qt, kt, vt = (torch.from_numpy(x) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=causal)
    sc = (qt @ kt.transpose(-1, -2))[0, 0] * scale
    if causal:
        sc = sc.masked_fill(~torch.ones(s, s, dtype=torch.bool).tril(), -math.inf)
    np.testing.assert_allclose(lse[0, 0], torch.logsumexp(sc, -1).numpy(), atol=1e-12)
    # dropped keys per row, from the block decisions taken on the exact scores
    nblk = s // 64
    bound = np.zeros(s)
    for qb in range(nblk):
        part = sc[64 * qb:64 * qb + 64].numpy().reshape(64, nblk, 64)
        bound[64 * qb:64 * qb + 64] = 64 * oracle.pv_skip_blocks(part, tau).sum()
    err = np.abs(o[0, 0] - ref.numpy()[0, 0]).max(axis=1)
    assert np.all(err <= bound * math.exp(-tau) * np.abs(v).max() + 1e-12)
    assert np.all(err[bound == 0] <= 1e-12)
