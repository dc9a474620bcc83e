"""Pins for the oracle on sequence lengths that are not multiples of 64 (CPU).

Reading R1 (CK page, "Status vs Upstream": per-block mean pool): the last
block of a ragged sequence holds fewer tokens and pools only those; in
attention it contributes only its existing keys, and a partial last Q-tile
writes only its existing rows.  The pins use facts outside the oracle's
formulas:
* attention over every block (or a LUT listing all of them) is torch's SDPA on
  the ragged tensors, causal included;
* a sparse LUT is SDPA with a boolean mask that keeps exactly the listed
  blocks' keys;
* duplicating each token of a partial block into a full block changes neither
  its mean nor its mean pairwise cosine, so the whole block map of the ragged
  sequence equals the map of the padded-by-duplication one;
* K smoothing removes the sequence mean, so shifting every K token by one
  vector leaves the smoothed map unchanged only if the mean is over the
  existing tokens;
* int8 inputs that are their own codes make the int8 path exact attention.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def _sdpa(q, k, v, mask=None, causal=False, scale=None):
    ratio = q.shape[1] // k.shape[1]
    kt = torch.from_numpy(np.repeat(k, ratio, axis=1))
    vt = torch.from_numpy(np.repeat(v, ratio, axis=1))
    qt = torch.from_numpy(q)
    m = None if mask is None else torch.from_numpy(mask)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, is_causal=causal,
                                                         scale=scale)
    sc = (qt @ kt.transpose(-1, -2)) * (scale if scale else 1.0 / math.sqrt(q.shape[-1]))
    if causal:
        sc = sc.masked_fill(~torch.ones(q.shape[2], k.shape[2], dtype=torch.bool).tril(), -math.inf)
    if m is not None:
        sc = sc.masked_fill(~m, -math.inf)
    return o.numpy(), torch.logsumexp(sc, -1).numpy()


def _rand(shape, seed, scale=1.0):
    return scale * np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("s_q,s_k", [(200, 333), (65, 64), (64, 1), (1, 130), (131, 131)])
def test_dense_ragged_is_sdpa(s_q, s_k):
    q = _rand((2, 4, s_q, 16), 1)
    k = _rand((2, 2, s_k, 16), 2)
    v = _rand((2, 2, s_k, 16), 3)
    o, lse = oracle.block_sparse_attention(q, k, v, None, None)
    ro, rl = _sdpa(q, k, v)
    np.testing.assert_allclose(o, ro, atol=1e-12, rtol=1e-12)
    np.testing.assert_allclose(lse, rl, atol=1e-12)
    # A LUT listing every block ascending is the same computation.
    nq, nk = -(-s_q // 64), -(-s_k // 64)
    lut = np.broadcast_to(np.arange(nk, dtype=np.int32), (2, 4, nq, nk)).copy()
    cnt = np.full((2, 4, nq), nk, np.int32)
    o2, l2 = oracle.block_sparse_attention(q, k, v, lut, cnt)
    np.testing.assert_allclose(o2, ro, atol=1e-12, rtol=1e-12)
    np.testing.assert_allclose(l2, rl, atol=1e-12)


@pytest.mark.parametrize("s", [131, 200, 255])
def test_causal_ragged_is_sdpa(s):
    q, k, v = _rand((1, 2, s, 16), 4), _rand((1, 2, s, 16), 5), _rand((1, 2, s, 16), 6)
    o, lse = oracle.block_sparse_attention(q, k, v, None, None, causal=True)
    ro, rl = _sdpa(q, k, v, causal=True)
    np.testing.assert_allclose(o, ro, atol=1e-12, rtol=1e-12)
    np.testing.assert_allclose(lse, rl, atol=1e-12)


def test_sparse_ragged_is_masked_sdpa():
    s_q, s_k = 150, 300                       # nq = 3, nk = 5, last K block of 44 keys
    q, k, v = _rand((1, 2, s_q, 16), 7), _rand((1, 2, s_k, 16), 8), _rand((1, 2, s_k, 16), 9)
    nq, nk = 3, 5
    rows = {0: [0, 4], 1: [4], 2: [1, 2, 3]}
    lut = np.full((1, 2, nq, nk), -1, np.int32)
    cnt = np.zeros((1, 2, nq), np.int32)
    mask = np.zeros((1, 2, s_q, s_k), bool)
    for qb, blocks in rows.items():
        for hh in range(2):
            lut[0, hh, qb, :len(blocks)] = blocks
            cnt[0, hh, qb] = len(blocks)
            for kb in blocks:
                mask[0, hh, qb * 64:(qb + 1) * 64, kb * 64:(kb + 1) * 64] = True
    o, lse = oracle.block_sparse_attention(q, k, v, lut, cnt)
    ro, rl = _sdpa(q, k, v, mask=mask)
    np.testing.assert_allclose(o, ro, atol=1e-12, rtol=1e-12)
    np.testing.assert_allclose(lse, rl, atol=1e-12)


def _duplicate_tail(x, n_tail):
    """x [b, h, 64 m + n_tail, d] with 64 % n_tail == 0: the tail's tokens each
    repeated 64 / n_tail times (in place) to fill a whole block."""
    head, tail = x[:, :, :x.shape[2] - n_tail], x[:, :, x.shape[2] - n_tail:]
    return np.concatenate([head, np.repeat(tail, 64 // n_tail, axis=2)], axis=2)


@pytest.mark.parametrize("n_tail", [32, 16, 1])
@pytest.mark.parametrize("opts", [dict(), dict(causal=True, attention_sink=True)])
def test_partial_block_pools_like_its_duplicated_block(n_tail, opts):
    b, h, d = 1, 2, 32
    s = 64 * 4 + n_tail
    rng = np.random.default_rng(n_tail)
    centre = rng.standard_normal((b, h, 1, d))
    q = centre + 0.6 * rng.standard_normal((b, h, s, d))
    k = centre + 0.6 * rng.standard_normal((b, h, s, d))
    thr = [0.3, 0.5]
    ragged = oracle.block_map(q, k, [0.4, 0.6], thr, **opts)
    full = oracle.block_map(_duplicate_tail(q, n_tail), _duplicate_tail(k, n_tail), [0.4, 0.6], thr, **opts)
    assert ragged["lut"].shape == (b, h, 5, 5)
    for key in ("q_mean", "k_mean", "sim_q_val", "sim_k_val", "prob"):
        np.testing.assert_allclose(ragged[key], full[key], rtol=1e-12, atol=1e-14, err_msg=key)
    for key in ("lut", "count", "bitmap", "sim_q", "sim_k"):
        assert np.array_equal(ragged[key], full[key]), key
    if n_tail == 1:
        # One token: its own mean, and a self-similarity of exactly 1.
        np.testing.assert_allclose(ragged["q_mean"][:, :, -1], q[:, :, -1], rtol=1e-15)
        np.testing.assert_allclose(ragged["sim_q_val"][:, :, -1], 1.0, rtol=1e-15)


def test_smoothing_mean_is_over_existing_keys():
    b, h, s, d = 1, 2, 64 * 3 + 20, 32
    rng = np.random.default_rng(11)
    q, k = rng.standard_normal((b, h, s, d)), rng.standard_normal((b, h, s, d))
    shift = 5.0 * rng.standard_normal((b, h, 1, d))
    a = oracle.block_map(q, k, [0.5, 0.5], [0.0, 0.0], smooth_k=True)
    c = oracle.block_map(q, k + shift, [0.5, 0.5], [0.0, 0.0], smooth_k=True)
    for key in ("k_mean", "sim_k_val", "prob"):
        np.testing.assert_allclose(a[key], c[key], rtol=1e-9, atol=1e-12, err_msg=key)
    assert np.array_equal(a["lut"], c["lut"])


def test_int8_ragged_own_codes_exact():
    rng = np.random.default_rng(12)
    b, h, s, d = 1, 2, 64 * 2 + 37, 16
    q = rng.integers(-127, 128, (b, h, s, d)).astype(np.float64)
    k = rng.integers(-127, 128, (b, h, s, d)).astype(np.float64)
    q[:, :, ::64, 0] = 127.0                 # a 127 in every block, the partial one included
    k[:, :, ::64, 0] = -127.0
    v = rng.standard_normal((b, h, s, d))
    codes, scales = oracle.quantize_int8(q)
    assert scales.shape == (b, h, 3) and np.all(scales == 1.0)
    assert np.array_equal(codes.astype(np.float64), q)
    sc = 1.0 / 2048.0
    for causal in (False, True):
        o, lse = oracle.block_sparse_attention_qk_int8(q, k, v, None, None, scale=sc, causal=causal)
        ro, rl = _sdpa(q, k, v, causal=causal, scale=sc)
        np.testing.assert_allclose(o, ro, atol=1e-12, rtol=1e-12)
        np.testing.assert_allclose(lse, rl, atol=1e-12)


def test_int8_partial_block_scale_is_its_own():
    rng = np.random.default_rng(13)
    x = rng.standard_normal((1, 1, 64 + 10, 8)).astype(np.float16).astype(np.float32)
    c1, s1 = oracle.quantize_int8(x)
    x2 = x.copy()
    x2[0, 0, 64:] *= 4.0                     # only the 10-token block changes scale
    c2, s2 = oracle.quantize_int8(x2)
    assert np.array_equal(c1, c2)
    assert s2[0, 0, 0] == s1[0, 0, 0] and s2[0, 0, 1] == 4.0 * s1[0, 0, 1]
    assert s1[0, 0, 1] == np.float32(np.abs(x[0, 0, 64:]).max()) / np.float32(127)


def test_pv_skip_ragged_reduces_to_exact_and_keeps_lse():
    s_q, s_k = 100, 170
    q, k, v = _rand((1, 2, s_q, 16), 14, 2.0), _rand((1, 2, s_k, 16), 15), _rand((1, 2, s_k, 16), 16)
    # K block t scaled by 4^-t: later blocks, the partial one of 42 keys
    # included, fall below the running maximum of every row of a tile.
    k = k * (4.0 ** -(np.arange(s_k) // 64))[None, None, :, None]
    ro, rl = _sdpa(q, k, v)
    # A threshold nothing falls below: exact attention, no unit skipped.
    o, lse, n_skip, _ = oracle.block_sparse_attention_pv_skip(q, k, v, None, None, 1e9,
                                                              return_skips=True)
    assert n_skip == 0
    np.testing.assert_allclose(o, ro, atol=1e-12, rtol=1e-12)
    np.testing.assert_allclose(lse, rl, atol=1e-12)
    # A small one: the LSE stays exact and O moves within the skip bound.
    o, lse, n_skip, _ = oracle.block_sparse_attention_pv_skip(q, k, v, None, None, 1.0,
                                                              return_skips=True)
    assert n_skip > 0
    np.testing.assert_allclose(lse, rl, atol=1e-12)
    bound = s_k * math.exp(-1.0) * np.abs(v).max()
    assert np.abs(o - ro).max() <= bound
