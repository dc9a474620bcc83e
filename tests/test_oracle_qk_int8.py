"""Pins for the oracle's int8 Q/K block quantisation (CPU).

CK page, "Status vs Upstream", not-yet-ported list: Q/K int8 quantisation in
the pool kernel for an int8 QK product in the attention kernel.  Reading R27
fixes the formula (per 64-token block, scale absmax / 127, round half to
even in fp32).  The pins: closed forms where the scale is a power of two (so
every product is exact and ties are real ties), torch's own int8 quantiser
away from ties, exact equality with torch's SDPA when the inputs are their
own codes, scale equivariance, and the per-score error bound of rounding.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def test_codes_round_half_to_even_at_unit_scale():
    x = np.zeros((64, 8), np.float32)
    vals = [127.0, -127.0, 0.5, 1.5, 2.5, -2.5, 63.5, 126.5, -0.5, 3.25]
    x[0, :8] = vals[:8]
    x[1, :2] = vals[8:]
    codes, scale = oracle.quantize_block_int8(x)
    assert scale == np.float32(1.0)
    assert list(codes[0, :8]) == [127, -127, 0, 2, 2, -2, 64, 126]
    assert list(codes[1, :2]) == [0, 3]


def test_codes_at_scale_two():
    x = np.zeros((64, 4), np.float32)
    x[0] = [254.0, 1.0, 3.0, -5.0]
    codes, scale = oracle.quantize_block_int8(x)
    assert scale == np.float32(2.0)
    assert list(codes[0]) == [127, 0, 2, -2]


def test_zero_block():
    codes, scale = oracle.quantize_block_int8(np.zeros((64, 16), np.float32))
    assert scale == 0.0 and not codes.any()


def test_codes_agree_with_torch_quantize_away_from_ties():
    rng = np.random.default_rng(0)
    for trial in range(20):
        x = (rng.standard_normal((64, 128)) * 10 ** rng.uniform(-3, 3)).astype(np.float16).astype(np.float32)
        codes, scale = oracle.quantize_block_int8(x)
        ref = torch.quantize_per_tensor(torch.from_numpy(x), float(scale), 0, torch.qint8).int_repr().numpy()
        t = x.astype(np.float64) / float(scale)
        far = np.abs(np.abs(t - np.floor(t)) - 0.5) > 1e-3
        assert np.array_equal(codes[far], ref[far])
        assert np.abs(codes).max() == 127


@pytest.mark.parametrize("causal", [False, True])
def test_inputs_that_are_their_own_codes_give_exact_attention(causal):
    # Integer Q and K in [-127, 127] with a 127 in every block: scale 1 and
    # codes = inputs, so the int8 path is exact attention.
    rng = np.random.default_rng(1)
    b, h, s, d = 1, 2, 256, 16
    q = rng.integers(-127, 128, (b, h, s, d)).astype(np.float64)
    k = rng.integers(-127, 128, (b, h, s, d)).astype(np.float64)
    q[:, :, ::64, 0] = 127.0
    k[:, :, ::64, 0] = -127.0
    v = rng.standard_normal((b, h, s, d))
    sc = 1.0 / 2048.0                      # keeps exp() in range for these scores
    o, lse = oracle.block_sparse_attention_qk_int8(q, k, v, None, None, scale=sc, causal=causal)
    qt, kt, vt = (torch.from_numpy(x) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=causal, scale=sc)
    np.testing.assert_allclose(o, ref.numpy(), atol=1e-12, rtol=1e-12)
    scores = (qt @ kt.transpose(-1, -2)) * sc
    if causal:
        scores = scores.masked_fill(~torch.ones(s, s, dtype=torch.bool).tril(), -math.inf)
    np.testing.assert_allclose(lse, torch.logsumexp(scores, -1).numpy(), atol=1e-12)


def test_scaling_a_block_by_a_power_of_two_scales_only_its_scale():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((1, 1, 128, 32)).astype(np.float16).astype(np.float32)
    c1, s1 = oracle.quantize_int8(x)
    x2 = x.copy()
    x2[0, 0, 64:] *= 8.0
    c2, s2 = oracle.quantize_int8(x2)
    assert np.array_equal(c1, c2)
    assert s2[0, 0, 0] == s1[0, 0, 0] and s2[0, 0, 1] == 8.0 * s1[0, 0, 1]


def test_score_error_within_the_rounding_bound():
    # Codes are within half a step of x / scale, so
    # |s_q - s| <= scale * sum_d (sq/2 |k| + sk/2 |q| + sq sk / 4).  The fp32
    # roundings of 127 / absmax and absmax / 127 stretch the half step by a
    # few parts in 10^6 (a margin of 1e-4 covers them).
    rng = np.random.default_rng(3)
    b, h, s, d = 1, 1, 256, 64
    q = (3.0 * rng.standard_normal((b, h, s, d))).astype(np.float16).astype(np.float64)
    k = (rng.standard_normal((b, h, s, d)) + 2.0).astype(np.float16).astype(np.float64)
    cq, sq = oracle.quantize_int8(q)
    ck, sk = oracle.quantize_int8(k)
    qd, kd = oracle.dequantize_int8(cq, sq), oracle.dequantize_int8(ck, sk)
    assert np.all(np.abs(qd - q) <= np.repeat(sq, 64, axis=2)[..., None] / 2 * (1 + 1e-4))
    scale = 1.0 / math.sqrt(d)
    err = np.abs(qd[0, 0] @ kd[0, 0].T - q[0, 0] @ k[0, 0].T) * scale
    sqr = np.repeat(sq[0, 0], 64)[:, None].astype(np.float64)
    skr = np.repeat(sk[0, 0], 64)[None, :].astype(np.float64)
    bound = scale * (sqr / 2 * np.abs(k[0, 0]).sum(1)[None, :] + skr / 2 * np.abs(q[0, 0]).sum(1)[:, None]
                     + d * sqr * skr / 4)
    assert np.all(err <= bound * (1 + 1e-4))
    assert err.max() > 0.05 * bound.max()          # the bound is not vacuous here
