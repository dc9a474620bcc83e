"""Pins for the oracle's fp8 e4m3 Q/K quantisation (reading R29).

CK page, "Status vs Upstream", not-yet-ported list: Q/K quantisation fused
into the pool kernel for a low-precision QK product in the attention kernel;
the aiter 6841 page runs fp8 Q/K recipes.  The oracle's e4m3 rounding is
pinned to torch's float8_e4m3fn conversion (an independent library routine)
and to closed forms of the OCP e4m3 grid; the block quantisation to closed
forms, its error bound, and exact attention when the inputs are their own
codes.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def test_rounding_equals_torch_float8_e4m3fn():
    rng = np.random.default_rng(11)
    # Below 464 (the midpoint between 448 and the next binade's first value);
    # the quantisation never goes past 448 * (1 + 2^-23), and torch turns
    # values from 464 up into NaN where the oracle saturates.
    x = np.concatenate([
        rng.uniform(-463.9, 463.9, 100000),      # normals, and the rounding range above 448
        rng.uniform(-2.0 ** -5, 2.0 ** -5, 100000),   # subnormals and the smallest normals
        rng.standard_normal(100000) * 30,
    ]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    assert np.array_equal(oracle.round_e4m3(x), ref)


def test_byte_values_equal_torch_float8_view():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    val = oracle.e4m3_value(codes)
    assert np.array_equal(np.isnan(val), np.isnan(ref))
    assert np.array_equal(val[~np.isnan(val)], ref[~np.isnan(ref)])
    assert np.isnan(val).sum() == 2                          # 0x7F and 0xFF


def test_grid_closed_forms():
    grid = oracle.e4m3_value(np.arange(128, dtype=np.uint8))[:127]     # +0 .. 448
    assert grid[1] == 2.0 ** -9 and grid[7] == 7 * 2.0 ** -9 and grid[8] == 2.0 ** -6
    assert grid[0x38] == 1.0 and grid[0x7E] == oracle.E4M3_MAX == 448.0
    # every grid value rounds to itself, and its byte is recovered
    assert np.array_equal(oracle.round_e4m3(grid.astype(np.float32)), grid)
    assert np.array_equal(oracle.e4m3_code(grid), np.arange(127, dtype=np.uint8))
    # midpoints between neighbours go to the even mantissa (even byte)
    mids = (grid[1:] + grid[:-1]) / 2
    r = oracle.round_e4m3(mids.astype(np.float32))
    even = np.where(np.arange(126) % 2 == 0, grid[:-1], grid[1:])
    assert np.array_equal(r, even)
    # above 448 the rounding saturates; signs are kept
    assert np.all(oracle.round_e4m3(np.float32([448.5, 460, 1e6])) == 448.0)
    assert np.array_equal(oracle.round_e4m3(-grid.astype(np.float32)), -grid)


def test_block_quantisation_closed_forms():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((64, 32)).astype(np.float32)
    codes, scale = oracle.quantize_block_fp8(x)
    amax = np.float32(np.abs(x).max())
    assert scale == amax / np.float32(448)
    assert np.abs(codes).max() == 448.0                      # the largest element lands on 448
    assert np.array_equal(oracle.round_e4m3(codes.astype(np.float32)), codes)
    # each code is within half a grid step of x / scale
    y = x.astype(np.float64) * float(np.float32(448) / amax)
    a = np.abs(y)
    step = np.where(a >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(a, 1e-30))) - 3), 2.0 ** -9)
    assert np.all(np.abs(codes - y) <= step / 2 + 1e-12 * a)
    # power-of-two input scaling leaves the codes and scales the scale exactly
    c2, s2 = oracle.quantize_block_fp8(x * np.float32(4))
    assert np.array_equal(c2, codes) and s2 == 4 * scale
    # an all-zero block
    cz, sz = oracle.quantize_block_fp8(np.zeros((64, 8), np.float32))
    assert sz == 0 and not cz.any()


def test_partial_block_has_its_own_scale():
    x = np.random.default_rng(6).standard_normal((1, 1, 64 + 10, 16)).astype(np.float32)
    _, s1 = oracle.quantize_fp8(x)
    x2 = x.copy()
    x2[0, 0, 64:] *= 8.0
    c2, s2 = oracle.quantize_fp8(x2)
    assert s2[0, 0, 0] == s1[0, 0, 0] and s2[0, 0, 1] == 8 * s1[0, 0, 1]


@pytest.mark.parametrize("causal", [False, True])
def test_inputs_that_are_their_own_codes_give_exact_attention(causal):
    # Every block of Q and K holds 448 and values on the e4m3 grid, so its
    # scale is exactly 1 and its codes are the inputs: attention on the codes
    # is attention on the inputs.
    rng = np.random.default_rng(7)
    grid = oracle.e4m3_value(np.arange(127, dtype=np.uint8))
    small = grid[(grid > 0) & (grid <= 8)]

    def on_grid(shape):
        x = rng.choice(small, size=shape) * rng.choice([-1.0, 1.0], size=shape)
        x[..., ::64, 0] = 448.0
        return x

    q, k = on_grid((1, 2, 192, 16)), on_grid((1, 2, 192, 16))
    v = rng.standard_normal((1, 2, 192, 16))
    _, sq = oracle.quantize_fp8(q)
    assert np.all(sq == 1.0)
    o, lse = oracle.block_sparse_attention_qk_fp8(q, k, v, None, None, scale=0.01, causal=causal)
    ro = torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(t) for t in (q, k, v)), scale=0.01, is_causal=causal)
    assert np.abs(o - ro.numpy()).max() < 1e-12
    sc = 0.01 * torch.from_numpy(q) @ torch.from_numpy(k).transpose(-1, -2)
    if causal:
        sc = sc.masked_fill(~torch.ones(192, 192, dtype=torch.bool).tril(), -math.inf)
    assert np.abs(lse - torch.logsumexp(sc, -1).numpy()).max() < 1e-12


def test_scores_within_the_rounding_bound():
    # |q.k - cq.ck sq sk| <= sum |q_i| |dk_i| + |dq_i| |k_i| + |dq_i| |dk_i|
    # with |dx| <= half a grid step times the scale.
    rng = np.random.default_rng(8)
    q = rng.standard_normal((1, 1, 64, 32)).astype(np.float32)
    k = rng.standard_normal((1, 1, 64, 32)).astype(np.float32)
    cq, sq = oracle.quantize_fp8(q)
    ck, sk = oracle.quantize_fp8(k)
    dq = oracle.dequantize_int8(cq, sq)[0, 0]
    dk = oracle.dequantize_int8(ck, sk)[0, 0]
    qq, kk = q[0, 0].astype(np.float64), k[0, 0].astype(np.float64)
    eq, ek = np.abs(dq - qq), np.abs(dk - kk)
    # e4m3 has 3 mantissa bits: relative error <= 2^-4 for normals
    assert np.all(eq <= np.maximum(2.0 ** -4 * np.abs(qq), 2.0 ** -10 * float(sq[0, 0, 0])) + 1e-12)
    bound = np.abs(qq) @ ek.T + eq @ np.abs(kk).T + eq @ ek.T
    assert np.all(np.abs(dq @ dk.T - qq @ kk.T) <= bound + 1e-9)
