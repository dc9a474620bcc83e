"""GPU parity with a softmax_scale other than 1/sqrt(d).

Reading R4: the pooled scores use the attention's softmax scale (it moves the
pooled softmax, so it changes cdf-mode selections; top-k is scale-invariant).
Reading R11: the LSE is the natural log of sum_j exp(scale * q.k_j), scale
included.  Every entry point that takes softmax_scale is run with scales
below and above the default and compared with the oracle given the same scale,
at the bars of the other parity tests.
"""
import numpy as np
import pytest
import torch

import oracle
from block_sparse_attention_sparge_amd import ops, synth

pytestmark = pytest.mark.gpu

O_ATOL, O_RTOL, LSE_TOL = 4e-2, 1e-2, 2e-3


def np64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    ops.load_library()
    return torch.device("cuda:0")


def check_o(o_gpu, o_ref):
    err = np.abs(np64(o_gpu) - o_ref)
    bad = err > O_ATOL + O_RTOL * np.abs(o_ref)
    assert not bad.any(), f"O: {bad.sum()} of {bad.size} outside atol/rtol; max err {err.max():.3e}"


def check_lse(l_gpu, l_ref):
    g = np64(l_gpu)
    assert np.array_equal(np.isneginf(g), np.isneginf(l_ref)), "-inf rows differ"
    fin = ~np.isneginf(l_ref)
    if fin.any():
        assert np.abs(g[fin] - l_ref[fin]).max() <= LSE_TOL


def _qkv(dev, b, h, s, d, dtype, seed):
    gam = [0.5 + 1.5 * i / max(1, h - 1) for i in range(h)]
    q = synth.centroid_noise(b, h, s, d, 64, gam, 0.5, seed, 1, dtype, dev)
    k = synth.centroid_noise(b, h, s, d, 64, gam, 0.5, seed, 2, dtype, dev)
    v = synth.normal((b, h, s, d), seed, 3, dtype, dev)
    return q, k, v


@pytest.mark.parametrize("scale", [0.02, 0.3])
@pytest.mark.parametrize("causal", [False, True])
def test_map_and_fmha(dev, scale, causal):
    q, k, v = _qkv(dev, 1, 4, 1024, 128, torch.float16, 7)
    cdf = [0.5, 0.8, 0.9, 0.95]
    res = ops.build_block_map(q, k, [0.0] * 4, [0.001] * 4, cdfthreshd=cdf, softmax_scale=scale,
                              causal=causal, return_debug=True)
    torch.cuda.synchronize()
    ref = oracle.block_map(np64(q), np64(k), [0.0] * 4, [0.001] * 4, cdfthreshd=cdf, scale=scale,
                           causal=causal)
    gp = np64(res["prob"])
    assert (np.abs(gp - ref["prob"]) <= 1e-3 * np.abs(ref["prob"]) + 1e-7).all(), "pooled prob"
    lut, cnt, _ = oracle.select_from_probs(gp, np64(res["sim_q"]).astype(bool),
                                           np64(res["sim_k"]).astype(bool), [0.0] * 4, cdf, causal=causal)
    assert np.array_equal(res["lut"].cpu().numpy(), lut) and np.array_equal(res["count"].cpu().numpy(), cnt)
    # The scale matters here: the default scale selects different counts.
    dflt = oracle.block_map(np64(q), np64(k), [0.0] * 4, [0.001] * 4, cdfthreshd=cdf, causal=causal)
    assert not np.array_equal(dflt["count"], ref["count"])
    o, lse = ops.sparse_fmha_fwd(q, k, v, res["lut"], res["count"], softmax_scale=scale, causal=causal)
    torch.cuda.synchronize()
    ro, rl = oracle.block_sparse_attention(np64(q), np64(k), np64(v), res["lut"].cpu().numpy(),
                                           res["count"].cpu().numpy(), scale=scale, causal=causal)
    check_o(o, ro)
    check_lse(lse, rl)


@pytest.mark.parametrize("scale", [0.02, 0.3])
def test_int8_fmha(dev, scale):
    q, k, v = _qkv(dev, 1, 4, 1000, 64, torch.bfloat16, 8)
    bm = ops.build_block_map(q, k, [0.5] * 4, [0.001] * 4, softmax_scale=scale, quantize_int8=True)
    o, lse = ops.sparse_fmha_fwd_qk_int8(bm["q_i8"], bm["q_i8_scale"], bm["k_i8"], bm["k_i8_scale"], v,
                                         bm["lut"], bm["count"], softmax_scale=scale)
    torch.cuda.synchronize()
    ro, rl = oracle.block_sparse_attention_qk_int8(np64(q), np64(k), np64(v), bm["lut"].cpu().numpy(),
                                                   bm["count"].cpu().numpy(), scale=scale)
    check_o(o, ro)
    check_lse(lse, rl)


@pytest.mark.parametrize("scale", [0.02, 0.3])
def test_decode(dev, scale):
    b, h_q, h_kv, s_k, d, L = 4, 8, 2, 3000, 128, 300
    q = synth.normal((b, h_q, 1, d), 9, 1, torch.bfloat16, dev, scale=4.0)
    k = synth.normal((b, h_kv, s_k, d), 9, 2, torch.bfloat16, dev)
    v = synth.normal((b, h_kv, s_k, d), 9, 3, torch.bfloat16, dev)
    lists = synth.token_lists(b, h_kv, L, s_k, 9, 4, True).to(dev)
    op, lp = ops.sparse_fmha_fwd(q, k, v, lists, None, blk_q=1, blk_k=1, num_splits=4, softmax_scale=scale)
    o, lse = ops.attn_combine(op, lp, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ro, rl = oracle.token_list_attention(np64(q), np64(k), np64(v), lists.cpu().numpy(), scale=scale)
    check_o(o, ro)
    check_lse(lse, rl)
