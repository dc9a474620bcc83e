"""GPU parity for block maps with fewer K heads than query heads.

Reading R28: query head j pools against K head j // (h / h_kv) (the GQA
mapping of attention, aiter 6841 page) and gates that head's K blocks with its
own simthreshd1[j].  The bars are those of the other block-map tests: the LUT,
counts and bitmap bit-exact against the oracle's selection run on the GPU's
pooled probabilities and flags; pooled means and probabilities within 1e-3
relative; flags equal wherever the similarity is not within 1e-5 of the
threshold; int8 codes and scales bit-exact.  End to end, the map feeds the
sparse FMHA with K/V of h_kv heads (O atol 4e-2 / rtol 1e-2, LSE 2e-3 nats).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from block_sparse_attention_sparge_amd import ops, synth

pytestmark = pytest.mark.gpu


def np64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    ops.load_library()
    return torch.device("cuda:0")


def _case(dev, b, h, h_kv, s, d, dtype, seed):
    gam = [0.5 + 1.5 * i / max(1, h - 1) for i in range(h)]
    q = synth.centroid_noise(b, h, s, d, 64, gam, 0.5, seed, 1, dtype, dev)
    k = synth.centroid_noise(b, h_kv, s, d, 64, gam[:h_kv], 0.5, seed, 2, dtype, dev)
    v = synth.normal((b, h_kv, s, d), seed, 3, dtype, dev)
    return q, k, v


def _check_map(res, q, k, topk, thr, cdf=None, **opts):
    h, h_kv = q.shape[1], k.shape[1]
    ref = oracle.block_map(np64(q), np64(k), topk=topk, simthreshd1=thr, cdfthreshd=cdf, **opts)
    assert tuple(res["k_mean"].shape) == (q.shape[0], h_kv, k.shape[2] // 64, q.shape[3])
    for key in ("q_mean", "k_mean"):
        g, r = np64(res[key]), ref[key]
        rms = math.sqrt(float((r * r).mean()))
        assert (np.abs(g - r) <= 1e-3 * np.abs(r) + 1e-6 * rms).all(), key
    thr_a = np.array(thr)[None, :, None]
    far_q = np.abs(ref["sim_q_val"] - thr_a) > 1e-5
    assert np.array_equal(np64(res["sim_q"]).astype(bool)[far_q], ref["sim_q"][far_q])
    simk_val = np.repeat(ref["sim_k_val"], h // h_kv, axis=1)          # as each query head sees it
    far_k = np.abs(simk_val - thr_a) > 1e-5
    assert np.array_equal(np64(res["sim_k"]).astype(bool)[far_k], ref["sim_k"][far_k])
    gp = np64(res["prob"])
    assert (np.abs(gp - ref["prob"]) <= 1e-3 * np.abs(ref["prob"]) + 1e-7).all(), "pooled prob"
    lut, cnt, bm = oracle.select_from_probs(
        gp, np64(res["sim_q"]).astype(bool), np64(res["sim_k"]).astype(bool), topk, cdf,
        causal=opts.get("causal", False), attention_sink=opts.get("attention_sink", False))
    assert np.array_equal(res["lut"].cpu().numpy(), lut), "LUT not bit-exact"
    assert np.array_equal(res["count"].cpu().numpy(), cnt), "count not bit-exact"
    assert np.array_equal(res["bitmap"].cpu().numpy(), bm), "bitmap not bit-exact"
    return ref


@pytest.mark.parametrize("h,h_kv", [(4, 2), (8, 2), (8, 1)])
@pytest.mark.parametrize("dtype,d", [(torch.float16, 64), (torch.bfloat16, 128)])
def test_grouped_block_map(dev, h, h_kv, dtype, d):
    q, k, _ = _case(dev, 2, h, h_kv, 1024, d, dtype, 20 + h + h_kv)
    topk = [0.25 + 0.125 * (i % 3) for i in range(h)]
    thr = [0.47 + 0.04 * (i % 2) for i in range(h)]       # K gates differ within a group
    res = ops.build_block_map(q, k, topk, thr, return_debug=True)
    torch.cuda.synchronize()
    ref = _check_map(res, q, k, topk, thr)
    assert (ref["sim_k"][:, 0] != ref["sim_k"][:, 1]).any()


@pytest.mark.parametrize("opts", [dict(smooth_k=True), dict(causal=True, attention_sink=True),
                                  dict(smooth_k=True, causal=True, attention_sink=True)])
def test_grouped_block_map_options(dev, opts):
    q, k, _ = _case(dev, 1, 8, 2, 2048, 128, torch.bfloat16, 31)
    topk, thr = [0.4] * 8, [0.001] * 8
    res = ops.build_block_map(q, k, topk, thr, return_debug=True, **opts)
    torch.cuda.synchronize()
    _check_map(res, q, k, topk, thr, **opts)


def test_grouped_block_map_cdf_mode(dev):
    q, k, _ = _case(dev, 1, 4, 2, 1024, 128, torch.float16, 41)
    cdf = [0.3, 0.6, 0.9, 0.99]
    res = ops.build_block_map(q, k, [0.0] * 4, [0.001] * 4, cdfthreshd=cdf, return_debug=True)
    torch.cuda.synchronize()
    _check_map(res, q, k, [0.0] * 4, [0.001] * 4, cdf=cdf)


def test_grouped_int8_codes_per_k_head(dev):
    q, k, v = _case(dev, 2, 8, 2, 1024, 128, torch.float16, 51)
    res = ops.build_block_map(q, k, [0.4] * 8, [0.001] * 8, quantize_int8=True)
    torch.cuda.synchronize()
    for x, key in ((q, "q_i8"), (k, "k_i8")):
        codes, scales = oracle.quantize_int8(x.float().cpu().numpy())
        assert np.array_equal(res[key].cpu().numpy(), codes), key
        assert np.array_equal(res[key + "_scale"].cpu().numpy(), scales), key
    o, lse = ops.sparse_fmha_fwd_qk_int8(res["q_i8"], res["q_i8_scale"], res["k_i8"], res["k_i8_scale"], v,
                                         res["lut"], res["count"])
    torch.cuda.synchronize()
    ro, rl = oracle.block_sparse_attention_qk_int8(np64(q), np64(k), np64(v), res["lut"].cpu().numpy(),
                                                   res["count"].cpu().numpy())
    err = np.abs(np64(o) - ro)
    assert (err <= 4e-2 + 1e-2 * np.abs(ro)).all()
    assert np.abs(np64(lse) - rl).max() <= 2e-3


@pytest.mark.parametrize("causal", [False, True])
def test_grouped_end_to_end(dev, causal):
    # The grouped map gives one LUT row per query head; the FMHA reads K/V of
    # h_kv heads with those rows.
    q, k, v = _case(dev, 2, 8, 2, 2048, 128, torch.bfloat16, 61)
    bm = ops.build_block_map(q, k, [0.3] * 8, [0.001] * 8, causal=causal, attention_sink=causal)
    o, lse = ops.sparse_fmha_fwd(q, k, v, bm["lut"], bm["count"], causal=causal)
    torch.cuda.synchronize()
    ro, rl = oracle.block_sparse_attention(np64(q), np64(k), np64(v), bm["lut"].cpu().numpy(),
                                           bm["count"].cpu().numpy(), causal=causal)
    err = np.abs(np64(o) - ro)
    assert (err <= 4e-2 + 1e-2 * np.abs(ro)).all(), f"max err {err.max():.3e}"
    g = np64(lse)
    assert np.array_equal(np.isneginf(g), np.isneginf(rl))
    fin = ~np.isneginf(rl)
    assert np.abs(g[fin] - rl[fin]).max() <= 2e-3
