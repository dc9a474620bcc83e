"""Seeded sweep of the block map against the fp64 oracle.

Each case draws its own shape and options: ragged s_q / s_k, d 64 or 128,
fp16 or bf16, grouped-query ratios 1 / 2 / 4, per-head top-k fractions or cdf
thresholds, per-head gate thresholds placed among the blocks' similarities
(so that Q and K gates fire), K smoothing, the causal block mask and the
attention sink.  Every case is held to the stated bars: pooled means and
probabilities within 1e-3 relative, gate flags equal wherever the similarity
is more than 1e-5 from the threshold, and LUT, count and bitmap bit-exact
against the oracle's selection run on the GPU's probabilities and flags.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from block_sparse_attention_sparge_amd import ops, synth

pytestmark = pytest.mark.gpu

N_CASES = 48


def np64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    ops.load_library()          # raises if the HIP library is missing
    return torch.device("cuda:0")


def draw_case(i):
    r = np.random.RandomState(2000 + i)
    c = dict(
        b=int(r.choice([1, 2])),
        h_kv=int(r.choice([1, 2])),
        ratio=int(r.choice([1, 2, 4])),
        d=int(r.choice([64, 128])),
        dtype=[torch.float16, torch.bfloat16][r.randint(2)],
        gamma=float(r.choice([0.0, 0.5, 1.0, 2.0])),
        sigma=float(r.choice([0.3, 0.5, 1.0])),
        smooth_k=bool(r.rand() < 0.3),
        causal=bool(r.rand() < 0.3),
        sink=bool(r.rand() < 0.3),
        cdf_mode=bool(r.rand() < 0.3),
    )
    h = c["h_kv"] * c["ratio"]
    c["s_q"] = int(r.randint(1, 1500))
    c["s_k"] = c["s_q"] if c["causal"] else int(r.randint(1, 1500))
    c["topk"] = [0.0] * h if c["cdf_mode"] else [float(r.uniform(0.01, 1.0)) for _ in range(h)]
    c["cdf"] = [float(r.uniform(0.2, 0.99)) for _ in range(h)] if c["cdf_mode"] else None
    # Thresholds between about 0 and the blocks' typical similarity, so that
    # some gates close: a block of centroid + noise has a mean pairwise cosine
    # near gamma^2 / (gamma^2 + sigma^2), pure noise near 1 / 64.
    typ = c["gamma"] ** 2 / (c["gamma"] ** 2 + c["sigma"] ** 2) + 1.0 / 64
    c["thr"] = [float(r.choice([0.001, r.uniform(0.5, 1.5) * typ])) for _ in range(h)]
    return c


def describe(c):
    return (f"b{c['b']} h_kv{c['h_kv']}x{c['ratio']} s_q{c['s_q']} s_k{c['s_k']} d{c['d']} "
            f"{str(c['dtype']).split('.')[-1]} gamma{c['gamma']} sigma{c['sigma']} "
            f"smooth={c['smooth_k']} causal={c['causal']} sink={c['sink']} cdf={c['cdf_mode']}")


@pytest.mark.parametrize("i", range(N_CASES))
def test_block_map_random_case(dev, i):
    c = draw_case(i)
    print(describe(c), flush=True)
    h = c["h_kv"] * c["ratio"]
    gq = [c["gamma"]] * h
    q = synth.centroid_noise(c["b"], h, c["s_q"], c["d"], 64, gq, c["sigma"], 700 + i, 1, c["dtype"], dev)
    k = synth.centroid_noise(c["b"], c["h_kv"], c["s_k"], c["d"], 64, gq[:c["h_kv"]], c["sigma"], 700 + i, 2,
                             c["dtype"], dev)
    opts = dict(smooth_k=c["smooth_k"], causal=c["causal"], attention_sink=c["sink"])
    res = ops.build_block_map(q, k, c["topk"], c["thr"], cdfthreshd=c["cdf"], return_debug=True, **opts)
    torch.cuda.synchronize()
    ref = oracle.block_map(np64(q), np64(k), topk=c["topk"], simthreshd1=c["thr"], cdfthreshd=c["cdf"], **opts)
    # The absolute floor is 1e-6 of the larger of the means' rms and the
    # tokens' rms: with K smoothing and a single K block the exact mean is 0,
    # and the fp32 mean of the smoothed tokens is then rounding noise at the
    # tokens' scale.
    for key, x in (("q_mean", q), ("k_mean", k)):
        g, rr = np64(res[key]), ref[key]
        rms = max(math.sqrt(float((rr * rr).mean())), math.sqrt(float((np64(x) ** 2).mean())))
        assert (np.abs(g - rr) <= 1e-3 * np.abs(rr) + 1e-6 * rms).all(), f"{describe(c)}: {key}"
    thr_a = np.array(c["thr"])[None, :, None]
    far_q = np.abs(ref["sim_q_val"] - thr_a) > 1e-5
    assert np.array_equal(np64(res["sim_q"]).astype(bool)[far_q], ref["sim_q"][far_q]), f"{describe(c)}: sim_q"
    simk_val = np.repeat(ref["sim_k_val"], c["ratio"], axis=1)
    far_k = np.abs(simk_val - thr_a) > 1e-5
    assert np.array_equal(np64(res["sim_k"]).astype(bool)[far_k], ref["sim_k"][far_k]), f"{describe(c)}: sim_k"
    gp = np64(res["prob"])
    assert (np.abs(gp - ref["prob"]) <= 1e-3 * np.abs(ref["prob"]) + 1e-7).all(), f"{describe(c)}: prob"
    lut, cnt, bm = oracle.select_from_probs(gp, np64(res["sim_q"]).astype(bool), np64(res["sim_k"]).astype(bool),
                                            c["topk"], c["cdf"], causal=c["causal"], attention_sink=c["sink"])
    assert np.array_equal(res["lut"].cpu().numpy(), lut), f"{describe(c)}: LUT not bit-exact"
    assert np.array_equal(res["count"].cpu().numpy(), cnt), f"{describe(c)}: count not bit-exact"
    assert np.array_equal(res["bitmap"].cpu().numpy(), bm), f"{describe(c)}: bitmap not bit-exact"
