"""GPU selection with exactly equal pooled probabilities at the cut.

The selection takes blocks by pooled probability, largest first, and equal
probabilities go to the lower block index: the Vulkan page (llama.cpp pull
request 10) emits ties at a top-k threshold in ascending index order.  Here K
is built from a few distinct blocks, each repeated at several positions, so
every row holds only a few distinct pooled scores, each shared by several
blocks (identical tokens pool to identical means, so the GPU's scores and
probabilities of the copies are bit-identical).  Most cuts then fall inside
a group of equal probabilities, and only the tie rule decides which copies
are taken.  The LUT, count and bitmap must equal the oracle's selection run
on the GPU's own probabilities and gate flags, bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from block_sparse_attention_sparge_amd import ops, synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    ops.load_library()
    return torch.device("cuda:0")


def _tied(dev, b, h, s, d, dtype, n_distinct, seed):
    """Q as block-centroid + noise; K block j is a copy of K block
    perm[j % n_distinct], so the distinct blocks interleave along the row."""
    q = synth.centroid_noise(b, h, s, d, 64, [1.5] * h, 0.5, seed, 1, dtype, dev)
    k0 = synth.centroid_noise(b, h, s, d, 64, [1.5] * h, 0.5, seed, 2, dtype, dev)
    nk = s // 64
    src = torch.arange(nk, device=dev) % n_distinct
    src = torch.randperm(n_distinct, generator=torch.Generator().manual_seed(seed))[src.cpu()].to(dev)
    k = k0.view(b, h, nk, 64, d)[:, :, src].reshape(b, h, s, d).contiguous()
    return q, k


def _check(res, topk, cdf, causal=False):
    gp = res["prob"].double().cpu().numpy()
    sq = res["sim_q"].cpu().numpy().astype(bool)
    sk = res["sim_k"].cpu().numpy().astype(bool)
    lut, cnt, bm = oracle.select_from_probs(gp, sq, sk, topk, cdf, causal=causal)
    assert np.array_equal(res["lut"].cpu().numpy(), lut), "LUT not bit-exact"
    assert np.array_equal(res["count"].cpu().numpy(), cnt), "count not bit-exact"
    assert np.array_equal(res["bitmap"].cpu().numpy(), bm), "bitmap not bit-exact"
    return gp, cnt


def _cut_is_tied(p_row, n):
    """The n-th and (n+1)-th largest probabilities are exactly equal."""
    ps = np.sort(p_row)[::-1]
    return n < len(ps) and ps[n - 1] == ps[n]


@pytest.mark.parametrize("dtype,d", [(torch.float16, 128), (torch.bfloat16, 64)])
def test_topk_ties_at_the_cut_go_to_the_lower_block(dev, dtype, d):
    b, h, s = 2, 4, 2048                       # nk = 32: 4 distinct blocks x 8 copies
    q, k = _tied(dev, b, h, s, d, dtype, 4, 7)
    topk = [5 / 32, 11 / 32, 13 / 32, 21 / 32]  # cuts at 5, 11, 13, 21 (never a multiple of 8)
    res = ops.build_block_map(q, k, topk, [0.001] * h, return_debug=True)
    torch.cuda.synchronize()
    gp, cnt = _check(res, topk, None)
    assert np.all(res["sim_q"].cpu().numpy()) and np.all(res["sim_k"].cpu().numpy())
    tied = [_cut_is_tied(gp[ib, ih, qb], int(cnt[ib, ih, qb]))
            for ib in range(b) for ih in range(h) for qb in range(s // 64)]
    assert np.mean(tied) > 0.9, f"only {np.mean(tied):.2f} of the rows cut inside a tie group"


def test_cdf_ties_at_the_cut_go_to_the_lower_block(dev):
    b, h, s, d = 1, 4, 2048, 128
    q, k = _tied(dev, b, h, s, d, torch.float16, 4, 9)
    cdf = [0.1, 0.3, 0.55, 0.8]
    res = ops.build_block_map(q, k, [0.0] * h, [0.001] * h, cdfthreshd=cdf, return_debug=True)
    torch.cuda.synchronize()
    gp, cnt = _check(res, [0.0] * h, cdf)
    tied = [_cut_is_tied(gp[0, ih, qb], int(cnt[0, ih, qb])) for ih in range(h) for qb in range(s // 64)]
    assert np.mean(tied) > 0.5, f"only {np.mean(tied):.2f} of the rows cut inside a tie group"


def test_causal_ties(dev):
    # Causal rows see only blocks kb <= qb; the copies of each distinct block
    # among them still tie.  Two distinct blocks repeat along the row.
    b, h, s, d = 1, 2, 2048, 64
    q, k = _tied(dev, b, h, s, d, torch.bfloat16, 2, 13)
    topk = [7 / 32, 0.5]
    res = ops.build_block_map(q, k, topk, [0.001] * h, causal=True, return_debug=True)
    torch.cuda.synchronize()
    gp, cnt = _check(res, topk, None, causal=True)
    tied = [_cut_is_tied(gp[0, ih, qb], int(cnt[0, ih, qb])) for ih in range(h) for qb in range(s // 64)]
    assert np.mean(tied) > 0.5, f"only {np.mean(tied):.2f} of the rows cut inside a tie group"


@pytest.mark.parametrize("nk", [256, 384, 1024])
def test_topk_ties_on_long_rows(dev, nk):
    # Rows of more than 128 blocks take the radix select (histograms of the
    # probabilities' bytes) instead of the bisection, with 4, 8 and 16 key
    # slots per lane (384 blocks fill 6 of the 8).  K repeats 4 distinct
    # blocks along the row and the cuts fall inside groups of equal
    # probabilities.
    b, h, sq, d = 1, 4, 1024, 64
    sk = 64 * nk
    q = synth.centroid_noise(b, h, sq, d, 64, [1.5] * h, 0.5, 21, 1, torch.float16, dev)
    k0 = synth.centroid_noise(b, h, 64 * 4, d, 64, [1.5] * h, 0.5, 21, 2, torch.float16, dev)
    src = torch.randperm(4, generator=torch.Generator().manual_seed(nk))[torch.arange(nk) % 4].to(dev)
    k = k0.view(b, h, 4, 64, d)[:, :, src].reshape(b, h, sk, d).contiguous()
    cuts = [37, nk // 3 + 5, nk // 2 + 3, nk - 11]
    topk = [(n + 0.5) / nk for n in cuts]
    res = ops.build_block_map(q, k, topk, [0.001] * h, return_debug=True)
    torch.cuda.synchronize()
    gp, cnt = _check(res, topk, None)
    assert np.array_equal(cnt[0], np.array(cuts)[:, None].repeat(sq // 64, 1))
    tied = [_cut_is_tied(gp[0, ih, qb], int(cnt[0, ih, qb])) for ih in range(h) for qb in range(sq // 64)]
    assert np.mean(tied) > 0.9, f"only {np.mean(tied):.2f} of the rows cut inside a tie group"
