"""GPU parity at the limits the boundary states.

* The block map's per-head knobs up to SPARGE_MAX_HEADS = 128 heads (topk,
  simthreshd1 and cdfthreshd differ from head to head; CK page, "Status vs
  Upstream": per-head topk / simthreshd1 / cdfthreshd).
* The token-list mode at its limit of 65536 query rows per KV head (aiter
  4919 page: gfx950 sparse decode with split-K).
* num_splits = 1024, the most split partials attn_combine takes (Updating Log
  page, Stage 1: the LSE combine; an empty split is the identity).

Bars as in the other parity tests: LUT, count and bitmap bit-exact against
the oracle's selection on the GPU's P and flags, P within 1e-3 relative, O
within atol 4e-2 / rtol 1e-2, LSE within 2e-3 nats with -inf matching.
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


def _map_case(dev, h, seed):
    # Heads from flat (gamma 0.3) to peaked (gamma 2.5) pooled softmax, K with
    # a quarter of the heads' blocks made of +-v pairs (similarity 0, so the
    # K gate fails there at any positive threshold).
    b, s, d = 1, 512, 64
    gam = [0.3 + 2.2 * i / (h - 1) for i in range(h)]
    q = synth.centroid_noise(b, h, s, d, 64, gam, 0.5, seed, 1, torch.float16, dev)
    k = synth.centroid_noise(b, h, s, d, 64, gam, 0.5, seed, 2, torch.float16, dev)
    for hh in range(0, h, 4):
        kb = (hh // 4) % (s // 64)
        v = k[0, hh, 64 * kb].clone()
        k[0, hh, 64 * kb:64 * kb + 64:2] = v
        k[0, hh, 64 * kb + 1:64 * kb + 64:2] = -v
    return q, k


def _check_against_oracle(res, q, k, topk, thr, cdf):
    ref = oracle.block_map(np64(q), np64(k), topk=topk, simthreshd1=thr, cdfthreshd=cdf)
    thr_a = np.array(thr)[None, :, None]
    for g_key, r_key, v_key in (("sim_q", "sim_q", "sim_q_val"), ("sim_k", "sim_k", "sim_k_val")):
        far = np.abs(ref[v_key] - thr_a) > 1e-5
        assert np.array_equal(np64(res[g_key]).astype(bool)[far], ref[r_key][far]), g_key
    gp = np64(res["prob"])
    assert (np.abs(gp - ref["prob"]) <= 1e-3 * np.abs(ref["prob"]) + 1e-7).all(), "pooled prob"
    lut, cnt, bm = oracle.select_from_probs(gp, np64(res["sim_q"]).astype(bool),
                                            np64(res["sim_k"]).astype(bool), topk, cdf)
    assert np.array_equal(res["lut"].cpu().numpy(), lut), "LUT not bit-exact"
    assert np.array_equal(res["count"].cpu().numpy(), cnt), "count not bit-exact"
    assert np.array_equal(res["bitmap"].cpu().numpy(), bm), "bitmap not bit-exact"
    return ref


def test_block_map_128_heads_topk(dev):
    h = 128
    q, k = _map_case(dev, h, 3)
    topk = [(1 + i % 8) / 8 for i in range(h)]                   # 1..8 of 8 blocks
    thr = [0.001 if i % 3 else 0.5 for i in range(h)]            # 0.5 closes some Q and K gates
    res = ops.build_block_map(q, k, topk, thr, return_debug=True)
    torch.cuda.synchronize()
    ref = _check_against_oracle(res, q, k, topk, thr, None)
    cnt = res["count"].cpu().numpy()[0]
    # The per-head count reaches the last head: heads with an open Q gate and
    # no forced K block select exactly floor(topk * 8) blocks.
    open_rows = ref["sim_q"][0] & ~(~ref["sim_k"][0]).any(-1)[:, None]
    expect = np.array([int(np.floor(np.float32(t) * 8)) for t in topk])[:, None]
    assert open_rows[-8:].any()
    assert np.array_equal(cnt[open_rows], np.broadcast_to(expect, cnt.shape)[open_rows])


def test_block_map_128_heads_cdf(dev):
    h = 128
    q, k = _map_case(dev, h, 4)
    cdf = [0.2 + 0.79 * i / (h - 1) for i in range(h)]
    thr = [0.001] * h
    res = ops.build_block_map(q, k, [0.0] * h, thr, cdfthreshd=cdf, return_debug=True)
    torch.cuda.synchronize()
    _check_against_oracle(res, q, k, [0.0] * h, thr, cdf)


def test_decode_65536_rows_per_kv_head(dev):
    # h_q / h_kv * s_q = 8 * 8192 = 65536 query rows share each KV head's list.
    b, h_q, h_kv, s_q, s_k, d, L = 1, 16, 2, 8192, 4096, 128, 96
    q = synth.normal((b, h_q, s_q, d), 81, 1, torch.bfloat16, dev, scale=4.0)
    k = synth.normal((b, h_kv, s_k, d), 81, 2, torch.bfloat16, dev)
    v = synth.normal((b, h_kv, s_k, d), 81, 3, torch.bfloat16, dev)
    lists = synth.token_lists(b, h_kv, L, s_k, 81, 4, True).to(dev)
    o, lse = ops.sparse_fmha_fwd(q, k, v, lists, None, blk_q=1, blk_k=1)
    op, lp = ops.sparse_fmha_fwd(q, k, v, lists, None, blk_q=1, blk_k=1, num_splits=3)
    oc, lc = ops.attn_combine(op, lp, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ro, rl = oracle.token_list_attention(np64(q), np64(k), np64(v), lists.cpu().numpy())
    for oo, ll in ((o, lse), (oc, lc)):
        check_o(oo, ro)
        check_lse(ll, rl)


@pytest.mark.parametrize("causal", [False, True])
def test_fmha_1024_splits(dev, causal):
    # Rows of up to 6 blocks split 1024 ways: almost every partial is empty
    # (O = 0, LSE = -inf) and the combine must treat them as the identity.
    b, h, s, d = 1, 2, 384, 64
    q = synth.normal((b, h, s, d), 91, 1, torch.float16, dev)
    k = synth.normal((b, h, s, d), 91, 2, torch.float16, dev)
    v = synth.normal((b, h, s, d), 91, 3, torch.float16, dev)
    op, lp = ops.sparse_fmha_fwd(q, k, v, None, None, num_splits=1024, causal=causal)
    assert op.shape[0] == 1024
    oc, lc = ops.attn_combine(op, lp, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.isneginf(lp[6:]).all() and (op[6:] == 0).all()
    ro, rl = oracle.block_sparse_attention(np64(q), np64(k), np64(v), None, None, causal=causal)
    check_o(oc, ro)
    check_lse(lc, rl)
