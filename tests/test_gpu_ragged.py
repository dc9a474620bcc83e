"""GPU parity on sequence lengths that are not multiples of 64.

Reading R1 (CK page, "Status vs Upstream": per-block mean pool): the last
block of a ragged sequence pools, gates and quantises only its own tokens; in
attention a partial last K block contributes only its existing keys and a
partial last Q-tile writes only its existing rows.  The bars are those of the
other parity tests: LUT, count and bitmap bit-exact against the oracle's
selection run on the GPU's pooled probabilities and flags; pooled means and
probabilities within 1e-3 relative; flags equal away from the threshold; int8
codes and scales bit-exact; O within atol 4e-2 / rtol 1e-2; LSE within 2e-3
nats with -inf exactly where the oracle has it.  Memory past the end of every
output is checked to be untouched.
"""
import math

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


def check_o(o_gpu, o_ref, keep=None):
    err = np.abs(np64(o_gpu) - o_ref)
    bad = err > O_ATOL + O_RTOL * np.abs(o_ref)
    if keep is not None:
        bad = bad[keep]
    assert not bad.any(), f"O: {bad.sum()} of {bad.size} outside atol/rtol; max err {err.max():.3e}"


def check_lse(l_gpu, l_ref):
    g = np64(l_gpu)
    assert np.array_equal(np.isneginf(g), np.isneginf(l_ref)), "-inf rows differ"
    fin = ~np.isneginf(l_ref)
    if fin.any():
        assert np.abs(g[fin] - l_ref[fin]).max() <= LSE_TOL


def _qkv(dev, b, h, h_kv, s_q, s_k, d, dtype, seed):
    gam = [0.5 + 1.5 * i / max(1, h - 1) for i in range(h)]
    q = synth.centroid_noise(b, h, s_q, d, 64, gam, 0.5, seed, 1, dtype, dev)
    k = synth.centroid_noise(b, h_kv, s_k, d, 64, gam[:h_kv], 0.5, seed, 2, dtype, dev)
    v = synth.normal((b, h_kv, s_k, d), seed, 3, dtype, dev)
    return q, k, v


def _check_map(res, q, k, topk, thr, cdf=None, **opts):
    h, h_kv = q.shape[1], k.shape[1]
    nq, nk = -(-q.shape[2] // 64), -(-k.shape[2] // 64)
    ref = oracle.block_map(np64(q), np64(k), topk=topk, simthreshd1=thr, cdfthreshd=cdf, **opts)
    assert tuple(res["lut"].shape) == (q.shape[0], h, nq, nk)
    for key in ("q_mean", "k_mean"):
        g, r = np64(res[key]), ref[key]
        rms = math.sqrt(float((r * r).mean()))
        assert (np.abs(g - r) <= 1e-3 * np.abs(r) + 1e-6 * rms).all(), key
    thr_a = np.array(thr)[None, :, None]
    far_q = np.abs(ref["sim_q_val"] - thr_a) > 1e-5
    assert np.array_equal(np64(res["sim_q"]).astype(bool)[far_q], ref["sim_q"][far_q])
    far_k = np.abs(np.repeat(ref["sim_k_val"], h // h_kv, axis=1) - thr_a) > 1e-5
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


# (s_q, s_k, h, h_kv): partial blocks of 1, 5, 8, 15, 40, 63 tokens, a query
# or key sequence shorter than one block, and GQA.
SHAPES = [(1000, 1000, 4, 4), (200, 333, 4, 2), (65, 130, 2, 2), (1, 64, 2, 1), (64, 1, 2, 2),
          (4033, 3000, 4, 2)]


@pytest.mark.parametrize("s_q,s_k,h,h_kv", SHAPES)
@pytest.mark.parametrize("dtype,d", [(torch.float16, 128), (torch.bfloat16, 64)])
def test_block_map(dev, s_q, s_k, h, h_kv, dtype, d):
    q, k, _ = _qkv(dev, 2, h, h_kv, s_q, s_k, d, dtype, s_q + s_k)
    topk = [0.25 + 0.125 * (i % 3) for i in range(h)]
    thr = [0.47 + 0.04 * (i % 2) for i in range(h)]
    res = ops.build_block_map(q, k, topk, thr, return_debug=True)
    torch.cuda.synchronize()
    _check_map(res, q, k, topk, thr)


@pytest.mark.parametrize("opts", [dict(smooth_k=True), dict(causal=True, attention_sink=True),
                                  dict(smooth_k=True, causal=True)])
def test_block_map_options(dev, opts):
    q, k, _ = _qkv(dev, 1, 4, 2, 1000, 1000, 128, torch.bfloat16, 5)
    topk, thr = [0.4] * 4, [0.001] * 4
    res = ops.build_block_map(q, k, topk, thr, return_debug=True, **opts)
    torch.cuda.synchronize()
    _check_map(res, q, k, topk, thr, **opts)


def test_block_map_cdf_mode(dev):
    q, k, _ = _qkv(dev, 1, 4, 4, 777, 901, 64, torch.float16, 6)
    cdf = [0.3, 0.6, 0.9, 0.99]
    res = ops.build_block_map(q, k, [0.0] * 4, [0.001] * 4, cdfthreshd=cdf, return_debug=True)
    torch.cuda.synchronize()
    _check_map(res, q, k, [0.0] * 4, [0.001] * 4, cdf=cdf)


@pytest.mark.parametrize("dtype,d", [(torch.float16, 128), (torch.bfloat16, 64)])
def test_int8_codes_and_no_write_past_the_end(dev, dtype, d):
    b, h, h_kv, s_q, s_k = 2, 4, 2, 300, 170
    q = synth.normal((b, h, s_q, d), 8, 1, dtype, dev, scale=3.0)
    k = synth.normal((b, h_kv, s_k, d), 8, 2, dtype, dev)
    q[1, 3, 256:] *= 50.0                        # the partial block of the last head: its own scale
    nq, nk = 5, 3
    sentinel = 77
    flat_q = torch.full((b * h * s_q * d + 4096,), sentinel, dtype=torch.int8, device=dev)
    flat_k = torch.full((b * h_kv * s_k * d + 4096,), sentinel, dtype=torch.int8, device=dev)
    out = dict(q_i8=flat_q[:b * h * s_q * d].view(b, h, s_q, d),
               k_i8=flat_k[:b * h_kv * s_k * d].view(b, h_kv, s_k, d))
    res = ops.build_block_map(q, k, [0.5] * h, [0.001] * h, quantize_int8=True, out=out)
    torch.cuda.synchronize()
    assert res["q_i8_scale"].shape == (b, h, nq) and res["k_i8_scale"].shape == (b, h_kv, nk)
    for x, key in ((q, "q_i8"), (k, "k_i8")):
        codes, scales = oracle.quantize_int8(x.float().cpu().numpy())
        assert np.array_equal(res[key].cpu().numpy(), codes), key
        assert np.array_equal(res[key + "_scale"].cpu().numpy(), scales), key
    assert (flat_q[b * h * s_q * d:] == sentinel).all() and (flat_k[b * h_kv * s_k * d:] == sentinel).all()


FMHA_SHAPES = [(1000, 1000, 4, 4), (200, 333, 4, 2), (65, 130, 2, 2), (1, 64, 2, 1), (64, 1, 2, 2),
               (127, 1, 2, 1), (130, 65, 2, 2), (63, 63, 2, 2)]


@pytest.mark.parametrize("s_q,s_k,h,h_kv", FMHA_SHAPES)
@pytest.mark.parametrize("dtype,d", [(torch.float16, 128), (torch.bfloat16, 64)])
def test_fmha_dense(dev, s_q, s_k, h, h_kv, dtype, d):
    q, k, v = _qkv(dev, 2, h, h_kv, s_q, s_k, d, dtype, 3 * s_q + s_k)
    o, lse = ops.sparse_fmha_fwd(q, k, v, None, None)
    torch.cuda.synchronize()
    ro, rl = oracle.block_sparse_attention(np64(q), np64(k), np64(v), None, None)
    check_o(o, ro)
    check_lse(lse, rl)


@pytest.mark.parametrize("s", [1000, 131, 63, 1])
@pytest.mark.parametrize("dtype,d", [(torch.float16, 128), (torch.bfloat16, 64)])
def test_fmha_causal_dense(dev, s, dtype, d):
    q, k, v = _qkv(dev, 1, 2, 2, s, s, d, dtype, 11 + s)
    o, lse = ops.sparse_fmha_fwd(q, k, v, None, None, causal=True)
    torch.cuda.synchronize()
    ro, rl = oracle.block_sparse_attention(np64(q), np64(k), np64(v), None, None, causal=True)
    check_o(o, ro)
    check_lse(lse, rl)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype,d", [(torch.float16, 128), (torch.bfloat16, 64)])
def test_map_then_fmha_with_splits(dev, causal, dtype, d):
    # The block map's LUT (partial last block listed or not), then the FMHA:
    # direct, fp32 partials over 3 splits merged by attn_combine.
    s = 2000
    q, k, v = _qkv(dev, 2, 4, 2, s, s, d, dtype, 21)
    bm = ops.build_block_map(q, k, [0.3] * 4, [0.001] * 4, causal=causal, attention_sink=causal)
    lut, cnt = bm["lut"], bm["count"]
    ro, rl = oracle.block_sparse_attention(np64(q), np64(k), np64(v), lut.cpu().numpy(), cnt.cpu().numpy(),
                                           causal=causal)
    last = (lut == 31).any(-1)
    assert last.any() and (~last).any()          # rows with and without the 16-key block
    o, lse = ops.sparse_fmha_fwd(q, k, v, lut, cnt, causal=causal)
    op, lp = ops.sparse_fmha_fwd(q, k, v, lut, cnt, causal=causal, num_splits=3)
    oc, lc = ops.attn_combine(op, lp, out_dtype=torch.float32)
    torch.cuda.synchronize()
    for oo, ll in ((o, lse), (oc, lc)):
        check_o(oo, ro)
        check_lse(ll, rl)


def test_fmha_empty_rows_and_no_write_past_the_end(dev):
    b, h, s_q, s_k, d = 2, 3, 150, 170, 128
    q, k, v = _qkv(dev, b, h, h, s_q, s_k, d, torch.float16, 31)
    nq, nk = 3, 3
    rng = np.random.default_rng(31)
    lut = np.full((b, h, nq, nk), -1, np.int32)
    cnt = np.zeros((b, h, nq), np.int32)
    for idx in np.ndindex(b, h, nq):
        m = 0 if rng.random() < 0.25 else int(rng.integers(1, nk + 1))
        sel = np.sort(rng.choice(nk, size=m, replace=False))
        lut[idx][:m] = sel
        cnt[idx] = m
    lut_t, cnt_t = torch.from_numpy(lut).to(dev), torch.from_numpy(cnt).to(dev)
    big = torch.full((b, h, s_q + 64, d), float("nan"), dtype=torch.float16, device=dev)
    o = big[:, :, :s_q]
    flat = torch.full((b * h * s_q + 256,), 123.0, dtype=torch.float32, device=dev)
    lse = flat[:b * h * s_q].view(b, h, s_q)
    ops.sparse_fmha_fwd(q, k, v, lut_t, cnt_t, o=o, lse=lse)
    torch.cuda.synchronize()
    ro, rl = oracle.block_sparse_attention(np64(q), np64(k), np64(v), lut, cnt)
    check_o(o, ro)
    check_lse(lse, rl)
    assert torch.isnan(big[:, :, s_q:]).all(), "rows past s_q were written"
    assert (flat[b * h * s_q:] == 123.0).all(), "LSE past the end was written"


@pytest.mark.parametrize("tau", [0.5, 1.5])
def test_pv_threshold(dev, tau):
    # Keys that decay block by block, so many blocks fall below the running
    # maximum of every row of a tile; a partial Q-tile of 40 rows and a
    # partial K block of 44.
    b, h, s_q, s_k, d = 1, 2, 424, 940, 128
    g = torch.Generator(device=dev).manual_seed(41)
    q = (4.0 * torch.randn(b, h, s_q, d, generator=g, device=dev)).half()
    scale = torch.pow(2.0, -0.5 * (torch.arange(s_k, device=dev) // 64).float())
    k = (torch.randn(b, h, s_k, d, generator=g, device=dev) * scale[:, None]).half()
    v = torch.randn(b, h, s_k, d, generator=g, device=dev).half()
    o, lse = ops.sparse_fmha_fwd(q, k, v, None, None, pv_threshold=tau)
    torch.cuda.synchronize()
    ro, rl, ns, nu, near = oracle.block_sparse_attention_pv_skip(
        np64(q), np64(k), np64(v), None, None, tau, return_skips=True, return_margins=True)
    assert 0 < ns < nu
    keep = np.repeat(near >= 1e-3, 64, axis=-1)[:, :, :s_q]
    assert keep.mean() > 0.8
    check_o(o, ro, keep=np.broadcast_to(keep[..., None], ro.shape))
    check_lse(lse, rl)
    ex, _ = oracle.block_sparse_attention(np64(q), np64(k), np64(v), None, None)
    assert np.abs(ro - ex)[keep].max() > 1.5 * O_ATOL, "the skips in this case are too small to see"


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype,d", [(torch.float16, 128), (torch.bfloat16, 64)])
def test_int8_end_to_end(dev, causal, dtype, d):
    s = 1000
    q, k, v = _qkv(dev, 2, 4, 2, s, s, d, dtype, 51)
    bm = ops.build_block_map(q, k, [0.4] * 4, [0.001] * 4, causal=causal, attention_sink=causal,
                             quantize_int8=True)
    o, lse = ops.sparse_fmha_fwd_qk_int8(bm["q_i8"], bm["q_i8_scale"], bm["k_i8"], bm["k_i8_scale"], v,
                                         bm["lut"], bm["count"], causal=causal)
    torch.cuda.synchronize()
    ro, rl = oracle.block_sparse_attention_qk_int8(np64(q), np64(k), np64(v), bm["lut"].cpu().numpy(),
                                                   bm["count"].cpu().numpy(), causal=causal)
    check_o(o, ro)
    check_lse(lse, rl)


def _nan_padded(x):
    """x viewed at the start of a buffer that holds whole 64-row blocks; the
    elements past x are NaN."""
    b, h, s, d = x.shape
    assert b * h == 1
    buf = torch.full((-(-s // 64) * 64 * d,), float("nan"), dtype=x.dtype, device=x.device)
    buf[: s * d] = x.reshape(-1)
    return buf[: s * d].view(b, h, s, d)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype,d", [(torch.float16, 128), (torch.bfloat16, 64)])
def test_fmha_tail_rows_read_as_zeros(dev, causal, dtype, d):
    # K and V sit at the start of buffers whose elements past the sequence
    # are NaN.  The missing rows of the last 64-key block must arrive as
    # zeros (the loads' range check ends at the last existing row), never as
    # the NaN behind them: P = 0 times NaN would make O NaN.
    s = 1000
    q, k, v = _qkv(dev, 1, 1, 1, s, s, d, dtype, 71)
    k, v = _nan_padded(k), _nan_padded(v)
    o, lse = ops.sparse_fmha_fwd(q, k, v, None, None, causal=causal)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and not torch.isnan(lse).any()
    ro, rl = oracle.block_sparse_attention(np64(q), np64(k), np64(v), None, None, causal=causal)
    check_o(o, ro)
    check_lse(lse, rl)
    bm = ops.build_block_map(q, k, [1.0], [0.001], causal=causal, quantize_int8=True)
    o8, l8 = ops.sparse_fmha_fwd_qk_int8(bm["q_i8"], bm["q_i8_scale"], bm["k_i8"], bm["k_i8_scale"], v,
                                         bm["lut"], bm["count"], causal=causal)
    torch.cuda.synchronize()
    assert torch.isfinite(o8).all() and not torch.isnan(l8).any()
    ro8, rl8 = oracle.block_sparse_attention_qk_int8(np64(q), np64(k), np64(v), bm["lut"].cpu().numpy(),
                                                     bm["count"].cpu().numpy(), causal=causal)
    check_o(o8, ro8)
    check_lse(l8, rl8)


@pytest.mark.parametrize("s_q,s_k", [(200, 333), (1, 64), (130, 65)])
def test_int8_dense_ragged_shapes(dev, s_q, s_k):
    q, k, v = _qkv(dev, 1, 4, 2, s_q, s_k, 128, torch.float16, 61)
    cq, sq = oracle.quantize_int8(q.float().cpu().numpy())
    ck, sk = oracle.quantize_int8(k.float().cpu().numpy())
    o, lse = ops.sparse_fmha_fwd_qk_int8(torch.from_numpy(cq).to(dev), torch.from_numpy(sq).to(dev),
                                         torch.from_numpy(ck).to(dev), torch.from_numpy(sk).to(dev), v)
    torch.cuda.synchronize()
    ro, rl = oracle.block_sparse_attention_qk_int8(np64(q), np64(k), np64(v), None, None)
    check_o(o, ro)
    check_lse(lse, rl)


@pytest.mark.parametrize("s", [640, 1000])
def test_int8_causal_with_all_zero_blocks(dev, s):
    # An all-zero Q block and an all-zero K block have scale 0; under the
    # causal mask their removed keys must still score -inf (not -inf * 0).
    q, k, v = _qkv(dev, 1, 2, 2, s, s, 128, torch.bfloat16, 71)
    q[0, 0, 128:192] = 0
    q[0, 1, 64 * (s // 64):] = 0                 # the last (partial when s = 1000) Q block
    k[0, 0, 128:192] = 0
    k[0, 1, 0:64] = 0
    bm = ops.build_block_map(q, k, [1.0, 1.0], [0.001, 0.001], causal=True, quantize_int8=True)
    assert bm["q_i8_scale"][0, 0, 2].item() == 0.0 and bm["k_i8_scale"][0, 1, 0].item() == 0.0
    o, lse = ops.sparse_fmha_fwd_qk_int8(bm["q_i8"], bm["q_i8_scale"], bm["k_i8"], bm["k_i8_scale"], v,
                                         None, None, causal=True)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    ro, rl = oracle.block_sparse_attention_qk_int8(np64(q), np64(k), np64(v), None, None, causal=True)
    check_o(o, ro)
    check_lse(lse, rl)
