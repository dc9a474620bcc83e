"""GPU parity for the fp8 (e4m3) Q/K path: quantisation in the block map and
the fp8-QK sparse FMHA.

CK page, "Status vs Upstream", not-yet-ported list: Q/K quantisation in the
pool kernel feeding a low-precision QK product in the attention kernel; the
aiter 6841 page runs fp8 Q/K recipes (reading R29: per 64-token block, scale
absmax / 448, x * (448 / absmax) rounded to the OCP e4m3 grid to nearest even,
in fp32).  The codes are decided in fp32 and must have the oracle's values
bit for bit (compared as e4m3 values: a negative zero equals zero).
Attention on the codes is held to the bars of the other attention tests (O
atol 4e-2 / rtol 1e-2, LSE 2e-3 nats, -inf exact) against the oracle's
attention on its own codes.
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


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    ops.load_library()
    return torch.device("cuda:0")


def _check_codes(res, q, k):
    for x, key in ((q, "q_fp8"), (k, "k_fp8")):
        codes, scales = oracle.quantize_fp8(x.float().cpu().numpy())
        got = oracle.e4m3_value(res[key].cpu().numpy())
        bad = got != codes
        assert not bad.any(), f"{key}: {bad.sum()} codes differ, e.g. {got[bad][:4]} vs {codes[bad][:4]}"
        assert np.array_equal(res[key + "_scale"].cpu().numpy(), scales), f"{key} scales not bit-exact"


def _attn_ref(q, k, v, lut, cnt, per_kv=False, causal=False):
    return oracle.block_sparse_attention_qk_fp8(
        np64(q), np64(k), np64(v), None if lut is None else lut.cpu().numpy(),
        None if cnt is None else cnt.cpu().numpy(), lut_per_kv_head=per_kv, causal=causal)


def _fmha(bm, v, lut, cnt, **kw):
    return ops.sparse_fmha_fwd_qk_fp8(bm["q_fp8"], bm["q_fp8_scale"], bm["k_fp8"], bm["k_fp8_scale"], v,
                                      lut, cnt, **kw)


@pytest.mark.parametrize("smooth_k", [False, True])
def test_block_map_codes_tiny_and_unchanged_selection(dev, smooth_k):
    case = synth.tiny_case(dev, seed=3)
    plain = ops.build_block_map(case.q, case.k, case.topk, case.simthreshd1, return_debug=True,
                                smooth_k=smooth_k)
    res = ops.build_block_map(case.q, case.k, case.topk, case.simthreshd1, return_debug=True,
                              smooth_k=smooth_k, quantize_fp8=True)
    torch.cuda.synchronize()
    _check_codes(res, case.q, case.k)
    for key in ("lut", "count", "bitmap", "prob", "q_mean", "k_mean"):
        assert torch.equal(plain[key], res[key]), key


@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 128), (torch.float16, 64)])
def test_block_map_codes_with_zero_tiny_and_extreme_blocks(dev, dtype, d):
    b, h, s = 2, 3, 1024
    q = synth.normal((b, h, s, d), 31, 1, dtype, dev, scale=3.0)
    k = synth.normal((b, h, s, d), 31, 2, dtype, dev)
    q[0, 0, 64:128] = 0                      # an all-zero block: scale 0, codes 0
    k[1, 2, :64] *= 1000.0                   # a block of large values
    k[0, 1, 128:192] *= 1e-3                 # small values: many subnormal codes
    k[0, 1, 130, 5] = 50.0                   # one large entry: the rest fall to tiny codes
    res = ops.build_block_map(q, k, [0.5] * h, [0.001] * h, quantize_fp8=True)
    torch.cuda.synchronize()
    _check_codes(res, q, k)
    assert res["q_fp8_scale"][0, 0, 1].item() == 0.0
    sub = oracle.e4m3_value(res["k_fp8"][0, 1, 128:192].cpu().numpy())
    assert np.any((sub != 0) & (np.abs(sub) < 2.0 ** -6)), "no subnormal code was exercised"


def test_block_map_codes_mid_and_ragged(dev):
    case = synth.mid_case(dev)
    res = ops.build_block_map(case.q, case.k, case.topk, case.simthreshd1, quantize_fp8=True)
    torch.cuda.synchronize()
    _check_codes(res, case.q, case.k)
    q, k = case.q[:, :, :1000], case.k[:, :, :1000]     # a partial last block of 40 tokens
    res = ops.build_block_map(q, k, case.topk, case.simthreshd1, quantize_fp8=True)
    torch.cuda.synchronize()
    _check_codes(res, q, k)


@pytest.mark.parametrize("topk", [0.4, 1.0])
def test_end_to_end_mid(dev, topk):
    case = synth.mid_case(dev, topk=topk)
    bm = ops.build_block_map(case.q, case.k, case.topk, case.simthreshd1, quantize_fp8=True)
    o, lse = _fmha(bm, case.v, bm["lut"], bm["count"])
    torch.cuda.synchronize()
    ro, rl = _attn_ref(case.q, case.k, case.v, bm["lut"], bm["count"])
    check_o(o, ro)
    check_lse(lse, rl)


def test_end_to_end_tiny_fp16_d64(dev):
    case = synth.tiny_case(dev)
    bm = ops.build_block_map(case.q, case.k, case.topk, case.simthreshd1, quantize_fp8=True)
    o, lse = _fmha(bm, case.v, bm["lut"], bm["count"])
    torch.cuda.synchronize()
    ro, rl = _attn_ref(case.q, case.k, case.v, bm["lut"], bm["count"])
    check_o(o, ro)
    check_lse(lse, rl)


@pytest.mark.parametrize("per_kv", [False, True])
def test_gqa_empty_rows_fp32_out(dev, per_kv):
    b, hq, hkv, s, d = 2, 4, 2, 512, 128
    q = synth.centroid_noise(b, hq, s, d, 64, [1.0, 1.5, 2.0, 0.5], 0.4, 9, 1, torch.bfloat16, dev)
    k = synth.centroid_noise(b, hkv, s, d, 64, [1.0, 1.5], 0.4, 9, 2, torch.bfloat16, dev)
    v = synth.normal((b, hkv, s, d), 9, 3, torch.bfloat16, dev)
    bm = ops.build_block_map(q, k, [0.5] * hq, [0.001] * hq, quantize_fp8=True)
    hl = hkv if per_kv else hq
    nq = s // 64
    g = torch.Generator().manual_seed(5)
    lut = torch.full((b, hl, nq, nq), -1, dtype=torch.int32)
    cnt = torch.zeros((b, hl, nq), dtype=torch.int32)
    for i in range(b * hl * nq):
        n = int(torch.randint(0, nq + 1, (1,), generator=g)) if i % 5 else 0     # every fifth row empty
        sel = torch.sort(torch.randperm(nq, generator=g)[:n]).values
        lut.view(-1, nq)[i, :n] = sel.to(torch.int32)
        cnt.view(-1)[i] = n
    lut, cnt = lut.to(dev), cnt.to(dev)
    o, lse = _fmha(bm, v, lut, cnt, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ro, rl = _attn_ref(q, k, v, lut, cnt, per_kv=per_kv)
    check_o(o, ro)
    check_lse(lse, rl)


@pytest.mark.parametrize("splits", [2, 5])
def test_splits_then_combine(dev, splits):
    case = synth.mid_case(dev)
    bm = ops.build_block_map(case.q, case.k, case.topk, case.simthreshd1, quantize_fp8=True)
    op, lp = _fmha(bm, case.v, bm["lut"], bm["count"], num_splits=splits)
    o, lse = ops.attn_combine(op, lp, out_dtype=case.v.dtype)
    torch.cuda.synchronize()
    ro, rl = _attn_ref(case.q, case.k, case.v, bm["lut"], bm["count"])
    check_o(o, ro)
    check_lse(lse, rl)


@pytest.mark.parametrize("s", [1024, 1000])
def test_causal_block_map_end_to_end(dev, s):
    # Causal mask, sink and smoothing in the block map; the causal fp8 FMHA
    # (also the ragged-K kernel when s is not a multiple of 64).
    case = synth.mid_case(dev)
    q, k, v = case.q[:, :, :s], case.k[:, :, :s], case.v[:, :, :s]
    bm = ops.build_block_map(q, k, case.topk, case.simthreshd1, causal=True, attention_sink=True,
                             smooth_k=True, quantize_fp8=True)
    o, lse = _fmha(bm, v, bm["lut"], bm["count"], causal=True)
    torch.cuda.synchronize()
    ro, rl = _attn_ref(q, k, v, bm["lut"], bm["count"], causal=True)
    check_o(o, ro)
    check_lse(lse, rl)


def test_headline_codes_and_sampled_heads(dev):
    case = synth.headline_case(dev, topk=0.4)
    bm = ops.build_block_map(case.q, case.k, case.topk, case.simthreshd1, quantize_fp8=True)
    o, lse = _fmha(bm, case.v, bm["lut"], bm["count"])
    torch.cuda.synchronize()
    heads = [0, 31]
    sub = {key: bm[key][:, heads] for key in ("q_fp8", "q_fp8_scale", "k_fp8", "k_fp8_scale")}
    _check_codes(sub, case.q[:, heads], case.k[:, heads])
    ro, rl = _attn_ref(case.q[:, heads], case.k[:, heads], case.v[:, heads], bm["lut"][:, heads],
                       bm["count"][:, heads])
    check_o(o[:, heads], ro)
    check_lse(lse[:, heads], rl)


def test_binding_refuses_int8_codes_for_fp8(dev):
    case = synth.tiny_case(dev)
    bm = ops.build_block_map(case.q, case.k, case.topk, case.simthreshd1, quantize_int8=True)
    with pytest.raises(ops.SpargeError):
        ops.sparse_fmha_fwd_qk_fp8(bm["q_i8"], bm["q_i8_scale"], bm["k_i8"], bm["k_i8_scale"], case.v,
                                   bm["lut"], bm["count"])
