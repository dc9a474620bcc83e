"""GPU parity for the int8 Q/K path: quantisation in the block map and the
int8-QK sparse FMHA.

CK page, "Status vs Upstream", not-yet-ported list: Q/K int8 quantisation in
the pool kernel feeding an int8 QK product in the attention kernel (reading
R27: per 64-token block, scale absmax / 127, round half to even in fp32).
The codes and scales are integer work decided in fp32 and must match the
oracle bit for bit.  Attention on the codes is held to the bars of the other
attention tests (O atol 4e-2 / rtol 1e-2, LSE 2e-3 nats, -inf exact) against
the oracle's attention on its own codes.
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
    for x, key in ((q, "q_i8"), (k, "k_i8")):
        codes, scales = oracle.quantize_int8(x.float().cpu().numpy())
        assert np.array_equal(res[key].cpu().numpy(), codes), f"{key} codes not bit-exact"
        assert np.array_equal(res[key + "_scale"].cpu().numpy(), scales), f"{key} scales not bit-exact"


@pytest.mark.parametrize("smooth_k", [False, True])
def test_block_map_codes_tiny_and_unchanged_selection(dev, smooth_k):
    case = synth.tiny_case(dev, seed=3)
    plain = ops.build_block_map(case.q, case.k, case.topk, case.simthreshd1, return_debug=True,
                                smooth_k=smooth_k)
    res = ops.build_block_map(case.q, case.k, case.topk, case.simthreshd1, return_debug=True,
                              smooth_k=smooth_k, quantize_int8=True)
    torch.cuda.synchronize()
    _check_codes(res, case.q, case.k)
    for key in ("lut", "count", "bitmap", "prob", "q_mean", "k_mean"):
        assert torch.equal(plain[key], res[key]), key


@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 128), (torch.float16, 64)])
def test_block_map_codes_with_zero_and_extreme_blocks(dev, dtype, d):
    b, h, s = 2, 3, 1024
    q = synth.normal((b, h, s, d), 31, 1, dtype, dev, scale=3.0)
    k = synth.normal((b, h, s, d), 31, 2, dtype, dev)
    q[0, 0, 64:128] = 0                      # an all-zero block: scale 0, codes 0
    k[1, 2, :64] *= 1000.0                   # a block of large values
    k[0, 1, 128:192] = 0
    k[0, 1, 130, 5] = -1e-3                  # a block with one tiny entry (code -127)
    res = ops.build_block_map(q, k, [0.5] * h, [0.001] * h, quantize_int8=True)
    torch.cuda.synchronize()
    _check_codes(res, q, k)
    assert res["q_i8_scale"][0, 0, 1].item() == 0.0


def test_block_map_codes_mid(dev):
    case = synth.mid_case(dev)
    res = ops.build_block_map(case.q, case.k, case.topk, case.simthreshd1, quantize_int8=True)
    torch.cuda.synchronize()
    _check_codes(res, case.q, case.k)


def _attn_ref(q, k, v, lut, cnt, per_kv=False, causal=False):
    return oracle.block_sparse_attention_qk_int8(
        np64(q), np64(k), np64(v), None if lut is None else lut.cpu().numpy(),
        None if cnt is None else cnt.cpu().numpy(), lut_per_kv_head=per_kv, causal=causal)


@pytest.mark.parametrize("topk", [0.4, 1.0])
def test_end_to_end_mid(dev, topk):
    case = synth.mid_case(dev, topk=topk)
    bm = ops.build_block_map(case.q, case.k, case.topk, case.simthreshd1, quantize_int8=True)
    o, lse = ops.sparse_fmha_fwd_qk_int8(bm["q_i8"], bm["q_i8_scale"], bm["k_i8"], bm["k_i8_scale"],
                                         case.v, bm["lut"], bm["count"])
    torch.cuda.synchronize()
    ro, rl = _attn_ref(case.q, case.k, case.v, bm["lut"], bm["count"])
    check_o(o, ro)
    check_lse(lse, rl)


def test_end_to_end_tiny_fp16_d64(dev):
    case = synth.tiny_case(dev)
    bm = ops.build_block_map(case.q, case.k, case.topk, case.simthreshd1, quantize_int8=True)
    o, lse = ops.sparse_fmha_fwd_qk_int8(bm["q_i8"], bm["q_i8_scale"], bm["k_i8"], bm["k_i8_scale"],
                                         case.v, bm["lut"], bm["count"])
    torch.cuda.synchronize()
    ro, rl = _attn_ref(case.q, case.k, case.v, bm["lut"], bm["count"])
    check_o(o, ro)
    check_lse(lse, rl)


def _codes_on_gpu(x, dev):
    codes, scales = oracle.quantize_int8(x.float().cpu().numpy())
    return torch.from_numpy(codes).to(dev), torch.from_numpy(scales).to(dev)


@pytest.mark.parametrize("dtype,d", [(torch.float16, 128), (torch.bfloat16, 64)])
@pytest.mark.parametrize("per_kv", [False, True])
def test_gqa_empty_rows_fp32_out_and_splits(dev, dtype, d, per_kv):
    b, hq, hkv, s = 2, 4, 2, 768
    nq = s // 64
    q = synth.normal((b, hq, s, d), 41, 1, dtype, dev, scale=2.0)
    k = synth.normal((b, hkv, s, d), 41, 2, dtype, dev)
    v = synth.normal((b, hkv, s, d), 41, 3, dtype, dev)
    q8, qs = _codes_on_gpu(q, dev)
    k8, ks = _codes_on_gpu(k, dev)
    hl = hkv if per_kv else hq
    rng = np.random.default_rng(42)
    lut = np.full((b, hl, nq, nq), -1, dtype=np.int32)
    cnt = np.zeros((b, hl, nq), dtype=np.int32)
    for idx in np.ndindex(b, hl, nq):
        m = 0 if rng.random() < 0.15 else int(rng.integers(1, nq + 1))
        sel = np.sort(rng.choice(nq, size=m, replace=False))
        lut[idx][:m] = sel
        cnt[idx] = m
    lut_t, cnt_t = torch.from_numpy(lut).to(dev), torch.from_numpy(cnt).to(dev)
    ro, rl = _attn_ref(q, k, v, lut_t, cnt_t, per_kv=per_kv)
    o, lse = ops.sparse_fmha_fwd_qk_int8(q8, qs, k8, ks, v, lut_t, cnt_t, out_dtype=torch.float32)
    torch.cuda.synchronize()
    check_o(o, ro)
    check_lse(lse, rl)
    op, lp = ops.sparse_fmha_fwd_qk_int8(q8, qs, k8, ks, v, lut_t, cnt_t, num_splits=3)
    oc, lc = ops.attn_combine(op, lp, out_dtype=dtype)
    torch.cuda.synchronize()
    check_o(oc, ro)
    check_lse(lc, rl)


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
def test_causal_dense(dev, dtype):
    b, h, s, d = 1, 3, 640, 128
    q = synth.normal((b, h, s, d), 51, 1, dtype, dev)
    k = synth.normal((b, h, s, d), 51, 2, dtype, dev)
    v = synth.normal((b, h, s, d), 51, 3, dtype, dev)
    q8, qs = _codes_on_gpu(q, dev)
    k8, ks = _codes_on_gpu(k, dev)
    o, lse = ops.sparse_fmha_fwd_qk_int8(q8, qs, k8, ks, v, None, None, causal=True)
    torch.cuda.synchronize()
    ro, rl = _attn_ref(q, k, v, None, None, causal=True)
    check_o(o, ro)
    check_lse(lse, rl)


def test_headline_sampled_heads(dev):
    # b2 h32 s16384 d128 fp16 at topk 0.4: codes of the whole workload bit-exact,
    # attention of heads 0 and 31 of both batches against the oracle.
    case = synth.headline_case(dev, topk=0.4)
    bm = ops.build_block_map(case.q, case.k, case.topk, case.simthreshd1, quantize_int8=True)
    o, lse = ops.sparse_fmha_fwd_qk_int8(bm["q_i8"], bm["q_i8_scale"], bm["k_i8"], bm["k_i8_scale"],
                                         case.v, bm["lut"], bm["count"])
    torch.cuda.synchronize()
    _check_codes(bm, case.q, case.k)
    heads = [0, 31]
    ro, rl = _attn_ref(case.q[:, heads], case.k[:, heads], case.v[:, heads], bm["lut"][:, heads],
                       bm["count"][:, heads])
    check_o(o[:, heads], ro)
    check_lse(lse[:, heads], rl)


def test_causal_end_to_end_with_smoothing_and_sink(dev):
    # Causal block map (K smoothing, attention sink) with the int8 codes, then
    # the causal int8-QK FMHA on its LUT.
    case = synth.mid_case(dev)
    bm = ops.build_block_map(case.q, case.k, case.topk, case.simthreshd1, smooth_k=True, causal=True,
                             attention_sink=True, quantize_int8=True)
    o, lse = ops.sparse_fmha_fwd_qk_int8(bm["q_i8"], bm["q_i8_scale"], bm["k_i8"], bm["k_i8_scale"],
                                         case.v, bm["lut"], bm["count"], causal=True)
    torch.cuda.synchronize()
    _check_codes(bm, case.q, case.k)
    ro, rl = _attn_ref(case.q, case.k, case.v, bm["lut"], bm["count"], causal=True)
    check_o(o, ro)
    check_lse(lse, rl)


def test_strided_views(dev):
    # Codes and V read through views with padded rows and a transposed
    # (b, s, h, d) storage order; the output written into a padded view.
    b, h, s, d = 2, 3, 512, 128
    q = synth.normal((b, h, s, d), 71, 1, torch.float16, dev)
    k = synth.normal((b, h, s, d), 71, 2, torch.float16, dev)
    v = synth.normal((b, h, s, d), 71, 3, torch.float16, dev)
    q8, qs = _codes_on_gpu(q, dev)
    k8, ks = _codes_on_gpu(k, dev)
    q8p = torch.zeros((b, h, s, d + 32), dtype=torch.int8, device=dev)[..., :d]
    q8p.copy_(q8)
    k8t = k8.transpose(1, 2).contiguous().transpose(1, 2)           # (b, s, h, d) storage
    vt = v.transpose(1, 2).contiguous().transpose(1, 2)
    o = torch.zeros((b, h, s, d + 64), dtype=torch.float16, device=dev)[..., :d]
    nq = s // 64
    lut = torch.arange(nq, dtype=torch.int32, device=dev).flip(0).sort().values.repeat(b, h, nq, 1).contiguous()
    cnt = torch.full((b, h, nq), nq, dtype=torch.int32, device=dev)
    _, lse = ops.sparse_fmha_fwd_qk_int8(q8p, qs, k8t, ks, vt, lut, cnt, o=o)
    torch.cuda.synchronize()
    ro, rl = _attn_ref(q, k, v, lut, cnt)
    check_o(o, ro)
    check_lse(lse, rl)
