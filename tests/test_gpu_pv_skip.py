"""GPU parity for the pv_threshold skip in the block-mode FMHA.

CK page, "Status vs Upstream", not-yet-ported list: pv_threshold, a per-Q-tile
skip inside the attention kernel.  The kernel takes one decision per (Q-tile,
listed block), from all 64 query rows of the tile against their running
maxima over the row's whole list, as the oracle's rule does.  Its output is
compared with the oracle's skip rule at the bars of the other attention tests
(O atol 4e-2 / rtol 1e-2, LSE 2e-3 nats).  Q-tiles with a block whose
decision lies within 1e-3 nats of the threshold are left out: there fp32 and
fp64 scores may decide differently.  Each case also checks that the skips it
exercises move O by more than the tolerance, so a kernel that never skipped
would fail.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from block_sparse_attention_sparge_amd import ops, synth

pytestmark = pytest.mark.gpu

O_ATOL, O_RTOL, LSE_TOL = 4e-2, 1e-2, 2e-3
NEAR = 1e-3


def np64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    ops.load_library()
    return torch.device("cuda:0")


def _compare(o_gpu, lse_gpu, q, k, v, lut, cnt, tau, causal=False, per_kv=False, sensitive=True):
    qn, kn, vn = np64(q), np64(k), np64(v)
    lut_n = None if lut is None else lut.cpu().numpy()
    cnt_n = None if cnt is None else cnt.cpu().numpy()
    ro, rl, ns, nu, near = oracle.block_sparse_attention_pv_skip(
        qn, kn, vn, lut_n, cnt_n, tau, lut_per_kv_head=per_kv, causal=causal, return_skips=True,
        return_margins=True)
    assert 0 < ns < nu, (ns, nu)
    keep = np.repeat(near >= NEAR, 64, axis=-1)[..., :ro.shape[2]]    # [b, h, s_q]
    assert keep.mean() > 0.8
    og, lg = np64(o_gpu), np64(lse_gpu)
    err = np.abs(og - ro)[keep]
    bad = err > O_ATOL + O_RTOL * np.abs(ro[keep])
    assert not bad.any(), f"O: {bad.sum()} of {bad.size} outside atol/rtol; max err {err.max():.3e}"
    # LSE is the exact one, skip or not
    assert np.array_equal(np.isneginf(lg), np.isneginf(rl))
    fin = ~np.isneginf(rl)
    assert np.abs(lg[fin] - rl[fin]).max() <= LSE_TOL
    if sensitive:
        ex, _ = oracle.block_sparse_attention(qn, kn, vn, lut_n, cnt_n, lut_per_kv_head=per_kv,
                                              causal=causal)
        assert np.abs(ro - ex)[keep].max() > 1.5 * O_ATOL, "the skips in this case are too small to see"
    return ns / nu


def _decaying(dev, b, h, s, d, dtype, seed, rate=0.5):
    """K block t scaled by 2^(-rate t): later blocks score lower, so many of
    them fall below the running maximum of every row of a tile."""
    g = torch.Generator(device=dev).manual_seed(seed)
    q = (4.0 * torch.randn(b, h, s, d, generator=g, device=dev)).to(dtype)
    scale = torch.pow(2.0, -rate * (torch.arange(s, device=dev) // 64).float())
    k = (torch.randn(b, h, s, d, generator=g, device=dev) * scale[:, None]).to(dtype)
    v = torch.randn(b, h, s, d, generator=g, device=dev).to(dtype)
    return q, k, v


@pytest.mark.parametrize("dtype,d", [(torch.float16, 128), (torch.bfloat16, 64)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("tau", [0.5, 1.5])
def test_pv_skip_dense_decaying_keys(dev, dtype, d, causal, tau):
    q, k, v = _decaying(dev, 1, 2, 1024, d, dtype, 100 + d)
    o, lse = ops.sparse_fmha_fwd(q, k, v, None, None, causal=causal, pv_threshold=tau)
    torch.cuda.synchronize()
    _compare(o, lse, q, k, v, None, None, tau, causal=causal)


def test_pv_skip_takes_one_pass_per_row(dev):
    # The rule compares each block with the maximum over the blocks before it
    # in the row, so a split of the row is refused on the host.
    q, k, v = _decaying(dev, 1, 2, 256, 128, torch.float16, 7)
    with pytest.raises(ops.SpargeError):
        ops.sparse_fmha_fwd(q, k, v, None, None, num_splits=2, pv_threshold=2.0)


@pytest.mark.parametrize("tau", [0.25, 0.5])
def test_pv_skip_mid_block_map(dev, tau):
    case = synth.mid_case(dev)
    bm = ops.build_block_map(case.q, case.k, case.topk, case.simthreshd1)
    o, lse = ops.sparse_fmha_fwd(case.q, case.k, case.v, bm["lut"], bm["count"], pv_threshold=tau)
    torch.cuda.synchronize()
    _compare(o, lse, case.q, case.k, case.v, bm["lut"], bm["count"], tau)


def test_pv_skip_gqa_shared_lut_causal(dev):
    b, hq, hkv, s, d = 1, 4, 2, 768, 128
    q, k, v = _decaying(dev, b, hkv, s, d, torch.bfloat16, 11)
    q = torch.cat([q, q.flip(2)], dim=1).reshape(b, hq, s, d).contiguous()
    nq = s // 64
    lut = torch.arange(nq, dtype=torch.int32, device=dev).repeat(b, hkv, nq, 1).contiguous()
    cnt = torch.full((b, hkv, nq), nq, dtype=torch.int32, device=dev)
    o, lse = ops.sparse_fmha_fwd(q, k, v, lut, cnt, causal=True, pv_threshold=1.0)
    torch.cuda.synchronize()
    _compare(o, lse, q, k, v, lut, cnt, 1.0, causal=True, per_kv=True)


def test_pv_threshold_zero_is_the_plain_kernel(dev):
    case = synth.mid_case(dev)
    bm = ops.build_block_map(case.q, case.k, case.topk, case.simthreshd1)
    o0, l0 = ops.sparse_fmha_fwd(case.q, case.k, case.v, bm["lut"], bm["count"])
    o1, l1 = ops.sparse_fmha_fwd(case.q, case.k, case.v, bm["lut"], bm["count"], pv_threshold=0.0)
    # a threshold far above any score gap skips nothing: same bits as no skip
    o2, l2 = ops.sparse_fmha_fwd(case.q, case.k, case.v, bm["lut"], bm["count"], pv_threshold=1e4)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
    assert torch.equal(o0, o2) and torch.equal(l0, l2)


@pytest.mark.parametrize("tau", [2.0, 4.0])
def test_pv_skip_headline_sampled_heads(dev, tau):
    # Headline workload at topk 0.4: the flattest (h 0, nothing dropped) and
    # most peaked (h 31, 43% of its pairs dropped at tau 4 and 67% at tau 2)
    # heads of both batches against the oracle.
    case = synth.headline_case(dev, topk=0.4)
    bm = ops.build_block_map(case.q, case.k, case.topk, case.simthreshd1)
    o, lse = ops.sparse_fmha_fwd(case.q, case.k, case.v, bm["lut"], bm["count"], pv_threshold=tau)
    torch.cuda.synchronize()
    heads = [0, 31]
    frac = _compare(o[:, heads], lse[:, heads], case.q[:, heads], case.k[:, heads],
                    case.v[:, heads], bm["lut"][:, heads], bm["count"][:, heads], tau,
                    sensitive=False)
    print(f"headline tau {tau}: {frac:.3f} of the (tile, block) pairs of heads 0 and 31 dropped")
