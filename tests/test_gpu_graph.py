"""The path captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

Callers under graph capture cannot allocate; the allocation-free block map
(sparge_build_block_map_noalloc), the sparse FMHA, the split-K decode and the
combine take caller-owned outputs and enqueue only kernels, so they can be
captured.  Each graph is replayed several times with the program's own eager
work and synchronisations between replays, and every replay must give the
bits of the eager calls.
"""
import pytest
import torch

from block_sparse_attention_sparge_amd import ops, synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    ops.load_library()
    return torch.device("cuda:0")


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()                                     # warm outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def _eager_noise(dev, i):
    # Unrelated eager work between replays: it reuses the caching allocator
    # and the device, then synchronises.
    x = torch.randn(1 << 20, device=dev) * (i + 1)
    torch.cuda.synchronize()
    return float(x.abs().sum())


def test_block_map_and_fmha_replay_bitwise(dev):
    case = synth.mid_case(dev)
    q, k, v = case.q, case.k, case.v
    b, h, s, d = q.shape
    nq = s // 64
    out = dict(lut=torch.empty((b, h, nq, nq), dtype=torch.int32, device=dev),
               count=torch.empty((b, h, nq), dtype=torch.int32, device=dev))
    o = torch.empty_like(q)
    lse = torch.empty((b, h, s), dtype=torch.float32, device=dev)

    def step():
        ops.build_block_map_noalloc(q, k, case.topk, case.simthreshd1, out=out, smooth_k=True)
        ops.sparse_fmha_fwd(q, k, v, out["lut"], out["count"], o=o, lse=lse)

    ref = ops.build_block_map(q, k, case.topk, case.simthreshd1, smooth_k=True)
    ref_o, ref_l = ops.sparse_fmha_fwd(q, k, v, ref["lut"], ref["count"])
    g = _capture(step)
    for i in range(4):
        for t in (out["lut"], out["count"], o, lse):
            t.fill_(-7)                           # stale values must not survive
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out["lut"], ref["lut"]) and torch.equal(out["count"], ref["count"]), i
        assert torch.equal(o, ref_o) and torch.equal(lse, ref_l), i
        _eager_noise(dev, i)


def test_split_decode_and_combine_replay_bitwise(dev):
    case = synth.decode_case(dev, b=8)
    splits = 8
    p = torch.empty((splits, 8, 32, 1, 128), device=dev)
    pl = torch.empty((splits, 8, 32, 1), device=dev)
    o = torch.empty_like(case.q)
    lse = torch.empty((8, 32, 1), device=dev)

    def step():
        ops.sparse_fmha_fwd(case.q, case.k, case.v, case.lists, None, blk_q=1, blk_k=1,
                            num_splits=splits, o=p, lse=pl)
        ops.attn_combine(p, pl, o=o, lse=lse)

    rp, rpl = ops.sparse_fmha_fwd(case.q, case.k, case.v, case.lists, None, blk_q=1, blk_k=1,
                                  num_splits=splits)
    ref_o, ref_l = ops.attn_combine(rp, rpl, out_dtype=case.q.dtype)
    g = _capture(step)
    for i in range(4):
        o.fill_(0)
        lse.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, ref_o) and torch.equal(lse, ref_l), i
        _eager_noise(dev, i)
