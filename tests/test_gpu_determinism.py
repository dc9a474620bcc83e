"""Bitwise run-to-run stability of the hot path under relaunch.

The aiter 6841 page checks its sparse attention kernels over hundreds of frozen
relaunches and reports them bitwise-stable over 256 launches.  The path here
has no atomics and fixed reduction orders (the LUT is written by prefix scan,
blocks are accumulated in LUT order, splits merge in part order), so every
relaunch must give the same bits.  Each launch here runs while a memory-bound
copy runs on a second stream of the same (default) priority, so the kernels
meet different timing and cache states from launch to launch; the loop stops
at the first launch that differs.
"""
import pytest
import torch

from block_sparse_attention_sparge_amd import ops, synth

pytestmark = pytest.mark.gpu

LAUNCHES = 256


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    ops.load_library()
    return torch.device("cuda:0")


def _traffic(dev):
    """A memory-bound copy to run beside the launches (512 MiB each way)."""
    src = torch.zeros(512 << 20, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    side = torch.cuda.Stream(device=dev)        # default priority, like the main stream
    side.wait_stream(torch.cuda.current_stream(dev))

    def issue():
        with torch.cuda.stream(side):
            for _ in range(4):
                dst.copy_(src)
    return side, issue


def test_headline_step_is_bitwise_stable_over_256_launches(dev):
    # b2 h32 s16384 d128 fp16 with the mixed per-head topk {0.1 .. 0.8}.
    case = synth.headline_case(dev, topk=synth.mixed_topk(32))
    ref = ops.build_block_map(case.q, case.k, case.topk, case.simthreshd1, return_debug=True)
    ref_o, ref_l = ops.sparse_fmha_fwd(case.q, case.k, case.v, ref["lut"], ref["count"])
    bufs = {key: torch.empty_like(ref[key]) for key in ("lut", "count", "bitmap", "prob", "sim_q", "sim_k",
                                                        "q_mean", "k_mean", "workspace")}
    o, lse = torch.empty_like(ref_o), torch.empty_like(ref_l)
    side, issue = _traffic(dev)
    torch.cuda.synchronize()
    for i in range(LAUNCHES):
        issue()
        bm = ops.build_block_map(case.q, case.k, case.topk, case.simthreshd1, return_debug=True, out=bufs)
        ops.sparse_fmha_fwd(case.q, case.k, case.v, bm["lut"], bm["count"], o=o, lse=lse)
        for key in ("lut", "count", "prob"):
            assert torch.equal(bm[key], ref[key]), f"launch {i}: {key} differs"
        assert torch.equal(o, ref_o), f"launch {i}: O differs"
        assert torch.equal(lse, ref_l), f"launch {i}: LSE differs"
    side.synchronize()


def test_split_decode_and_combine_are_bitwise_stable_over_256_launches(dev):
    # The decode workload's shape on 16 batches: token lists of 2048 per KV
    # head, 8 splits merged by attn_combine.
    case = synth.decode_case(dev, b=16)
    ref_p, ref_pl = ops.sparse_fmha_fwd(case.q, case.k, case.v, case.lists, None, blk_q=1, blk_k=1,
                                        num_splits=8)
    ref_o, ref_l = ops.attn_combine(ref_p, ref_pl, out_dtype=case.q.dtype)
    p, pl = torch.empty_like(ref_p), torch.empty_like(ref_pl)
    o, lse = torch.empty_like(ref_o), torch.empty_like(ref_l)
    side, issue = _traffic(dev)
    torch.cuda.synchronize()
    for i in range(LAUNCHES):
        issue()
        ops.sparse_fmha_fwd(case.q, case.k, case.v, case.lists, None, blk_q=1, blk_k=1, num_splits=8,
                            o=p, lse=pl)
        ops.attn_combine(p, pl, o=o, lse=lse)
        assert torch.equal(p, ref_p) and torch.equal(pl, ref_pl), f"launch {i}: partials differ"
        assert torch.equal(o, ref_o) and torch.equal(lse, ref_l), f"launch {i}: combined result differs"
    side.synchronize()
