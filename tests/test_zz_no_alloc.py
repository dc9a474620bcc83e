"""The allocation-free block map (sparge_build_block_map_noalloc) against the
workspace entry point (sparge_build_block_map), through the C ABI.

Both run the same kernels; the only difference is where the scratch lives
(the library's static per-GPU array instead of a caller workspace), so every
output must agree bit for bit.  Calls follow one another on one stream, each
smaller than the one before, so a later call that read stale scratch from an
earlier, larger one would show.
"""
import pytest
import torch

from block_sparse_attention_sparge_amd import ops, synth

pytestmark = pytest.mark.gpu

KEYS = ("lut", "count", "bitmap", "prob", "sim_q", "sim_k", "q_mean", "k_mean")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    ops.load_library()
    return torch.device("cuda:0")


def _both(case, **opts):
    ref = ops.build_block_map(case.q, case.k, case.topk, case.simthreshd1, return_debug=True, **opts)
    got = ops.build_block_map_noalloc(case.q, case.k, case.topk, case.simthreshd1, return_debug=True,
                                      **opts)
    torch.cuda.synchronize()
    return ref, got


def _same(ref, got, keys):
    for key in keys:
        assert torch.equal(ref[key], got[key]), key


def test_noalloc_matches_workspace_entry_point_on_shrinking_calls(dev):
    # 1) the headline block map (b2 h32 s16384 d128 fp16, ~17 MiB of scratch)
    big = synth.headline_case(dev, topk=synth.mixed_topk(32))
    ref, got = _both(big)
    _same(ref, got, KEYS)
    # 2) right after it, a smaller mid case with K smoothing (the per-chunk
    #    sums of K also live in the scratch) and int8 codes
    mid = synth.mid_case(dev)
    ref, got = _both(mid, smooth_k=True, quantize_int8=True)
    _same(ref, got, KEYS + ("q_i8", "q_i8_scale", "k_i8", "k_i8_scale"))
    # 3) the tiny case, causal with the sink
    tiny = synth.tiny_case(dev)
    ref, got = _both(tiny, causal=True, attention_sink=True)
    _same(ref, got, KEYS)


def test_noalloc_refuses_sizes_beyond_its_scratch(dev):
    q = torch.empty((4, 32, 16384, 128), dtype=torch.float16, device=dev)
    with pytest.raises(ops.SpargeError, match="scratch"):
        ops.build_block_map_noalloc(q, q, [0.4] * 32, [0.001] * 32)
