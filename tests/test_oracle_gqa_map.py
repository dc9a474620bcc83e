"""Pin for the oracle's block map with fewer KV heads than query heads (CPU).

Reading R28: query head j pools against KV head j // (h / h_kv), the GQA
mapping attention uses (aiter 6841 page).  That is by construction the block
map of the same Q against K with every KV head repeated for its query heads,
so the oracle's grouped path is pinned against its already pinned per-head
path on an explicitly expanded K (numpy repeat, not the oracle's indexing).
"""
import numpy as np
import pytest

import oracle


@pytest.mark.parametrize("ratio", [2, 4])
@pytest.mark.parametrize("opts", [dict(), dict(smooth_k=True), dict(causal=True, attention_sink=True),
                                  dict(smooth_k=True, causal=True)])
def test_grouped_map_equals_map_on_expanded_keys(ratio, opts):
    rng = np.random.default_rng(ratio)
    b, h, s, d = 2, 4, 512, 16
    h_kv = h // ratio
    q = rng.standard_normal((b, h, s, d))
    k = rng.standard_normal((b, h_kv, s, d)) + np.repeat(rng.standard_normal((b, h_kv, s // 64, d)), 64, axis=2)
    topk = [0.25, 0.5, 0.125, 0.375]
    thr = [0.3, 0.6, 0.45, 0.2]            # per query head: the K gate differs within a group
    g = oracle.block_map(q, k, topk, thr, **opts)
    e = oracle.block_map(q, np.repeat(k, ratio, axis=1), topk, thr, **opts)
    for key in ("lut", "count", "bitmap", "prob", "scores", "q_mean", "sim_q", "sim_k"):
        np.testing.assert_array_equal(g[key], e[key], err_msg=key)
    np.testing.assert_array_equal(g["k_mean"], e["k_mean"][:, ::ratio])
    np.testing.assert_array_equal(g["sim_k_val"], e["sim_k_val"][:, ::ratio])
    # the groups really see different gates on the same K blocks
    assert (g["sim_k"][:, 0] != g["sim_k"][:, 1]).any()


def test_grouped_map_rejects_a_non_divisor():
    q, k = np.zeros((1, 3, 128, 8)), np.zeros((1, 2, 128, 8))
    with pytest.raises(ValueError):
        oracle.block_map(q, k, [0.5] * 3, [0.0] * 3)
