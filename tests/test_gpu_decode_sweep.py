"""Seeded sweep of the token-list (decode) attention against the fp64 oracle.

Each case draws b, the number of KV heads, the query heads per KV head (1 to
16), the query positions sharing a list (1 to 3), s_k, the list length
(1 to 2000, ragged rows with -1 holes and empty rows), d 64 or 128, fp16 or
bf16, a peaked or flat query scale, and splits merged by attn_combine.  It
covers every row count the kernel is built for, several workgroups per KV
head, and chunks that end inside a list.  Held to O atol 4e-2 / rtol 1e-2 and
LSE 2e-3 nats, -inf exactly where the oracle has it.
"""
import numpy as np
import pytest
import torch

import oracle
from block_sparse_attention_sparge_amd import ops, synth

pytestmark = pytest.mark.gpu

O_ATOL, O_RTOL, LSE_TOL = 4e-2, 1e-2, 2e-3
N_CASES = 32


def np64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    ops.load_library()          # raises if the HIP library is missing
    return torch.device("cuda:0")


def draw_case(i):
    r = np.random.RandomState(3000 + i)
    return dict(
        b=int(r.randint(1, 5)),
        h_kv=int(r.choice([1, 2, 4])),
        ratio=int(r.choice([1, 2, 3, 4, 8, 16])),
        s_q=int(r.choice([1, 1, 2, 3])),
        s_k=int(r.randint(1, 6000)),
        L=int(r.randint(1, 2000)),
        d=int(r.choice([64, 128])),
        dtype=[torch.float16, torch.bfloat16][r.randint(2)],
        q_scale=float(r.choice([1.0, 4.0])),
        splits=int(r.choice([1, 1, 2, 5, 8])),
    )


def describe(c):
    return (f"b{c['b']} h_kv{c['h_kv']}x{c['ratio']} s_q{c['s_q']} s_k{c['s_k']} L{c['L']} d{c['d']} "
            f"{str(c['dtype']).split('.')[-1]} q_scale={c['q_scale']} splits={c['splits']}")


@pytest.mark.parametrize("i", range(N_CASES))
def test_decode_random_case(dev, i):
    c = draw_case(i)
    print(describe(c), flush=True)
    h_q = c["h_kv"] * c["ratio"]
    L = min(c["L"], c["s_k"])
    q = synth.normal((c["b"], h_q, c["s_q"], c["d"]), 900 + i, 1, c["dtype"], dev, scale=c["q_scale"])
    k = synth.normal((c["b"], c["h_kv"], c["s_k"], c["d"]), 900 + i, 2, c["dtype"], dev)
    v = synth.normal((c["b"], c["h_kv"], c["s_k"], c["d"]), 900 + i, 3, c["dtype"], dev)
    lists = synth.token_lists(c["b"], c["h_kv"], L, c["s_k"], 900 + i, 4, ragged=True).to(dev)
    if c["splits"] == 1:
        o, lse = ops.sparse_fmha_fwd(q, k, v, lists, None, blk_q=1, blk_k=1)
    else:
        op, lp = ops.sparse_fmha_fwd(q, k, v, lists, None, blk_q=1, blk_k=1, num_splits=c["splits"])
        o, lse = ops.attn_combine(op, lp, out_dtype=c["dtype"])
    torch.cuda.synchronize()
    ro, rl = oracle.token_list_attention(np64(q), np64(k), np64(v), lists.cpu().numpy())
    g = np64(o)
    err = np.abs(g - ro)
    bad = err > O_ATOL + O_RTOL * np.abs(ro)
    assert not bad.any(), f"{describe(c)}: {bad.sum()} O entries outside the bar; max err {err.max():.3e}"
    gl = np64(lse)
    assert np.array_equal(np.isneginf(gl), np.isneginf(rl)), f"{describe(c)}: -inf rows differ"
    fin = ~np.isneginf(rl)
    if fin.any():
        e = np.abs(gl[fin] - rl[fin]).max()
        assert e <= LSE_TOL, f"{describe(c)}: LSE max err {e:.3e} nats"
