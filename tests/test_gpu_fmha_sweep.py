"""Seeded sweep of the block-mode FMHA against the fp64 oracle.

Each case draws its own shape and options: ragged s_q / s_k (partial first
and last tiles and blocks), d 64 or 128, fp16 or bf16, grouped-query ratios
1 / 2 / 4, LUT rows per query head or per KV head, random LUT densities with
empty rows, the dense mode, the causal mask (s_q = s_k), splits merged by
attn_combine with fp32 or 16-bit partials, and output in the input type or
fp32.  Every case is held to the stated bars: O within atol 4e-2 / rtol 1e-2,
LSE within 2e-3 nats, -inf exactly where the oracle has it.  Eight larger
cases (over 4096 rows, so non-causal ones take the interleaved XCD order)
are checked on their first and last query head.
"""
import numpy as np
import pytest
import torch

import oracle
from block_sparse_attention_sparge_amd import ops, synth

pytestmark = pytest.mark.gpu

O_ATOL, O_RTOL, LSE_TOL = 4e-2, 1e-2, 2e-3
N_CASES = 64


def np64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    ops.load_library()          # raises if the HIP library is missing
    return torch.device("cuda:0")


def draw_case(i):
    r = np.random.RandomState(1000 + i)
    c = dict(
        b=int(r.choice([1, 2])),
        h_kv=int(r.choice([1, 2])),
        ratio=int(r.choice([1, 2, 4])),
        d=int(r.choice([64, 128])),
        dtype=[torch.float16, torch.bfloat16][r.randint(2)],
        causal=bool(r.rand() < 0.3),
        dense=bool(r.rand() < 0.2),
        per_kv=bool(r.rand() < 0.3),
        splits=int(r.choice([1, 1, 2, 3])),
        out_f32=bool(r.rand() < 0.3),
        q_scale=float(r.choice([1.0, 3.0])),
    )
    c["s_q"] = int(r.randint(1, 700))
    c["s_k"] = c["s_q"] if c["causal"] else int(r.randint(1, 700))
    nq, nk = -(-c["s_q"] // 64), -(-c["s_k"] // 64)
    h_lut = c["h_kv"] if c["per_kv"] else c["h_kv"] * c["ratio"]
    lut = np.full((c["b"], h_lut, nq, nk), -1, np.int32)
    cnt = np.zeros((c["b"], h_lut, nq), np.int32)
    for idx in np.ndindex(c["b"], h_lut, nq):
        n = 0 if r.rand() < 0.1 else int(r.randint(1, nk + 1))
        sel = np.sort(r.choice(nk, size=n, replace=False)).astype(np.int32)
        lut[idx][:n] = sel
        cnt[idx] = n
    c["lut"], c["cnt"] = lut, cnt
    return c


def describe(c):
    return (f"b{c['b']} h_kv{c['h_kv']}x{c['ratio']} s_q{c['s_q']} s_k{c['s_k']} d{c['d']} "
            f"{str(c['dtype']).split('.')[-1]} causal={c['causal']} dense={c['dense']} "
            f"per_kv={c['per_kv']} splits={c['splits']} out_f32={c['out_f32']} q_scale={c['q_scale']}")


@pytest.mark.parametrize("i", range(N_CASES))
def test_fmha_random_case(dev, i):
    c = draw_case(i)
    print(describe(c), flush=True)
    h_q = c["h_kv"] * c["ratio"]
    q = synth.normal((c["b"], h_q, c["s_q"], c["d"]), 500 + i, 1, c["dtype"], dev, scale=c["q_scale"])
    k = synth.normal((c["b"], c["h_kv"], c["s_k"], c["d"]), 500 + i, 2, c["dtype"], dev)
    v = synth.normal((c["b"], c["h_kv"], c["s_k"], c["d"]), 500 + i, 3, c["dtype"], dev)
    lut = None if c["dense"] else torch.from_numpy(c["lut"]).to(dev)
    cnt = None if c["dense"] else torch.from_numpy(c["cnt"]).to(dev)
    out_dt = torch.float32 if c["out_f32"] else c["dtype"]
    if c["splits"] == 1:
        o, lse = ops.sparse_fmha_fwd(q, k, v, lut, cnt, causal=c["causal"], out_dtype=out_dt)
    else:
        part_dt = torch.float32 if c["out_f32"] else c["dtype"]
        op, lp = ops.sparse_fmha_fwd(q, k, v, lut, cnt, causal=c["causal"], num_splits=c["splits"],
                                     out_dtype=part_dt)
        o, lse = ops.attn_combine(op, lp, out_dtype=out_dt)
    torch.cuda.synchronize()
    ro, rl = oracle.block_sparse_attention(np64(q), np64(k), np64(v),
                                           None if c["dense"] else c["lut"],
                                           None if c["dense"] else c["cnt"],
                                           lut_per_kv_head=c["per_kv"], causal=c["causal"])
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


# Cases above 4096 rows: non-causal launches of that size deal their tiles
# across the XCDs (every eighth tile of each head per XCD); causal ones keep
# contiguous heads.  The oracle runs on the first and last query head.
N_LARGE = 8


def draw_large_case(i):
    r = np.random.RandomState(7000 + i)
    c = dict(b=int(r.choice([1, 2])), h_kv=int(r.choice([4, 8, 16])), ratio=int(r.choice([1, 2, 4])),
             d=int(r.choice([64, 128])), dtype=[torch.float16, torch.bfloat16][r.randint(2)],
             causal=bool(r.rand() < 0.25), splits=int(r.choice([1, 1, 2])), out_f32=bool(r.rand() < 0.3))
    h_q = c["h_kv"] * c["ratio"]
    tiles = 4096 // (c["b"] * h_q * c["splits"]) + 1
    c["s"] = int(min(12000, max(tiles * 64 - int(r.randint(0, 63)), 256)))
    nb = -(-c["s"] // 64)
    lut = np.full((c["b"], h_q, nb, nb), -1, np.int32)
    cnt = np.zeros((c["b"], h_q, nb), np.int32)
    for idx in np.ndindex(c["b"], h_q, nb):
        n = 0 if r.rand() < 0.05 else int(r.randint(1, min(nb, 40) + 1))
        lut[idx][:n] = np.sort(r.choice(nb, size=n, replace=False)).astype(np.int32)
        cnt[idx] = n
    c["lut"], c["cnt"] = lut, cnt
    return c


@pytest.mark.parametrize("i", range(N_LARGE))
def test_fmha_random_large_case(dev, i):
    c = draw_large_case(i)
    h_q = c["h_kv"] * c["ratio"]
    s = c["s"]
    print(f"b{c['b']} h_kv{c['h_kv']}x{c['ratio']} s{s} d{c['d']} {str(c['dtype']).split('.')[-1]} "
          f"causal={c['causal']} splits={c['splits']} out_f32={c['out_f32']}", flush=True)
    q = synth.normal((c["b"], h_q, s, c["d"]), 900 + i, 1, c["dtype"], dev, scale=1.5)
    k = synth.normal((c["b"], c["h_kv"], s, c["d"]), 900 + i, 2, c["dtype"], dev)
    v = synth.normal((c["b"], c["h_kv"], s, c["d"]), 900 + i, 3, c["dtype"], dev)
    lut = None if c["causal"] else torch.from_numpy(c["lut"]).to(dev)
    cnt = None if c["causal"] else torch.from_numpy(c["cnt"]).to(dev)
    out_dt = torch.float32 if c["out_f32"] else c["dtype"]
    if c["splits"] == 1:
        o, lse = ops.sparse_fmha_fwd(q, k, v, lut, cnt, causal=c["causal"], out_dtype=out_dt)
    else:
        op, lp = ops.sparse_fmha_fwd(q, k, v, lut, cnt, causal=c["causal"], num_splits=2,
                                     out_dtype=torch.float32 if c["out_f32"] else c["dtype"])
        o, lse = ops.attn_combine(op, lp, out_dtype=out_dt)
    torch.cuda.synchronize()
    for ih in (0, h_q - 1):
        hk = ih // c["ratio"]
        ro, rl = oracle.block_sparse_attention(
            np64(q[:, ih:ih + 1]), np64(k[:, hk:hk + 1]), np64(v[:, hk:hk + 1]),
            None if c["causal"] else c["lut"][:, ih:ih + 1], None if c["causal"] else c["cnt"][:, ih:ih + 1],
            causal=c["causal"])
        g = np64(o[:, ih:ih + 1])
        err = np.abs(g - ro)
        bad = err > O_ATOL + O_RTOL * np.abs(ro)
        assert not bad.any(), f"case {i} head {ih}: {bad.sum()} O entries outside the bar; max err {err.max():.3e}"
        gl = np64(lse[:, ih:ih + 1])
        assert np.array_equal(np.isneginf(gl), np.isneginf(rl)), f"case {i} head {ih}: -inf rows differ"
        fin = ~np.isneginf(rl)
        if fin.any():
            assert np.abs(gl[fin] - rl[fin]).max() <= LSE_TOL, f"case {i} head {ih}: LSE outside the bar"
