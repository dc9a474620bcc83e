"""Seeded sweep of the int8-QK and fp8-QK paths against the fp64 oracle.

Each case draws a shape (ragged s_q / s_k, d 64 or 128, GQA ratio 1 / 2 / 4),
the V type (fp16 or bf16), a random LUT (per query head or per KV head, empty
rows) or the dense mode, the causal mask, splits and fp32 output.  The int8
or fp8 (e4m3) codes and scales come from the block map's fused quantisation
and must equal the oracle's bit for bit (fp8 codes compared as values);
attention on them is held to O atol 4e-2 / rtol 1e-2 and LSE 2e-3 nats
against the oracle's attention on its own codes.
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
    r = np.random.RandomState(4000 + i)
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
        lut[idx][:n] = np.sort(r.choice(nk, size=n, replace=False)).astype(np.int32)
        cnt[idx] = n
    c["lut"], c["cnt"] = lut, cnt
    return c


def describe(c):
    return (f"b{c['b']} h_kv{c['h_kv']}x{c['ratio']} s_q{c['s_q']} s_k{c['s_k']} d{c['d']} "
            f"{str(c['dtype']).split('.')[-1]} causal={c['causal']} dense={c['dense']} "
            f"per_kv={c['per_kv']} splits={c['splits']} out_f32={c['out_f32']} q_scale={c['q_scale']}")


@pytest.mark.parametrize("code", ["int8", "fp8"])
@pytest.mark.parametrize("i", range(N_CASES))
def test_qk_int8_random_case(dev, i, code):
    c = draw_case(i)
    print(describe(c), flush=True)
    h_q = c["h_kv"] * c["ratio"]
    q = synth.normal((c["b"], h_q, c["s_q"], c["d"]), 1100 + i, 1, c["dtype"], dev, scale=c["q_scale"])
    k = synth.normal((c["b"], c["h_kv"], c["s_k"], c["d"]), 1100 + i, 2, c["dtype"], dev)
    v = synth.normal((c["b"], c["h_kv"], c["s_k"], c["d"]), 1100 + i, 3, c["dtype"], dev)
    fp8 = code == "fp8"
    bm = ops.build_block_map(q, k, [0.5] * h_q, [0.001] * h_q, quantize_int8=not fp8, quantize_fp8=fp8)
    torch.cuda.synchronize()
    sfx = "fp8" if fp8 else "i8"
    for x, key in ((q, "q_" + sfx), (k, "k_" + sfx)):
        xn = x.float().cpu().numpy()
        codes, scales = oracle.quantize_fp8(xn) if fp8 else oracle.quantize_int8(xn)
        got = oracle.e4m3_value(bm[key].cpu().numpy()) if fp8 else bm[key].cpu().numpy()
        assert np.array_equal(got, codes), f"{describe(c)}: {key}"
        assert np.array_equal(bm[key + "_scale"].cpu().numpy(), scales), f"{describe(c)}: {key} scale"
    lut = None if c["dense"] else torch.from_numpy(c["lut"]).to(dev)
    cnt = None if c["dense"] else torch.from_numpy(c["cnt"]).to(dev)
    args = (bm["q_" + sfx], bm["q_" + sfx + "_scale"], bm["k_" + sfx], bm["k_" + sfx + "_scale"], v, lut, cnt)
    fmha = ops.sparse_fmha_fwd_qk_fp8 if fp8 else ops.sparse_fmha_fwd_qk_int8
    out_dt = torch.float32 if c["out_f32"] else c["dtype"]
    if c["splits"] == 1:
        o, lse = fmha(*args, causal=c["causal"], out_dtype=out_dt)
    else:
        op, lp = fmha(*args, causal=c["causal"], num_splits=c["splits"],
                      out_dtype=torch.float32 if c["out_f32"] else c["dtype"])
        o, lse = ops.attn_combine(op, lp, out_dtype=out_dt)
    torch.cuda.synchronize()
    ref = oracle.block_sparse_attention_qk_fp8 if fp8 else oracle.block_sparse_attention_qk_int8
    ro, rl = ref(np64(q), np64(k), np64(v), None if c["dense"] else c["lut"],
                 None if c["dense"] else c["cnt"], lut_per_kv_head=c["per_kv"], causal=c["causal"])
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
