"""Seeded sweep of attn_combine against the fp64 oracle.

Each case draws the number of parts (1 to 40, across the small-grid kernel's
limits of 4 and 16 parts), a shape whose grid falls on either side of the
small-grid limit (2048 workgroups), d 64 or 128, fp32 / fp16 / bf16 partials,
fp32 / fp16 / bf16 output, and -inf LSE on random parts and on whole rows.
fp32 partials are held to 2e-6 (their format error after the merge), 16-bit
partials to 8e-3; LSE to 1e-5; all-empty rows must give O = 0, LSE = -inf.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from block_sparse_attention_sparge_amd import ops

pytestmark = pytest.mark.gpu

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
    r = np.random.RandomState(5000 + i)
    d = int(r.choice([64, 128]))
    big = bool(r.rand() < 0.3)
    # 2048 workgroups of 256 threads, 8 d values per thread.
    limit_rows = 2048 * 256 * 8 // d
    rows = limit_rows + int(r.randint(256, 8000)) if big else int(r.randint(1, 30000))
    b = int(r.choice([1, 2]))
    h = int(r.choice([1, 2, 4, 8]))
    s = max(1, -(-rows // (b * h)))
    n = int(r.choice([2, 4, 8])) if big else int(r.choice([1, 2, 3, 4, 5, 8, 16, 17, 40]))
    return dict(n=n, b=b, h=h, s=s, d=d,
                pdt=[torch.float32, torch.float16, torch.bfloat16][r.randint(3)],
                odt=[torch.float32, torch.float16, torch.bfloat16][r.randint(3)],
                p_empty=float(r.choice([0.0, 0.3, 0.9])))


@pytest.mark.parametrize("i", range(N_CASES))
def test_combine_random_case(dev, i):
    c = draw_case(i)
    desc = (f"n{c['n']} b{c['b']} h{c['h']} s{c['s']} d{c['d']} parts {str(c['pdt']).split('.')[-1]} "
            f"out {str(c['odt']).split('.')[-1]} p_empty {c['p_empty']}")
    print(desc, flush=True)
    g = torch.Generator(device=dev).manual_seed(6000 + i)
    n, b, h, s, d = c["n"], c["b"], c["h"], c["s"], c["d"]
    parts = torch.randn(n, b, h, s, d, generator=g, device=dev).to(c["pdt"])
    lse = torch.randn(n, b, h, s, generator=g, device=dev) * 3
    lse[torch.rand(n, b, h, s, generator=g, device=dev) < c["p_empty"]] = -math.inf
    lse[:, 0, 0, : min(s, 3)] = -math.inf                       # rows with every part empty
    o, l = ops.attn_combine(parts, lse, out_dtype=c["odt"])
    torch.cuda.synchronize()
    ro, rl = oracle.combine(list(np64(parts)), list(np64(lse)))
    tol = 2e-6 if c["pdt"] == torch.float32 else 8e-3
    if c["odt"] != torch.float32:
        tol = max(tol, 8e-3)                                     # the output's own rounding
    go = np64(o)
    err = np.abs(go - ro)
    assert (err <= tol + tol * np.abs(ro)).all(), f"{desc}: max O err {err.max():.3e}"
    gl = np64(l)
    assert np.array_equal(np.isneginf(gl), np.isneginf(rl)), f"{desc}: -inf rows differ"
    fin = ~np.isneginf(rl)
    if fin.any():
        assert np.abs(gl[fin] - rl[fin]).max() <= 1e-5, f"{desc}: LSE"
    assert (go[0, 0, : min(s, 3)] == 0).all(), f"{desc}: empty rows not zero"
