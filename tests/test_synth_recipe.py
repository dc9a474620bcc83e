"""CPU checks that the seeded input generators follow the stated recipe, and
of the benchmark's command-line contract.

Recipe (the workloads' shapes, value distributions and index structure):
block-centroid + noise Q/K (per (b, h) and 64-token block, c ~ gamma_h N(0, I),
token = c + sigma N(0, I)), gamma_h linear from 0.5 to 2 over the heads of the
headline workload, V ~ N(0, 1); two-pass combine LUTs (A = the last 4 blocks,
B = 64 distinct earlier blocks per row, ascending, about 10% of rows empty);
decode lists (ascending distinct positions, -1 padded; Q = 4 N(0, 1)).
"""
import math
import subprocess
import sys
from pathlib import Path

import numpy as np
import pytest
import torch

from block_sparse_attention_sparge_amd import synth

ROOT = Path(__file__).resolve().parents[1]


def test_seeded_and_tensor_ids_independent():
    a = synth.normal((4, 64), 3, 1)
    b = synth.normal((4, 64), 3, 1)
    c = synth.normal((4, 64), 3, 2)
    d = synth.normal((4, 64), 4, 1)
    assert torch.equal(a, b)
    assert not torch.equal(a, c) and not torch.equal(a, d)


def test_normal_scale_and_rounding():
    x = synth.normal((256, 256), 0, 1, dtype=torch.float32, scale=4.0)
    assert abs(float(x.std()) - 4.0) < 0.05 and abs(float(x.mean())) < 0.05
    h = synth.normal((64,), 0, 1, dtype=torch.float16)
    f = synth.normal((64,), 0, 1, dtype=torch.float32)
    assert torch.equal(h, f.to(torch.float16))            # drawn in fp32, rounded once


def test_headline_gammas_linear_half_to_two():
    g = synth.headline_gammas(32)
    assert g[0] == 0.5 and g[-1] == 2.0 and len(g) == 32
    assert np.allclose(np.diff(g), 1.5 / 31)


def test_mixed_topk_cycles_the_sweep():
    assert synth.mixed_topk(12) == [0.1, 0.2, 0.4, 0.6, 0.8] * 2 + [0.1, 0.2]


@pytest.mark.parametrize("gamma,sigma", [(0.5, 0.5), (2.0, 0.5), (1.0, 0.3)])
def test_centroid_noise_statistics(gamma, sigma):
    b, h, s, d = 1, 1, 64 * 256, 64
    x = synth.centroid_noise(b, h, s, d, 64, [gamma], sigma, 5, 1, torch.float32)
    blocks = x.view(256, 64, d)
    means = blocks.mean(1)                                  # c + sigma * mean of 64 noise draws
    within = blocks - means[:, None, :]
    # block means spread as gamma (plus the noise's sigma / 8); tokens scatter
    # around them with sigma * sqrt(63 / 64)
    assert abs(float(means.std()) - math.sqrt(gamma ** 2 + sigma ** 2 / 64)) < 0.03 * gamma + 0.01
    assert abs(float(within.std()) - sigma * math.sqrt(63 / 64)) < 0.01
    # every token of a block shares its centroid: high intra-block cosine
    # similarity, the property the block map's gate measures
    xn = blocks / blocks.norm(dim=-1, keepdim=True)
    sim = (xn.sum(1).norm(dim=-1) ** 2 / 64 ** 2).mean()
    expect = gamma ** 2 / (gamma ** 2 + sigma ** 2)
    assert abs(float(sim) - expect) < 0.05


def test_partial_last_block_keeps_its_centroid():
    x = synth.centroid_noise(1, 1, 64 + 10, 32, 64, [1.0], 0.0, 2, 1, torch.float32)
    assert torch.equal(x[0, 0, 64], x[0, 0, 73]) and not torch.equal(x[0, 0, 0], x[0, 0, 64])


def test_headline_case_per_head_scale():
    c = synth.headline_case("cpu", topk=0.4, b=1, h=4, s=64 * 128, d=64)
    assert c.q.shape == (1, 4, 64 * 128, 64) and c.q.dtype == torch.float16
    spread = [float(c.q[0, i].float().view(128, 64, 64).mean(1).std()) for i in range(4)]
    assert spread == sorted(spread)                         # gamma grows with the head index
    assert abs(float(c.v.float().std()) - 1.0) < 0.02
    assert c.topk == [0.4] * 4 and c.simthreshd1 == [0.001] * 4


def test_random_block_lists_structure():
    lut, cnt = synth.random_block_lists(2000, 64, 508, 0.1, 0, 4, 512)
    empty = cnt == 0
    assert abs(float(empty.float().mean()) - 0.1) < 0.03
    for r in range(0, 2000, 37):
        row = lut[r]
        if empty[r]:
            assert (row == -1).all()
            continue
        sel = row[:64]
        assert int(cnt[r]) == 64 and (row[64:] == -1).all()
        assert (sel[1:] > sel[:-1]).all() and int(sel.min()) >= 0 and int(sel.max()) < 508


def test_combine_case_luts():
    c = synth.combine_case("cpu", h=2, s_q=256, s_k=8192)
    nk = 8192 // 64
    a = c.lut_a.view(-1, nk)
    assert (a[:, :4] == torch.arange(nk - 4, nk, dtype=torch.int32)).all() and (a[:, 4:] == -1).all()
    assert (c.count_a == 4).all()
    bl = c.lut_b.view(-1, nk)
    live = bl[bl >= 0]
    assert int(live.max()) < nk - 4                          # B never overlaps A


@pytest.mark.parametrize("ragged", [False, True])
def test_token_lists_structure(ragged):
    lists = synth.token_lists(4, 3, 256, 4096, 0, 4, ragged)
    assert lists.shape == (4, 3, 256)
    counts = []
    for row in lists.view(-1, 256):
        valid = row[row >= 0]
        counts.append(len(valid))
        assert (valid[1:] > valid[:-1]).all()
        assert len(valid) == 0 or int(valid.max()) < 4096
    if ragged:
        assert len(set(counts)) > 1
        assert any(((row[:-1] == -1) & (row[1:] >= 0)).any() for row in lists.view(-1, 256))
    else:
        assert counts == [256] * 12


def test_decode_case_query_scale():
    dc = synth.decode_case("cpu", b=2, h_q=8, h_kv=2, s_k=2048, L=256)
    assert dc.q.shape == (2, 8, 1, 128) and dc.k.shape == (2, 2, 2048, 128)
    assert abs(float(dc.q.float().std()) - 4.0) < 0.3
    assert dc.lists.dtype == torch.int32 and dc.lists.shape == (2, 2, 256)


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2", "--no-cpu"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""                           # no JSON line
