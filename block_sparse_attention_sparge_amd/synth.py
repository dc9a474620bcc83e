"""Seeded synthetic inputs for block-sparse attention.

This module only draws random tensors and index lists; it holds none of the
attention or block-map arithmetic, so both the GPU path and the CPU oracle can
be fed from it.  Every tensor comes from its own torch.Generator seeded from
(seed, tensor id), on the device it is requested on (a CUDA tensor and a CPU
tensor drawn with the same seed differ; tests that compare GPU and oracle copy
the GPU inputs to the host).

Workloads (shapes, value distributions and index structure):

* block-centroid + noise Q/K: for every (b, h) and every block of `blk`
  tokens, a centroid c ~ gamma_h * N(0, I_d); token = c + sigma * N(0, I_d).
  This gives blocks with high intra-block similarity and pooled scores whose
  spread grows with gamma_h, standing in for the video-model activations the
  CK page's figure was measured on (not available here).
* V ~ N(0, 1).
* two-pass combine: LUT A = the last 4 KV blocks; LUT B = 64 distinct random
  blocks below them per row, ascending; about 10% of B's rows empty.
* decode: Q = 4 * N(0, 1) (peaked logits), K, V ~ N(0, 1); per (b, KV head)
  ascending lists of distinct token positions, -1 padded.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import torch


def _gen(device, seed: int, tensor_id: int) -> torch.Generator:
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed((int(seed) * 1_000_003 + int(tensor_id) * 7919 + 17) & 0x7FFF_FFFF_FFFF)
    return g


def normal(shape, seed: int, tensor_id: int, dtype=torch.float16, device="cpu",
           scale: float = 1.0) -> torch.Tensor:
    """scale * N(0, 1) of the given shape, drawn in fp32 and rounded to `dtype`."""
    g = _gen(device, seed, tensor_id)
    x = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    if scale != 1.0:
        x = x * scale
    return x.to(dtype)


def centroid_noise(b: int, h: int, s: int, d: int, blk: int, gammas, sigma: float,
                   seed: int, tensor_id: int, dtype=torch.float16,
                   device="cpu") -> torch.Tensor:
    """Block-centroid + noise tokens [b, h, s, d]; gammas has one entry per head.
    When s is not a multiple of blk the last block is partial (same centroid)."""
    g = _gen(device, seed, tensor_id)
    gam = torch.as_tensor(list(gammas), dtype=torch.float32, device=device).view(1, h, 1, 1)
    c = torch.randn(b, h, -(-s // blk), d, generator=g, device=device, dtype=torch.float32) * gam
    n = torch.randn(b, h, s, d, generator=g, device=device, dtype=torch.float32)
    x = c.repeat_interleave(blk, dim=2)[:, :, :s] + sigma * n
    return x.to(dtype)


@dataclass
class BlockSparseCase:
    """One block-sparse forward workload (stage 1 + stage 2)."""
    name: str
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    topk: List[float]
    simthreshd1: List[float]
    cdfthreshd: Optional[List[float]] = None
    blk_q: int = 64
    blk_k: int = 64
    meta: dict = field(default_factory=dict)


def tiny_case(device="cpu", seed: int = 0) -> BlockSparseCase:
    """b1 h2 s512 d64 fp16, gamma 1, sigma 0.3, topk 0.5, simthreshd1 0.001."""
    b, h, s, d = 1, 2, 512, 64
    q = centroid_noise(b, h, s, d, 64, [1.0] * h, 0.3, seed, 1, torch.float16, device)
    k = centroid_noise(b, h, s, d, 64, [1.0] * h, 0.3, seed, 2, torch.float16, device)
    v = normal((b, h, s, d), seed, 3, torch.float16, device)
    return BlockSparseCase("tiny", q, k, v, [0.5] * h, [0.001] * h,
                           meta=dict(gamma=1.0, sigma=0.3, seed=seed))


def mid_case(device="cpu", seed: int = 0, topk: float = 0.4) -> BlockSparseCase:
    """b1 h8 s4096 d128 bf16, gamma 1, sigma 0.5, cdf off."""
    b, h, s, d = 1, 8, 4096, 128
    q = centroid_noise(b, h, s, d, 64, [1.0] * h, 0.5, seed, 1, torch.bfloat16, device)
    k = centroid_noise(b, h, s, d, 64, [1.0] * h, 0.5, seed, 2, torch.bfloat16, device)
    v = normal((b, h, s, d), seed, 3, torch.bfloat16, device)
    return BlockSparseCase("mid", q, k, v, [topk] * h, [0.001] * h,
                           meta=dict(gamma=1.0, sigma=0.5, seed=seed))


def headline_gammas(h: int = 32) -> List[float]:
    """Centroid scale per head, linear from 0.5 to 2 over the heads."""
    return [0.5 + 1.5 * i / (h - 1) for i in range(h)]


def headline_case(device="cpu", seed: int = 0, topk=0.4, b: int = 2, h: int = 32,
                  s: int = 16384, d: int = 128, dtype=torch.float16) -> BlockSparseCase:
    """b2 h32 s16384 d128 fp16; gamma_h in [0.5, 2], sigma 0.5; simthreshd1 0.001.

    `topk` is one fraction for every head, or a per-head list.
    """
    gam = headline_gammas(h)
    q = centroid_noise(b, h, s, d, 64, gam, 0.5, seed, 1, dtype, device)
    k = centroid_noise(b, h, s, d, 64, gam, 0.5, seed, 2, dtype, device)
    v = normal((b, h, s, d), seed, 3, dtype, device)
    tk = list(topk) if isinstance(topk, (list, tuple)) else [float(topk)] * h
    return BlockSparseCase("headline", q, k, v, tk, [0.001] * h,
                           meta=dict(gamma="0.5+1.5*h/(H-1)", sigma=0.5, seed=seed))


def mixed_topk(h: int, sweep=(0.1, 0.2, 0.4, 0.6, 0.8)) -> List[float]:
    """Per-head top-k fractions: head i takes sweep[i mod len(sweep)]."""
    return [float(sweep[i % len(sweep)]) for i in range(h)]


def random_block_lists(rows: int, n_pick: int, n_range: int, p_empty: float,
                       seed: int, tensor_id: int, row_len: int):
    """Per row, `n_pick` distinct blocks from [0, n_range), ascending, -1 padded to
    `row_len`; a row is empty with probability p_empty.  Returns (lut, count) int32 (CPU)."""
    g = _gen("cpu", seed, tensor_id)
    lut = torch.full((rows, row_len), -1, dtype=torch.int32)
    count = torch.zeros(rows, dtype=torch.int32)
    empty = torch.rand(rows, generator=g) < p_empty
    for r in range(rows):
        picks = torch.randperm(n_range, generator=g)[:n_pick]
        if bool(empty[r]):
            continue
        sel = torch.sort(picks).values.to(torch.int32)
        lut[r, :n_pick] = sel
        count[r] = n_pick
    return lut, count


@dataclass
class CombineCase:
    """Two-pass workload: a dense pass over the most recent KV blocks (A) and a
    sparse pass over listed earlier blocks (B), merged by the LSE combine."""
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    lut_a: torch.Tensor
    count_a: torch.Tensor
    lut_b: torch.Tensor
    count_b: torch.Tensor
    blk: int = 64


def combine_case(device="cpu", seed: int = 0, b: int = 1, h: int = 16, s_q: int = 1024,
                 s_k: int = 32768, d: int = 128, dtype=torch.bfloat16,
                 n_recent: int = 4, n_pick: int = 64, p_empty: float = 0.1) -> CombineCase:
    """b1 h16 s_q1024 s_k32768 d128 bf16.  LUT rows are [b, h, nq, nk]."""
    blk = 64
    nq, nk = s_q // blk, s_k // blk
    q = normal((b, h, s_q, d), seed, 1, dtype, device)
    k = normal((b, h, s_k, d), seed, 2, dtype, device)
    v = normal((b, h, s_k, d), seed, 3, dtype, device)
    rows = b * h * nq
    lut_a = torch.full((rows, nk), -1, dtype=torch.int32)
    lut_a[:, :n_recent] = torch.arange(nk - n_recent, nk, dtype=torch.int32)
    count_a = torch.full((rows,), n_recent, dtype=torch.int32)
    lut_b, count_b = random_block_lists(rows, n_pick, nk - n_recent, p_empty, seed, 4, nk)
    shp = (b, h, nq, nk)
    return CombineCase(q, k, v, lut_a.view(shp).to(device), count_a.view(b, h, nq).to(device),
                       lut_b.view(shp).to(device), count_b.view(b, h, nq).to(device), blk)


@dataclass
class DecodeCase:
    """Decode-style grouped-query attention over per-(b, KV head) token lists."""
    q: torch.Tensor          # [b, h_q, 1, d]
    k: torch.Tensor          # [b, h_kv, s_k, d]
    v: torch.Tensor          # [b, h_kv, s_k, d]
    lists: torch.Tensor      # [b, h_kv, L] int32, ascending, -1 padded


def token_lists(b: int, h_kv: int, L: int, s_k: int, seed: int, tensor_id: int,
                ragged: bool = False) -> torch.Tensor:
    """[b, h_kv, L] int32 ascending distinct positions in [0, s_k), -1 padded.

    With `ragged`, each row keeps a random number of valid entries (0..L) and
    some rows also carry -1 entries between valid ones."""
    g = _gen("cpu", seed, tensor_id)
    out = torch.full((b * h_kv, L), -1, dtype=torch.int32)
    for r in range(b * h_kv):
        n = L
        if ragged:
            n = int(torch.randint(0, L + 1, (1,), generator=g))
        sel = torch.sort(torch.randperm(s_k, generator=g)[:n]).values.to(torch.int32)
        out[r, :n] = sel
        if ragged and n > 2 and r % 3 == 0:
            holes = torch.randperm(n, generator=g)[: max(1, n // 8)]
            out[r, holes] = -1
    return out.view(b, h_kv, L)


def decode_case(device="cpu", seed: int = 0, b: int = 64, h_q: int = 32, h_kv: int = 8,
                s_k: int = 32768, d: int = 128, L: int = 2048, dtype=torch.bfloat16,
                q_scale: float = 4.0, ragged: bool = False) -> DecodeCase:
    """b64 h_q32 h_kv8 d128 bf16, s_k 32768, lists of 2048 positions; Q = 4 * N(0, 1)."""
    q = normal((b, h_q, 1, d), seed, 1, dtype, device, scale=q_scale)
    k = normal((b, h_kv, s_k, d), seed, 2, dtype, device)
    v = normal((b, h_kv, s_k, d), seed, 3, dtype, device)
    lists = token_lists(b, h_kv, L, s_k, seed, 4, ragged).to(device)
    return DecodeCase(q, k, v, lists)
