"""Plain fp64 CPU oracle for SpargeAttn-style block-sparse attention (forward).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  The product path (the
HIP library and its Python binding) never calls it and shares no code with it.

Every function works in float64 on NumPy arrays and follows the pages'
description step by step, with no blocking, fusion or reordering:

* "Sparge Attention (Composable Kernel)" page, "Status vs Upstream" list: the
  block-map pipeline is per-block mean-pool, cosine similarity, pooled QK, then
  top-k / cdfthreshd block selection into a BlockMap LUT, with per-head
  topk / simthreshd1 / cdfthreshd.
* "Updating Log -- Speculative Sparse Attention" page, Stage 1: attention with a
  natural-log LSE, the online-softmax combine of two partials
  (FA(A u B) = Combine(FA(A), FA(B))) and the empty partial (LSE = -inf).
  Stage 3: a row that selects no block writes O = 0 and LSE = -inf.
* aiter pull request 6841 page (sorted-sparse MHA v4 LSE): an empty LUT row
  exports LSE = -inf.
* aiter pull request 4919 page (gfx950 sparse decode): -1 entries in an index
  list are skipped; the reduce masks partials whose maximum is -inf.
* llama.cpp pull request 10 page (Vulkan sparse prefill): index lists are
  ascending; ties at a top-k threshold are emitted in ascending index order.

Where the pages leave a step open, the reading taken is stated at the function
(readings R1..R14 in the design notes).  Parity of these readings with the
upstream SpargeAttn code is unpinned (no upstream code is available); the GPU
path is pinned against this oracle.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np

NEG_INF = -math.inf


# ----------------------------------------------------------------------------
# Stage 1: block map
# ----------------------------------------------------------------------------

def block_mean(x_blk: np.ndarray) -> np.ndarray:
    """Mean token of one block: (1/n) * sum_i x_i.

    CK page, "Status vs Upstream": per-block mean-pool.  Reading R1: a plain
    mean over the block's tokens; the last block of a sequence whose length is
    not a multiple of the block size holds fewer tokens, and its mean divides
    by that count.
    """
    x = np.asarray(x_blk, dtype=np.float64)
    return x.sum(axis=0) / x.shape[0]


def block_self_similarity(x_blk: np.ndarray) -> float:
    """Mean pairwise cosine similarity of the block's tokens, diagonal included.

    CK page, "Status vs Upstream": cosine similarity, gated by simthreshd1.
    Reading R2: the average of all n*n cosines cos(x_i, x_j), i = j included.
    A zero-norm token has no direction and contributes the zero vector.  The
    average of the Gram matrix of unit vectors equals |sum_i xhat_i|^2 / n^2,
    which is what is computed here.
    """
    x = np.asarray(x_blk, dtype=np.float64)
    n = x.shape[0]
    norms = np.sqrt((x * x).sum(axis=1))
    xhat = np.zeros_like(x)
    nz = norms > 0.0
    xhat[nz] = x[nz] / norms[nz, None]
    s = xhat.sum(axis=0)
    return float(s @ s) / float(n * n)


def pool_and_gate(x: np.ndarray, blk: int, simthreshd1: float):
    """Pool one (b, h) slice x [s, d] into blocks of `blk` tokens.

    Returns (means [nb, d], sims [nb], flags [nb] bool) where
    flag = sim > simthreshd1 (reading R3: strict comparison).  nb =
    ceil(s / blk); a partial last block pools its own tokens (reading R1).
    """
    x = np.asarray(x, dtype=np.float64)
    s, _ = x.shape
    nb = -(-s // blk)
    means = np.stack([block_mean(x[i * blk:(i + 1) * blk]) for i in range(nb)])
    sims = np.array([block_self_similarity(x[i * blk:(i + 1) * blk]) for i in range(nb)])
    flags = sims > float(simthreshd1)
    return means, sims, flags


def smooth_keys(k: np.ndarray) -> np.ndarray:
    """K with its mean over the sequence removed: k - km, km = mean_s k.

    CK page, "Status vs Upstream", not-yet-ported list: K smoothing, the
    pre-pool step k -= km.  Reading R22: km is the plain mean over all s_k
    positions of the (b, h) slice, and smoothing feeds only the block map (the
    pooled means and the K similarity gate); attention keeps the original K,
    so its LSE stays the exact log-sum-exp of the true scores.
    """
    k = np.asarray(k, np.float64)
    return k - k.mean(axis=-2, keepdims=True)


def causal_valid(nq: int, nk: int) -> np.ndarray:
    """valid[qb, kb]: K block kb holds a key at or before some query of Q-tile qb.

    CK page, not-yet-ported list: the is_causal mask in the pooled score.
    Reading R23 (blk_q = blk_k, s_q = s_k): block kb is entirely in the future
    of tile qb exactly when kb > qb.
    """
    return np.arange(nk)[None, :] <= np.arange(nq)[:, None]


def pooled_scores(qbar: np.ndarray, kbar: np.ndarray, sim_k: np.ndarray,
                  scale: float, causal: bool = False) -> np.ndarray:
    """S[qb, kb] = scale * <qbar[qb], kbar[kb]>, and -inf on non-similar K blocks.

    CK page, "Status vs Upstream": pooled QK.  Reading R4: the attention
    softmax scale (1/sqrt(d) by default).  Reading R5: a K block that fails the
    similarity gate is kept out of the pooled softmax (its column is -inf) and
    is forced on later, in `select_row`.  With `causal`, blocks in the future
    of the tile are -inf as well (reading R23).
    """
    s = float(scale) * (np.asarray(qbar, np.float64) @ np.asarray(kbar, np.float64).T)
    s[:, ~np.asarray(sim_k, bool)] = NEG_INF
    if causal:
        s[~causal_valid(s.shape[0], s.shape[1])] = NEG_INF
    return s


def row_softmax(scores: np.ndarray) -> np.ndarray:
    """Softmax over the last axis in fp64; a row of all -inf maps to all zeros.

    Reading R6: a row with every pooled score at -inf has no distribution; it is
    set to zero (and every block of that row is then forced on by the gate).
    """
    s = np.asarray(scores, dtype=np.float64)
    out = np.zeros_like(s)
    for idx in np.ndindex(*s.shape[:-1]):
        row = s[idx]
        m = row.max()
        if m == NEG_INF:
            continue
        e = np.exp(row - m)
        out[idx] = e / e.sum()
    return out


def topk_count(topk: float, nk: int) -> int:
    """Number of blocks a top-k fraction selects: clamp(floor(topk * nk), 1, nk).

    CK page, "Performance" and "Usage": topk is a fraction of the row (e.g.
    -topk=0.4).  Reading R7: the fraction arrives as fp32; it is widened to
    fp64, multiplied by nk and truncated.
    """
    n = int(math.floor(float(np.float32(topk)) * nk))
    return min(max(n, 1), nk)


def selection_order(prob_row: np.ndarray) -> np.ndarray:
    """Block indices ordered by pooled probability, largest first.

    Equal probabilities are ordered by ascending block index (the lower index
    wins), as the Vulkan page emits ties at a top-k threshold in ascending index
    order.
    """
    p = np.asarray(prob_row, dtype=np.float64)
    kb = np.arange(p.shape[0])
    return np.lexsort((kb, -p))


def cdf_count(prob_row: np.ndarray, order: np.ndarray, cdfthreshd: float) -> int:
    """Fewest leading blocks of `order` whose summed probability reaches the threshold.

    CK page, "Status vs Upstream": cdfthreshd block selection.  Reading R8: the
    running sum is accumulated one block at a time in fp64 in `order`; the
    count is the first n >= 1 with sum >= cdfthreshd, else every block.
    """
    thr = float(np.float32(cdfthreshd))
    c = 0.0
    for n, kb in enumerate(order, start=1):
        c = c + float(prob_row[kb])
        if c >= thr:
            return n
    return len(order)


def select_row(prob_row: np.ndarray, sim_q_flag: bool, sim_k: np.ndarray,
               topk: float, cdfthreshd: Optional[float],
               valid: Optional[np.ndarray] = None, attention_sink: bool = False) -> np.ndarray:
    """Selected K blocks of one Q-tile row, ascending.

    * If the Q block fails the similarity gate, every K block is selected
      (reading R5: its mean does not stand for the block).
    * Otherwise take the first n blocks of `selection_order`: n from
      `topk_count` when topk > 0, else from `cdf_count` (reading R8: top-k wins
      when both are set).
    * Then add every K block that failed the gate (reading R9: these are
      added after the count, so a row may hold more than n blocks).
    * `valid` (causal mode, reading R23) limits every one of these steps to the
      blocks at or before the tile: "every block" means every valid block, n is
      clamped to the number of valid blocks, and forced blocks must be valid.
      Invalid blocks have probability 0 and a larger index than any valid
      block, so the first n of the order are valid.
    * `attention_sink` (CK page, not-yet-ported list: column 0 forced on)
      adds block 0 to every row.
    """
    nk = prob_row.shape[0]
    if valid is None:
        valid = np.ones(nk, dtype=bool)
    valid = np.asarray(valid, bool)
    n_valid = int(valid.sum())
    if not sim_q_flag:
        chosen = set(int(kb) for kb in np.nonzero(valid)[0])
    else:
        order = selection_order(prob_row)
        if topk is not None and float(np.float32(topk)) > 0.0:
            n = topk_count(topk, nk)
        else:
            if cdfthreshd is None:
                raise ValueError("either topk > 0 or cdfthreshd must be given")
            n = cdf_count(prob_row, order, cdfthreshd)
        n = min(n, n_valid)
        chosen = set(int(kb) for kb in order[:n])
        chosen |= set(int(kb) for kb in np.nonzero(~np.asarray(sim_k, bool) & valid)[0])
    if attention_sink:
        chosen.add(0)
    return np.array(sorted(chosen), dtype=np.int64)


def lut_from_selection(rows: Sequence[np.ndarray], nk: int):
    """Encode per-row selections as (lut [rows, nk] int32 ascending, -1 padded,
    count [rows] int32, bitmap [rows, nk] uint8).  Reading R10."""
    nrows = len(rows)
    lut = np.full((nrows, nk), -1, dtype=np.int32)
    count = np.zeros(nrows, dtype=np.int32)
    bitmap = np.zeros((nrows, nk), dtype=np.uint8)
    for r, sel in enumerate(rows):
        sel = np.asarray(sel, dtype=np.int64)
        lut[r, :len(sel)] = sel
        count[r] = len(sel)
        bitmap[r, sel] = 1
    return lut, count, bitmap


def select_from_probs(prob: np.ndarray, sim_q: np.ndarray, sim_k: np.ndarray,
                      topk: Sequence[float], cdfthreshd: Optional[Sequence[float]],
                      causal: bool = False, attention_sink: bool = False):
    """Selection steps applied to given pooled probabilities and gate flags.

    prob [b, h, nq, nk]; sim_q [b, h, nq]; sim_k [b, h, nk]; topk / cdfthreshd
    per head.  Returns (lut, count, bitmap) shaped [b, h, nq, nk] / [b, h, nq].
    Used both by `block_map` and to re-run the selection on probabilities and
    flags produced elsewhere.
    """
    prob = np.asarray(prob, dtype=np.float64)
    b, h, nq, nk = prob.shape
    lut = np.full((b, h, nq, nk), -1, dtype=np.int32)
    count = np.zeros((b, h, nq), dtype=np.int32)
    bitmap = np.zeros((b, h, nq, nk), dtype=np.uint8)
    for ib in range(b):
        for ih in range(h):
            cdf = None if cdfthreshd is None else cdfthreshd[ih]
            valid = causal_valid(nq, nk) if causal else np.ones((nq, nk), dtype=bool)
            rows = [select_row(prob[ib, ih, qb], bool(sim_q[ib, ih, qb]),
                               sim_k[ib, ih], topk[ih], cdf, valid[qb], attention_sink)
                    for qb in range(nq)]
            l, c, m = lut_from_selection(rows, nk)
            lut[ib, ih], count[ib, ih], bitmap[ib, ih] = l, c, m
    return lut, count, bitmap


def block_map(q: np.ndarray, k: np.ndarray, topk: Sequence[float],
              simthreshd1: Sequence[float], cdfthreshd: Optional[Sequence[float]] = None,
              blk_q: int = 64, blk_k: int = 64, scale: Optional[float] = None,
              smooth_k: bool = False, causal: bool = False,
              attention_sink: bool = False) -> dict:
    """Whole stage 1 for q [b, h, s_q, d] and k [b, h_kv, s_k, d], h % h_kv == 0.

    With h_kv < h (grouped-query attention, reading R28) query head j pools
    against KV head j // (h / h_kv), as attention does (aiter 6841 page, GQA
    mapping): its pooled scores use that head's K block means, and the K gate
    of row j compares that head's K block similarity with simthreshd1[j].
    `smooth_k` pools and gates K after `smooth_keys`; `causal` applies the
    causal block mask (requires s_q = s_k and blk_q = blk_k); `attention_sink`
    forces block 0 in every row.  Returns a dict with q_mean [b, h, nq, d],
    k_mean [b, h_kv, nk, d] (of the smoothed K when smoothing), sim_q_val,
    sim_k_val [b, h_kv, nk], sim_q, sim_k [b, h, nk] (the K gate as row j sees
    it), scores, prob, lut, count, bitmap.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    if causal and (q.shape[2] != k.shape[2] or blk_q != blk_k):
        raise ValueError("causal block map needs s_q = s_k and blk_q = blk_k")
    if smooth_k:
        k = smooth_keys(k)
    b, h, s_q, d = q.shape
    h_kv, s_k = k.shape[1], k.shape[2]
    if h % h_kv:
        raise ValueError("the query heads must be a multiple of the KV heads")
    ratio = h // h_kv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    nq, nk = -(-s_q // blk_q), -(-s_k // blk_k)       # a partial last block counts
    q_mean = np.zeros((b, h, nq, d))
    k_mean = np.zeros((b, h_kv, nk, d))
    sim_q_val = np.zeros((b, h, nq))
    sim_k_val = np.zeros((b, h_kv, nk))
    sim_q = np.zeros((b, h, nq), dtype=bool)
    sim_k = np.zeros((b, h, nk), dtype=bool)
    scores = np.zeros((b, h, nq, nk))
    for ib in range(b):
        for ik in range(h_kv):
            k_mean[ib, ik], sim_k_val[ib, ik], _ = pool_and_gate(k[ib, ik], blk_k, 0.0)
        for ih in range(h):
            ik = ih // ratio
            q_mean[ib, ih], sim_q_val[ib, ih], sim_q[ib, ih] = pool_and_gate(
                q[ib, ih], blk_q, simthreshd1[ih])
            sim_k[ib, ih] = sim_k_val[ib, ik] > simthreshd1[ih]
            scores[ib, ih] = pooled_scores(q_mean[ib, ih], k_mean[ib, ik],
                                           sim_k[ib, ih], scale, causal)
    prob = row_softmax(scores)
    lut, count, bitmap = select_from_probs(prob, sim_q, sim_k, topk, cdfthreshd,
                                           causal, attention_sink)
    return dict(q_mean=q_mean, k_mean=k_mean, sim_q_val=sim_q_val, sim_k_val=sim_k_val,
               sim_q=sim_q, sim_k=sim_k, scores=scores, prob=prob,
               lut=lut, count=count, bitmap=bitmap)


# ----------------------------------------------------------------------------
# Stage 2: attention over the selected keys, and the LSE combine
# ----------------------------------------------------------------------------

def attend(qi: np.ndarray, keys: np.ndarray, values: np.ndarray, scale: float,
           allowed: Optional[np.ndarray] = None):
    """Exact softmax attention of query rows qi [m, d] over keys/values [n, d].

    LSE is the natural log of sum_j exp(scale * q.k_j) (reading R11: the scale is
    inside the LSE).  With no keys, O = 0 and LSE = -inf (Updating Log page,
    Stage 3; aiter 6841 page; reading R12).  `allowed` [m, n] (causal mode)
    removes key j from row i where it is False; a row left with no key gets
    O = 0 and LSE = -inf.
    """
    qi = np.asarray(qi, np.float64)
    m_rows = qi.shape[0]
    if keys.shape[0] == 0:
        return np.zeros((m_rows, values.shape[1])), np.full(m_rows, NEG_INF)
    s = float(scale) * (qi @ np.asarray(keys, np.float64).T)
    if allowed is not None:
        s = np.where(np.asarray(allowed, bool), s, NEG_INF)
    m = s.max(axis=1, keepdims=True)
    empty = m[:, 0] == NEG_INF                      # rows with no allowed key
    m = np.where(empty[:, None], 0.0, m)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    l_safe = np.where(empty[:, None], 1.0, l)
    lse = np.where(empty, NEG_INF, (m + np.log(l_safe))[:, 0])
    o = np.where(empty[:, None], 0.0, (e @ np.asarray(values, np.float64)) / l_safe)
    return o, lse


def block_sparse_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                           lut: Optional[np.ndarray], count: Optional[np.ndarray],
                           blk_q: int = 64, blk_k: int = 64,
                           scale: Optional[float] = None, lut_per_kv_head: bool = False,
                           causal: bool = False):
    """Attention of every Q-tile over the K blocks its LUT row lists.

    q [b, h_q, s_q, d]; k, v [b, h_kv, s_k, d]; query head j reads KV head
    j // (h_q / h_kv) (aiter 6841 page, GQA mapping).  lut [b, h_lut, nq, L]
    with count [b, h_lut, nq]; h_lut = h_kv when `lut_per_kv_head`, else h_q.
    lut = None means every block (dense).  With `causal` (s_q = s_k, reading
    R23) query position i attends only to listed keys j <= i.  Lengths need
    not be multiples of the blocks: the last Q-tile and the last K block are
    partial, and a listed partial block contributes only its existing keys.
    Returns O [b, h_q, s_q, d], LSE [b, h_q, s_q].
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    b, h_q, s_q, d = q.shape
    h_kv, s_k = k.shape[1], k.shape[2]
    ratio = h_q // h_kv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    nq, nk = -(-s_q // blk_q), -(-s_k // blk_k)
    o = np.zeros((b, h_q, s_q, v.shape[3]))
    lse = np.zeros((b, h_q, s_q))
    for ib in range(b):
        for ih in range(h_q):
            hk = ih // ratio
            hl = hk if lut_per_kv_head else ih
            for qb in range(nq):
                if lut is None:
                    blocks = np.arange(nk)
                else:
                    n = int(count[ib, hl, qb])
                    blocks = np.asarray(lut[ib, hl, qb, :n], dtype=np.int64)
                idx = (blocks[:, None] * blk_k + np.arange(blk_k)[None, :]).reshape(-1)
                idx = idx[idx < s_k]
                rows = slice(qb * blk_q, min((qb + 1) * blk_q, s_q))
                allowed = None
                if causal:
                    qpos = np.arange(rows.start, rows.stop)
                    allowed = idx[None, :] <= qpos[:, None]
                o[ib, ih, rows], lse[ib, ih, rows] = attend(
                    q[ib, ih, rows], k[ib, hk, idx], v[ib, hk, idx], scale, allowed)
    return o, lse


def pv_skip_blocks(scores: np.ndarray, tau: float, return_margin: bool = False):
    """Which listed blocks of one Q-tile the pv_threshold rule drops.

    CK page, "Status vs Upstream", not-yet-ported list: pv_threshold is a
    per-Q-tile skip inside the attention kernel, a pure speed measure.  The
    unit is therefore one Q-tile against one listed block.  The pages give no
    test; reading R25 takes the plainest one that leaves the result an
    approximation of the same attention:

    * the listed blocks are visited in LUT order, as by an online softmax, in
      one pass over the row;
    * for query row i of the tile, M_i is its running maximum: the largest
      score of row i over the keys of the blocks visited so far, this block
      included; r_i is its largest score over this block's keys;
    * the block is dropped for the whole tile when r_i < M_i - tau holds for
      every row i of the tile.

    A row with no key in the block has r_i = -inf; while M_i is still -inf
    (the row has met no key yet) the block is kept.

    scores [rows, n_blocks, blk_k] (scaled, -inf where masked).  Returns a bool
    array [n_blocks], True = dropped.  With `return_margin`, also, per block,
    max_i (r_i - (M_i - tau)) over the rows with a key in the block (-inf if
    none): the decision flips where this crosses 0, so it says how far the
    decision lies from the threshold.
    """
    rows, n, _ = scores.shape
    skip = np.zeros(n, dtype=bool)
    margin = np.full(n, NEG_INF)
    run = np.full(rows, NEG_INF)
    for t in range(n):
        r = scores[:, t, :].max(axis=1)                 # [rows]
        run = np.maximum(run, r)
        skip[t] = bool(np.all(r < run - tau))
        live = r > NEG_INF
        if live.any():
            margin[t] = float(np.max(r[live] - (run[live] - tau)))
    return (skip, margin) if return_margin else skip


def block_sparse_attention_pv_skip(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                                   lut: Optional[np.ndarray], count: Optional[np.ndarray],
                                   pv_threshold: float, scale: Optional[float] = None,
                                   lut_per_kv_head: bool = False, causal: bool = False,
                                   return_skips: bool = False, return_margins: bool = False):
    """block_sparse_attention with the pv_threshold skip (reading R25).

    A dropped block's keys still count in each row's softmax denominator and in
    its LSE; only their P.V terms leave the numerator:
        O_i = sum_{j kept} exp(s_ij - m_i) v_j / sum_{j all} exp(s_ij - m_i),
        LSE_i = m_i + ln sum_{j all} exp(s_ij - m_i),
    with m_i the maximum over all of row i's keys.  The LSE therefore equals the
    exact one, and |O_i - O_exact,i| <= (dropped keys of row i) * exp(-tau) *
    max |v|, since every dropped score lies more than tau below m_i.  The blocks
    of 64 queries and 64 keys are the ones of block_sparse_attention.  A
    partial last K block is completed with masked keys (score -inf) and a
    partial last Q-tile with copies of its last row: a copy repeats a decision
    the tile already takes, so the blocks are decided by the tile's own rows.
    With `return_skips`, also returns the number of dropped (tile, block)
    pairs and of all listed pairs; with `return_margins`, then [b, h_q, nq]
    the smallest |margin| (pv_skip_blocks) over the tile's blocks: decisions
    closer than rounding to the threshold may fall either way in another
    precision.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    b, h_q, s_q, d = q.shape
    h_kv, s_k = k.shape[1], k.shape[2]
    ratio = h_q // h_kv
    blk = 64
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    nq, nk = -(-s_q // blk), -(-s_k // blk)
    o = np.zeros((b, h_q, s_q, v.shape[3]))
    lse = np.zeros((b, h_q, s_q))
    n_skip = n_pairs = 0
    near = np.full((b, h_q, nq), math.inf)
    for ib in range(b):
        for ih in range(h_q):
            hk = ih // ratio
            hl = hk if lut_per_kv_head else ih
            for qb in range(nq):
                if lut is None:
                    blocks = np.arange(nk)
                else:
                    blocks = np.asarray(lut[ib, hl, qb, :int(count[ib, hl, qb])], dtype=np.int64)
                rows = slice(qb * blk, min((qb + 1) * blk, s_q))
                nr = rows.stop - rows.start
                n = len(blocks)
                if n == 0:
                    o[ib, ih, rows], lse[ib, ih, rows] = 0.0, NEG_INF
                    continue
                idx = (blocks[:, None] * blk + np.arange(blk)[None, :]).reshape(-1)
                exists = idx < s_k                                         # keys of a partial block
                idx = np.where(exists, idx, 0)
                qpos = np.minimum(np.arange(qb * blk, (qb + 1) * blk), s_q - 1)   # copies of the last row
                s = scale * (q[ib, ih, qpos] @ k[ib, hk, idx].T)          # [64, n * 64]
                allowed = exists[None, :] & (idx[None, :] <= qpos[:, None] if causal else True)
                s = np.where(allowed, s, NEG_INF)
                skip, margin = pv_skip_blocks(s.reshape(blk, n, blk), pv_threshold, return_margin=True)
                near[ib, ih, qb] = np.abs(margin).min()
                n_skip += int(skip.sum())
                n_pairs += n
                # kept[j]: key j of the row's list stays in the numerator
                kept = ~np.repeat(skip, blk)
                m = s.max(axis=1, keepdims=True)
                empty = m[:, 0] == NEG_INF
                m = np.where(empty[:, None], 0.0, m)
                e = np.exp(s - m)
                l = e.sum(axis=1, keepdims=True)
                l_safe = np.where(empty[:, None], 1.0, l)
                num = (e * kept[None, :]) @ v[ib, hk, idx]
                o[ib, ih, rows] = np.where(empty[:, None], 0.0, num / l_safe)[:nr]
                lse[ib, ih, rows] = np.where(empty, NEG_INF, (m + np.log(l_safe))[:, 0])[:nr]
    out = (o, lse)
    if return_skips:
        out += (n_skip, n_pairs)
    if return_margins:
        out += (near,)
    return out


def quantize_block_int8(x_blk: np.ndarray):
    """Symmetric int8 codes of one block of tokens, with one fp32 scale.

    CK page, "Status vs Upstream", not-yet-ported list: Q/K int8 quantisation
    fused into the pool kernel, feeding an int8 QK GEMM in the attention
    kernel.  The pages give no formula.  Reading R27: the block is the
    64-token pooling block; scale = absmax / 127 and
    code = round-half-even(x * (127 / absmax)), clamped to [-127, 127], each
    operation in fp32 (the codes are integers decided by floating point, so
    the oracle takes the decision in the kernel's precision).  An all-zero
    block has scale 0 and codes 0.  x_blk holds values exact in fp32 (the
    fp16 / bf16 inputs).  Returns (int8 codes, np.float32 scale).
    """
    x = np.asarray(x_blk, np.float32)
    amax = np.float32(np.abs(x).max()) if x.size else np.float32(0)
    if amax == 0:
        return np.zeros(x.shape, np.int8), np.float32(0)
    inv = np.float32(127) / amax
    codes = np.clip(np.rint(x * inv), -127, 127).astype(np.int8)
    return codes, amax / np.float32(127)


def quantize_int8(x: np.ndarray, blk: int = 64):
    """quantize_block_int8 over every block of `blk` tokens of x [b, h, s, d]
    (a partial last block quantises its own tokens, reading R1).
    Returns codes [b, h, s, d] int8 and scales [b, h, ceil(s / blk)] fp32."""
    b, h, s, d = x.shape
    nb = -(-s // blk)
    codes = np.zeros((b, h, s, d), np.int8)
    scales = np.zeros((b, h, nb), np.float32)
    for ib in range(b):
        for ih in range(h):
            for j in range(nb):
                rows = slice(j * blk, (j + 1) * blk)
                codes[ib, ih, rows], scales[ib, ih, j] = quantize_block_int8(x[ib, ih, rows])
    return codes, scales


def dequantize_int8(codes: np.ndarray, scales: np.ndarray, blk: int = 64) -> np.ndarray:
    """codes * scale of their block, in fp64 (exact: an int8 code, or an fp8
    e4m3 code value, times an fp32)."""
    per_row = np.repeat(scales.astype(np.float64), blk, axis=2)[:, :, :codes.shape[2]]
    return codes.astype(np.float64) * per_row[..., None]


def block_sparse_attention_qk_int8(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                                   lut: Optional[np.ndarray], count: Optional[np.ndarray],
                                   scale: Optional[float] = None, lut_per_kv_head: bool = False,
                                   causal: bool = False):
    """block_sparse_attention with Q and K replaced by their int8 block codes
    times their scales (reading R27): scores are scale * sq * sk * (cq . ck),
    everything after them as in block_sparse_attention (V unquantised)."""
    cq, sq = quantize_int8(q)
    ck, sk = quantize_int8(k)
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[3])
    return block_sparse_attention(dequantize_int8(cq, sq), dequantize_int8(ck, sk), v, lut, count,
                                  scale=scale, lut_per_kv_head=lut_per_kv_head, causal=causal)


E4M3_MAX = 448.0     # largest finite OCP fp8 e4m3 value: 1.75 * 2^8


def round_e4m3(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the OCP fp8 e4m3 grid, to nearest with ties to
    even, saturating at +-448 (reading R29).

    The grid: 4 exponent bits with bias 7 and 3 mantissa bits; normal values
    (1 + m/8) * 2^e for e in [-6, 8] (the top binade stops at 1.75 * 2^8 =
    448), subnormal values m * 2^-9.  In a binade [2^e, 2^(e+1)) the spacing
    is 2^(e-3); below 2^-6 it is 2^-9.  Values from 464 up (past the
    midpoint above 448) never arise in the quantisation, whose inputs stay
    within 448 * (1 + 2^-23); they saturate here.  Returns float64 values on
    the grid.
    """
    x = np.asarray(x, np.float64)
    a = np.abs(x)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    step = np.where(a >= 2.0 ** -6, 2.0 ** (e - 3), 2.0 ** -9)
    q = np.round(a / step) * step            # np.round: half to even on the exact quotient
    q = np.minimum(q, E4M3_MAX)
    return np.where(a > 0, np.sign(x) * q, 0.0)


def e4m3_value(codes: np.ndarray) -> np.ndarray:
    """Value of OCP fp8 e4m3 bytes (sign, 4 exponent bits with bias 7, 3
    mantissa bits; exponent 0 is subnormal, 0x7F / 0xFF are NaN)."""
    b = np.asarray(codes, np.uint8).astype(np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    ex, m = (b >> 3) & 0xF, b & 0x7
    mag = np.where(ex == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * 2.0 ** (ex - 7.0))
    return np.where((b & 0x7F) == 0x7F, np.nan, sign * mag)


def e4m3_code(values: np.ndarray) -> np.ndarray:
    """The OCP fp8 e4m3 byte of values already on the grid (zero as 0x00)."""
    v = np.asarray(values, np.float64)
    table = e4m3_value(np.arange(256, dtype=np.uint8))
    table = np.where(np.isnan(table), np.inf, table)
    table[0x80] = np.inf                         # -0 never produced: zero encodes as 0x00
    idx = np.abs(table[None, :] - v.reshape(-1, 1)).argmin(axis=1)
    if not np.all(table[idx] == v.reshape(-1)):
        raise ValueError("values off the e4m3 grid")
    return idx.astype(np.uint8).reshape(v.shape)


def quantize_block_fp8(x_blk: np.ndarray):
    """fp8 e4m3 codes of one block of tokens, with one fp32 scale.

    CK page, "Status vs Upstream", not-yet-ported list: Q/K quantisation in
    the pool kernel for a low-precision QK product in the attention kernel;
    the aiter 6841 page runs fp8 Q/K recipes.  Reading R29, the fp8 twin of
    R27: the 64-token pooling block, symmetric, scale = absmax / 448 and code =
    round_e4m3(x * (448 / absmax)), each operation in fp32 (the division
    correctly rounded), the last rounding to the e4m3 grid to nearest even.
    An all-zero block has scale 0 and codes 0.  Returns (code values on the
    e4m3 grid as float64, np.float32 scale).
    """
    x = np.asarray(x_blk, np.float32)
    amax = np.float32(np.abs(x).max()) if x.size else np.float32(0)
    if amax == 0:
        return np.zeros(x.shape), np.float32(0)
    inv = np.float32(E4M3_MAX) / amax
    return round_e4m3(x * inv), amax / np.float32(E4M3_MAX)


def quantize_fp8(x: np.ndarray, blk: int = 64):
    """quantize_block_fp8 over every block of `blk` tokens of x [b, h, s, d]
    (a partial last block quantises its own tokens, reading R1).  Returns code
    values [b, h, s, d] (float64, on the e4m3 grid) and scales
    [b, h, ceil(s / blk)] fp32."""
    b, h, s, d = x.shape
    nb = -(-s // blk)
    codes = np.zeros((b, h, s, d))
    scales = np.zeros((b, h, nb), np.float32)
    for ib in range(b):
        for ih in range(h):
            for j in range(nb):
                rows = slice(j * blk, (j + 1) * blk)
                codes[ib, ih, rows], scales[ib, ih, j] = quantize_block_fp8(x[ib, ih, rows])
    return codes, scales


def block_sparse_attention_qk_fp8(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                                  lut: Optional[np.ndarray], count: Optional[np.ndarray],
                                  scale: Optional[float] = None, lut_per_kv_head: bool = False,
                                  causal: bool = False):
    """block_sparse_attention with Q and K replaced by their fp8 e4m3 block
    codes times their scales (reading R29): scores are
    scale * sq * sk * (cq . ck), everything after them as in
    block_sparse_attention (V unquantised)."""
    cq, sq = quantize_fp8(q)
    ck, sk = quantize_fp8(k)
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[3])
    return block_sparse_attention(dequantize_int8(cq, sq), dequantize_int8(ck, sk), v, lut, count,
                                  scale=scale, lut_per_kv_head=lut_per_kv_head, causal=causal)


def token_list_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                         lists: np.ndarray, scale: Optional[float] = None):
    """Decode-style attention over per-(b, KV head) token index lists.

    q [b, h_q, s_q, d] (s_q usually 1); k, v [b, h_kv, s_k, d]; lists
    [b, h_kv, L] int with -1 = skip (aiter 4919 page: -1 sentinels; reading
    R14: one list per KV head, shared by its query-head group, applied to
    every query position).  Query head j reads KV head j // (h_q / h_kv).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    b, h_q, s_q, d = q.shape
    h_kv = k.shape[1]
    ratio = h_q // h_kv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = np.zeros((b, h_q, s_q, v.shape[3]))
    lse = np.zeros((b, h_q, s_q))
    for ib in range(b):
        for ih in range(h_q):
            hk = ih // ratio
            row = np.asarray(lists[ib, hk], dtype=np.int64)
            idx = row[row >= 0]
            o[ib, ih], lse[ib, ih] = attend(q[ib, ih], k[ib, hk, idx], v[ib, hk, idx], scale)
    return o, lse


def combine(o_parts: Sequence[np.ndarray], lse_parts: Sequence[np.ndarray]):
    """Merge partial attention results by their LSE.

    Updating Log page, Stage 1: Combine(FA(A), FA(B)) = FA(A u B) with the
    running-max trick; an empty partial (LSE = -inf) is the identity.  aiter
    4919 page: partials whose maximum is -inf are masked before the
    exponential.  Reading R13: when every partial is -inf the result is O = 0,
    LSE = -inf.

    o_parts: n arrays [..., d]; lse_parts: n arrays [...].
    """
    lse = np.stack([np.asarray(x, np.float64) for x in lse_parts])   # [n, ...]
    o = np.stack([np.asarray(x, np.float64) for x in o_parts])       # [n, ..., d]
    m = lse.max(axis=0)                                              # [...]
    finite = lse > NEG_INF
    safe_m = np.where(m > NEG_INF, m, 0.0)
    w = np.where(finite, np.exp(np.where(finite, lse, 0.0) - safe_m), 0.0)
    total = w.sum(axis=0)
    empty = ~(total > 0.0)
    denom = np.where(empty, 1.0, total)
    out = (w[..., None] * o).sum(axis=0) / denom[..., None]
    out[empty] = 0.0
    lse_out = np.where(empty, NEG_INF, safe_m + np.log(denom))
    return out, lse_out


def dense_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                    scale: Optional[float] = None):
    """softmax(scale * Q K^T) V and its LSE over every key, per (b, h); the
    definition the sparse path reduces to when every block is selected."""
    q = np.asarray(q, np.float64)
    b, h_q, s_q, d = q.shape
    h_kv = k.shape[1]
    ratio = h_q // h_kv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = np.zeros((b, h_q, s_q, v.shape[3]))
    lse = np.zeros((b, h_q, s_q))
    for ib in range(b):
        for ih in range(h_q):
            o[ib, ih], lse[ib, ih] = attend(q[ib, ih], np.asarray(k[ib, ih // ratio], np.float64),
                                            np.asarray(v[ib, ih // ratio], np.float64), scale)
    return o, lse
