"""Benchmark of the block-sparse attention forward on one MI355X.

Workload: b=2 h=32 s=16384 d=128 fp16, 64-token blocks, simthreshd1 0.001,
block-centroid + noise Q/K (centroid scale 0.5..2 over the heads, noise 0.5),
V ~ N(0, 1), seeded synthetic data resident in HBM before timing starts.

One step = the whole block-sparse forward: sparge_build_block_map (pool +
gate kernel, score + select kernel) then sparse_fmha_fwd over the LUT, at
topk 0.4 for every head.  `value` is the dense-equivalent throughput of a
step, 4*b*h*s*s*d / step time, in TFLOP/s, over exactly --steps timed steps.
The same line carries:
  * interleaved arms at topk 0.1, 0.2, 0.4, 0.6, 0.8 and the mixed per-head
    sweep, and the dense FMHA baseline (the same kernel, every block);
  * the roofline of the sparse FMHA kernel, from HIP events around each of
    its launches in the timed region, with two ceilings measured beside it
    (the fp16 MFMA rate on realistic operands, and a loop of the FMHA's
    instruction volume without its dependences);
  * rows outside the headline: the b1 h8 s4096 bf16 config, the two-pass
    combine, the combine on headline-sized partials and the split-K decode
    (short launch sequences timed as HIP graphs, warm and with the caches
    flushed), causal prefill, pv_threshold, a ragged length, bf16, int8 and
    fp8 Q/K;
  * the fp64 CPU oracle timed on a bounded sample in a process pool.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-extras]
       python bench.py --profile-arm {0.1,...,mixed,dense} --steps K --warmup W
       python bench.py --ceilings-only
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_FP16_TFLOPS = 2500.0     # MI355X dense fp16 / bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
# rocprofv3 FETCH_SIZE / WRITE_SIZE summary of the sparse FMHA (bytes per launch,
# copy-calibrated); quoted only while it matches the current kernel source.
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "fmha_block_headline_traffic.md")
B, H, S, D = 2, 32, 16384, 128
F_BLK = 4 * 64 * 64 * D          # flop per (64-query tile, 64-key block) pair


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def median(x):
    s = sorted(x)
    n = len(s)
    return s[n // 2] if n % 2 else 0.5 * (s[n // 2 - 1] + s[n // 2])


def timed_steps(step, steps, warmup, torch, fmha_events=None):
    """The contract's timed region: `warmup` untimed steps, then exactly `steps`
    steps between two synchronisations, timed with HIP events on the launching
    stream (and the host clock).  step(i) may record per-step events.
    Returns (event ms per step, wall ms per step)."""
    for i in range(warmup):
        step(None)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for i in range(steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    return e0.elapsed_time(e1) / steps, wall


def interleaved(fns, rounds, warmup, torch):
    """A/B timing: every round runs each arm once, in an order that rotates
    from round to round, with HIP events around each call.  Returns
    {name: [ms per call]}."""
    names = list(fns)
    for _ in range(warmup):
        for n in names:
            fns[n]()
    torch.cuda.synchronize()
    evs = {n: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(rounds)] for n in names}
    for r in range(rounds):
        order = names[r % len(names):] + names[:r % len(names)]
        for n in order:
            a, b = evs[n][r]
            a.record()
            fns[n]()
            b.record()
    torch.cuda.synchronize()
    return {n: [a.elapsed_time(b) for a, b in evs[n]] for n in names}


def graph_ms(fn, torch, reps=20, replays=10):
    """Device time per call of a short launch sequence with no host gaps:
    `reps` calls of fn captured in one HIP graph, replayed `replays` times
    between HIP events.  fn must allocate nothing.  Returns (median ms per
    call, the graph)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            fn()
    g.replay()
    torch.cuda.synchronize()
    per = []
    for _ in range(replays):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        per.append(a.elapsed_time(b) / reps)
    return median(per), g


def graph_cold_ms(fn, torch, flush, replays=10):
    """Device time of one call captured in a graph, each replay preceded (outside
    the timed events) by a read of a 1 GiB buffer, which leaves L2 and MALL
    holding none of the call's data.  A read, not a write: a flushing write
    leaves dirty lines whose write-back to HBM would run inside the timed call
    (a sequential 512 MiB read measured 3.7 TB/s after a 512 MiB write, 5.9
    after a 1 GiB read or warm)."""
    _, g = graph_ms(fn, torch, reps=1, replays=1)
    per = []
    for _ in range(replays):
        flush.sum(dtype=torch.int32)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        per.append(a.elapsed_time(b))
    return median(per)


def _oracle_slice(job):
    """One (b, h) slice of the CPU baseline in a worker process: the fp64
    oracle's block map and attention over the selected blocks, on one BLAS
    thread.  Returns (seconds, selected block pairs, block-map seconds,
    attention seconds)."""
    q, k, v, topk = job
    from threadpoolctl import threadpool_limits
    import oracle
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        bm = oracle.block_map(q, k, topk=[topk], simthreshd1=[0.001])
        t1 = time.perf_counter()
        oracle.block_sparse_attention(q, k, v, bm["lut"], bm["count"])
        t2 = time.perf_counter()
        return t2 - t0, int(bm["count"].sum()), t1 - t0, t2 - t1


def cpu_baseline(topk=0.4, max_workers=16):
    """The fp64 oracle timed on the host cores, before the GPU is touched
    (the workers are forked).  Sample: the 32 heads of batch 0 of the
    headline workload (drawn on the host: same recipe, other random draws),
    one (b, h) slice per task, over min(16, host CPUs) worker processes with
    one BLAS thread each.  Value: dense-equivalent TFLOP/s of the sample."""
    import multiprocessing as mp
    import concurrent.futures as cf
    import torch
    from block_sparse_attention_sparge_amd import synth
    torch.set_num_threads(1)
    case = synth.headline_case("cpu", topk=topk, b=1)
    jobs = [(case.q[:, h:h + 1].double().numpy(), case.k[:, h:h + 1].double().numpy(),
             case.v[:, h:h + 1].double().numpy(), topk) for h in range(H)]
    del case
    workers = max(1, min(max_workers, os.cpu_count() or 1))
    t0 = time.perf_counter()
    with cf.ProcessPoolExecutor(max_workers=workers, mp_context=mp.get_context("fork")) as ex:
        res = list(ex.map(_oracle_slice, jobs))
    dt = time.perf_counter() - t0
    dense_flops = 4.0 * len(jobs) * S * S * D
    return dict(value=dense_flops / dt / 1e12, unit="TFLOP/s (dense-equivalent)", cores=workers,
                kind="oracle",
                sample=f"32 (b, h) slices (b=0, h=0..31) of b2 h32 s16384 d128 at topk {topk}: fp64 oracle "
                       f"block map + attention over the selected blocks, {workers} worker processes with one "
                       f"BLAS thread each, {dt:.1f} s wall ({sum(r[0] for r in res):.0f} s of CPU work)",
                seconds=dt, cpu_seconds=sum(r[0] for r in res),
                cpu_seconds_block_map=sum(r[2] for r in res), cpu_seconds_attention=sum(r[3] for r in res),
                host_cpus=os.cpu_count())


def step_arms(ops, case, arms, rounds, warmup, torch):
    """Interleaved timing of the block map, the sparse FMHA and the whole step
    for each top-k arm (one fraction for every head, or a per-head list), and
    of the dense FMHA."""
    o = torch.empty_like(case.q)
    lse = torch.empty(case.q.shape[:3], dtype=torch.float32, device=case.q.device)
    fns, maps = {}, {}
    for name, tk in arms.items():
        ws = {}
        ws.update(ops.build_block_map(case.q, case.k, tk, case.simthreshd1, out=ws))
        maps[name] = ws

        def bm(tk=tk, ws=ws):
            ops.build_block_map(case.q, case.k, tk, case.simthreshd1, out=ws)

        def fm(ws=ws):
            ops.sparse_fmha_fwd(case.q, case.k, case.v, ws["lut"], ws["count"], o=o, lse=lse)

        fns[f"{name}/block_map"] = bm
        fns[f"{name}/fmha"] = fm
        fns[f"{name}/step"] = lambda bm=bm, fm=fm: (bm(), fm())
    fns["dense"] = lambda: ops.dense_fmha_fwd(case.q, case.k, case.v, o=o, lse=lse)
    t = interleaved(fns, rounds, warmup, torch)
    out = {}
    for name in arms:
        out[name] = dict(block_map_ms=median(t[f"{name}/block_map"]), fmha_ms=median(t[f"{name}/fmha"]),
                         step_ms=median(t[f"{name}/step"]), pairs=int(maps[name]["count"].sum().item()),
                         fmha_spread=(max(t[f"{name}/fmha"]) - min(t[f"{name}/fmha"])) / median(t[f"{name}/fmha"]))
    return out, median(t["dense"])


def extras(ops, synth, torch, steps, warmup):
    out = {}
    dev = torch.device("cuda:0")
    flush = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
    # M: b1 h8 s4096 d128 bf16 (centroid scale 1, noise 0.5), topk 0.4 and 1.0,
    # and the dense FMHA; short launches, so each sequence is timed as a HIP
    # graph of 20 back-to-back calls.
    log("M config b1 h8 s4096 d128 bf16")
    mc = synth.mid_case(dev)
    om = torch.empty_like(mc.q)
    lm = torch.empty(mc.q.shape[:3], dtype=torch.float32, device=dev)
    dense_m, _ = graph_ms(lambda: ops.dense_fmha_fwd(mc.q, mc.k, mc.v, o=om, lse=lm), torch)
    mrow = dict(workload="b1 h8 s4096 d128 bf16, centroid scale 1, noise 0.5", dense_fmha_ms=dense_m,
                timing="HIP graph of 20 back-to-back calls, median of 10 replays")
    flops_m = 4.0 * 1 * 8 * 4096 * 4096 * 128
    for tk in (0.4, 1.0):
        ws = {}
        ws.update(ops.build_block_map(mc.q, mc.k, [tk] * 8, mc.simthreshd1, out=ws))

        def bm(tk=tk, ws=ws):
            ops.build_block_map(mc.q, mc.k, [tk] * 8, mc.simthreshd1, out=ws)

        def fm(ws=ws):
            ops.sparse_fmha_fwd(mc.q, mc.k, mc.v, ws["lut"], ws["count"], o=om, lse=lm)

        bms, _ = graph_ms(bm, torch)
        fms, _ = graph_ms(fm, torch)
        sts, _ = graph_ms(lambda: (bm(), fm()), torch)
        pairs = int(ws["count"].sum().item())
        mrow[f"topk_{tk}"] = dict(step_ms=sts, block_map_ms=bms, fmha_ms=fms, pairs=pairs,
                                  dense_equiv_tflops=flops_m / sts / 1e9,
                                  actual_tflops_fmha=pairs * F_BLK / fms / 1e9,
                                  speedup_vs_dense_step=dense_m / sts)
    out["m_config"] = mrow
    del mc, om, lm
    # Two-pass combine, b1 h16 s_q1024 s_k32768 d128 bf16: pass A (last 4 blocks)
    # and pass B (64 listed blocks, 10% of rows empty) into fp32 partials, then
    # attn_combine.  Graph-timed (no host gaps), warm and with L2/MALL flushed.
    log("two-pass combine")
    c = synth.combine_case(dev)
    oa, la = ops.sparse_fmha_fwd(c.q, c.k, c.v, c.lut_a, c.count_a, out_dtype=torch.float32)
    ob, lb = ops.sparse_fmha_fwd(c.q, c.k, c.v, c.lut_b, c.count_b, out_dtype=torch.float32)
    parts, lses = torch.stack([oa, ob]), torch.stack([la, lb])
    oc = torch.empty_like(c.q)
    lc = torch.empty_like(la)

    def two_pass():
        ops.sparse_fmha_fwd(c.q, c.k, c.v, c.lut_a, c.count_a, o=parts[0], lse=lses[0],
                            out_dtype=torch.float32)
        ops.sparse_fmha_fwd(c.q, c.k, c.v, c.lut_b, c.count_b, o=parts[1], lse=lses[1],
                            out_dtype=torch.float32)
        ops.attn_combine(parts, lses, o=oc, lse=lc)

    def comb():
        ops.attn_combine(parts, lses, o=oc, lse=lc)

    tp, _ = graph_ms(two_pass, torch)
    cm, _ = graph_ms(comb, torch)
    tp_cold = graph_cold_ms(two_pass, torch, flush)
    cm_cold = graph_cold_ms(comb, torch, flush)
    comb_bytes = parts.numel() * 4 + lses.numel() * 4 + oc.numel() * 2 + lc.numel() * 4
    out["two_pass_combine"] = dict(workload="b1 h16 s_q1024 s_k32768 d128 bf16", ms=tp, combine_ms=cm,
                                   combine_gbs=comb_bytes / cm / 1e6, cold_ms=tp_cold, cold_combine_ms=cm_cold,
                                   cold_combine_gbs=comb_bytes / cm_cold / 1e6, combine_bytes=comb_bytes,
                                   timing="HIP graph of 20 back-to-back sequences (warm); one sequence per "
                                          "graph replay after a 1 GiB read that evicts L2 and MALL (cold)")
    del c, oa, ob, parts, lses, oc, lc
    # Combine on headline-shaped fp32 partials: 2 x [2, 32, 16384, 128].
    parts = torch.randn(2, B, H, S, D, device=dev)
    lses = torch.randn(2, B, H, S, device=dev)
    oc = torch.empty((B, H, S, D), dtype=torch.float16, device=dev)
    lc = torch.empty((B, H, S), device=dev)
    cm, _ = graph_ms(lambda: ops.attn_combine(parts, lses, o=oc, lse=lc), torch, reps=5)
    comb_bytes = parts.numel() * 4 + lses.numel() * 4 + oc.numel() * 2 + lc.numel() * 4
    out["combine_headline_partials"] = dict(workload="2 x [2,32,16384,128] fp32 -> fp16", ms=cm,
                                            gbs=comb_bytes / cm / 1e6, frac_hbm=comb_bytes / cm / 1e6 / PEAK_HBM_GBS)
    del parts, lses, oc, lc
    # Decode GQA, b64 h_q32 h_kv8 s_k32768 d128 bf16, 2048-entry lists, 4 splits + combine
    # (split + combine measured fastest at 4 splits for this shape, of 2 to 16).
    log("decode")
    dc = synth.decode_case(dev)
    S_SPLIT = 4
    op = torch.empty((S_SPLIT, 64, 32, 1, 128), device=dev)
    lp = torch.empty((S_SPLIT, 64, 32, 1), device=dev)
    od = torch.empty_like(dc.q)
    ld = torch.empty((64, 32, 1), device=dev)

    def dec_fmha():
        ops.sparse_fmha_fwd(dc.q, dc.k, dc.v, dc.lists, None, blk_q=1, blk_k=1,
                            num_splits=S_SPLIT, o=op, lse=lp, out_dtype=torch.float32)

    def decode():
        dec_fmha()
        ops.attn_combine(op, lp, o=od, lse=ld)

    dm, _ = graph_ms(decode, torch)
    dfm, _ = graph_ms(dec_fmha, torch)
    dm_cold = graph_cold_ms(decode, torch, flush)
    dfm_cold = graph_cold_ms(dec_fmha, torch, flush)
    gathered = 64 * 8 * 2048 * 128 * 2 * 2
    # n_eff = 1 / sum p^2 of each query row's attention over its listed keys
    # (aiter 6841 page, input distributions), from fp32 scores of the same inputs.
    idx = dc.lists.long().clamp_min(0)                           # [64, 8, 2048]
    kg = torch.gather(dc.k, 2, idx[..., None].expand(-1, -1, -1, 128)).float()
    qg = dc.q.float().reshape(64, 8, 4, 128)
    p = torch.softmax(torch.matmul(qg, kg.transpose(-1, -2).contiguous()) / math.sqrt(128), dim=-1)
    neff = (1.0 / (p * p).sum(-1)).flatten().sort().values.cpu()
    del kg, qg, p
    out["decode_gqa"] = dict(
        workload="b64 h_q32 h_kv8 s_k32768 d128 bf16, 2048 listed keys, 4 splits + combine",
        ms=dm, fmha_ms=dfm, gathered_gbs=gathered / dm / 1e6, frac_hbm=gathered / dm / 1e6 / PEAK_HBM_GBS,
        fmha_gathered_gbs=gathered / dfm / 1e6,
        cold_ms=dm_cold, cold_fmha_ms=dfm_cold, cold_gathered_gbs=gathered / dm_cold / 1e6,
        cold_frac_hbm=gathered / dm_cold / 1e6 / PEAK_HBM_GBS,
        n_eff_median=float(neff[len(neff) // 2]), n_eff_p10=float(neff[len(neff) // 10]),
        n_eff_p90=float(neff[(9 * len(neff)) // 10]),
        timing="HIP graph of 20 back-to-back calls (warm); one call per graph replay after a 1 GiB read that "
               "evicts L2 and MALL (cold)")
    del dc, op, lp, od, ld, flush
    # Causal prefill at the headline shape (b2 h32 s16384 d128 fp16, topk 0.4):
    # block map with K smoothing, the causal block mask and the attention sink,
    # then the causal sparse FMHA; the causal dense FMHA is the baseline.
    log("causal, pv_threshold, ragged, bf16, int8 rows")
    hc = synth.headline_case(dev, topk=0.4)
    ws = {}

    def causal_map():
        return ops.build_block_map(hc.q, hc.k, hc.topk, hc.simthreshd1, out=ws, smooth_k=True,
                                   causal=True, attention_sink=True)

    bm = causal_map()
    ws.update(bm)                 # later calls reuse these outputs
    o = torch.empty_like(hc.q)
    l = torch.empty((B, H, S), device=dev)
    t = interleaved({"map": causal_map,
                     "fmha": lambda: ops.sparse_fmha_fwd(hc.q, hc.k, hc.v, bm["lut"], bm["count"], o=o, lse=l,
                                                         causal=True),
                     "dense": lambda: ops.sparse_fmha_fwd(hc.q, hc.k, hc.v, None, None, o=o, lse=l, causal=True)},
                    max(5, steps // 2), 1, torch)
    bmt, ft, dt = median(t["map"]), median(t["fmha"]), median(t["dense"])
    pairs = int(bm["count"].sum().item())
    dense_pairs = B * H * (S // 64) * (S // 64 + 1) // 2
    out["causal_headline"] = dict(
        workload="b2 h32 s16384 d128 fp16, topk 0.4, smooth_k + causal + attention_sink",
        block_map_ms=bmt, fmha_ms=ft, pairs=pairs, fmha_tflops_computed=pairs * F_BLK / ft / 1e9,
        dense_causal_ms=dt, dense_causal_pairs=dense_pairs,
        dense_causal_tflops_computed=dense_pairs * F_BLK / dt / 1e9,
        speedup_vs_dense_step=dt / (bmt + ft))
    # pv_threshold (one decision per Q-tile and listed block), topk 0.4: on the
    # whole headline, and on its peaked heads 21..31 (centroid scale 1.47..2),
    # where most listed blocks lie far below the tile's running maxima.
    bm = ops.build_block_map(hc.q, hc.k, hc.topk, hc.simthreshd1, out=ws)
    pk = slice(21, 32)
    qp, kp, vp = hc.q[:, pk], hc.k[:, pk], hc.v[:, pk]
    lutp, cntp = bm["lut"][:, pk].contiguous(), bm["count"][:, pk].contiguous()
    op_ = torch.empty_like(qp)
    lp_ = torch.empty(qp.shape[:3], device=dev)
    fns = {}
    for tau in (0.0, 1.0, 2.0, 4.0):
        fns[f"all/{tau}"] = lambda tau=tau: ops.sparse_fmha_fwd(hc.q, hc.k, hc.v, bm["lut"], bm["count"], o=o,
                                                                lse=l, pv_threshold=tau)
        fns[f"peaked/{tau}"] = lambda tau=tau: ops.sparse_fmha_fwd(qp, kp, vp, lutp, cntp, o=op_, lse=lp_,
                                                                   pv_threshold=tau)
    t = interleaved(fns, steps, warmup, torch)
    pv = {k: median(v) for k, v in t.items()}
    out["pv_skip_headline"] = dict(
        workload="b2 h32 s16384 d128 fp16, topk 0.4, pv_threshold 0 / 1 / 2 / 4; 'peaked' = heads 21..31",
        fmha_ms={k: round(v, 4) for k, v in pv.items()},
        speedup_all_tau1=pv["all/0.0"] / pv["all/1.0"],
        speedup_all_tau2=pv["all/0.0"] / pv["all/2.0"], speedup_all_tau4=pv["all/0.0"] / pv["all/4.0"],
        speedup_peaked_tau1=pv["peaked/0.0"] / pv["peaked/1.0"],
        speedup_peaked_tau2=pv["peaked/0.0"] / pv["peaked/2.0"],
        speedup_peaked_tau4=pv["peaked/0.0"] / pv["peaked/4.0"])
    del qp, kp, vp, lutp, cntp, op_, lp_
    # A ragged length at the headline shape: s = 16347 (255 full blocks and
    # one of 27 tokens), the same tensors viewed shorter.  The block map pools
    # the partial block; the FMHA runs its masked kernel for it.
    SR = 16347
    qr, kr, vr = hc.q[:, :, :SR], hc.k[:, :, :SR], hc.v[:, :, :SR]
    bmr = ops.build_block_map(qr, kr, hc.topk, hc.simthreshd1)
    orr = torch.empty((B, H, SR, qr.shape[3]), dtype=qr.dtype, device=dev)
    lr = torch.empty((B, H, SR), device=dev)
    t = interleaved({"map": lambda: ops.build_block_map(qr, kr, hc.topk, hc.simthreshd1, out=bmr),
                     "fmha": lambda: ops.sparse_fmha_fwd(qr, kr, vr, bmr["lut"], bmr["count"], o=orr, lse=lr)},
                    steps, warmup, torch)
    pairs = int(bmr["count"].sum().item())
    out["ragged_headline"] = dict(
        workload="b2 h32 s16347 d128 fp16 (last block 27 tokens), topk 0.4",
        block_map_ms=median(t["map"]), fmha_ms=median(t["fmha"]), pairs=pairs,
        fmha_tflops_computed=pairs * F_BLK / median(t["fmha"]) / 1e9)
    del bmr, orr, lr
    # The same shape in bf16 (topk 0.4): block map and sparse FMHA.
    hb = synth.headline_case(dev, topk=0.4, dtype=torch.bfloat16)
    bmb = ops.build_block_map(hb.q, hb.k, hb.topk, hb.simthreshd1)
    ob = torch.empty_like(hb.q)
    t = interleaved({"map": lambda: ops.build_block_map(hb.q, hb.k, hb.topk, hb.simthreshd1, out=bmb),
                     "fmha": lambda: ops.sparse_fmha_fwd(hb.q, hb.k, hb.v, bmb["lut"], bmb["count"], o=ob, lse=l)},
                    steps, warmup, torch)
    pairs = int(bmb["count"].sum().item())
    out["bf16_headline_topk_0.4"] = dict(
        workload="b2 h32 s16384 d128 bf16, topk 0.4", block_map_ms=median(t["map"]), fmha_ms=median(t["fmha"]),
        pairs=pairs, fmha_tflops_computed=pairs * F_BLK / median(t["fmha"]) / 1e9,
        mfma_frac_fmha=pairs * F_BLK / median(t["fmha"]) / 1e9 / PEAK_FP16_TFLOPS)
    del hb, bmb, ob
    # int8 and fp8 (e4m3) Q/K at the headline shape: the block map with the
    # fused per-block quantisation, then the 8-bit-QK sparse FMHA (V and P
    # stay fp16), against the fp16 FMHA on the same LUT.
    for topk in (0.4, 0.1):
        tk = [topk] * H
        q8 = ops.build_block_map(hc.q, hc.k, tk, hc.simthreshd1, quantize_int8=True)
        f8 = ops.build_block_map(hc.q, hc.k, tk, hc.simthreshd1, quantize_fp8=True)
        t = interleaved({
            "map8": lambda: ops.build_block_map(hc.q, hc.k, tk, hc.simthreshd1, out=q8, quantize_int8=True),
            "mapf8": lambda: ops.build_block_map(hc.q, hc.k, tk, hc.simthreshd1, out=f8, quantize_fp8=True),
            "fmha8": lambda: ops.sparse_fmha_fwd_qk_int8(q8["q_i8"], q8["q_i8_scale"], q8["k_i8"], q8["k_i8_scale"],
                                                         hc.v, q8["lut"], q8["count"], o=o, lse=l),
            "fmhaf8": lambda: ops.sparse_fmha_fwd_qk_fp8(f8["q_fp8"], f8["q_fp8_scale"], f8["k_fp8"],
                                                         f8["k_fp8_scale"], hc.v, f8["lut"], f8["count"], o=o, lse=l),
            "fmha16": lambda: ops.sparse_fmha_fwd(hc.q, hc.k, hc.v, q8["lut"], q8["count"], o=o, lse=l)},
            steps, warmup, torch)
        pairs = int(q8["count"].sum().item())
        ft, ftf, ft16 = median(t["fmha8"]), median(t["fmhaf8"]), median(t["fmha16"])
        out[f"qk_int8_topk_{topk}"] = dict(
            workload=f"b2 h32 s16384 d128, int8 Q/K codes per 64-token block, fp16 V, topk {topk}",
            block_map_ms=median(t["map8"]), fmha_ms=ft, fmha_fp16_same_lut_ms=ft16,
            fmha_speedup_vs_fp16=ft16 / ft, pairs=pairs, fmha_tflops_computed=pairs * F_BLK / ft / 1e9)
        out[f"qk_fp8_topk_{topk}"] = dict(
            workload=f"b2 h32 s16384 d128, fp8 e4m3 Q/K codes per 64-token block, fp16 V, topk {topk}",
            block_map_ms=median(t["mapf8"]), fmha_ms=ftf, fmha_fp16_same_lut_ms=ft16,
            fmha_speedup_vs_fp16=ft16 / ftf, pairs=int(f8["count"].sum().item()),
            fmha_tflops_computed=int(f8["count"].sum().item()) * F_BLK / ftf / 1e9)
        del q8, f8
    del hc, bm, o, l, ws
    return out


ARMS = ("0.1", "0.2", "0.4", "0.6", "0.8", "mixed")


def attainable(torch, achieved):
    """Ceilings measured live beside the FMHA, from libsparge_probe.so (the
    kernels of csrc/ceiling_probe.hip, three workgroups per CU like the
    FMHA): the fp16 MFMA rate on zero-mean operands held in registers, and
    the rate of a loop with the FMHA's per-wavefront volume per 64-key block
    (16 MFMAs, 16 KB of LDS reads feeding them, 8 KB of LDS writes, the
    softmax's VALU work) but none of its dependences, barriers or memory."""
    import ctypes
    from block_sparse_attention_sparge_amd import build as _build
    if not os.path.exists(_build.PROBE_LIB):
        raise RuntimeError(f"{_build.PROBE_LIB} not found: build it with "
                           "`python -m block_sparse_attention_sparge_amd.build`")
    lib = ctypes.CDLL(_build.PROBE_LIB)
    lib.sparge_probe_launch.restype = ctypes.c_int
    lib.sparge_probe_launch.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.sparge_probe_flops.restype = ctypes.c_double
    lib.sparge_probe_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    wg = 3 * torch.cuda.get_device_properties(0).multi_processor_count
    iters = 2000
    out = torch.empty(wg * 256, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    res = {}
    for kind, name in ((0, "mfma_only"), (1, "loop_volume")):
        def launch():
            rc = lib.sparge_probe_launch(kind, wg, iters, ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(stream))
            if rc != 0:
                raise RuntimeError(f"sparge_probe_launch({name}) failed: hip error {rc}")
        for _ in range(2):
            launch()
        ts = []
        for _ in range(7):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            launch()
            b.record()
            b.synchronize()
            ts.append(a.elapsed_time(b))
        res[f"{name}_tflops"] = round(lib.sparge_probe_flops(wg, iters) / (median(ts) * 1e-3) / 1e12, 1)
    if achieved is not None:
        res["frac_of_mfma_only"] = round(achieved / res["mfma_only_tflops"], 4)
        res["frac_of_loop_volume"] = round(achieved / res["loop_volume_tflops"], 4)
    res["probe"] = f"csrc/ceiling_probe.hip, {wg} workgroups x 4 wavefronts x {iters} iterations of 16 MFMAs"
    return res


def _topk_of(name):
    from block_sparse_attention_sparge_amd import synth
    return synth.mixed_topk(H) if name == "mixed" else [float(name)] * H


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-extras", action="store_true", help="skip the rows outside the headline")
    ap.add_argument("--ceilings-only", action="store_true",
                    help="run only the two throughput probes of roofline.attainable (for profiler runs)")
    ap.add_argument("--profile-arm", choices=ARMS + ("dense",), default=None,
                    help="run only warmup + steps headline steps of this arm (for profiler runs)")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this path has no multi-GPU mode (--gpus {args.gpus}).",
              file=sys.stderr)
        return 2
    if args.ceilings_only:
        import torch
        print(json.dumps({"attainable": attainable(torch, None)}), flush=True)
        return 0
    cpu = None
    if not args.no_cpu and args.profile_arm is None:
        # Before the GPU is touched: the workers are forked.
        log("cpu baseline: fp64 oracle over 32 (b, h) slices in a process pool")
        cpu = cpu_baseline(0.4)
    import torch
    from block_sparse_attention_sparge_amd import ops, synth

    torch.set_num_threads(min(16, os.cpu_count() or 1))
    ops.load_library()
    dev = torch.device("cuda:0")
    log(f"device {torch.cuda.get_device_name(dev)}; generating b{B} h{H} s{S} d{D} fp16")
    case = synth.headline_case(dev, topk=0.4)
    o = torch.empty_like(case.q)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    if args.profile_arm is not None:
        # Profiler mode: the only FMHA launches are the ones of this arm.
        if args.profile_arm == "dense":
            step = lambda i: ops.dense_fmha_fwd(case.q, case.k, case.v, o=o, lse=lse)
        else:
            tk, ws = _topk_of(args.profile_arm), {}

            def step(i):
                ws.update(ops.build_block_map(case.q, case.k, tk, case.simthreshd1, out=ws))
                ops.sparse_fmha_fwd(case.q, case.k, case.v, ws["lut"], ws["count"], o=o, lse=lse)
        ms, _ = timed_steps(step, args.steps, args.warmup, torch)
        log(f"profile arm {args.profile_arm}: {ms:.4f} ms per step")
        return 0

    # The timed region: exactly `steps` headline steps (block map + sparse
    # FMHA at topk 0.4) after `warmup` untimed ones, with HIP events around
    # each FMHA launch on the stream it runs on.
    log(f"headline: {args.warmup} warmup + {args.steps} timed steps at topk 0.4")
    ws = {}
    fm_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(args.steps)]

    def step(i):
        ws.update(ops.build_block_map(case.q, case.k, case.topk, case.simthreshd1, out=ws))
        if i is not None:
            fm_ev[i][0].record()
        ops.sparse_fmha_fwd(case.q, case.k, case.v, ws["lut"], ws["count"], o=o, lse=lse)
        if i is not None:
            fm_ev[i][1].record()

    step_ms, step_wall = timed_steps(step, args.steps, args.warmup, torch)
    fmha_ms = [a.elapsed_time(b) for a, b in fm_ev]
    fmha_mean = sum(fmha_ms) / len(fmha_ms)
    pairs = int(ws["count"].sum().item())
    del ws

    log("arms: topk 0.1 / 0.2 / 0.4 / 0.6 / 0.8 / mixed per head, and dense, interleaved")
    arms, dense_ms = step_arms(ops, case, {a: _topk_of(a) for a in ARMS}, args.steps, 2, torch)

    dense_flops = 4.0 * B * H * S * S * D
    value = dense_flops / (step_ms * 1e-3) / 1e12
    from block_sparse_attention_sparge_amd import profile_summary
    traffic = profile_summary.read_traffic(TRAFFIC_PROFILE, "topk 0.4")
    act = F_BLK * pairs / (fmha_mean * 1e-3) / 1e12
    res = {
        "metric": "sparse attn fwd ms + dense-equiv TFLOPS & speedup vs dense FMHA, s=16k topk 0.4/0.1",
        "value": round(value, 2),
        "unit": "TFLOP/s (dense-equivalent)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {"workload": "b2 h32 s16384 d128 fp16, blk 64x64, topk 0.4, simthreshd1 0.001, "
                               "block-centroid+noise Q/K", "global_batch": B, "seq_len": S,
                   "heads": H, "head_dim": D, "topk": 0.4, "parallelism": "single-gpu"},
        "roofline": {"bound": "mfma", "achieved": round(act, 1), "peak": PEAK_FP16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(act / PEAK_FP16_TFLOPS, 4),
                     "traffic": None if traffic is None else round(traffic),
                     "kernel": "fmha_block_kernel (sparse_fmha_fwd)",
                     "flops_per_launch": F_BLK * pairs, "pairs": pairs,
                     "avg_launch_ms": round(fmha_mean, 4),
                     "attainable": attainable(torch, act)},
        "step_wall_ms": round(step_wall, 4),
        "arms": {},
        "dense_fmha_ms": round(dense_ms, 4),
        "dense_fmha_tflops": round(dense_flops / (dense_ms * 1e-3) / 1e12, 1),
    }
    for name, a in arms.items():
        res["arms"][f"topk_{name}"] = {
            "step_ms": round(a["step_ms"], 4), "block_map_ms": round(a["block_map_ms"], 4),
            "fmha_ms": round(a["fmha_ms"], 4), "pairs": a["pairs"],
            "dense_equiv_tflops": round(dense_flops / (a["step_ms"] * 1e-3) / 1e12, 1),
            "actual_tflops_fmha": round(F_BLK * a["pairs"] / (a["fmha_ms"] * 1e-3) / 1e12, 1),
            "mfma_frac_fmha": round(F_BLK * a["pairs"] / (a["fmha_ms"] * 1e-3) / 1e12 / PEAK_FP16_TFLOPS, 4),
            "speedup_vs_dense_step": round(dense_ms / a["step_ms"], 3),
            "speedup_vs_dense_fmha": round(dense_ms / a["fmha_ms"], 3),
            "block_map_share": round(a["block_map_ms"] / a["step_ms"], 3),
            "block_map_gbs": round((2 * B * H * S * D * 2) / (a["block_map_ms"] * 1e-3) / 1e9, 1),
            "fmha_spread": round(a["fmha_spread"], 3),
        }
    if not args.no_extras:
        res["other_rows"] = extras(ops, synth, torch, args.steps, args.warmup)
    if cpu is not None:
        res["cpu_baseline"] = cpu
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
