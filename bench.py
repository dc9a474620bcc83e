"""Benchmark of the block-sparse attention forward on one MI355X.

Workload: b=2 h=32 s=16384 d=128 fp16, 64-token blocks, simthreshd1 0.001,
block-centroid + noise Q/K (centroid scale 0.5..2 over the heads, noise 0.5),
V ~ N(0, 1), seeded synthetic data resident in HBM before timing starts.

One step = the whole block-sparse forward: sparge_build_block_map (pool +
gate kernel, score + select kernel) then sparse_fmha_fwd over the LUT, at
topk 0.4 for every head.  `value` is the dense-equivalent throughput of a
step, 4*b*h*s*s*d / step time, in TFLOP/s.  The same line carries the topk 0.1
arm, the dense FMHA baseline (the same kernel with every block selected), the
other rows of the path (two-pass combine, decode), the roofline of the sparse
FMHA kernel, and the fp64 CPU oracle timed on a bounded sample.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-extras]
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


def time_arm(fn, steps, warmup, torch):
    """Run fn() warmup times, then time `steps` calls with HIP events on the
    current stream.  Returns (wall ms per call, list of per-call event ms)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    evs[0].record()
    for i in range(steps):
        fn()
        evs[i + 1].record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    per = [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]
    return wall, per


def time_cold(fn, steps, torch, flush):
    """Per-call HIP-event times of fn() with L2 and MALL flushed first: a
    512 MiB write precedes every call, outside the timed events."""
    per = []
    for _ in range(steps):
        flush.fill_(1)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        per.append(e0.elapsed_time(e1))
    return per


def median(x):
    s = sorted(x)
    n = len(s)
    return s[n // 2] if n % 2 else 0.5 * (s[n // 2 - 1] + s[n // 2])


def run_step_arm(ops, case, topk, steps, warmup, torch):
    """Time block map and sparse FMHA separately and as one step."""
    ws = {}
    bm = ops.build_block_map(case.q, case.k, [topk] * H, case.simthreshd1, out=ws)
    ws.update(bm)
    o = torch.empty_like(case.q)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=case.q.device)

    def block_map():
        ops.build_block_map(case.q, case.k, [topk] * H, case.simthreshd1, out=ws)

    def fmha():
        ops.sparse_fmha_fwd(case.q, case.k, case.v, ws["lut"], ws["count"], o=o, lse=lse)

    def step():
        block_map()
        fmha()

    _, bm_ms = time_arm(block_map, steps, warmup, torch)
    _, fm_ms = time_arm(fmha, steps, warmup, torch)
    wall, st_ms = time_arm(step, steps, warmup, torch)
    pairs = int(ws["count"].sum().item())     # selected (q tile, k block) pairs
    return dict(step_ms=median(st_ms), step_wall_ms=wall, block_map_ms=median(bm_ms),
                fmha_ms=median(fm_ms), fmha_ms_mean=sum(fm_ms) / len(fm_ms),
                fmha_spread=(max(fm_ms) - min(fm_ms)) / median(fm_ms), pairs=pairs)


def cpu_baseline(case, topk, heads=16):
    """The fp64 oracle on `heads` heads (b=0, h=0..heads-1) of the workload:
    block map + attention over the selected blocks."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = 1
    q = case.q[:1, :heads].double().cpu().numpy()
    k = case.k[:1, :heads].double().cpu().numpy()
    v = case.v[:1, :heads].double().cpu().numpy()
    t0 = time.perf_counter()
    bm = oracle.block_map(q, k, topk=[topk] * heads, simthreshd1=[0.001] * heads)
    oracle.block_sparse_attention(q, k, v, bm["lut"], bm["count"])
    dt = time.perf_counter() - t0
    dense_flops = 4.0 * heads * S * S * D
    return dict(value=dense_flops / dt / 1e12, unit="TFLOP/s (dense-equivalent)",
                cores=int(threads), kind="oracle",
                sample=f"{heads} heads (b=0, h=0..{heads - 1}) of b2 h32 s16384 d128 at topk {topk}: fp64 oracle "
                       f"block map + attention over the selected blocks, {dt:.1f} s",
                seconds=dt, host_cpus=os.cpu_count())


def extras(ops, synth, torch, steps, warmup):
    out = {}
    dev = torch.device("cuda:0")
    # Two-pass combine, b1 h16 s_q1024 s_k32768 d128 bf16.
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

    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    _, tp = time_arm(two_pass, steps, warmup, torch)
    _, cm = time_arm(comb, steps, warmup, torch)
    tp_cold = time_cold(two_pass, steps, torch, flush)
    cm_cold = time_cold(comb, steps, torch, flush)
    comb_bytes = parts.numel() * 4 + lses.numel() * 4 + oc.numel() * 2 + lc.numel() * 4
    out["two_pass_combine"] = dict(workload="b1 h16 s_q1024 s_k32768 d128 bf16", ms=median(tp),
                                   combine_ms=median(cm), combine_gbs=comb_bytes / median(cm) / 1e6,
                                   cold_ms=median(tp_cold), cold_combine_ms=median(cm_cold),
                                   cold_combine_gbs=comb_bytes / median(cm_cold) / 1e6)
    del c, oa, ob, parts, lses, oc, lc
    # Combine on headline-shaped fp32 partials: 2 x [2, 32, 16384, 128].
    parts = torch.randn(2, B, H, S, D, device=dev)
    lses = torch.randn(2, B, H, S, device=dev)
    oc = torch.empty((B, H, S, D), dtype=torch.float16, device=dev)
    lc = torch.empty((B, H, S), device=dev)
    _, cm = time_arm(lambda: ops.attn_combine(parts, lses, o=oc, lse=lc), steps, warmup, torch)
    comb_bytes = parts.numel() * 4 + lses.numel() * 4 + oc.numel() * 2 + lc.numel() * 4
    out["combine_headline_partials"] = dict(workload="2 x [2,32,16384,128] fp32 -> fp16",
                                            ms=median(cm), gbs=comb_bytes / median(cm) / 1e6,
                                            frac_hbm=comb_bytes / median(cm) / 1e6 / PEAK_HBM_GBS)
    del parts, lses, oc, lc
    # Decode GQA, b64 h_q32 h_kv8 s_k32768 d128 bf16, 2048-entry lists, 8 splits + combine.
    dc = synth.decode_case(dev)
    S_SPLIT = 8
    op = torch.empty((S_SPLIT, 64, 32, 1, 128), device=dev)
    lp = torch.empty((S_SPLIT, 64, 32, 1), device=dev)
    od = torch.empty_like(dc.q)
    ld = torch.empty((64, 32, 1), device=dev)

    def decode():
        ops.sparse_fmha_fwd(dc.q, dc.k, dc.v, dc.lists, None, blk_q=1, blk_k=1,
                            num_splits=S_SPLIT, o=op, lse=lp, out_dtype=torch.float32)
        ops.attn_combine(op, lp, o=od, lse=ld)

    _, dm = time_arm(decode, steps, warmup, torch)
    dm_cold = time_cold(decode, steps, torch, flush)
    gathered = 64 * 8 * 2048 * 128 * 2 * 2
    out["decode_gqa"] = dict(workload="b64 h_q32 h_kv8 s_k32768 d128 bf16, 2048 listed keys, 8 splits",
                             ms=median(dm), gathered_gbs=gathered / median(dm) / 1e6,
                             frac_hbm=gathered / median(dm) / 1e6 / PEAK_HBM_GBS,
                             cold_ms=median(dm_cold), cold_gathered_gbs=gathered / median(dm_cold) / 1e6,
                             cold_frac_hbm=gathered / median(dm_cold) / 1e6 / PEAK_HBM_GBS)
    del flush
    # Causal prefill at the headline shape (b2 h32 s16384 d128 fp16, topk 0.4):
    # block map with K smoothing, the causal block mask and the attention sink,
    # then the causal sparse FMHA; the causal dense FMHA is the baseline.
    hc = synth.headline_case(dev, topk=0.4)
    ws = {}

    def causal_map():
        return ops.build_block_map(hc.q, hc.k, hc.topk, hc.simthreshd1, out=ws, smooth_k=True,
                                   causal=True, attention_sink=True)

    bm = causal_map()
    ws.update(bm)                 # later calls reuse these outputs
    o = torch.empty_like(hc.q)
    l = torch.empty((B, H, S), device=dev)
    _, bmt = time_arm(causal_map, steps, warmup, torch)
    _, ft = time_arm(lambda: ops.sparse_fmha_fwd(hc.q, hc.k, hc.v, bm["lut"], bm["count"], o=o, lse=l,
                                                 causal=True), steps, warmup, torch)
    _, dt = time_arm(lambda: ops.sparse_fmha_fwd(hc.q, hc.k, hc.v, None, None, o=o, lse=l, causal=True),
                     max(3, steps // 4), 1, torch)
    pairs = int(bm["count"].sum().item())
    dense_pairs = B * H * (S // 64) * (S // 64 + 1) // 2
    out["causal_headline"] = dict(
        workload="b2 h32 s16384 d128 fp16, topk 0.4, smooth_k + causal + attention_sink",
        block_map_ms=median(bmt), fmha_ms=median(ft), pairs=pairs,
        fmha_tflops_computed=pairs * F_BLK / median(ft) / 1e9,
        dense_causal_ms=median(dt), dense_causal_pairs=dense_pairs,
        dense_causal_tflops_computed=dense_pairs * F_BLK / median(dt) / 1e9,
        speedup_vs_dense_step=median(dt) / (median(bmt) + median(ft)))
    # pv_threshold at the headline shape (plain block map, topk 0.4): the same
    # FMHA with no skip and with thresholds of 4 and 8 nats.
    bm = ops.build_block_map(hc.q, hc.k, hc.topk, hc.simthreshd1, out=ws)
    pv = {}
    for tau in (0.0, 4.0, 8.0):
        _, t = time_arm(lambda: ops.sparse_fmha_fwd(hc.q, hc.k, hc.v, bm["lut"], bm["count"], o=o, lse=l,
                                                    pv_threshold=tau), steps, warmup, torch)
        pv[tau] = median(t)
    out["pv_skip_headline"] = dict(
        workload="b2 h32 s16384 d128 fp16, topk 0.4, pv_threshold 0 / 4 / 8",
        fmha_ms_no_skip=pv[0.0], fmha_ms_tau4=pv[4.0], fmha_ms_tau8=pv[8.0],
        speedup_tau4=pv[0.0] / pv[4.0], speedup_tau8=pv[0.0] / pv[8.0])
    # A ragged length at the headline shape: s = 16347 (255 full blocks and
    # one of 27 tokens), the same tensors viewed shorter.  The block map pools
    # the partial block; the FMHA runs its masked kernel for it.
    SR = 16347
    qr, kr, vr = hc.q[:, :, :SR], hc.k[:, :, :SR], hc.v[:, :, :SR]
    bmr = ops.build_block_map(qr, kr, hc.topk, hc.simthreshd1)
    orr = torch.empty((B, H, SR, qr.shape[3]), dtype=qr.dtype, device=dev)
    lr = torch.empty((B, H, SR), device=dev)
    _, bmt = time_arm(lambda: ops.build_block_map(qr, kr, hc.topk, hc.simthreshd1, out=bmr), steps, warmup,
                      torch)
    _, ft = time_arm(lambda: ops.sparse_fmha_fwd(qr, kr, vr, bmr["lut"], bmr["count"], o=orr, lse=lr),
                     steps, warmup, torch)
    pairs = int(bmr["count"].sum().item())
    out["ragged_headline"] = dict(
        workload="b2 h32 s16347 d128 fp16 (last block 27 tokens), topk 0.4",
        block_map_ms=median(bmt), fmha_ms=median(ft), pairs=pairs,
        fmha_tflops_computed=pairs * F_BLK / median(ft) / 1e9)
    del bmr, orr, lr
    # The same shape in bf16 (topk 0.4): block map and sparse FMHA.
    hb = synth.headline_case(dev, topk=0.4, dtype=torch.bfloat16)
    bmb = ops.build_block_map(hb.q, hb.k, hb.topk, hb.simthreshd1)
    ob = torch.empty_like(hb.q)
    _, bmt = time_arm(lambda: ops.build_block_map(hb.q, hb.k, hb.topk, hb.simthreshd1, out=bmb), steps, warmup,
                      torch)
    _, ft = time_arm(lambda: ops.sparse_fmha_fwd(hb.q, hb.k, hb.v, bmb["lut"], bmb["count"], o=ob, lse=l),
                     steps, warmup, torch)
    pairs = int(bmb["count"].sum().item())
    out["bf16_headline_topk_0.4"] = dict(
        workload="b2 h32 s16384 d128 bf16, topk 0.4", block_map_ms=median(bmt), fmha_ms=median(ft),
        pairs=pairs, fmha_tflops_computed=pairs * F_BLK / median(ft) / 1e9,
        mfma_frac_fmha=pairs * F_BLK / median(ft) / 1e9 / PEAK_FP16_TFLOPS)
    del hb, bmb, ob
    # int8 Q/K at the headline shape: the block map with the fused per-block
    # quantisation, then the int8-QK sparse FMHA (V and P stay fp16).
    for topk in (0.4, 0.1):
        tk = [topk] * H
        q8 = ops.build_block_map(hc.q, hc.k, tk, hc.simthreshd1, quantize_int8=True)

        def map8():
            ops.build_block_map(hc.q, hc.k, tk, hc.simthreshd1, out=q8, quantize_int8=True)

        def fmha8():
            ops.sparse_fmha_fwd_qk_int8(q8["q_i8"], q8["q_i8_scale"], q8["k_i8"], q8["k_i8_scale"], hc.v,
                                        q8["lut"], q8["count"], o=o, lse=l)

        _, bmt = time_arm(map8, steps, warmup, torch)
        _, ft = time_arm(fmha8, steps, warmup, torch)
        _, ft16 = time_arm(lambda: ops.sparse_fmha_fwd(hc.q, hc.k, hc.v, q8["lut"], q8["count"], o=o, lse=l),
                           steps, warmup, torch)
        pairs = int(q8["count"].sum().item())
        out[f"qk_int8_topk_{topk}"] = dict(
            workload=f"b2 h32 s16384 d128, int8 Q/K codes per 64-token block, fp16 V, topk {topk}",
            block_map_ms=median(bmt), fmha_ms=median(ft), fmha_fp16_same_lut_ms=median(ft16),
            fmha_speedup_vs_fp16=median(ft16) / median(ft), pairs=pairs,
            fmha_tflops_computed=pairs * F_BLK / median(ft) / 1e9)
        del q8
    del hc, bm, o, l, ws
    return out


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-extras", action="store_true", help="skip combine / decode rows")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this path has no multi-GPU mode (--gpus {args.gpus}).",
              file=sys.stderr)
        return 2
    import torch
    from block_sparse_attention_sparge_amd import ops, synth

    ops.load_library()
    dev = torch.device("cuda:0")
    log(f"device {torch.cuda.get_device_name(dev)}; generating b{B} h{H} s{S} d{D} fp16")
    case = synth.headline_case(dev, topk=0.4)
    torch.cuda.synchronize()

    dense_flops = 4.0 * B * H * S * S * D
    f_blk = 4.0 * 64 * 64 * D
    arms = {}
    for tk in (0.4, 0.1):
        log(f"arm topk {tk}")
        arms[tk] = run_step_arm(ops, case, tk, args.steps, args.warmup, torch)
    log("arm dense")
    o = torch.empty_like(case.q)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=dev)
    _, dn = time_arm(lambda: ops.dense_fmha_fwd(case.q, case.k, case.v, o=o, lse=lse),
                     max(5, args.steps // 2), 2, torch)
    dense_ms = median(dn)

    main_arm = arms[0.4]
    value = dense_flops / (main_arm["step_ms"] * 1e-3) / 1e12
    from block_sparse_attention_sparge_amd import profile_summary
    traffic = profile_summary.read_traffic(TRAFFIC_PROFILE, "topk 0.4")
    act = f_blk * main_arm["pairs"] / (main_arm["fmha_ms_mean"] * 1e-3) / 1e12
    res = {
        "metric": "sparse attn fwd ms + dense-equiv TFLOPS & speedup vs dense FMHA, s=16k topk 0.4/0.1",
        "value": round(value, 2),
        "unit": "TFLOP/s (dense-equivalent)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_arm["step_ms"], 4),
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
                     "flops_per_launch": f_blk * main_arm["pairs"],
                     "avg_launch_ms": round(main_arm["fmha_ms_mean"], 4)},
        "arms": {},
        "dense_fmha_ms": round(dense_ms, 4),
        "dense_fmha_tflops": round(dense_flops / (dense_ms * 1e-3) / 1e12, 1),
    }
    for tk, a in arms.items():
        res["arms"][f"topk_{tk}"] = {
            "step_ms": round(a["step_ms"], 4), "block_map_ms": round(a["block_map_ms"], 4),
            "fmha_ms": round(a["fmha_ms"], 4), "pairs": a["pairs"],
            "dense_equiv_tflops": round(dense_flops / (a["step_ms"] * 1e-3) / 1e12, 1),
            "actual_tflops_fmha": round(f_blk * a["pairs"] / (a["fmha_ms"] * 1e-3) / 1e12, 1),
            "mfma_frac_fmha": round(f_blk * a["pairs"] / (a["fmha_ms"] * 1e-3) / 1e12 / PEAK_FP16_TFLOPS, 4),
            "speedup_vs_dense_step": round(dense_ms / a["step_ms"], 3),
            "speedup_vs_dense_fmha": round(dense_ms / a["fmha_ms"], 3),
            "block_map_share": round(a["block_map_ms"] / a["step_ms"], 3),
            "block_map_gbs": round((2 * B * H * S * D * 2) / (a["block_map_ms"] * 1e-3) / 1e9, 1),
            "fmha_spread": round(a["fmha_spread"], 3),
        }
    if not args.no_extras:
        log("extras: two-pass combine, combine at headline size, decode")
        res["other_rows"] = extras(ops, synth, torch, args.steps, args.warmup)
    if not args.no_cpu:
        log("cpu baseline (oracle, 16 heads)")
        res["cpu_baseline"] = cpu_baseline(case, 0.4)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
