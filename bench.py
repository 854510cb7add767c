#!/usr/bin/env python3
"""Throughput of the routed-expert MoE FFN path on one MI355X.

Default workload: the Phi-3.5-MoE-shaped layer (hidden 4096, 16 experts,
top-2, SwiGLU intermediate 6400, no shared expert).  One step is one INT4
draft decode step (T = 1: routing + ELB count + gather folded into the gate/up
launch, the down projection, combine -- or with --draft split the fused
routing plan, the W4A16 FFN and combine; launched call by call, or replayed
as a captured HIP graph with --graph on) followed by one
FP16 verification of K+1 = 17 tokens (route, gather,
regrouped verify FFN, combine), every step through the C ABI of libsmoe.so
on seeded synthetic inputs already resident in HBM.  Steps cycle over a pool
of 8 seeded token batches.

Printed JSON line (rank 0):
  value       draft INT4 weight GB/s: INT4 bytes (packed codes + fp16 scales
              + packed zeros) of the experts each draft step touches, over
              the wall time of the draft half of the step (HIP events around
              all of its calls)
  verify      the verify half: TFLOP/s (2 x rows x 3 H I), % of FP16 MFMA
              peak, and its FP16 weight GB/s
  roofline    the dominant kernel of the step (verify_grouped_gemm, HBM
              bound): touched FP16 weight bytes per call / average call time
  roofline_draft  the same for w4a16_grouped_ffn (INT4 bytes)
  ds_draft, qwen_verify, qwen_chunk  the other configurations' layers: the
              DeepSeek-V2-Lite draft step at T = 1/4/16, the Qwen1.5-MoE
              verify layer at K+1 = 9, the 24-layer Qwen chunk (16 draft steps,
              ELB snapshot, placement, staged verify)
  cpu_baseline    the CPU oracle on a bounded sample of draft steps
"""
from __future__ import annotations

import argparse
import gc
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
MFMA_F16_PEAK_TFS = 2516.6   # dense FP16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk
POOL = 8                     # distinct seeded batches
STREAM_BLOCKS = 2048         # workgroups of the streaming-read ceiling (best of 1024/2048/4096)


def idx_all(args, K):
    """Pool indexes of the K timed steps."""
    return [(args.warmup + st) % POOL for st in range(K)]


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-sample", type=int, default=30,
                    help="draft steps of the oracle timed for cpu_baseline (0 = skip)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a 1 GiB device copy (counter calibration for rocprofv3 --pmc)")
    ap.add_argument("--workload", default="phi_layer",
                    choices=["phi_layer", "qwen_chunk", "route_fidelity", "qwen_rounds",
                             "draft_formats", "ds_draft", "qwen_verify"],
                    help="phi_layer (default): one draft + verify step of the Phi-3.5-MoE-shaped "
                         "layer; qwen_chunk: 24 Qwen-shaped layers, 16 draft steps, ELB snapshot, "
                         "top-16 residency, 17-token verify with staged misses; route_fidelity: INT4 draft vs "
                         "FP16 target routing agreement and distinct experts vs depth; qwen_rounds: speculation "
                         "rounds with the prefetch planner vs boundary placement; draft_formats: the "
                         "one-token draft step with 2-, 4- and 8-bit experts (Phi and DeepSeek shapes); "
                         "ds_draft: the DeepSeek-V2-Lite-shaped draft layer step (routing, ELB, INT4 "
                         "experts, 2 FP16 shared experts, combine) at T = 1, 4 and 16; qwen_verify: "
                         "the Qwen1.5-MoE-shaped verify layer at K+1 = 9 (routed and shared expert)")
    ap.add_argument("--layers", type=int, default=24, help="qwen_chunk: number of layers")
    ap.add_argument("--rounds", type=int, default=4, help="qwen_rounds: speculation rounds")
    ap.add_argument("--rho", type=float, default=0.8,
                    help="qwen_rounds: lag-one correlation of the token stream (0.8 gives about "
                         "7x distinct experts from depth 1 to 16 on these layers)")
    ap.add_argument("--no-dense-point", dest="dense_point", action="store_false",
                    help="phi_layer: skip the supplementary T=2048 verify point")
    ap.add_argument("--no-context", dest="context", action="store_false",
                    help="qwen_verify: skip the context pass that times the routed and the "
                         "shared expert as separate calls (a clean kernel trace of the step)")
    ap.add_argument("--no-other-configs", dest="other_configs", action="store_false",
                    help="phi_layer: skip the DeepSeek-V2-Lite draft (T=1/4/16) and Qwen1.5-MoE "
                         "verify (T=9) sub-objects of the line")
    ap.add_argument("--draft", choices=["fused", "split"], default="fused",
                    help="phi_layer draft step: moe_draft_route_ffn + moe_combine (fused: routing "
                         "folded into the gate/up launch, 3 launches) or moe_route_plan + "
                         "w4a16_grouped_ffn + moe_combine (split, 4 launches)")
    ap.add_argument("--graph", choices=["on", "off"], default="off",
                    help="replay the draft step as a captured HIP graph (on) or launch its calls "
                         "one by one (off, the default: measured faster on this platform for "
                         "the Phi layer step and the 24-layer Qwen chunk alike)")
    return ap.parse_args()


def main():
    args = parse()
    args.no_graph = args.graph == "off"
    if args.gpus != 1:
        print(f"bench.py: measures one GPU only (asked for --gpus {args.gpus}); the path is "
              "single-GPU and no multi-GPU figure is produced.", file=sys.stderr)
        sys.exit(2)
    # no cyclic-garbage pass inside a timed region (a host pause there leaves
    # the GPU idle between a step's events); the run is short-lived
    gc.collect()
    gc.disable()
    if args.workload == "qwen_chunk":
        return bench_qwen_chunk(args)
    if args.workload == "route_fidelity":
        return bench_route_fidelity(args)
    if args.workload == "qwen_rounds":
        return bench_qwen_rounds(args)
    if args.workload == "draft_formats":
        return bench_draft_formats(args)
    if args.workload == "ds_draft":
        return bench_ds_draft(args)
    if args.workload == "qwen_verify":
        return bench_qwen_verify(args)

    import numpy as np
    import torch

    import fp16_verify_expert_amd as fve
    import synth

    fve.lib()
    torch.cuda.set_device(0)
    dev = torch.device("cuda")
    s = synth.PHI
    T_D, T_V = 1, 17
    H, I, E, k = s.H, s.I, s.E, s.k

    # ---- weights: all experts resident (INT4 draft + FP16 target) ----
    t0 = time.perf_counter()
    layer = synth.make_layer(s)
    gen_s = time.perf_counter() - t0
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    w4 = [{key: tuple(up(t) for t in ex[key]) for key in ("w13", "w2")} for ex in layer["int4"]]
    w16 = [(up(a), up(b)) for a, b in layer["f16"]]
    t4 = fve.w4_expert_table(w4)
    t16 = fve.f16_expert_table(w16)
    router = up(layer["router"])
    xs_d = [up(synth.tokens(s, T_D, step=i)) for i in range(POOL)]
    xs_v = [up(synth.tokens(s, T_V, step=100 + i)) for i in range(POOL)]

    # ---- preallocated buffers (no allocation inside the timed loop) ----
    def bufs(T):
        n = T * k
        return dict(ids=torch.empty((T, k), dtype=torch.int32, device=dev),
                    w=torch.empty((T, k), dtype=torch.float32, device=dev),
                    maps=dict(offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
                              sorted_token=torch.empty(n, dtype=torch.int32, device=dev),
                              sorted_pair=torch.empty(n, dtype=torch.int32, device=dev),
                              pair_pos=torch.empty(n, dtype=torch.int32, device=dev),
                              active=torch.empty(E, dtype=torch.int32, device=dev),
                              n_active=torch.empty(1, dtype=torch.int32, device=dev)),
                    y=torch.empty((n, H), dtype=torch.float16, device=dev),
                    out=torch.empty((T, H), dtype=torch.float16, device=dev),
                    lg=torch.empty(T * (E + 1), dtype=torch.float32, device=dev))
    bd, bv = bufs(T_D), bufs(T_V)
    ws_d = fve.new_workspace(0, T_D, k, H, I, E)
    ws_v = fve.new_workspace(1, T_V, k, H, I, E)
    counters = torch.zeros((1, E), dtype=torch.int32, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)

    def draft_split(i, ev=None):
        x = xs_d[i % POOL]
        fve.moe_route_plan(x, router, k, counters=counters, layer=0, err_word=err,
                           topk_ids=bd["ids"], topk_w=bd["w"], maps=bd["maps"],
                           logits_ws=bd["lg"])
        if ev: ev[0].record()
        fve.w4a16_grouped_ffn(x, bd["maps"], t4, T_D, k, H, I, E, ws_d, y_sorted=bd["y"],
                              err_word=err)
        if ev: ev[1].record()
        fve.moe_combine(bd["y"], bd["maps"]["pair_pos"], bd["w"], out=bd["out"])

    def draft_fused(i, ev=None):
        x = xs_d[i % POOL]
        if ev: ev[0].record()
        fve.moe_draft_route_ffn(x, router, k, t4, I, ws_d, counters=counters, layer=0,
                                err_word=err, topk_ids=bd["ids"], topk_w=bd["w"],
                                maps=bd["maps"], y_sorted=bd["y"])
        if ev: ev[1].record()
        fve.moe_combine(bd["y"], bd["maps"]["pair_pos"], bd["w"], out=bd["out"])

    draft = draft_fused if args.draft == "fused" else draft_split

    def verify(i, ev=None):
        x = xs_v[i % POOL]
        # routing and maps in one plan (no ELB update for verification)
        fve.moe_route_plan(x, router, k, err_word=err, topk_ids=bv["ids"], topk_w=bv["w"],
                           maps=bv["maps"], logits_ws=bv["lg"])
        if ev: ev[0].record()
        fve.verify_grouped_gemm(x, bv["maps"]["sorted_token"], bv["maps"]["offsets"], t16, T_V,
                                T_V * k, H, I, E, ws_v, active=bv["maps"]["active"],
                                n_active=bv["maps"]["n_active"], y_sorted=bv["y"], err_word=err)
        if ev: ev[1].record()
        fve.moe_combine(bv["y"], bv["maps"]["pair_pos"], bv["w"], out=bv["out"])

    # ---- per-batch algorithmic work (routing is deterministic); the two
    #      draft paths must agree bit for bit ----
    touched_d, touched_v = [], []
    for i in range(POOL):
        draft_split(i)
        torch.cuda.synchronize()
        ref_out = bd["out"].clone()
        draft(i)
        verify(i)
        torch.cuda.synchronize()
        assert torch.equal(bd["out"], ref_out), "fused and split draft steps differ"
        touched_d.append(int(bd["maps"]["n_active"].item()))
        touched_v.append(int(bv["maps"]["n_active"].item()))
    assert int(err.item()) == 0, "device error word set"
    b4 = s.int4_bytes_per_expert
    b16 = s.f16_bytes_per_expert
    flop_v = lambda i: 2.0 * T_V * k * 3 * H * I

    for i in range(args.warmup):
        draft(i)
        verify(i)
    torch.cuda.synchronize()

    # ---- the draft step as one HIP graph per pooled input (launch-free) ----
    graphs = None
    if not args.no_graph:
        graphs = []
        for i in range(POOL):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                draft(i)
            graphs.append(g)
        torch.cuda.synchronize()
        # replays must reproduce the eager outputs (checked on the pool)
        for i in range(POOL):
            draft(i)
            torch.cuda.synchronize()
            ref = bd["out"].clone()
            graphs[i].replay()
            torch.cuda.synchronize()
            assert torch.equal(bd["out"], ref), "draft graph replay differs from eager"

    # ---- timed region ----
    K = args.steps
    mk = lambda: torch.cuda.Event(enable_timing=True)
    ph = [(mk(), mk(), mk()) for _ in range(K)]            # draft start / verify start / end
    kd = [(mk(), mk()) for _ in range(K)]                  # fused call (pass after the loop)
    kv = [(mk(), mk()) for _ in range(K)]                  # verify call
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for st in range(K):
        i = args.warmup + st
        ph[st][0].record()
        if graphs is not None:
            graphs[i % POOL].replay()
        else:
            draft(i)
        ph[st][1].record()
        verify(i, kv[st])
        ph[st][2].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    assert int(err.item()) == 0, "device error word set"
    # the draft entry points' own durations, from eager passes after the timed
    # loop with events around each call (kept out of the timed draft half, so
    # that its wall time holds no event markers; the fused call also holds the
    # routing)
    kw = [(mk(), mk()) for _ in range(K)]
    for st in range(K):
        draft_split(args.warmup + st, kw[st])
        verify(args.warmup + st)
    torch.cuda.synchronize()
    if args.draft == "fused":
        for st in range(K):
            draft_fused(args.warmup + st, kd[st])
            verify(args.warmup + st)
        torch.cuda.synchronize()

    # every call of the split draft step and of the verify step on its own,
    # and the ELB update (HIP events around each; launch gaps excluded)
    nl = min(K, 20)
    calls = {n: [(mk(), mk()) for _ in range(nl)] for n in
             ("moe_route_plan", "w4a16_grouped_ffn", "moe_combine_draft", "moe_route_topk",
              "elb_count", "moe_gather", "verify_grouped_gemm", "moe_combine_verify")}
    # a first pass is not timed: the standalone routing, ELB and gather entry
    # points are not part of the timed steps, so their first launches land here
    warm = {n: (mk(), mk()) for n in calls}
    for st in range(nl + 1):
        i = args.warmup + st
        x = xs_d[i % POOL]
        ev = lambda n: warm[n] if st == 0 else calls[n][st - 1]
        ev("moe_route_plan")[0].record()
        fve.moe_route_plan(x, router, k, counters=counters, layer=0, err_word=err,
                           topk_ids=bd["ids"], topk_w=bd["w"], maps=bd["maps"],
                           logits_ws=bd["lg"])
        ev("moe_route_plan")[1].record()
        ev("w4a16_grouped_ffn")[0].record()
        fve.w4a16_grouped_ffn(x, bd["maps"], t4, T_D, k, H, I, E, ws_d, y_sorted=bd["y"],
                              err_word=err)
        ev("w4a16_grouped_ffn")[1].record()
        ev("moe_combine_draft")[0].record()
        fve.moe_combine(bd["y"], bd["maps"]["pair_pos"], bd["w"], out=bd["out"])
        ev("moe_combine_draft")[1].record()
        xv = xs_v[i % POOL]
        ev("moe_route_topk")[0].record()
        fve.moe_route_topk(xv, router, k, topk_ids=bv["ids"], topk_w=bv["w"])
        ev("moe_route_topk")[1].record()
        # the ELB update of the same ids on its own (the draft steps fold it
        # into their routing launch)
        ev("elb_count")[0].record()
        fve.elb_count(bv["ids"], E, 0, counters, err)
        ev("elb_count")[1].record()
        ev("moe_gather")[0].record()
        fve.moe_gather(bv["ids"], E, err, out=bv["maps"])
        ev("moe_gather")[1].record()
        ev("verify_grouped_gemm")[0].record()
        fve.verify_grouped_gemm(xv, bv["maps"]["sorted_token"], bv["maps"]["offsets"], t16,
                                T_V, T_V * k, H, I, E, ws_v, active=bv["maps"]["active"],
                                n_active=bv["maps"]["n_active"], y_sorted=bv["y"],
                                err_word=err)
        ev("verify_grouped_gemm")[1].record()
        ev("moe_combine_verify")[0].record()
        fve.moe_combine(bv["y"], bv["maps"]["pair_pos"], bv["w"], out=bv["out"])
        ev("moe_combine_verify")[1].record()
    torch.cuda.synchronize()
    call_us = {n: round(1e3 * sum(a.elapsed_time(b) for a, b in v) / nl, 2)
               for n, v in calls.items()}

    # ---- attainable ceiling of the draft FFN: streaming reads of the same
    #      gate/up and down byte counts (the touched experts' INT4 bytes of
    #      each projection) in two dependent launches, HIP events around
    #      both, each preceded by a verify step as in the per-call pass ----
    def int4_bytes(Kd, N):
        return Kd * N // 2 + (Kd // 128) * N * 2 + (Kd // 128) * (N // 8) * 4
    nt = sum(touched_d[i] for i in idx_all(args, K)) / K
    gu_b = int(round(nt * int4_bytes(H, 2 * I))) // 16 * 16
    dn_b = int(round(nt * int4_bytes(I, H))) // 16 * 16
    src_gu = torch.empty(gu_b // 2, dtype=torch.float16, device=dev)
    src_dn = torch.empty(dn_b // 2, dtype=torch.float16, device=dev)
    sink = torch.zeros(STREAM_BLOCKS, dtype=torch.int32, device=dev)
    ev_st = [(mk(), mk()) for _ in range(nl)]
    for st in range(nl + 1):
        verify(args.warmup + st)
        if st:
            ev_st[st - 1][0].record()
        fve.smoe_stream_read(src_gu, sink, STREAM_BLOCKS)
        fve.smoe_stream_read(src_dn, sink, STREAM_BLOCKS)
        if st:
            ev_st[st - 1][1].record()
    torch.cuda.synchronize()
    stream_us = 1e3 * sum(a.elapsed_time(b) for a, b in ev_st) / nl
    del src_gu, src_dn

    # ---- the layer's draft step as one launch (moe_draft_layer: routing,
    #      INT4 FFN and combine, logits computed inside) against the split
    #      step on the same batches, HIP events around each, each after a
    #      verify step; outputs bit-identical ----
    single = None
    if fve.draft_layer_supported(H, I, E, k):
        wsl = fve.new_layer_workspace(k, H, I, E)
        out1 = torch.empty((1, H), dtype=torch.float16, device=dev)
        ev_sl = [(mk(), mk()) for _ in range(nl)]
        ev_sp = [(mk(), mk()) for _ in range(nl)]
        for st in range(nl + 1):
            i = args.warmup + st
            verify(i)
            if st:
                ev_sp[st - 1][0].record()
            draft_fused(i)
            if st:
                ev_sp[st - 1][1].record()
            verify(i)
            if st:
                ev_sl[st - 1][0].record()
            fve.moe_draft_layer(xs_d[i % POOL], router, k, t4, I, wsl, err_word=err, out=out1)
            if st:
                ev_sl[st - 1][1].record()
            torch.cuda.synchronize()
            assert torch.equal(out1, bd["out"]), "one-launch layer differs from the split step"
        assert int(err.item()) == 0, "device error word set"
        single = {"what": "moe_draft_layer (one launch: logits, routing, ELB, INT4 FFN, combine) "
                          "vs moe_draft_route_ffn + moe_combine, HIP events around each, after "
                          "a verify step; bit-identical outputs",
                  "one_launch_us": round(1e3 * sum(a.elapsed_time(b) for a, b in ev_sl) / nl, 2),
                  "split_us": round(1e3 * sum(a.elapsed_time(b) for a, b in ev_sp) / nl, 2)}
        del wsl

    idx = idx_all(args, K)
    draft_ms = sum(ph[st][0].elapsed_time(ph[st][1]) for st in range(K))
    verify_ms = sum(ph[st][1].elapsed_time(ph[st][2]) for st in range(K))
    w4_ms = [kw[st][0].elapsed_time(kw[st][1]) for st in range(K)]
    fused_ms = ([kd[st][0].elapsed_time(kd[st][1]) for st in range(K)]
                if args.draft == "fused" else None)
    vg_ms = [kv[st][0].elapsed_time(kv[st][1]) for st in range(K)]
    bytes_d = sum(touched_d[i] * b4 for i in idx)
    bytes_v = sum(touched_v[i] * b16 for i in idx)
    flops_v = sum(flop_v(i) for i in idx)
    step_ms = (draft_ms + verify_ms) / K

    value = bytes_d / (draft_ms * 1e-3) / 1e9
    # attainable verify roofline: min(MFMA peak, arithmetic intensity x HBM peak)
    v_attain = min(MFMA_F16_PEAK_TFS, flops_v / bytes_v * HBM_PEAK_GBS / 1e3)
    v_tfs = flops_v / (verify_ms * 1e-3) / 1e12
    v_gbs = bytes_v / (verify_ms * 1e-3) / 1e9
    rv_ach = bytes_v / (sum(vg_ms) * 1e-3) / 1e9
    rd_ach = bytes_d / (sum(w4_ms) * 1e-3) / 1e9
    prof_dir = os.path.join(ROOT, "profiles")

    def pmc_traffic(name):
        """HBM bytes per call from the committed rocprofv3 --pmc summary
        (FETCH_SIZE + WRITE_SIZE, scaled by a 1 GiB copy), or None when the
        kernel sources changed since the counters were taken."""
        import hashlib
        p = os.path.join(prof_dir, "pmc_traffic.json")
        if not os.path.exists(p):
            return None
        with open(p) as f:
            d = json.load(f)
        for src, h in d.get("sources_sha256", {}).items():
            path = os.path.join(ROOT, "fp16_verify_expert_amd", "csrc", src)
            with open(path, "rb") as f:
                if hashlib.sha256(f.read()).hexdigest()[:16] != h:
                    return None
        v = d.get(name)
        return None if v is None else round(float(v))

    res = {
        "metric": "MoE-layer INT4 draft weight GB/s (% HBM peak); verify TFLOP/s (% MFMA)",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4-w/fp16-a (draft), fp16 (verify); fp32 accumulate",
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1) tokens; RTN GPTQ INT4 g128 draft)",
        "config": {"workload": "phi35_moe_layer: H=4096 E=16 top-2 I=6400; draft T=1 INT4 + "
                               "verify K+1=17 FP16; all experts HBM-resident",
                   "draft_tokens": T_D, "verify_tokens": T_V, "batch_pool": POOL},
        "draft": {"ms": round(draft_ms / K, 4), "gbps": round(value, 2),
                  "launch": "hip_graph" if graphs is not None else "eager",
                  "path": ("moe_draft_route_ffn + moe_combine" if args.draft == "fused" else
                           "moe_route_plan + w4a16_grouped_ffn + moe_combine"),
                  "fused_call_us": (None if fused_ms is None else
                                    round(1e3 * sum(fused_ms) / K, 3)),
                  "frac_hbm": round(value / HBM_PEAK_GBS, 4),
                  "touched_experts_avg": round(sum(touched_d[i] for i in idx) / K, 3),
                  "int4_bytes_avg": round(bytes_d / K)},
        "verify": {"ms": round(verify_ms / K, 4), "tflops": round(v_tfs, 3),
                   "frac_mfma": round(v_tfs / MFMA_F16_PEAK_TFS, 5), "gbps": round(v_gbs, 2),
                   "attainable_tflops": round(v_attain, 2),
                   "frac_attainable": round(v_tfs / v_attain, 4),
                   "frac_hbm": round(v_gbs / HBM_PEAK_GBS, 4),
                   "touched_experts_avg": round(sum(touched_v[i] for i in idx) / K, 3),
                   "f16_bytes_avg": round(bytes_v / K)},
        "roofline": {"kernel": "verify_grouped_gemm (gate/up + down launches)", "bound": "hbm",
                     "achieved": round(rv_ach, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(rv_ach / HBM_PEAK_GBS, 4),
                     "avg_us": round(1e3 * sum(vg_ms) / K, 3),
                     "traffic": pmc_traffic("verify_grouped_gemm")},
        "roofline_draft": {"kernel": "w4a16_grouped_ffn (gate/up + down launches)",
                           "bound": "hbm", "achieved": round(rd_ach, 2), "peak": HBM_PEAK_GBS,
                           "unit": "GB/s", "frac": round(rd_ach / HBM_PEAK_GBS, 4),
                           "avg_us": round(1e3 * sum(w4_ms) / K, 3),
                           "traffic": pmc_traffic("w4a16_grouped_ffn"),
                           "attainable": {
                               "what": "smoe_stream_read of the same gate/up and down byte "
                                       "counts in two dependent launches, HIP events around "
                                       "both, after a verify step",
                               "bytes": gu_b + dn_b, "us": round(stream_us, 3),
                               "gbps": round((gu_b + dn_b) / stream_us / 1e3, 1),
                               "frac_hbm": round((gu_b + dn_b) / stream_us / 1e3
                                                 / HBM_PEAK_GBS, 4)},
                           "frac_attainable": round(rd_ach / ((gu_b + dn_b) / stream_us / 1e3),
                                                    4)},
        "call_us": call_us,
        "draft_single_launch": single,
        "host_wall_s": round(wall, 4),
        "gen_s": round(gen_s, 2),
    }

    # ---- supplementary dense point (outside the benchmark configurations):
    #      the same layer's FP16 experts over T = 2048 tokens, k = 2, i.e. about
    #      256 rows per expert, where the verify FFN is a real contraction ----
    if args.dense_point:
        T_X = 2048
        xd = up(synth.tokens(s, T_X, step=500))
        idsd, _, _ = fve.moe_route_topk(xd, router, k)
        md = fve.moe_gather(idsd, E, err)
        rows_d = T_X * k
        ws_x = fve.new_workspace(1, T_X, k, H, I, E)
        yd = torch.empty((rows_d, H), dtype=torch.float16, device=dev)
        call = lambda: fve.verify_grouped_gemm(xd, md["sorted_token"], md["offsets"], t16, T_X,
                                               rows_d, H, I, E, ws_x, active=md["active"],
                                               n_active=md["n_active"], y_sorted=yd,
                                               err_word=err)
        for _ in range(3):
            call()
        torch.cuda.synchronize()
        nd = 20
        evd = [(mk(), mk()) for _ in range(nd)]
        for i in range(nd):
            evd[i][0].record()
            call()
            evd[i][1].record()
        torch.cuda.synchronize()
        assert int(err.item()) == 0, "device error word set"
        us_d = 1e3 * sum(a.elapsed_time(b) for a, b in evd) / nd
        nact = int(md["n_active"].item())
        fl = 2.0 * rows_d * 3 * H * I
        res["dense_point"] = {
            "note": "supplementary, outside the benchmark configurations: phi35 experts, T=2048 "
                    "tokens, k=2 (verify_grouped_gemm in its tiled-GEMM regime)",
            "rows": rows_d, "touched_experts": nact, "rows_per_expert": round(rows_d / nact, 1),
            "us": round(us_d, 2), "tflops": round(fl / (us_d * 1e-6) / 1e12, 2),
            "frac_mfma": round(fl / (us_d * 1e-6) / 1e12 / MFMA_F16_PEAK_TFS, 4),
            "weight_gbps": round(nact * b16 / (us_d * 1e-6) / 1e9, 1),
            "attainable_tflops": round(min(MFMA_F16_PEAK_TFS,
                                           fl / (nact * b16) * HBM_PEAK_GBS / 1e3), 1)}
        del xd, ws_x, yd

    # ---- the other configurations' layers, for the same line: the
    #      DeepSeek-V2-Lite draft step and the Qwen1.5-MoE verify layer ----
    if args.other_configs:
        K_o = min(max(K, 5), 20)
        ds_res, _, _ = ds_draft_results(K_o, min(args.warmup, 3))
        res["ds_draft"] = {"config": DS_WORKLOAD, "steps": K_o, "results": ds_res}
        res["qwen_verify"] = {"config": QWEN_VERIFY_WORKLOAD, "steps": K_o,
                              **qwen_verify_results(K_o, min(args.warmup, 3))}
        # the 24-layer chunk (one timed chunk after an untimed one)
        c5 = qwen_chunk_results(24, 1, 1)
        res["qwen_chunk"] = {k2: c5[k2] for k2 in ("config", "draft", "placement",
                                                     "verify_staged", "verify_all_resident")}

    if args.calib_copy:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    if args.cpu_sample > 0:
        res["cpu_baseline"] = cpu_baseline(layer, s, args.cpu_sample)
    print(json.dumps(res), flush=True)


def qwen_layers(L, dev):
    """L Qwen-shaped layers generated on the device: ChunkLayer list (FP16
    target experts also in page-locked host memory) and every FP16 expert in
    HBM as [L, E, 3HI]."""
    import torch

    import synth
    from fp16_verify_expert_amd.chunk import ChunkLayer
    s = synth.QWEN_CHUNK
    layers, full = [], torch.empty((L, s.E, 3 * s.H * s.I), dtype=torch.float16, device=dev)
    for l in range(L):
        g = synth.torch_layer(s, l, dev)
        for e, (w13, w2) in enumerate(g["f16"]):
            full[l, e, :2 * s.I * s.H].copy_(w13.reshape(-1))
            full[l, e, 2 * s.I * s.H:].copy_(w2.reshape(-1))
        del g["f16"]
        host_f16 = torch.empty((s.E, 3 * s.H * s.I), dtype=torch.float16, pin_memory=True)
        host_f16.copy_(full[l])
        layers.append(ChunkLayer(router=g["router"], int4=g["int4"], host_f16=host_f16,
                                 shared=(g["shared"]["w13"], g["shared"]["w2"]),
                                 shared_gate=g["shared"]["gate"]))
        print(f"generated layer {l}", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    return layers, full


def bench_draft_formats(args):
    """The draft step at other code widths ([S1] Main Findings and Future
    Directions: draft fidelity is compared at 2-, 4- and 8-bit precision, and
    the precision trades prediction accuracy for memory).  For each width, on
    the Phi-3.5-MoE shape (T = 1) and the DeepSeek-V2-Lite shape (T = 1, 4,
    16): the draft step (moe_route_plan, wq_grouped_ffn, moe_combine) over
    seeded synthetic inputs, every expert in HBM, RTN GPTQ-layout weights of
    the same fp16 experts.  Reported: the weight bytes a step reads, the step
    wall time and the FFN call time (HIP events), and GB/s of both."""
    import numpy as np
    import torch

    import fp16_verify_expert_amd as fve
    import synth

    fve.lib()
    torch.cuda.set_device(0)
    dev = torch.device("cuda")
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    mk = lambda: torch.cuda.Event(enable_timing=True)
    K = max(args.steps, 5)
    results = []
    t_all = time.perf_counter()
    for shape, Ts in ((synth.PHI, (1,)), (synth.DS, (1, 4, 16))):
        f16 = [synth.expert_f16(shape, 0, e) for e in range(shape.E)]
        router = up(synth.router(shape))
        for fmt in (2, 4, 8, "awq4"):
            awq = fmt == "awq4"
            bits = 4 if awq else fmt
            if awq:
                q = [synth.expert_awq(shape, 0, e, w13, w2) for e, (w13, w2) in enumerate(f16)]
            else:
                q = [synth.expert_int4(w13, w2, bits) for w13, w2 in f16]
            gq = [{key: tuple(up(t) for t in ex[key]) for key in ("w13", "w2")} for ex in q]
            table = fve.w4_expert_table(gq)
            sc = [(up(ex["a13"]), up(ex["a2"])) for ex in q] if awq else None
            stab = fve.awq_scale_table(sc) if awq else None
            # codes + scales + zeros (+ the fp16 input-channel factors of AWQ)
            bpe = synth.quant_bytes_per_expert(shape, bits) + (
                2 * (shape.H + shape.I) if awq else 0)
            for T in Ts:
                xs = [up(synth.tokens(shape, T, step=i)) for i in range(POOL)]
                ws = fve.new_workspace(0, T, shape.k, shape.H, shape.I, shape.E)
                y = torch.empty((T * shape.k, shape.H), dtype=torch.float16, device=dev)
                out = torch.empty((T, shape.H), dtype=torch.float16, device=dev)
                ids_b = torch.empty((T, shape.k), dtype=torch.int32, device=dev)
                w_b = torch.empty((T, shape.k), dtype=torch.float32, device=dev)
                maps_b = fve._new_maps(T, shape.k, shape.E, dev)
                lg_b = torch.empty(T * (shape.E + 1), dtype=torch.float32, device=dev)
                touched = []

                def step(i, ev=None):
                    x = xs[i % POOL]
                    ids, w, _, m = fve.moe_route_plan(x, router, shape.k, topk_ids=ids_b,
                                                      topk_w=w_b, maps=maps_b, logits_ws=lg_b)
                    if ev: ev[0].record()
                    if awq:
                        fve.awq_grouped_ffn(x, m, table, stab, T, shape.k, shape.H, shape.I,
                                            shape.E, ws, y_sorted=y)
                    else:
                        fve.wq_grouped_ffn(x, m, table, T, shape.k, shape.H, shape.I, shape.E,
                                           ws, bits, y_sorted=y)
                    if ev: ev[1].record()
                    fve.moe_combine(y, m["pair_pos"], w, out=out)
                    return m

                for i in range(POOL):
                    m = step(i)
                    torch.cuda.synchronize()
                    touched.append(int(m["n_active"].item()))
                for i in range(args.warmup):
                    step(i)
                ph = [(mk(), mk()) for _ in range(K)]
                kf = [(mk(), mk()) for _ in range(K)]
                torch.cuda.synchronize()
                for st in range(K):
                    ph[st][0].record()
                    step(args.warmup + st, kf[st])
                    ph[st][1].record()
                torch.cuda.synchronize()
                idx = [(args.warmup + st) % POOL for st in range(K)]
                nbytes = sum(touched[i] * bpe for i in idx)
                step_ms = sum(a.elapsed_time(b) for a, b in ph)
                ffn_ms = sum(a.elapsed_time(b) for a, b in kf)
                results.append({
                    "shape": shape.name, "bits": bits, "format": "awq" if awq else "gptq",
                    "T": T,
                    "touched_experts_avg": round(sum(touched[i] for i in idx) / K, 2),
                    "weight_bytes_avg": round(nbytes / K),
                    "step_us": round(1e3 * step_ms / K, 2),
                    "step_gbps": round(nbytes / (step_ms * 1e-3) / 1e9, 1),
                    "ffn_us": round(1e3 * ffn_ms / K, 2),
                    "ffn_gbps": round(nbytes / (ffn_ms * 1e-3) / 1e9, 1),
                    "ffn_frac_hbm": round(nbytes / (ffn_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)})
                print(json.dumps(results[-1]), file=sys.stderr, flush=True)
            del gq, table, sc, stab
            torch.cuda.empty_cache()
    phi4 = next(r for r in results if r["shape"] == synth.PHI.name and r["bits"] == 4)
    out = {"metric": "draft step weight GB/s by code width", "value": phi4["step_gbps"],
           "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
           "higher_is_better": True, "vs_baseline": None,
           "dtype": "int2/int4/int8-w (GPTQ layout, g128; AWQ-style int4 with fp16 input-channel "
                    "divisors), fp16-a; fp32 accumulate",
           "data": "synthetic (seeded N(0,0.02) fp16 experts, RTN at each width, N(0,1) tokens)",
           "config": {"workload": "draft_formats: one draft step (route plan, wq_grouped_ffn or "
                                  "awq_grouped_ffn, combine) at 2/4/8 bits and AWQ-style 4 "
                                  "bits; phi35 T=1, ds_v2_lite T=1/4/16"},
           "results": results, "run_s": round(time.perf_counter() - t_all, 1)}
    print(json.dumps(out), flush=True)


def bench_ds_draft(args):
    """The DeepSeek-V2-Lite-shaped draft layer step as a line of its own
    (ds_draft_results)."""
    results, gen_s, K = ds_draft_results(max(args.steps, 5), args.warmup)
    r1 = results[0]
    res = {"metric": "MoE-layer INT4 draft weight GB/s (% HBM peak); verify TFLOP/s (% MFMA)",
           "value": r1["int4_gbps"], "unit": "GB/s", "n_gpus": 1, "steps": K,
           "warmup": args.warmup, "ms_per_step": round(r1["step_us"] / 1e3, 5),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "int4-w/fp16-a (routed experts), fp16 (shared experts); fp32 accumulate",
           "data": "synthetic (seeded N(0,0.02) weights from torch Philox, RTN GPTQ INT4 g128; "
                   "N(0,1) tokens)",
           "config": {"workload": DS_WORKLOAD},
           "results": results, "gen_s": round(gen_s, 1)}
    print(json.dumps(res), flush=True)


DS_WORKLOAD = ("ds_v2_lite draft layer step: H=2048 E=64 top-6 I=1408 + 2 shared experts (as one "
               "of I=2816); T=1/4/16; ELB [1,64]; 1 GiB read before each timed step")


def ds_draft_results(K, warmup):
    """The DeepSeek-V2-Lite-shaped draft layer step (hidden 2048, 64 routed
    experts, top-6, intermediate 1408, 2 FP16 shared experts run as one of
    intermediate 2816, ELB counters over one layer) at T = 1, 4 and 16 tokens,
    every weight in HBM.  T = 1: moe_draft_route_ffn (routing, ELB, maps,
    routed INT4 FFN and the shared experts in three launches) + moe_combine;
    T > 1: moe_route_plan + w4a16_grouped_ffn_shared (the routed INT4 FFN and
    the shared experts; up to 4 rows the shared columns ride in the two
    multi-row launches) + moe_combine.  A read of 1 GiB runs before each timed
    step, outside its events, so the weights come from HBM.  Reported per T:
    the step's wall time (HIP events around its calls, no markers inside),
    the INT4 bytes of the touched experts and the shared experts' FP16 bytes,
    and GB/s of the INT4 bytes and of all weight bytes."""
    import numpy as np
    import torch

    import fp16_verify_expert_amd as fve
    import synth

    fve.lib()
    torch.cuda.set_device(0)
    dev = torch.device("cuda")
    s = synth.DS
    H, E, k, I, Is = s.H, s.E, s.k, s.I, s.shared_I
    t0 = time.perf_counter()
    g = synth.torch_layer(s, 0, dev)
    del g["f16"]
    table = fve.w4_expert_table(g["int4"])
    router = g["router"]
    shared = (g["shared"]["w13"], g["shared"]["w2"])
    gen_s = time.perf_counter() - t0
    scrub = torch.empty(1 << 29, dtype=torch.float16, device=dev)  # 1 GiB
    counters = torch.zeros((1, E), dtype=torch.int32, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    mk = lambda: torch.cuda.Event(enable_timing=True)
    b4 = s.int4_bytes_per_expert
    results = []
    for T in (1, 4, 16):
        xs = [torch.from_numpy(synth.tokens(s, T, step=i)).to(dev) for i in range(POOL)]
        ws = fve.new_workspace(0, T, k, H, I, E)
        sh_h = torch.empty((T, Is), dtype=torch.float16, device=dev)
        sh_out = torch.empty((T, H), dtype=torch.float16, device=dev)
        y = torch.empty((T * k, H), dtype=torch.float16, device=dev)
        out = torch.empty((T, H), dtype=torch.float16, device=dev)
        ids_b = torch.empty((T, k), dtype=torch.int32, device=dev)
        w_b = torch.empty((T, k), dtype=torch.float32, device=dev)
        maps_b = fve._new_maps(T, k, E, dev)
        lg_b = torch.empty(T * (E + 1), dtype=torch.float32, device=dev)

        def step(i):
            x = xs[i % POOL]
            if T == 1:
                fve.moe_draft_route_ffn(x, router, k, table, I, ws, counters=counters,
                                        err_word=err, topk_ids=ids_b, topk_w=w_b, maps=maps_b,
                                        y_sorted=y, shared=shared, shared_h=sh_h,
                                        shared_out=sh_out)
            else:
                # one stream: the shared experts on a side stream were slower
                # (the join before the combine cost about 6 us, and the two
                # streams slowed each other's kernels)
                fve.moe_route_plan(x, router, k, counters=counters, err_word=err,
                                   topk_ids=ids_b, topk_w=w_b, maps=maps_b, logits_ws=lg_b)
                fve.w4a16_grouped_ffn_shared(x, maps_b, table, T, k, H, I, E, ws, shared,
                                             y_sorted=y, shared_h=sh_h, shared_out=sh_out,
                                             err_word=err)
            fve.moe_combine(y, maps_b["pair_pos"], w_b, sh_out, out=out)

        touched = []
        for i in range(POOL):
            step(i)
            torch.cuda.synchronize()
            touched.append(int(maps_b["n_active"].item()))
        for i in range(warmup):
            step(i)
        ev = [(mk(), mk()) for _ in range(K)]
        torch.cuda.synchronize()
        for st in range(K):
            scrub.sum()  # read-only: leaves no dirty lines to write back during the step
            ev[st][0].record()
            step(warmup + st)
            ev[st][1].record()
        torch.cuda.synchronize()
        assert int(err.item()) == 0, "device error word set"
        idx = [(warmup + st) % POOL for st in range(K)]
        b_int4 = sum(touched[i] * b4 for i in idx) / K
        b_sh = s.shared_f16_bytes
        per = sorted(1e3 * a.elapsed_time(b) for a, b in ev)
        us = sum(per) / K
        results.append({"T": T, "touched_experts_avg": round(sum(touched[i] for i in idx) / K, 2),
                        "int4_bytes_avg": round(b_int4), "shared_f16_bytes": b_sh,
                        "step_us": round(us, 2), "step_us_median": round(per[K // 2], 2),
                        "step_us_max": round(per[-1], 2),
                        "int4_gbps": round(b_int4 / us / 1e3, 1),
                        "all_weight_gbps": round((b_int4 + b_sh) / us / 1e3, 1),
                        "all_weight_frac_hbm": round((b_int4 + b_sh) / us / 1e3 / HBM_PEAK_GBS, 4),
                        "path": ("moe_draft_route_ffn (shared experts inside) + moe_combine"
                                 if T == 1 else "moe_route_plan + w4a16_grouped_ffn_shared + "
                                 "moe_combine")})
        print(json.dumps(results[-1]), file=sys.stderr, flush=True)
    del g, table, scrub
    torch.cuda.empty_cache()
    return results, gen_s, K


def bench_qwen_verify(args):
    """The Qwen1.5-MoE-shaped verify layer (qwen_verify_results) as a line of
    its own."""
    import torch

    import fp16_verify_expert_amd as fve
    fve.lib()
    torch.cuda.set_device(0)
    K = max(args.steps, 5)
    r = qwen_verify_results(K, args.warmup, args.context)
    res = {"metric": "MoE-layer INT4 draft weight GB/s (% HBM peak); verify TFLOP/s (% MFMA)",
           "value": round(r["verify"]["bytes"] / r["verify"]["us"] / 1e3, 2),
           "unit": "GB/s (verify FP16 weights)",
           "n_gpus": 1, "steps": K, "warmup": args.warmup,
           "ms_per_step": round(r["layer_step_us"] / 1e3, 5), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "fp16; fp32 accumulate",
           "data": "synthetic (seeded N(0,0.02) weights from torch Philox, N(0,1) tokens)",
           "config": {"workload": QWEN_VERIFY_WORKLOAD}, **r}
    print(json.dumps(res), flush=True)


QWEN_VERIFY_WORKLOAD = ("qwen15_moe verify layer: H=2048 E=60 top-4 I=1408 + gated shared expert "
                        "I=5632; K+1=9 tokens; 1 GiB read before each timed step")


def qwen_verify_results(K, warmup, context=True):
    """The Qwen1.5-MoE-shaped verification layer at K+1 = 9 tokens, every
    weight in HBM: routing plan, verify_grouped_gemm_shared (the routed
    experts and the gated shared expert in the same two launches), combine.
    A read of 1 GiB runs before each timed step, outside its events.
    Reported: the verify call (HIP events around it) as FP16 weight TB/s,
    fraction of HBM peak, TFLOP/s and fraction of FP16 MFMA peak, the layer
    step's wall time, and (context) the routed experts and the shared expert
    as two separate verify_grouped_gemm calls."""
    import torch

    import fp16_verify_expert_amd as fve
    import synth

    dev = torch.device("cuda")
    s = synth.QWEN
    H, E, k, I, Is, T = s.H, s.E, s.k, s.I, s.shared_I, 9
    g = synth.torch_layer(s, 0, dev, int4=False)
    table = fve.f16_expert_table(g["f16"])
    shared = (g["shared"]["w13"], g["shared"]["w2"])
    tsh = fve.f16_expert_table([shared])
    gate = g["shared"]["gate"]
    router = g["router"]
    scrub = torch.empty(1 << 29, dtype=torch.float16, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    mk = lambda: torch.cuda.Event(enable_timing=True)
    xs = [torch.from_numpy(synth.tokens(s, T, step=200 + i)).to(dev) for i in range(POOL)]
    ws = fve.new_workspace(1, T, k, H, I, E)
    wsv = fve.new_workspace(1, T, 1, H, Is, 1)
    iota = torch.arange(T, dtype=torch.int32, device=dev)
    offs = torch.tensor([0, T], dtype=torch.int32, device=dev)
    ids_b = torch.empty((T, k), dtype=torch.int32, device=dev)
    w_b = torch.empty((T, k), dtype=torch.float32, device=dev)
    gate_b = torch.empty((T,), dtype=torch.float32, device=dev)
    maps_b = fve._new_maps(T, k, E, dev)
    lg_b = torch.empty(T * (E + 1), dtype=torch.float32, device=dev)
    y = torch.empty((T * k, H), dtype=torch.float16, device=dev)
    sh_h = torch.empty((T, Is), dtype=torch.float16, device=dev)
    sh_out = torch.empty((T, H), dtype=torch.float16, device=dev)
    out = torch.empty((T, H), dtype=torch.float16, device=dev)

    def plan(i):
        fve.moe_route_plan(xs[i % POOL], router, k, False, gate, err_word=err, topk_ids=ids_b,
                           topk_w=w_b, shared_gate=gate_b, maps=maps_b, logits_ws=lg_b)

    def step(i, ev=None):
        x = xs[i % POOL]
        plan(i)
        if ev: ev[1].record()
        fve.verify_grouped_gemm_shared(x, maps_b["sorted_token"], maps_b["offsets"], table, T,
                                       T * k, H, I, E, ws, shared, active=maps_b["active"],
                                       n_active=maps_b["n_active"], y_sorted=y, shared_h=sh_h,
                                       shared_out=sh_out, err_word=err)
        if ev: ev[2].record()
        fve.moe_combine(y, maps_b["pair_pos"], w_b, sh_out, gate_b, out=out)

    touched = []
    for i in range(POOL):
        step(i)
        torch.cuda.synchronize()
        touched.append(int(maps_b["n_active"].item()))
    for i in range(warmup):
        step(i)
    evs = [[mk() for _ in range(4)] for _ in range(K)]
    torch.cuda.synchronize()
    for st in range(K):
        scrub.sum()
        evs[st][0].record()
        step(warmup + st, evs[st])
        evs[st][3].record()
    # context: the routed experts and the shared expert as separate calls
    sep = [[mk() for _ in range(3)] for _ in range(K)] if context else []
    for st in range(len(sep)):
        i = warmup + st
        x = xs[i % POOL]
        plan(i)
        scrub.sum()
        sep[st][0].record()
        fve.verify_grouped_gemm(x, maps_b["sorted_token"], maps_b["offsets"], table, T, T * k,
                                H, I, E, ws, active=maps_b["active"],
                                n_active=maps_b["n_active"], y_sorted=y, err_word=err)
        sep[st][1].record()
        fve.verify_grouped_gemm(x, iota, offs, tsh, T, T, H, Is, 1, wsv, y_sorted=sh_out,
                                err_word=err)
        sep[st][2].record()
    torch.cuda.synchronize()
    assert int(err.item()) == 0, "device error word set"
    idx = [(warmup + st) % POOL for st in range(K)]
    avg = lambda ev, a, b: 1e3 * sum(e[a].elapsed_time(e[b]) for e in ev) / K
    verify_us, step_us = avg(evs, 1, 2), avg(evs, 0, 3)
    nt = sum(touched[i] for i in idx) / K
    rb = nt * s.f16_bytes_per_expert
    sb = s.shared_f16_bytes
    rf = 2.0 * T * k * 3 * H * I
    sf = 2.0 * T * 3 * H * Is

    def part(nbytes, flops, us):
        return {"bytes": round(nbytes), "us": round(us, 2),
                "tbps": round(nbytes / us / 1e6, 3),
                "frac_hbm": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4),
                "tflops": round(flops / us / 1e6, 3),
                "frac_mfma": round(flops / us / 1e6 / MFMA_F16_PEAK_TFS, 5)}
    res = {"T": T, "touched_experts_avg": round(nt, 2),
           "verify": dict(part(rb + sb, rf + sf, verify_us),
                          call="verify_grouped_gemm_shared (routed + shared expert)"),
           "separate": None if not context else {
               "routed": part(rb, rf, avg(sep, 0, 1)), "shared": part(sb, sf, avg(sep, 1, 2)),
               "note": "the same work as two verify_grouped_gemm calls (context)"},
           "layer_step_us": round(step_us, 2),
           "note": "HIP events around each call inside the step (about 2-4 us each)"}
    del g, table, scrub
    torch.cuda.empty_cache()
    return res


def bench_route_fidelity(args):
    """Draft/target routing agreement and expert demand vs speculation depth
    on residual-chained synthetic Qwen-shaped layers ([S1] Key Contributions
    1: the INT4 copy preserves expert routing; Main Findings: distinct experts
    per layer grow with the depth).  For token streams of lag-one correlation
    rho (a routing-locality knob), every token runs through all layers twice,
    with the INT4 draft experts and with the FP16 target experts (each chain
    on its own outputs, as in drafting and verification).  Reported per rho:
    the mean top-k expert-ID overlap |draft ∩ target| / k per layer and
    overall, and the distinct target experts per layer among K consecutive
    tokens for K = 1..32.  Synthetic weights: the numbers describe this
    kernel stack on random layers, not the pages' trained models."""
    import numpy as np
    import torch

    import fp16_verify_expert_amd as fve
    import synth
    from fp16_verify_expert_amd.chunk import ChunkEngine, distinct_experts, topk_agreement

    fve.lib()
    torch.cuda.set_device(0)
    dev = torch.device("cuda")
    s = synth.QWEN_CHUNK
    L, N = args.layers, 256
    t0 = time.perf_counter()
    layers, full = qwen_layers(L, dev)
    eng = ChunkEngine(layers, s.H, s.E, s.k, s.I, s.shared_I, 16, 17, device=dev)
    gen_s = time.perf_counter() - t0
    depths = [1, 2, 4, 8, 16, 32]
    per_rho = {}
    t1 = time.perf_counter()
    for rho in (0.0, 0.5, 0.8, 0.9, 0.95):
        x = torch.from_numpy(synth.token_stream(s, N, rho)).to(dev)
        rd, rt = [], []
        eng.forward(x, "int4", record=rd)
        eng.forward(x, "f16", full, record=rt)
        torch.cuda.synchronize()
        assert int(eng.err.item()) == 0, "device error word set"
        d = torch.stack([r["ids"] for r in rd]).cpu().numpy()     # [L, N, k]
        t = torch.stack([r["ids"] for r in rt]).cpu().numpy()
        match = topk_agreement(d, t)
        distinct = distinct_experts(t, depths)
        per_rho[str(rho)] = {
            "topk_match_mean": round(float(match.mean()), 4),
            "topk_match_per_layer": [round(float(v), 3) for v in match.mean(axis=1)],
            "distinct_experts_vs_depth": {str(K): round(v, 2) for K, v in distinct.items()},
            "growth_1_to_16": round(distinct[16] / distinct[1], 2)}
    out = {"metric": "draft/target top-k expert-ID agreement; distinct experts vs depth",
           "value": per_rho["0.0"]["topk_match_mean"], "unit": "fraction", "n_gpus": 1,
           "higher_is_better": True, "vs_baseline": None, "data": "synthetic",
           "config": {"workload": f"route_fidelity: {L} Qwen-shaped layers (H=2048 E=60 top-4 "
                                  f"I=1408 + gated shared 5632), {N} tokens per stream, INT4 "
                                  f"RTN g128 draft vs FP16 target, pre-norm residual chain"},
           "per_rho": per_rho, "gen_s": round(gen_s, 1),
           "run_s": round(time.perf_counter() - t1, 1)}
    print(json.dumps(out), flush=True)


def bench_qwen_rounds(args):
    """Speculation rounds with offloaded FP16 target experts ([S1] Key
    Contributions 3: the Layer-Aware Prefetch Planner with Cold Start,
    Prefetch Overlap and Final Cleanup, then the residency manager computing
    hits while misses load).  R consecutive rounds over one AR(1) token
    stream (lag-one correlation --rho: a routing-locality knob); each round
    drafts 16 tokens (INT4, graph-replayed) through 24 Qwen-shaped layers and
    verifies 17 (FP16), with 16 of 60 experts per layer resident.  Two
    policies: boundary placement (draft all, then place the top-16 per layer,
    then verify) and the planner (chunked drafting with ELB-driven prefetch
    overlapped, per-layer events, residency carried across rounds).  The same
    rounds with every expert in HBM give the compute-only time; the exposed
    H2D time of a round is its wall time minus that."""
    import numpy as np
    import torch

    import fp16_verify_expert_amd as fve
    import synth
    from fp16_verify_expert_amd.chunk import ChunkEngine

    fve.lib()
    torch.cuda.set_device(0)
    dev = torch.device("cuda")
    s = synth.QWEN_CHUNK
    L, STEPS, R = args.layers, 16, args.rounds
    t0 = time.perf_counter()
    layers, full = qwen_layers(L, dev)
    eng = ChunkEngine(layers, s.H, s.E, s.k, s.I, s.shared_I, 16, 17, device=dev)
    eng.capture_draft()
    gen_s = time.perf_counter() - t0
    stream = torch.from_numpy(synth.token_stream(s, STEPS * R + 1, args.rho)).to(dev)

    def round_inputs(r):
        xs = [stream[STEPS * r + st:STEPS * r + st + 1] for st in range(STEPS)]
        return xs, stream[STEPS * r:STEPS * r + STEPS + 1]

    # compute only: the same drafts and verifies with every expert in HBM
    comp = []
    for r in range(R):
        xs, xv = round_inputs(r)
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record()
        for x in xs:
            eng.draft_step_graph(x)
        e[1].record()
        eng.verify(xv, all_resident=full)
        e[2].record()
        torch.cuda.synchronize()
        comp.append((e[0].elapsed_time(e[1]), e[1].elapsed_time(e[2])))
    step_s = float(np.mean([c[0] for c in comp])) / STEPS * 1e-3
    res = {}
    for name, planner in (("boundary", False), ("planner", True)):
        eng.resident = [[-1] * eng.nres for _ in range(L)]
        eng.stats = dict(staged_experts=0, staged_bytes=0, hit_experts=0, miss_experts=0,
                         prefetched_experts=0)
        rounds = []
        for r in range(R):
            xs, xv = round_inputs(r)
            before = dict(eng.stats)
            tm = {}
            eng.run_round(xs, xv, planner=planner, step_s=step_s, timing=tm)
            torch.cuda.synchronize()
            assert int(eng.err.item()) == 0, "device error word set"
            d = {k2: eng.stats[k2] - before.get(k2, 0) for k2 in eng.stats}
            wall = tm["start"].elapsed_time(tm["end"])
            rounds.append(dict(ms=round(wall, 2),
                               draft_ms=round(tm["start"].elapsed_time(tm["drafted"]), 2),
                               exposed_h2d_ms=round(wall - sum(comp[r]), 2),
                               placed_or_prefetched=(d.get("prefetched_experts", 0) if planner
                                                     else L * eng.nres),
                               hits=d["hit_experts"], misses=d["miss_experts"]))
        warm = rounds[1:] if R > 1 else rounds
        res[name] = {"rounds": rounds,
                     "mean_ms_after_cold": round(float(np.mean([x["ms"] for x in warm])), 2),
                     "mean_exposed_h2d_ms_after_cold":
                         round(float(np.mean([x["exposed_h2d_ms"] for x in warm])), 2),
                     "hit_rate": round(sum(x["hits"] for x in rounds) /
                                       max(1, sum(x["hits"] + x["misses"] for x in rounds)), 3)}
    out = {"metric": "exposed H2D time per speculation round (ms)",
           "value": res["planner"]["mean_exposed_h2d_ms_after_cold"], "unit": "ms",
           "n_gpus": 1, "higher_is_better": False, "vs_baseline": None,
           "data": f"synthetic (AR(1) token stream, rho={args.rho})",
           "config": {"workload": f"qwen_rounds: {R} rounds x (16 INT4 draft steps + 17-token "
                                  f"FP16 verify), {L} Qwen-shaped layers, 16/60 experts resident "
                                  f"per layer, pinned-host staging"},
           "compute_only_ms": [round(a + b, 2) for a, b in comp],
           "policies": res, "gen_s": round(gen_s, 1)}
    print(json.dumps(out), flush=True)


def bench_qwen_chunk(args):
    """The Qwen-shaped draft chunk + verify (qwen_chunk_results) as a line of
    its own."""
    out = qwen_chunk_results(args.layers, args.steps, args.warmup, args.no_graph)
    print(json.dumps(out), flush=True)


def qwen_chunk_results(L, steps, warmup, no_graph=True):
    """Draft chunk + verify over L Qwen-shaped layers with 16 of 60 FP16
    experts resident per layer.  One step = 16 INT4 draft decode steps through
    all layers (ELB table [L, 60]), the chunk-boundary snapshot and placement of
    the top-16 experts per layer, then the 17-token FP16 verify where misses
    are staged from pinned host memory on a side stream behind the hit GEMMs.
    The same verify with every expert in HBM gives the PCIe-free figure."""
    import numpy as np
    import torch

    import fp16_verify_expert_amd as fve
    import synth
    from fp16_verify_expert_amd.chunk import ChunkEngine, ChunkLayer

    fve.lib()
    torch.cuda.set_device(0)
    dev = torch.device("cuda")
    s = synth.QWEN_CHUNK
    STEPS, TV, NRES = 16, 17, 16
    t0 = time.perf_counter()
    layers, full = qwen_layers(L, dev)
    gen_s = time.perf_counter() - t0
    eng = ChunkEngine(layers, s.H, s.E, s.k, s.I, s.shared_I, NRES, TV, device=dev)
    mk = lambda: torch.cuda.Event(enable_timing=True)

    def chunk(c, timed):
        xs = [torch.from_numpy(synth.tokens(s, 1, step=1000 * c + st)).to(dev)
              for st in range(STEPS)]
        xv = torch.cat(xs + [torch.from_numpy(synth.tokens(s, 1, step=1000 * c + STEPS)).to(dev)])
        ev = [mk() for _ in range(5)]
        eng.clear_counters()
        before = dict(eng.stats)
        ev[0].record()
        for st in range(STEPS):
            if no_graph:
                eng.draft_step(xs[st])
            else:
                eng.draft_step_graph(xs[st])
        ev[1].record()
        counts = eng.snapshot()
        eng.place_residents(counts)
        ev[2].record()
        eng.verify(xv)
        ev[3].record()
        eng.verify(xv, all_resident=full)
        ev[4].record()
        torch.cuda.synchronize()
        assert int(eng.err.item()) == 0, "device error word set"
        d = {k2: eng.stats[k2] - before[k2] for k2 in eng.stats}
        return dict(draft_ms=ev[0].elapsed_time(ev[1]), place_ms=ev[1].elapsed_time(ev[2]),
                    verify_ms=ev[2].elapsed_time(ev[3]), verify_res_ms=ev[3].elapsed_time(ev[4]),
                    # T = 1: each layer-step reads exactly k distinct INT4 experts
                    int4_bytes=STEPS * L * s.k * s.int4_bytes_per_expert,
                    shared_bytes=STEPS * L * s.shared_f16_bytes, stats=d,
                    place_bytes=L * NRES * s.f16_bytes_per_expert)

    if not no_graph:
        eng.capture_draft()
    for c in range(warmup and 1):
        chunk(c, False)
    res_list = [chunk(100 + c, True) for c in range(max(1, min(steps, 3)))]
    n = len(res_list)
    avg = lambda key: sum(r[key] for r in res_list) / n
    draft_ms, verify_ms, verify_res_ms, place_ms = (avg("draft_ms"), avg("verify_ms"),
                                                    avg("verify_res_ms"), avg("place_ms"))
    int4_b, sh_b = avg("int4_bytes"), avg("shared_bytes")
    staged = sum(r["stats"]["staged_bytes"] for r in res_list) / n
    hits = sum(r["stats"]["hit_experts"] for r in res_list) / n
    misses = sum(r["stats"]["miss_experts"] for r in res_list) / n
    flops_v = 2.0 * TV * s.k * 3 * s.H * s.I * L + 2.0 * TV * 3 * s.H * s.shared_I * L
    touched_v = (hits + misses)
    vbytes = touched_v * s.f16_bytes_per_expert + L * s.shared_f16_bytes
    value = int4_b / (draft_ms * 1e-3) / 1e9
    out = {
        "metric": "MoE-layer INT4 draft weight GB/s (% HBM peak); verify TFLOP/s (% MFMA)",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": n, "warmup": 1,
        "ms_per_step": round(draft_ms + place_ms + verify_ms, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "int4-w/fp16-a (draft), fp16 (verify); fp32 accumulate",
        "data": "synthetic (seeded N(0,0.02) weights from torch Philox, N(0,1) tokens)",
        "config": {"workload": f"qwen15_moe_chunk: {L} layers H=2048 E=60 top-4 I=1408 + shared "
                               f"5632 gated; 16 draft steps (T=1), ELB [{L},60], 16/60 resident, "
                               f"verify K+1=17 with staged misses"},
        "draft": {"ms": round(draft_ms, 3), "int4_gbps": round(value, 2),
                  "int4_plus_shared_gbps": round((int4_b + sh_b) / (draft_ms * 1e-3) / 1e9, 2),
                  "int4_bytes": round(int4_b), "shared_f16_bytes": round(sh_b),
                  "launch": "eager" if no_graph else "hip_graph",
                  "us_per_layer_step": round(1e3 * draft_ms / (STEPS * L), 2)},
        "placement": {"ms": round(place_ms, 3), "bytes": res_list[0]["place_bytes"],
                      "h2d_gbps": round(res_list[0]["place_bytes"] / (place_ms * 1e-3) / 1e9, 2)},
        "verify_staged": {"ms": round(verify_ms, 3), "hits": hits, "misses": misses,
                          "staged_bytes": round(staged),
                          "staged_gbps_over_verify": round(staged / (verify_ms * 1e-3) / 1e9, 2)},
        "verify_all_resident": {"ms": round(verify_res_ms, 3),
                                "tflops": round(flops_v / (verify_res_ms * 1e-3) / 1e12, 3),
                                "frac_mfma": round(flops_v / (verify_res_ms * 1e-3) / 1e12
                                                   / MFMA_F16_PEAK_TFS, 5),
                                "weight_gbps": round(vbytes / (verify_res_ms * 1e-3) / 1e9, 2)},
        "gen_s": round(gen_s, 1),
    }
    del eng, layers, full
    torch.cuda.empty_cache()
    return out


def cpu_baseline(layer, s, n):
    """The oracle (as it stands) on n draft steps of the same workload."""
    import numpy as np
    import oracle
    import synth
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))
    nbytes = 0
    t0 = time.perf_counter()
    for i in range(n):
        x = synth.tokens(s, 1, step=i)
        r = oracle.route_topk(x, layer["router"], s.k)
        m = oracle.gather_maps(r["ids"], s.E)
        y = oracle.grouped_ffn(x, m, layer["int4"], "int4")
        oracle.combine(y, m["pair_pos"], r["weights"])
        nbytes += int(m["n_active"]) * s.int4_bytes_per_expert
    dt = time.perf_counter() - t0
    out = {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": cores,
           "kind": "oracle",
           "sample": f"{n} INT4 draft steps (T=1, route+gather+dequant+fp64 FFN+combine) of the "
                     f"phi35 layer in {dt:.1f} s"}
    try:
        model = next(l.split(":", 1)[1].strip() for l in open("/proc/cpuinfo")
                     if l.startswith("model name"))
    except Exception:
        model = None
    out["cpu_model"] = model
    # context: one step single-threaded, and the matmuls alone on pre-dequantised
    # fp32 weights (the touched experts of one step)
    try:
        from threadpoolctl import threadpool_limits
        x = synth.tokens(s, 1, step=0)
        r = oracle.route_topk(x, layer["router"], s.k)
        m = oracle.gather_maps(r["ids"], s.E)
        b1 = int(m["n_active"]) * s.int4_bytes_per_expert
        with threadpool_limits(1):
            t1 = time.perf_counter()
            oracle.grouped_ffn(x, m, layer["int4"], "int4")
            d1 = time.perf_counter() - t1
        out["single_thread_gbps"] = round(b1 / d1 / 1e9, 4)
        ws = []
        for e in [int(v) for v in m["active"] if v >= 0]:
            q = layer["int4"][e]
            ws.append((oracle.dequant_gptq(*q["w13"], dtype=np.float32),
                       oracle.dequant_gptq(*q["w2"], dtype=np.float32)))
        xf = x.astype(np.float32)
        t2 = time.perf_counter()
        for w13, w2 in ws:
            oracle.swiglu_ffn(xf, w13[:, :s.I], w13[:, s.I:], w2)
        d2 = time.perf_counter() - t2
        out["matmul_only_gbps"] = round(b1 / d2 / 1e9, 4)
        out["matmul_only_note"] = ("fp32 BLAS on pre-dequantised weights of one step's touched "
                                   "experts, same algorithmic INT4 bytes")
    except Exception as exc:  # context only
        out["extra_error"] = str(exc)[:200]
    return out


if __name__ == "__main__":
    main()
