#!/usr/bin/env python3
"""Benchmark of one CP rank's causal attention share on one MI355X.

A step is one pass of the share's hot path over one synthetic batch: the
forward (out + LSE) and, where built, the backward (dQ and partial dK/dV) of
the Colossal (all-gather) share of rank 7 of cp=8 at S = 32768: B = 1, 32 query
heads over 8 KV heads (GQA), head_dim 128, bf16 inputs with fp32 accumulation,
query rows 28672..32767 against all 32768 keys. Inputs are iid N(0, 1) rounded
to bf16 (seed 0) and resident in HBM before timing starts.

FLOPs are causal-effective: only visible (query, key) pairs count, 4*D per pair
for the forward and 10*D per pair for the backward (its five contractions,
including the recomputed Q K^T). Peak: 2.5 PFLOP/s dense bf16 MFMA.

Prints ONE JSON line. `--detail` adds every other share of the workload list
(forward only) to that line under "detail".
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

PEAK_BF16_TFLOPS = 2500.0
WORKLOAD = "colossal_cp8_r7_s32k_gqa32x8_d128"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--detail", action="store_true", help="also time every other share (forward)")
    return ap.parse_args()


def share_for(spec, rank):
    kind = spec["kind"]
    return kind, spec["cp"], rank, spec.get("ulysses", 2)


def time_share(spec, prob, rank, steps, warmup, with_bwd):
    import torch
    from context_causal_attention_attn_amd import api, cut_share

    dev = torch.device("cuda")
    q, k, v = prob.q.to(dev), prob.k.to(dev), prob.v.to(dev)
    kind, cp, r, U = share_for(spec, rank)
    sh = cut_share(kind, q, k, v, cp, r, ulysses=U)
    D = q.shape[-1]
    scale = 1.0 / math.sqrt(D)
    d = api.make_desc(sh.q, sh.k, sh.v, sh.q.stride(), sh.q_chunk_pos, [0], sh.layout, True, scale)
    pairs = api.cp_attn_share_pairs(d)
    B, Hq = sh.q.shape[0], sh.q.shape[1]
    f_fwd = 4.0 * D * B * Hq * pairs
    f_bwd = 10.0 * D * B * Hq * pairs
    out = torch.empty(sh.q.shape, dtype=sh.q.dtype, device=dev)
    lse = torch.empty(sh.q.shape[:3], dtype=torch.float32, device=dev)
    dout = sh.take_rows(prob.dout.to(dev)).contiguous() if (with_bwd and prob.dout is not None) else None

    def fwd():
        api.cp_attn_fwd(sh.q, sh.k, sh.v, sh.q_chunk_pos, layout=sh.layout, softmax_scale=scale,
                        out=out, lse=lse)

    def bwd():
        return api.cp_attn_bwd(sh.q, sh.k, sh.v, out, lse, dout, sh.q_chunk_pos, layout=sh.layout,
                               softmax_scale=scale)

    for _ in range(warmup):
        fwd()
        if dout is not None:
            bwd()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(steps):
        ev[i][0].record(stream)
        fwd()
        ev[i][1].record(stream)
        if dout is not None:
            bwd()
        ev[i][2].record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(end)
    fwd_ms = [a.elapsed_time(b) for a, b, _ in ev]
    bwd_ms = [b.elapsed_time(c) for _, b, c in ev] if dout is not None else []
    return dict(pairs=pairs, f_fwd=f_fwd, f_bwd=f_bwd if dout is not None else 0.0, total_ms=total_ms,
                wall_s=wall, fwd_ms=fwd_ms, bwd_ms=bwd_ms, hq=Hq, batch=B, sq=sh.q.shape[2])


def cpu_baseline(spec, prob):
    """The oracle as it stands, on a bounded sample of the same share: query
    head 0 (its KV head 0), every local row, forward + backward."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle.cp_share as oc

    kind, cp, r, U = share_for(spec, spec["ranks"][0])
    S, Hq, Hkv = spec["seq"], spec["hq"], spec["hkv"]
    if kind == "contiguous":
        sh = oc.contiguous_share(S, Hq, Hkv, cp, r)
    elif kind == "head_tail":
        sh = oc.head_tail_share(S, Hq, Hkv, cp, r)
    elif kind == "ulysses":
        sh = oc.ulysses_share(S, Hq, Hkv, cp, r)
    else:
        sh = oc.hybrid_share(S, Hq, Hkv, cp, U, r)
    h, hk = int(sh["q_heads"][0]), int(sh["kv_heads"][0])
    D = spec["head_dim"]
    q = prob.q[:1, h:h + 1].double().numpy()[:, :, sh["q_pos"]]
    k = prob.k[:1, hk:hk + 1].double().numpy()
    v = prob.v[:1, hk:hk + 1].double().numpy()
    do = (prob.dout[:1, h:h + 1].double().numpy()[:, :, sh["q_pos"]] if prob.dout is not None
          else np.random.default_rng(0).standard_normal(q.shape))
    scale = 1.0 / math.sqrt(D)
    t0 = time.perf_counter()
    oc.attention_rows_bwd(q, k, v, do, sh["q_pos"], sh["kv_pos"], scale, True)
    dt = time.perf_counter() - t0
    pairs = oc.share_pairs(sh["q_pos"], sh["kv_pos"])
    flops = 14.0 * D * pairs   # forward (4D) + backward (10D) per visible pair
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{kind} share rank {r}: query head {h} only (1 of {len(sh['q_heads'])}), "
                      f"all {len(sh['q_pos'])} local rows, forward+backward in fp64 NumPy; "
                      f"{dt:.1f} s for {flops / 1e9:.1f} causal-effective GFLOP",
            "seconds": dt}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share; --gpus {args.gpus} is not supported: every share "
              "runs on one GPU with the gathered K/V as an input, and no collective is part of this "
              "build.", file=sys.stderr)
        sys.exit(2)
    import torch

    from context_causal_attention_attn_amd import build as b
    if not os.path.exists(b.LIB_PATH):
        b.build()
    from context_causal_attention_attn_amd import _lib
    from synthetic import WORKLOADS, workload

    lib = _lib.load()
    spec, prob = workload(args.workload, seed=0)
    with_bwd = True
    if with_bwd and prob.dout is None:
        from synthetic import global_problem
        prob = global_problem(spec["batch"], spec["hq"], spec["hkv"], spec["seq"], spec["head_dim"],
                              spec["dtype"], 0, with_dout=True)
    res = time_share(spec, prob, spec["ranks"][0], args.steps, args.warmup, with_bwd)
    ms_per_step = res["total_ms"] / args.steps
    flops_step = res["f_fwd"] + res["f_bwd"]
    value = flops_step / (ms_per_step * 1e-3) / 1e12
    fwd_avg = sum(res["fwd_ms"]) / len(res["fwd_ms"])
    bwd_avg = sum(res["bwd_ms"]) / len(res["bwd_ms"]) if res["bwd_ms"] else 0.0
    fwd_tflops = res["f_fwd"] / (fwd_avg * 1e-3) / 1e12
    bwd_tflops = res["f_bwd"] / (bwd_avg * 1e-3) / 1e12 if bwd_avg else None
    if bwd_avg > fwd_avg:
        dom, achieved = "cp_attn_bwd (bwd_main_kernel<128> + pre/convert)", bwd_tflops
    else:
        dom, achieved = "fwd_bf16_kernel<128,1>", fwd_tflops
    line = {
        "metric": "causal-effective TFLOP/s per CP-rank share (fwd, bwd) and % of bf16 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "kind": spec["kind"], "cp": spec["cp"],
                   "rank": spec["ranks"][0], "batch": spec["batch"], "hq": spec["hq"], "hkv": spec["hkv"],
                   "head_dim": spec["head_dim"], "seq_global": spec["seq"], "sq_local": res["sq"],
                   "causal_pairs_per_head": res["pairs"],
                   "passes": "fwd+bwd" if with_bwd else "fwd (backward not built yet)"},
        "fwd": {"ms": round(fwd_avg, 4), "tflops": round(fwd_tflops, 2),
                "frac_of_peak": round(fwd_tflops / PEAK_BF16_TFLOPS, 4)},
        "bwd": ({"ms": round(bwd_avg, 4), "tflops": round(bwd_tflops, 2),
                 "frac_of_peak": round(bwd_tflops / PEAK_BF16_TFLOPS, 4)} if bwd_avg else None),
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None},
        "device": torch.cuda.get_device_name(0),
    }
    if args.detail:
        detail = {}
        for name, sp in WORKLOADS.items():
            if sp["dtype"] != "bf16":
                continue
            bw = bool(sp.get("backward"))
            _, pr = workload(name, seed=0)
            for r in sp["ranks"]:
                rr = time_share(sp, pr, r, max(5, args.steps // 2), 2, bw)
                avg = sum(rr["fwd_ms"]) / len(rr["fwd_ms"])
                tf = rr["f_fwd"] / (avg * 1e-3) / 1e12
                ent = {"fwd_ms": round(avg, 4), "fwd_tflops": round(tf, 2),
                       "fwd_frac": round(tf / PEAK_BF16_TFLOPS, 4)}
                if bw:
                    bavg = sum(rr["bwd_ms"]) / len(rr["bwd_ms"])
                    btf = rr["f_bwd"] / (bavg * 1e-3) / 1e12
                    ent.update({"bwd_ms": round(bavg, 4), "bwd_tflops": round(btf, 2),
                                "bwd_frac": round(btf / PEAK_BF16_TFLOPS, 4)})
                detail[f"{name}/r{r}"] = ent
            del pr
        line["detail"] = detail
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(spec, prob)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
