#!/usr/bin/env python3
"""Benchmark of one CP rank's causal attention share on one MI355X.

A step is one pass of the share's hot path over one synthetic batch: the
forward (out + LSE) and the backward (Delta pass, dK/dV kernel, dQ kernel) of
the Colossal (all-gather) share of rank 7 of cp=8 at S = 32768: B = 1, 32 query
heads over 8 KV heads (GQA), head_dim 128, bf16 inputs with fp32 accumulation,
query rows 28672..32767 against all 32768 keys. Inputs are iid N(0, 1) rounded
to bf16 (seed 0) and resident in HBM before timing starts. `value` is that
step's throughput.

FLOPs are causal-effective: only visible (query, key) pairs count, 4*D per pair
for the forward and 10*D per pair for the backward (its five contractions,
including the recomputed Q K^T). Peak: 2516.6 TFLOP/s dense bf16 MFMA (256 CUs x
4096 flop per clock x 2.4 GHz).

Each kernel's time is the average, over the timed steps, of HIP events the
library records on the launch stream around it (cp_attn_bwd_timed); the
roofline object describes the kernel with the largest average. Its "traffic"
comes from the rocprofv3 counter summaries in profiles/ when one matches the
kernel's current source text, else null.

After the headline share, the line times every other share the workloads
state a target for ("configs", forward and backward each): the Head-Tail
shares of all 8 ranks (with their max/min spread under "balance"), the Ulysses
cp=8 rank-0 share, the Hybrid U=2 x C=4 rank-4 share and the Head-Tail B = 2
backward shares of ranks 0 and 7, and the Colossal rank-7 share over eight
packed sequences; the Ulysses share also runs straight from the all-to-all's
received blocks (".../in_place": no unpack or pack pass); the headline share
also runs under a boolean, an additive and an additive padding user mask
(".../user_mask_*": 10 % of the pairs hidden at random, FLOPs still over
the causal pairs). While the headline step keeps running for
about 2.5 s, amd-smi reads the GFX clocks and socket power ("clock"; the chip
runs at its power cap, below the 2.4 GHz the peak assumes). The oracle's CPU
baseline runs last, in a child process. Prints ONE JSON line. `--detail` adds
every bf16 workload share (K/V in all-gather order, packed sequences) and the
Ulysses re-layouts under "detail".
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

PEAK_BF16_TFLOPS = 2516.6   # 256 CUs x 4096 bf16 flop/clock x 2.4 GHz, dense
PEAK_HBM_GBS = 8000.0
WORKLOAD = "colossal_cp8_r7_s32k_gqa32x8_d128"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--warm-s", type=float, default=1.0,
                    help="seconds of untimed steps of the headline share before its warm-up steps")
    ap.add_argument("--workload", default=WORKLOAD)
    ap.add_argument("--rank", type=int, default=None,
                    help="CP rank of the workload's share (default: the workload's first listed rank)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-clock", action="store_true", help="skip the amd-smi clock/power sample")
    ap.add_argument("--detail", action="store_true",
                    help="also time every bf16 workload share (gathered K/V orders, packed sequences) "
                         "and the Ulysses re-layouts")
    ap.add_argument("--no-configs", action="store_true",
                    help="time only the headline share (skip the other target shares)")
    ap.add_argument("--kv-order", choices=["natural", "gathered"], default="natural",
                    help="K/V in natural order, or as an all-gather delivers them (a KV chunk table)")
    ap.add_argument("--relayout-only", action="store_true",
                    help="only time the Ulysses exchange re-layouts (prints their JSON object)")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="after timing, run one plain device copy of this many MiB (counter calibration)")
    return ap.parse_args()


def share_for(spec, rank):
    kind = spec["kind"]
    return kind, spec["cp"], rank, spec.get("ulysses", 2)


KERNEL_SOURCES = {   # files whose text determines each kernel's machine code
    "fwd": ["fwd_bf16_kernel.h", "fwd_bf16_m0.hip", "gfx950_common.h", "plan.h", "../../include/cp_attn.h"],
    "pre": ["bwd_bf16_kernels.h", "bwd_bf16.hip", "gfx950_common.h", "plan.h", "../../include/cp_attn.h"],
    "dkdv": ["bwd_bf16_kernels.h", "bwd_dkdv_m0.hip", "gfx950_common.h", "plan.h", "../../include/cp_attn.h"],
    "dq": ["bwd_bf16_kernels.h", "bwd_dq_m0.hip", "gfx950_common.h", "plan.h", "../../include/cp_attn.h"],
}
KERNEL_NAMES = {"fwd": "fwd_bf16_kernel<128, 2, 0>", "pre": "bwd_pre_kernel<128>",
                "dkdv": "bwd_dkdv_kernel<128, 0>", "dq": "bwd_dq_kernel<128, 2, 0>"}


def sources_sha256(part):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[part]:
        with open(os.path.join(ROOT, "context_causal_attention_attn_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def kernel_name(part, spec, kv_order):
    """The instantiation a share runs: mode 0 for keys in natural order, 1 for
    a KV chunk table, 2 for packed sequences (the dK/dV kernel: 0, or 1 for
    packed sequences). The workloads all have GQA groups of 4 (two row blocks
    per forward and dQ work item)."""
    name = KERNEL_NAMES[part]
    mode = 2 if spec.get("doc_lengths") else (1 if kv_order == "gathered" else 0)
    if part in ("fwd", "dq"):
        return name.replace(", 0>", f", {mode}>")
    if part == "dkdv" and mode == 2:
        return name.replace(", 0>", ", 1>")
    return name


def traffic_record(part):
    """HBM bytes per launch of a kernel from the rocprofv3 counter summaries in
    profiles/ (FETCH_SIZE and WRITE_SIZE passes, scaled by a plain copy of known
    size), or None when no summary matches the kernel's current source text."""
    import glob
    import re
    want = sources_sha256(part)
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        for line in open(path):
            m = re.match(r"traffic-record kernel=(\S+) sources_sha256=([0-9a-f]+) "
                         r"fetch_bytes=(\d+) write_bytes=(\d+)", line.strip())
            if m and m.group(1) == KERNEL_NAMES[part].replace(" ", "") and m.group(2) == want:
                return {"fetch_bytes": int(m.group(3)), "write_bytes": int(m.group(4)),
                        "source": os.path.relpath(path, ROOT)}
    return None


class BlockShare:
    """A Ulysses head shard as the sequence->head all-to-all delivers it: the
    received blocks [u, B, H, L, D] of Q, K, V (and dO), read in place by the
    share kernels (chunked layout, block p at positions p*L..)."""

    def __init__(self, prob, U, rank, dev):
        import torch
        from context_causal_attention_attn_amd import seq_to_head_pack
        L = prob.q.shape[2] // U

        def recv(t):
            # rank `rank`'s receive buffer: block `rank` of every source rank's send buffer
            return torch.stack([seq_to_head_pack(t[:, :, p * L:(p + 1) * L].to(dev), U)[rank]
                                for p in range(U)]).contiguous()

        self.q, self.k, self.v = recv(prob.q), recv(prob.k), recv(prob.v)
        self._dout = recv(prob.dout) if prob.dout is not None else None
        self.q_chunk_pos = [p * L for p in range(U)]
        self.kv_chunk_pos = list(self.q_chunk_pos)
        self.layout = "chunked"

    def take_rows(self, _dout):
        return self._dout


def share_user_mask(kind, B, Sq, Skv, dev):
    """A seeded user mask for a share, broadcast over heads: "bool", 10 % of
    the (row, key) pairs hidden at random; "additive", N(0, 1) biases with the
    same 10 % at -inf; "padding", 0 with the same 10 % at -inf."""
    import torch
    g = torch.Generator(device="cpu").manual_seed(11)
    keep = torch.rand((1, 1, Sq, Skv), generator=g) >= 0.1
    if kind == "bool":
        return keep.to(dev)
    bias = torch.randn((1, 1, Sq, Skv), generator=g) if kind == "additive" else torch.zeros((1, 1, Sq, Skv))
    return torch.where(keep, bias, torch.full((), float("-inf"))).to(dev)


def time_share(spec, prob, rank, steps, warmup, with_bwd, kv_order="natural", warm_s=0.0, in_place=False,
               user_mask=None):
    import torch
    from context_causal_attention_attn_amd import api, cut_share

    dev = torch.device("cuda")
    kind, cp, r, U = share_for(spec, rank)
    from synthetic import doc_starts
    if in_place:   # Ulysses share straight from the exchange's blocks
        sh = BlockShare(prob, cp, r, dev)
    else:
        q, k, v = prob.q.to(dev), prob.k.to(dev), prob.v.to(dev)
        sh = cut_share(kind, q, k, v, cp, r, ulysses=U, kv_order=kv_order)
    kvp = sh.kv_chunk_pos
    docs = doc_starts(spec)
    D = sh.q.shape[-1]
    scale = 1.0 / math.sqrt(D)
    B, Hq, Sq = api._geom(sh.q)[:3]
    Hkv, Skv = api._geom(sh.k)[1:3]
    mask = share_user_mask(user_mask, B, Sq, Skv, dev) if user_mask else None
    d = api.make_desc(sh.q, sh.k, sh.v, sh.q, sh.q_chunk_pos, kvp, sh.layout, True, scale, docs, mask)
    pairs = api.cp_attn_share_pairs(d)
    out = torch.empty(sh.q.shape, dtype=sh.q.dtype, device=dev)
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=dev)
    dout = (sh.take_rows(prob.dout.to(dev)).contiguous() if not in_place else sh.take_rows(None)) \
        if (with_bwd and prob.dout is not None) else None
    if dout is not None:
        grads = (torch.empty_like(out), torch.empty((B, Hkv, Skv, D), dtype=torch.float32, device=dev),
                 torch.empty((B, Hkv, Skv, D), dtype=torch.float32, device=dev))
        ws = torch.empty(max(1, api.cp_attn_workspace_bytes(d, True)), dtype=torch.uint8, device=dev)

    def fwd():
        api.cp_attn_fwd(sh.q, sh.k, sh.v, sh.q_chunk_pos, layout=sh.layout, softmax_scale=scale,
                        out=out, lse=lse, kv_chunk_pos=kvp, doc_starts=docs, attn_mask=mask)

    def bwd(events):
        api.cp_attn_bwd_timed(sh.q, sh.k, sh.v, out, lse, dout, sh.q_chunk_pos, events,
                              layout=sh.layout, softmax_scale=scale, workspace=ws, grads=grads,
                              kv_chunk_pos=kvp, doc_starts=docs, attn_mask=mask)

    def new_events():
        return [torch.cuda.Event(enable_timing=True) for _ in range(5)]

    # Steps for warm_s seconds (clocks ramp up over a few hundred
    # milliseconds after the GPU idled), then exactly `warmup` steps.
    def untimed():
        ev = new_events()
        fwd()
        if dout is not None:
            bwd(ev[1:])

    t_warm = time.perf_counter()
    while time.perf_counter() - t_warm < warm_s:
        for _ in range(4):
            untimed()
        torch.cuda.synchronize()
    for _ in range(warmup):
        untimed()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = [new_events() for _ in range(steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(steps):
        ev = evs[i]
        ev[0].record(stream)
        fwd()
        ev[1].record(stream)
        if dout is not None:
            bwd(ev[1:])   # records ev[1] again (same point: nothing runs in between) .. ev[4]
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(end)

    def avg(i, j):
        return sum(e[i].elapsed_time(e[j]) for e in evs) / steps

    ms = {"fwd": avg(0, 1)}
    if dout is not None:
        ms.update(pre=avg(1, 2), dkdv=avg(2, 3), dq=avg(3, 4), bwd=avg(1, 4))
    fl = {"fwd": 4.0 * D * B * Hq * pairs, "bwd": 10.0 * D * B * Hq * pairs,
          # contractions each kernel performs on visible pairs: dK/dV recomputes
          # S and dP and forms dV, dK (4 x 2D); dQ recomputes S and dP and forms dQ (3 x 2D)
          "dkdv": 8.0 * D * B * Hq * pairs, "dq": 6.0 * D * B * Hq * pairs}
    el = 2 if sh.q.dtype == torch.bfloat16 else 4
    io = {"pre": 2 * B * Hq * Sq * D * el + 4 * B * Hq * Sq,   # read out, dout; write Delta
          "fwd": (B * Hq * Sq * D * el * 2 + 2 * B * Hkv * Skv * D * el + 4 * B * Hq * Sq),
          "dkdv": (2 * B * Hq * Sq * D * el + 2 * B * Hkv * Skv * D * el + 8 * B * Hq * Sq
                   + 2 * B * Hkv * Skv * D * 4),
          "dq": (3 * B * Hq * Sq * D * el + 2 * B * Hkv * Skv * D * el + 8 * B * Hq * Sq)}
    def step():
        fwd()
        if dout is not None:
            bwd(new_events()[1:])

    return dict(pairs=pairs, flops=fl, bytes=io, ms=ms, total_ms=total_ms, wall_s=wall,
                hq=Hq, batch=B, sq=Sq, has_bwd=dout is not None, step=step)


def parse_smi_metric(text):
    """GFX clocks (MHz, one per XCD) and socket power (W) from the text of
    `amd-smi metric -c -p` (sections GFX_<n>: with a CLK: line each)."""
    import re
    clocks, power, in_gfx = [], None, False
    for line in text.splitlines():
        m = re.match(r"\s*SOCKET_POWER:\s*([0-9.]+)\s*W", line)
        if m and power is None:
            power = float(m.group(1))
        if re.match(r"\s*GFX_\d+:\s*$", line):
            in_gfx = True
            continue
        if re.match(r"\s*[A-Z][A-Z0-9_]*:\s*$", line):
            in_gfx = False
            continue
        m = re.match(r"\s*CLK:\s*([0-9.]+)\s*MHz", line)
        if m and in_gfx:
            clocks.append(float(m.group(1)))
            in_gfx = False
    return clocks, power


def sample_clock(step, seconds=2.5, samples=3):
    """Run `step` back to back for about `seconds` and read the GFX clocks and
    socket power `samples` times with amd-smi (the timed region itself is too
    short for the tool). A read can land in a lull, so the sample drawn at the
    highest socket power is the one reported; all reads are listed. None when
    amd-smi is not available."""
    import shutil
    import subprocess
    import threading

    import torch
    exe = shutil.which("amd-smi")
    if exe is None:
        return None
    texts = []

    def probe():
        for i in range(samples):
            time.sleep(seconds / (samples + 1))
            try:
                r = subprocess.run([exe, "metric", "-c", "-p"], capture_output=True, text=True, timeout=20)
                texts.append(r.stdout)
            except (OSError, subprocess.SubprocessError):
                pass

    th = threading.Thread(target=probe)
    th.start()
    t0 = time.perf_counter()
    while th.is_alive() or time.perf_counter() - t0 < seconds:
        for _ in range(4):
            step()
        torch.cuda.synchronize()
    th.join()
    reads = []
    for text in texts:
        clocks, power = parse_smi_metric(text)
        if clocks:
            clocks.sort()
            n = len(clocks)
            med = clocks[n // 2] if n % 2 else 0.5 * (clocks[n // 2 - 1] + clocks[n // 2])
            reads.append({"gfx_mhz_median": med, "gfx_mhz_min": clocks[0], "gfx_mhz_max": clocks[-1],
                          "socket_power_w": power})
    if not reads:
        return None
    best = max(reads, key=lambda r: r["socket_power_w"] or 0.0)
    return dict(best, reads=reads, source="amd-smi metric -c -p while the step loop ran "
                                          "(the read at the highest socket power)")


def copy_calibration(mib):
    """One plain device-to-device copy of `mib` MiB, for scaling the HBM byte
    counters of a rocprofv3 --pmc pass over this process."""
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def time_ulysses_relayout(prob, U, reps=24, sets=6):
    """The four local steps of the Ulysses exchange on one rank's share of the
    Ulysses workload (its sequence shard of Q [B, N, S/U, D] and, in the
    inverse direction, a head shard [B, N/U, S, D] of the output): HIP-event
    time per call and the HBM rate counting every byte read once and written
    once. The calls rotate over `sets` independent buffer sets (6 x 96 MiB),
    more than the 256 MB Infinity Cache holds, so each call streams from HBM."""
    import torch
    from context_causal_attention_attn_amd import (head_to_seq_pack, head_to_seq_unpack, seq_to_head_pack,
                                                   seq_to_head_unpack)

    dev = torch.device("cuda")
    B, N, S, D = prob.q.shape
    L = S // U
    xs = [prob.q[:, :, :L].to(dev).contiguous() for _ in range(sets)]
    bs = [seq_to_head_pack(x, U) for x in xs]
    ys = [seq_to_head_unpack(b) for b in bs]
    steps = {"seq_to_head_pack": lambda i: seq_to_head_pack(xs[i], U, out=bs[i]),
             "seq_to_head_unpack": lambda i: seq_to_head_unpack(bs[i], out=ys[i]),
             "head_to_seq_pack": lambda i: head_to_seq_pack(ys[i], U, out=bs[i]),
             "head_to_seq_unpack": lambda i: head_to_seq_unpack(bs[i], out=xs[i])}
    x = xs[0]
    nbytes = 2 * x.numel() * x.element_size()
    res = {}
    for name, fn in steps.items():
        for i in range(sets):
            fn(i)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        ev[0].record()
        for i in range(reps):
            fn(i % sets)
        ev[1].record()
        torch.cuda.synchronize()
        ms = ev[0].elapsed_time(ev[1]) / reps
        gbs = nbytes / (ms * 1e-3) / 1e9
        res[name] = {"ms": round(ms, 4), "bytes": nbytes, "achieved": round(gbs, 1), "unit": "GB/s",
                     "bound": "hbm", "peak": PEAK_HBM_GBS, "frac": round(gbs / PEAK_HBM_GBS, 4)}
    return {"tensor": f"[{B}, {N}, {L}, {D}] <-> [{B}, {N // U}, {S}, {D}] {str(x.dtype).split('.')[-1]}, u = {U}",
            "steps": res}


CPU_SAMPLE = r"""
import json, math, os, sys, time
sys.path.insert(0, sys.argv[1])
import numpy as np
from threadpoolctl import threadpool_info
import oracle.cp_share as oc
from synthetic import workload
spec, prob = workload(sys.argv[2], seed=0)
rank = int(sys.argv[3])
kind, cp, U = spec["kind"], spec["cp"], spec.get("ulysses", 2)
S, Hq, Hkv, D = spec["seq"], spec["hq"], spec["hkv"], spec["head_dim"]
if kind == "contiguous":
    sh = oc.contiguous_share(S, Hq, Hkv, cp, rank)
elif kind == "head_tail":
    sh = oc.head_tail_share(S, Hq, Hkv, cp, rank)
elif kind == "ulysses":
    sh = oc.ulysses_share(S, Hq, Hkv, cp, rank)
else:
    sh = oc.hybrid_share(S, Hq, Hkv, cp, U, rank)
G = len(sh["q_heads"]) // len(sh["kv_heads"])
h, hk = int(sh["q_heads"][0]), int(sh["kv_heads"][0])
q = prob.q[:1, h:h + G].double().numpy()[:, :, sh["q_pos"]]
k = prob.k[:1, hk:hk + 1].double().numpy()
v = prob.v[:1, hk:hk + 1].double().numpy()
do = np.random.default_rng(0).standard_normal(q.shape)
t0 = time.perf_counter()
oc.attention_rows_bwd(q, k, v, do, sh["q_pos"], sh["kv_pos"], 1.0 / math.sqrt(D), True)
dt = time.perf_counter() - t0
pairs = oc.share_pairs(sh["q_pos"], sh["kv_pos"])
threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
print(json.dumps({"seconds": dt, "pairs": int(pairs), "G": G, "h": h, "hk": hk, "threads": threads,
                  "rows": int(len(sh["q_pos"])), "heads": int(len(sh["q_heads"]))}))
"""


def cpu_model_name():
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(spec, name, rank):
    """The oracle as it stands, on a bounded sample of the same share, in a
    child process of its own (NumPy fp64 with its BLAS threads over every CPU
    this process may run on): the query heads of the first GQA group (they
    read KV head 0), every local row, forward + backward (about 10 s on 16
    host threads). The child regenerates the seeded problem; only the oracle
    call is timed."""
    import subprocess
    D = spec["head_dim"]
    r = subprocess.run([sys.executable, "-c", CPU_SAMPLE, ROOT, name, str(rank)], capture_output=True,
                       text=True, timeout=600)
    if r.returncode != 0:
        return {"value": None, "error": r.stderr[-400:]}
    res = json.loads(r.stdout.strip().splitlines()[-1])
    flops = 14.0 * D * res["G"] * res["pairs"]   # forward (4D) + backward (10D) per visible pair and head
    dt = res["seconds"]
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": res["threads"], "kind": "oracle",
            "cpu_model": cpu_model_name(), "cpus_available": len(os.sched_getaffinity(0)),
            "sample": f"{spec['kind']} share rank {rank}: query heads {res['h']}..{res['h'] + res['G'] - 1} "
                      f"(the GQA group of KV head {res['hk']}; {res['G']} of {res['heads']}), all {res['rows']} "
                      f"local rows, forward+backward in fp64 NumPy in a child process; "
                      f"{dt:.1f} s for {flops / 1e9:.1f} causal-effective GFLOP",
            "seconds": dt}


# Every other share the workload list states a target for, timed on the
# default line after the headline share: (workload, ranks), plus the
# packed-sequence Colossal share. The Colossal, Head-Tail, Ulysses, Hybrid and
# packed shares are all cut from the same seeded B = 1 problem; the Head-Tail
# backward shares from their own B = 2 one.
CONFIG_SHARES = [
    ("head_tail_cp8_s32k_gqa32x8_d128", list(range(8))),
    ("ulysses_cp8_s32k_gqa32x8_d128", [0]),
    ("hybrid_u2_c4_s32k_gqa32x8_d128", [4]),
    ("head_tail_bwd_b2_cp8_s32k_gqa32x8_d128", [0, 7]),
    ("colossal_packed_cp8_r7_s32k_gqa32x8_d128", [7]),
]


def share_entry(rr):
    """Per-share timing record: forward and (when timed) backward, with the
    three backward kernels."""
    t, fl = rr["ms"], rr["flops"]

    def tf(f, ms):
        return f / (ms * 1e-3) / 1e12

    ent = {"fwd_ms": round(t["fwd"], 4), "fwd_tflops": round(tf(fl["fwd"], t["fwd"]), 2),
           "fwd_frac": round(tf(fl["fwd"], t["fwd"]) / PEAK_BF16_TFLOPS, 4)}
    if rr["has_bwd"]:
        btf = tf(fl["bwd"], t["bwd"])
        ent.update({"bwd_ms": round(t["bwd"], 4), "bwd_tflops": round(btf, 2),
                    "bwd_frac": round(btf / PEAK_BF16_TFLOPS, 4),
                    "dkdv_ms": round(t["dkdv"], 4), "dq_ms": round(t["dq"], 4),
                    "dkdv_frac": round(tf(fl["dkdv"], t["dkdv"]) / PEAK_BF16_TFLOPS, 4),
                    "dq_frac": round(tf(fl["dq"], t["dq"]) / PEAK_BF16_TFLOPS, 4)})
    return ent


def problem_key(sp):
    return (sp["batch"], sp["hq"], sp["hkv"], sp["seq"], sp["head_dim"], sp["dtype"])


def config_problems(shared):
    """The seeded global problems of CONFIG_SHARES (with dO), generated before
    any timing starts, so that no share is timed on a GPU that sat idle while
    the host drew its inputs; `shared` is (spec, problem) of the headline."""
    from synthetic import WORKLOADS, global_problem
    probs = {problem_key(shared[0]): shared[1]}
    for name, _ in CONFIG_SHARES:
        key = problem_key(WORKLOADS[name])
        if key not in probs:
            probs[key] = global_problem(*key, 0, with_dout=True)
    return probs


def time_configs(steps, warmup, probs):
    """Time every share of CONFIG_SHARES (forward and backward) after a
    0.3 s warm-up each."""
    from synthetic import WORKLOADS
    out = {}
    for name, ranks in CONFIG_SHARES:
        sp = dict(WORKLOADS[name])
        pr = probs[problem_key(sp)]
        for r in ranks:
            rr = time_share(sp, pr, r, steps, warmup, True, warm_s=0.3)
            out[f"{name}/r{r}"] = share_entry(rr)
            del rr
            if sp["kind"] == "ulysses":
                # The same share read straight from the all-to-all's blocks.
                rr = time_share(sp, pr, r, steps, warmup, True, warm_s=0.3, in_place=True)
                out[f"{name}/r{r}/in_place"] = share_entry(rr)
                del rr
    # The headline share under a user mask (FLOPs still counted over the causal
    # pairs: the kernels visit every causal tile whatever the mask hides).
    for kind in ("bool", "additive", "padding"):
        sp = dict(WORKLOADS[WORKLOAD])
        rr = time_share(sp, probs[problem_key(sp)], 7, steps, warmup, True, warm_s=0.3, user_mask=kind)
        out[f"{WORKLOAD}/r7/user_mask_{kind}"] = share_entry(rr)
        del rr
    bal = {}
    for name, ranks in CONFIG_SHARES:
        fw = [out[f"{name}/r{r}"]["fwd_ms"] for r in ranks]
        if len(fw) > 1:
            bal[name] = {"fwd_ms_min": min(fw), "fwd_ms_max": max(fw), "spread": round(max(fw) / min(fw) - 1.0, 4)}
            if all("bwd_ms" in out[f"{name}/r{r}"] for r in ranks):
                bw = [out[f"{name}/r{r}"]["bwd_ms"] for r in ranks]
                bal[name].update(bwd_ms_min=min(bw), bwd_ms_max=max(bw),
                                 bwd_spread=round(max(bw) / min(bw) - 1.0, 4))
    return out, bal


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share; --gpus {args.gpus} is not supported: every share "
              "runs on one GPU with the gathered K/V as an input, and this library runs no collective."
              , file=sys.stderr)
        sys.exit(2)
    import torch

    from context_causal_attention_attn_amd import build as b
    if not b.is_current():
        b.build()
    from context_causal_attention_attn_amd import _lib
    from synthetic import WORKLOADS, workload

    _lib.load()
    if args.relayout_only:
        usp, upr = workload("ulysses_cp8_s32k_gqa32x8_d128", seed=0)
        print(json.dumps({"ulysses_relayout": time_ulysses_relayout(upr, usp["cp"])}), flush=True)
        if args.copy_calib_mib:
            copy_calibration(args.copy_calib_mib)
        return
    spec, prob = workload(args.workload, seed=0)
    if prob.dout is None:
        from synthetic import global_problem
        prob = global_problem(spec["batch"], spec["hq"], spec["hkv"], spec["seq"], spec["head_dim"],
                              spec["dtype"], 0, with_dout=True)
    rank = spec["ranks"][0] if args.rank is None else args.rank
    if not 0 <= rank < spec["cp"]:
        print(f"--rank {rank} is outside 0..{spec['cp'] - 1} for {args.workload}", file=sys.stderr)
        sys.exit(2)
    configs = not args.no_configs and args.workload == WORKLOAD
    probs = config_problems((spec, prob)) if configs else None
    # The W warm-up steps run after at least args.warm_s seconds of the same
    # step, so the timed steps see the clocks of a busy GPU, not of one that
    # idled while the host drew the inputs.
    res = time_share(spec, prob, rank, args.steps, args.warmup, True, args.kv_order, warm_s=args.warm_s)
    ms, fl, io = res["ms"], res["flops"], res["bytes"]
    ms_per_step = res["total_ms"] / args.steps
    flops_step = fl["fwd"] + (fl["bwd"] if res["has_bwd"] else 0.0)
    value = flops_step / (ms_per_step * 1e-3) / 1e12

    def tf(f, t):
        return f / (t * 1e-3) / 1e12

    kernels = {}
    for part in ("fwd", "pre", "dkdv", "dq"):
        if part not in ms:
            continue
        ent = {"kernel": kernel_name(part, spec, args.kv_order), "ms": round(ms[part], 4)}
        if part == "pre":
            gbs = io[part] / (ms[part] * 1e-3) / 1e9
            ent.update(bound="hbm", achieved=round(gbs, 1), unit="GB/s", peak=PEAK_HBM_GBS,
                       frac=round(gbs / PEAK_HBM_GBS, 4))
        else:
            a = tf(fl[part], ms[part])
            ent.update(bound="mfma", achieved=round(a, 2), unit="TFLOP/s", peak=PEAK_BF16_TFLOPS,
                       frac=round(a / PEAK_BF16_TFLOPS, 4))
        ent["algorithmic_bytes"] = io[part]
        kernels[part] = ent
    dom = max(kernels, key=lambda p: ms[p])
    # The committed counter summaries were measured on the Colossal cp=8 rank-7
    # share in natural order: other shares report no traffic.
    measured = (args.workload, rank, args.kv_order) == ("colossal_cp8_r7_s32k_gqa32x8_d128", 7, "natural")
    tr = traffic_record(dom) if measured else None
    roof = dict(kernels[dom])
    roof["traffic"] = (tr["fetch_bytes"] + tr["write_bytes"]) if tr else None
    if tr:
        roof["traffic_detail"] = tr
    roof["flops_per_launch"] = fl.get(dom)
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
                   "rank": rank, "batch": spec["batch"], "hq": spec["hq"], "hkv": spec["hkv"],
                   "head_dim": spec["head_dim"], "seq_global": spec["seq"], "sq_local": res["sq"],
                   "causal_pairs_per_head": res["pairs"],
                   "passes": "fwd+bwd" if res["has_bwd"] else "fwd",
                   **({"kv_order": args.kv_order} if args.kv_order != "natural" else {}),
                   **({"packed_sequences": len(spec["doc_lengths"])} if spec.get("doc_lengths") else {})},
        "fwd": {"ms": round(ms["fwd"], 4), "tflops": round(tf(fl["fwd"], ms["fwd"]), 2),
                "frac_of_peak": round(tf(fl["fwd"], ms["fwd"]) / PEAK_BF16_TFLOPS, 4)},
        "bwd": ({"ms": round(ms["bwd"], 4), "tflops": round(tf(fl["bwd"], ms["bwd"]), 2),
                 "frac_of_peak": round(tf(fl["bwd"], ms["bwd"]) / PEAK_BF16_TFLOPS, 4)}
                if res["has_bwd"] else None),
        "roofline": roof,
        "kernels": kernels,
        "device": torch.cuda.get_device_name(0),
        "peak_bf16_tflops": PEAK_BF16_TFLOPS,
        "warm_s": args.warm_s,
    }
    if not args.no_clock:
        clk = sample_clock(res["step"])
        line["clock"] = clk
    del res
    if configs:
        cfg, bal = time_configs(max(5, args.steps // 2), args.warmup, probs)
        del probs
        line["configs"] = cfg
        line["balance"] = bal
    if args.detail:
        detail = {}
        for name, sp in WORKLOADS.items():
            if sp["dtype"] != "bf16":
                continue
            bw = bool(sp.get("backward"))
            _, pr = workload(name, seed=0)
            # The Head-Tail backward shares also run with K/V in all-gather
            # order (16 KV chunks out of position order).
            orders = ["natural", "gathered"] if (bw and sp["kind"] == "head_tail") else ["natural"]
            for r, order in [(r, o) for r in sp["ranks"] for o in orders]:
                # Input generation leaves the GPU idle for seconds: warm it
                # back up for half a second before timing.
                rr = time_share(sp, pr, r, max(5, args.steps // 2), args.warmup, bw, order, warm_s=0.5)
                detail[f"{name}/r{r}" + ("" if order == "natural" else "/gathered_kv")] = share_entry(rr)
            del pr
        line["detail"] = detail
        usp, upr = workload("ulysses_cp8_s32k_gqa32x8_d128", seed=0)
        line["ulysses_relayout"] = time_ulysses_relayout(upr, usp["cp"])
        del upr
    if args.copy_calib_mib:
        copy_calibration(args.copy_calib_mib)
    del prob
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(spec, args.workload, rank)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
