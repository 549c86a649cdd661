"""Shared helpers of the GPU parity tests: cut shares on both sides of the
parity check, each side with its own code (the oracle's share builders on the
CPU side, the package's cut_share on the HIP side), from one seeded global
problem."""
import math

import numpy as np
import torch

import oracle.cp_share as oc
from context_causal_attention_attn_amd import cut_share
from synthetic import global_problem


def oracle_share(kind, S, Hq, Hkv, cp, rank, U=2):
    if kind == "contiguous":
        return oc.contiguous_share(S, Hq, Hkv, cp, rank)
    if kind == "head_tail":
        return oc.head_tail_share(S, Hq, Hkv, cp, rank)
    if kind == "ulysses":
        return oc.ulysses_share(S, Hq, Hkv, cp, rank)
    if kind == "hybrid":
        return oc.hybrid_share(S, Hq, Hkv, cp, U, rank)
    raise ValueError(kind)


def gathered_key_rows(kind, S, cp, U=2):
    """Global key rows in the order a K/V all-gather delivers them, from the
    oracle's own chunk geometry: rank after rank of the gathering group (all
    CP ranks, or the Colossal sub-group of a Hybrid share), each rank's chunks
    in its local order. The global problem is in natural order, so a row
    index is also the key's global position."""
    group, layout = (cp // U, "contiguous") if kind == "hybrid" else (cp, kind)
    parts = []
    for r in range(group):
        pos, n = oc.share_chunks(layout, S, group, r)
        parts += [np.arange(p, p + n, dtype=np.int64) for p in pos]
    return np.concatenate(parts)


def to_f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def oracle_rows(prob, sh, scale, rows=None, heads=None, causal=True, key_rows=None):
    """Oracle out/lse of a share, optionally only for some local rows/heads.
    key_rows, if given, lists the global key rows in storage order (the keys
    and their positions are taken in that order). Returns arrays indexed
    [b, local_head, local_row]."""
    q = prob.q[:, sh["q_heads"]]
    q_pos = sh["q_pos"]
    qsel = q[:, :, torch.from_numpy(q_pos)]
    k = prob.k[:, sh["kv_heads"]]
    v = prob.v[:, sh["kv_heads"]]
    kv_pos = sh["kv_pos"]
    if key_rows is not None:
        k, v, kv_pos = k[:, :, torch.from_numpy(key_rows)], v[:, :, torch.from_numpy(key_rows)], kv_pos[key_rows]
    hq_loc = len(sh["q_heads"])
    G = hq_loc // len(sh["kv_heads"])
    heads = list(range(hq_loc)) if heads is None else list(heads)
    rows = np.arange(len(q_pos)) if rows is None else np.asarray(rows)
    outs, lses = [], []
    for h in heads:
        hk = h // G
        o, l = oc.attention_rows(to_f64(qsel[:, h:h + 1, torch.from_numpy(rows)]),
                                 to_f64(k[:, hk:hk + 1]), to_f64(v[:, hk:hk + 1]),
                                 q_pos[rows], kv_pos, scale, causal)
        outs.append(o[:, 0])
        lses.append(l[:, 0])
    return np.stack(outs, 1), np.stack(lses, 1)


def spiked_problem(seed=7, with_dout=False):
    """A 1024-token bf16 problem whose keys 600..615 are scaled by 30. Rows
    after them meet scores tens of log2 units above (and below) everything in
    their earlier key tiles, so the forward's running reference must be
    replaced, and O rescaled, on a tile after the first; the backward sees
    rows whose LSE is dominated by a few keys."""
    prob = global_problem(1, 4, 2, 1024, 128, dtype="bf16", seed=seed, with_dout=with_dout)
    k = prob.k.float()
    k[:, :, 600:616] *= 30.0
    prob.k = k.to(torch.bfloat16)
    return prob
