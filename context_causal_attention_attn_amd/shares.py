"""Cut one CP rank's share out of a global (unsharded) problem, HIP side.

This stands in for the collectives that would deliver a rank's inputs
(all-gather of K/V, the Ulysses all-to-all), which a single GPU does not run:
it selects the rank's heads and query rows from global tensors and returns
the chunk table the kernels need. Positions come from the library's own
cp_attn_share_positions.

  contiguous : all heads, rows [r*S/P, (r+1)*S/P)          ("新流程 CP 多通信模式迁移设计方案" §6.1, §8)
  head_tail  : all heads, rows of chunk r then chunk 2P-1-r ("HyperModels 新 Trainer Context Parallel 接入设计方案" §4.4)
  ulysses    : heads [r*H/P, (r+1)*H/P) of Q and K/V, all rows, offset 0   (§6.2)
  hybrid     : P = C*U, co = r // U, u = r % U: heads [u*H/U, ...), rows [co*S/C, ...)  (§6.3)

K/V come in natural order (one KV chunk at position 0) or, with
kv_order="gathered", in the order an all-gather over the CP group delivers
them: rank after rank, each rank's own chunks in its local order (Head-Tail:
chunks 0, 2P-1, 1, 2P-2, ...; "HyperModels 新 Trainer Context Parallel 接入设计方案"
§4.4 zigzag order), with the matching KV chunk table.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List

import torch

from .api import cp_attn_share_positions


@dataclass
class Share:
    q: torch.Tensor            # [B, hq_local, sq_local, D] (a view, or a copy for head_tail)
    k: torch.Tensor            # [B, hkv_local, S, D] view
    v: torch.Tensor
    q_heads: List[int]         # global head indices of the local query heads
    kv_heads: List[int]
    rows: List[List[int]]      # [start, stop) of each local chunk in the global sequence
    q_chunk_pos: List[int]
    layout: str                # "contiguous" or "head_tail" (the kernel layout)
    kv_chunk_pos: List[int] = None   # global position of each KV chunk (storage order)

    def __post_init__(self):
        if self.kv_chunk_pos is None:
            self.kv_chunk_pos = [0]

    def kv_positions(self) -> List[int]:
        """Global position of every K/V row, in storage order."""
        n = self.k.shape[2] // len(self.kv_chunk_pos)
        return [p + i for p in self.kv_chunk_pos for i in range(n)]

    def take_rows(self, t: torch.Tensor) -> torch.Tensor:
        """The same rows/heads of another query-shaped global tensor (e.g. dO)."""
        t = t[:, self.q_heads[0]:self.q_heads[-1] + 1]
        parts = [t[:, :, a:b] for a, b in self.rows]
        return parts[0] if len(parts) == 1 else torch.cat(parts, dim=2)


def cut_share(kind: str, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cp: int, rank: int,
              ulysses: int = 1, kv_order: str = "natural") -> Share:
    if kv_order not in ("natural", "gathered"):
        raise ValueError(f"kv_order must be 'natural' or 'gathered', got {kv_order!r}")
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    if kind in ("contiguous", "head_tail"):
        pos, n = cp_attn_share_positions(kind, S, cp, rank)
        qh, kh = list(range(Hq)), list(range(Hkv))
        layout = kind
    elif kind == "ulysses":
        if Hq % cp or Hkv % cp:
            raise ValueError("Ulysses needs Hq and Hkv divisible by the Ulysses degree")
        qh = list(range(rank * Hq // cp, (rank + 1) * Hq // cp))
        kh = list(range(rank * Hkv // cp, (rank + 1) * Hkv // cp))
        pos, n, layout = [0], S, "contiguous"
    elif kind == "hybrid":
        if not (1 < ulysses < cp) or cp % ulysses:
            raise ValueError("Hybrid needs 1 < U < P and P % U == 0")
        if Hq % ulysses or Hkv % ulysses:
            raise ValueError("Hybrid needs Hq and Hkv divisible by the Ulysses degree")
        c = cp // ulysses
        co, u = rank // ulysses, rank % ulysses
        pos, n = cp_attn_share_positions("contiguous", S, c, co)
        qh = list(range(u * Hq // ulysses, (u + 1) * Hq // ulysses))
        kh = list(range(u * Hkv // ulysses, (u + 1) * Hkv // ulysses))
        layout = "contiguous"
    else:
        raise ValueError(f"unknown share kind {kind!r}")
    rows = [[p, p + n] for p in pos]
    qs = q[:, qh[0]:qh[-1] + 1]
    parts = [qs[:, :, a:b] for a, b in rows]
    qloc = parts[0] if len(parts) == 1 else torch.cat(parts, dim=2)
    kloc, vloc = k[:, kh[0]:kh[-1] + 1], v[:, kh[0]:kh[-1] + 1]
    kv_pos = [0]
    if kv_order == "gathered":
        if kind == "ulysses":
            raise ValueError("a Ulysses share holds the whole sequence: there is no K/V all-gather")
        # The group whose K/V shards are gathered: every CP rank (contiguous,
        # head_tail) or the Colossal sub-group of the Hybrid share.
        group, lay = (cp // ulysses, "contiguous") if kind == "hybrid" else (cp, kind)
        kv_pos = []
        for r in range(group):
            kv_pos += cp_attn_share_positions(lay, S, group, r)[0]
        n_kv = S // len(kv_pos)
        if kv_pos != sorted(kv_pos):
            kloc = torch.cat([kloc[:, :, p:p + n_kv] for p in kv_pos], dim=2)
            vloc = torch.cat([vloc[:, :, p:p + n_kv] for p in kv_pos], dim=2)
    return Share(q=qloc, k=kloc, v=vloc, q_heads=qh, kv_heads=kh,
                 rows=rows, q_chunk_pos=list(pos), layout=layout, kv_chunk_pos=kv_pos)
