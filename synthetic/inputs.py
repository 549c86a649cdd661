"""Seeded global problems for one context-parallel attention share.

Every share in the tests and the benchmark is sliced out of ONE global problem
(Q, K, V and, for the backward pass, dO over the whole sequence), so that shares
of different ranks are mutually consistent and reassemble to the unsharded
problem. The generator below fixes the draw order and the value distribution:

* ``torch.Generator('cpu').manual_seed(seed)``;
* draw order: global Q ``[B, Hq, S, D]``, then K ``[B, Hkv, S, D]``, then V
  ``[B, Hkv, S, D]``, then dO ``[B, Hq, S, D]`` (only when asked for);
* values iid N(0, 1) in float32; for bfloat16 problems each value is rounded to
  the nearest bfloat16 (ties to even), which is what ``Tensor.to(torch.bfloat16)``
  does.

The workloads are the shapes of the context-parallel shares that the pages
describe (cp=8 contiguous all-gather shares, Head-Tail shares of 16 chunks of
2048 tokens, pure Ulysses and Ulysses x Colossal hybrid shares at S=32768, and a
tiny fp32 case). No dataset is involved: the inputs are synthetic by design.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import torch


@dataclass
class GlobalProblem:
    q: torch.Tensor                 # [B, Hq, S, D]
    k: torch.Tensor                 # [B, Hkv, S, D]
    v: torch.Tensor                 # [B, Hkv, S, D]
    dout: Optional[torch.Tensor]    # [B, Hq, S, D] or None
    dtype: str                      # "bf16" or "fp32"
    seed: int


def global_problem(batch: int, hq: int, hkv: int, seq: int, head_dim: int,
                   dtype: str = "bf16", seed: int = 0,
                   with_dout: bool = False) -> GlobalProblem:
    """Draw one global problem on the CPU with the fixed draw order above."""
    if dtype not in ("bf16", "fp32"):
        raise ValueError(f"dtype must be 'bf16' or 'fp32', got {dtype!r}")
    g = torch.Generator("cpu").manual_seed(seed)
    q = torch.randn(batch, hq, seq, head_dim, generator=g, dtype=torch.float32)
    k = torch.randn(batch, hkv, seq, head_dim, generator=g, dtype=torch.float32)
    v = torch.randn(batch, hkv, seq, head_dim, generator=g, dtype=torch.float32)
    dout = None
    if with_dout:
        dout = torch.randn(batch, hq, seq, head_dim, generator=g, dtype=torch.float32)
    if dtype == "bf16":
        q, k, v = q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)
        if dout is not None:
            dout = dout.to(torch.bfloat16)
    return GlobalProblem(q=q, k=k, v=v, dout=dout, dtype=dtype, seed=seed)


# Named workloads: the global problem plus how the share is cut from it.
# "kind" is one of contiguous / head_tail / ulysses / hybrid; the share is cut
# by the consumer (oracle or HIP side), each with its own slicing code.
WORKLOADS = {
    "tiny_fp32_contiguous_cp4_r1": dict(
        batch=1, hq=2, hkv=2, seq=256, head_dim=64, dtype="fp32",
        kind="contiguous", cp=4, ranks=[1]),
    "colossal_cp8_r7_s32k_gqa32x8_d128": dict(
        batch=1, hq=32, hkv=8, seq=32768, head_dim=128, dtype="bf16",
        kind="contiguous", cp=8, ranks=[7]),
    "head_tail_cp8_s32k_gqa32x8_d128": dict(
        batch=1, hq=32, hkv=8, seq=32768, head_dim=128, dtype="bf16",
        kind="head_tail", cp=8, ranks=list(range(8))),
    "ulysses_cp8_s32k_gqa32x8_d128": dict(
        batch=1, hq=32, hkv=8, seq=32768, head_dim=128, dtype="bf16",
        kind="ulysses", cp=8, ranks=[0]),
    "hybrid_u2_c4_s32k_gqa32x8_d128": dict(
        batch=1, hq=32, hkv=8, seq=32768, head_dim=128, dtype="bf16",
        kind="hybrid", cp=8, ulysses=2, ranks=[4]),   # co_rank 2, u_rank 0
    "head_tail_bwd_b2_cp8_s32k_gqa32x8_d128": dict(
        batch=2, hq=32, hkv=8, seq=32768, head_dim=128, dtype="bf16",
        kind="head_tail", cp=8, ranks=[0, 7], backward=True),
    # Eight packed sequences over the 32K tokens (a global cu_seqlens), with a
    # length mix after the FLA CP tests: sequences cut by rank boundaries,
    # boundaries on rank boundaries, one sequence over two ranks.
    "colossal_packed_cp8_r7_s32k_gqa32x8_d128": dict(
        batch=1, hq=32, hkv=8, seq=32768, head_dim=128, dtype="bf16",
        kind="contiguous", cp=8, ranks=[7], backward=True,
        doc_lengths=[3000, 4000, 3240, 5120, 5120, 7000, 3240, 2048]),
}


def doc_starts(spec: dict) -> list:
    """Global start positions of a workload's packed sequences ([] for one sequence)."""
    lengths = spec.get("doc_lengths")
    if not lengths:
        return []
    out, pos = [], 0
    for n in lengths:
        out.append(pos)
        pos += n
    return out


def workload(name: str, seed: int = 0) -> tuple[dict, GlobalProblem]:
    spec = dict(WORKLOADS[name])
    prob = global_problem(spec["batch"], spec["hq"], spec["hkv"], spec["seq"],
                          spec["head_dim"], spec["dtype"], seed,
                          with_dout=spec.get("backward", False))
    return spec, prob
