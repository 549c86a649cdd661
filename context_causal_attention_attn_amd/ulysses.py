"""The Ulysses exchange's local steps, same names as the C ABI's
cp_attn_ulysses_relayout steps ("新流程 CP 多通信模式迁移设计方案" §6.2: Q/K/V
[B, N, S/P, D] are split by head and all-to-all'd into [B, N/P, S, D]; the
output returns by the inverse exchange; §6.3 runs it inside the Hybrid's
Ulysses sub-group).

    x       [B, u*H, L, D]   a rank's sequence shard (every head)
    y       [B, H, u*L, D]   its head shard over the group's sequence
    blocks  [u, B, H, L, D]  block p goes to (pack) / came from (unpack) rank p

An all_to_all_single over the group (not part of this package) moves block p of
every rank's packed buffer to rank p. These functions only marshal arguments;
every copy runs in the library's kernel.

The share kernels can also take the received blocks as they are
(`ulysses_fwd_in_place`, `ulysses_bwd_in_place`): block p holds sequence rows
p*L .. p*L+L-1 of the head shard, so it is query (and key) chunk p of a
"chunked" share, and the output comes back in the blocks layout the reverse
exchange sends. No unpack or pack pass runs around the attention.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import _lib
from .api import _stream_handle, cp_attn_bwd, cp_attn_fwd

_DTYPES = {torch.bfloat16: _lib.DTYPE_BF16, torch.float32: _lib.DTYPE_FP32}


def cp_attn_ulysses_relayout(step: str, src: torch.Tensor, dst: torch.Tensor, side: torch.Tensor, u: int, heads: int,
                             rows: int) -> None:
    """One step of the exchange (same name as the C entry point): `side` is
    the x or y tensor the step names (its strides are passed), the other of
    src/dst is the contiguous blocks tensor."""
    if src.dtype != dst.dtype or src.dtype not in _DTYPES:
        raise ValueError("src and dst must both be bfloat16 or both float32")
    if src.device != dst.device or src.device.type != "cuda":
        raise ValueError("src and dst must be on the same GPU")
    if side.stride(3) != 1:
        raise ValueError("head_dim must be contiguous")
    st = (ctypes.c_int64 * 3)(side.stride(0), side.stride(1), side.stride(2))
    lib = _lib.load()
    _lib.check(lib.cp_attn_ulysses_relayout(_lib.ULYSSES_STEPS[step], _DTYPES[src.dtype], u, side.shape[0],
                                            heads, rows, side.shape[3], src.data_ptr(), dst.data_ptr(), st,
                                            _stream_handle(src)), f"cp_attn_ulysses_relayout({step})")


def _blocks_for(t: torch.Tensor, u: int, heads: int, rows: int, out: Optional[torch.Tensor]) -> torch.Tensor:
    shape = (u, t.shape[0], heads, rows, t.shape[3])
    if out is None:
        return torch.empty(shape, dtype=t.dtype, device=t.device)
    if tuple(out.shape) != shape or out.dtype != t.dtype or not out.is_contiguous():
        raise ValueError(f"blocks must be a contiguous {shape} tensor of {t.dtype}")
    return out


def seq_to_head_pack(x: torch.Tensor, u: int, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """x [B, u*H, L, D] -> blocks [u, B, H, L, D] (block p: heads p*H .. of x)."""
    B, N, L, D = x.shape
    if N % u:
        raise ValueError("the head count must divide by the Ulysses degree")
    blocks = _blocks_for(x, u, N // u, L, out)
    cp_attn_ulysses_relayout("seq_to_head_pack", x, blocks, x, u, N // u, L)
    return blocks


def seq_to_head_unpack(blocks: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Received blocks [u, B, H, L, D] (block p from rank p) -> y [B, H, u*L, D]."""
    u, B, H, L, D = blocks.shape
    if not blocks.is_contiguous():
        raise ValueError("blocks must be contiguous")
    y = torch.empty((B, H, u * L, D), dtype=blocks.dtype, device=blocks.device) if out is None else out
    if tuple(y.shape) != (B, H, u * L, D) or y.dtype != blocks.dtype:
        raise ValueError("out must be a [B, H, u*L, D] tensor of the blocks' dtype")
    cp_attn_ulysses_relayout("seq_to_head_unpack", blocks, y, y, u, H, L)
    return y


def head_to_seq_pack(y: torch.Tensor, u: int, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y [B, H, u*L, D] -> blocks [u, B, H, L, D] (block p: rows p*L .. of y)."""
    B, H, S, D = y.shape
    if S % u:
        raise ValueError("the sequence length must divide by the Ulysses degree")
    blocks = _blocks_for(y, u, H, S // u, out)
    cp_attn_ulysses_relayout("head_to_seq_pack", y, blocks, y, u, H, S // u)
    return blocks


def head_to_seq_unpack(blocks: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Received blocks [u, B, H, L, D] (block p from rank p) -> x [B, u*H, L, D]."""
    u, B, H, L, D = blocks.shape
    if not blocks.is_contiguous():
        raise ValueError("blocks must be contiguous")
    x = torch.empty((B, u * H, L, D), dtype=blocks.dtype, device=blocks.device) if out is None else out
    if tuple(x.shape) != (B, u * H, L, D) or x.dtype != blocks.dtype:
        raise ValueError("out must be a [B, u*H, L, D] tensor of the blocks' dtype")
    cp_attn_ulysses_relayout("head_to_seq_unpack", blocks, x, x, u, H, L)
    return x


def _chunk_pos(blocks: torch.Tensor, offset: int):
    return [offset + p * blocks.shape[3] for p in range(blocks.shape[0])]


def ulysses_fwd_in_place(qb: torch.Tensor, kb: torch.Tensor, vb: torch.Tensor, *, causal: bool = True,
                         softmax_scale: Optional[float] = None, q_offset: int = 0, kv_offset: int = 0,
                         out: Optional[torch.Tensor] = None):
    """Forward of a Ulysses head shard read straight from the received blocks
    qb [u, B, H, L, D] and kb, vb [u, B, Hkv, L, D] (block p: sequence rows
    p*L.., global positions offset + p*L..; with several K/V blocks, L a
    multiple of 128). Returns (out [u, B, H, L, D], the blocks the head->seq
    exchange sends, and lse [B, H, u*L])."""
    return cp_attn_fwd(qb, kb, vb, _chunk_pos(qb, q_offset), layout="chunked", kv_chunk_pos=_chunk_pos(kb, kv_offset),
                       causal=causal, softmax_scale=softmax_scale, out=out)


def ulysses_bwd_in_place(qb, kb, vb, outb, lse, doutb, *, causal: bool = True,
                         softmax_scale: Optional[float] = None, q_offset: int = 0, kv_offset: int = 0):
    """Backward of the same share from blocks: returns (dq [u, B, H, L, D] in
    the blocks layout, dk, dv float32 [B, Hkv, u*L, D] in sequence order)."""
    return cp_attn_bwd(qb, kb, vb, outb, lse, doutb, _chunk_pos(qb, q_offset), layout="chunked",
                       kv_chunk_pos=_chunk_pos(kb, kv_offset), causal=causal, softmax_scale=softmax_scale)
