"""Python binding of the C ABI (include/cp_attn.h), same names.

Argument marshalling only: shapes and strides are read from the tensors, the
descriptor is filled in, outputs are allocated with torch on the inputs'
device, and the call is enqueued on torch's current stream. Every step of the
attention itself runs in the HIP kernels of libcpattn.so.
"""
from __future__ import annotations

import ctypes
import math
from typing import Optional, Sequence

import torch

from . import _lib
from ._lib import CpAttnDesc, CpAttnPlanStats, check

_DT = {torch.bfloat16: _lib.DTYPE_BF16, torch.float32: _lib.DTYPE_FP32}


def cp_attn_share_positions(layout: str, s_global: int, cp_size: int, cp_rank: int):
    """Global start positions of a rank's query chunks and the chunk length."""
    lib = _lib.load()
    pos = (ctypes.c_int64 * 2)()
    n = ctypes.c_int32()
    length = ctypes.c_int64()
    check(lib.cp_attn_share_positions(_lib.LAYOUTS[layout], s_global, cp_size, cp_rank,
                                      pos, ctypes.byref(n), ctypes.byref(length)),
          "cp_attn_share_positions")
    return [pos[i] for i in range(n.value)], length.value


class _Desc:
    """A filled cp_attn_desc plus the host arrays it points to."""

    def __init__(self, *, dtype, batch, hq, hkv, head_dim, sq_local, skv, q_chunk_pos,
                 kv_chunk_pos, layout, causal, softmax_scale, q_strides, kv_strides, o_strides,
                 doc_starts=(), attn_mask=None, mask_strides=(0, 0, 0), chunk_strides=(0, 0, 0)):
        additive = attn_mask is not None and attn_mask.dtype == torch.float32
        self.qpos = (ctypes.c_int64 * max(1, len(q_chunk_pos)))(*q_chunk_pos)
        self.kvpos = (ctypes.c_int64 * max(1, len(kv_chunk_pos)))(*kv_chunk_pos)
        doc_starts = [int(x) for x in doc_starts]
        self.docs = (ctypes.c_int64 * max(1, len(doc_starts)))(*doc_starts)
        d = CpAttnDesc()
        d.abi_version = _lib.ABI_VERSION
        d.dtype = dtype
        d.batch, d.hq, d.hkv, d.head_dim = batch, hq, hkv, head_dim
        d.sq_local, d.skv = sq_local, skv
        d.n_q_chunks = len(q_chunk_pos)
        d.q_chunk_pos = ctypes.cast(self.qpos, ctypes.POINTER(ctypes.c_int64))
        d.n_kv_chunks = len(kv_chunk_pos)
        d.kv_chunk_pos = ctypes.cast(self.kvpos, ctypes.POINTER(ctypes.c_int64))
        d.layout = _lib.LAYOUTS[layout] if isinstance(layout, str) else int(layout)
        d.causal = int(bool(causal))
        d.softmax_scale = float(softmax_scale)
        for i in range(3):
            d.q_strides[i], d.kv_strides[i], d.o_strides[i] = q_strides[i], kv_strides[i], o_strides[i]
        d.n_docs = len(doc_starts)
        d.doc_starts = ctypes.cast(self.docs, ctypes.POINTER(ctypes.c_int64))
        self.mask = attn_mask   # keeps the tensor alive as long as the descriptor
        d.attn_mask = attn_mask.data_ptr() if attn_mask is not None else None
        for i in range(3):
            d.mask_strides[i] = int(mask_strides[i]) * (4 if additive else 1)   # elements -> bytes
        d.mask_additive = 1 if additive else 0
        for i in range(3):
            d.chunk_strides[i] = int(chunk_strides[i])
        self.desc = d

    def ref(self):
        return ctypes.byref(self.desc)


def _geom(t):
    """(batch, heads, rows, head_dim, (batch, head, row) strides, chunk stride,
    chunks) of a [batch, heads, rows, head_dim] tensor, or of a
    [chunks, batch, heads, rows per chunk, head_dim] one whose chunks lie
    stride(0) elements apart (e.g. the blocks a Ulysses all-to-all delivers)."""
    if t.dim() == 4:
        B, H, S, D = t.shape
        return B, H, S, D, tuple(t.stride()[:3]), 0, None
    if t.dim() == 5:
        C, B, H, L, D = t.shape
        return B, H, C * L, D, tuple(t.stride()[1:4]), t.stride(0), C
    raise ValueError("tensors must be [batch, heads, rows, head_dim] or [chunks, batch, heads, rows, head_dim]")


def _check_inputs(q, k, v):
    if q.dtype not in _DT or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must all be bfloat16 or all float32")
    if k.shape != v.shape or k.stride() != v.stride():
        raise ValueError("k and v must have the same shape and strides")
    gq, gk = _geom(q), _geom(k)
    if gq[0] != gk[0] or gq[3] != gk[3]:
        raise ValueError("q and k/v disagree on batch or head_dim")
    for t in (q, k, v):
        if t.stride(-1) != 1:
            raise ValueError("the head_dim axis must be contiguous")
        if not t.is_cuda:
            raise ValueError("tensors must be on the GPU")


def _mask_args(attn_mask, q, k):
    """A user attention mask as (tensor, byte strides): bool or uint8,
    [B or 1, Hq or 1, Sq, Skv] on q's device with the key dim contiguous;
    size-1 batch or head dims broadcast (stride 0)."""
    if attn_mask is None:
        return None, (0, 0, 0)
    if attn_mask.dtype not in (torch.bool, torch.uint8, torch.float32) or attn_mask.dim() != 4:
        raise ValueError("attn_mask must be a 4-D bool, uint8 or float32 (additive) tensor [B|1, Hq|1, Sq, Skv]")
    B, Hq, Sq = _geom(q)[:3]
    Skv = _geom(k)[2]
    if (attn_mask.shape[0] not in (1, B) or attn_mask.shape[1] not in (1, Hq) or attn_mask.shape[2] != Sq
            or attn_mask.shape[3] != Skv):
        raise ValueError(f"attn_mask shape {tuple(attn_mask.shape)} does not broadcast to {(B, Hq, Sq, Skv)}")
    if attn_mask.device != q.device or attn_mask.stride(3) != 1:
        raise ValueError("attn_mask must be on q's device with a contiguous key dim")
    st = tuple(0 if attn_mask.shape[i] == 1 else attn_mask.stride(i) for i in range(3))
    return attn_mask, st


def make_desc(q, k, v, o, q_chunk_pos: Sequence[int], kv_chunk_pos: Sequence[int],
              layout, causal: bool, softmax_scale: Optional[float], doc_starts: Sequence[int] = (),
              attn_mask=None) -> _Desc:
    """Descriptor of a share. q, k, v (and o, whose strides out, dout and dq
    share: a tensor, or a stride tuple of a 4-D one) are 4-D, or 5-D with
    their chunks stride(0) apart; a 5-D q or o needs one chunk per entry of
    q_chunk_pos, a 5-D k one per entry of kv_chunk_pos."""
    B, Hq, Sq, D, q_st, q_cs, q_nc = _geom(q)
    _, Hkv, Skv, _, kv_st, kv_cs, kv_nc = _geom(k)
    if isinstance(o, torch.Tensor):
        _, _, _, _, o_st, o_cs, o_nc = _geom(o)
    else:
        o_st, o_cs, o_nc = tuple(o)[:3], 0, None
    for n, want, what in ((q_nc, len(q_chunk_pos), "q"), (o_nc, len(q_chunk_pos), "out"),
                          (kv_nc, len(kv_chunk_pos), "k/v")):
        if n is not None and n != want:
            raise ValueError(f"a 5-D {what} has {n} chunks, its chunk table {want}")
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else softmax_scale
    m, mst = _mask_args(attn_mask, q, k)
    return _Desc(dtype=_DT.get(q.dtype, -1), batch=B, hq=Hq, hkv=Hkv, head_dim=D, sq_local=Sq, skv=Skv,
                 q_chunk_pos=list(q_chunk_pos), kv_chunk_pos=list(kv_chunk_pos), layout=layout,
                 causal=causal, softmax_scale=scale, q_strides=q_st, kv_strides=kv_st, o_strides=o_st,
                 doc_starts=doc_starts, attn_mask=m, mask_strides=mst, chunk_strides=(q_cs, kv_cs, o_cs))


def _stream_handle(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def cp_attn_validate(q, k, v, q_chunk_pos, *, layout="contiguous", kv_chunk_pos=(0,), causal=True,
                     softmax_scale=None, doc_starts=(), attn_mask=None) -> None:
    d = make_desc(q, k, v, q, q_chunk_pos, kv_chunk_pos, layout, causal, softmax_scale, doc_starts, attn_mask)
    check(_lib.load().cp_attn_validate(d.ref()), "cp_attn_validate")


def cp_attn_share_pairs(d: _Desc) -> int:
    out = ctypes.c_int64()
    check(_lib.load().cp_attn_share_pairs(d.ref(), ctypes.byref(out)), "cp_attn_share_pairs")
    return out.value


def cp_attn_workspace_bytes(d: _Desc, backward: bool) -> int:
    out = ctypes.c_size_t()
    check(_lib.load().cp_attn_workspace_bytes(d.ref(), int(bool(backward)), ctypes.byref(out)),
          "cp_attn_workspace_bytes")
    return out.value


def cp_attn_plan_stats_fwd(d: _Desc) -> dict:
    st = CpAttnPlanStats()
    check(_lib.load().cp_attn_plan_stats_fwd(d.ref(), ctypes.byref(st)), "cp_attn_plan_stats_fwd")
    return {name: getattr(st, name) for name, _ in CpAttnPlanStats._fields_}


def cp_attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, q_chunk_pos: Sequence[int], *,
                layout="contiguous", kv_chunk_pos: Sequence[int] = (0,), causal: bool = True,
                softmax_scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                lse: Optional[torch.Tensor] = None, doc_starts: Sequence[int] = (),
                attn_mask: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """Forward of one share: returns (out [B, Hq, Sq, D] in q's dtype, lse [B, Hq, Sq] float32).

    q is the local query shard (rows in chunk order), k/v the gathered K/V.
    q_chunk_pos gives each chunk's global start position (see
    cp_attn_share_positions). kv_chunk_pos gives the global start position of
    each of the equal KV chunks in storage order: (p0,) for keys in natural
    order from p0, or one entry per chunk for K/V in any chunk order (e.g. as
    an all-gather delivers them; chunk length a multiple of 128 then).
    doc_starts, if not empty, gives the global start positions of packed
    variable-length sequences (a global cu_seqlens without its final total):
    a key is then visible only to queries of its own sequence. attn_mask, if
    given, is a bool/uint8 [B|1, Hq|1, Sq, Skv] device tensor ANDed with the
    CP mask (True / nonzero: may attend), or a float32 one added to the scaled
    scores (-inf hides a key).

    q (and out) may also be 5-D [chunks, B, Hq, L, D], one chunk per entry of
    q_chunk_pos stride(0) apart (layout "chunked"), and k/v 5-D
    [chunks, B, Hkv, Lkv, D], one per entry of kv_chunk_pos: e.g. the blocks
    a Ulysses all-to-all delivers, read in place; out then defaults to q's
    shape, the layout the reverse exchange sends. lse is always [B, Hq, Sq].

    A bf16 share's attn_mask is first packed into a bit table in device
    memory: workspace, if given and large enough, holds it, else one is
    allocated.
    """
    lib = _lib.load()
    _check_inputs(q, k, v)
    B, Hq, Sq, D = _geom(q)[:4]
    if out is None:
        out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    if out.shape != q.shape or out.dtype != q.dtype or out.stride(-1) != 1 or out.device != q.device:
        raise ValueError("out must match q's shape, dtype and device, with a contiguous head_dim")
    if lse.shape != (B, Hq, Sq) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, Hq, Sq] tensor")
    d = make_desc(q, k, v, out, q_chunk_pos, kv_chunk_pos, layout, causal, softmax_scale, doc_starts,
                  attn_mask)
    need = cp_attn_workspace_bytes(d, False)
    ws_ptr, ws_bytes = None, 0
    if need > 0:
        if workspace is None or workspace.numel() * workspace.element_size() < need:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    check(lib.cp_attn_fwd(d.ref(), q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                          lse.data_ptr(), ws_ptr, ws_bytes, _stream_handle(q)), "cp_attn_fwd")
    return out, lse


def cp_attn_bwd(q, k, v, out, lse, dout, q_chunk_pos: Sequence[int], *, layout="contiguous",
                kv_chunk_pos: Sequence[int] = (0,), causal: bool = True,
                softmax_scale: Optional[float] = None, workspace: Optional[torch.Tensor] = None,
                grads: Optional[tuple] = None, doc_starts: Sequence[int] = (),
                attn_mask: Optional[torch.Tensor] = None):
    """Backward of one share: returns (dq in q's dtype, dk, dv float32 partials over the gathered K/V).

    grads, if given, is a (dq, dk, dv) triple of preallocated outputs: dq with
    out's shape and strides, dk/dv contiguous float32 [B, Hkv, Skv, D]. dk/dv
    rows follow the k/v rows (the KV chunk table's storage order). q, out,
    dout (and dq) may be 5-D chunked like in cp_attn_fwd, and so may k/v.
    """
    return _bwd(q, k, v, out, lse, dout, q_chunk_pos, layout, kv_chunk_pos, causal,
                softmax_scale, workspace, grads, None, doc_starts, attn_mask)


def cp_attn_bwd_timed(q, k, v, out, lse, dout, q_chunk_pos: Sequence[int], events, *,
                      layout="contiguous", kv_chunk_pos: Sequence[int] = (0,), causal: bool = True,
                      softmax_scale: Optional[float] = None, workspace: Optional[torch.Tensor] = None,
                      grads: Optional[tuple] = None, doc_starts: Sequence[int] = (),
                      attn_mask: Optional[torch.Tensor] = None):
    """cp_attn_bwd with four torch.cuda.Event (enable_timing=True) recorded by the
    library on the current stream around its phases (for bf16: Delta pass,
    dK/dV kernel, dQ kernel), so events[i].elapsed_time(events[i+1]) is phase i+1."""
    if len(events) != 4:
        raise ValueError("cp_attn_bwd_timed needs exactly four events")
    stream = torch.cuda.current_stream(q.device)
    for e in events:
        if not e.cuda_event:   # torch creates the HIP event on first record
            e.record(stream)
    handles = (ctypes.c_void_p * 4)(*[e.cuda_event for e in events])
    return _bwd(q, k, v, out, lse, dout, q_chunk_pos, layout, kv_chunk_pos, causal,
                softmax_scale, workspace, grads, handles, doc_starts, attn_mask)


def _bwd(q, k, v, out, lse, dout, q_chunk_pos, layout, kv_chunk_pos, causal, softmax_scale,
         workspace, grads, events, doc_starts=(), attn_mask=None):
    lib = _lib.load()
    _check_inputs(q, k, v)
    B, Hq, Sq, D = _geom(q)[:4]
    Hkv, Skv = _geom(k)[1:3]
    if dout.shape != q.shape or out.shape != q.shape or dout.dtype != q.dtype or out.dtype != q.dtype:
        raise ValueError("out and dout must match q's shape and dtype")
    if dout.stride() != out.stride() or out.stride(-1) != 1:
        out, dout = out.contiguous(), dout.contiguous()
    if lse.shape != (B, Hq, Sq) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, Hq, Sq] tensor")
    if grads is None:
        dq = torch.empty_strided(out.shape, out.stride(), dtype=q.dtype, device=q.device)
        dk = torch.empty((B, Hkv, Skv, D), dtype=torch.float32, device=q.device)
        dv = torch.empty((B, Hkv, Skv, D), dtype=torch.float32, device=q.device)
    else:
        dq, dk, dv = grads
        if dq.shape != q.shape or dq.dtype != q.dtype or dq.stride() != out.stride():
            raise ValueError("dq must match q's shape and dtype, with out's strides")
        for t in (dk, dv):
            if t.shape != (B, Hkv, Skv, D) or t.dtype != torch.float32 or not t.is_contiguous():
                raise ValueError("dk and dv must be contiguous float32 [B, Hkv, Skv, D] tensors")
    d = make_desc(q, k, v, out, q_chunk_pos, kv_chunk_pos, layout, causal, softmax_scale, doc_starts,
                  attn_mask)
    need = cp_attn_workspace_bytes(d, True)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    args = (d.ref(), q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
            dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(),
            workspace.numel() * workspace.element_size(), _stream_handle(q))
    if events is None:
        check(lib.cp_attn_bwd(*args), "cp_attn_bwd")
    else:
        check(lib.cp_attn_bwd_timed(*args, events, 4), "cp_attn_bwd_timed")
    return dq, dk, dv
