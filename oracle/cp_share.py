"""TEST INFRASTRUCTURE ONLY -- the fp64 CPU oracle of one context-parallel (CP)
rank's causal attention share.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module. It is plain NumPy in float64, written from
the definitions on the source pages; it shares no code, header, table or helper
with the HIP library and never imports it.

Sources (page title, then the section used):

* [CP-migration] "新流程 CP 多通信模式迁移设计方案" (hyper-parallel issue 7):
  §6.1 AllGather / Pure Colossal, §6.2 Pure Ulysses, §6.3 Hybrid, §8 Causal
  mask (the offset table), §9.1 TP + Ulysses, §9.2 GQA/MQA, §9.3 Layout.
* [Trainer-CP] "HyperModels 新 Trainer Context Parallel 接入设计方案"
  (hyper-parallel issue 324): §0 terms (Head-Tail load balance), §4.2 padding
  policy, §4.3 the three synchronous strategies, §4.4 Async and load balance.
* [FLA-CP] "flash-linear-attention 上下文并行CP 从 CP2TP、Ring CP 到 True CP
  的设计取舍与源码实现": §3.2 FLACPContext (contiguous vs zigzag layout), §3.3
  hard constraints of the partitioner.

The pages never write the attention formula itself; they call a scaled
dot-product attention primitive. The oracle takes the plain reading: softmax of
``scale * q.k`` over the visible keys, weights applied to ``v``, with the
log-sum-exp (natural log, of the scaled scores) returned beside the output.

Parity pins (tests/test_oracle_pins.py): every function below is pinned by at
least one check that does not re-run its own arithmetic -- brute-force Python
loops, torch's float64 SDPA, closed forms, reassembly of all rank shares into
the unsharded result, and central finite differences for the backward pass.
No function here is "parity unpinned".
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

__all__ = [
    "kv_head_of", "visible", "share_chunks", "chunk_row_positions",
    "attention_rows", "attention_rows_bwd", "contiguous_share",
    "head_tail_share", "ulysses_share", "hybrid_share", "share_pairs",
    "ulysses_seq_to_head", "ulysses_head_to_seq", "doc_of",
]


# Reading of the additive user mask ([CP-migration] §8: a float attn_mask is
# added to the scores and hidden keys get -inf): padding masks write "hidden"
# as -inf or as a large negative number (-1e4, -1e9, the float32 minimum).
# Values at or below MASK_HIDE hide their key exactly like -inf; values above
# it are biases added to the scaled score.
MASK_HIDE = -1.0e4


# ----------------------------------------------------------------------------
# Head mapping and visibility
# ----------------------------------------------------------------------------
def kv_head_of(hq: int, n_q_heads: int, n_kv_heads: int) -> int:
    """KV head read by query head ``hq`` under GQA/MQA.

    [CP-migration] §9.2 requires Q and KV head counts to divide separately and
    forbids silently repeating KV heads. The grouping is contiguous: query
    heads ``[g*G, (g+1)*G)`` read KV head ``g`` with ``G = Hq / Hkv``; this is
    the only grouping under which a head slice taken by the Ulysses all-to-all
    ([CP-migration] §6.2) stays a self-contained set of groups.
    """
    if n_q_heads % n_kv_heads != 0:
        raise ValueError("GQA needs Hq % Hkv == 0")
    return hq // (n_q_heads // n_kv_heads)


def doc_of(pos: np.ndarray, doc_starts: Sequence[int]) -> np.ndarray:
    """Index of the packed sequence (document) holding each global position:
    the sequences start at ``doc_starts`` (a global cu_seqlens without its
    final total, [FLA-CP] §3.1), each running up to the next start. Positions
    before the first start form document -1."""
    return np.searchsorted(np.asarray(doc_starts, dtype=np.int64), np.asarray(pos, dtype=np.int64),
                           side="right") - 1


def visible(q_pos: np.ndarray, kv_pos: np.ndarray, causal: bool,
            doc_starts: Optional[Sequence[int]] = None) -> np.ndarray:
    """Boolean [Sq, Skv]: may the query at global position q_pos[i] see the key
    at global position kv_pos[j]?

    [CP-migration] §8: the causal mask compares GLOBAL token positions (each
    strategy supplies the global start of its local Q range); a key is visible
    when its position is not after the query's, the diagonal included, as in
    standard ``is_causal`` attention which Ulysses keeps unchanged. Without the
    causal flag every key is visible.

    With ``doc_starts`` (packed variable-length sequences, [FLA-CP] §3.1 and
    §3.3: a global cu_seqlens partitioned across ranks) a key must also lie in
    the query's own sequence: each sequence is causal attention on its own.
    """
    q_pos = np.asarray(q_pos, dtype=np.int64)
    kv_pos = np.asarray(kv_pos, dtype=np.int64)
    if not causal:
        if doc_starts is not None:
            raise ValueError("packed sequences are defined for causal attention only")
        return np.ones((q_pos.size, kv_pos.size), dtype=bool)
    vis = kv_pos[None, :] <= q_pos[:, None]
    if doc_starts is not None:
        vis &= doc_of(kv_pos, doc_starts)[None, :] == doc_of(q_pos, doc_starts)[:, None]
    return vis


# ----------------------------------------------------------------------------
# Share geometry
# ----------------------------------------------------------------------------
def share_chunks(layout: str, s_global: int, cp_size: int, cp_rank: int):
    """Global start positions of a rank's local Q chunks, and the chunk length.

    * ``contiguous``: one chunk ``[r*S/P, (r+1)*S/P)`` -- the all-gather offset
      ``cp_rank * q_len`` of [CP-migration] §8 and the contiguous layout of
      [FLA-CP] §3.2. Needs ``S % P == 0`` ([Trainer-CP] §4.2).
    * ``head_tail``: the sequence is cut into 2P equal chunks and rank r holds
      chunk r (front) followed by chunk 2P-1-r (back), concatenated as
      ``[front; back]`` ([FLA-CP] §3.2 zigzag; [Trainer-CP] §0 and §4.4: each
      Q half keeps its own global interval, [CP-migration] §8 last row). Needs
      ``S % 2P == 0`` ([Trainer-CP] §4.2; [FLA-CP] §3.3).
    """
    if cp_size < 1 or not (0 <= cp_rank < cp_size):
        raise ValueError("need cp_size >= 1 and 0 <= cp_rank < cp_size")
    if layout == "contiguous":
        if s_global % cp_size:
            raise ValueError("contiguous layout needs S divisible by cp_size")
        n = s_global // cp_size
        return [cp_rank * n], n
    if layout == "head_tail":
        if s_global % (2 * cp_size):
            raise ValueError("head_tail layout needs S divisible by 2*cp_size")
        n = s_global // (2 * cp_size)
        return [cp_rank * n, (2 * cp_size - 1 - cp_rank) * n], n
    raise ValueError(f"unknown layout {layout!r}")


def chunk_row_positions(chunk_pos: Sequence[int], chunk_len: int) -> np.ndarray:
    """Global position of every local row: the chunks laid end to end in the
    order given, row t of chunk c at ``chunk_pos[c] + t``."""
    return np.concatenate([np.arange(p, p + chunk_len, dtype=np.int64)
                           for p in chunk_pos]) if len(chunk_pos) else np.zeros(0, np.int64)


# ----------------------------------------------------------------------------
# Forward
# ----------------------------------------------------------------------------
def _as_f64(x) -> np.ndarray:
    if hasattr(x, "detach"):            # a torch tensor
        x = x.detach().to("cpu")
        import torch
        x = x.to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def attention_rows(q, k, v, q_pos, kv_pos, scale: float, causal: bool = True,
                   row_block: int = 1024, doc_starts: Optional[Sequence[int]] = None,
                   user_mask: Optional[np.ndarray] = None):
    """Attention of local query rows against the gathered keys/values.

    q: [B, Hq, Sq, D]; k, v: [B, Hkv, Skv, D]; q_pos [Sq] and kv_pos [Skv] are
    global token positions. Returns (out [B, Hq, Sq, D], lse [B, Hq, Sq]) in
    float64.

    This is the Attention(Q_local, K_global, V_global) call of [CP-migration]
    §6.1 (and of §6.2/§6.3 on head-sliced inputs), with the global-position mask
    of §8. Per row i, over its visible set A_i:
        s_ij  = scale * sum_d q[i, d] k[j, d]
        LSE_i = ln sum_{j in A_i} exp(s_ij)      (with the row max subtracted)
        out_i = sum_{j in A_i} exp(s_ij - LSE_i) v_j
    A row with no visible key gets out = 0 and LSE = -inf. ``doc_starts``
    restricts A_i to the row's own packed sequence (see ``visible``).
    ``user_mask`` (broadcastable to [B, Hq, Sq, Skv]) is the caller's
    attention mask, merged with the CP mask and never replacing it
    ([CP-migration] §8): a boolean mask by logical AND (a key must be visible
    under both); a floating-point mask is additive (added to the scaled
    scores; a value at or below MASK_HIDE, -inf included, hides the key) and
    the CP mask hides what it hides. The LSE then includes the bias:
    LSE_i = ln sum_{j in A_i} exp(s_ij + mask_ij).

    Rows are independent, so they are visited in blocks of ``row_block`` only to
    bound memory; nothing is reordered within a row.
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    kv_pos = np.asarray(kv_pos, dtype=np.int64)
    B, Hq, Sq, D = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    assert k.shape == (B, Hkv, Skv, D) and v.shape == k.shape
    assert q_pos.shape == (Sq,) and kv_pos.shape == (Skv,)
    out = np.zeros((B, Hq, Sq, D))
    lse = np.full((B, Hq, Sq), -np.inf)
    for b in range(B):
        for h in range(Hq):
            hk = kv_head_of(h, Hq, Hkv)
            for r0 in range(0, Sq, row_block):
                r1 = min(Sq, r0 + row_block)
                vis = visible(q_pos[r0:r1], kv_pos, causal, doc_starts)
                s = scale * (q[b, h, r0:r1] @ k[b, hk].T)
                if user_mask is not None:
                    um = np.broadcast_to(user_mask, (B, Hq, Sq, Skv))[b, h, r0:r1]
                    if um.dtype == bool:
                        vis = vis & um
                    else:
                        hidden = um <= MASK_HIDE
                        s = s + np.where(hidden, 0.0, um)
                        vis = vis & ~hidden
                s = np.where(vis, s, -np.inf)
                m = s.max(axis=1)
                has = np.isfinite(m)
                m_safe = np.where(has, m, 0.0)
                w = np.exp(s - m_safe[:, None])          # exp(-inf) = 0 for hidden keys
                l = w.sum(axis=1)
                l_safe = np.where(has, l, 1.0)
                lse[b, h, r0:r1] = np.where(has, m_safe + np.log(l_safe), -np.inf)
                out[b, h, r0:r1] = (w / l_safe[:, None]) @ v[b, hk]
    return out, lse


# ----------------------------------------------------------------------------
# Backward
# ----------------------------------------------------------------------------
def attention_rows_bwd(q, k, v, dout, q_pos, kv_pos, scale: float,
                       causal: bool = True, kv_index: Optional[np.ndarray] = None,
                       row_block: int = 1024, want_dq: bool = True,
                       doc_starts: Optional[Sequence[int]] = None,
                       user_mask: Optional[np.ndarray] = None):
    """Gradients of ``sum(dout * out)`` for one share.

    Returns (dq [B, Hq, Sq, D], dk, dv) in float64, where dk/dv are this share's
    PARTIAL gradients over the gathered K/V ([B, Hkv, Skv, D], or only the rows
    listed in ``kv_index``). [CP-migration] §6.1 backward: dQ needs no CP
    communication, and the dK/dV of the global K/V are reduce-scattered (summed)
    over ranks, so each share contributes a partial sum; under GQA each KV head
    collects the sum over its group of query heads (§9.2).

    The pages only describe the communication around the primitive; the
    primitive's own gradient is the standard one of softmax attention:
        P_ij  = exp(s_ij - LSE_i) on visible pairs, else 0
        dV_j  = sum_i P_ij dout_i
        dP_ij = dout_i . v_j
        Delta_i = dout_i . out_i
        dS_ij = P_ij (dP_ij - Delta_i)
        dQ_i  = scale * sum_j dS_ij k_j
        dK_j  = scale * sum_i dS_ij q_i
    ``out`` and ``LSE`` are recomputed here in float64 with ``attention_rows``.
    Rows of dQ are independent of each other, so dQ of a subset of rows is
    obtained by passing only those rows; dK/dV need every row and are computed
    only for the keys in ``kv_index``. ``want_dq=False`` skips dQ (zeros).
    """
    q, k, v, dout = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(dout)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    kv_pos = np.asarray(kv_pos, dtype=np.int64)
    B, Hq, Sq, D = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    out, lse = attention_rows(q, k, v, q_pos, kv_pos, scale, causal, row_block, doc_starts, user_mask)
    sel = np.arange(Skv) if kv_index is None else np.asarray(kv_index, dtype=np.int64)
    dq = np.zeros_like(q)
    dk = np.zeros((B, Hkv, sel.size, D))
    dv = np.zeros((B, Hkv, sel.size, D))

    um_all = None if user_mask is None else np.broadcast_to(user_mask, (B, Hq, Sq, Skv))

    def grads(qb, dob, delta, lse_b, has, pos_b, kk, vv, kpos, um=None):
        """P and dS of a block of rows against the keys kk/vv at positions kpos
        (um: the user mask of those rows and keys)."""
        vis = visible(pos_b, kpos, causal, doc_starts) & has[:, None]
        s = scale * (qb @ kk.T)
        if um is not None:
            if um.dtype == bool:
                vis = vis & um
            else:
                hidden = um <= MASK_HIDE
                s = s + np.where(hidden, 0.0, um)
                vis = vis & ~hidden
        lse_safe = np.where(has, lse_b, 0.0)
        p = np.where(vis, np.exp(np.where(vis, s, 0.0) - lse_safe[:, None]), 0.0)
        dp = dob @ vv.T
        return p, p * (dp - delta[:, None])

    for b in range(B):
        for h in range(Hq):
            hk = kv_head_of(h, Hq, Hkv)
            for r0 in range(0, Sq, row_block):
                r1 = min(Sq, r0 + row_block)
                lse_b = lse[b, h, r0:r1]
                has = np.isfinite(lse_b)
                delta = np.sum(dout[b, h, r0:r1] * out[b, h, r0:r1], axis=1)
                qb, dob = q[b, h, r0:r1], dout[b, h, r0:r1]
                um = None if um_all is None else um_all[b, h, r0:r1]
                if want_dq:
                    _, ds = grads(qb, dob, delta, lse_b, has, q_pos[r0:r1], k[b, hk], v[b, hk], kv_pos, um)
                    dq[b, h, r0:r1] = scale * (ds @ k[b, hk])
                if sel.size:
                    p_sel, ds_sel = grads(qb, dob, delta, lse_b, has, q_pos[r0:r1],
                                          k[b, hk][sel], v[b, hk][sel], kv_pos[sel],
                                          None if um is None else um[:, sel])
                    dv[b, hk] += p_sel.T @ dob
                    dk[b, hk] += scale * (ds_sel.T @ qb)
    return dq, dk, dv


# ----------------------------------------------------------------------------
# Shares cut from one global problem
# ----------------------------------------------------------------------------
def _share(q_heads, kv_heads, q_pos, kv_pos, chunk_pos, chunk_len):
    return dict(q_heads=np.asarray(q_heads, np.int64), kv_heads=np.asarray(kv_heads, np.int64),
                q_pos=np.asarray(q_pos, np.int64), kv_pos=np.asarray(kv_pos, np.int64),
                q_chunk_pos=list(chunk_pos), chunk_len=int(chunk_len))


def contiguous_share(s_global: int, hq: int, hkv: int, cp_size: int, cp_rank: int):
    """Colossal / all-gather share ([CP-migration] §6.1; [Trainer-CP] §4.3):
    all heads, local rows ``[r*S/P, (r+1)*S/P)`` against every key ``[0, S)``.

    Returns the global head and row indices of the share; because the global
    problem is in natural order, a row's index is its global position.
    """
    pos, n = share_chunks("contiguous", s_global, cp_size, cp_rank)
    return _share(np.arange(hq), np.arange(hkv), chunk_row_positions(pos, n),
                  np.arange(s_global), pos, n)


def head_tail_share(s_global: int, hq: int, hkv: int, cp_size: int, cp_rank: int):
    """Head-Tail load-balanced all-gather share ([Trainer-CP] §0, §4.4;
    [FLA-CP] §3.2): rows of chunk r then rows of chunk 2P-1-r, against every
    key in natural order (the output order is restored by the caller, which
    [Trainer-CP] §4.4 requires of the wrapper)."""
    pos, n = share_chunks("head_tail", s_global, cp_size, cp_rank)
    return _share(np.arange(hq), np.arange(hkv), chunk_row_positions(pos, n),
                  np.arange(s_global), pos, n)


def ulysses_share(s_global: int, hq: int, hkv: int, cp_size: int, cp_rank: int):
    """Pure Ulysses share ([CP-migration] §6.2, §9.1, §9.2): after the
    sequence-to-head all-to-all, rank r holds Q heads ``[r*Hq/P, (r+1)*Hq/P)``
    and KV heads ``[r*Hkv/P, (r+1)*Hkv/P)`` over the whole sequence; causal
    offset 0 ([CP-migration] §8). Q and KV head counts must both divide by P."""
    if hq % cp_size or hkv % cp_size:
        raise ValueError("Ulysses needs Hq and Hkv divisible by the Ulysses degree")
    nq, nk = hq // cp_size, hkv // cp_size
    return _share(np.arange(cp_rank * nq, (cp_rank + 1) * nq),
                  np.arange(cp_rank * nk, (cp_rank + 1) * nk),
                  np.arange(s_global), np.arange(s_global), [0], s_global)


def hybrid_share(s_global: int, hq: int, hkv: int, cp_size: int, ulysses: int,
                 cp_rank: int):
    """Hybrid (Ulysses x Colossal) share ([CP-migration] §6.3, §8).

    P = C*U; the derived (C, U) mesh is named ("cp_co", "cp_ulysses"), read here
    row-major: ``co_rank = r // U``, ``u_rank = r % U``. After the all-to-all
    in the Ulysses group the rank holds heads ``[u*H/U, (u+1)*H/U)`` of Q and
    K/V; after the K/V all-gather in the co group its Q rows are
    ``[co*S/C, (co+1)*S/C)`` (causal offset ``co_rank * q_len_after_a2a``) and
    its K/V cover ``[0, S)``. Needs ``1 < U < P`` and ``P % U == 0``.
    """
    if not (1 < ulysses < cp_size) or cp_size % ulysses:
        raise ValueError("Hybrid needs 1 < U < P and P % U == 0")
    if hq % ulysses or hkv % ulysses:
        raise ValueError("Hybrid needs Hq and Hkv divisible by the Ulysses degree")
    c = cp_size // ulysses
    if s_global % c:
        raise ValueError("Hybrid needs S divisible by the co-group size")
    co, u = cp_rank // ulysses, cp_rank % ulysses
    n = s_global // c
    nq, nk = hq // ulysses, hkv // ulysses
    return _share(np.arange(u * nq, (u + 1) * nq), np.arange(u * nk, (u + 1) * nk),
                  np.arange(co * n, (co + 1) * n), np.arange(s_global), [co * n], n)


def share_pairs(q_pos, kv_pos, causal: bool = True, doc_starts: Optional[Sequence[int]] = None) -> int:
    """Number of visible (query, key) pairs per head: the causal work of a
    share, which Head-Tail balancing equalises across ranks ([Trainer-CP] §0).
    With packed sequences a row counts only the keys of its own sequence."""
    q_pos = np.asarray(q_pos, np.int64)
    kv_sorted = np.sort(np.asarray(kv_pos, np.int64))
    if not causal:
        return int(q_pos.size * kv_sorted.size)
    upto = np.searchsorted(kv_sorted, q_pos, side="right")
    if doc_starts is None:
        return int(upto.sum())
    starts = np.asarray(doc_starts, np.int64)
    d = doc_of(q_pos, starts)
    lo = np.where(d >= 0, starts[np.maximum(d, 0)], np.iinfo(np.int64).min)
    return int((upto - np.searchsorted(kv_sorted, lo, side="left")).sum())


# ----------------------------------------------------------------------------
# Ulysses exchange (the data movement around the all-to-all)
# ----------------------------------------------------------------------------
def ulysses_seq_to_head(shards: Sequence[np.ndarray]) -> list:
    """Sequence-to-head exchange of a Ulysses group of U ranks ([CP-migration]
    §6.2: ``[B, N, S/P, D]`` -- split heads, all-to-all -> ``[B, N/P, S, D]``;
    §6.3 runs the same exchange inside the ``cp_ulysses`` sub-group).

    ``shards[p]`` is rank p's sequence shard ``[B, N, L, D]`` (rows p*L ..
    p*L+L-1 of the group's sequence). Rank u ends up with heads
    ``[u*N/U, (u+1)*N/U)`` of every shard, the shards in rank order along the
    sequence: ``[B, N/U, U*L, D]``. Pure data movement, exact for any dtype.
    """
    U = len(shards)
    N = shards[0].shape[1]
    if N % U:
        raise ValueError("the head count must divide by the Ulysses degree")
    n = N // U
    return [np.concatenate([shards[p][:, u * n:(u + 1) * n] for p in range(U)], axis=2)
            for u in range(U)]


def ulysses_head_to_seq(head_shards: Sequence[np.ndarray]) -> list:
    """The inverse exchange ([CP-migration] §6.2 "inverse all_to_all" of the
    output): rank u holds heads ``[u*n, (u+1)*n)`` over the group's whole
    sequence ``[B, n, U*L, D]``; afterwards rank p holds every head of its
    sequence shard p, ``[B, U*n, L, D]``."""
    U = len(head_shards)
    S = head_shards[0].shape[2]
    if S % U:
        raise ValueError("the sequence length must divide by the Ulysses degree")
    L = S // U
    return [np.concatenate([head_shards[u][:, :, p * L:(p + 1) * L] for u in range(U)], axis=1)
            for p in range(U)]
