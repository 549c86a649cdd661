"""GPU parity of the Ulysses exchange re-layouts against the oracle's
exchange ("新流程 CP 多通信模式迁移设计方案" §6.2, §6.3), bit-exact.

Each test runs every rank of a Ulysses group on the one GPU: pack on every
rank, the all-to-all emulated by plain indexing (block p of rank r's send
buffer becomes block r of rank p's receive buffer -- the collective, which is
not part of the library), unpack on every rank; then compares each rank's
result with oracle.ulysses_seq_to_head / ulysses_head_to_seq on the same
inputs. The last tests run the whole Ulysses forward: exchange, the share
kernel on the head shards, the inverse exchange of the output.
"""
import math

import numpy as np
import pytest
import torch

import oracle.cp_share as oc
from context_causal_attention_attn_amd import (cp_attn_bwd, cp_attn_fwd, head_to_seq_pack, head_to_seq_unpack,
                                               seq_to_head_pack, seq_to_head_unpack, ulysses_bwd_in_place,
                                               ulysses_fwd_in_place)
from synthetic import global_problem, workload
from tests._share_cases import oracle_rows, oracle_share, to_f64

pytestmark = pytest.mark.gpu


def bits(t: torch.Tensor) -> np.ndarray:
    """The raw bits of a tensor (bf16 as int16, fp32 as int32): exact comparison."""
    t = t.detach().cpu().contiguous()
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).numpy()


def all_to_all(sends):
    """Rank r receives block r of every rank's send buffer, in rank order."""
    U = len(sends)
    return [torch.stack([sends[p][r] for p in range(U)]).contiguous() for r in range(U)]


CASES = [
    # dtype, U, B, heads per rank after the exchange, rows per shard, D
    ("bf16", 2, 2, 3, 100, 128),
    ("bf16", 4, 1, 2, 257, 64),
    ("fp32", 4, 2, 1, 64, 128),
    ("fp32", 3, 1, 2, 33, 64),
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-u{c[1]}-b{c[2]}-h{c[3]}-L{c[4]}-D{c[5]}" for c in CASES])
def test_seq_to_head_and_back_bit_exact(case):
    dtype, U, B, H, L, D = case
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    g = torch.Generator().manual_seed(U * 100 + L)
    dev = torch.device("cuda")
    # Rank p's sequence shard, as a strided view (every other row of a taller tensor).
    tall = [torch.randn(B, U * H, 2 * L, D, generator=g).to(tdt) for _ in range(U)]
    shards = [t[:, :, ::2] for t in tall]
    ref = oc.ulysses_seq_to_head([bits(x) for x in shards])
    ys = [seq_to_head_unpack(r) for r in all_to_all([seq_to_head_pack(x.to(dev), U) for x in
                                                     [t.to(dev)[:, :, ::2] for t in tall]])]
    torch.cuda.synchronize()
    for u in range(U):
        assert ys[u].shape == (B, H, U * L, D)
        np.testing.assert_array_equal(bits(ys[u]), ref[u], err_msg=f"seq->head rank {u}")
    # The inverse exchange, from head shards that are themselves strided views.
    heads_tall = [torch.randn(B, 2 * H, U * L, D, generator=g).to(tdt) for _ in range(U)]
    ys = [t[:, 1::2] for t in heads_tall]
    ref = oc.ulysses_head_to_seq([bits(y) for y in ys])
    xs = [head_to_seq_unpack(r) for r in all_to_all([head_to_seq_pack(t.to(dev)[:, 1::2], U)
                                                      for t in heads_tall])]
    torch.cuda.synchronize()
    for p in range(U):
        assert xs[p].shape == (B, U * H, L, D)
        np.testing.assert_array_equal(bits(xs[p]), ref[p], err_msg=f"head->seq rank {p}")


def test_preallocated_outputs_and_empty_shards():
    dev = torch.device("cuda")
    x = torch.randn(1, 4, 16, 128, device=dev).to(torch.bfloat16)
    out = torch.full((2, 1, 2, 16, 128), 7.0, device=dev, dtype=torch.bfloat16)
    blocks = seq_to_head_pack(x, 2, out=out)
    torch.cuda.synchronize()
    assert blocks.data_ptr() == out.data_ptr()
    assert torch.equal(blocks[1, 0], x[0, 2:4])
    empty = seq_to_head_pack(x[:, :, :0], 2)
    assert empty.shape == (2, 1, 2, 0, 128)


@pytest.mark.parametrize("U", [2, 4])
def test_ulysses_forward_through_the_exchange(U):
    """Sequence shards of Q/K/V -> exchange -> the share kernel on each rank's
    head shard (whole sequence, offset 0) -> inverse exchange of the output:
    each rank's output rows (all heads) match the oracle's attention of that
    sequence shard."""
    S, Hq, Hkv, D = 2048, 8, 4, 128
    prob = global_problem(1, Hq, Hkv, S, D, dtype="bf16", seed=12)
    dev = torch.device("cuda")
    L = S // U
    sh_q = [prob.q[:, :, p * L:(p + 1) * L].to(dev) for p in range(U)]
    sh_k = [prob.k[:, :, p * L:(p + 1) * L].to(dev) for p in range(U)]
    sh_v = [prob.v[:, :, p * L:(p + 1) * L].to(dev) for p in range(U)]
    exch = lambda shards: [seq_to_head_unpack(r) for r in all_to_all([seq_to_head_pack(x, U) for x in shards])]
    qh, kh, vh = exch(sh_q), exch(sh_k), exch(sh_v)
    scale = 1.0 / math.sqrt(D)
    outs = [cp_attn_fwd(qh[u], kh[u], vh[u], [0], softmax_scale=scale)[0] for u in range(U)]
    o_seq = [head_to_seq_unpack(r) for r in all_to_all([head_to_seq_pack(o, U) for o in outs])]
    torch.cuda.synchronize()
    for p in range(U):
        osh = oracle_share("contiguous", S, Hq, Hkv, U, p)
        ref_o, _ = oracle_rows(prob, osh, scale)
        err = np.max(np.abs(to_f64(o_seq[p]) - ref_o))
        rel = np.linalg.norm(to_f64(o_seq[p]) - ref_o) / np.linalg.norm(ref_o)
        print(f"ulysses u={U} rank {p}: out max-abs {err:.3e} rel-L2 {rel:.3e}", flush=True)
        assert err <= 2e-2 and rel <= 1e-2


def test_full_size_exchange_of_the_ulysses_workload():
    """The 32K Ulysses workload's Q (32 heads, 8 ranks of 4096 rows): every
    rank's head shard after the exchange, bit-exact."""
    spec, prob = workload("ulysses_cp8_s32k_gqa32x8_d128")
    U, S = spec["cp"], spec["seq"]
    L = S // U
    dev = torch.device("cuda")
    q = prob.q.to(dev)
    ys = [seq_to_head_unpack(r) for r in all_to_all([seq_to_head_pack(q[:, :, p * L:(p + 1) * L], U)
                                                     for p in range(U)])]
    torch.cuda.synchronize()
    qb = bits(prob.q)
    ref = oc.ulysses_seq_to_head([qb[:, :, p * L:(p + 1) * L] for p in range(U)])
    for u in range(U):
        np.testing.assert_array_equal(bits(ys[u]), ref[u], err_msg=f"rank {u}")


@pytest.mark.parametrize("U,dtype", [(2, "bf16"), (4, "bf16"), (4, "fp32")])
def test_ulysses_in_place_forward_and_backward(U, dtype):
    """The share kernels on the received blocks themselves: sequence shards ->
    pack -> all-to-all -> forward and backward straight from the blocks (no
    unpack) -> the output and dQ blocks go back through the all-to-all and are
    unpacked on the sequence side (no pack). Each rank's output and dQ rows
    (all heads) and each head rank's dK/dV match the oracle; the in-place
    results equal the unpacked path's."""
    S, Hq, Hkv, D = (2048, 8, 4, 128) if dtype == "bf16" else (512, 4, 4, 64)
    prob = global_problem(1, Hq, Hkv, S, D, dtype=dtype, seed=13, with_dout=True)
    dev = torch.device("cuda")
    L = S // U
    shard = lambda t, p: t[:, :, p * L:(p + 1) * L].to(dev)
    recv = lambda t: all_to_all([seq_to_head_pack(shard(t, p), U) for p in range(U)])
    qb, kb, vb, gb = recv(prob.q), recv(prob.k), recv(prob.v), recv(prob.dout)
    scale = 1.0 / math.sqrt(D)
    res = [ulysses_fwd_in_place(qb[u], kb[u], vb[u], softmax_scale=scale) for u in range(U)]
    grads = [ulysses_bwd_in_place(qb[u], kb[u], vb[u], res[u][0], res[u][1], gb[u], softmax_scale=scale)
             for u in range(U)]
    o_seq = [head_to_seq_unpack(r) for r in all_to_all([o for o, _ in res])]
    dq_seq = [head_to_seq_unpack(r) for r in all_to_all([g[0] for g in grads])]
    # The unpacked path on the same head shards.
    for u in range(U):
        qh, kh, vh, gh = (seq_to_head_unpack(x[u]) for x in (qb, kb, vb, gb))
        o_ref, l_ref = cp_attn_fwd(qh, kh, vh, [0], softmax_scale=scale)
        g_ref = cp_attn_bwd(qh, kh, vh, o_ref, l_ref, gh, [0], softmax_scale=scale)
        torch.cuda.synchronize()
        assert res[u][0].shape == (U, 1, Hq // U, L, D) and res[u][1].shape == (1, Hq // U, S)
        assert torch.equal(seq_to_head_unpack(res[u][0]), o_ref) and torch.equal(res[u][1], l_ref), f"fwd u{u}"
        assert torch.equal(seq_to_head_unpack(grads[u][0]), g_ref[0]), f"dq u{u}"
        for a, b in zip(grads[u][1:], g_ref[1:]):
            assert float((a - b).norm() / b.norm()) <= 1e-5, f"dk/dv u{u}"
    tol_o, tol_g = (2e-2, 1e-2) if dtype == "bf16" else (1e-4, 1e-4)
    for p in range(U):
        osh = oracle_share("contiguous", S, Hq, Hkv, U, p)
        ref_o, _ = oracle_rows(prob, osh, scale)
        err = np.max(np.abs(to_f64(o_seq[p]) - ref_o))
        rows = torch.from_numpy(osh["q_pos"])
        ref_dq, _, _ = oc.attention_rows_bwd(to_f64(prob.q[:, :, rows]), to_f64(prob.k), to_f64(prob.v),
                                             to_f64(prob.dout[:, :, rows]), osh["q_pos"], np.arange(S), scale, True,
                                             kv_index=np.array([], dtype=np.int64))
        e_dq = np.linalg.norm(to_f64(dq_seq[p]) - ref_dq) / np.linalg.norm(ref_dq)
        print(f"ulysses in place u={U} {dtype} rank {p}: out max-abs {err:.3e} dq rel-L2 {e_dq:.3e}", flush=True)
        assert err <= tol_o and e_dq <= tol_g
    for u in range(U):
        kh = list(range(u * Hkv // U, (u + 1) * Hkv // U))
        qh = list(range(u * Hq // U, (u + 1) * Hq // U))
        _, rdk, rdv = oc.attention_rows_bwd(to_f64(prob.q[:, qh]), to_f64(prob.k[:, kh]), to_f64(prob.v[:, kh]),
                                            to_f64(prob.dout[:, qh]), np.arange(S), np.arange(S), scale, True,
                                            want_dq=False)
        for got, ref in ((grads[u][1], rdk), (grads[u][2], rdv)):
            e = np.linalg.norm(to_f64(got) - ref) / np.linalg.norm(ref)
            assert e <= tol_g, f"head rank {u}: dk/dv rel-L2 {e}"


def test_full_size_ulysses_in_place_forward():
    """Rank 0 of the 32K Ulysses workload from its received blocks (8 blocks
    of 4096 rows, 4 query heads, 1 KV head): identical to the unpacked share."""
    spec, prob = workload("ulysses_cp8_s32k_gqa32x8_d128")
    U, S = spec["cp"], spec["seq"]
    L = S // U
    dev = torch.device("cuda")
    blocks = [all_to_all([seq_to_head_pack(t.to(dev)[:, :, p * L:(p + 1) * L], U) for p in range(U)])[0]
              for t in (prob.q, prob.k, prob.v)]
    scale = 1.0 / math.sqrt(spec["head_dim"])
    out_b, lse_b = ulysses_fwd_in_place(*blocks, softmax_scale=scale)
    qh, kh, vh = (seq_to_head_unpack(b) for b in blocks)
    out, lse = cp_attn_fwd(qh, kh, vh, [0], softmax_scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(seq_to_head_unpack(out_b), out) and torch.equal(lse_b, lse)
