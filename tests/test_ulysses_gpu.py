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
from context_causal_attention_attn_amd import (cp_attn_fwd, head_to_seq_pack, head_to_seq_unpack,
                                               seq_to_head_pack, seq_to_head_unpack)
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
