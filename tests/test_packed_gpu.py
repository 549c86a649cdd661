"""GPU parity of packed variable-length sequences (a global cu_seqlens split
across CP ranks: a key is visible only inside its query's own sequence)
against the oracle, forward and backward, on every rank of contiguous and
Head-Tail shares, with sequences shorter than a key tile, boundaries on and
off tile boundaries, and sequences cut by rank boundaries."""
import math

import numpy as np
import pytest
import torch

import oracle.cp_share as oc
from context_causal_attention_attn_amd import cp_attn_bwd, cp_attn_fwd, cut_share
from synthetic import global_problem, workload
from tests._share_cases import oracle_share, to_f64

pytestmark = pytest.mark.gpu

OUT_TOL_BF16, LSE_TOL_BF16, TOL_FP32 = 2e-2, 1e-3, 1e-4


def starts_of(lengths):
    return [int(x) for x in np.concatenate([[0], np.cumsum(lengths)[:-1]])]


def rel_l2(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def run_share(prob, kind, cp, rank, starts, with_bwd):
    dev = torch.device("cuda")
    q, k, v = prob.q.to(dev), prob.k.to(dev), prob.v.to(dev)
    sh = cut_share(kind, q, k, v, cp, rank)
    scale = 1.0 / math.sqrt(q.shape[-1])
    out, lse = cp_attn_fwd(sh.q, sh.k, sh.v, sh.q_chunk_pos, layout=sh.layout, softmax_scale=scale,
                           doc_starts=starts)
    grads = None
    if with_bwd:
        dout = sh.take_rows(prob.dout.to(dev))
        grads = cp_attn_bwd(sh.q, sh.k, sh.v, out, lse, dout, sh.q_chunk_pos, layout=sh.layout,
                            softmax_scale=scale, doc_starts=starts)
    torch.cuda.synchronize()
    return sh, out, lse, grads, scale


def oracle_fwd_bwd(prob, osh, scale, starts, with_bwd, rows=None, heads=None):
    qh, kh = osh["q_heads"], osh["kv_heads"]
    q_pos = osh["q_pos"] if rows is None else osh["q_pos"][rows]
    q = to_f64(prob.q[:, qh][:, :, torch.from_numpy(q_pos)])
    if heads is not None:
        q = q[:, heads]
    k, v = to_f64(prob.k[:, kh]), to_f64(prob.v[:, kh])
    if heads is not None:
        G = len(qh) // len(kh)
        assert all(h // G == 0 for h in heads), "sampled heads of the first GQA group only"
        k, v = k[:, :1], v[:, :1]
    out, lse = oc.attention_rows(q, k, v, q_pos, osh["kv_pos"], scale, True, doc_starts=starts)
    if not with_bwd:
        return out, lse, None
    do = to_f64(prob.dout[:, qh][:, :, torch.from_numpy(osh["q_pos"])])
    return out, lse, oc.attention_rows_bwd(to_f64(prob.q[:, qh][:, :, torch.from_numpy(osh["q_pos"])]), k, v, do,
                                          osh["q_pos"], osh["kv_pos"], scale, True, doc_starts=starts)


def check_fwd(out, lse, ref_o, ref_l, tol_o, tol_l, what):
    o, l = to_f64(out), to_f64(lse)
    err_o = float(np.max(np.abs(o - ref_o)))
    err_l = float(np.max(np.abs(l - ref_l)))
    print(f"{what}: out max-abs {err_o:.3e} rel-L2 {rel_l2(o, ref_o):.3e} lse max-abs {err_l:.3e}", flush=True)
    assert err_o <= tol_o and err_l <= tol_l and rel_l2(o, ref_o) <= 1e-2, what


MIXES = {
    "cut": [700, 900, 448],                     # boundaries inside ranks and tiles
    "aligned": [512, 512, 1024],                # boundaries on rank and tile boundaries
    "short": [30, 5, 64, 1, 90, 200, 17, 300, 1341],   # sequences shorter than a tile
    "late_start": [1300, 748],                  # rows before the first boundary's rank
}


@pytest.mark.parametrize("mix", list(MIXES), ids=list(MIXES))
@pytest.mark.parametrize("kind", ["contiguous", "head_tail"])
def test_packed_bf16_fwd_bwd_all_ranks(kind, mix):
    S, Hq, Hkv, D, cp = 2048, 8, 2, 128, 4
    starts = starts_of(MIXES[mix])
    prob = global_problem(1, Hq, Hkv, S, D, dtype="bf16", seed=13, with_dout=True)
    for r in range(cp):
        sh, out, lse, grads, scale = run_share(prob, kind, cp, r, starts, True)
        osh = oracle_share(kind, S, Hq, Hkv, cp, r)
        ref_o, ref_l, ref_g = oracle_fwd_bwd(prob, osh, scale, starts, True)
        check_fwd(out, lse, ref_o, ref_l, OUT_TOL_BF16, LSE_TOL_BF16, f"packed {kind} {mix} r{r}")
        errs = [rel_l2(to_f64(g), rg) for g, rg in zip(grads, ref_g)]
        print(f"  dq {errs[0]:.3e} dk {errs[1]:.3e} dv {errs[2]:.3e}", flush=True)
        assert max(errs) <= 1e-2


def test_packed_fp32_and_offset_start():
    """fp32 path (tolerance 1e-4), and a first boundary after position 0
    (rows before it form one more sequence)."""
    S, Hq, Hkv, D, cp = 512, 2, 2, 64, 4
    prob = global_problem(1, Hq, Hkv, S, D, dtype="fp32", seed=14, with_dout=True)
    for starts in (starts_of([100, 3, 200, 209]), [37, 300]):
        for kind in ("contiguous", "head_tail"):
            for r in range(cp):
                sh, out, lse, grads, scale = run_share(prob, kind, cp, r, starts, True)
                osh = oracle_share(kind, S, Hq, Hkv, cp, r)
                ref_o, ref_l, ref_g = oracle_fwd_bwd(prob, osh, scale, starts, True)
                check_fwd(out, lse, ref_o, ref_l, TOL_FP32, TOL_FP32, f"fp32 packed {kind} {starts[:2]} r{r}")
                for g, rg in zip(grads, ref_g):
                    assert rel_l2(to_f64(g), rg) <= TOL_FP32


def test_packed_full_size_sampled_rows():
    """The benchmarked 32K Colossal rank-7 share with eight packed sequences
    (boundaries cut the rank's rows): sampled rows of two heads against the
    oracle."""
    spec, prob = workload("colossal_cp8_r7_s32k_gqa32x8_d128")
    starts = starts_of([3000, 4000, 3240, 5120, 5120, 7000, 3240, 2048])
    sh, out, lse, _, scale = run_share(prob, "contiguous", 8, 7, starts, False)
    osh = oracle_share("contiguous", spec["seq"], spec["hq"], spec["hkv"], 8, 7)
    rng = np.random.default_rng(5)
    # Rows around the boundary at 30720 inside the share and random rows.
    edge = [30720 - 28672 + d for d in (-2, -1, 0, 1, 63, 64)]
    rows = np.unique(np.concatenate([edge, [0, 4095], rng.integers(0, 4096, 24)]))
    heads = [0, 3]
    ref_o, ref_l, _ = oracle_fwd_bwd(prob, osh, scale, starts, False, rows=rows, heads=heads)
    r_t = torch.from_numpy(rows).to(out.device)
    check_fwd(out[:, heads][:, :, r_t], lse[:, heads][:, :, r_t], ref_o, ref_l, OUT_TOL_BF16, LSE_TOL_BF16,
              "32K packed colossal r7")


OTHER = [
    # kind, S, Hq, Hkv, D, cp, B: the other kernel instantiations
    ("head_tail", 1024, 6, 3, 64, 2, 1),     # D = 64, GQA groups of 2
    ("contiguous", 1024, 4, 4, 128, 4, 2),   # MHA (one head per work item), B = 2
]


@pytest.mark.parametrize("case", OTHER, ids=[f"{c[0]}-D{c[4]}-{c[2]}x{c[3]}-B{c[6]}" for c in OTHER])
def test_packed_other_shapes(case):
    kind, S, Hq, Hkv, D, cp, B = case
    starts = starts_of([200, 63, 129, 1, 631])
    prob = global_problem(B, Hq, Hkv, S, D, dtype="bf16", seed=15, with_dout=True)
    for r in range(cp):
        sh, out, lse, grads, scale = run_share(prob, kind, cp, r, starts, True)
        osh = oracle_share(kind, S, Hq, Hkv, cp, r)
        ref_o, ref_l, ref_g = oracle_fwd_bwd(prob, osh, scale, starts, True)
        check_fwd(out, lse, ref_o, ref_l, OUT_TOL_BF16, LSE_TOL_BF16, f"packed {case} r{r}")
        errs = [rel_l2(to_f64(g), rg) for g, rg in zip(grads, ref_g)]
        print(f"  dq {errs[0]:.3e} dk {errs[1]:.3e} dv {errs[2]:.3e}", flush=True)
        assert max(errs) <= 1e-2


def test_packed_full_size_head_tail_sampled_rows():
    """32K Head-Tail rank 2 with the eight-sequence mix: rows of both chunks
    (4096.. inside one sequence; 26624.. crossing the boundary at 27480)."""
    spec, prob = workload("colossal_cp8_r7_s32k_gqa32x8_d128")
    starts = starts_of([3000, 4000, 3240, 5120, 5120, 7000, 3240, 2048])
    sh, out, lse, _, scale = run_share(prob, "head_tail", 8, 2, starts, False)
    osh = oracle_share("head_tail", spec["seq"], spec["hq"], spec["hkv"], 8, 2)
    rng = np.random.default_rng(6)
    rows = np.unique(np.concatenate([[0, 2047, 2048, 4095], rng.integers(0, 4096, 28)]))
    heads = [1, 2]
    ref_o, ref_l, _ = oracle_fwd_bwd(prob, osh, scale, starts, False, rows=rows, heads=heads)
    r_t = torch.from_numpy(rows).to(out.device)
    check_fwd(out[:, heads][:, :, r_t], lse[:, heads][:, :, r_t], ref_o, ref_l, OUT_TOL_BF16, LSE_TOL_BF16,
              "32K packed head_tail r2")


@pytest.mark.parametrize("kind", ["contiguous", "head_tail"])
def test_tail_padding_needs_no_mask(kind):
    """A 2000-token sequence padded to 2048 so that it divides by cp (or 2cp)
    ([Trainer-CP] §4.2 padding policy): under the global-position causal mask
    no real token sees a padding key, so every real row equals the oracle's
    attention over the unpadded sequence, on every rank."""
    S, S_real, Hq, Hkv, D, cp = 2048, 2000, 8, 2, 128, 4
    prob = global_problem(1, Hq, Hkv, S, D, dtype="bf16", seed=16)
    for r in range(cp):
        sh, out, lse, _, scale = run_share(prob, kind, cp, r, [], False)
        osh = oracle_share(kind, S, Hq, Hkv, cp, r)
        real = np.nonzero(osh["q_pos"] < S_real)[0]
        if real.size == 0:
            continue
        q = to_f64(prob.q[:, :, torch.from_numpy(osh["q_pos"][real])])
        ref_o, ref_l = oc.attention_rows(q, to_f64(prob.k[:, :, :S_real]), to_f64(prob.v[:, :, :S_real]),
                                         osh["q_pos"][real], np.arange(S_real), scale, True)
        r_t = torch.from_numpy(real).to(out.device)
        check_fwd(out[:, :, r_t], lse[:, :, r_t], ref_o, ref_l, OUT_TOL_BF16, LSE_TOL_BF16,
                  f"padded {kind} r{r}")
