"""GPU parity of the backward share kernels against the fp64 oracle.

The GPU backward consumes the GPU forward's own out and LSE (as a training step
would); the oracle recomputes everything in float64 from the same seeded
inputs. Gate: relative L2 error <= 1e-2 for dQ, dK and dV each (fp32 inputs:
1e-4). Mid-size shares compare whole tensors; the 32K Head-Tail backward
(B = 2, ranks 0 and 7) compares sampled dQ rows and the dK/dV rows of sampled
keys of one KV head, plus the exact zeros of keys no local query can see.
"""
import math

import numpy as np
import pytest
import torch

import oracle.cp_share as oc
from context_causal_attention_attn_amd import cp_attn_bwd, cp_attn_fwd, cut_share
from synthetic import global_problem, workload
from tests._share_cases import gathered_key_rows, oracle_share, spiked_problem, to_f64

pytestmark = pytest.mark.gpu

REL_BF16 = 1e-2
REL_FP32 = 1e-4


def rel_l2(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


def gpu_share_grads(prob, kind, cp, rank, U=2, causal=True, kv_order="natural"):
    dev = torch.device("cuda")
    q, k, v = prob.q.to(dev), prob.k.to(dev), prob.v.to(dev)
    sh = cut_share(kind, q, k, v, cp, rank, ulysses=U, kv_order=kv_order)
    scale = 1.0 / math.sqrt(q.shape[-1])
    out, lse = cp_attn_fwd(sh.q, sh.k, sh.v, sh.q_chunk_pos, layout=sh.layout, causal=causal,
                           softmax_scale=scale, kv_chunk_pos=sh.kv_chunk_pos)
    dout = sh.take_rows(prob.dout.to(dev))
    dq, dk, dv = cp_attn_bwd(sh.q, sh.k, sh.v, out, lse, dout, sh.q_chunk_pos, layout=sh.layout,
                             causal=causal, softmax_scale=scale, kv_chunk_pos=sh.kv_chunk_pos)
    torch.cuda.synchronize()
    return sh, dq, dk, dv, scale


def oracle_share_grads(prob, osh, scale, causal=True, key_rows=None):
    """Oracle dq, dk, dv of a share; key_rows lists the global key rows in
    storage order (dk/dv come out in that order)."""
    qh, kh = osh["q_heads"], osh["kv_heads"]
    rows = torch.from_numpy(osh["q_pos"])
    q = to_f64(prob.q[:, qh][:, :, rows])
    do = to_f64(prob.dout[:, qh][:, :, rows])
    k, v = prob.k[:, kh], prob.v[:, kh]
    kv_pos = osh["kv_pos"]
    if key_rows is not None:
        k, v, kv_pos = k[:, :, torch.from_numpy(key_rows)], v[:, :, torch.from_numpy(key_rows)], kv_pos[key_rows]
    return oc.attention_rows_bwd(q, to_f64(k), to_f64(v), do, osh["q_pos"], kv_pos, scale, causal)


def check_grads(got, ref, tol, what):
    errs = {n: rel_l2(to_f64(g), r) for n, g, r in zip(("dq", "dk", "dv"), got, ref)}
    print(f"{what}: " + "  ".join(f"{n} rel-L2 {e:.3e}" for n, e in errs.items()), flush=True)
    for n, e in errs.items():
        assert e <= tol, f"{what}: {n} relative L2 {e}"


@pytest.mark.parametrize("kind,cp,rank", [("contiguous", 4, 1), ("contiguous", 4, 3), ("head_tail", 4, 0),
                                          ("head_tail", 4, 3)])
def test_tiny_fp32_backward(kind, cp, rank):
    spec, _ = workload("tiny_fp32_contiguous_cp4_r1")
    prob = global_problem(1, spec["hq"], spec["hkv"], spec["seq"], spec["head_dim"], "fp32", 0, with_dout=True)
    sh, dq, dk, dv, scale = gpu_share_grads(prob, kind, cp, rank)
    osh = oracle_share(kind, spec["seq"], spec["hq"], spec["hkv"], cp, rank)
    check_grads((dq, dk, dv), oracle_share_grads(prob, osh, scale), REL_FP32, f"fp32 {kind} r{rank}")


MID = [
    # kind, S, Hq, Hkv, D, cp, U, causal
    ("contiguous", 2000, 8, 2, 128, 4, 2, True),
    ("head_tail", 2000, 8, 2, 128, 4, 2, True),
    ("ulysses", 1000, 8, 2, 128, 2, 2, True),
    ("hybrid", 2000, 8, 2, 128, 4, 2, True),
    ("head_tail", 1200, 4, 4, 128, 3, 2, True),
    ("contiguous", 999, 8, 1, 128, 3, 2, True),
    ("head_tail", 1000, 6, 3, 64, 2, 2, True),
    ("contiguous", 1000, 4, 2, 64, 4, 2, False),
    ("head_tail", 1000, 8, 2, 128, 2, 2, False),
]


@pytest.mark.parametrize("case", MID, ids=[f"{c[0]}-S{c[1]}-{c[2]}x{c[3]}-D{c[4]}-cp{c[5]}-{'c' if c[7] else 'nc'}" for c in MID])
def test_bf16_mid_backward_all_ranks(case):
    kind, S, Hq, Hkv, D, cp, U, causal = case
    prob = global_problem(1, Hq, Hkv, S, D, dtype="bf16", seed=5, with_dout=True)
    dk_sum = None
    for r in range(cp):
        sh, dq, dk, dv, scale = gpu_share_grads(prob, kind, cp, r, U=U, causal=causal)
        osh = oracle_share(kind, S, Hq, Hkv, cp, r, U)
        ref = oracle_share_grads(prob, osh, scale, causal)
        check_grads((dq, dk, dv), ref, REL_BF16, f"{case} r{r}")
        if kind in ("contiguous", "head_tail") and causal:
            # Keys after every local query: partial dK/dV rows are exact zeros.
            last = int(osh["q_pos"].max())
            assert torch.all(dk[:, :, last + 1:] == 0) and torch.all(dv[:, :, last + 1:] == 0)
            dk_sum = dk.double().cpu() if dk_sum is None else dk_sum + dk.double().cpu()
    if dk_sum is not None:
        # reduce-scatter(sum) semantics: the rank partials add up to the full dK.
        full = oc.contiguous_share(S, Hq, Hkv, 1, 0)
        ref_full = oracle_share_grads(prob, full, 1.0 / math.sqrt(D), causal)
        assert rel_l2(dk_sum.numpy(), ref_full[1]) <= REL_BF16


GATHERED = [
    # kind, S, Hq, Hkv, D, cp, causal, dtype
    ("head_tail", 2048, 8, 2, 128, 4, True, "bf16"),
    ("head_tail", 1024, 4, 4, 64, 4, True, "bf16"),
    ("hybrid", 2048, 8, 2, 128, 4, True, "bf16"),
    ("head_tail", 2048, 8, 2, 128, 4, False, "bf16"),
    ("head_tail", 1024, 2, 2, 64, 4, True, "fp32"),
]


@pytest.mark.parametrize("case", GATHERED, ids=[f"{c[0]}-S{c[1]}-D{c[4]}-cp{c[5]}-{'c' if c[6] else 'nc'}-{c[7]}" for c in GATHERED])
def test_gathered_kv_order_backward_all_ranks(case):
    """K/V in all-gather order: dQ as in the natural order, partial dK/dV in
    the storage order of the K/V rows."""
    kind, S, Hq, Hkv, D, cp, causal, dtype = case
    prob = global_problem(1, Hq, Hkv, S, D, dtype=dtype, seed=10, with_dout=True)
    keys = gathered_key_rows(kind, S, cp)
    tol = REL_BF16 if dtype == "bf16" else REL_FP32
    for r in range(cp):
        sh, dq, dk, dv, scale = gpu_share_grads(prob, kind, cp, r, causal=causal, kv_order="gathered")
        osh = oracle_share(kind, S, Hq, Hkv, cp, r)
        ref = oracle_share_grads(prob, osh, scale, causal, key_rows=keys)
        check_grads((dq, dk, dv), ref, tol, f"gathered {case} r{r}")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_backward_kv_chunks_with_gap_and_invisible_chunk(dtype):
    """The forward test's scrambled table (positions 1280, 0, 2048, 512): the
    chunk no query sees gets exact-zero dK/dV rows."""
    prob = global_problem(1, 4, 2, 1024, 128, dtype=dtype, seed=11, with_dout=True)
    table = [1280, 0, 2048, 512]
    kv_pos = np.concatenate([np.arange(p, p + 256) for p in table])
    dev = torch.device("cuda")
    q, k, v = prob.q[:, :, :256].to(dev), prob.k.to(dev), prob.v.to(dev)
    do = prob.dout[:, :, :256].to(dev)
    out, lse = cp_attn_fwd(q, k, v, [1200], kv_chunk_pos=table, softmax_scale=0.1)
    dq, dk, dv = cp_attn_bwd(q, k, v, out, lse, do, [1200], kv_chunk_pos=table, softmax_scale=0.1)
    torch.cuda.synchronize()
    ref = oc.attention_rows_bwd(to_f64(prob.q[:, :, :256]), to_f64(prob.k), to_f64(prob.v),
                                to_f64(prob.dout[:, :, :256]), np.arange(1200, 1456), kv_pos, 0.1, True)
    check_grads((dq, dk, dv), ref, REL_BF16 if dtype == "bf16" else REL_FP32, f"kv chunk gap {dtype}")
    assert torch.all(dk[:, :, 512:768] == 0) and torch.all(dv[:, :, 512:768] == 0)


def test_backward_edge_cases():
    """Keys after some queries (rows with no visible key get dQ = 0) and a
    head_tail share of single-row chunks."""
    prob = global_problem(1, 4, 2, 512, 64, dtype="bf16", seed=6, with_dout=True)
    dev = torch.device("cuda")
    q, k, v = prob.q[:, :, :400].to(dev), prob.k[:, :, :200].to(dev), prob.v[:, :, :200].to(dev)
    do = prob.dout[:, :, :400].to(dev)
    out, lse = cp_attn_fwd(q, k, v, [100], kv_chunk_pos=[300], softmax_scale=0.125)
    dq, dk, dv = cp_attn_bwd(q, k, v, out, lse, do, [100], kv_chunk_pos=[300], softmax_scale=0.125)
    torch.cuda.synchronize()
    ref = oc.attention_rows_bwd(to_f64(prob.q[:, :, :400]), to_f64(prob.k[:, :, :200]),
                                to_f64(prob.v[:, :, :200]), to_f64(prob.dout[:, :, :400]),
                                np.arange(100, 500), np.arange(300, 500), 0.125, True)
    check_grads((dq, dk, dv), ref, REL_BF16, "kv offset")
    assert torch.all(dq[:, :, :200] == 0)
    prob = global_problem(1, 4, 2, 8, 128, dtype="bf16", seed=2, with_dout=True)
    for r in range(4):
        sh, dq, dk, dv, scale = gpu_share_grads(prob, "head_tail", 4, r)
        osh = oracle_share("head_tail", 8, 4, 2, 4, r)
        check_grads((dq, dk, dv), oracle_share_grads(prob, osh, scale), REL_BF16, f"S=8 r{r}")


@pytest.mark.parametrize("kind,cp,rank", [("contiguous", 2, 1), ("head_tail", 2, 0)])
def test_backward_with_late_score_spike(kind, cp, rank):
    """Gradients when a few keys dominate the rows after them (large LSE)."""
    prob = spiked_problem(with_dout=True)
    sh, dq, dk, dv, scale = gpu_share_grads(prob, kind, cp, rank)
    osh = oracle_share(kind, 1024, 4, 2, cp, rank)
    check_grads((dq, dk, dv), oracle_share_grads(prob, osh, scale), REL_BF16, f"spike {kind} r{rank}")


@pytest.fixture(scope="module")
def htbwd_problem():
    return workload("head_tail_bwd_b2_cp8_s32k_gqa32x8_d128")


def check_full_size_backward_sampled(spec, prob, kind, rank, b, hk, what):
    """Full-size share backward in the launch configuration bench.py times,
    checked on sampled outputs the oracle computes one by one: dQ of sampled
    rows (every head of one GQA group) and dK/dV of sampled keys (which need
    every local row of the group's heads)."""
    S, Hq, Hkv = spec["seq"], spec["hq"], spec["hkv"]
    sh, dq, dk, dv, scale = gpu_share_grads(prob, kind, spec["cp"], rank)
    osh = oracle_share(kind, S, Hq, Hkv, spec["cp"], rank)
    rng = np.random.default_rng(rank)
    G = Hq // Hkv
    heads = list(range(hk * G, hk * G + G))
    nrows = len(osh["q_pos"])
    rows = np.unique(np.concatenate([[0, 31, 32, nrows // 2 - 1, nrows // 2, nrows - 1],
                                     rng.integers(0, nrows, 40)]))
    pos = osh["q_pos"][rows]
    qd = to_f64(prob.q[b:b + 1, heads][:, :, torch.from_numpy(pos)])
    dod = to_f64(prob.dout[b:b + 1, heads][:, :, torch.from_numpy(pos)])
    kd, vd = to_f64(prob.k[b:b + 1, hk:hk + 1]), to_f64(prob.v[b:b + 1, hk:hk + 1])
    ref_dq, _, _ = oc.attention_rows_bwd(qd, kd, vd, dod, pos, osh["kv_pos"], scale, True,
                                         kv_index=np.array([], dtype=np.int64))
    got_dq = to_f64(dq[b:b + 1, heads][:, :, torch.from_numpy(rows).cuda()])
    e_dq = rel_l2(got_dq, ref_dq)
    last = int(osh["q_pos"].max())
    keys = np.unique(np.concatenate([[0, 1, 127, 128, 2047, 2048, last - 1, last],
                                     rng.integers(0, last + 1, 40)]))
    qa = to_f64(prob.q[b:b + 1, heads][:, :, torch.from_numpy(osh["q_pos"])])
    doa = to_f64(prob.dout[b:b + 1, heads][:, :, torch.from_numpy(osh["q_pos"])])
    _, ref_dk, ref_dv = oc.attention_rows_bwd(qa, kd, vd, doa, osh["q_pos"], osh["kv_pos"], scale, True,
                                              kv_index=keys, want_dq=False)
    kt = torch.from_numpy(keys).cuda()
    e_dk = rel_l2(to_f64(dk[b:b + 1, hk:hk + 1][:, :, kt]), ref_dk)
    e_dv = rel_l2(to_f64(dv[b:b + 1, hk:hk + 1][:, :, kt]), ref_dv)
    print(f"{what}: dq {e_dq:.3e} dk {e_dk:.3e} dv {e_dv:.3e}", flush=True)
    assert e_dq <= REL_BF16 and e_dk <= REL_BF16 and e_dv <= REL_BF16
    assert torch.all(dk[:, :, last + 1:] == 0) and torch.all(dv[:, :, last + 1:] == 0)
    assert torch.isfinite(dq).all() and torch.isfinite(dk).all() and torch.isfinite(dv).all()


@pytest.mark.parametrize("rank", [0, 7])
def test_full_size_head_tail_backward_sampled(htbwd_problem, rank):
    spec, prob = htbwd_problem
    check_full_size_backward_sampled(spec, prob, "head_tail", rank, 1, 5, f"32K head_tail bwd r{rank}")


def test_full_size_colossal_backward_sampled():
    """The benchmarked share (Colossal cp=8 rank 7, S = 32768) backward."""
    spec, _ = workload("colossal_cp8_r7_s32k_gqa32x8_d128")
    prob = global_problem(spec["batch"], spec["hq"], spec["hkv"], spec["seq"], spec["head_dim"],
                          spec["dtype"], 0, with_dout=True)
    check_full_size_backward_sampled(spec, prob, "contiguous", spec["ranks"][0], 0, 3, "32K colossal bwd r7")


@pytest.fixture(scope="module")
def s32k_dout_problem():
    spec, _ = workload("ulysses_cp8_s32k_gqa32x8_d128")
    prob = global_problem(spec["batch"], spec["hq"], spec["hkv"], spec["seq"], spec["head_dim"],
                          spec["dtype"], 0, with_dout=True)
    return spec, prob


@pytest.mark.parametrize("name,hk", [("ulysses_cp8_s32k_gqa32x8_d128", 0),
                                     ("hybrid_u2_c4_s32k_gqa32x8_d128", 2)])
def test_full_size_head_sharded_backward_sampled(s32k_dout_problem, name, hk):
    """Backward of the 32K head-sharded shares (Ulysses cp=8 rank 0: 4 query
    heads over the whole sequence; Hybrid U=2 x C=4 rank 4: 16 query heads,
    rows 16384..24575) in the launch configuration the benchmark times."""
    spec, _ = workload(name)
    _, prob = s32k_dout_problem
    check_full_size_backward_sampled(spec, prob, spec["kind"], spec["ranks"][0], 0, hk,
                                     f"32K {spec['kind']} bwd r{spec['ranks'][0]}")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_timed_backward_matches_untimed(dtype):
    # cp_attn_bwd_timed runs the same kernels with events between them: the
    # gradients must be bitwise those of cp_attn_bwd, and every phase's time
    # non-negative (the dK/dV phase strictly positive).
    from context_causal_attention_attn_amd import cp_attn_bwd_timed
    S, Hq, Hkv, D = (1200, 8, 2, 128) if dtype == "bf16" else (240, 2, 2, 64)
    prob = global_problem(1, Hq, Hkv, S, D, dtype, 3, with_dout=True)
    sh, dq, dk, dv, scale = gpu_share_grads(prob, "head_tail", 3, 1)
    dev = torch.device("cuda")
    out, lse = cp_attn_fwd(sh.q, sh.k, sh.v, sh.q_chunk_pos, layout=sh.layout, softmax_scale=scale)
    dout = sh.take_rows(prob.dout.to(dev))
    events = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    g = cp_attn_bwd_timed(sh.q, sh.k, sh.v, out, lse, dout, sh.q_chunk_pos, events, layout=sh.layout,
                          softmax_scale=scale)
    torch.cuda.synchronize()
    for a, b, n in zip((dq, dk, dv), g, ("dq", "dk", "dv")):
        assert torch.equal(a, b), n
    times = [events[i].elapsed_time(events[i + 1]) for i in range(3)]
    assert min(times) >= 0.0 and times[1] > 0.0, times
