"""Pins of the fp64 oracle to facts outside its own arithmetic (CPU only).

Each test checks the oracle against something it does not compute itself:
hand-derived worked examples (tests/golden), brute-force Python loops over the
unsharded problem, torch's float64 scaled-dot-product attention and its
autograd, closed forms, reassembly of every rank's share into the unsharded
result, and central finite differences. The last block plants plausible
mistakes in the oracle and checks that a pin catches each one.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle.cp_share as oc
from synthetic import global_problem

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _np(t):
    return t.to(torch.float64).numpy()


# ----------------------------------------------------------------------------
# Independent references
# ----------------------------------------------------------------------------
def brute_full_causal(q, k, v, scale):
    """Unsharded causal attention by explicit Python loops (positions = row
    index, key j visible to query i iff j <= i), written independently of the
    oracle: no NumPy reductions, math.exp on each score, math.fsum sums."""
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    out = np.zeros((B, Hq, S, D))
    lse = np.zeros((B, Hq, S))
    for b in range(B):
        for h in range(Hq):
            hk = h // G
            for i in range(S):
                scores = [scale * math.fsum(q[b, h, i, d] * k[b, hk, j, d] for d in range(D))
                          for j in range(i + 1)]
                mx = max(scores)
                w = [math.exp(s - mx) for s in scores]
                tot = math.fsum(w)
                lse[b, h, i] = mx + math.log(tot)
                for d in range(D):
                    out[b, h, i, d] = math.fsum(w[j] * v[b, hk, j, d] for j in range(i + 1)) / tot
    return out, lse


def torch_sdpa_full(q, k, v, scale, causal=True, mask=None):
    """torch's float64 SDPA on the CPU with K/V repeated per GQA group."""
    G = q.shape[1] // k.shape[1]
    kr = k.repeat_interleave(G, dim=1)
    vr = v.repeat_interleave(G, dim=1)
    if mask is not None:
        return F.scaled_dot_product_attention(q, kr, vr, attn_mask=mask, scale=scale)
    return F.scaled_dot_product_attention(q, kr, vr, is_causal=causal, scale=scale)


def small_problem(B=1, Hq=4, Hkv=2, S=24, D=5, seed=3, dout=False):
    p = global_problem(B, Hq, Hkv, S, D, dtype="fp32", seed=seed, with_dout=dout)
    return p


def share_of(kind, S, Hq, Hkv, cp, rank, U=None):
    if kind == "contiguous":
        return oc.contiguous_share(S, Hq, Hkv, cp, rank)
    if kind == "head_tail":
        return oc.head_tail_share(S, Hq, Hkv, cp, rank)
    if kind == "ulysses":
        return oc.ulysses_share(S, Hq, Hkv, cp, rank)
    if kind == "hybrid":
        return oc.hybrid_share(S, Hq, Hkv, cp, U, rank)
    raise ValueError(kind)


def run_share(sh, q, k, v, scale, causal=True):
    qs = q[:, sh["q_heads"]][:, :, sh["q_pos"]]
    ks = k[:, sh["kv_heads"]]
    vs = v[:, sh["kv_heads"]]
    return oc.attention_rows(qs, ks, vs, sh["q_pos"], sh["kv_pos"], scale, causal)


SHARE_CASES = [
    ("contiguous", 4, None), ("head_tail", 2, None), ("head_tail", 3, None),
    ("ulysses", 2, None), ("hybrid", 4, 2),
]


# ----------------------------------------------------------------------------
# Golden fixtures
# ----------------------------------------------------------------------------
def test_worked_example_mask():
    ex = json.load(open(os.path.join(GOLDEN, "worked_example_mask.json")))
    q = np.array(ex["q"]).reshape(1, 1, -1, 1)
    k = np.array(ex["k"]).reshape(1, 1, -1, 1)
    v = np.array(ex["v"]).reshape(1, 1, -1, 1)
    out, lse = oc.attention_rows(q, k, v, ex["q_pos"], ex["kv_pos"], ex["scale"], True)
    np.testing.assert_allclose(out[0, 0, :, 0], ex["out"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[0, 0], ex["lse"], rtol=0, atol=1e-12)


def test_share_geometry_golden():
    geo = json.load(open(os.path.join(GOLDEN, "share_geometry.json")))
    for c in geo["cases"]:
        pos, n = oc.share_chunks(c["layout"], c["S"], c["cp"], c["rank"])
        assert pos == c["chunk_pos"] and n == c["chunk_len"], c
        rows = oc.chunk_row_positions(pos, n)
        assert oc.share_pairs(rows, np.arange(c["S"])) == c["pairs"], c
    for c in geo["ulysses"]:
        sh = oc.ulysses_share(c["S"], c["Hq"], c["Hkv"], c["cp"], c["rank"])
        assert list(sh["q_heads"]) == c["q_heads"] and list(sh["kv_heads"]) == c["kv_heads"]
        assert sh["q_pos"][0] == c["rows"][0] and sh["q_pos"][-1] + 1 == c["rows"][1]
        assert oc.share_pairs(sh["q_pos"], sh["kv_pos"]) == c["pairs"]
    for c in geo["hybrid"]:
        sh = oc.hybrid_share(c["S"], c["Hq"], c["Hkv"], c["cp"], c["ulysses"], c["rank"])
        assert list(sh["q_heads"]) == c["q_heads"] and list(sh["kv_heads"]) == c["kv_heads"]
        assert sh["q_pos"][0] == c["rows"][0] and sh["q_pos"][-1] + 1 == c["rows"][1]
        assert oc.share_pairs(sh["q_pos"], sh["kv_pos"]) == c["pairs"]
    for c in geo["errors"]:
        with pytest.raises(ValueError):
            oc.share_chunks(c["layout"], c["S"], c["cp"], c["rank"])


def test_head_tail_work_is_balanced_closed_form():
    """Head-Tail balance ([Trainer-CP] §0) as an integer identity: with 2P
    chunks of L rows, every rank has 2P*L^2 + L visible pairs per head."""
    for P, L in [(2, 3), (4, 5), (8, 2048), (3, 7)]:
        S = 2 * P * L
        for r in range(P):
            pos, n = oc.share_chunks("head_tail", S, P, r)
            rows = oc.chunk_row_positions(pos, n)
            assert oc.share_pairs(rows, np.arange(S)) == 2 * P * L * L + L


# ----------------------------------------------------------------------------
# Brute force and library special cases
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("kind,cp,U", SHARE_CASES)
def test_share_equals_rows_of_bruteforce_full(kind, cp, U):
    S, Hq, Hkv, D = 24, 4, 2, 5
    p = small_problem(S=S, Hq=Hq, Hkv=Hkv, D=D)
    q, k, v = _np(p.q), _np(p.k), _np(p.v)
    scale = 0.7
    full_out, full_lse = brute_full_causal(q, k, v, scale)
    for r in range(cp):
        sh = share_of(kind, S, Hq, Hkv, cp, r, U)
        out, lse = run_share(sh, q, k, v, scale)
        exp_out = full_out[:, sh["q_heads"]][:, :, sh["q_pos"]]
        exp_lse = full_lse[:, sh["q_heads"]][:, :, sh["q_pos"]]
        np.testing.assert_allclose(out, exp_out, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, exp_lse, rtol=0, atol=1e-12)


def test_full_matches_torch_sdpa_fp64_gqa():
    p = small_problem(B=2, Hq=6, Hkv=2, S=40, D=8, seed=5)
    q, k, v = p.q.double(), p.k.double(), p.v.double()
    scale = 1 / math.sqrt(8)
    ref = torch_sdpa_full(q, k, v, scale).numpy()
    pos = np.arange(40)
    out, _ = oc.attention_rows(q.numpy(), k.numpy(), v.numpy(), pos, pos, scale, True)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    ref_nc = torch_sdpa_full(q, k, v, scale, causal=False).numpy()
    out_nc, _ = oc.attention_rows(q.numpy(), k.numpy(), v.numpy(), pos, pos, scale, False)
    np.testing.assert_allclose(out_nc, ref_nc, rtol=0, atol=1e-12)


def test_offset_share_matches_sdpa_with_explicit_mask():
    """A share with a global offset equals SDPA given the boolean mask built
    from global positions (the first-version adapter of [CP-migration] §8)."""
    p = small_problem(B=1, Hq=4, Hkv=1, S=48, D=6, seed=7)
    q, k, v = p.q.double(), p.k.double(), p.v.double()
    scale = 0.4
    for kind, cp in [("contiguous", 3), ("head_tail", 2)]:
        for r in range(cp):
            sh = share_of(kind, 48, 4, 1, cp, r)
            qpos = torch.from_numpy(sh["q_pos"])
            mask = torch.arange(48)[None, :] <= qpos[:, None]
            ref = torch_sdpa_full(q[:, :, qpos], k, v, scale, mask=mask).numpy()
            out, _ = run_share(sh, q.numpy(), k.numpy(), v.numpy(), scale)
            np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def test_bwd_matches_torch_autograd_fp64():
    p = small_problem(B=1, Hq=4, Hkv=2, S=32, D=6, seed=11, dout=True)
    scale = 0.5
    for kind, cp in [("contiguous", 4), ("head_tail", 2), ("ulysses", 2)]:
        for r in range(cp):
            sh = share_of(kind, 32, 4, 2, cp, r)
            qh, kh = torch.from_numpy(sh["q_heads"]), torch.from_numpy(sh["kv_heads"])
            qpos = torch.from_numpy(sh["q_pos"])
            q = p.q.double()[:, qh][:, :, qpos].clone().requires_grad_(True)
            k = p.k.double()[:, kh].clone().requires_grad_(True)
            v = p.v.double()[:, kh].clone().requires_grad_(True)
            do = p.dout.double()[:, qh][:, :, qpos]
            mask = torch.arange(32)[None, :] <= qpos[:, None]
            out = torch_sdpa_full(q, k, v, scale, mask=mask)
            (out * do).sum().backward()
            dq, dk, dv = oc.attention_rows_bwd(q.detach().numpy(), k.detach().numpy(),
                                               v.detach().numpy(), do.numpy(),
                                               sh["q_pos"], sh["kv_pos"], scale)
            np.testing.assert_allclose(dq, q.grad.numpy(), rtol=0, atol=1e-11)
            np.testing.assert_allclose(dk, k.grad.numpy(), rtol=0, atol=1e-11)
            np.testing.assert_allclose(dv, v.grad.numpy(), rtol=0, atol=1e-11)


# ----------------------------------------------------------------------------
# Closed forms
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("kind,cp,U", SHARE_CASES)
def test_closed_form_uniform_softmax(kind, cp, U):
    """q = 0: every visible key has weight 1/(p+1): out = prefix mean of v,
    LSE = ln(p+1)."""
    S, Hq, Hkv, D = 24, 4, 2, 3
    rng = np.random.default_rng(0)
    v = rng.standard_normal((1, Hkv, S, D))
    k = rng.standard_normal((1, Hkv, S, D))
    q = np.zeros((1, Hq, S, D))
    for r in range(cp):
        sh = share_of(kind, S, Hq, Hkv, cp, r, U)
        out, lse = run_share(sh, q, k, v, 0.9)
        G = Hq // Hkv
        for hi, h in enumerate(sh["q_heads"]):
            hk = h // G
            for i, pos in enumerate(sh["q_pos"]):
                np.testing.assert_allclose(out[0, hi, i], v[0, hk, :pos + 1].mean(0), atol=1e-12)
                assert abs(lse[0, hi, i] - math.log(pos + 1)) < 1e-12


def test_closed_form_equal_keys_and_unit_values():
    S, D = 20, 4
    rng = np.random.default_rng(1)
    q = rng.standard_normal((1, 2, S, D))
    u = rng.standard_normal(D)
    k = np.broadcast_to(u, (1, 1, S, D)).copy()
    v = rng.standard_normal((1, 1, S, D))
    scale = 0.8
    for cp, r in [(4, 2), (4, 3)]:
        sh = oc.contiguous_share(S, 2, 1, cp, r)
        out, lse = run_share(sh, q, k, v, scale)
        for i, pos in enumerate(sh["q_pos"]):
            for h in range(2):
                np.testing.assert_allclose(out[0, h, i], v[0, 0, :pos + 1].mean(0), atol=1e-12)
                assert abs(lse[0, h, i] - (scale * q[0, h, pos] @ u + math.log(pos + 1))) < 1e-12
    ones = np.ones_like(v)
    out, _ = oc.attention_rows(q, rng.standard_normal((1, 1, S, D)), ones,
                               np.arange(S), np.arange(S), scale, True)
    np.testing.assert_allclose(out, 1.0, atol=1e-13)


def test_closed_form_row_zero_sees_one_key():
    p = small_problem(S=16, Hq=2, Hkv=2, D=4)
    q, k, v = _np(p.q), _np(p.k), _np(p.v)
    out, lse = oc.attention_rows(q[:, :, :1], k, v, [0], np.arange(16), 0.3, True)
    np.testing.assert_allclose(out[0, :, 0], v[0, :, 0], atol=1e-14)
    np.testing.assert_allclose(lse[0, :, 0], 0.3 * np.sum(q[0, :, 0] * k[0, :, 0], axis=1), atol=1e-14)


def test_fully_masked_row_and_noncausal_uniform():
    q = np.zeros((1, 1, 2, 2))
    k = np.ones((1, 1, 3, 2))
    v = np.arange(6.0).reshape(1, 1, 3, 2)
    out, lse = oc.attention_rows(q, k, v, [4, 9], [10, 11, 12], 1.0, True)
    assert np.all(out == 0) and np.all(np.isneginf(lse))
    out, lse = oc.attention_rows(q, k, v, [4, 9], [10, 11, 12], 1.0, False)
    np.testing.assert_allclose(out[0, 0], [[2.0, 3.0]] * 2, atol=1e-14)
    np.testing.assert_allclose(lse, math.log(3), atol=1e-14)
    dq, dk, dv = oc.attention_rows_bwd(q, k, v, np.ones_like(q), [4, 9], [10, 11, 12], 1.0, True)
    assert np.all(dq == 0) and np.all(dk == 0) and np.all(dv == 0)


def test_kv_permutation_invariance():
    """Keys carry their own positions: permuting K/V rows with their positions
    (e.g. the raw rank order of a Head-Tail all-gather) changes nothing."""
    p = small_problem(S=24, Hq=2, Hkv=1, D=4, seed=9)
    q, k, v = _np(p.q), _np(p.k), _np(p.v)
    sh = oc.head_tail_share(24, 2, 1, 3, 1)
    out, lse = run_share(sh, q, k, v, 0.6)
    perm = np.random.default_rng(2).permutation(24)
    out2, lse2 = oc.attention_rows(q[:, :, sh["q_pos"]], k[:, :, perm], v[:, :, perm],
                                   sh["q_pos"], perm, 0.6, True)
    np.testing.assert_allclose(out2, out, atol=1e-12)
    np.testing.assert_allclose(lse2, lse, atol=1e-12)


def test_kv_permutation_equivariance_of_backward():
    """The backward with K/V rows permuted together with their positions: dQ
    is unchanged and dK/dV are the natural-order rows in the permuted order
    (the storage-order convention of the GPU path's partial dK/dV)."""
    p = small_problem(S=24, Hq=2, Hkv=1, D=4, seed=10, dout=True)
    q, k, v, do = _np(p.q), _np(p.k), _np(p.v), _np(p.dout)
    sh = oc.head_tail_share(24, 2, 1, 3, 2)
    qs, dos = q[:, :, sh["q_pos"]], do[:, :, sh["q_pos"]]
    dq, dk, dv = oc.attention_rows_bwd(qs, k, v, dos, sh["q_pos"], sh["kv_pos"], 0.6, True)
    perm = np.random.default_rng(4).permutation(24)
    dq2, dk2, dv2 = oc.attention_rows_bwd(qs, k[:, :, perm], v[:, :, perm], dos, sh["q_pos"], perm, 0.6, True)
    np.testing.assert_allclose(dq2, dq, atol=1e-12)
    np.testing.assert_allclose(dk2, dk[:, :, perm], atol=1e-12)
    np.testing.assert_allclose(dv2, dv[:, :, perm], atol=1e-12)
    assert np.abs(dk).max() > 1e-3   # not vacuous


# ----------------------------------------------------------------------------
# Reassembly and gradient-sharding invariants
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("kind,cp,U", SHARE_CASES)
def test_shares_reassemble_full_output_and_grads(kind, cp, U):
    S, Hq, Hkv, D = 24, 4, 2, 4
    p = small_problem(S=S, Hq=Hq, Hkv=Hkv, D=D, seed=13, dout=True)
    q, k, v, do = _np(p.q), _np(p.k), _np(p.v), _np(p.dout)
    scale = 0.55
    pos = np.arange(S)
    # The unsharded reference comes from torch (output) and torch autograd (grads).
    qt, kt, vt = (p.q.double().requires_grad_(True), p.k.double().requires_grad_(True),
                  p.v.double().requires_grad_(True))
    ref = torch_sdpa_full(qt, kt, vt, scale)
    (ref * p.dout.double()).sum().backward()
    out_full = np.full_like(q, np.nan)
    dq_full = np.full_like(q, np.nan)
    dk_sum = np.zeros_like(k)
    dv_sum = np.zeros_like(v)
    for r in range(cp):
        sh = share_of(kind, S, Hq, Hkv, cp, r, U)
        out, _ = run_share(sh, q, k, v, scale)
        ix = np.ix_(range(1), sh["q_heads"], sh["q_pos"])
        out_full[ix] = out
        dq, dk, dv = oc.attention_rows_bwd(q[ix], k[:, sh["kv_heads"]], v[:, sh["kv_heads"]],
                                           do[ix], sh["q_pos"], sh["kv_pos"], scale)
        dq_full[ix] = dq
        dk_sum[:, sh["kv_heads"]] += dk
        dv_sum[:, sh["kv_heads"]] += dv
    np.testing.assert_allclose(out_full, ref.detach().numpy(), atol=1e-12)
    np.testing.assert_allclose(dq_full, qt.grad.numpy(), atol=1e-11)
    # Summing every rank's partial dK/dV is the reduce-scatter(sum) of
    # [CP-migration] §6.1; for head-sharded shares each KV head has one owner.
    np.testing.assert_allclose(dk_sum, kt.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dv_sum, vt.grad.numpy(), atol=1e-11)


# ----------------------------------------------------------------------------
# Finite differences
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("kind,cp,rank", [("contiguous", 4, 2), ("head_tail", 2, 1)])
def test_bwd_central_finite_differences(kind, cp, rank):
    S, Hq, Hkv, D = 16, 4, 2, 3
    p = small_problem(S=S, Hq=Hq, Hkv=Hkv, D=D, seed=17, dout=True)
    sh = share_of(kind, S, Hq, Hkv, cp, rank)
    q = _np(p.q)[:, :, sh["q_pos"]]
    k, v = _np(p.k), _np(p.v)
    do = _np(p.dout)[:, :, sh["q_pos"]]
    scale = 0.8

    def loss(qq, kk, vv):
        o, _ = oc.attention_rows(qq, kk, vv, sh["q_pos"], sh["kv_pos"], scale)
        return float(np.sum(o * do))

    dq, dk, dv = oc.attention_rows_bwd(q, k, v, do, sh["q_pos"], sh["kv_pos"], scale)
    h = 1e-6
    rng = np.random.default_rng(0)
    for name, arr, grad in [("q", q, dq), ("k", k, dk), ("v", v, dv)]:
        for _ in range(12):
            idx = tuple(int(rng.integers(0, n)) for n in arr.shape)
            plus, minus = arr.copy(), arr.copy()
            plus[idx] += h
            minus[idx] -= h
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            args_p[name], args_m[name] = plus, minus
            fd = (loss(**{"qq": args_p["q"], "kk": args_p["k"], "vv": args_p["v"]})
                  - loss(**{"qq": args_m["q"], "kk": args_m["k"], "vv": args_m["v"]})) / (2 * h)
            assert abs(fd - grad[idx]) <= 1e-6 * max(1.0, abs(grad[idx])), (name, idx, fd, grad[idx])


def test_kv_index_subset_of_dk_dv():
    p = small_problem(S=20, Hq=2, Hkv=1, D=3, seed=19, dout=True)
    q, k, v, do = _np(p.q), _np(p.k), _np(p.v), _np(p.dout)
    pos = np.arange(20)
    _, dk, dv = oc.attention_rows_bwd(q, k, v, do, pos, pos, 0.5)
    sel = np.array([0, 7, 19])
    _, dk2, dv2 = oc.attention_rows_bwd(q, k, v, do, pos, pos, 0.5, kv_index=sel)
    np.testing.assert_allclose(dk2, dk[:, :, sel], atol=1e-14)
    np.testing.assert_allclose(dv2, dv[:, :, sel], atol=1e-14)
    dq3, dk3, _ = oc.attention_rows_bwd(q, k, v, do, pos, pos, 0.5, kv_index=sel, want_dq=False)
    assert np.all(dq3 == 0)
    np.testing.assert_allclose(dk3, dk[:, :, sel], atol=1e-14)
    # dQ of a subset of rows, computed from those rows alone.
    dq_all, _, _ = oc.attention_rows_bwd(q, k, v, do, pos, pos, 0.5)
    rows = np.array([3, 11, 19])
    dq4, _, _ = oc.attention_rows_bwd(q[:, :, rows], k, v, do[:, :, rows], pos[rows], pos, 0.5,
                                      kv_index=np.array([], dtype=np.int64))
    np.testing.assert_allclose(dq4, dq_all[:, :, rows], atol=1e-14)


# ----------------------------------------------------------------------------
# Planted mistakes: each must be caught by a pin above
# ----------------------------------------------------------------------------
def _fails(fn):
    try:
        fn()
    except AssertionError:
        return True
    return False


def test_planted_strict_causal_is_caught(monkeypatch):
    monkeypatch.setattr(oc, "visible", lambda qp, kp, c, docs=None: np.asarray(kp)[None, :] < np.asarray(qp)[:, None])
    assert _fails(lambda: test_share_equals_rows_of_bruteforce_full("contiguous", 4, None))


def test_planted_local_offset_is_caught(monkeypatch):
    """The bug [CP-migration] §8 warns about: masking with local row indices."""
    real = oc.visible
    monkeypatch.setattr(oc, "visible", lambda qp, kp, c, docs=None: real(np.asarray(qp) - np.asarray(qp)[0], kp, c, docs))
    assert _fails(lambda: test_share_equals_rows_of_bruteforce_full("contiguous", 4, None))


def test_planted_strided_gqa_is_caught(monkeypatch):
    monkeypatch.setattr(oc, "kv_head_of", lambda h, nq, nk: h % nk)
    assert _fails(test_full_matches_torch_sdpa_fp64_gqa)


def test_planted_head_tail_off_by_one_is_caught(monkeypatch):
    real = oc.share_chunks

    def bad(layout, S, P, r):
        pos, n = real(layout, S, P, r)
        if layout == "head_tail":
            pos = [pos[0], (2 * P - r) * n % S]
        return pos, n
    monkeypatch.setattr(oc, "share_chunks", bad)
    assert _fails(test_share_geometry_golden)


# ----------------------------------------------------------------------------
# Ulysses exchange
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("U", [2, 4])
def test_ulysses_exchange_matches_the_share_definition(U):
    """Sequence shards of one global tensor, exchanged, give each rank the
    global tensor's head slice over the whole sequence -- the Ulysses share
    the oracle defines independently (ulysses_share) -- and the inverse
    exchange restores the shards."""
    rng = np.random.default_rng(U)
    B, N, S, D = 2, 8, 24, 3
    X = rng.standard_normal((B, N, S, D))
    L = S // U
    shards = [X[:, :, p * L:(p + 1) * L] for p in range(U)]
    heads = oc.ulysses_seq_to_head(shards)
    for u in range(U):
        sh = oc.ulysses_share(S, N, N, U, u)
        np.testing.assert_array_equal(heads[u], X[:, sh["q_heads"]][:, :, sh["q_pos"]])
    back = oc.ulysses_head_to_seq(heads)
    for p in range(U):
        np.testing.assert_array_equal(back[p], shards[p])


def test_ulysses_exchange_brute_force_and_hybrid_subgroup():
    """Element by element: rank u's row p*L+t of local head h is rank p's row t
    of global head u*N/U+h. Inside a Hybrid co-group (U = 2 of P = 4) the
    exchange then the K/V all-gather over the co-group give hybrid_share's
    heads and rows."""
    rng = np.random.default_rng(7)
    U, B, N, L, D = 3, 1, 6, 2, 2
    shards = [rng.standard_normal((B, N, L, D)) for _ in range(U)]
    heads = oc.ulysses_seq_to_head(shards)
    n = N // U
    for u in range(U):
        for p in range(U):
            for h in range(n):
                for t in range(L):
                    assert np.array_equal(heads[u][0, h, p * L + t], shards[p][0, u * n + h, t])
    # Hybrid: P = 4 ranks, U = 2, C = 2; rank r = co*U + u holds rows of its
    # sequence shard r (length S/P) before the exchange.
    S, P, Uh = 16, 4, 2
    X = rng.standard_normal((1, 4, S, 2))
    Lr = S // P
    for co in range(P // Uh):
        group = [X[:, :, (co * Uh + u) * Lr:(co * Uh + u + 1) * Lr] for u in range(Uh)]
        after = oc.ulysses_seq_to_head(group)
        for u in range(Uh):
            sh = oc.hybrid_share(S, 4, 4, P, Uh, co * Uh + u)
            np.testing.assert_array_equal(after[u], X[:, sh["q_heads"]][:, :, sh["q_pos"]])


# ----------------------------------------------------------------------------
# Packed variable-length sequences
# ----------------------------------------------------------------------------
PACKED = [[7, 9, 8], [24], [3, 1, 5, 2, 13], [12, 12]]


def _starts(lengths):
    return np.concatenate([[0], np.cumsum(lengths)[:-1]]).astype(np.int64)


@pytest.mark.parametrize("lengths", PACKED, ids=["-".join(map(str, l)) for l in PACKED])
def test_packed_sequences_are_independent_causal_attentions(lengths):
    """Packed attention = each sequence's own causal attention (torch float64
    SDPA on the sequence alone), forward and backward (autograd), GQA."""
    S = 24
    p = small_problem(Hq=4, Hkv=2, S=S, D=5, seed=21, dout=True)
    q, k, v, do = p.q.double(), p.k.double(), p.v.double(), p.dout.double()
    starts = _starts(lengths)
    pos = np.arange(S)
    out, _ = oc.attention_rows(q.numpy(), k.numpy(), v.numpy(), pos, pos, 0.7, True, doc_starts=starts)
    dq, dk, dv = oc.attention_rows_bwd(q.numpy(), k.numpy(), v.numpy(), do.numpy(), pos, pos, 0.7, True,
                                       doc_starts=starts)
    qr, kr, vr = (t.clone().requires_grad_(True) for t in (q, k, v))
    outs = []
    for a, n in zip(starts, lengths):
        kk = kr[:, :, a:a + n].repeat_interleave(2, dim=1)
        vv = vr[:, :, a:a + n].repeat_interleave(2, dim=1)
        outs.append(F.scaled_dot_product_attention(qr[:, :, a:a + n], kk, vv, is_causal=True, scale=0.7))
    ref = torch.cat(outs, dim=2)
    ref.backward(do)
    np.testing.assert_allclose(out, ref.detach().numpy(), atol=1e-12)
    np.testing.assert_allclose(dq, qr.grad.numpy(), atol=1e-10)
    np.testing.assert_allclose(dk, kr.grad.numpy(), atol=1e-10)
    np.testing.assert_allclose(dv, vr.grad.numpy(), atol=1e-10)


def test_packed_closed_form_and_pair_count():
    """Q = 0: each row averages v over its own sequence up to itself, and
    LSE = ln(number of those keys). share_pairs counts the same keys."""
    S, lengths = 24, [3, 1, 5, 2, 13]
    starts = _starts(lengths)
    p = small_problem(Hq=2, Hkv=1, S=S, D=3, seed=22)
    v = p.v.double().numpy()
    pos = np.arange(S)
    out, lse = oc.attention_rows(np.zeros((1, 2, S, 3)), p.k.double().numpy(), v, pos, pos, 1.0, True,
                                 doc_starts=starts)
    for i in range(S):
        a = starts[starts <= i].max()
        np.testing.assert_allclose(out[0, :, i], np.broadcast_to(v[0, 0, a:i + 1].mean(axis=0), (2, 3)), atol=1e-13)
        np.testing.assert_allclose(lse[0, :, i], np.log(i - a + 1), atol=1e-13)
    brute = sum(1 for i in range(S) for j in range(S) if j <= i and starts[starts <= i].max() <= j)
    assert oc.share_pairs(pos, pos, True, starts) == brute
    # Keys permuted with their positions: same count.
    perm = np.random.default_rng(3).permutation(S)
    assert oc.share_pairs(pos[::-1], perm, True, starts) == brute


@pytest.mark.parametrize("kind,cp", [("contiguous", 3), ("head_tail", 3)])
def test_packed_shares_reassemble(kind, cp):
    """Every rank's share of a packed sequence (sequences cut at rank
    boundaries) equals the matching rows of the full packed attention."""
    S, lengths = 24, [7, 9, 8]
    starts = _starts(lengths)
    p = small_problem(Hq=2, Hkv=1, S=S, D=4, seed=23)
    q, k, v = _np(p.q), _np(p.k), _np(p.v)
    full, full_l = oc.attention_rows(q, k, v, np.arange(S), np.arange(S), 0.5, True, doc_starts=starts)
    for r in range(cp):
        sh = share_of(kind, S, 2, 1, cp, r)
        out, lse = oc.attention_rows(q[:, :, sh["q_pos"]], k, v, sh["q_pos"], sh["kv_pos"], 0.5, True,
                                     doc_starts=starts)
        np.testing.assert_allclose(out, full[:, :, sh["q_pos"]], atol=1e-13)
        np.testing.assert_allclose(lse, full_l[:, :, sh["q_pos"]], atol=1e-13)


def test_planted_sequence_boundary_off_by_one_is_caught(monkeypatch):
    real = oc.doc_of
    monkeypatch.setattr(oc, "doc_of", lambda pos, starts: real(np.asarray(pos) - 1, starts))
    assert _fails(lambda: test_packed_sequences_are_independent_causal_attentions([7, 9, 8]))


# ----------------------------------------------------------------------------
# User attention masks merged with the CP mask
# ----------------------------------------------------------------------------
def test_user_mask_is_anded_with_the_cp_mask():
    """A boolean user mask ([B, 1, S, S], broadcast over heads) merged by AND
    with the causal mask equals torch float64 SDPA given the AND of the two as
    its mask, forward and autograd backward; a share (global offset) sees the
    same rows of it."""
    S = 24
    p = small_problem(B=2, Hq=4, Hkv=2, S=S, D=5, seed=31, dout=True)
    q, k, v, do = p.q.double(), p.k.double(), p.v.double(), p.dout.double()
    rng = np.random.default_rng(31)
    um = rng.random((2, 1, S, S)) < 0.7
    um[:, :, np.arange(S), np.arange(S)] = True          # every row keeps its own key
    pos = np.arange(S)
    out, _ = oc.attention_rows(q.numpy(), k.numpy(), v.numpy(), pos, pos, 0.6, True, user_mask=um)
    dq, dk, dv = oc.attention_rows_bwd(q.numpy(), k.numpy(), v.numpy(), do.numpy(), pos, pos, 0.6, True,
                                       user_mask=um)
    both = torch.from_numpy(um & np.tril(np.ones((S, S), dtype=bool)))
    qr, kr, vr = (t.clone().requires_grad_(True) for t in (q, k, v))
    ref = F.scaled_dot_product_attention(qr, kr.repeat_interleave(2, dim=1), vr.repeat_interleave(2, dim=1),
                                         attn_mask=both, scale=0.6)
    ref.backward(do)
    np.testing.assert_allclose(out, ref.detach().numpy(), atol=1e-12)
    np.testing.assert_allclose(dq, qr.grad.numpy(), atol=1e-10)
    np.testing.assert_allclose(dk, kr.grad.numpy(), atol=1e-10)
    np.testing.assert_allclose(dv, vr.grad.numpy(), atol=1e-10)
    # A Head-Tail share with the mask rows of its own queries.
    sh = oc.head_tail_share(S, 4, 2, 3, 1)
    o2, _ = oc.attention_rows(q.numpy()[:, :, sh["q_pos"]], k.numpy(), v.numpy(), sh["q_pos"], pos, 0.6, True,
                              user_mask=um[:, :, sh["q_pos"]])
    np.testing.assert_allclose(o2, out[:, :, sh["q_pos"]], atol=1e-13)


def test_additive_user_mask_matches_sdpa():
    """An additive float mask (finite biases and -inf) on top of the causal
    mask equals torch float64 SDPA given causal -inf plus the same bias,
    forward and autograd backward."""
    S = 20
    p = small_problem(B=1, Hq=2, Hkv=1, S=S, D=4, seed=32, dout=True)
    q, k, v, do = p.q.double(), p.k.double(), p.v.double(), p.dout.double()
    rng = np.random.default_rng(32)
    bias = rng.normal(0.0, 2.0, (1, 2, S, S))
    bias[rng.random((1, 2, S, S)) < 0.2] = -np.inf
    bias[:, :, np.arange(S), np.arange(S)] = 0.0                     # every row keeps its own key
    pos = np.arange(S)
    out, lse = oc.attention_rows(q.numpy(), k.numpy(), v.numpy(), pos, pos, 0.5, True, user_mask=bias)
    dq, dk, dv = oc.attention_rows_bwd(q.numpy(), k.numpy(), v.numpy(), do.numpy(), pos, pos, 0.5, True,
                                       user_mask=bias)
    full = torch.from_numpy(np.where(np.tril(np.ones((S, S), dtype=bool)), bias, -np.inf))
    qr, kr, vr = (t.clone().requires_grad_(True) for t in (q, k, v))
    ref = F.scaled_dot_product_attention(qr, kr.repeat_interleave(2, dim=1), vr.repeat_interleave(2, dim=1),
                                         attn_mask=full, scale=0.5)
    ref.backward(do)
    np.testing.assert_allclose(out, ref.detach().numpy(), atol=1e-12)
    np.testing.assert_allclose(dq, qr.grad.numpy(), atol=1e-10)
    np.testing.assert_allclose(dk, kr.grad.numpy(), atol=1e-10)
    np.testing.assert_allclose(dv, vr.grad.numpy(), atol=1e-10)
    # LSE: logsumexp of the biased scaled scores (torch's own).
    sc = 0.5 * (q @ k.repeat_interleave(2, dim=1).transpose(-1, -2)) + full
    np.testing.assert_allclose(lse, torch.logsumexp(sc, dim=-1).numpy(), atol=1e-12)


def test_additive_hide_values_equal_the_boolean_mask():
    """Additive values at or below the hide threshold (-1e4, -1e9, -1e30, the
    float32 minimum, -inf) hide their key: such a mask (with 0 elsewhere)
    gives the same out, LSE and gradients as the boolean mask of its 0
    entries, whose AND with the CP mask is pinned against torch SDPA above.
    Rows where every key is hidden get out = 0, LSE = -inf and no gradient."""
    S = 24
    p = small_problem(B=1, Hq=4, Hkv=2, S=S, D=6, seed=33, dout=True)
    q, k, v, do = (t.double().numpy() for t in (p.q, p.k, p.v, p.dout))
    rng = np.random.default_rng(33)
    keep = rng.random((1, 4, S, S)) < 0.6
    keep[:, :, 5] = False                                          # a fully padded row
    hides = np.array([-1e4, -1e9, -1e30, float(np.finfo(np.float32).min), -np.inf])
    bias = np.where(keep, 0.0, hides[rng.integers(0, hides.size, keep.shape)])
    pos = np.arange(S)
    ob, lb = oc.attention_rows(q, k, v, pos, pos, 0.4, True, user_mask=keep)
    oa, la = oc.attention_rows(q, k, v, pos, pos, 0.4, True, user_mask=bias)
    np.testing.assert_array_equal(oa, ob)
    np.testing.assert_array_equal(la, lb)
    gb = oc.attention_rows_bwd(q, k, v, do, pos, pos, 0.4, True, user_mask=keep)
    ga = oc.attention_rows_bwd(q, k, v, do, pos, pos, 0.4, True, user_mask=bias)
    for x, y in zip(ga, gb):
        np.testing.assert_array_equal(x, y)
    assert np.all(oa[:, :, 5] == 0) and np.all(la[:, :, 5] == -np.inf)
    assert np.all(ga[0][:, :, 5] == 0)


def test_additive_bias_above_the_threshold_shifts_the_lse():
    """A bias just above the hide threshold is a bias: when every key of a
    row carries the same bias c, softmax is unchanged and the LSE moves by
    exactly c (closed form), for c = -9999 and for a large positive c."""
    S = 16
    p = small_problem(B=1, Hq=2, Hkv=1, S=S, D=4, seed=34, dout=True)
    q, k, v, do = (t.double().numpy() for t in (p.q, p.k, p.v, p.dout))
    pos = np.arange(S)
    o0, l0 = oc.attention_rows(q, k, v, pos, pos, 0.5, True)
    g0 = oc.attention_rows_bwd(q, k, v, do, pos, pos, 0.5, True)
    for c in (-9999.0, 5000.0):
        bias = np.full((1, 1, S, S), c)
        o1, l1 = oc.attention_rows(q, k, v, pos, pos, 0.5, True, user_mask=bias)
        np.testing.assert_allclose(o1, o0, atol=1e-12)
        np.testing.assert_allclose(l1, l0 + c, atol=1e-9)
        g1 = oc.attention_rows_bwd(q, k, v, do, pos, pos, 0.5, True, user_mask=bias)
        for x, y in zip(g1, g0):
            np.testing.assert_allclose(x, y, atol=1e-10)


def test_planted_hide_threshold_mistake_is_caught(monkeypatch):
    """Hiding only -inf (the threshold ignored) breaks the boolean-mask pin."""
    monkeypatch.setattr(oc, "MASK_HIDE", -np.inf)
    assert _fails(test_additive_hide_values_equal_the_boolean_mask)
