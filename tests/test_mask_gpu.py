"""GPU parity of user attention masks merged with the CP mask by AND
("新流程 CP 多通信模式迁移设计方案" §8: a boolean attn_mask and the CP mask are
combined, the user mask is never replaced) against the oracle, forward and
backward, on every rank: a sliding window broadcast over heads, a random
per-head mask, fully masked rows, a ragged key count and the fp32 path;
additive masks with finite biases, -inf, and the large negative values
padding masks use for "hidden" (-1e4, -1e9, -1e30, the float32 minimum: at or
below the hide threshold, so rows of them come out empty in both dtypes), plus
large positive biases."""
import math

import numpy as np
import pytest
import torch

import oracle.cp_share as oc
from context_causal_attention_attn_amd import cp_attn_bwd, cp_attn_fwd, cut_share
from synthetic import global_problem
from tests._share_cases import oracle_share, to_f64

pytestmark = pytest.mark.gpu


def rel_l2(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def make_mask(kind, osh, B, Hq, S, rng, dtype="bf16"):
    """Mask rows of the share's local queries: [B, 1 or Hq, Sq, S], bool or
    float32 (additive)."""
    q_pos = osh["q_pos"]
    if kind == "window":            # keys at most 300 positions back, all heads
        m = (q_pos[:, None] - np.arange(S)[None, :]) < 300
        m = np.broadcast_to(m, (B, 1) + m.shape).copy()
    elif kind == "additive":        # float biases, 15 % -inf, some rows fully hidden
        m = rng.normal(0.0, 1.5, (B, Hq, q_pos.size, S)).astype(np.float32)
        m[rng.random(m.shape) < 0.15] = -np.inf
        m[:, :, ::37] = -np.inf
    elif kind == "padding":         # additive: every padding style of "hidden", large biases
        shape = (B, Hq, q_pos.size, S)
        m = rng.normal(0.0, 1.5, shape).astype(np.float32)
        hides = np.array([-1e4, -1e9, -1e30, np.finfo(np.float32).min, -np.inf], dtype=np.float32)
        sel = rng.random(shape) < 0.15
        m[sel] = hides[rng.integers(0, hides.size, int(sel.sum()))]
        m[:, :, ::37] = -1e9                                # padding rows of each style
        m[:, :, 5::37] = np.finfo(np.float32).min
        m[:, :, 9::37] = -1e30
        m[rng.random(shape) < 0.003] = 60.0                 # late score spikes (the forward's redo path)
        # Rows that see these keys get an LSE near the bias (bf16: 1000; fp32,
        # whose LSE gate is 1e-4 absolute, 100: float32 keeps 1e-5 there).
        m[:, :, :, S // 2:S // 2 + 4] = 1000.0 if dtype == "bf16" else 100.0
        m[:, :, ::37] = -1e9
    elif kind == "additive_h1":     # float biases shared by every head, 15 % -inf, some rows hidden
        m = rng.normal(0.0, 1.5, (B, 1, q_pos.size, S)).astype(np.float32)
        m[rng.random(m.shape) < 0.15] = -np.inf
        m[:, :, ::37] = -np.inf
    elif kind == "random_b1":       # random per head, shared by the batch
        m = rng.random((1, Hq, q_pos.size, S)) < 0.75
        m[:, :, ::37] = False
    elif kind == "random_11":       # one random mask for every batch and head
        m = rng.random((1, 1, q_pos.size, S)) < 0.75
        m[:, :, ::37] = False
    else:                           # random per head, 25 % hidden, some rows fully hidden
        m = rng.random((B, Hq, q_pos.size, S)) < 0.75
        m[:, :, ::37] = False
    return m


CASES = [
    # mask, kind, S, Hq, Hkv, D, cp, dtype
    ("window", "contiguous", 2048, 8, 2, 128, 4, "bf16"),
    ("window", "head_tail", 2048, 8, 2, 128, 4, "bf16"),
    ("random", "contiguous", 1000, 4, 2, 64, 2, "bf16"),     # ragged key count (1000)
    ("random", "head_tail", 1024, 4, 4, 128, 4, "bf16"),
    ("random_b1", "head_tail", 1000, 8, 2, 128, 2, "bf16"),   # per-head mask broadcast over the batch
    ("random_11", "contiguous", 1100, 4, 2, 64, 2, "bf16"),   # one mask for all batches and heads
    ("random", "head_tail", 512, 2, 1, 64, 4, "fp32"),
    ("additive", "head_tail", 2048, 8, 2, 128, 4, "bf16"),
    ("additive", "contiguous", 1000, 4, 2, 64, 2, "bf16"),    # ragged key count
    ("additive_h1", "head_tail", 2048, 8, 2, 128, 4, "bf16"),  # biases shared by the heads
    ("additive_h1", "contiguous", 1000, 8, 2, 64, 2, "bf16"),  # ... with a ragged key count
    ("additive", "contiguous", 512, 2, 1, 64, 4, "fp32"),
    ("padding", "head_tail", 2048, 8, 2, 128, 4, "bf16"),
    ("padding", "contiguous", 1000, 4, 2, 64, 2, "bf16"),     # ragged key count
    ("padding", "head_tail", 512, 2, 1, 64, 4, "fp32"),
]


@pytest.mark.parametrize("case", CASES, ids=["-".join(map(str, c)) for c in CASES])
def test_user_mask_fwd_bwd_all_ranks(case):
    mask_kind, kind, S, Hq, Hkv, D, cp, dtype = case
    B = 2
    prob = global_problem(B, Hq, Hkv, S, D, dtype=dtype, seed=17, with_dout=True)
    rng = np.random.default_rng(17)
    dev = torch.device("cuda")
    tol_o, tol_l, tol_g = (2e-2, 1e-3, 1e-2) if dtype == "bf16" else (1e-4, 1e-4, 1e-4)
    for r in range(cp):
        q, k, v = prob.q.to(dev), prob.k.to(dev), prob.v.to(dev)
        sh = cut_share(kind, q, k, v, cp, r)
        osh = oracle_share(kind, S, Hq, Hkv, cp, r)
        m = make_mask(mask_kind, osh, B, Hq, S, rng, dtype)
        mt = torch.from_numpy(m).to(dev)
        scale = 1.0 / math.sqrt(D)
        out, lse = cp_attn_fwd(sh.q, sh.k, sh.v, sh.q_chunk_pos, layout=sh.layout, softmax_scale=scale,
                               attn_mask=mt)
        dout = sh.take_rows(prob.dout.to(dev))
        dq, dk, dv = cp_attn_bwd(sh.q, sh.k, sh.v, out, lse, dout, sh.q_chunk_pos, layout=sh.layout,
                                 softmax_scale=scale, attn_mask=mt)
        torch.cuda.synchronize()
        rows = torch.from_numpy(osh["q_pos"])
        qs, dos = to_f64(prob.q[:, :, rows]), to_f64(prob.dout[:, :, rows])
        mo = m if m.dtype == bool else m.astype(np.float64)
        ref_o, ref_l = oc.attention_rows(qs, to_f64(prob.k), to_f64(prob.v), osh["q_pos"], osh["kv_pos"], scale,
                                         True, user_mask=mo)
        ref_g = oc.attention_rows_bwd(qs, to_f64(prob.k), to_f64(prob.v), dos, osh["q_pos"], osh["kv_pos"],
                                      scale, True, user_mask=mo)
        o, l = to_f64(out), to_f64(lse)
        assert np.array_equal(np.isneginf(l), np.isneginf(ref_l)), "fully masked rows differ"
        fin = np.isfinite(ref_l)
        err_o = float(np.max(np.abs(o - ref_o)))
        err_l = float(np.max(np.abs(l[fin] - ref_l[fin])))
        errs = [rel_l2(to_f64(g), rg) for g, rg in zip((dq, dk, dv), ref_g)]
        print(f"mask {case} r{r}: out {err_o:.3e} lse {err_l:.3e} dq {errs[0]:.3e} dk {errs[1]:.3e} "
              f"dv {errs[2]:.3e}", flush=True)
        assert err_o <= tol_o and err_l <= tol_l and max(errs) <= tol_g
        if mask_kind in ("random", "random_b1", "random_11", "additive", "additive_h1", "padding"):
            assert torch.all(out[:, :, ::37] == 0) and torch.all(dq[:, :, ::37] == 0)


PURE_CASES = [
    # kind, S, Hq, Hkv, D, cp, rank, mask heads (1: broadcast over heads)
    ("contiguous", 1000, 4, 2, 64, 2, 1, 4),      # ragged key count, per-head mask
    ("head_tail", 2048, 8, 2, 128, 4, 2, 1),      # broadcast over heads
]


@pytest.mark.parametrize("case", PURE_CASES, ids=["-".join(map(str, c)) for c in PURE_CASES])
def test_additive_mask_of_zeros_and_hides_matches_the_boolean_mask(case):
    """An additive mask whose values are only 0 (either sign) and hiding
    values (-inf, -1e9, the float32 minimum, -1e4) takes the boolean mask's
    bit-table path: bitwise the results of the boolean mask it encodes, in
    both directions. A mask with one small nonzero bias does not, and the
    call after it (same workspace) is pure again."""
    kind, S, Hq, Hkv, D, cp, r, mh = case
    B = 2
    dev = torch.device("cuda")
    prob = global_problem(B, Hq, Hkv, S, D, dtype="bf16", seed=23, with_dout=True)
    sh = cut_share(kind, prob.q.to(dev), prob.k.to(dev), prob.v.to(dev), cp, r)
    Sq = sh.q.shape[2]
    g = torch.Generator(device="cpu").manual_seed(29)
    keep = torch.rand((B, mh, Sq, S), generator=g) < 0.8
    keep[:, :, ::37] = False
    hides = torch.tensor([float("-inf"), -1e9, torch.finfo(torch.float32).min, -1e4])
    hide = hides[torch.randint(0, 4, keep.shape, generator=g)]
    zero = torch.where(torch.rand(keep.shape, generator=g) < 0.5, torch.tensor(0.0), torch.tensor(-0.0))
    add = torch.where(keep, zero, hide).to(dev)
    keep = keep.to(dev)
    scale = 1.0 / math.sqrt(D)
    dout = sh.take_rows(prob.dout.to(dev))
    ws = torch.empty(64 << 20, dtype=torch.uint8, device=dev)

    def run(m):
        out, lse = cp_attn_fwd(sh.q, sh.k, sh.v, sh.q_chunk_pos, layout=sh.layout, softmax_scale=scale,
                               attn_mask=m, workspace=ws)
        grads = cp_attn_bwd(sh.q, sh.k, sh.v, out, lse, dout, sh.q_chunk_pos, layout=sh.layout,
                            softmax_scale=scale, attn_mask=m, workspace=ws)
        torch.cuda.synchronize()
        return [t.clone() for t in (out, lse, *grads)]

    names = ("out", "lse", "dq", "dk", "dv")
    ref = run(keep)
    got = run(add)
    for n, a, b in zip(names, got, ref):
        assert torch.equal(a, b), f"{case}: {n} of the 0/hide additive mask differs from the boolean mask's"
    impure = add.clone()
    ramp = (torch.arange(S, device=dev) % 7).float() * 0.3      # not a constant shift of the row
    impure[0, 0, 2, :] = torch.where(keep[0, 0, 2, :], ramp, impure[0, 0, 2, :])
    bias = run(impure)
    assert not torch.equal(bias[1][0, 0, 2], ref[1][0, 0, 2]), f"{case}: a biased mask gave the boolean mask's LSE"
    assert not torch.equal(bias[0][0, 0, 2], ref[0][0, 0, 2]), f"{case}: a biased mask gave the boolean mask's output"
    again = run(add)
    for n, a, b in zip(names, again, ref):
        assert torch.equal(a, b), f"{case}: {n} after a biased mask differs from the boolean mask's"
    # Which path ran: the forward's workspace holds the row table (256-byte
    # aligned), then the flag (0: only 0 and hiding values).
    words = B * mh * ((S + 63) // 64) * Sq
    at = (words * 8 + 255) // 256 * 256
    for m, want in ((impure, False), (add, True)):
        cp_attn_fwd(sh.q, sh.k, sh.v, sh.q_chunk_pos, layout=sh.layout, softmax_scale=scale, attn_mask=m,
                    workspace=ws)
        torch.cuda.synchronize()
        flag = int(ws[at:at + 4].view(torch.int32).item())
        assert (flag == 0) == want, f"{case}: flag {flag} after a {'pure' if want else 'biased'} mask"
    print(f"pure additive {case}: bitwise equal to the boolean mask", flush=True)


@pytest.mark.parametrize("additive", [0, 1])
def test_masked_share_without_keys(additive):
    """A share with no keys under a user mask, through the C ABI with a real
    mask pointer (torch gives a zero-width view no pointer): no bit table is
    built, every row comes out empty (out 0, LSE -inf) and dQ is 0, for a
    boolean and an additive mask."""
    from context_causal_attention_attn_amd import _lib
    from context_causal_attention_attn_amd.api import cp_attn_workspace_bytes, make_desc
    dev = torch.device("cuda")
    lib = _lib.load()
    q = torch.randn(1, 4, 64, 64, device=dev).to(torch.bfloat16)
    kv = torch.zeros(1, 2, 16, 64, dtype=torch.bfloat16, device=dev)[:, :, :0]
    base = torch.zeros(1, 4, 64, 16, dtype=torch.float32 if additive else torch.bool, device=dev)
    d = make_desc(q, kv, kv, q.stride(), [0], [0], "contiguous", True, 0.125)
    d.desc.attn_mask = base.data_ptr()
    d.desc.mask_additive = additive
    d.desc.mask_strides[0] = 0
    d.desc.mask_strides[1] = base.stride(1) * base.element_size()
    d.desc.mask_strides[2] = base.stride(2) * base.element_size()
    assert cp_attn_workspace_bytes(d, False) == 0
    out = torch.full_like(q, float("nan"))
    lse = torch.full((1, 4, 64), float("nan"), device=dev)
    fake = base.data_ptr()   # K/V pointers are not read without keys
    stream = torch.cuda.current_stream().cuda_stream
    _lib.check(lib.cp_attn_fwd(d.ref(), q.data_ptr(), fake, fake, out.data_ptr(), lse.data_ptr(), None, 0,
                               stream), "cp_attn_fwd")
    dout = torch.randn_like(q)
    dq = torch.full_like(q, float("nan"))
    need = cp_attn_workspace_bytes(d, True)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _lib.check(lib.cp_attn_bwd(d.ref(), q.data_ptr(), fake, fake, out.data_ptr(), lse.data_ptr(), dout.data_ptr(),
                               dq.data_ptr(), fake, fake, ws.data_ptr(), ws.numel(), stream), "cp_attn_bwd")
    torch.cuda.synchronize()
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))
    assert torch.all(dq == 0)
