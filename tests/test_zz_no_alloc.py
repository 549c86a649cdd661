"""GPU check of cp_attn_bwd_noalloc, the backward entry point that takes no
workspace (its per-row statistics live in a fixed scratch array inside the
library), called through the C ABI: two calls in a row, the second with a
smaller share, each compared with cp_attn_bwd given a caller workspace on the
same inputs. dQ comes from the same kernel and must agree bit for bit; dK/dV
too wherever cp_attn_bwd keeps each key tile in one workgroup. Where it splits
key tiles over several workgroups (few KV heads; partials summed afterwards),
the no-alloc call, whose scratch holds no partials, does not: only the fp32
summation order differs, so dK/dV agree to 1e-5 relative. A boolean user
mask's bit tables share the scratch too."""
import ctypes
import math

import pytest
import torch

from context_causal_attention_attn_amd import _lib, cp_attn_bwd, cp_attn_fwd, cut_share
from context_causal_attention_attn_amd.api import make_desc
from synthetic import global_problem

pytestmark = pytest.mark.gpu


def noalloc_bwd(sh, out, lse, dout, scale, mask=None):
    """dq, dk, dv from cp_attn_bwd_noalloc through the C ABI."""
    lib = _lib.load()
    q, k, v = sh.q, sh.k, sh.v
    B, Hq, Sq, D = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    dq = torch.full_like(out, float("nan"))
    dk = torch.full((B, Hkv, Skv, D), float("nan"), dtype=torch.float32, device=q.device)
    dv = torch.full_like(dk, float("nan"))
    d = make_desc(q, k, v, out.stride(), sh.q_chunk_pos, sh.kv_chunk_pos, sh.layout, True, scale, (), mask)
    st = lib.cp_attn_bwd_noalloc(d.ref(), q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                 lse.data_ptr(), dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                 torch.cuda.current_stream().cuda_stream)
    _lib.check(st, "cp_attn_bwd_noalloc")
    return dq, dk, dv


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_noalloc_backward_matches_workspace_backward_twice(dtype):
    dev = torch.device("cuda")
    # First a larger share, then a smaller one: the second call must not see
    # anything of the first in the shared scratch array.
    cases = [(2, 8, 2, 2048, 128, "head_tail", 4, 1), (1, 4, 2, 640, 64, "contiguous", 2, 1)]
    if dtype == "fp32":
        cases = [(1, 4, 2, 512, 64, "head_tail", 2, 0), (1, 2, 1, 256, 64, "contiguous", 4, 1)]
    for B, Hq, Hkv, S, D, kind, cp, r in cases:
        prob = global_problem(B, Hq, Hkv, S, D, dtype=dtype, seed=61, with_dout=True)
        sh = cut_share(kind, prob.q.to(dev), prob.k.to(dev), prob.v.to(dev), cp, r)
        scale = 1.0 / math.sqrt(D)
        out, lse = cp_attn_fwd(sh.q, sh.k, sh.v, sh.q_chunk_pos, layout=sh.layout, softmax_scale=scale)
        dout = sh.take_rows(prob.dout.to(dev)).contiguous()
        ref = cp_attn_bwd(sh.q, sh.k, sh.v, out, lse, dout, sh.q_chunk_pos, layout=sh.layout,
                          softmax_scale=scale)
        got = noalloc_bwd(sh, out, lse, dout, scale)
        torch.cuda.synchronize()
        assert torch.equal(got[0], ref[0]), f"{dtype} {kind} S={S}: dq differs from cp_attn_bwd"
        for name, a, b in zip(("dk", "dv"), got[1:], ref[1:]):
            assert torch.isfinite(a).all(), name
            rel = float((a - b).norm() / b.norm().clamp_min(1e-30))
            assert rel <= 1e-5, f"{dtype} {kind} S={S}: {name} relative difference {rel}"
        print(f"noalloc {dtype} {kind} B={B} S={S} r{r}: dq bitwise, dk/dv within 1e-5 of cp_attn_bwd", flush=True)


def test_noalloc_backward_with_user_masks():
    """User masks: the backward's bit tables of them (and an additive mask's
    flag) live in the same scratch. A boolean mask, an additive padding mask
    (0 or -inf: the bit path), an additive mask with biases (the value path)
    and an unmasked smaller share in a row, each against cp_attn_bwd."""
    dev = torch.device("cuda")
    g = torch.Generator(device="cpu").manual_seed(62)
    cases = [(2, 8, 2, 2048, 128, "head_tail", 4, 1, "bool"), (2, 8, 2, 2048, 128, "head_tail", 4, 1, "padding"),
             (2, 8, 2, 2048, 128, "head_tail", 4, 1, "bias"), (1, 4, 2, 640, 64, "contiguous", 2, 1, None)]
    for B, Hq, Hkv, S, D, kind, cp, r, masked in cases:
        prob = global_problem(B, Hq, Hkv, S, D, dtype="bf16", seed=63, with_dout=True)
        sh = cut_share(kind, prob.q.to(dev), prob.k.to(dev), prob.v.to(dev), cp, r)
        scale = 1.0 / math.sqrt(D)
        m = None
        if masked:
            keep = torch.rand((B, Hq, sh.q.shape[2], S), generator=g) < 0.75
            if masked == "bool":
                m = keep.to(dev)
            else:
                val = torch.randn(keep.shape, generator=g) if masked == "bias" else torch.zeros(keep.shape)
                m = torch.where(keep, val, torch.tensor(float("-inf"))).to(dev)
        out, lse = cp_attn_fwd(sh.q, sh.k, sh.v, sh.q_chunk_pos, layout=sh.layout, softmax_scale=scale,
                               attn_mask=m)
        dout = sh.take_rows(prob.dout.to(dev)).contiguous()
        ref = cp_attn_bwd(sh.q, sh.k, sh.v, out, lse, dout, sh.q_chunk_pos, layout=sh.layout,
                          softmax_scale=scale, attn_mask=m)
        got = noalloc_bwd(sh, out, lse, dout, scale, m)
        torch.cuda.synchronize()
        assert torch.equal(got[0], ref[0]), f"{kind} S={S} masked={masked}: dq differs from cp_attn_bwd"
        for name, a, b in zip(("dk", "dv"), got[1:], ref[1:]):
            assert torch.isfinite(a).all(), name
            rel = float((a - b).norm() / b.norm().clamp_min(1e-30))
            assert rel <= 1e-5, f"{kind} S={S} masked={masked}: {name} relative difference {rel}"
        print(f"noalloc {kind} B={B} S={S} masked={masked}: dq bitwise, dk/dv within 1e-5", flush=True)


def test_noalloc_rejects_shares_beyond_its_scratch():
    dev = torch.device("cuda")
    rows = _lib.NOALLOC_MAX_ROWS // 8 + 64        # B * Hq * Sq just above the limit with Hq = 8
    q = torch.empty((1, 8, rows, 64), dtype=torch.bfloat16, device=dev)
    k = torch.empty((1, 2, 128, 64), dtype=torch.bfloat16, device=dev)
    d = make_desc(q, k, k, q.stride(), [0], [0], "contiguous", True, 0.125)
    st = _lib.load().cp_attn_bwd_noalloc(d.ref(), q.data_ptr(), k.data_ptr(), k.data_ptr(), q.data_ptr(),
                                         q.data_ptr(), q.data_ptr(), q.data_ptr(), k.data_ptr(), k.data_ptr(),
                                         None)
    assert st == -11
