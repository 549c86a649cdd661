"""Host-side checks of the C ABI (CPU only; no kernel is launched).

The library must load and export every function include/cp_attn.h declares;
descriptor validation must reject each malformed input with its documented
status; the host-side share geometry, pair counts and the forward tile
schedule are checked against the oracle's geometry and the page-derived
golden tables.
"""
import ctypes
import json
import os
import re

import numpy as np
import pytest

import oracle.cp_share as oc
from context_causal_attention_attn_amd import _lib
from context_causal_attention_attn_amd.api import _Desc, cp_attn_plan_stats_fwd, cp_attn_share_pairs
from context_causal_attention_attn_amd.api import cp_attn_share_positions, cp_attn_workspace_bytes

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cp_attn.h")
GOLDEN = os.path.join(ROOT, "tests", "golden")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^[A-Za-z_][\w \t\*]*?\b(cp_attn_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    names = declared_functions()
    assert len(names) >= 9, names
    for n in names:
        assert hasattr(lib, n), f"libcpattn.so does not export {n}"
        assert n in _lib.SIGNATURES, f"binding has no signature for {n}"
    assert set(_lib.SIGNATURES) == set(names)
    assert lib.cp_attn_abi_version() == _lib.ABI_VERSION
    for st in list(_lib.STATUS) + [-99]:
        assert lib.cp_attn_error_string(st)


def test_share_positions_golden():
    geo = json.load(open(os.path.join(GOLDEN, "share_geometry.json")))
    for c in geo["cases"]:
        pos, n = cp_attn_share_positions(c["layout"], c["S"], c["cp"], c["rank"])
        assert pos == c["chunk_pos"] and n == c["chunk_len"]
    for c in geo["errors"]:
        with pytest.raises(_lib.CpAttnError) as e:
            cp_attn_share_positions(c["layout"], c["S"], c["cp"], c["rank"])
        assert e.value.status in (-10, -2)


def desc(**kw):
    base = dict(dtype=0, batch=1, hq=8, hkv=2, head_dim=128, sq_local=500, skv=2000,
                q_chunk_pos=[500], kv_chunk_pos=[0], layout="contiguous", causal=True,
                softmax_scale=0.088, q_strides=(8 * 2000 * 128, 2000 * 128, 128),
                kv_strides=(2 * 2000 * 128, 2000 * 128, 128), o_strides=(8 * 500 * 128, 500 * 128, 128))
    base.update(kw)
    return _Desc(**base)


def status(d):
    return _lib.load().cp_attn_validate(d.ref())


def test_validate_accepts_good_descriptors():
    assert status(desc()) == 0
    assert status(desc(layout="head_tail", q_chunk_pos=[250, 1750], sq_local=500)) == 0
    assert status(desc(dtype=1, head_dim=64, q_strides=(0, 0, 64), kv_strides=(0, 0, 64), o_strides=(0, 0, 64))) == 0
    assert status(desc(sq_local=0)) == 0
    # K/V in any chunk order: equal chunks of a multiple of 128 rows, disjoint positions.
    assert status(desc(skv=2048, kv_chunk_pos=[1024, 0])) == 0
    assert status(desc(skv=64 * 128, kv_chunk_pos=[128 * (63 - c) for c in range(64)])) == 0
    assert status(desc(skv=1024, kv_chunk_pos=[0, 4096])) == 0          # gaps between chunks


@pytest.mark.parametrize("kw,code", [
    (dict(hq=6, hkv=4), -2),                                  # hq % hkv
    (dict(batch=0), -2),
    (dict(head_dim=96), -5),                                  # unsupported head_dim
    (dict(dtype=7), -5),
    (dict(layout="head_tail"), -3),                           # head_tail needs 2 chunks
    (dict(q_chunk_pos=[0, 250], sq_local=500), -3),           # contiguous needs 1 chunk
    (dict(layout=5), -3),
    (dict(layout="head_tail", q_chunk_pos=[0, 100], sq_local=500), -4),   # overlapping chunks
    (dict(q_chunk_pos=[-1]), -4),
    (dict(layout="head_tail", q_chunk_pos=[0, 300], sq_local=501), -2),   # unequal chunks
    (dict(kv_chunk_pos=[0, 1000]), -5),                       # KV chunks of 1000 rows: not a multiple of 128
    (dict(skv=65 * 128, kv_chunk_pos=[128 * c for c in range(65)]), -3),   # more than 64 KV chunks
    (dict(skv=2048, kv_chunk_pos=[0, 512]), -4),               # overlapping KV chunks
    (dict(skv=2048, kv_chunk_pos=[1024, -1024]), -4),
    (dict(skv=2001, kv_chunk_pos=[0, 1000]), -2),              # unequal KV chunks
    (dict(softmax_scale=float("nan")), -2),
    (dict(softmax_scale=0.0), -2),
    (dict(q_strides=(8 * 2000 * 128, 2000 * 128, 132)), -9),   # row stride breaks 16-byte alignment
    (dict(kv_strides=(-1, 2000 * 128, 128)), -2),
    (dict(sq_local=2 ** 31), -5),
    (dict(q_strides=(0, 0, 2 ** 24)), -5),                     # row stride beyond 32-bit tile offsets
    (dict(o_strides=(0, 0, 2 ** 24 + 8)), -5),
])
def test_validate_rejects(kw, code):
    assert status(desc(**kw)) == code


def test_validate_abi_version_causal_flag_and_null():
    d = desc()
    d.desc.abi_version = 1
    assert status(d) == -8
    d = desc()
    d.desc.causal = 2
    assert status(d) == -2
    assert _lib.load().cp_attn_validate(None) == -1


CONFIGS = [
    ("contiguous", 256, 4, 1, 2, 2),
    ("contiguous", 32768, 8, 7, 32, 8),
    ("head_tail", 32768, 8, 0, 32, 8),
    ("head_tail", 32768, 8, 5, 32, 8),
    ("head_tail", 2000, 4, 2, 8, 2),
    ("ulysses", 32768, 8, 0, 32, 8),
    ("hybrid", 32768, 8, 4, 32, 8),
]


def _share(kind, S, cp, r, Hq, Hkv):
    if kind == "contiguous":
        return oc.contiguous_share(S, Hq, Hkv, cp, r)
    if kind == "head_tail":
        return oc.head_tail_share(S, Hq, Hkv, cp, r)
    if kind == "ulysses":
        return oc.ulysses_share(S, Hq, Hkv, cp, r)
    return oc.hybrid_share(S, Hq, Hkv, cp, 2, r)


def _desc_for(sh, S, Hq, Hkv, D=128, causal=True, kv_chunk_pos=(0,)):
    hq, hkv = len(sh["q_heads"]), len(sh["kv_heads"])
    n = sh["chunk_len"]
    layout = "head_tail" if len(sh["q_chunk_pos"]) == 2 else "contiguous"
    sq = n * len(sh["q_chunk_pos"])
    return desc(hq=hq, hkv=hkv, head_dim=D, sq_local=sq, skv=S, q_chunk_pos=sh["q_chunk_pos"],
                kv_chunk_pos=list(kv_chunk_pos), layout=layout, causal=causal, q_strides=(0, 0, D), kv_strides=(0, 0, D), o_strides=(0, 0, D))


@pytest.mark.parametrize("cfg", CONFIGS)
def test_share_pairs_match_oracle(cfg):
    kind, S, cp, r, Hq, Hkv = cfg
    sh = _share(kind, S, cp, r, Hq, Hkv)
    for causal in (True, False):
        d = _desc_for(sh, S, Hq, Hkv, causal=causal)
        assert cp_attn_share_pairs(d) == oc.share_pairs(sh["q_pos"], sh["kv_pos"], causal)


def test_share_pairs_with_kv_offset_and_masked_rows():
    # Keys start after some queries: those rows see nothing; later rows see all keys.
    d = desc(sq_local=100, skv=50, q_chunk_pos=[10], kv_chunk_pos=[40])
    exp = oc.share_pairs(np.arange(10, 110), np.arange(40, 90), True)
    assert cp_attn_share_pairs(d) == exp


def gathered_kv_pos(kind, S, cp):
    """KV chunk table of an all-gather over the CP group: rank after rank, each
    rank's chunks in its local order."""
    out = []
    for r in range(cp):
        out += cp_attn_share_positions(kind, S, cp, r)[0]
    return out


@pytest.mark.parametrize("kind,S,cp,rank", [("head_tail", 32768, 8, 0), ("head_tail", 32768, 8, 5),
                                            ("head_tail", 2048, 4, 3), ("contiguous", 32768, 8, 7)])
def test_gathered_kv_order_pairs_and_schedule(kind, S, cp, rank):
    """K/V in all-gather order: the same visible pairs as the natural order
    (checked against the oracle with per-key positions) and the same number
    of KV tile visits (chunk boundaries fall on tile boundaries)."""
    sh = _share(kind, S, cp, rank, 32, 8)
    table = gathered_kv_pos(kind, S, cp)
    n_kv = S // len(table)
    kv_pos = np.concatenate([np.arange(p, p + n_kv) for p in table])
    assert sorted(kv_pos.tolist()) == list(range(S))
    natural = _desc_for(sh, S, 32, 8)
    gathered = _desc_for(sh, S, 32, 8, kv_chunk_pos=table)
    for causal in (True, False):
        d_nat = _desc_for(sh, S, 32, 8, causal=causal)
        d_gat = _desc_for(sh, S, 32, 8, causal=causal, kv_chunk_pos=table)
        assert cp_attn_share_pairs(d_gat) == cp_attn_share_pairs(d_nat) == \
            oc.share_pairs(sh["q_pos"], kv_pos, causal)
    st_n, st_g = cp_attn_plan_stats_fwd(natural), cp_attn_plan_stats_fwd(gathered)
    assert st_g["kv_tile_visits"] == st_n["kv_tile_visits"]
    assert st_g["masked_tile_visits"] >= st_n["masked_tile_visits"]


def test_share_pairs_with_kv_chunk_gaps():
    # Two KV chunks with a gap between them, listed out of order.
    d = desc(sq_local=300, skv=256, q_chunk_pos=[100], kv_chunk_pos=[350, 0])
    kv_pos = np.concatenate([np.arange(350, 478), np.arange(0, 128)])
    assert cp_attn_share_pairs(d) == oc.share_pairs(np.arange(100, 400), kv_pos, True)


def test_head_tail_tile_schedule_is_balanced():
    """Every Head-Tail rank visits the same number of KV tiles, and the visits
    cover every visible pair (at most one partly masked tile per row tile)."""
    visits = set()
    for r in range(8):
        sh = oc.head_tail_share(32768, 32, 8, 8, r)
        st = cp_attn_plan_stats_fwd(_desc_for(sh, 32768, 32, 8))
        visits.add(st["kv_tile_visits"])
        rows_per_item = st["block_q_rows"] * st["heads_per_item"]
        area = st["kv_tile_visits"] * rows_per_item * st["block_kv_rows"]
        pairs = oc.share_pairs(sh["q_pos"], sh["kv_pos"]) * 32
        assert pairs <= area
        assert area - pairs <= st["work_items"] * rows_per_item * st["block_kv_rows"]
    assert len(visits) == 1


def test_workspace_bytes():
    """Forward: none. Backward: -Delta and LSE*log2e per row (each on a
    256-byte boundary), plus whole fp32 partial dK/dV tiles when the key tiles
    are split (this small share: 2 KV heads, 8 key tiles)."""
    d = desc()
    assert cp_attn_workspace_bytes(d, False) == 0
    rows = 1 * 8 * 500
    stats = 2 * ((rows * 4 + 255) // 256) * 256
    extra = cp_attn_workspace_bytes(d, True) - stats
    unit = 2 * 2 * 128 * 128 * 4                        # dK and dV of one key tile of both KV heads
    assert extra >= 0 and extra % unit == 0 and extra // unit in (0, 8, 24, 56)   # (parts - 1) x 8 tiles


def _aligned(n):
    return (n + 255) // 256 * 256


def test_workspace_holds_the_bit_tables_of_a_user_mask():
    """bf16 with a user mask. The forward's workspace holds the row table:
    one 64-bit word per query row, 64-key tile and mask batch/head. The
    backward's also holds the column table, one word per key, 64-row query
    tile of each chunk and mask batch/head, besides the row table (each
    256-byte aligned). An additive mask's tables come with 256 bytes more
    (the flag that says whether its values are only 0 and hiding ones). The
    fp32 path adds none."""
    def extra(backward, **kw):
        d0, dm = desc(**kw), desc(**kw)
        dm.desc.attn_mask = 1 << 40
        return cp_attn_workspace_bytes(dm, backward) - cp_attn_workspace_bytes(d0, backward)
    # contiguous 500 rows: 8 query tiles; 2000 keys: 32 key tiles;
    # broadcast mask: one batch, one head
    rows = _aligned(32 * 500 * 8)
    assert extra(False) == rows
    assert extra(True) == _aligned(8 * 2000 * 8) + rows
    # Head-Tail, two chunks of 250 rows: 4 tiles each; a per-head mask (stride != 0)
    d = desc(layout="head_tail", q_chunk_pos=[250, 1750], sq_local=500)
    f0, b0 = cp_attn_workspace_bytes(d, False), cp_attn_workspace_bytes(d, True)
    d.desc.attn_mask = 1 << 40
    d.desc.mask_strides[1] = 500 * 2000
    d.desc.mask_strides[2] = 2000
    rows = _aligned(8 * 32 * 500 * 8)
    assert cp_attn_workspace_bytes(d, False) - f0 == rows
    assert cp_attn_workspace_bytes(d, True) - b0 == _aligned(8 * 2 * 4 * 2000 * 8) + rows
    # additive: the same tables and the flag
    rows = _aligned(32 * 500 * 8)
    for backward, tables in ((False, rows), (True, _aligned(8 * 2000 * 8) + rows)):
        d = desc()
        d0 = cp_attn_workspace_bytes(d, backward)
        d.desc.attn_mask = 1 << 40
        d.desc.mask_additive = 1
        d.desc.mask_strides[2] = 2000 * 4
        assert cp_attn_workspace_bytes(d, backward) - d0 == tables + 256
    # fp32: none
    kw = dict(dtype=1, head_dim=64, q_strides=(0, 0, 64), kv_strides=(0, 0, 64), o_strides=(0, 0, 64))
    assert extra(False, **kw) == 0 and extra(True, **kw) == 0


def test_fwd_with_a_boolean_mask_needs_its_workspace():
    """cp_attn_fwd refuses a bf16 boolean-mask share whose workspace is
    missing, short or misaligned, before any HIP call."""
    lib = _lib.load()
    fake = 1 << 40
    d = desc()
    d.desc.attn_mask = fake
    need = cp_attn_workspace_bytes(d, False)
    args = (d.ref(), fake, fake, fake, fake, fake)
    assert lib.cp_attn_fwd(*args, None, 0, None) == -6
    assert lib.cp_attn_fwd(*args, fake, need - 8, None) == -6
    assert lib.cp_attn_fwd(*args, fake + 8, need, None) == -9


def test_noalloc_rejects_a_bit_table_beyond_its_scratch():
    """cp_attn_bwd_noalloc holds the bit table of a boolean mask in its fixed
    scratch: a share whose table does not fit is refused with
    CP_ATTN_ERR_SCRATCH_LIMIT before any HIP call."""
    lib = _lib.load()
    fake = 1 << 40
    S = 1 << 20                                          # 1 Mi keys x 8 tiles x 8 bytes = 64 MiB
    big = desc(skv=S, q_strides=(8 * S * 128, S * 128, 128), kv_strides=(2 * S * 128, S * 128, 128),
               q_chunk_pos=[S - 500])
    big.desc.attn_mask = fake
    big.desc.mask_strides[2] = S
    args = [fake] * 9 + [None]
    assert lib.cp_attn_bwd_noalloc(big.ref(), *args) == -11


def test_bwd_timed_rejects_bad_event_arrays_before_any_device_work():
    # Host-side checks only: every call below returns before touching a device.
    lib = _lib.load()
    d = desc()
    fake = [256 * (i + 1) for i in range(10)]
    ev4 = (ctypes.c_void_p * 4)(256, 512, 768, 1024)
    ev_null = (ctypes.c_void_p * 4)(256, None, 768, 1024)
    args = (d.ref(), *fake[:6], *fake[6:9], fake[9], 1 << 30, None)
    assert lib.cp_attn_bwd_timed(*args, ev4, 3) == -2
    assert lib.cp_attn_bwd_timed(*args, None, 4) == -1
    assert lib.cp_attn_bwd_timed(*args, ev_null, 4) == -1
    bad = desc(batch=0)
    assert lib.cp_attn_bwd_timed(bad.ref(), *args[1:], ev4, 4) == -2


@pytest.mark.parametrize("kind,cp,U", [("head_tail", 4, 1), ("contiguous", 4, 1), ("hybrid", 4, 2)])
def test_cut_share_gathered_kv_order(kind, cp, U):
    """cut_share(kv_order="gathered") on CPU tensors: K/V rows are the global
    rows at the positions the KV chunk table gives (the oracle's gathered key
    order), every position exactly once."""
    import torch
    from context_causal_attention_attn_amd import cut_share
    from tests._share_cases import gathered_key_rows
    S = 1024
    g = torch.Generator().manual_seed(0)
    q = torch.randn(1, 4, S, 8, generator=g)
    k = torch.randn(1, 2, S, 8, generator=g)
    for r in range(cp):
        sh = cut_share(kind, q, k, k, cp, r, ulysses=U, kv_order="gathered")
        pos = sh.kv_positions()
        assert sorted(pos) == list(range(S))
        assert pos == gathered_key_rows(kind, S, cp, U).tolist()
        assert torch.equal(sh.k, k[:, sh.kv_heads[0]:sh.kv_heads[-1] + 1][:, :, pos])
    with pytest.raises(ValueError):
        cut_share("ulysses", q, k, k, 2, 0, kv_order="gathered")


def _relayout_status(step=1, dtype=0, u=4, batch=1, heads=2, rows=64, head_dim=128, src=64, dst=1 << 40,
                     strides=(2 * 256 * 128, 256 * 128, 128)):
    st = None if strides is None else (ctypes.c_int64 * 3)(*strides)
    return _lib.load().cp_attn_ulysses_relayout(step, dtype, u, batch, heads, rows, head_dim, src, dst, st, None)


@pytest.mark.parametrize("kw,code", [
    (dict(step=4), -3), (dict(step=-1), -3),                  # unknown step
    (dict(dtype=7), -5),
    (dict(u=0), -2), (dict(batch=0), -2), (dict(heads=0), -2), (dict(rows=-1), -2),
    (dict(head_dim=96), -5),                                  # 192-byte rows: not a power of two
    (dict(head_dim=4), -5),                                   # 8-byte rows: below one 16-byte vector
    (dict(rows=2 ** 31), -5),
    (dict(strides=None), -1),
    (dict(strides=(-128, 128, 128)), -2),
    (dict(strides=(128, 128, 132)), -9),                      # row stride not a 16-byte multiple
    (dict(src=0), -1), (dict(dst=0), -1),
    (dict(src=72), -9),                                       # misaligned pointer
    (dict(src=1 << 40, dst=(1 << 40) + 4096), -2),            # overlapping buffers
])
def test_ulysses_relayout_rejects(kw, code):
    """Every rejected call returns before any device work (no GPU here)."""
    assert _relayout_status(**kw) == code


def test_ulysses_relayout_empty_is_a_no_op():
    assert _relayout_status(rows=0, src=0, dst=0) == 0


# Packed variable-length sequences: sequence-length mixes after the FLA CP
# test matrix (a sequence cut by rank boundaries, boundaries on rank
# boundaries, one sequence across several ranks, many short sequences).
PACKED_MIXES = {
    "cut": [3000, 4000, 3240, 5120, 5120, 7000, 3240, 2048],
    "aligned": [4096] * 8,
    "long_first": [21000, 11768],
    "short": [100] * 327 + [68],
}


def _doc_starts(lengths):
    return np.concatenate([[0], np.cumsum(lengths)[:-1]]).astype(np.int64).tolist()


def test_validate_packed_sequences():
    starts = _doc_starts([700, 800, 500])
    assert status(desc(doc_starts=starts)) == 0
    assert status(desc(doc_starts=[5])) == 0                           # positions before 5: one more sequence
    assert status(desc(doc_starts=[0, 700, 700])) == -4               # not strictly increasing
    assert status(desc(doc_starts=[-3, 700])) == -4
    assert status(desc(doc_starts=starts, causal=False)) == -5        # packed sequences are causal
    assert status(desc(doc_starts=starts, skv=2048, kv_chunk_pos=[0, 1024])) == -5
    # More than 256 boundaries that the share meets: unsupported.
    many = list(range(0, 2000, 3))
    assert status(desc(doc_starts=many)) == 0                          # 169 of them in the share
    many = list(range(0, 2000))
    assert status(desc(doc_starts=many)) == -5
    d = desc(doc_starts=starts)
    d.desc.doc_starts = None
    assert status(d) == -1


@pytest.mark.parametrize("mix", list(PACKED_MIXES), ids=list(PACKED_MIXES))
@pytest.mark.parametrize("kind,rank", [("contiguous", 7), ("contiguous", 2), ("head_tail", 0), ("head_tail", 5)])
def test_packed_share_pairs_match_oracle(mix, kind, rank):
    S = 32768
    starts = _doc_starts(PACKED_MIXES[mix])
    sh = _share(kind, S, 8, rank, 32, 8)
    d = _desc_for(sh, S, 32, 8)
    d = desc(hq=32, hkv=8, head_dim=128, sq_local=d.desc.sq_local, skv=S, q_chunk_pos=sh["q_chunk_pos"],
             layout="head_tail" if kind == "head_tail" else "contiguous", doc_starts=starts,
             q_strides=(0, 0, 128), kv_strides=(0, 0, 128), o_strides=(0, 0, 128))
    if mix == "short" and status(d) == -5:
        pytest.skip("more boundaries than the kernels take for this share")
    assert status(d) == 0
    pairs = cp_attn_share_pairs(d)
    assert pairs == oc.share_pairs(sh["q_pos"], sh["kv_pos"], True, starts)
    st = cp_attn_plan_stats_fwd(d)
    area = st["kv_tile_visits"] * st["block_q_rows"] * st["block_kv_rows"]
    assert pairs * 32 <= area * st["heads_per_item"]


def test_validate_user_mask():
    """A user attention mask (device bytes; validation reads only the pointer
    value and the strides): 4-byte alignment, a row stride below 32 MiB,
    natural key order, no packed sequences."""
    base = 1 << 40
    d = desc()
    d.desc.attn_mask = base
    for i, st in enumerate((0, 0, 2048)):
        d.desc.mask_strides[i] = st
    assert status(d) == 0
    d.desc.attn_mask = base + 2
    assert status(d) == -9
    d.desc.attn_mask = base
    d.desc.mask_strides[2] = 2046
    assert status(d) == -9
    d.desc.mask_strides[2] = -4
    assert status(d) == -2
    d.desc.mask_strides[2] = (1 << 25) - 4       # 64 rows stay below 2^31 bytes
    assert status(d) == 0
    d.desc.mask_strides[2] = 1 << 25
    assert status(d) == -2
    d2 = desc(skv=2048, kv_chunk_pos=[1024, 0])
    d2.desc.attn_mask = base
    assert status(d2) == -5
    d3 = desc(doc_starts=[0, 700])
    d3.desc.attn_mask = base
    assert status(d3) == -5


def test_validate_additive_user_mask():
    """An additive float32 mask is read with 16-byte vector loads: its pointer
    and every stride must be 16-byte multiples (4- or 8-byte alignment is
    CP_ATTN_ERR_ALIGNMENT); mask_additive must be 0 or 1."""
    base = 1 << 40
    d = desc()
    d.desc.attn_mask = base
    d.desc.mask_additive = 1
    for i, st in enumerate((0, 4 * 2048 * 1024, 4 * 2048)):
        d.desc.mask_strides[i] = st
    assert status(d) == 0
    for off in (4, 8, 12):
        d.desc.attn_mask = base + off
        assert status(d) == -9, off
    d.desc.attn_mask = base
    for i in range(3):
        for bad in (4, 8, 4 * 2048 + 4):
            saved = d.desc.mask_strides[i]
            d.desc.mask_strides[i] = bad
            assert status(d) == -9, (i, bad)
            d.desc.mask_strides[i] = saved
    assert status(d) == 0
    d.desc.mask_additive = 2
    assert status(d) == -2
    d.desc.mask_additive = -1
    assert status(d) == -2
    # The byte mask keeps its 4-byte rule: 4-aligned pointers pass.
    d.desc.mask_additive = 0
    d.desc.attn_mask = base + 4
    assert status(d) == 0


def test_header_constants_match_the_binding():
    """The binding's ABI version and limits are the header's."""
    hdr = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                            "include", "cp_attn.h")).read()
    def define(name):
        return re.search(rf"#define {name} \(?(-?[0-9.e]+)f?\)?", hdr).group(1)
    assert int(define("CP_ATTN_ABI_VERSION")) == _lib.ABI_VERSION
    assert int(define("CP_ATTN_MAX_Q_CHUNKS")) == _lib.MAX_Q_CHUNKS
    assert int(define("CP_ATTN_MAX_KV_CHUNKS")) == _lib.MAX_KV_CHUNKS
    assert float(define("CP_ATTN_MASK_HIDE")) == oc.MASK_HIDE
    assert _lib.load().cp_attn_abi_version() == _lib.ABI_VERSION


def test_noalloc_backward_rejects_beyond_its_scratch_before_device_work():
    """cp_attn_bwd_noalloc: a share with more than CP_ATTN_NOALLOC_MAX_ROWS rows
    (batch * hq * sq_local) is refused with CP_ATTN_ERR_SCRATCH_LIMIT before any
    HIP call (no GPU needed); an invalid descriptor gets validation's status."""
    lib = _lib.load()
    fake = 1 << 40
    big = desc(sq_local=_lib.NOALLOC_MAX_ROWS // 4 + 256)     # hq = 8 in desc(): twice the limit
    args = [fake] * 9 + [None]
    assert lib.cp_attn_bwd_noalloc(big.ref(), *args) == -11
    assert "scratch" in lib.cp_attn_error_string(-11).decode()
    bad = desc()
    bad.desc.abi_version = 1
    assert lib.cp_attn_bwd_noalloc(bad.ref(), *args) == -8


def test_workspace_holds_split_key_tile_partials():
    """The backward splits the key tiles of shares with few KV heads over
    several workgroups and needs room for their fp32 partial dK/dV; shares
    with many workgroups (the Colossal and Head-Tail cp=8 shares) need only
    the per-row statistics."""
    def ws(B, Hq, Hkv, sq, skv, qpos):
        d = desc(batch=B, hq=Hq, hkv=Hkv, sq_local=sq, skv=skv, q_chunk_pos=qpos,
                 layout="contiguous" if len(qpos) == 1 else "head_tail",
                 q_strides=(Hq * sq * 128, sq * 128, 128), kv_strides=(Hkv * skv * 128, skv * 128, 128),
                 o_strides=(Hq * sq * 128, sq * 128, 128))
        stats = 2 * ((B * Hq * sq * 4 + 255) // 256 * 256)
        return cp_attn_workspace_bytes(d, True) - stats
    assert ws(1, 32, 8, 4096, 32768, [28672]) == 0                       # Colossal cp=8 rank 7
    assert ws(2, 32, 8, 4096, 32768, [0, 30720]) == 0                     # Head-Tail B=2 rank 0
    part = ws(1, 4, 1, 32768, 32768, [0])                                  # Ulysses cp=8 rank 0
    unit = 2 * 128 * 128 * 4                                               # dK and dV of one key tile
    assert part > 0 and part % (256 * unit) == 0                           # whole extra parts of 256 tiles


def test_validate_chunked_layout_and_chunk_strides():
    """The chunked layout takes 1..16 equal query chunks at disjoint
    positions; chunk strides (q, k/v, out) are non-negative element counts
    that keep rows 16-byte aligned (bf16: multiples of 8 elements)."""
    u, H, L, D = 8, 4, 256, 128
    blocks = (1 * H * L * D, L * D, D)            # batch, head, row strides of one received block
    d = desc(hq=H, hkv=1, sq_local=u * L, skv=u * L, q_chunk_pos=[p * L for p in range(u)],
             kv_chunk_pos=[p * L for p in range(u)], layout="chunked", q_strides=blocks, kv_strides=(L * D, L * D, D),
             o_strides=blocks, chunk_strides=(H * L * D, L * D, H * L * D))
    assert status(d) == 0
    for i in range(3):
        saved = d.desc.chunk_strides[i]
        d.desc.chunk_strides[i] = -8
        assert status(d) == -2
        d.desc.chunk_strides[i] = saved + 4
        assert status(d) == -9
        d.desc.chunk_strides[i] = saved
    assert status(d) == 0
    over = desc(sq_local=17 * 16, q_chunk_pos=[p * 16 for p in range(17)], layout="chunked")
    assert status(over) == -3                       # more than 16 query chunks
    two = desc(sq_local=512, q_chunk_pos=[0, 1000], layout="contiguous")
    assert status(two) == -3                        # contiguous takes exactly one chunk
    d.desc.layout = 3
    assert status(d) == -3
