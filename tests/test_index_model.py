"""Host-side check of the kernels' address arithmetic over the planner's shapes.

For each shape the library's own planner (gqa_decode_plan / gqla_absorb_plan through
the C ABI, no device work) gives the launch; tests/index_model.py then walks every
workgroup of that launch with the kernels' tile, page and partial-slot index math and
checks that every access stays inside its buffer, that every tile is consumed once and
that the merge reads exactly the partials the decode kernel wrote.
"""
from __future__ import annotations

import ctypes
import sys

import numpy as np
import pytest

from gqa_kv_cache_03_amd import _lib
from gqa_kv_cache_03_amd._lib import Plan
from gqa_synth import WORKLOADS
from gqa_synth.generate import draw_block_table, draw_lengths

import index_model as im

POLICY = {"auto": _lib.GQA_POLICY_AUTO, "valu": _lib.GQA_POLICY_VALU, "mfma": _lib.GQA_POLICY_MFMA}


def plan_of(shape: im.Shape, *, num_splits=0, policy="auto", dtype=_lib.GQA_DTYPE_BF16, latent_G=0):
    o = _lib.default_opts()
    o.dtype = dtype
    o.causal = 1
    o.num_splits = num_splits
    o.policy = POLICY[policy]
    if shape.page_size:
        o.page_size = shape.page_size
        o.max_blocks_per_seq = shape.max_blocks
        o.num_pages = shape.num_pages
    else:
        o.cache_capacity = shape.capacity
    pl = Plan()
    if latent_G:
        st = _lib.lib().gqla_absorb_plan(shape.B, shape.H, latent_G, 128, 512, shape.q_len,
                                         ctypes.byref(o), ctypes.byref(pl))
    else:
        st = _lib.lib().gqa_decode_plan(shape.B, shape.H, shape.G, shape.d_h, shape.q_len,
                                        ctypes.byref(o), ctypes.byref(pl))
    assert st == _lib.GQA_OK, _lib.lib().gqa_status_string(st)
    return {"schedule": pl.schedule, "rows": pl.rows, "row_blocks": pl.row_blocks,
            "tile_tokens": pl.tile_tokens, "chunk_tokens": pl.chunk_tokens, "max_splits": pl.max_splits,
            "workgroups": pl.workgroups, "grid": list(pl.grid), "workspace_bytes": pl.workspace_bytes}


def check(shape, **kw):
    pl = plan_of(shape, **kw)
    if pl["schedule"] == 1:
        return im.check_persistent(shape, pl)
    return im.check_split_grid(shape, pl)


def contiguous(B, H, G, d, q_len, lens, cap=None):
    lens = [int(x) for x in lens]
    return im.Shape(B, H, G, d, q_len, lens, cap or max(lens))


def paged(B, H, G, d, q_len, lens, P, slack_blocks=0):
    lens = [int(x) for x in lens]
    mb = max(-(-L // P) for L in lens) + slack_blocks
    return im.Shape(B, H, G, d, q_len, lens, mb * P, page_size=P,
                    num_pages=sum(-(-L // P) for L in lens) + 3, max_blocks=mb)


RNG = np.random.default_rng(7)
RAGGED = [int(x) for x in RNG.integers(1, 5000, size=13)]

SHAPES = [
    # (id, shape builder)
    ("decode_g8", lambda: contiguous(4, 32, 8, 128, 1, [4096] * 4)),
    ("ragged_g4", lambda: contiguous(13, 32, 4, 128, 1, RAGGED)),
    ("ragged_q4_g1", lambda: contiguous(13, 32, 1, 128, 4, [max(4, x) for x in RAGGED])),
    ("ragged_d64", lambda: contiguous(13, 16, 2, 64, 2, [max(2, x) for x in RAGGED])),
    ("len_eq_qlen", lambda: contiguous(5, 8, 2, 128, 3, [3, 3, 3, 3, 3])),
    ("len_one", lambda: contiguous(7, 4, 4, 128, 1, [1] * 7)),
    ("cap_not_tile_multiple", lambda: contiguous(3, 8, 1, 128, 1, [77, 1, 100], cap=100)),
    ("row_blocks_512", lambda: contiguous(3, 32, 1, 128, 16, [2000, 33, 700])),
    ("row_blocks_300", lambda: contiguous(2, 60, 1, 128, 5, [999, 64])),
    ("paged16_d128", lambda: paged(9, 32, 4, 128, 1, RAGGED[:9], 16)),
    ("paged16_d64", lambda: paged(9, 32, 4, 64, 1, RAGGED[:9], 16)),
    ("paged32_q16", lambda: paged(4, 32, 4, 128, 16, [max(16, x) for x in RAGGED[:4]], 32)),
    ("paged256_slack", lambda: paged(6, 16, 2, 128, 2, [max(2, x) for x in RAGGED[:6]], 256, slack_blocks=3)),
    ("many_sequences", lambda: contiguous(200, 8, 2, 128, 1, RNG.integers(1, 300, size=200))),
]


@pytest.mark.parametrize("num_splits", [0, 1, 3, 7, 2048])
@pytest.mark.parametrize("sid,build", SHAPES, ids=[s[0] for s in SHAPES])
def test_persistent_schedule_index_math(sid, build, num_splits):
    shape = build()
    rep = check(shape, num_splits=num_splits, policy="mfma")
    assert rep.tiles > 0


@pytest.mark.parametrize("num_splits", [0, 1, 5])
@pytest.mark.parametrize("sid,build", SHAPES[:8] + SHAPES[9:11], ids=[s[0] for s in SHAPES[:8] + SHAPES[9:11]])
def test_split_grid_index_math(sid, build, num_splits):
    shape = build()
    rep = check(shape, num_splits=num_splits, policy="valu")
    assert rep.tiles > 0


def test_more_workgroups_than_tiles_leaves_idle_workgroups_harmless():
    # 16 tiles in all, 512 workgroups: most own nothing and must write nothing; each
    # two-tile segment of the third sequence is cut in two (two partials each)
    shape = contiguous(3, 4, 4, 128, 1, [1, 32, 33])
    pl = plan_of(shape, num_splits=512, policy="mfma")
    rep = im.check_persistent(shape, pl)
    assert rep.tiles == 4 * (1 + 1 + 2) and rep.partial_writes == 8 and rep.merged_segments == 4


def test_latent_attention_plan_index_math():
    # the GQLA absorbed attention: one 512-wide latent head read by every query head
    lens = [int(x) for x in np.random.default_rng(3).integers(8, 3000, size=6)]
    for P in (0, 16):
        if P:
            shape = paged(6, 16, 1, 512, 1, lens, P)
        else:
            shape = contiguous(6, 16, 1, 512, 1, lens)
        pl = plan_of(shape, policy="mfma", latent_G=2)
        assert pl["rows"] == 16
        im.check_persistent(shape, pl)


def workload_shape(name):
    wl = WORKLOADS[name]
    lens = [int(x) for x in draw_lengths(wl)]
    if wl.d_c:
        H, G, d = wl.H, 1, wl.d_c
    else:
        H, G, d = wl.H, wl.G, wl.d_h
    if wl.layout == "paged":
        table, num_pages = draw_block_table(wl, np.asarray(lens))
        return wl, im.Shape(wl.B, H, G, d, wl.q_len, lens, table.shape[1] * wl.page_size,
                            page_size=wl.page_size, num_pages=num_pages, max_blocks=table.shape[1])
    return wl, contiguous(wl.B, H, G, d, wl.q_len, lens)


@pytest.mark.parametrize("name", sorted(WORKLOADS))
def test_full_size_workload_index_math(name):
    wl, shape = workload_shape(name)
    if wl.dtype != "bfloat16":
        pytest.skip("the persistent schedule is the bf16 matrix-core path")
    rep = check(shape, policy="mfma", latent_G=wl.G if wl.d_c else 0)
    assert rep.tiles > 0


def test_model_catches_a_planted_ownership_mistake(monkeypatch):
    # a merge that finds one segment's last owner one workgroup too far must be caught
    shape = contiguous(4, 32, 1, 128, 4, [5000, 3000, 4000, 100])
    pl = plan_of(shape, policy="mfma", num_splits=37)
    im.check_persistent(shape, pl)  # the real arithmetic passes
    real = im.tile_owner
    hit = {"n": 0}

    def shifted_owner(f, W, nwg):
        # the second call is the owner of the first segment's last tile
        hit["n"] += 1
        w = real(f, W, nwg)
        return w + 1 if hit["n"] == 2 else w

    monkeypatch.setattr(im, "tile_owner", shifted_owner)
    with pytest.raises(im.ModelError):
        im.check_persistent(shape, pl)
    assert hit["n"] == 2


def test_model_catches_a_planted_slot_mistake(monkeypatch):
    # every partial written to slot 0: a workgroup with a cut first and a cut last
    # segment then writes one slot twice
    shape = contiguous(4, 32, 1, 128, 4, [5000, 3000, 4000, 100])
    pl = plan_of(shape, policy="mfma", num_splits=37)
    assert "slot = 0 if first else 1" in open(im.__file__).read()
    patched = open(im.__file__).read().replace("slot = 0 if first else 1", "slot = 0")
    ns = {"__name__": "index_model_planted"}
    sys.modules["index_model_planted"] = type(sys)("index_model_planted")
    exec(compile(patched, im.__file__, "exec"), ns)
    with pytest.raises(ns["ModelError"]):
        ns["check_persistent"](shape, pl)
