"""Host-side tests of the C ABI (no GPU needed: every check below returns before
any HIP call). The library must load, export every declared symbol and reject bad
arguments with the documented status codes."""
import ctypes
import os
import re
import subprocess

import pytest

from gqa_kv_cache_03_amd import _lib
from gqa_kv_cache_03_amd._lib import DecodeOpts, Plan

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

OK, INV, UNS, WS = (_lib.GQA_OK, _lib.GQA_ERR_INVALID_ARGUMENT, _lib.GQA_ERR_UNSUPPORTED,
                    _lib.GQA_ERR_WORKSPACE)
P = 4096  # a fake, aligned, non-null address: validation never dereferences it


def declared_symbols():
    names = set()
    for h in ("gqa_decode.h", "gqa_bench.h", "gqla_absorb.h"):
        txt = open(os.path.join(ROOT, "include", h)).read()
        txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
        for m in re.finditer(r"\b(?:int|void|size_t|const char\*)\s+(gql?a_\w+)\s*\(", txt):
            names.add(m.group(1))
    return names


def test_library_exports_every_declared_symbol():
    L = _lib.lib()
    decl = declared_symbols()
    assert decl == set(_lib.EXPORTED)
    for name in decl:
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert decl <= exported


def _c_offsets(tmp_path, struct, fields):
    """offsetof() of each field, as the C compiler lays out the public header."""
    src = tmp_path / "off.c"
    body = "".join(f'  printf("%zu\\n", offsetof({struct}, {f}));\n' for f in fields)
    src.write_text(f"""#include <stdio.h>
#include <stddef.h>
#include "gqa_decode.h"
int main(void) {{
  printf("%zu\\n", sizeof({struct}));
{body}  return 0;
}}
""")
    exe = tmp_path / "off"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    vals = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    return vals[0], vals[1:]


@pytest.mark.parametrize("cls,struct", [(DecodeOpts, "gqa_decode_opts"), (Plan, "gqa_plan")])
def test_struct_layout_matches_header(tmp_path, cls, struct):
    fields = [f for f, _ in cls._fields_]
    size, offs = _c_offsets(tmp_path, struct, fields)
    assert ctypes.sizeof(cls) == size
    assert [getattr(cls, f).offset for f in fields] == offs


def test_default_opts():
    o = _lib.default_opts()
    assert o.struct_size == ctypes.sizeof(DecodeOpts)
    assert o.dtype == _lib.GQA_DTYPE_BF16 and o.causal == 1 and o.policy == 0
    assert _lib.lib().gqa_abi_version() == 1


def opts(**kw):
    o = _lib.default_opts()
    o.cache_capacity = 256
    for k, v in kw.items():
        setattr(o, k, v)
    return o


def call(B=2, H=8, G=2, d=128, q_len=1, scale=0.1, o=None, q=P, k=P, v=P, sl=P, bt=None, out=P):
    o = opts() if o is None else o
    return _lib.lib().gqa_decode(q, k, v, sl, bt, out, B, H, G, d, q_len, ctypes.c_float(scale), None,
                                 ctypes.byref(o) if o is not False else None)


def plan(B=2, H=8, G=2, d=128, q_len=1, o=None):
    o = opts() if o is None else o
    pl = Plan()
    st = _lib.lib().gqa_decode_plan(B, H, G, d, q_len, ctypes.byref(o), ctypes.byref(pl))
    return st, pl


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INV), (dict(k=None), INV), (dict(v=None), INV), (dict(sl=None), INV), (dict(out=None), INV),
    (dict(q=P + 8), INV), (dict(out=P + 4), INV), (dict(sl=P + 2), INV),
    (dict(B=0), INV), (dict(H=0), INV), (dict(G=0), INV), (dict(d=0), INV), (dict(q_len=0), INV),
    (dict(H=8, G=3), INV), (dict(H=4, G=8), INV),
    (dict(scale=float("nan")), INV), (dict(scale=float("inf")), INV),
    (dict(d=96), UNS), (dict(d=256), UNS),
    (dict(H=64, G=1, q_len=17), UNS),                 # R = 1088 > 1024
    (dict(o=False), INV),
])
def test_invalid_arguments_are_rejected(kw, status):
    assert call(**kw) == status


def test_opts_checks():
    assert call(o=opts(struct_size=8)) == INV
    assert call(o=opts(dtype=7)) == UNS
    assert call(o=opts(causal=2)) == INV
    assert call(o=opts(cache_capacity=0)) == INV
    assert call(q_len=4, o=opts(cache_capacity=3)) == INV
    assert call(o=opts(num_splits=-1)) == INV
    assert call(o=opts(policy=9)) == INV
    assert call(o=opts(dtype=_lib.GQA_DTYPE_F32, policy=_lib.GQA_POLICY_MFMA)) == UNS
    assert call(o=opts(page_size=16)) == INV           # page size without a block table


def test_paged_geometry_checks():
    good = dict(page_size=16, max_blocks_per_seq=8, num_pages=40, num_splits=1)
    assert call(bt=P, o=opts(**good)) != INV
    for bad in (dict(page_size=0), dict(page_size=8), dict(page_size=24), dict(page_size=512),
                dict(max_blocks_per_seq=0), dict(num_pages=0)):
        assert call(bt=P, o=opts(**{**good, **bad})) == INV, bad
    assert call(bt=P + 2, o=opts(**good)) == INV


def test_workspace_required_when_split():
    for o in (opts(num_splits=4, policy=_lib.GQA_POLICY_VALU), opts(num_splits=7)):
        assert call(o=o) == WS
        st, pl = plan(o=o)
        assert st == OK and pl.workspace_bytes > 0
        o.workspace = 1000                                   # misaligned
        o.workspace_bytes = pl.workspace_bytes
        assert call(o=o) == WS
        o.workspace = 4096
        o.workspace_bytes = pl.workspace_bytes - 1
        assert call(o=o) == WS


ro = lambda x: -(-x // 256) * 256


def test_plan_policy_and_workspace_formula():
    st, pl = plan(H=32, G=8, q_len=1, o=opts(cache_capacity=4096))
    assert st == OK and pl.policy == _lib.GQA_POLICY_MFMA and pl.rows == 4
    st, pl = plan(H=8, G=8, q_len=1, o=opts())                     # R = 1
    assert pl.policy == _lib.GQA_POLICY_VALU and pl.rows == 1
    st, pl = plan(H=8, G=2, o=opts(dtype=_lib.GQA_DTYPE_F32))
    assert pl.policy == _lib.GQA_POLICY_VALU
    # split-K grid (VALU): chunk is ceil(cap / n) rounded up to the tile
    st, pl = plan(B=3, H=16, G=4, q_len=2, o=opts(cache_capacity=1000, num_splits=3,
                                                  policy=_lib.GQA_POLICY_VALU))
    assert st == OK and pl.schedule == 0
    assert pl.chunk_tokens % pl.tile_tokens == 0
    assert pl.chunk_tokens >= -(-1000 // 3)
    assert pl.max_splits == -(-1000 // pl.chunk_tokens) <= 3
    rows = 3 * 2 * 16 * pl.max_splits
    assert pl.workspace_bytes == ro(rows * 128 * 4) + ro(rows * 4)
    assert list(pl.grid) == [pl.max_splits, 4, 3]
    st, pl = plan(o=opts(num_splits=1, policy=_lib.GQA_POLICY_VALU))   # one split: no workspace
    assert pl.max_splits == 1 and pl.workspace_bytes == 0


@pytest.mark.parametrize("nwg", [1, 5, 600])
def test_persistent_plan_and_workspace_formula(nwg):
    """MFMA policy: num_splits is the persistent workgroup count; each holds two
    partial slots of R rows (one row block here), plus B + 1 prefix sums."""
    B, H, G, q_len, d = 3, 16, 4, 2, 128
    st, pl = plan(B=B, H=H, G=G, q_len=q_len, d=d, o=opts(cache_capacity=1000, num_splits=nwg))
    assert st == OK and pl.policy == _lib.GQA_POLICY_MFMA and pl.schedule == 1
    R = H // G * q_len
    assert pl.workgroups == nwg and list(pl.grid) == [nwg, 1, 1] and pl.max_splits == 2
    assert pl.workspace_bytes == ro(nwg * 2 * R * d * 4) + ro(nwg * 2 * R * 4) + ro((B + 1) * 4)


def test_persistent_default_fills_the_device():
    """Without a device to query, the default is two workgroups on each of 256 CUs."""
    st, pl = plan(H=32, G=8, o=opts(cache_capacity=4096))
    assert st == OK and pl.schedule == 1
    assert pl.workgroups == 512


@pytest.mark.parametrize("R", [1, 2, 3, 4, 8, 16, 17, 32, 64, 65, 128, 256, 257, 300, 512, 520, 1024])
def test_every_row_count_up_to_the_maximum_plans(R):
    st, pl = plan(H=R, G=1, q_len=1, o=opts(cache_capacity=1 << 16))
    assert st == OK and pl.rows == R
    # a 64 MiB K+V cache: the matrix cores at any R (below R = 4 only from 16 MiB on)
    assert pl.policy == _lib.GQA_POLICY_MFMA
    assert pl.lds_bytes <= 160 * 1024
    if pl.policy == _lib.GQA_POLICY_MFMA:
        # one block up to 256 rows; a larger group in blocks of at most 128 rows
        assert pl.row_blocks == (1 if R <= 256 else -(-R // 128))


@pytest.mark.parametrize("R", [1, 2, 3])
def test_small_row_counts_take_the_matrix_cores_from_16_mib_of_cache(R):
    # K+V capacity bytes = 2 * 2 * B * G * capacity * d_h; the threshold is 16 MiB
    B, G, d = 2, 8, 128
    cap_at = (16 << 20) // (4 * B * G * d)          # exactly 16 MiB
    for cap, want in ((cap_at - 1, _lib.GQA_POLICY_VALU), (cap_at, _lib.GQA_POLICY_MFMA)):
        st, pl = plan(B=B, H=G * R, G=G, d=d, q_len=1, o=opts(cache_capacity=cap))
        assert st == OK and pl.rows == R and pl.policy == want, (cap, pl.policy)
    # fp32 always on the vector ALUs; R >= 4 always on the matrix cores
    st, pl = plan(B=B, H=G * R, G=G, d=d, q_len=1, o=opts(cache_capacity=cap_at, dtype=_lib.GQA_DTYPE_F32))
    assert pl.policy == _lib.GQA_POLICY_VALU
    st, pl = plan(B=B, H=G * 4, G=G, d=d, q_len=1, o=opts(cache_capacity=16))
    assert pl.policy == _lib.GQA_POLICY_MFMA


def test_status_strings():
    L = _lib.lib()
    for s in range(5):
        assert L.gqa_status_string(s)
    assert L.gqa_status_string(99) == b"unknown status"


def test_bench_helper_validation():
    L = _lib.lib()
    assert L.gqa_bench_read_stream(None, 16, P, None) == INV
    assert L.gqa_bench_read_stream(P, 15, P, None) == INV
    assert L.gqa_bench_read_stream(P + 4, 16, P, None) == INV
    assert L.gqa_bench_read_stream_lds(None, 16, 8, 16384, None) == INV
    assert L.gqa_bench_read_stream_lds(P, 15, 8, 16384, None) == INV
    assert L.gqa_bench_read_stream_lds(P, 16, 0, 16384, None) == INV
    assert L.gqa_bench_read_stream_lds(P, 16, 8, 8192, None) == INV


def call_append(kn=P, vn=P, **kw):
    o = kw.pop("o", None) or opts()
    args = dict(B=2, H=8, G=2, d=128, q_len=1, scale=0.1, q=P, k=P, v=P, sl=P, bt=None, out=P)
    args.update(kw)
    return _lib.lib().gqa_decode_append(args["q"], kn, vn, args["k"], args["v"], args["sl"], args["bt"],
                                        args["out"], args["B"], args["H"], args["G"], args["d"], args["q_len"],
                                        ctypes.c_float(args["scale"]), None, ctypes.byref(o))


@pytest.mark.parametrize("kw,status", [
    (dict(kn=None), INV), (dict(vn=None), INV), (dict(kn=P + 8), INV), (dict(vn=P + 2), INV),
    (dict(q=None), INV), (dict(H=8, G=3), INV), (dict(d=96), UNS),
])
def test_append_invalid_arguments_are_rejected(kw, status):
    assert call_append(**kw) == status


def test_append_workspace_checked():
    assert call_append(o=opts(num_splits=7)) == WS


def test_row_blocks_split_large_groups_evenly():
    """R = 16 tokens x 32 heads = 512 rows: four blocks of 128; R = 300: three of 112
    (100 rounded up to 16); the partial slots hold one block's rows."""
    for q_len, H, rb_rows in ((16, 32, 128), (10, 30, 112)):
        st, pl = plan(B=2, H=H, G=1, q_len=q_len, o=opts(cache_capacity=4096, num_splits=64))
        R = H * q_len
        assert st == OK and pl.row_blocks == -(-R // 128)
        assert pl.row_blocks * rb_rows >= R and rb_rows % 16 == 0
        assert pl.workspace_bytes == ro(64 * 2 * rb_rows * 128 * 4) + ro(64 * 2 * rb_rows * 4) + ro(3 * 4)


def test_grouping_variant_checks():
    hg = P  # a fake aligned device pointer; validation never dereferences it
    # bf16 with a head map: any H, G with G <= H; the plan sizes rows by max_group_heads
    st, pl = plan(H=40, G=6, q_len=2, o=opts(head_group=hg))
    assert st == OK and pl.policy == _lib.GQA_POLICY_MFMA and pl.rows == 40 * 2
    st, pl = plan(H=40, G=6, q_len=2, o=opts(head_group=hg, max_group_heads=10))
    assert st == OK and pl.rows == 20
    assert plan(H=8, G=9, o=opts(head_group=hg))[0] == INV             # G > H
    assert plan(H=40, G=6, o=opts(head_group=hg, max_group_heads=41))[0] == INV
    assert plan(H=40, G=6, o=opts(head_group=hg, max_group_heads=-1))[0] == INV
    assert plan(H=40, G=6, o=opts(head_group=hg + 2))[0] == INV        # misaligned map
    assert plan(H=300, G=6, o=opts(head_group=hg))[0] == UNS           # more than 256 heads
    assert plan(H=8, G=2, o=opts(head_group=hg, dtype=_lib.GQA_DTYPE_F32))[0] == UNS
    assert plan(H=8, G=2, o=opts(head_active=P, policy=_lib.GQA_POLICY_VALU))[0] == UNS
    st, pl = plan(H=8, G=8, o=opts(head_active=P))                      # R = 1 still on MFMA
    assert st == OK and pl.policy == _lib.GQA_POLICY_MFMA
    assert plan(H=8, G=2, o=opts(reserved0=1))[0] == INV
    assert plan(H=40, G=6)[0] == INV                                      # no map: H % G must be 0


# --------------------------------------------- GQLA, absorbed execution

def lcall(B=2, H=16, G=2, d=128, d_c=512, q_len=1, scale=0.1, o=None, q=P, lat=P, wk=P, wv=P, sl=P, bt=None,
          out=P):
    o = opts() if o is None else o
    return _lib.lib().gqla_absorb_decode(q, lat, wk, wv, sl, bt, out, B, H, G, d, d_c, q_len, ctypes.c_float(scale),
                                         None, ctypes.byref(o) if o is not False else None)


def lplan(B=2, H=16, G=2, d=128, d_c=512, q_len=1, o=None):
    o = opts() if o is None else o
    pl = Plan()
    st = _lib.lib().gqla_absorb_plan(B, H, G, d, d_c, q_len, ctypes.byref(o), ctypes.byref(pl))
    return st, pl


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INV), (dict(lat=None), INV), (dict(wk=None), INV), (dict(wv=None), INV),
    (dict(sl=None), INV), (dict(out=None), INV), (dict(wk=P + 8), INV), (dict(lat=P + 2), INV),
    (dict(B=0), INV), (dict(H=0), INV), (dict(G=0), INV), (dict(d=0), INV), (dict(d_c=0), INV),
    (dict(q_len=0), INV), (dict(H=16, G=3), INV), (dict(H=2, G=4), INV),
    (dict(scale=float("nan")), INV),
    (dict(d=96), UNS), (dict(d_c=256), UNS), (dict(d_c=576), UNS),
    (dict(H=128, q_len=9), UNS),                     # H q_len = 1152 > 1024 rows
    (dict(o=False), INV),
])
def test_latent_invalid_arguments_are_rejected(kw, status):
    assert lcall(**kw) == status


def test_latent_opts_checks():
    assert lcall(o=opts(dtype=_lib.GQA_DTYPE_F32)) == UNS
    assert lcall(o=opts(policy=_lib.GQA_POLICY_VALU)) == UNS
    assert lcall(o=opts(head_active=P)) == UNS
    assert lcall(o=opts(head_group=P)) == UNS
    assert lcall(o=opts(page_size=16)) == INV          # page size without a block table
    assert lcall() == WS                               # the workspace is always needed


@pytest.mark.parametrize("H,G,q_len,rows,blocks", [(16, 2, 1, 16, 1), (16, 16, 2, 32, 1), (128, 16, 1, 128, 4),
                                                   (8, 1, 3, 24, 1), (40, 5, 1, 40, 2)])
def test_latent_plan(H, G, q_len, rows, blocks):
    """Every query head reads the one latent: H q_len rows, in blocks of at most 32
    (the 512-wide query fragments fill the registers); the workspace holds the
    absorbed queries (bf16), the weighted latents (fp32) and the split partials."""
    B = 3
    st, pl = lplan(B=B, H=H, G=G, q_len=q_len, o=opts(num_splits=100))
    assert st == OK
    assert pl.policy == _lib.GQA_POLICY_MFMA and pl.schedule == 1
    assert pl.rows == rows and pl.row_blocks == blocks and pl.workgroups == 100
    rb = -(-rows // blocks)
    rb = rows if blocks == 1 else -(-rb // 16) * 16
    up = lambda x: -(-x // 256) * 256  # noqa: E731
    n = B * q_len * H
    attn = up(100 * 2 * rb * 512 * 4) + up(100 * 2 * rb * 4) + up((B + 1) * 4)
    assert pl.workspace_bytes == up(n * 512 * 2) + up(n * 512 * 4) + attn
    # two stages of 32 latent rows, staged once, and the 8 KiB where the waves add their
    # partial QK^T scores
    assert pl.lds_bytes == 2 * 32 * 512 * 2 + 8192
    size = ctypes.c_size_t(0)
    o = opts(num_splits=100)
    assert _lib.lib().gqla_absorb_workspace_size(B, H, G, 128, 512, q_len, ctypes.byref(o), ctypes.byref(size)) == OK
    assert size.value == pl.workspace_bytes


def test_latent_paged_geometry_checks():
    good = dict(page_size=16, max_blocks_per_seq=8, num_pages=40, num_splits=1)
    assert lcall(bt=P, o=opts(**good)) == WS              # valid; only the workspace is missing
    for bad in (dict(page_size=8), dict(max_blocks_per_seq=0), dict(num_pages=0)):
        assert lcall(bt=P, o=opts(**{**good, **bad})) == INV, bad


def call_noalloc(B=2, H=8, G=2, d=128, q_len=1, scale=0.1, o=None, q=P, k=P, v=P, sl=P, bt=None, out=P):
    o = opts() if o is None else o
    return _lib.lib().gqa_decode_noalloc(q, k, v, sl, bt, out, B, H, G, d, q_len, ctypes.c_float(scale), None,
                                         ctypes.byref(o) if o is not False else None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INV), (dict(out=P + 4), INV), (dict(B=0), INV), (dict(H=8, G=3), INV),
    (dict(scale=float("nan")), INV), (dict(d=96), UNS), (dict(o=False), INV),
])
def test_noalloc_rejects_what_gqa_decode_rejects(kw, status):
    assert call_noalloc(**kw) == status == call(**kw)


def test_noalloc_refuses_plans_beyond_its_scratch():
    """Plans whose partials exceed the fixed scratch return GQA_ERR_SCRATCH before any
    HIP call; the limit is the one the header states."""
    SCR = _lib.GQA_ERR_SCRATCH
    assert _lib.NOALLOC_SCRATCH_BYTES == 65 << 20
    hdr = open(os.path.join(ROOT, "include", "gqa_decode.h")).read()
    assert re.search(r"#define GQA_NOALLOC_SCRATCH_BYTES \(\(size_t\)65 << 20\)", hdr)
    # 256 packed rows per group (G = 1, H = 32, q_len = 8): 512 workgroups x 2 slots x
    # 256 rows x 128 x 4 bytes = 128 MiB of partials
    o = opts(cache_capacity=4096)
    st, pl = plan(B=8, H=32, G=1, q_len=8, o=o)
    assert st == OK and pl.workspace_bytes > _lib.NOALLOC_SCRATCH_BYTES
    assert call_noalloc(B=8, H=32, G=1, q_len=8, o=o) == SCR
    # the same shape at 128 rows needs 64.5 MiB and is not refused on size (it proceeds
    # to the device, which this host test does not reach: checked on the GPU)
    st, pl = plan(B=8, H=32, G=1, q_len=4, o=o)
    assert st == OK and pl.workspace_bytes <= _lib.NOALLOC_SCRATCH_BYTES
    assert "scratch" in _lib.status_string(SCR)


def ccall(sl=P, bt=None, B=2, q_len=1, o=None, report=P):
    o = opts() if o is None else o
    return _lib.lib().gqa_decode_check_inputs(sl, bt, B, q_len, None, ctypes.byref(o) if o is not False else None,
                                              report)


@pytest.mark.parametrize("kw,status", [
    (dict(sl=None), INV), (dict(report=None), INV), (dict(o=False), INV),
    (dict(sl=P + 2), INV), (dict(report=P + 2), INV), (dict(bt=P + 2, o="paged"), INV),
    (dict(B=0), INV), (dict(q_len=0), INV),
    (dict(o=dict(page_size=16)), INV),                          # page size without a table
    (dict(o=dict(cache_capacity=0)), INV),
    (dict(bt=P, o=dict(page_size=24, max_blocks_per_seq=4, num_pages=8)), INV),
    (dict(bt=P, o=dict(page_size=16, max_blocks_per_seq=0, num_pages=8)), INV),
    (dict(bt=P, o=dict(page_size=16, max_blocks_per_seq=4, num_pages=0)), INV),
    (dict(bt=P, B=65536, o=dict(page_size=16, max_blocks_per_seq=40000, num_pages=8)), UNS),
])
def test_check_inputs_rejects_bad_arguments(kw, status):
    """Argument errors of gqa_decode_check_inputs come back before any HIP call."""
    kw = dict(kw)
    o = kw.pop("o", None)
    if o == "paged":
        o = opts(page_size=16, max_blocks_per_seq=4, num_pages=8)
    elif isinstance(o, dict):
        o = opts(**o)
    assert ccall(o=o, **kw) == status


def lacall(cn=P, B=2, H=16, G=2, d=128, d_c=512, q_len=1, o=None, q=P, lat=P, wk=P, wv=P, sl=P, bt=None, out=P):
    o = opts() if o is None else o
    return _lib.lib().gqla_absorb_decode_append(q, cn, wk, wv, lat, sl, bt, out, B, H, G, d, d_c, q_len,
                                                ctypes.c_float(0.1), None, ctypes.byref(o))


@pytest.mark.parametrize("kw,status", [
    (dict(cn=None), INV), (dict(cn=P + 8), INV), (dict(lat=None), INV), (dict(q=P + 4), INV),
    (dict(d_c=256), UNS), (dict(H=16, G=3), INV),
    (dict(), WS),                                  # every argument valid: only the workspace is missing
])
def test_latent_append_rejects_bad_arguments(kw, status):
    """gqla_absorb_decode_append checks what gqla_absorb_decode checks, plus c_new,
    on the host before any HIP call."""
    assert lacall(**kw) == status


def test_plain_c_client(tmp_path):
    """The public headers are plain C: a C program compiles against include/ alone, links
    against the library and gets the host-side results the Python binding gets."""
    lib_dir = os.path.dirname(_lib.LIB_PATH)
    exe = tmp_path / "c_client"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c_client.c"), "-L", lib_dir, "-lgqa_decode",
                    f"-Wl,-rpath,{lib_dir}", "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.count("ok ") == 12
