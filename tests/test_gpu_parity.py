"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Sizes are small enough for the oracle to finish in seconds but span several tiles
(64 keys), several splits and ragged tails. Inputs come from gqa_synth with NaN in
every cache slot the step must not read (contiguous padding, page tails, unused
pages).
"""
import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from gpu_cases import (assert_parity, host64, make, oracle_for, small_workload)  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gqa_kv_cache_03_amd  # noqa: F401  (fails loudly if the library is missing)


def run(inp, **kw):
    from gqa_kv_cache_03_amd import gqa_decode
    wl = inp.wl
    out = gqa_decode(inp.q, inp.k_cache, inp.v_cache, inp.seq_lens, inp.block_table,
                     scale=wl.scale, causal=wl.causal, **kw)
    torch.cuda.synchronize()
    return host64(out)


CASES = [
    # B, H, G, d, q_len, lens, dtype, page
    (1, 8, 2, 64, 1, [128], "float32", 0),            # the fp32 single-token shape
    (2, 8, 2, 128, 1, [77, 300], "float32", 0),
    (3, 16, 16, 64, 2, [5, 64, 190], "float32", 0),    # MHA, fp32
    (2, 4, 1, 64, 3, [40, 129], "float32", 16),        # MQA, fp32, paged
    (2, 32, 8, 128, 1, [4096, 1000], "bfloat16", 0),   # R = 4
    (3, 64, 8, 128, 1, [1, 65, 2049], "bfloat16", 0),  # R = 8, L = 1
    (2, 32, 4, 128, 1, [700, 3000], "bfloat16", 16),   # R = 8, paged 16
    (2, 32, 4, 128, 1, [33, 2500], "bfloat16", 32),    # R = 8, paged 32
    (2, 32, 8, 128, 4, [4, 1500], "bfloat16", 0),      # R = 16, causal, L = q_len
    (2, 32, 4, 128, 4, [300, 1777], "bfloat16", 0),    # R = 32
    (2, 32, 2, 128, 4, [1200, 64], "bfloat16", 16),    # R = 64, paged
    (2, 32, 1, 128, 4, [999, 2100], "bfloat16", 0),    # R = 128 (MQA)
    (1, 64, 1, 128, 4, [1300], "bfloat16", 0),         # R = 256
    (2, 32, 32, 128, 4, [513, 2000], "bfloat16", 0),   # R = 4 (MHA), causal
    (2, 16, 16, 128, 1, [300, 1025], "bfloat16", 0),   # R = 1 -> VALU, bf16
    (2, 16, 8, 128, 1, [100, 700], "bfloat16", 16),    # R = 2 -> VALU, paged
    (2, 12, 4, 128, 1, [100, 700], "bfloat16", 0),     # R = 3 -> VALU
    (2, 24, 4, 128, 2, [100, 701], "bfloat16", 0),     # R = 12
    (2, 8, 2, 64, 2, [90, 260], "bfloat16", 0),        # d = 64 on MFMA
    (2, 32, 1, 64, 4, [90, 1000], "bfloat16", 16),     # d = 64, R = 128, paged
    (1, 32, 1, 128, 16, [1500], "bfloat16", 0),        # R = 512: four row blocks of 128
    (2, 30, 1, 128, 10, [900, 40], "bfloat16", 32),    # R = 300: three blocks of 112, paged 32
    (2, 64, 1, 64, 9, [300, 50], "bfloat16", 0),       # R = 576: five blocks of 128, d = 64
    (2, 32, 2, 128, 12, [700, 64], "bfloat16", 32),    # q_len 12, R = 192, paged 32
    (1, 32, 1, 128, 16, [600], "float32", 0),          # fp32, R = 512 on the vector ALUs
    (2, 16, 2, 64, 16, [300, 17], "float32", 32),      # fp32, q_len 16, paged 32, L ~ q_len
    (3, 8, 8, 128, 1, [1, 2, 3], "bfloat16", 0),       # MHA, R = 1, tiny sequences
    (2, 64, 8, 128, 1, [131, 32768], "bfloat16", 0),   # one long, one short sequence
    (1, 64, 1, 128, 16, [700], "bfloat16", 0),         # R = 1024, the most rows a group may pack: 8 blocks
    (1, 64, 1, 64, 16, [300], "bfloat16", 256),        # R = 1024, d = 64, the largest page (256)
    (2, 32, 4, 128, 1, [5000, 300], "bfloat16", 128),  # paged 128
]


@pytest.mark.parametrize("B,H,G,d,q_len,lens,dtype,page", CASES)
@pytest.mark.parametrize("splits", [0, 1, 3, 37])
def test_matches_oracle(B, H, G, d, q_len, lens, dtype, page, splits):
    wl, lens = small_workload(B, H, G, d, q_len, lens, dtype=dtype, paged=page,
                              seed=1000 + B * 7 + H + G + d + q_len + page)
    inp = make(wl, lens)
    got = run(inp, num_splits=splits)
    ref = oracle_for(inp)
    assert_parity(got, ref, dtype, f"{wl.name} splits={splits}")


@pytest.mark.parametrize("R_case", [(32, 8, 1, 4), (32, 4, 1, 4), (32, 2, 4, 2), (32, 1, 4, 2), (64, 1, 4, 2),
                                    (32, 1, 16, 2)])
@pytest.mark.parametrize("nwg", [1, 2, 5, 64, 333, 5000])
def test_persistent_boundaries(R_case, nwg):
    """Persistent workgroup counts from one (every segment inside one workgroup, many
    segment switches) to more workgroups than tiles (empty workgroups, one-tile
    shares): exercises the ring's prologue, steady state and drain, segment switches
    and both partial slots for every wave layout."""
    H, G, q_len, B = R_case
    wl, lens = small_workload(B, H, G, 128, q_len, [3000, 97, 1, 650][:B], seed=77 + H + G)
    inp = make(wl, lens)
    got = run(inp, num_splits=nwg, policy="mfma")
    assert_parity(got, oracle_for(inp), "bfloat16", f"nwg={nwg} R={H // G * q_len}")


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("policy", ["valu", "mfma"])
def test_policies_and_causality(causal, policy):
    wl, lens = small_workload(2, 32, 8, 128, 3, [500, 1300], seed=31, causal=causal)
    inp = make(wl, lens)
    got = run(inp, policy=policy, num_splits=2)
    ref = oracle_for(inp, causal=causal)
    assert_parity(got, ref, "bfloat16", f"{policy} causal={causal}")


@pytest.mark.parametrize("R_case", [(32, 8, 1), (32, 4, 2), (32, 2, 4)])
def test_split_invariance(R_case):
    """num_splits in {1,2,3,7,auto} and odd chunk sizes: identical up to fp32 rounding."""
    H, G, q_len = R_case
    wl, lens = small_workload(3, H, G, 128, q_len, [2000, 64, 1111], seed=41, key_norm_std=0.25)
    inp = make(wl, lens)
    outs = [run(inp, num_splits=s) for s in (1, 2, 3, 7, 0)]
    outs.append(run(inp, chunk_tokens=128))
    ref = oracle_for(inp)
    for o in outs:
        assert_parity(o, ref, "bfloat16")
        # bf16 outputs: two roundings of fp32 values that agree to ~1e-6 relative
        assert np.abs(o - outs[0]).max() <= 2 ** -7 * np.abs(outs[0]).max()


def test_split_invariance_fp32_tight():
    wl, lens = small_workload(2, 8, 2, 128, 1, [1000, 333], dtype="float32", seed=43)
    inp = make(wl, lens)
    base = run(inp, num_splits=1)
    for s in (2, 3, 7, 0):
        o = run(inp, num_splits=s)
        assert np.abs(o - base).max() <= 1e-6 * max(1.0, np.abs(base).max())


@pytest.mark.parametrize("page", [16, 32, 64, 128, 256])
def test_paged_equals_contiguous(page):
    """Same keys in a permuted pool: bitwise-equal output for the same split plan."""
    from gqa_synth.generate import paginate
    wl, lens = small_workload(3, 32, 4, 128, 2, [1500, 17, 800], seed=51)
    inp = make(wl, lens)
    cap = inp.k_cache.shape[2]
    pk, tbl, npages = paginate(torch, inp.k_cache, lens, page, seed=9, extra_pages=5)
    pv, _, _ = paginate(torch, inp.v_cache, lens, page, seed=9, extra_pages=5)
    from gqa_kv_cache_03_amd import gqa_decode
    kw = dict(scale=wl.scale, chunk_tokens=256)
    a = gqa_decode(inp.q, inp.k_cache, inp.v_cache, inp.seq_lens, **kw)
    bt = torch.as_tensor(tbl, device="cuda")
    b = gqa_decode(inp.q, pk, pv, inp.seq_lens, bt, **kw)
    torch.cuda.synchronize()
    assert cap >= 1500
    assert torch.equal(a, b)
    assert_parity(host64(b), oracle_for(inp), "bfloat16")


# ------------------------------------------------- structured inputs with |out| ~ 1

def _structured(kind, dtype="bfloat16", paged=0):
    B, H, G, d, q_len = 2, 32, 4, 128, 4
    wl, lens = small_workload(B, H, G, d, q_len, [1000, 2222], dtype=dtype, paged=paged, seed=61)
    inp = make(wl, lens)
    rng = np.random.default_rng(5)
    tdt = inp.q.dtype
    q, k, v = inp.q, inp.k_cache, inp.v_cache
    hpg = H // G
    if kind in ("one_hot",):
        scale = 1.0
        picks = {}
        for b in range(B):
            L = int(lens[b])
            for g in range(G):
                u = rng.standard_normal(d)
                u /= np.linalg.norm(u)
                j = int(rng.integers(0, L - q_len + 1))
                picks[(b, g)] = j
                q[b, :, g * hpg:(g + 1) * hpg] = torch.as_tensor(u, dtype=tdt, device="cuda")
                _set_rows(inp, b, g, slice(0, L), lambda n: torch.as_tensor(
                    0.01 * rng.standard_normal((n, d)), dtype=tdt, device="cuda"), which="k")
                _set_rows(inp, b, g, slice(j, j + 1), lambda n: torch.as_tensor(
                    60.0 * u[None, :], dtype=tdt, device="cuda"), which="k")
        return inp, scale, picks
    if kind == "v_const_per_group":
        for b in range(B):
            for g in range(G):
                _set_rows(inp, b, g, slice(0, int(lens[b])), lambda n: torch.full(
                    (n, d), float(g + 1), dtype=tdt, device="cuda"), which="v")
        return inp, 1.0, None
    if kind == "v_ramp":
        for b in range(B):
            L = int(lens[b])
            for g in range(G):
                _set_rows(inp, b, g, slice(0, L), lambda n: (torch.arange(n, device="cuda", dtype=torch.float32)
                                                            [:, None] / L).expand(n, d).to(tdt), which="v")
        return inp, 1.0, None
    if kind == "identical_keys":
        for b in range(B):
            for g in range(G):
                kk = torch.as_tensor(rng.standard_normal(d), dtype=tdt, device="cuda")
                _set_rows(inp, b, g, slice(0, int(lens[b])), lambda n: kk.expand(n, d), which="k")
        return inp, 1.0, None
    raise ValueError(kind)


def _set_rows(inp, b, g, sl, fn, which):
    cache = inp.k_cache if which == "k" else inp.v_cache
    j = np.arange(sl.start, sl.stop)
    vals = fn(len(j))
    if inp.block_table is None:
        cache[b, g, sl.start:sl.stop] = vals
    else:
        P = inp.wl.page_size
        pages = torch.as_tensor(inp.table[b][j // P].astype(np.int64), device="cuda")
        slots = torch.as_tensor(j % P, device="cuda")
        cache[pages, g, slots] = vals


@pytest.mark.parametrize("kind", ["one_hot", "v_const_per_group", "v_ramp", "identical_keys"])
@pytest.mark.parametrize("paged", [0, 16])
def test_structured_inputs(kind, paged):
    inp, scale, picks = _structured(kind, paged=paged)
    wl = inp.wl
    from gqa_kv_cache_03_amd import gqa_decode
    out = gqa_decode(inp.q, inp.k_cache, inp.v_cache, inp.seq_lens, inp.block_table, scale=scale, num_splits=3)
    torch.cuda.synchronize()
    got = host64(out)
    assert_parity(got, _oracle_scale(inp, scale), "bfloat16", kind)
    hpg = wl.H // wl.G
    if kind == "one_hot":
        for (b, g), j in picks.items():
            vrow = _row(inp, b, g, j, "v")
            np.testing.assert_allclose(got[b, :, g * hpg:(g + 1) * hpg],
                                       np.broadcast_to(vrow, (wl.q_len, hpg, wl.d_h)), atol=2e-2, rtol=1e-2)
    if kind == "v_const_per_group":
        for g in range(wl.G):
            np.testing.assert_array_equal(got[:, :, g * hpg:(g + 1) * hpg], float(g + 1))


def _row(inp, b, g, j, which):
    cache = inp.k_cache if which == "k" else inp.v_cache
    if inp.block_table is None:
        return host64(cache[b, g, j])
    P = inp.wl.page_size
    return host64(cache[int(inp.table[b][j // P]), g, j % P])


def _oracle_scale(inp, scale):
    import oracle as O
    wl = inp.wl
    q, k, v = host64(inp.q), host64(inp.k_cache), host64(inp.v_cache)
    if inp.block_table is None:
        return O.gqa_decode(q, k, v, inp.lens, scale, wl.G)
    return O.gqa_decode(q, k, v, inp.lens, scale, wl.G, block_table=inp.table, page_size=wl.page_size)


def test_nan_canaries_never_reach_output():
    wl, lens = small_workload(3, 32, 8, 128, 1, [65, 1, 300], seed=71, paged=16, extra_pages=7)
    inp = make(wl, lens)
    got = run(inp, num_splits=4)
    assert np.isfinite(got).all()
    assert_parity(got, oracle_for(inp), "bfloat16")


def test_output_overwritten_and_inputs_untouched():
    wl, lens = small_workload(2, 32, 8, 128, 1, [900, 100], seed=73)
    inp = make(wl, lens)
    snap = [t.clone() for t in (inp.q, inp.k_cache, inp.v_cache, inp.seq_lens)]
    from gqa_kv_cache_03_amd import gqa_decode
    out = torch.full_like(inp.q, float("nan"))
    gqa_decode(inp.q, inp.k_cache, inp.v_cache, inp.seq_lens, scale=wl.scale, out=out, num_splits=2)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    for a, b in zip(snap, (inp.q, inp.k_cache, inp.v_cache, inp.seq_lens)):
        assert torch.equal(a.nan_to_num(7.0), b.nan_to_num(7.0))


def test_scale_argument_is_applied():
    wl, lens = small_workload(1, 8, 2, 64, 1, [128], dtype="float32", seed=75)
    inp = make(wl, lens)
    from gqa_kv_cache_03_amd import gqa_decode
    for s in (0.0, 0.03125, 0.5, 1.3):
        out = gqa_decode(inp.q, inp.k_cache, inp.v_cache, inp.seq_lens, scale=s)
        torch.cuda.synchronize()
        assert_parity(host64(out), _oracle_scale(inp, s), "float32", f"scale={s}")


@pytest.mark.parametrize("B,page", [(65, 0), (130, 16), (200, 0)])
@pytest.mark.parametrize("splits", [0, 37])
def test_many_sequences(B, page, splits):
    """More than 64 sequences: the kernel's schedule scan and the merge's prefix sums
    take several 64-lane chunks of seq_lens."""
    rng = np.random.default_rng(5000 + B + page)
    lens = rng.integers(1, 300, size=B).astype(np.int32)
    lens[B // 2] = 2048                                   # one long sequence mid-batch
    wl, lens = small_workload(B, 32, 8, 128, 1, list(lens), paged=page, seed=5100 + B)
    inp = make(wl, lens)
    print(f"[parity] many sequences B={B} page={page} splits={splits}", flush=True)
    got = run(inp, num_splits=splits)
    assert_parity(got, oracle_for(inp), "bfloat16", f"B={B} page={page} splits={splits}")


# The persistent merge takes one of two forms: a wave per (segment, row) while
# segments average at most 2 * 4 * (256 / d) partials (nwg <= 8 * (256 / d) * B * G *
# row blocks), else a workgroup per (segment, row). Each case below lands in the form
# named, with segments of a few to a few hundred partials.
MERGE_FORM_CASES = [
    # B, H, G, d, q_len, lens, nwg, form
    (16, 32, 8, 128, 1, (300, 2600), 64, "wave"),
    (16, 32, 8, 128, 1, (300, 2600), 1024, "wave"),
    (4, 16, 4, 64, 2, (700, 3000), 512, "wave"),
    (2, 32, 1, 128, 4, (9000, 12000), 512, "workgroup"),
    (1, 8, 1, 128, 2, (5000, 5000), 300, "workgroup"),
    (2, 16, 2, 64, 1, (4000, 9000), 700, "workgroup"),
]


@pytest.mark.parametrize("B,H,G,d,q_len,lens,nwg,form", MERGE_FORM_CASES)
def test_merge_forms(B, H, G, d, q_len, lens, nwg, form):
    R = H // G * q_len
    n_rb = 1 if R <= 256 else -(-R // 128)
    assert (nwg <= 8 * (256 // d) * B * G * n_rb) == (form == "wave")
    rng = np.random.default_rng(5200 + B * H + nwg)
    L = rng.integers(lens[0], lens[1] + 1, size=B).astype(np.int32)
    wl, L = small_workload(B, H, G, d, q_len, list(L), seed=5300 + nwg)
    inp = make(wl, L)
    print(f"[parity] merge form {form}: B={B} H={H} G={G} d={d} q_len={q_len} nwg={nwg}", flush=True)
    got = run(inp, num_splits=nwg)
    assert_parity(got, oracle_for(inp), "bfloat16", f"{form} form nwg={nwg}")


@pytest.mark.parametrize("H,G,d,q_len,page", [(8, 8, 128, 1, 0), (16, 8, 128, 1, 16), (24, 8, 128, 1, 0),
                                              (8, 8, 128, 3, 32), (8, 8, 64, 2, 0), (24, 8, 64, 1, 16)])
def test_small_row_counts_on_a_large_cache_take_the_matrix_cores(H, G, d, q_len, page):
    """Fewer than 4 packed rows over a cache of 16 MiB or more: AUTO picks the persistent
    matrix-core kernel, whose 16-row tiles then hold 13-15 padding rows; every unit still
    matches the oracle."""
    from gqa_kv_cache_03_amd import gqa_decode, plan
    from gpu_cases import all_units_parity
    lens = [20000, 9000 + q_len, 16384, 33]
    wl, lens = small_workload(4, H, G, d, q_len, lens, paged=page, seed=8800 + H + d + q_len)
    inp = make(wl, lens)
    pl = plan(inp.q, inp.k_cache, inp.block_table, causal=wl.causal)
    assert pl["policy"] == "mfma" and pl["rows"] == H // G * q_len < 4, pl
    print(f"[small R] H={H} G={G} d={d} q_len={q_len} page={page} R={pl['rows']}", flush=True)
    out = gqa_decode(inp.q, inp.k_cache, inp.v_cache, inp.seq_lens, inp.block_table, scale=wl.scale,
                     causal=wl.causal)
    torch.cuda.synchronize()
    worst = all_units_parity(inp, out, f"small R H={H} G={G} d={d} q_len={q_len}", log=lambda m: None)
    assert worst["units"] == wl.B * wl.G
