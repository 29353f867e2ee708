"""GPU parity of the grouping variants against the fp64 oracle.

- A call-time head -> KV head map (non-uniform groups, KDGQA/DGQA style): unequal
  groups, idle KV heads, every head on one KV head, and a bound on the group size.
- A per-(token, head) active mask (Grouped Query Experts style): inactive pairs must
  be exactly 0 and active ones match the oracle.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from gpu_cases import assert_parity, host64, make, oracle_for, small_workload  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gqa_kv_cache_03_amd  # noqa: F401  (fails loudly if the library is missing)


def oracle_variant(inp, head_group=None, head_active=None):
    wl = inp.wl
    kw = dict(head_group=head_group, head_active=head_active, causal=wl.causal)
    if inp.block_table is None:
        cap = int(inp.lens.max())
        return oracle.gqa_decode(host64(inp.q), host64(inp.k_cache[:, :, :cap]), host64(inp.v_cache[:, :, :cap]),
                                 inp.lens, wl.scale, wl.G, **kw)
    return oracle.gqa_decode(host64(inp.q), host64(inp.k_cache), host64(inp.v_cache), inp.lens, wl.scale, wl.G,
                             block_table=inp.table.astype(np.int64), page_size=wl.page_size, **kw)


def random_map(rng, H, G, max_heads=None, idle=()):
    """A seeded allocation of H query heads to the G KV heads (none to `idle`),
    with at most max_heads per KV head."""
    live = [g for g in range(G) if g not in idle]
    while True:
        m = rng.choice(live, size=H)
        counts = np.bincount(m, minlength=G)
        if max_heads is None or counts.max() <= max_heads:
            return m.astype(np.int32)


MAP_CASES = [
    # B, H, G, d, q_len, lens, page, map kind, max_group_heads
    (2, 32, 8, 128, 1, [300, 1025], 0, "random", 0),
    (2, 32, 4, 128, 4, [33, 700], 16, "random", 0),
    (2, 32, 8, 128, 2, [500, 64], 0, "idle", 0),
    (2, 16, 4, 128, 1, [200, 90], 0, "all_one", 0),
    (2, 64, 8, 64, 3, [150, 400], 32, "bounded", 12),
    (2, 48, 6, 128, 1, [257, 1200], 0, "random", 0),     # H % G == 0 not needed, but here it is
    (2, 40, 6, 128, 2, [800, 90], 0, "random", 0),       # H % G != 0
]


@pytest.mark.parametrize("B,H,G,d,q_len,lens,page,kind,maxh", MAP_CASES)
@pytest.mark.parametrize("splits", [0, 7])
def test_head_map_matches_oracle(B, H, G, d, q_len, lens, page, kind, maxh, splits):
    from gqa_kv_cache_03_amd import gqa_decode
    rng = np.random.default_rng(3000 + H + G + q_len)
    if kind == "random":
        m = random_map(rng, H, G)
    elif kind == "idle":
        m = random_map(rng, H, G, idle=(1, 5))
    elif kind == "all_one":
        m = np.full(H, 2, dtype=np.int32)
    else:
        m = random_map(rng, H, G, max_heads=maxh)
    # a G-group cache: the workload helper wants H % G == 0, so build it with a
    # divisible head count and use q's first H heads
    Hb = H if H % G == 0 else (H // G + 1) * G
    wl, lens = small_workload(B, Hb, G, d, q_len, lens, paged=page, seed=3100 + H + G)
    inp = make(wl, lens)
    inp.q = inp.q[:, :, :H].contiguous()
    hg = torch.as_tensor(m, device="cuda")
    print(f"[variants] map {kind} H={H} G={G} counts={np.bincount(m, minlength=G).tolist()} splits={splits}",
          flush=True)
    out = gqa_decode(inp.q, inp.k_cache, inp.v_cache, inp.seq_lens, inp.block_table, scale=wl.scale,
                     causal=wl.causal, num_splits=splits, head_group=hg, max_group_heads=maxh)
    torch.cuda.synchronize()
    ref = oracle_variant(inp, head_group=m)
    assert_parity(host64(out), ref, "bfloat16", f"map {kind}")


@pytest.mark.parametrize("B,H,G,d,q_len,lens,page", [
    (2, 32, 8, 128, 1, [300, 1025], 0),
    (2, 32, 4, 128, 4, [33, 700], 16),
    (2, 16, 16, 128, 2, [100, 700], 0),     # R = 2: the variant runs on the matrix cores
])
@pytest.mark.parametrize("splits", [0, 7])
def test_active_mask_matches_oracle(B, H, G, d, q_len, lens, page, splits):
    from gqa_kv_cache_03_amd import gqa_decode
    rng = np.random.default_rng(3200 + H + G + q_len)
    wl, lens = small_workload(B, H, G, d, q_len, lens, paged=page, seed=3300 + H)
    inp = make(wl, lens)
    act = (rng.random((B, q_len, H)) < 0.5).astype(np.uint8)
    out = gqa_decode(inp.q, inp.k_cache, inp.v_cache, inp.seq_lens, inp.block_table, scale=wl.scale,
                     causal=wl.causal, num_splits=splits, head_active=torch.as_tensor(act, device="cuda"))
    torch.cuda.synchronize()
    got = host64(out)
    assert (got[act == 0] == 0).all()
    assert_parity(got, oracle_variant(inp, head_active=act), "bfloat16", "active mask")


def test_map_and_mask_together_and_with_append():
    from gqa_kv_cache_03_amd import gqa_decode, gqa_decode_append
    rng = np.random.default_rng(3400)
    wl, lens = small_workload(2, 32, 4, 128, 2, [400, 70], seed=3500)
    inp = make(wl, lens)
    m = random_map(rng, 32, 4)
    act = (rng.random((2, 2, 32)) < 0.6).astype(np.uint8)
    kw = dict(scale=wl.scale, head_group=torch.as_tensor(m, device="cuda"),
              head_active=torch.as_tensor(act, device="cuda"))
    ref = oracle_variant(inp, head_group=m, head_active=act)
    out = gqa_decode(inp.q, inp.k_cache, inp.v_cache, inp.seq_lens, **kw)
    torch.cuda.synchronize()
    assert_parity(host64(out), ref, "bfloat16", "map + mask")
    # the same through the fused append: new rows from k_new / v_new
    k_new = torch.stack([inp.k_cache[b, :, int(lens[b]) - 2:int(lens[b])].transpose(0, 1)
                         for b in range(2)]).contiguous()
    v_new = torch.stack([inp.v_cache[b, :, int(lens[b]) - 2:int(lens[b])].transpose(0, 1)
                         for b in range(2)]).contiguous()
    for b in range(2):
        inp.k_cache[b, :, int(lens[b]) - 2:int(lens[b])] = float("nan")
        inp.v_cache[b, :, int(lens[b]) - 2:int(lens[b])] = float("nan")
    out2 = gqa_decode_append(inp.q, k_new, v_new, inp.k_cache, inp.v_cache, inp.seq_lens, **kw)
    torch.cuda.synchronize()
    assert torch.equal(out2, out)


def test_variants_reject_unsupported():
    from gqa_kv_cache_03_amd import GqaError, gqa_decode
    wl, lens = small_workload(1, 8, 2, 64, 1, [64], dtype="float32", seed=3600)
    inp = make(wl, lens)
    hg = torch.zeros(8, dtype=torch.int32, device="cuda")
    with pytest.raises(GqaError):            # fp32: the variants run on the matrix cores only
        gqa_decode(inp.q, inp.k_cache, inp.v_cache, inp.seq_lens, head_group=hg)


@pytest.mark.parametrize("splits", [0, 5])
def test_oversize_group_and_stray_entries_give_nan_rows(splits):
    """A map whose group exceeds max_group_heads, and entries outside [0, G): the
    (token, head) rows no packed tile holds come back NaN, every other row matches
    the oracle, and nothing is left unwritten (out starts out as a finite canary)."""
    from gqa_kv_cache_03_amd import gqa_decode, plan
    B, H, G, d, q_len, maxh = 2, 32, 4, 128, 2, 6
    wl, lens = small_workload(B, H, G, d, q_len, [300, 900], seed=3700)
    inp = make(wl, lens)
    rng = np.random.default_rng(3710)
    m = rng.permutation(np.concatenate([np.zeros(10), np.repeat([1, 2, 3], 6), [-1, 7],
                                        rng.integers(1, 4, H - 30)])).astype(np.int32)
    pl = plan(inp.q, inp.k_cache, causal=True, head_group=torch.as_tensor(m, device="cuda"),
              max_group_heads=maxh)
    assert pl["row_blocks"] == 1 and pl["rows"] == maxh * q_len
    cap = maxh * q_len
    drop = np.zeros((q_len, H), dtype=bool)
    for h in range(H):
        g = int(m[h])
        if not 0 <= g < G:
            drop[:, h] = True
            continue
        members = [x for x in range(H) if m[x] == g]
        k = members.index(h)
        for t in range(q_len):
            drop[t, h] = t * len(members) + k >= cap
    assert drop.any() and (~drop).any()
    out = torch.full_like(inp.q, 7.0)
    gqa_decode(inp.q, inp.k_cache, inp.v_cache, inp.seq_lens, scale=wl.scale, out=out, num_splits=splits,
               head_group=torch.as_tensor(m, device="cuda"), max_group_heads=maxh)
    torch.cuda.synchronize()
    got = host64(out)
    safe = np.where((m >= 0) & (m < G), m, 0).astype(np.int32)
    ref = oracle_variant(inp, head_group=safe)
    for b in range(B):
        assert np.isnan(got[b][drop]).all()
        assert_parity(got[b][~drop], ref[b][~drop], "bfloat16", f"kept rows b={b}")


def draw_map_case(seed):
    """A seeded head-map case: sizes, a map with optional stray entries, an optional
    group-size bound that may cut a group, an optional active mask."""
    rng = np.random.default_rng(seed)
    G = int(rng.choice([1, 2, 4, 6, 8, 16]))
    H = int(rng.integers(G, 129))
    q_len = int(rng.choice([1, 1, 2, 3, 4]))
    d = int(rng.choice([64, 128]))
    B = int(rng.integers(1, 9))
    lens = [int(rng.integers(q_len, 3000)) for _ in range(B)]
    page = int(rng.choice([0, 16, 32, 64]))
    splits = int(rng.choice([0, 0, 1, 3, 9, 200]))
    m = rng.integers(0, G, size=H).astype(np.int32)
    if rng.random() < 0.3:
        idx = rng.choice(H, size=min(int(rng.integers(1, 4)), H), replace=False)
        m[idx] = rng.choice([-1, G, G + 3], size=len(idx))
    counts = np.bincount(m[(m >= 0) & (m < G)], minlength=G)
    maxh = int(rng.integers(1, counts.max() + 1)) if rng.random() < 0.4 and counts.max() > 1 else 0
    active = (rng.random((B, q_len, H)) < 0.6).astype(np.uint8) if rng.random() < 0.3 else None
    return B, H, G, d, q_len, lens, page, splits, m, maxh, active


def packed_row_cap(H, q_len, maxh):
    """Rows a group's packed tiles hold: the planner's row blocks for maxh (0 = H) heads."""
    R = (H if maxh == 0 else maxh) * q_len
    n_rb = 1 if R <= 256 else -(-R // 128)
    rb = R if n_rb == 1 else (-(-R // n_rb) + 15) // 16 * 16
    return n_rb * rb


@pytest.mark.parametrize("seed", range(24))
def test_random_head_map(seed):
    """Random maps, stray entries, group-size bounds and active masks on random shapes,
    through both merge forms: kept rows match the oracle, rows no packed tile holds are
    NaN, and no row is left unwritten (out starts as a finite canary)."""
    from gqa_kv_cache_03_amd import gqa_decode
    B, H, G, d, q_len, lens, page, splits, m, maxh, active = draw_map_case(92000 + seed)
    Hb = ((H + G - 1) // G) * G
    wl, lens = small_workload(B, Hb, G, d, q_len, lens, paged=page, seed=92000 + seed)
    inp = make(wl, lens)
    inp.q = inp.q[:, :, :H].contiguous()
    print(f"[variants] random map seed={seed} B={B} H={H} G={G} d={d} q_len={q_len} page={page} "
          f"splits={splits} maxh={maxh} mask={active is not None}", flush=True)
    out = torch.full_like(inp.q, 7.0)
    kw = dict(head_group=torch.as_tensor(m, device="cuda"), max_group_heads=maxh)
    if active is not None:
        kw["head_active"] = torch.as_tensor(active, device="cuda")
    gqa_decode(inp.q, inp.k_cache, inp.v_cache, inp.seq_lens, inp.block_table, scale=wl.scale, causal=wl.causal,
               num_splits=splits, out=out, **kw)
    torch.cuda.synchronize()
    got = host64(out)
    cap = packed_row_cap(H, q_len, maxh)
    drop = np.zeros((q_len, H), dtype=bool)
    for h in range(H):
        g = int(m[h])
        if not 0 <= g < G:
            drop[:, h] = True
            continue
        members = [x for x in range(H) if m[x] == g]
        k = members.index(h)
        for t in range(q_len):
            drop[t, h] = t * len(members) + k >= cap
    safe = np.where((m >= 0) & (m < G), m, 0).astype(np.int32)
    ref = oracle_variant(inp, head_group=safe, head_active=active)
    for b in range(B):
        assert np.isnan(got[b][drop]).all()
        assert_parity(got[b][~drop], ref[b][~drop], "bfloat16", f"random map seed {seed} b={b}")
