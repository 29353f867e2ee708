"""Seeded random shapes against the fp64 oracle, GPU.

Each case draws its sizes from a fixed seed, so the set is the same on every run:
batch, heads, groups, head width, new tokens, ragged lengths, contiguous or paged
(page 16 / 32 / 64 / 128), forced workgroup or split counts, causal or not, bf16 or
fp32, either kernel policy.
The point is to cross the plans' decision boundaries at combinations no hand-written
case names: row blocks, policies, partial-slot layouts, page crossings and ragged
tails, together. The fused appends (GQA and GQLA) run on such shapes too, their caches
checked bit for bit. A few larger draws (up to 130 sequences, contexts up to 20k
tokens, pages up to 256) are checked on every (sequence, group) unit.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from gpu_cases import all_units_parity, assert_parity, host64, make, oracle_for, small_workload  # noqa: E402
from gqa_synth import Workload, make_latent_inputs  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gqa_kv_cache_03_amd  # noqa: F401  (fails loudly if the library is missing)


def draw_case(seed):
    rng = np.random.default_rng(seed)
    G = int(rng.choice([1, 2, 4, 8, 16]))
    hpg = int(rng.choice([1, 2, 3, 4, 6, 8, 16, 32]))
    H = G * hpg
    q_len = int(rng.choice([1, 1, 1, 2, 3, 4, 8, 16]))
    while hpg * q_len > 1024 or H > 256:
        q_len = max(1, q_len // 2)
        if hpg * q_len <= 1024 and H <= 256:
            break
        hpg = max(1, hpg // 2)
        H = G * hpg
    d = int(rng.choice([64, 128]))
    B = int(rng.integers(1, 6))
    lens = [int(rng.integers(q_len, 700)) for _ in range(B)]
    page = int(rng.choice([0, 0, 16, 32, 64, 128]))
    dtype = "float32" if rng.random() < 0.2 else "bfloat16"
    causal = bool(rng.random() < 0.8)
    splits = int(rng.choice([0, 0, 1, 2, 7, 50, 300]))
    policy = str(rng.choice(["auto", "auto", "valu", "mfma"] if dtype == "bfloat16" else ["auto", "valu"]))
    return B, H, G, d, q_len, lens, page, dtype, causal, splits, policy


@pytest.mark.parametrize("seed", range(40))
def test_random_gqa_shape(seed):
    from gqa_kv_cache_03_amd import gqa_decode
    B, H, G, d, q_len, lens, page, dtype, causal, splits, policy = draw_case(7000 + seed)
    wl, lens = small_workload(B, H, G, d, q_len, lens, dtype=dtype, paged=page, seed=7100 + seed, causal=causal)
    inp = make(wl, lens)
    print(f"[random] seed={seed} B={B} H={H} G={G} d={d} q_len={q_len} page={page} {dtype} causal={causal} "
          f"splits={splits} policy={policy} lens={list(lens)}", flush=True)
    out = gqa_decode(inp.q, inp.k_cache, inp.v_cache, inp.seq_lens, inp.block_table, scale=wl.scale,
                     causal=causal, num_splits=splits, policy=policy)
    torch.cuda.synchronize()
    assert_parity(host64(out), oracle_for(inp, causal=causal), dtype, f"seed {seed}")


def draw_large_case(seed):
    rng = np.random.default_rng(seed)
    G = int(rng.choice([1, 2, 4, 8, 16, 32]))
    hpg = int(rng.choice([1, 2, 4, 8, 16, 32, 64]))
    if G * hpg > 256:
        hpg = max(1, 256 // G)
    H = G * hpg
    q_len = int(rng.choice([1, 1, 2, 4, 8, 16]))
    while hpg * q_len > 1024:
        q_len //= 2
    d = int(rng.choice([64, 128]))
    B = int(rng.choice([1, 3, 17, 65, 130]))
    l_max = int(rng.choice([300, 3000, 20000]))
    if B * G * l_max > 40_000_000:  # at most 40M cached rows per tensor
        l_max = max(q_len + 1, 40_000_000 // (B * G))
    lens = [int(rng.integers(q_len, max(q_len + 1, l_max))) for _ in range(B)]
    page = int(rng.choice([0, 16, 32, 64, 128, 256]))
    causal = bool(rng.random() < 0.8)
    splits = int(rng.choice([0, 0, 0, 1, 13, 1000]))
    return B, H, G, d, q_len, lens, page, causal, splits


@pytest.mark.parametrize("seed", range(8))
def test_random_large_gqa_shape(seed):
    from gqa_kv_cache_03_amd import gqa_decode
    B, H, G, d, q_len, lens, page, causal, splits = draw_large_case(50000 + seed)
    wl, lens = small_workload(B, H, G, d, q_len, lens, dtype="bfloat16", paged=page, seed=50000 + seed,
                              causal=causal)
    inp = make(wl, lens)
    print(f"[random large] seed={seed} B={B} H={H} G={G} d={d} q_len={q_len} page={page} causal={causal} "
          f"splits={splits} max L={max(lens)}", flush=True)
    out = gqa_decode(inp.q, inp.k_cache, inp.v_cache, inp.seq_lens, inp.block_table, scale=wl.scale,
                     causal=causal, num_splits=splits)
    torch.cuda.synchronize()
    worst = all_units_parity(inp, out, f"large seed {seed}", log=lambda m: None)
    assert worst["units"] == B * G


@pytest.mark.parametrize("seed", range(12))
def test_random_gqla_shape(seed):
    from gqa_kv_cache_03_amd import gqla_absorb_decode
    rng = np.random.default_rng(7500 + seed)
    G = int(rng.choice([1, 2, 4]))
    H = G * int(rng.choice([1, 4, 8]))
    q_len = int(rng.choice([1, 1, 2, 3]))
    B = int(rng.integers(1, 5))
    d = int(rng.choice([64, 128]))
    lens = np.array([int(rng.integers(q_len, 900)) for _ in range(B)], dtype=np.int32)
    page = int(rng.choice([0, 16, 32]))
    causal = bool(rng.random() < 0.8)
    splits = int(rng.choice([0, 1, 9, 200]))
    wl = Workload(name=f"t_rand_gqla_{seed}", B=B, H=H, G=G, d_h=d, q_len=q_len, dtype="bfloat16",
                  len_lo=int(lens.min()), len_hi=int(lens.max()), layout="paged" if page else "contiguous",
                  page_size=page, causal=causal, seed=7600 + seed, extra_pages=2 if page else 0, d_c=512)
    inp = make_latent_inputs(wl, device="cuda", lens=lens)
    print(f"[random gqla] seed={seed} B={B} H={H} G={G} d={d} q_len={q_len} page={page} causal={causal} "
          f"splits={splits} lens={list(lens)}", flush=True)
    out = gqla_absorb_decode(inp.q, inp.latent, inp.w_uk, inp.w_uv, inp.seq_lens, inp.block_table,
                             scale=wl.scale, causal=causal, num_splits=splits)
    torch.cuda.synchronize()
    wk, wv = host64(inp.w_uk), host64(inp.w_uv)
    if page:
        tbl = inp.table.astype(np.int64)
        ref = oracle.gqla_decode(host64(inp.q), host64(inp.latent), wk, wv, lens, wl.scale, block_table=tbl,
                                 page_size=page, causal=causal)
    else:
        ref = oracle.gqla_decode(host64(inp.q), host64(inp.latent), wk, wv, lens, wl.scale, causal=causal)
    assert_parity(host64(out), ref, "bfloat16", f"gqla seed {seed}")


@pytest.mark.parametrize("seed", range(20))
def test_random_gqa_append_shape(seed):
    """The fused append on the same kind of random shapes (lengths seven times longer
    for every other seed): the output and both caches against the oracle."""
    from gqa_kv_cache_03_amd import gqa_decode_append
    from test_gpu_append import split_new_rows
    B, H, G, d, q_len, lens, page, dtype, causal, splits, policy = draw_case(7800 + seed)
    if seed % 2:
        lens = [q_len + (L - q_len) * 7 for L in lens]
    wl, lens = small_workload(B, H, G, d, q_len, lens, dtype=dtype, paged=page, seed=7900 + seed, causal=causal)
    inp = make(wl, lens)
    k_new, v_new = split_new_rows(inp)
    tbl = None if inp.table is None else inp.table.astype(np.int64)
    exp_k = oracle.append_kv(host64(inp.k_cache), host64(k_new), inp.lens, tbl, wl.page_size)
    exp_v = oracle.append_kv(host64(inp.v_cache), host64(v_new), inp.lens, tbl, wl.page_size)
    print(f"[random append] seed={seed} B={B} H={H} G={G} d={d} q_len={q_len} page={page} {dtype} "
          f"causal={causal} splits={splits} policy={policy} lens={list(lens)}", flush=True)
    out = gqa_decode_append(inp.q, k_new, v_new, inp.k_cache, inp.v_cache, inp.seq_lens, inp.block_table,
                            scale=wl.scale, causal=causal, num_splits=splits, policy=policy)
    torch.cuda.synchronize()
    for got, exp in ((host64(inp.k_cache), exp_k), (host64(inp.v_cache), exp_v)):
        np.testing.assert_array_equal(np.isnan(got), np.isnan(exp))
        np.testing.assert_array_equal(np.nan_to_num(got), np.nan_to_num(exp))
    ref = oracle.gqa_decode(host64(inp.q), exp_k, exp_v, inp.lens, wl.scale, wl.G, block_table=tbl,
                            page_size=wl.page_size, causal=causal)
    assert_parity(host64(out), ref, dtype, f"append seed {seed}")


@pytest.mark.parametrize("seed", range(8))
def test_random_gqla_append_shape(seed):
    """The fused latent append on random GQLA shapes: output and latent cache against the
    oracle."""
    from gqa_kv_cache_03_amd import gqla_absorb_decode_append
    from test_gpu_gqla_append import split_new_latents
    rng = np.random.default_rng(7700 + seed)
    G = int(rng.choice([1, 2, 4]))
    H = G * int(rng.choice([1, 4, 8, 16]))
    q_len = int(rng.choice([1, 2, 3, 4]))
    B = int(rng.integers(1, 5))
    d = int(rng.choice([64, 128]))
    lens = np.array([int(rng.integers(q_len, 900)) for _ in range(B)], dtype=np.int32)
    page = int(rng.choice([0, 16, 32]))
    causal = bool(rng.random() < 0.8)
    splits = int(rng.choice([0, 1, 9, 200]))
    wl = Workload(name=f"t_rand_gqla_app_{seed}", B=B, H=H, G=G, d_h=d, q_len=q_len, dtype="bfloat16",
                  len_lo=int(lens.min()), len_hi=int(lens.max()), layout="paged" if page else "contiguous",
                  page_size=page, causal=causal, seed=7750 + seed, extra_pages=2 if page else 0, d_c=512)
    inp = make_latent_inputs(wl, device="cuda", lens=lens)
    c_new = split_new_latents(inp)
    tbl = None if inp.table is None else inp.table.astype(np.int64)
    exp = oracle.append_latent(host64(inp.latent), host64(c_new), inp.lens, tbl, page)
    print(f"[random gqla append] seed={seed} B={B} H={H} G={G} d={d} q_len={q_len} page={page} "
          f"causal={causal} splits={splits} lens={list(lens)}", flush=True)
    out = gqla_absorb_decode_append(inp.q, c_new, inp.latent, inp.w_uk, inp.w_uv, inp.seq_lens, inp.block_table,
                                    scale=wl.scale, causal=causal, num_splits=splits)
    torch.cuda.synchronize()
    got = host64(inp.latent)
    np.testing.assert_array_equal(np.isnan(got), np.isnan(exp))
    np.testing.assert_array_equal(np.nan_to_num(got), np.nan_to_num(exp))
    ref = oracle.gqla_decode(host64(inp.q), exp, host64(inp.w_uk), host64(inp.w_uv), inp.lens, wl.scale,
                             block_table=tbl, page_size=page, causal=causal)
    assert_parity(host64(out), ref, "bfloat16", f"gqla append seed {seed}")
