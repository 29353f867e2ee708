"""GPU parity of the GQLA absorbed execution (gqla_absorb_decode) against the fp64 oracle.

The oracle (oracle.gqla_decode) expands the latent through each group's
up-projections and runs the plain GQA step over the expanded cache. The HIP path
instead folds W_UK into the queries, attends over the latent itself (the matrix-core
decode kernel with one 512-wide KV head that is both K and V), merges, and applies
W_UV. Covered here:

- small shapes over several tiles with ragged tails, paged and contiguous;
- causal q_len > 1;
- more than 32 packed rows (row blocks);
- forced workgroup counts, including a single workgroup;
- the library's GQA path on the expanded cache, which must agree;
- the full-size workload, every sequence.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from gpu_cases import assert_parity, host64  # noqa: E402
from gqa_synth import Workload, make_latent_inputs, workload  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gqa_kv_cache_03_amd  # noqa: F401  (fails loudly if the library is missing)


def latent_workload(B, H, G, d_h, q_len, lens, paged=0, seed=11, causal=True, extra_pages=3):
    wl = Workload(name=f"t_gqla_B{B}_H{H}_G{G}_d{d_h}_q{q_len}", B=B, H=H, G=G, d_h=d_h, q_len=q_len,
                  dtype="bfloat16", len_lo=min(lens), len_hi=max(lens),
                  layout="paged" if paged else "contiguous", page_size=paged, causal=causal, seed=seed,
                  extra_pages=extra_pages if paged else 0, d_c=512)
    return wl, np.asarray(lens, dtype=np.int32)


def oracle_latent(inp, bs=None):
    """fp64 oracle for the sequences bs (all by default)."""
    wl = inp.wl
    bs = list(range(wl.B)) if bs is None else list(bs)
    q = host64(inp.q[bs])
    lens = inp.lens[bs]
    wk, wv = host64(inp.w_uk), host64(inp.w_uv)
    if inp.block_table is None:
        lat = host64(inp.latent[bs, :int(lens.max())])
        return oracle.gqla_decode(q, lat, wk, wv, lens, wl.scale, causal=wl.causal)
    # a pool of just these sequences' pages, with a remapped table
    P = wl.page_size
    tbl = inp.table[bs]
    used = sorted({int(p) for i in range(len(bs)) for p in tbl[i, :-(-int(lens[i]) // P)]})
    remap = {p: i for i, p in enumerate(used)}
    pool = host64(inp.latent[torch.as_tensor(used, dtype=torch.long, device=inp.latent.device)])
    t2 = np.full(tbl.shape, -1, dtype=np.int64)
    for i in range(len(bs)):
        n = -(-int(lens[i]) // P)
        t2[i, :n] = [remap[int(p)] for p in tbl[i, :n]]
    return oracle.gqla_decode(q, pool, wk, wv, lens, wl.scale, block_table=t2, page_size=P, causal=wl.causal)


CASES = [
    # B, H, G, d_h, q_len, lens, page
    (2, 16, 2, 128, 1, [100, 1500], 0),        # one GPU's share at TP 8: 16 rows
    (3, 16, 2, 128, 1, [33, 700, 4097], 16),   # paged 16, ragged tails
    (2, 16, 16, 128, 2, [64, 300], 0),         # 32 rows, causal q_len 2
    (2, 8, 1, 64, 3, [40, 129], 32),           # d_h 64, paged 32, 24 rows
    (1, 128, 16, 128, 1, [513], 0),            # a whole layer: 128 rows in 4 row blocks
    (2, 40, 5, 128, 1, [200, 90], 16),         # 40 rows: 2 blocks of 32 (the second partial)
    (2, 4, 2, 128, 1, [5, 70], 0),             # 4 rows
    (2, 16, 2, 128, 1, [1, 2], 0),             # a single visible token
    (2, 16, 2, 128, 4, [4, 37], 16),           # L = q_len: the first new token sees one key
    (1, 64, 2, 128, 1, [300], 0),              # 32 heads per group: two 16-row projection rounds
    (2, 48, 1, 64, 2, [50, 333], 16),          # 48 heads in one group, d_h 64: three rounds
]


@pytest.mark.parametrize("B,H,G,d_h,q_len,lens,page", CASES)
@pytest.mark.parametrize("splits", [0, 1, 7])
def test_absorbed_matches_oracle(B, H, G, d_h, q_len, lens, page, splits):
    from gqa_kv_cache_03_amd import gqla_absorb_decode, gqla_plan
    wl, lens = latent_workload(B, H, G, d_h, q_len, lens, paged=page, seed=4000 + H + G + q_len + page)
    inp = make_latent_inputs(wl, device="cuda", lens=lens)
    pl = gqla_plan(inp.q, inp.latent, inp.w_uk, inp.block_table, num_splits=splits)
    print(f"[gqla] {wl.name} lens={list(lens)} page={page} splits={splits} rows={pl['rows']} "
          f"blocks={pl['row_blocks']} wgs={pl['workgroups']}", flush=True)
    out = gqla_absorb_decode(inp.q, inp.latent, inp.w_uk, inp.w_uv, inp.seq_lens, inp.block_table,
                             scale=wl.scale, causal=wl.causal, num_splits=splits)
    torch.cuda.synchronize()
    assert_parity(host64(out), oracle_latent(inp), "bfloat16", f"{wl.name} splits={splits}")


def test_non_causal():
    from gqa_kv_cache_03_amd import gqla_absorb_decode
    wl, lens = latent_workload(2, 16, 2, 128, 3, [50, 333], causal=False, seed=4100)
    inp = make_latent_inputs(wl, device="cuda", lens=lens)
    out = gqla_absorb_decode(inp.q, inp.latent, inp.w_uk, inp.w_uv, inp.seq_lens, scale=wl.scale, causal=False)
    torch.cuda.synchronize()
    assert_parity(host64(out), oracle_latent(inp), "bfloat16", "non-causal")


def test_absorbed_and_expanded_executions_agree():
    """The abstract's claim at the library level: the absorbed call over the latent and
    gqa_decode over the expanded caches (W c_j, formed here in fp32 and rounded to
    bf16) give the same output within the bf16 tolerance."""
    from gqa_kv_cache_03_amd import gqa_decode, gqla_absorb_decode
    wl, lens = latent_workload(3, 16, 2, 128, 1, [300, 2048, 77], seed=4200)
    inp = make_latent_inputs(wl, device="cuda", lens=lens)
    lat = inp.latent.float()                                       # [B, cap, d_c]
    k = torch.stack([torch.matmul(lat, inp.w_uk[g].float().t().contiguous()) for g in range(wl.G)], 1)
    v = torch.stack([torch.matmul(lat, inp.w_uv[g].float().t().contiguous()) for g in range(wl.G)], 1)
    k, v = k.to(torch.bfloat16).contiguous(), v.to(torch.bfloat16).contiguous()
    absorbed = gqla_absorb_decode(inp.q, inp.latent, inp.w_uk, inp.w_uv, inp.seq_lens, scale=wl.scale)
    expanded = gqa_decode(inp.q, k, v, inp.seq_lens, scale=wl.scale)
    torch.cuda.synchronize()
    ref = oracle_latent(inp)
    assert_parity(host64(absorbed), ref, "bfloat16", "absorbed")
    assert_parity(host64(expanded), ref, "bfloat16", "expanded")
    assert_parity(host64(absorbed), host64(expanded), "bfloat16", "absorbed vs expanded")


def test_repeated_calls_reuse_the_workspace():
    """Two calls in a row on one workspace, the second smaller: no state leaks."""
    from gqa_kv_cache_03_amd import gqla_absorb_decode, gqla_plan
    wl, lens = latent_workload(3, 16, 2, 128, 2, [900, 64, 1500], paged=16, seed=4300)
    inp = make_latent_inputs(wl, device="cuda", lens=lens)
    ws = torch.empty(gqla_plan(inp.q, inp.latent, inp.w_uk, inp.block_table)["workspace_bytes"],
                     dtype=torch.uint8, device="cuda")
    out1 = gqla_absorb_decode(inp.q, inp.latent, inp.w_uk, inp.w_uv, inp.seq_lens, inp.block_table,
                              scale=wl.scale, workspace=ws)
    short = torch.as_tensor([30, 64, 9], dtype=torch.int32, device="cuda")
    out2 = gqla_absorb_decode(inp.q[:, :, :, :].contiguous(), inp.latent, inp.w_uk, inp.w_uv, short,
                              inp.block_table, scale=wl.scale, workspace=ws)
    torch.cuda.synchronize()
    assert_parity(host64(out1), oracle_latent(inp), "bfloat16", "first call")
    inp.lens = np.asarray([30, 64, 9], dtype=np.int32)
    assert_parity(host64(out2), oracle_latent(inp), "bfloat16", "second call")


def test_rejects_bad_arguments():
    from gqa_kv_cache_03_amd import GqaError, gqla_absorb_decode
    wl, lens = latent_workload(1, 16, 2, 128, 1, [64], seed=4400)
    inp = make_latent_inputs(wl, device="cuda", lens=lens)
    with pytest.raises(ValueError):
        gqla_absorb_decode(inp.q, inp.latent, inp.w_uk, inp.w_uv[:1].contiguous(), inp.seq_lens)
    with pytest.raises(GqaError):       # a latent width the kernel is not built for
        gqla_absorb_decode(inp.q, inp.latent[:, :, :256].contiguous(), inp.w_uk[:, :, :256].contiguous(),
                           inp.w_uv[:, :, :256].contiguous(), inp.seq_lens)


def test_full_size_parity_every_sequence():
    """The benchmark's GQLA workload at full size, default plan; every sequence against
    the oracle (each an 8K-64K token expansion in fp64), on host threads."""
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    from gpu_cases import host_workers
    from gqa_kv_cache_03_amd import gqla_absorb_decode
    wl = workload("gqla_absorb_tp8_bf16_B16_H16_G2_d128_c512_n8k_64k")
    print(f"[gqla] {wl.name}: generating", flush=True)
    inp = make_latent_inputs(wl, device="cuda")
    out = gqla_absorb_decode(inp.q, inp.latent, inp.w_uk, inp.w_uv, inp.seq_lens, inp.block_table,
                             scale=wl.scale, causal=wl.causal)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all())
    got = host64(out)
    wk, wv = host64(inp.w_uk), host64(inp.w_uv)
    P = wl.page_size

    def one(b, q, lat):
        ref = oracle.gqla_decode(q, lat, wk, wv, inp.lens[b:b + 1], wl.scale, causal=wl.causal)
        return b, assert_parity(got[b:b + 1], ref, "bfloat16", f"{wl.name} b={b}")

    with threadpool_limits(limits=1, user_api="blas"), ThreadPoolExecutor(max_workers=host_workers()) as ex:
        futs = []
        for b in range(wl.B):
            L = int(inp.lens[b])
            n = -(-L // P)
            pages = torch.as_tensor(inp.table[b, :n].astype(np.int64), device=inp.latent.device)
            lat = host64(inp.latent[pages].reshape(1, n * P, wl.d_c)[:, :L])
            futs.append(ex.submit(one, b, host64(inp.q[b:b + 1]), lat))
        for f in futs:
            b, e = f.result()
            print(f"[gqla] {wl.name} b={b} L={int(inp.lens[b])}: max_abs {e['max_abs']:.2e} "
                  f"rel_l2 {e['rel_l2']:.2e}", flush=True)


def test_full_size_latent_append():
    """The fused latent append on the benchmark's GQLA workload at full size: afterwards
    the latent pool equals the generated one bit for bit, and every sequence of the
    output matches the oracle over it (the oracle on host threads, as above)."""
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    from gpu_cases import host_workers
    from gqa_kv_cache_03_amd import gqla_absorb_decode_append
    from test_gpu_gqla_append import split_new_latents
    wl = workload("gqla_absorb_tp8_bf16_B16_H16_G2_d128_c512_n8k_64k")
    print(f"[gqla append] {wl.name}: generating", flush=True)
    inp = make_latent_inputs(wl, device="cuda")
    full = inp.latent.clone()
    c_new = split_new_latents(inp)
    out = gqla_absorb_decode_append(inp.q, c_new, inp.latent, inp.w_uk, inp.w_uv, inp.seq_lens, inp.block_table,
                                    scale=wl.scale, causal=wl.causal)
    torch.cuda.synchronize()
    assert torch.equal(inp.latent.view(torch.int16), full.view(torch.int16)), "latent cache bytes"
    del full
    got = host64(out)
    wk, wv = host64(inp.w_uk), host64(inp.w_uv)
    P = wl.page_size

    def one(b, q, lat):
        ref = oracle.gqla_decode(q, lat, wk, wv, inp.lens[b:b + 1], wl.scale, causal=wl.causal)
        return b, assert_parity(got[b:b + 1], ref, "bfloat16", f"{wl.name} +append b={b}")

    with threadpool_limits(limits=1, user_api="blas"), ThreadPoolExecutor(max_workers=host_workers()) as ex:
        futs = []
        for b in range(wl.B):
            L = int(inp.lens[b])
            n = -(-L // P)
            pages = torch.as_tensor(inp.table[b, :n].astype(np.int64), device=inp.latent.device)
            lat = host64(inp.latent[pages].reshape(1, n * P, wl.d_c)[:, :L])
            futs.append(ex.submit(one, b, host64(inp.q[b:b + 1]), lat))
        for f in futs:
            f.result()


@pytest.mark.parametrize("splits", [0, 37])
def test_many_sequences(splits):
    """More than 64 sequences (several chunks of the schedule scan), ragged, paged."""
    from gqa_kv_cache_03_amd import gqla_absorb_decode
    rng = np.random.default_rng(4500)
    lens = rng.integers(1, 200, size=100).astype(np.int32)
    lens[70] = 1500
    wl, lens = latent_workload(100, 16, 2, 128, 1, list(lens), paged=16, seed=4600)
    inp = make_latent_inputs(wl, device="cuda", lens=lens)
    out = gqla_absorb_decode(inp.q, inp.latent, inp.w_uk, inp.w_uv, inp.seq_lens, inp.block_table,
                             scale=wl.scale, num_splits=splits)
    torch.cuda.synchronize()
    assert_parity(host64(out), oracle_latent(inp), "bfloat16", f"B=100 splits={splits}")
