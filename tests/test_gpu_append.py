"""GPU parity of the fused cache append (gqa_decode_append) against the fp64 oracle.

The cache handed to the call holds NaN at the new tokens' positions, so the step
must take those rows from k_new / v_new. Checked afterwards:

- the output against the oracle's decode over the appended cache (oracle.append_kv);
- the cache against oracle.append_kv bit for bit: the new rows are written exactly,
  and every other byte, NaN padding included, is untouched.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from gpu_cases import assert_parity, host64, make, small_workload  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gqa_kv_cache_03_amd  # noqa: F401  (fails loudly if the library is missing)


def split_new_rows(inp):
    """Take the new tokens' K/V rows out of the generated cache ([B, q_len, G, d])
    and overwrite their cache slots with NaN."""
    wl = inp.wl
    B, q_len, G, d = wl.B, wl.q_len, wl.G, wl.d_h
    k_new = torch.empty((B, q_len, G, d), dtype=inp.q.dtype, device="cuda")
    v_new = torch.empty_like(k_new)
    for b in range(B):
        L = int(inp.lens[b])
        for t in range(q_len):
            pos = L - q_len + t
            if inp.block_table is None:
                k_new[b, t], v_new[b, t] = inp.k_cache[b, :, pos], inp.v_cache[b, :, pos]
                inp.k_cache[b, :, pos] = float("nan")
                inp.v_cache[b, :, pos] = float("nan")
            else:
                P = wl.page_size
                pg, sl = int(inp.table[b, pos // P]), pos % P
                k_new[b, t], v_new[b, t] = inp.k_cache[pg, :, sl], inp.v_cache[pg, :, sl]
                inp.k_cache[pg, :, sl] = float("nan")
                inp.v_cache[pg, :, sl] = float("nan")
    return k_new, v_new


def bits(t):
    """Raw bit patterns, so that NaN compares equal to itself."""
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu().numpy()


CASES = [
    # B, H, G, d, q_len, lens, dtype, page, policy-forcing note
    (3, 32, 8, 128, 1, [1, 77, 300], "bfloat16", 0),     # R = 4, MFMA
    (2, 32, 8, 128, 4, [4, 1500], "bfloat16", 0),       # R = 16, causal, L = q_len
    (2, 32, 4, 128, 4, [33, 700], "bfloat16", 16),      # R = 32, paged 16
    (2, 32, 2, 128, 3, [40, 129], "bfloat16", 32),      # R = 48, paged 32, rows span pages
    (2, 32, 1, 128, 4, [1000, 64], "bfloat16", 0),      # R = 128
    (2, 8, 2, 64, 2, [90, 260], "bfloat16", 16),        # d = 64, R = 8
    (2, 16, 16, 128, 1, [300, 1025], "bfloat16", 0),    # R = 1 -> vector-ALU path
    (2, 8, 2, 128, 2, [77, 300], "float32", 0),         # fp32 -> vector-ALU path
    (2, 4, 1, 64, 3, [40, 129], "float32", 16),         # fp32, paged
    (1, 32, 1, 128, 16, [700], "bfloat16", 32),         # R = 512: two row blocks, paged 32
    (2, 32, 8, 128, 16, [40, 16], "bfloat16", 0),       # new rows span two tiles; all rows new
    (2, 16, 4, 128, 8, [70, 33], "bfloat16", 16),       # new rows across a tile and a page edge
]


@pytest.mark.parametrize("B,H,G,d,q_len,lens,dtype,page", CASES)
@pytest.mark.parametrize("splits", [0, 1, 7])
def test_append_matches_oracle(B, H, G, d, q_len, lens, dtype, page, splits):
    from gqa_kv_cache_03_amd import gqa_decode_append
    wl, lens = small_workload(B, H, G, d, q_len, lens, dtype=dtype, paged=page,
                              seed=2000 + B + H + G + d + q_len + page)
    inp = make(wl, lens)
    k_new, v_new = split_new_rows(inp)
    old_k, old_v = inp.k_cache.clone(), inp.v_cache.clone()
    tbl = None if inp.table is None else inp.table.astype(np.int64)
    exp_k = oracle.append_kv(host64(old_k), host64(k_new), inp.lens, tbl, wl.page_size)
    exp_v = oracle.append_kv(host64(old_v), host64(v_new), inp.lens, tbl, wl.page_size)
    print(f"[append] {wl.name} lens={list(lens)} page={page} splits={splits}", flush=True)
    out = gqa_decode_append(inp.q, k_new, v_new, inp.k_cache, inp.v_cache, inp.seq_lens, inp.block_table,
                            scale=wl.scale, causal=wl.causal, num_splits=splits)
    torch.cuda.synchronize()
    # the cache, bit for bit (the exact values of the expected cache are the inputs')
    got_k, got_v = host64(inp.k_cache), host64(inp.v_cache)
    np.testing.assert_array_equal(np.isnan(got_k), np.isnan(exp_k))
    np.testing.assert_array_equal(np.nan_to_num(got_k), np.nan_to_num(exp_k))
    np.testing.assert_array_equal(np.isnan(got_v), np.isnan(exp_v))
    np.testing.assert_array_equal(np.nan_to_num(got_v), np.nan_to_num(exp_v))
    # the output: the oracle's decode over the appended cache
    ref = oracle.gqa_decode(host64(inp.q), exp_k, exp_v, inp.lens, wl.scale, wl.G, block_table=tbl,
                            page_size=wl.page_size, causal=wl.causal)
    assert_parity(host64(out), ref, dtype, f"append {wl.name} splits={splits}")


def test_append_equals_write_then_decode():
    """The fused call gives the same output as writing the rows and calling
    gqa_decode (same plan), and leaves the same cache bytes."""
    from gqa_kv_cache_03_amd import gqa_decode, gqa_decode_append
    wl, lens = small_workload(3, 32, 8, 128, 2, [500, 33, 1200], seed=91)
    inp = make(wl, lens)
    full_k, full_v = inp.k_cache.clone(), inp.v_cache.clone()
    ref = gqa_decode(inp.q, full_k, full_v, inp.seq_lens, scale=wl.scale)
    k_new, v_new = split_new_rows(inp)
    out = gqa_decode_append(inp.q, k_new, v_new, inp.k_cache, inp.v_cache, inp.seq_lens, scale=wl.scale)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    assert (bits(inp.k_cache) == bits(full_k)).all() and (bits(inp.v_cache) == bits(full_v)).all()


def test_append_rejects_bad_new_rows():
    from gqa_kv_cache_03_amd import gqa_decode_append
    wl, lens = small_workload(2, 32, 8, 128, 1, [100, 200], seed=93)
    inp = make(wl, lens)
    k_new, v_new = split_new_rows(inp)
    with pytest.raises(ValueError):
        gqa_decode_append(inp.q, k_new[:, :, :4], v_new, inp.k_cache, inp.v_cache, inp.seq_lens)
