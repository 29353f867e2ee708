"""Pins for the CPU oracle: each test ties it to something other than itself.

Mechanisms: the MHA and MQA reductions, a library routine (torch fp64
scaled_dot_product_attention on repeat_interleave'd K/V, the aiwiki listing's own
call), closed forms, 50-digit brute force, invariants, and the KV byte counts the
pages print. Mutation tests plant mistakes in the oracle (on the CPU) and check
that the pins catch them.
"""
import json
import math
import os
from decimal import Decimal, getcontext

import numpy as np
import pytest

import oracle
from oracle import gqa_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_case(rng, B, H, G, d, q_len, lens, cap=None, paged_P=0):
    cap = cap or int(max(lens))
    q = rng.standard_normal((B, q_len, H, d))
    k = rng.standard_normal((B, G, cap, d))
    v = rng.standard_normal((B, G, cap, d))
    for b, L in enumerate(lens):
        k[b, :, L:] = np.nan
        v[b, :, L:] = np.nan
    return q, k, v, np.asarray(lens, dtype=np.int32)


def paginate_np(rng, cache, lens, P, extra=2):
    B, G, cap, d = cache.shape
    need = [-(-int(L) // P) for L in lens]
    n_pages = sum(need) + extra
    perm = rng.permutation(n_pages)
    table = np.full((B, -(-cap // P)), -1, dtype=np.int32)
    pool = np.full((n_pages, G, P, d), np.nan)
    pos = 0
    for b, L in enumerate(lens):
        table[b, :need[b]] = perm[pos:pos + need[b]]
        pos += need[b]
        for j in range(int(L)):
            pool[table[b, j // P], :, j % P] = cache[b, :, j]
    return pool, table


# --------------------------------------------------------------- P1: MHA (G = H)

def single_head_attention(qrows, K, V, scale, n_visible):
    """One head, written independently: scalar loops, math.fsum and math.exp."""
    out = []
    for t, qv in enumerate(qrows):
        n = n_visible[t]
        logits = [scale * math.fsum(float(a) * float(b) for a, b in zip(qv, K[j])) for j in range(n)]
        m = max(logits)
        e = [math.exp(x - m) for x in logits]
        z = math.fsum(e)
        out.append([math.fsum(e[j] * float(V[j][c]) for j in range(n)) / z for c in range(len(qv))])
    return np.array(out)


@pytest.mark.parametrize("q_len,causal", [(1, True), (3, True), (2, False)])
def test_mha_reduction_head_by_head(q_len, causal):
    rng = np.random.default_rng(11)
    B, H, d = 2, 4, 8
    lens = [7, 12]
    q, k, v, lens = rand_case(rng, B, H, H, d, q_len, lens)
    scale = 0.37
    ref = oracle.gqa_decode(q, k, v, lens, scale, G=H, causal=causal)
    s32 = float(np.float32(scale))
    for b in range(B):
        L = int(lens[b])
        nvis = [L - q_len + t + 1 if causal else L for t in range(q_len)]
        for h in range(H):
            mine = single_head_attention(q[b, :, h], k[b, h, :L], v[b, h, :L], s32, nvis)
            np.testing.assert_allclose(ref[b, :, h], mine, rtol=0, atol=1e-12)


# --------------------------------------------------------------- P2: MQA einsum (G = 1)

@pytest.mark.parametrize("q_len", [1, 4])
def test_mqa_reduction_literal_einsum(q_len):
    """The MQA einsum block of the llms.blog page, written literally, at G = 1."""
    rng = np.random.default_rng(12)
    B, H, d, m = 3, 6, 16, 21
    q, k, v, lens = rand_case(rng, B, H, 1, d, q_len, [m] * B)
    scale = 0.25
    Q = q.transpose(0, 2, 1, 3)              # bhnk
    K = k[:, 0]                              # bmk
    V = v[:, 0]                              # bmv
    logits = np.einsum("bhnk,bmk->bhnm", Q, K) * scale
    mask = np.zeros((q_len, m))
    for t in range(q_len):
        mask[t, m - q_len + t + 1:] = -np.inf
    x = logits + mask
    w = np.exp(x - x.max(axis=-1, keepdims=True))
    w /= w.sum(axis=-1, keepdims=True)
    Ob = np.einsum("bhnm,bmv->bhnv", w, V)
    ref = oracle.gqa_decode(q, k, v, lens, scale, G=1)
    np.testing.assert_allclose(ref, Ob.transpose(0, 2, 1, 3), rtol=0, atol=1e-12)


# --------------------------------------------------------------- P3: library routine

def sdpa_reference(q, k, v, lens, scale, G, causal=True, enable_gqa=False):
    """torch fp64 SDPA on repeat_interleave'd K/V with an explicit bottom-right mask."""
    import torch
    import torch.nn.functional as F
    B, q_len, H, d = q.shape
    out = np.empty_like(q)
    for b in range(B):
        L = int(lens[b])
        qt = torch.from_numpy(q[b:b + 1]).transpose(1, 2)          # [1,H,q_len,d]
        kt = torch.from_numpy(np.ascontiguousarray(k[b:b + 1, :, :L]))
        vt = torch.from_numpy(np.ascontiguousarray(v[b:b + 1, :, :L]))
        if not enable_gqa:
            kt = kt.repeat_interleave(H // G, dim=1)
            vt = vt.repeat_interleave(H // G, dim=1)
        mask = torch.ones(q_len, L, dtype=torch.bool)
        if causal:
            mask = torch.ones(q_len, L, dtype=torch.bool).tril(diagonal=L - q_len)
        o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=float(np.float32(scale)),
                                           enable_gqa=enable_gqa)
        out[b] = o.transpose(1, 2).numpy()[0]
    return out


SHAPES = [  # B, H, G, d, q_len, lens
    (2, 8, 2, 16, 1, [9, 33]),
    (1, 6, 3, 8, 4, [5]),
    (3, 12, 4, 32, 2, [40, 2, 17]),
    (2, 4, 1, 8, 3, [3, 11]),
    (2, 4, 4, 8, 1, [1, 6]),
]


@pytest.mark.parametrize("B,H,G,d,q_len,lens", SHAPES)
@pytest.mark.parametrize("enable_gqa", [False, True])
def test_matches_repeat_interleave_sdpa(B, H, G, d, q_len, lens, enable_gqa):
    rng = np.random.default_rng(13 + B * H + G)
    q, k, v, lens = rand_case(rng, B, H, G, d, q_len, lens)
    scale = 1 / math.sqrt(d)
    ref = oracle.gqa_decode(q, k, v, lens, scale, G)
    lib = sdpa_reference(q, k, v, lens, scale, G, enable_gqa=enable_gqa)
    np.testing.assert_allclose(ref, lib, rtol=0, atol=1e-12)


def test_non_causal_matches_sdpa():
    rng = np.random.default_rng(14)
    q, k, v, lens = rand_case(rng, 2, 8, 2, 16, 3, [10, 4])
    ref = oracle.gqa_decode(q, k, v, lens, 0.3, 2, causal=False)
    lib = sdpa_reference(q, k, v, lens, 0.3, 2, causal=False)
    np.testing.assert_allclose(ref, lib, rtol=0, atol=1e-12)


# --------------------------------------------------------------- P4: mean of V

@pytest.mark.parametrize("mode", ["identical_keys", "zero_query", "zero_scale"])
def test_uniform_attention_is_mean_of_visible_v(mode):
    rng = np.random.default_rng(15)
    B, H, G, d, q_len = 2, 6, 2, 8, 3
    lens = [5, 13]
    q, k, v, lens = rand_case(rng, B, H, G, d, q_len, lens)
    scale = 0.5
    if mode == "identical_keys":
        for b, L in enumerate(lens):
            k[b, :, :L] = rng.standard_normal((G, 1, d))
    elif mode == "zero_query":
        q[:] = 0.0
    else:
        scale = 0.0
    ref = oracle.gqa_decode(q, k, v, lens, scale, G)
    for b, L in enumerate(lens):
        for t in range(q_len):
            n = L - q_len + t + 1           # bottom-right causal extent
            for h in range(H):
                g = h * G // H
                np.testing.assert_allclose(ref[b, t, h], v[b, g, :n].mean(axis=0), rtol=0, atol=1e-13)


# --------------------------------------------------------------- P5: one-hot

@pytest.mark.parametrize("paged", [False, True])
def test_dominant_logit_returns_that_value_row(paged):
    rng = np.random.default_rng(16)
    B, H, G, d, q_len = 2, 8, 4, 16, 2
    lens = [37, 50]
    q, k, v, lens = rand_case(rng, B, H, G, d, q_len, lens)
    scale = 0.125
    alpha = 400.0                      # scale * alpha = 50 nats above the rest
    picks = {}
    for b, L in enumerate(lens):
        for g in range(G):
            u = rng.standard_normal(d)
            u /= np.linalg.norm(u)
            k[b, g, :L] = 1e-3 * rng.standard_normal((L, d))
            j = int(rng.integers(0, L - q_len + 1))   # visible to every new token
            k[b, g, j] = alpha * u
            picks[(b, g)] = j
            for h in range(H):
                if h * G // H == g:
                    q[b, :, h] = u
    tbl, P = None, 0
    kk, vv = k, v
    if paged:
        P = 4
        kk, tbl = paginate_np(np.random.default_rng(3), k, lens, P)
        vv, _ = paginate_np(np.random.default_rng(3), v, lens, P)
    ref = oracle.gqa_decode(q, kk, vv, lens, scale, G, block_table=tbl, page_size=P)
    for (b, g), j in picks.items():
        for h in range(H):
            if h * G // H == g:
                for t in range(q_len):
                    np.testing.assert_allclose(ref[b, t, h], v[b, g, j], rtol=0, atol=1e-12)


# --------------------------------------------------------------- P6: brute force

def brute_force_decimal(q, k, v, lens, scale, G, block_table=None, P=0, causal=True):
    getcontext().prec = 50
    B, q_len, H, d = q.shape
    out = np.empty(q.shape)
    sc = Decimal(float(np.float32(scale)))
    for b in range(B):
        L = int(lens[b])
        for h in range(H):
            g = h * G // H
            for t in range(q_len):
                last = L - q_len + t if causal else L - 1
                rows = []
                for j in range(last + 1):
                    if block_table is None:
                        rows.append((k[b, g, j], v[b, g, j]))
                    else:
                        pg = block_table[b][j // P]
                        rows.append((k[pg, g, j % P], v[pg, g, j % P]))
                s = [sc * sum(Decimal(float(q[b, t, h, c])) * Decimal(float(kr[c])) for c in range(d))
                     for kr, _ in rows]
                m = max(s)
                e = [(x - m).exp() for x in s]
                z = sum(e)
                for c in range(d):
                    out[b, t, h, c] = float(sum(e[j] * Decimal(float(rows[j][1][c])) for j in range(len(rows))) / z)
    return out


BRUTE = []
for H in range(1, 9):
    for G in [g for g in range(1, H + 1) if H % g == 0]:
        BRUTE.append((H, G))


@pytest.mark.parametrize("H,G", BRUTE)
def test_brute_force_all_groupings(H, G):
    rng = np.random.default_rng(100 + 10 * H + G)
    q_len = 1 + (H + G) % 3
    d = 1 + (H * 3 + G) % 8
    lens = [int(rng.integers(q_len, 21)), int(rng.integers(q_len, 21))]
    q, k, v, lens = rand_case(rng, 2, H, G, d, q_len, lens)
    scale = float(rng.uniform(0.1, 1.5))
    for causal in (True, False):
        ref = oracle.gqa_decode(q, k, v, lens, scale, G, causal=causal)
        bf = brute_force_decimal(q, k, v, lens, scale, G, causal=causal)
        np.testing.assert_allclose(ref, bf, rtol=0, atol=1e-13)


@pytest.mark.parametrize("P", [2, 3, 4])
def test_brute_force_paged(P):
    rng = np.random.default_rng(200 + P)
    H, G, d, q_len = 6, 3, 5, 2
    lens = [11, 19]
    q, k, v, lens = rand_case(rng, 2, H, G, d, q_len, lens)
    pk, tbl = paginate_np(np.random.default_rng(P), k, lens, P)
    pv, _ = paginate_np(np.random.default_rng(P), v, lens, P)
    ref = oracle.gqa_decode(q, pk, pv, lens, 0.7, G, block_table=tbl, page_size=P)
    bf = brute_force_decimal(q, pk, pv, lens, 0.7, G, block_table=tbl, P=P)
    np.testing.assert_allclose(ref, bf, rtol=0, atol=1e-13)


# --------------------------------------------------------------- P7: bytes

def test_page_printed_reduction_factors():
    with open(os.path.join(GOLDEN, "kv_reduction_factors.json")) as f:
        entries = json.load(f)["entries"]
    lens = [1000, 37]
    for e in entries:
        if e["kind"] == "ratio":
            mha = oracle.kv_bytes(e["H"], 128, 2, lens)
            gqa = oracle.kv_bytes(e["G"], 128, 2, lens)
            assert mha == e["factor"] * gqa, e["cite"]
        else:
            one = oracle.kv_bytes(1, e["d_h"], e["itemsize"], [e["tokens"]]) // 2   # one tensor
            assert one == e["bytes_one_kv_head"], e["cite"]
            assert e["heads_mha"] * one == e["bytes_mha"], e["cite"]


@pytest.mark.parametrize("paged", [False, True])
def test_byte_count_equals_distinct_rows_read(paged):
    rng = np.random.default_rng(17)
    B, H, G, d = 3, 8, 2, 4
    lens = [5, 16, 9]
    q, k, v, lens = rand_case(rng, B, H, G, d, 1, lens, cap=20)
    tbl, P = None, 0
    if paged:
        P = 4
        k, tbl = paginate_np(np.random.default_rng(1), k, lens, P)
        v, _ = paginate_np(np.random.default_rng(1), v, lens, P)
    rows = oracle.touched_kv_rows(k, v, lens, G, tbl, P)
    assert rows * d * 2 == oracle.kv_bytes(G, d, 2, lens)
    # The H/G-times larger repeat_interleave traffic is what is avoided.
    assert oracle.kv_bytes(H, d, 2, lens) == (H // G) * oracle.kv_bytes(G, d, 2, lens)


# --------------------------------------------------------------- P9 (CPU side): paged == contiguous

def test_paged_gather_equals_contiguous_exactly():
    rng = np.random.default_rng(18)
    q, k, v, lens = rand_case(rng, 3, 8, 4, 16, 2, [30, 17, 64])
    ref = oracle.gqa_decode(q, k, v, lens, 0.2, 4)
    pk, tbl = paginate_np(np.random.default_rng(5), k, lens, 16)
    pv, _ = paginate_np(np.random.default_rng(5), v, lens, 16)
    pg = oracle.gqa_decode(q, pk, pv, lens, 0.2, 4, block_table=tbl, page_size=16)
    assert np.array_equal(ref, pg)


# --------------------------------------------------------------- P10: linearity, permutation

def test_linear_in_values():
    rng = np.random.default_rng(19)
    q, k, v1, lens = rand_case(rng, 2, 8, 2, 8, 2, [9, 14])
    v2 = rng.standard_normal(v1.shape)
    a, b = 0.7, -1.9
    o1 = oracle.gqa_decode(q, k, v1, lens, 0.4, 2)
    o2 = oracle.gqa_decode(q, k, v2, lens, 0.4, 2)
    o3 = oracle.gqa_decode(q, k, a * v1 + b * v2, lens, 0.4, 2)
    np.testing.assert_allclose(o3, a * o1 + b * o2, rtol=0, atol=1e-12)


def test_joint_key_value_permutation_invariance():
    rng = np.random.default_rng(20)
    q, k, v, lens = rand_case(rng, 2, 8, 4, 8, 1, [13, 13])
    ref = oracle.gqa_decode(q, k, v, lens, 0.4, 4)
    perm = rng.permutation(13)
    out = oracle.gqa_decode(q, k[:, :, perm], v[:, :, perm], lens, 0.4, 4)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-13)


# --------------------------------------------------------------- P12: invariants

def test_weights_are_a_distribution_and_output_in_hull():
    rng = np.random.default_rng(21)
    q, k, v, lens = rand_case(rng, 2, 8, 2, 8, 3, [6, 40])
    q *= 4.0
    out, w = oracle.gqa_decode(q, k, v, lens, 0.35, 2, return_weights=True)
    for (b, t, h), wt in w.items():
        assert abs(wt.sum() - 1.0) <= 1e-14
        assert (wt >= 0).all()
        n = len(wt)
        assert n == int(lens[b]) - 3 + t + 1
        Vv = v[b, h * 2 // 8, :n]
        assert (out[b, t, h] <= Vv.max(axis=0) + 1e-12).all()
        assert (out[b, t, h] >= Vv.min(axis=0) - 1e-12).all()


def test_bf16_upcast_matches_library_conversion():
    import torch
    bits = np.arange(65536, dtype=np.uint16)
    mine = oracle.bf16_bits_to_float64(bits)
    lib = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    finite = np.isfinite(lib)
    assert np.array_equal(mine[finite], lib[finite])
    assert np.array_equal(np.isnan(mine), np.isnan(lib))


# --------------------------------------------------------------- planted mistakes

def _pins_fail(monkeypatch, name, wrong):
    monkeypatch.setattr(O, name, wrong)
    rng = np.random.default_rng(22)
    q, k, v, lens = rand_case(rng, 2, 8, 2, 16, 3, [9, 20])
    ref = O.gqa_decode(q, k, v, lens, 0.3, 2)
    lib = sdpa_reference(q, k, v, lens, 0.3, 2)
    return not np.allclose(ref, lib, rtol=0, atol=1e-6)


def test_planted_strided_group_map_is_caught(monkeypatch):
    assert _pins_fail(monkeypatch, "group_of_head", lambda h, H, G: h % G)


def test_planted_top_left_causal_is_caught(monkeypatch):
    assert _pins_fail(monkeypatch, "visible_keys", lambda L, q_len, t, causal: t + 1)


def test_planted_off_by_one_extent_is_caught(monkeypatch):
    assert _pins_fail(monkeypatch, "visible_keys", lambda L, q_len, t, causal: L - q_len + t)


def test_planted_page_slot_mistake_is_caught(monkeypatch):
    real = O.kv_rows

    def wrong(cache, b, g, L, block_table=None, page_size=0, touched=None):
        if block_table is None:
            return real(cache, b, g, L, block_table, page_size, touched)
        j = np.arange(L)
        return np.asarray(cache[np.asarray(block_table[b])[j % page_size], g, j // page_size], dtype=np.float64)

    monkeypatch.setattr(O, "kv_rows", wrong)
    rng = np.random.default_rng(23)
    q, k, v, lens = rand_case(rng, 1, 4, 2, 4, 3, [9])    # causal: key order matters
    pk, tbl = paginate_np(np.random.default_rng(2), k, lens, 3, extra=0)
    pv, _ = paginate_np(np.random.default_rng(2), v, lens, 3, extra=0)
    ref = O.gqa_decode(q, pk, pv, lens, 0.6, 2, block_table=tbl, page_size=3)
    bf = brute_force_decimal(q, pk, pv, lens, 0.6, 2, block_table=tbl, P=3)
    assert not np.allclose(ref, bf, rtol=0, atol=1e-6)


# --------------------------------------------- cache append (the step's new tokens)

def _append_case(rng, paged_P=0):
    B, H, G, d, q_len = 3, 8, 2, 8, 3
    lens = np.array([5, 3, 11], dtype=np.int32)
    old_lens = lens - q_len
    cap = 14
    old_k = rng.standard_normal((B, G, cap, d))
    old_v = rng.standard_normal((B, G, cap, d))
    for b in range(B):                       # rows of this step and beyond: not yet written
        old_k[b, :, old_lens[b]:] = np.nan
        old_v[b, :, old_lens[b]:] = np.nan
    k_new = rng.standard_normal((B, q_len, G, d))
    v_new = rng.standard_normal((B, q_len, G, d))
    q = rng.standard_normal((B, q_len, H, d))
    return q, old_k, old_v, k_new, v_new, lens, old_lens, G


def _concatenated(old, new, old_lens, lens):
    """Expected cache, built independently: each sequence's old rows followed by its
    new tokens (np.concatenate along positions), padded with NaN."""
    B, G, cap, d = old.shape
    full = np.full_like(old, np.nan)
    for b in range(B):
        rows = np.concatenate([old[b, :, :old_lens[b]], new[b].transpose(1, 0, 2)], axis=1)
        assert rows.shape[1] == lens[b]
        full[b, :, :lens[b]] = rows
    return full


def test_append_places_new_rows_after_the_old_ones():
    q, ok, ov, kn, vn, lens, old_lens, G = _append_case(np.random.default_rng(81))
    k = oracle.append_kv(ok, kn, lens)
    exp = _concatenated(ok, kn, old_lens, lens)
    for b in range(len(lens)):
        np.testing.assert_array_equal(k[b, :, :lens[b]], exp[b, :, :lens[b]])
        assert np.isnan(k[b, :, lens[b]:]).all()          # nothing past the sequence
    assert np.isnan(ok[0, :, old_lens[0]:]).all()          # the input is not modified


def test_append_then_decode_equals_decode_on_concatenated_cache():
    q, ok, ov, kn, vn, lens, old_lens, G = _append_case(np.random.default_rng(82))
    got = oracle.gqa_decode(q, oracle.append_kv(ok, kn, lens), oracle.append_kv(ov, vn, lens), lens, 0.4, G)
    ref = oracle.gqa_decode(q, _concatenated(ok, kn, old_lens, lens), _concatenated(ov, vn, old_lens, lens),
                            lens, 0.4, G)
    np.testing.assert_array_equal(got, ref)


@pytest.mark.parametrize("P", [2, 4])
def test_append_paged_equals_contiguous(P):
    rng = np.random.default_rng(83)
    q, ok, ov, kn, vn, lens, old_lens, G = _append_case(rng)
    zk = np.nan_to_num(ok, nan=0.0)
    pool, table = paginate_np(np.random.default_rng(5), zk, lens, P)   # pages for all lens rows
    pool_after = oracle.append_kv(pool, kn, lens, block_table=table, page_size=P)
    contig_after = oracle.append_kv(zk, kn, lens)
    for b in range(len(lens)):
        for j in range(lens[b]):
            np.testing.assert_array_equal(pool_after[table[b, j // P], :, j % P], contig_after[b, :, j])


def test_planted_append_position_mistake_is_caught():
    q, ok, ov, kn, vn, lens, old_lens, G = _append_case(np.random.default_rng(84))
    wrong = np.array(ok, copy=True)
    for b in range(len(lens)):                  # off by one: the new rows one slot late
        for t in range(kn.shape[1]):
            pos = lens[b] - kn.shape[1] + t + 1
            if pos < ok.shape[2]:
                wrong[b, :, pos] = kn[b, t]
    exp = _concatenated(ok, kn, old_lens, lens)
    assert not all(np.array_equal(wrong[b, :, :lens[b]], exp[b, :, :lens[b]]) for b in range(len(lens)))


# ------------------------------ grouping variants: call-time head map, active mask

def sdpa_gather_reference(q, k, v, lens, scale, head_group, causal=True):
    """torch fp64 SDPA with each query head's K/V gathered by index_select through the
    map (the non-uniform counterpart of repeat_interleave), explicit bottom-right mask."""
    import torch
    import torch.nn.functional as F
    B, q_len, H, d = q.shape
    idx = torch.as_tensor(np.asarray(head_group, dtype=np.int64))
    out = np.empty_like(q)
    for b in range(B):
        L = int(lens[b])
        qt = torch.from_numpy(q[b:b + 1]).transpose(1, 2)
        kt = torch.from_numpy(np.ascontiguousarray(k[b:b + 1, :, :L])).index_select(1, idx)
        vt = torch.from_numpy(np.ascontiguousarray(v[b:b + 1, :, :L])).index_select(1, idx)
        mask = torch.ones(q_len, L, dtype=torch.bool)
        if causal:
            mask = mask.tril(diagonal=L - q_len)
        o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=float(np.float32(scale)))
        out[b] = o.transpose(1, 2).numpy()[0]
    return out


def test_uniform_head_map_equals_contiguous_groups():
    rng = np.random.default_rng(91)
    q, k, v, lens = rand_case(rng, 2, 8, 2, 16, 3, [9, 20])
    a = O.gqa_decode(q, k, v, lens, 0.3, 2)
    b = O.gqa_decode(q, k, v, lens, 0.3, 2, head_group=[h // 4 for h in range(8)])
    np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("head_group", [
    [2, 0, 0, 1, 2, 2, 2, 0],        # unequal groups, interleaved
    [1, 1, 1, 1, 1, 1, 1, 1],        # every head on one KV head; KV heads 0 and 2 idle
    [0, 1, 2, 0, 1, 2, 0, 1],        # strided
])
def test_head_map_matches_gathered_sdpa(head_group):
    rng = np.random.default_rng(92)
    q, k, v, lens = rand_case(rng, 2, 8, 3, 16, 3, [9, 20])
    ref = sdpa_gather_reference(q, k, v, lens, 0.3, head_group)
    got = O.gqa_decode(q, k, v, lens, 0.3, 3, head_group=head_group)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_planted_head_map_ignored_is_caught():
    rng = np.random.default_rng(93)
    q, k, v, lens = rand_case(rng, 1, 8, 2, 8, 2, [12])
    hg = [1, 0, 1, 0, 0, 0, 1, 1]
    ref = sdpa_gather_reference(q, k, v, lens, 0.5, hg)
    wrong = O.gqa_decode(q, k, v, lens, 0.5, 2)          # contiguous groups instead of the map
    assert not np.allclose(wrong, ref, rtol=0, atol=1e-6)


def test_inactive_pairs_are_zero_and_others_unchanged():
    rng = np.random.default_rng(94)
    q, k, v, lens = rand_case(rng, 2, 8, 2, 16, 3, [9, 20])
    act = (rng.random((2, 3, 8)) < 0.5).astype(np.uint8)
    full = O.gqa_decode(q, k, v, lens, 0.3, 2)
    got = O.gqa_decode(q, k, v, lens, 0.3, 2, head_active=act)
    np.testing.assert_array_equal(got[act == 0], 0.0)
    np.testing.assert_array_equal(got[act == 1], full[act == 1])
