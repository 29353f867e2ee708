"""Pins for the GQLA part of the CPU oracle (oracle.gqla_decode).

The oracle expands the latent cache through each group's up-projections and runs the
plain GQA step over it. Each test ties that to something other than itself:

- the absorbed order of evaluation, which the GQLA abstract (thelatestinai page for
  2604.07766) says is equivalent: every head attends over the latent with the
  key projection folded into its query, and the value projection is applied after
  the weighted sum;
- two special cases that reduce to the plain paths: identity projections give MQA
  over the latent, and slice-selecting projections give GQA over slices of it;
- 50-digit brute force on tiny shapes;
- paged against contiguous, and the byte count;
- planted mistakes, which the pins must catch.
"""
from decimal import Decimal, getcontext

import numpy as np
import pytest

import oracle
from oracle import gqla_oracle as GL


def rand_gqla(rng, B, H, G, d_h, d_c, q_len, lens, cap=None):
    cap = cap or int(max(lens))
    q = rng.standard_normal((B, q_len, H, d_h))
    lat = rng.standard_normal((B, cap, d_c))
    for b, L in enumerate(lens):
        lat[b, L:] = np.nan       # positions past the end must never be read
    w_uk = rng.standard_normal((G, d_h, d_c)) / np.sqrt(d_c)
    w_uv = rng.standard_normal((G, d_h, d_c)) / np.sqrt(d_c)
    return q, lat, w_uk, w_uv, np.asarray(lens, dtype=np.int32)


def paginate_latent(rng, lat, lens, P, extra=2):
    B, cap, d_c = lat.shape
    need = [-(-int(L) // P) for L in lens]
    n_pages = sum(need) + extra
    perm = rng.permutation(n_pages)
    table = np.full((B, -(-cap // P)), -1, dtype=np.int32)
    pool = np.full((n_pages, P, d_c), np.nan)
    pos = 0
    for b, L in enumerate(lens):
        table[b, :need[b]] = perm[pos:pos + need[b]]
        pos += need[b]
        for j in range(int(L)):
            pool[table[b, j // P], j % P] = lat[b, j]
    return pool, table


def absorbed(q, lat, w_uk, w_uv, lens, scale, causal=True):
    """The MQA-absorb order, written out independently: fold W_UK into the query,
    attend over the latent itself, apply W_UV to the weighted latent sum."""
    B, q_len, H, d_h = q.shape
    G = w_uk.shape[0]
    out = np.empty(q.shape)
    sc = float(np.float32(scale))
    for b in range(B):
        L = int(lens[b])
        C = np.asarray(lat[b, :L], dtype=np.float64)
        for h in range(H):
            g = h // (H // G)
            for t in range(q_len):
                n = L - q_len + t + 1 if causal else L
                qt = w_uk[g].T @ q[b, t, h]              # [d_c]
                s = sc * (C[:n] @ qt)
                e = np.exp(s - s.max())
                u = (e / e.sum()) @ C[:n]                # weighted latent, [d_c]
                out[b, t, h] = w_uv[g] @ u
    return out


SHAPES = [
    # B, H, G, d_h, d_c, q_len, lens
    (2, 4, 2, 3, 7, 1, [5, 12]),
    (2, 8, 2, 4, 6, 3, [9, 4]),
    (1, 6, 3, 5, 5, 2, [17]),
    (3, 4, 1, 2, 9, 1, [1, 8, 3]),
    (2, 8, 8, 3, 4, 2, [6, 11]),
]


@pytest.mark.parametrize("B,H,G,d_h,d_c,q_len,lens", SHAPES)
@pytest.mark.parametrize("causal", [True, False])
def test_absorbed_order_equals_expanded_cache(B, H, G, d_h, d_c, q_len, lens, causal):
    rng = np.random.default_rng(700 + H * 10 + G + d_c)
    q, lat, w_uk, w_uv, lens = rand_gqla(rng, B, H, G, d_h, d_c, q_len, lens)
    ref = oracle.gqla_decode(q, lat, w_uk, w_uv, lens, 0.45, causal=causal)
    np.testing.assert_allclose(ref, absorbed(q, lat, w_uk, w_uv, lens, 0.45, causal), rtol=0, atol=1e-12)


def test_identity_projections_reduce_to_mqa_over_the_latent():
    rng = np.random.default_rng(710)
    B, H, G, d, q_len = 2, 6, 3, 5, 2
    q, lat, _, _, lens = rand_gqla(rng, B, H, G, d, d, q_len, [7, 13])
    eye = np.broadcast_to(np.eye(d), (G, d, d))
    ref = oracle.gqla_decode(q, lat, eye, eye, lens, 0.8)
    cache = lat[:, None]                        # one KV head that every query head reads
    np.testing.assert_allclose(ref, oracle.gqa_decode(q, cache, cache, lens, 0.8, 1), rtol=0, atol=1e-13)


def test_slice_projections_reduce_to_gqa_over_latent_slices():
    """W_UK[g] picks latent dims [g d_h, (g+1) d_h), W_UV[g] the next group's slice:
    the expanded caches are those slices, so the step is plain GQA over them."""
    rng = np.random.default_rng(720)
    B, H, G, d_h, q_len = 2, 8, 4, 3, 2
    d_c = G * d_h
    q, lat, _, _, lens = rand_gqla(rng, B, H, G, d_h, d_c, q_len, [6, 10])
    sel = np.zeros((G, d_h, d_c))
    for g in range(G):
        sel[g, :, g * d_h:(g + 1) * d_h] = np.eye(d_h)
    sel_v = np.roll(sel, 1, axis=0)             # group g reads slice g - 1 as its values
    ref = oracle.gqla_decode(q, lat, sel, sel_v, lens, 0.6)
    k = np.stack([lat[:, :, g * d_h:(g + 1) * d_h] for g in range(G)], axis=1)
    v = np.stack([lat[:, :, ((g - 1) % G) * d_h:((g - 1) % G + 1) * d_h] for g in range(G)], axis=1)
    np.testing.assert_allclose(ref, oracle.gqa_decode(q, k, v, lens, 0.6, G), rtol=0, atol=1e-13)


def brute_force_absorbed(q, lat, w_uk, w_uv, lens, scale, causal=True):
    """50-digit decimal arithmetic, in the absorbed order."""
    getcontext().prec = 50
    B, q_len, H, d_h = q.shape
    G, _, d_c = w_uk.shape
    D = lambda x: Decimal(float(x))  # noqa: E731
    sc = D(np.float32(scale))
    out = np.empty(q.shape)
    for b in range(B):
        L = int(lens[b])
        for h in range(H):
            g = h * G // H
            for t in range(q_len):
                n = L - q_len + t + 1 if causal else L
                qt = [sum(D(q[b, t, h, i]) * D(w_uk[g, i, c]) for i in range(d_h)) for c in range(d_c)]
                s = [sc * sum(qt[c] * D(lat[b, j, c]) for c in range(d_c)) for j in range(n)]
                m = max(s)
                e = [(x - m).exp() for x in s]
                z = sum(e)
                u = [sum(e[j] * D(lat[b, j, c]) for j in range(n)) / z for c in range(d_c)]
                for i in range(d_h):
                    out[b, t, h, i] = float(sum(D(w_uv[g, i, c]) * u[c] for c in range(d_c)))
    return out


@pytest.mark.parametrize("H,G,d_h,d_c,q_len", [(2, 1, 2, 3, 1), (4, 2, 3, 2, 2), (6, 3, 2, 4, 3)])
def test_brute_force(H, G, d_h, d_c, q_len):
    rng = np.random.default_rng(730 + H + d_c)
    q, lat, w_uk, w_uv, lens = rand_gqla(rng, 2, H, G, d_h, d_c, q_len, [q_len + 4, q_len + 9])
    for causal in (True, False):
        ref = oracle.gqla_decode(q, lat, w_uk, w_uv, lens, 0.9, causal=causal)
        bf = brute_force_absorbed(q, lat, w_uk, w_uv, lens, 0.9, causal=causal)
        np.testing.assert_allclose(ref, bf, rtol=0, atol=1e-13)


@pytest.mark.parametrize("P", [2, 4, 5])
def test_paged_latent_equals_contiguous_exactly(P):
    rng = np.random.default_rng(740 + P)
    q, lat, w_uk, w_uv, lens = rand_gqla(rng, 3, 4, 2, 3, 6, 2, [5, 17, 11])
    pool, tbl = paginate_latent(np.random.default_rng(P), lat, lens, P)
    ref = oracle.gqla_decode(q, lat, w_uk, w_uv, lens, 0.5)
    got = oracle.gqla_decode(q, pool, w_uk, w_uv, lens, 0.5, block_table=tbl, page_size=P)
    assert np.array_equal(ref, got)


@pytest.mark.parametrize("P", [0, 3, 4])
def test_latent_bytes_count_each_token_once(P):
    """latent_bytes against an explicit count of the distinct latent rows (storage
    locations) the step reads, contiguous and paged with a permuted table: every
    visible token's latent is read once, whatever the number of heads and groups."""
    rng = np.random.default_rng(760 + P)
    lens = [9, 2, 14, 5]
    d_c = 6
    lat = rng.standard_normal((len(lens), max(lens) + 3, d_c))
    if P:
        pool, tbl = paginate_latent(np.random.default_rng(P), lat, np.asarray(lens), P)
        rows = oracle.touched_latent_rows(pool, lens, tbl, P)
    else:
        rows = oracle.touched_latent_rows(lat, lens)
    assert rows == sum(lens)
    assert oracle.latent_bytes(d_c, 2, lens) == d_c * 2 * rows
    # the expanded cache of the same layer reads 2 G d_h numbers per token instead of d_c
    G, d_h = 3, 4
    k = np.zeros((len(lens), G, max(lens), d_h))
    assert oracle.kv_bytes(G, d_h, 2, lens) == oracle.touched_kv_rows(k, k, lens, G) * d_h * 2
    assert oracle.kv_bytes(G, d_h, 2, lens) * d_c == oracle.latent_bytes(d_c, 2, lens) * 2 * G * d_h


# --------------------------------------------------------------- planted mistakes

def _caught(monkeypatch, name, wrong, d_h=4, d_c=4):
    monkeypatch.setattr(GL, name, wrong)
    rng = np.random.default_rng(750)
    q, lat, w_uk, w_uv, lens = rand_gqla(rng, 2, 6, 3, d_h, d_c, 2, [7, 12])
    ref = GL.gqla_decode(q, lat, w_uk, w_uv, lens, 0.7)
    return not np.allclose(ref, absorbed(q, lat, w_uk, w_uv, lens, 0.7), rtol=0, atol=1e-6)


def test_planted_transposed_projection_is_caught(monkeypatch):
    real = GL.expand_cache
    assert _caught(monkeypatch, "expand_cache",
                   lambda lat, w, lens, bt=None, P=0: real(lat, np.swapaxes(np.asarray(w), 1, 2), lens, bt, P))


def test_planted_wrong_group_weights_is_caught(monkeypatch):
    real = GL.expand_cache
    assert _caught(monkeypatch, "expand_cache",
                   lambda lat, w, lens, bt=None, P=0: real(lat, np.roll(np.asarray(w), 1, axis=0), lens, bt, P),
                   d_h=3, d_c=5)


def test_planted_page_slot_mistake_is_caught(monkeypatch):
    real = GL.latent_rows

    def wrong(lat, b, L, block_table=None, page_size=0):
        if block_table is None:
            return real(lat, b, L)
        j = np.arange(L)
        return np.asarray(lat[np.asarray(block_table[b])[j % page_size], j // page_size], dtype=np.float64)

    monkeypatch.setattr(GL, "latent_rows", wrong)
    rng = np.random.default_rng(760)
    # 9 tokens in 3-token pages, 3 new ones: the mistake swaps which keys the first
    # new token sees
    q, lat, w_uk, w_uv, lens = rand_gqla(rng, 1, 4, 2, 3, 5, 3, [9])
    pool, tbl = paginate_latent(np.random.default_rng(3), lat, lens, 3, extra=0)
    ref = GL.gqla_decode(q, pool, w_uk, w_uv, lens, 0.6, block_table=tbl, page_size=3)
    assert not np.allclose(ref, absorbed(q, lat, w_uk, w_uv, lens, 0.6), rtol=0, atol=1e-6)


# ------------------------------ the latent append (oracle.append_latent)

def _latent_append_case(rng, q_len=3):
    old_lens = np.array([5, 1, 9], dtype=np.int32)
    lens = old_lens + q_len
    cap = int(lens.max()) + 2
    B, d_c = len(lens), 6
    old = np.full((B, cap, d_c), np.nan)
    for b in range(B):
        old[b, :old_lens[b]] = rng.standard_normal((old_lens[b], d_c))
    new = rng.standard_normal((B, q_len, d_c))
    return old, new, old_lens, lens


def test_latent_append_places_new_rows_after_the_old_ones():
    old, new, old_lens, lens = _latent_append_case(np.random.default_rng(91))
    got = oracle.append_latent(old, new, lens)
    for b in range(len(lens)):
        exp = np.concatenate([old[b, :old_lens[b]], new[b]], axis=0)     # the sequence grows by q_len rows
        np.testing.assert_array_equal(got[b, :lens[b]], exp)
        assert np.isnan(got[b, lens[b]:]).all()                           # nothing past the sequence
    assert np.isnan(old[1, old_lens[1]:]).all()                           # the input is not modified


def test_latent_append_then_expand_equals_expand_then_gqa_append():
    """Appending a latent row and expanding it through the group's projections gives the
    row the plain GQA append writes for that group (W c_new): the two oracle appends agree
    through expand_cache."""
    rng = np.random.default_rng(92)
    old, new, old_lens, lens = _latent_append_case(rng, q_len=2)
    G, d_h = 2, 3
    w = rng.standard_normal((G, d_h, old.shape[2]))
    via_latent = GL.expand_cache(oracle.append_latent(old, new, lens), w, lens)
    new_kv = np.einsum("gic,btc->btgi", w, new)                             # [B, q_len, G, d_h]
    via_kv = oracle.append_kv(GL.expand_cache(old, w, lens), new_kv, lens)
    for b in range(len(lens)):
        np.testing.assert_allclose(via_latent[b, :, :lens[b]], via_kv[b, :, :lens[b]], rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("P", [2, 4])
def test_latent_append_paged_equals_contiguous(P):
    old, new, old_lens, lens = _latent_append_case(np.random.default_rng(93))
    zero = np.nan_to_num(old, nan=0.0)
    pool, tbl = paginate_latent(np.random.default_rng(P), zero, lens, P)
    pool_after = oracle.append_latent(pool, new, lens, block_table=tbl, page_size=P)
    contig_after = oracle.append_latent(zero, new, lens)
    for b in range(len(lens)):
        for j in range(lens[b]):
            np.testing.assert_array_equal(pool_after[tbl[b, j // P], j % P], contig_after[b, j])


def test_planted_latent_append_position_mistake_is_caught():
    old, new, old_lens, lens = _latent_append_case(np.random.default_rng(94))
    wrong = np.array(old, copy=True)
    for b in range(len(lens)):                  # off by one: the new rows one slot late
        for t in range(new.shape[1]):
            wrong[b, lens[b] - new.shape[1] + t + 1] = new[b, t]
    assert not all(np.array_equal(wrong[b, :lens[b]], np.concatenate([old[b, :old_lens[b]], new[b]]))
                   for b in range(len(lens)))
