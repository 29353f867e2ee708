"""Plain fp64 CPU oracle for one grouped-query-attention decode step.

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
benchmark's CPU-baseline leg, never by the product path. It shares no code with
the HIP library or its binding.

Sources (page title, section):

* "Grouped-Query Attention and Multi-Query Attention: Mathematical Foundations ..."
  (llms.blog), section "Multi-Query Attention" > "Mathematical Formulation": the
  einsum block -- logits = einsum(bhnk, bmk -> bhnm), weights = softmax(logits +
  mask), O = einsum(bhnm, bmv -> bhnv) -- and the decode cache shapes [b, H, m, d_k]
  (MHA) and [b, m, d_k] (MQA).
* same page, "Grouped-Query Attention" > "Mathematical Formulation": H query heads
  in G groups of H/G; the group's one key and value head is shared by the group's
  H/G query heads; the cache is [b, G, m, d_k].
* "Grouped-Query Attention" (aiwiki), the PyTorch listing: KV head g is expanded
  with repeat_interleave(h // g) -- contiguous blocks of H/G query heads share one
  KV head -- and attention is scaled_dot_product_attention(q, k, v, is_causal),
  whose default scale is 1/sqrt(d_head). The note after the listing: the kernel
  computes the KV head index from the query head index instead of copying.
* llms.blog page, section "PagedAttention": the cache is kept in fixed-size blocks
  of tokens; the aiwiki page's "Interaction with the cache": a page is shared by
  the h/g query heads of its group.

Readings where the pages leave a point open (each also listed in the design notes):

* scale is an explicit argument (the einsum block has none; the listing's SDPA
  default is 1/sqrt(d_head)); the fp32 value passed is applied exactly.
* with q_len > 1 new tokens and causal masking, query token t is the
  (L - q_len + t)-th position of its sequence and sees keys 0 .. L - q_len + t
  (the bottom-right alignment of verifying drafted tokens against a cache, as in
  the "Speculative Decoding" section); seq_lens counts the new tokens.
* masked keys are excluded exactly (weight 0), never given a large negative logit;
  cache slots at or past L do not exist for the step.
* bf16 inputs are taken at their exact (upcast) values.

Parity: pinned (see tests/test_oracle.py) by the MHA and MQA reductions, the
library-routine cross-check with repeat_interleave + SDPA, closed forms (mean of V,
one-hot), 50-digit brute force on tiny shapes, invariants and the byte count. One
part is parity unpinned: with head_active, an inactive (token, head) pair's output is
0 -- a reading (no page gives a value for a head the router leaves out), restated by
its test, not derived from anything the pages fix.
"""
from __future__ import annotations

import numpy as np


def bf16_bits_to_float64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 numbers given as their uint16 bit patterns."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def group_of_head(h: int, H: int, G: int) -> int:
    """KV head read by query head h: contiguous blocks of H/G heads per group
    (repeat_interleave in the aiwiki listing; on the llms.blog page each group's
    single key/value head serves all H/G query heads of that group)."""
    return h // (H // G)


def heads_of_group(g: int, H: int, G: int, head_group=None) -> list[int]:
    """Query heads that read KV head g: the contiguous block, or, with a call-time
    map (one KV head index per query head; the key-norm driven, non-uniform
    allocation of "Beyond Uniform Query Distribution: Key-Driven Grouped Query
    Attention", Figure 1), every head the map sends to g, in ascending order."""
    if head_group is None:
        return [h for h in range(H) if group_of_head(h, H, G) == g]
    return [h for h in range(H) if int(head_group[h]) == g]


def visible_keys(L: int, q_len: int, t: int, causal: bool) -> int:
    """Number of cache positions query token t of this step may attend to."""
    if not causal:
        return L
    return L - q_len + t + 1


def kv_rows(cache, b: int, g: int, L: int, block_table=None, page_size: int = 0,
            touched: set | None = None) -> np.ndarray:
    """The first L rows of KV head g of sequence b, as float64 [L, d].

    Contiguous cache: cache[b, g, j]. Paged pool: row j of sequence b lives in page
    block_table[b, j // page_size] at slot j % page_size.
    """
    if block_table is None:
        rows = np.asarray(cache[b, g, :L], dtype=np.float64)
        if touched is not None:
            touched.update(("c", b, g, j) for j in range(L))
        return rows
    j = np.arange(L)
    pages = np.asarray(block_table[b])[j // page_size]
    slots = j % page_size
    if touched is not None:
        touched.update(("p", int(p), g, int(s)) for p, s in zip(pages, slots))
    return np.asarray(cache[pages, g, slots], dtype=np.float64)


def gqa_decode(q, k_cache, v_cache, seq_lens, scale: float, G: int,
               block_table=None, page_size: int = 0, causal: bool = True,
               return_weights: bool = False, touched: set | None = None,
               head_group=None, head_active=None):
    """Attention output for every (sequence, new token, query head).

    q        [B, q_len, H, d]  (any real dtype; upcast to float64)
    k_cache  [B, G, cap, d] contiguous, or [num_pages, G, page_size, d] paged
    v_cache  same layout as k_cache
    seq_lens [B] visible keys per sequence, counting the q_len new tokens
    head_group  optional [H] KV head of each query head (non-uniform groups)
    head_active optional [B, q_len, H]; 0 marks a (token, head) pair left inactive by a
             per-token router over each group's query heads (Grouped Query Experts,
             thelatestinai page), whose output is 0: the pair is not computed (a
             reading the pages do not fix: parity unpinned)
    returns  out [B, q_len, H, d] float64 (and, if asked, a dict of weights
             {(b, t, h): w[visible]}).
    """
    q = np.asarray(q, dtype=np.float64)
    B, q_len, H, d = q.shape
    if head_group is None:
        assert G >= 1 and H % G == 0, "query heads must split evenly into KV groups"
    else:
        assert len(head_group) == H and all(0 <= int(x) < G for x in head_group)
    scale = float(np.float32(scale))
    out = np.empty((B, q_len, H, d), dtype=np.float64)
    weights = {} if return_weights else None
    for b in range(B):
        L = int(seq_lens[b])
        assert q_len <= L, "every new token must be in the cache"
        for g in range(G):
            K = kv_rows(k_cache, b, g, L, block_table, page_size, touched)
            V = kv_rows(v_cache, b, g, L, block_table, page_size, touched)
            for h in heads_of_group(g, H, G, head_group):
                Qh = q[b, :, h, :]                       # [q_len, d]
                logits = scale * (Qh @ K.T)              # [q_len, L]
                for t in range(q_len):
                    n = visible_keys(L, q_len, t, causal)
                    s = logits[t, :n]
                    e = np.exp(s - s.max())
                    w = e / e.sum()
                    out[b, t, h] = w @ V[:n]
                    if weights is not None:
                        weights[(b, t, h)] = w
    if head_active is not None:
        out[np.asarray(head_active) == 0] = 0.0
    if return_weights:
        return out, weights
    return out


def append_kv(cache, new, seq_lens, block_table=None, page_size: int = 0):
    """The cache after a step's new tokens are added to it, as a float64 copy.

    Keys and values are projections of the memory positions and, during incremental
    decoding, live in a cache with one row per position (llms.blog page,
    "Multi-Query Attention" > "Mathematical Formulation"); every step then rereads
    the whole cache ("The KV-Cache Bandwidth Wall"). Reading: the step's q_len new
    tokens occupy the last q_len of the seq_lens[b] positions, so row t of
    new[b, :, g] (new is [B, q_len, G, d]) becomes position seq_lens[b] - q_len + t of
    KV head g -- cache[b, g, pos] when contiguous, or slot pos % page_size of page
    block_table[b, pos // page_size] when paged ("PagedAttention"). No other row
    changes.
    """
    out = np.array(cache, dtype=np.float64, copy=True)
    new = np.asarray(new, dtype=np.float64)
    B, q_len, G, d = new.shape
    for b in range(B):
        L = int(seq_lens[b])
        assert q_len <= L, "every new token must be in the cache"
        for t in range(q_len):
            pos = L - q_len + t
            for g in range(G):
                if block_table is None:
                    out[b, g, pos] = new[b, t, g]
                else:
                    out[int(block_table[b, pos // page_size]), g, pos % page_size] = new[b, t, g]
    return out


def kv_bytes(G: int, d_h: int, itemsize: int, seq_lens) -> int:
    """K and V bytes one decode step must read when each group is read once:
    2 * G * d_h * itemsize * sum_b L_b. With uniform lengths n this is the
    2 * b * g * n * d_h elements of the aiwiki intro (times itemsize); with G = H it
    is the 2 * b * H * n * d_k elements of the bandwidth-wall section."""
    return 2 * G * d_h * itemsize * int(np.sum(np.asarray(seq_lens, dtype=np.int64)))


def touched_kv_rows(k_cache, v_cache, seq_lens, G: int, block_table=None,
                    page_size: int = 0) -> int:
    """Distinct cache rows (one row = d_h elements of one tensor) the oracle
    reads, counted explicitly: the independent side of the byte-count pin."""
    seen_k: set = set()
    seen_v: set = set()
    for b in range(len(seq_lens)):
        L = int(seq_lens[b])
        for g in range(G):
            kv_rows(k_cache, b, g, L, block_table, page_size, seen_k)
            kv_rows(v_cache, b, g, L, block_table, page_size, seen_v)
    return len(seen_k) + len(seen_v)
