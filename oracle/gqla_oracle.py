"""Plain fp64 CPU oracle for the decode step of Group-Query Latent Attention (GQLA).

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
benchmark's CPU-baseline leg, never by the product path. It shares no code with
the HIP library or its binding.

Source: the thelatestinai page for paper 2604.07766, the GQLA abstract. Each group of
query heads shares one pair of up-projections. Every cached token keeps one joint
latent vector. The group's keys and values are that latent mapped through the group's
up-projections: this is the expanded, per-group cache that the GQA execution reads.
The same weights can instead run as MQA with the projections absorbed: every query
head attends over the latent itself. The two executions are equivalent.

Readings where the abstract leaves a point open (each also listed in the design notes):

* the latent is one vector of d_c numbers per token, shared by all groups (the
  abstract's "joint latent"); there is no separate positional part.
* group g has W_UK[g] and W_UV[g], each d_h x d_c; its key for token j is
  W_UK[g] @ c_j and its value W_UV[g] @ c_j.
* query head h belongs to group h // (H/G), as in the plain GQA path.
* scale, causal masking, seq_lens and paging mean what they mean for the plain path;
  a paged latent pool is [num_pages, page_size, d_c].

What is computed here is the plain definition: the expanded cache, then the plain GQA
decode step over it (gqa_oracle.gqa_decode, pinned on its own). The absorbed order of
evaluation is the method's claim, and the tests use it as an independent check.
"""
from __future__ import annotations

import numpy as np

from .gqa_oracle import gqa_decode


def latent_rows(latent, b: int, L: int, block_table=None, page_size: int = 0,
                touched: set | None = None) -> np.ndarray:
    """The first L latent vectors of sequence b, as float64 [L, d_c]: latent[b, j]
    when contiguous, else slot j % page_size of page block_table[b, j // page_size].
    With `touched`, the storage location of every row read is added to it."""
    if block_table is None:
        if touched is not None:
            touched.update(("c", b, j) for j in range(L))
        return np.asarray(latent[b, :L], dtype=np.float64)
    j = np.arange(L)
    pages = np.asarray(block_table[b])[j // page_size]
    if touched is not None:
        touched.update(("p", int(pg), int(sl)) for pg, sl in zip(pages, j % page_size))
    return np.asarray(latent[pages, j % page_size], dtype=np.float64)


def touched_latent_rows(latent, seq_lens, block_table=None, page_size: int = 0) -> int:
    """Distinct latent rows (d_c numbers each) that the step reads, counted explicitly
    from the storage locations of every visible position of every sequence: the
    independent side of the latent byte-count pin (every group and head derives its
    keys and values from these same rows)."""
    seen: set = set()
    for b in range(len(seq_lens)):
        latent_rows(latent, b, int(seq_lens[b]), block_table, page_size, seen)
    return len(seen)


def expand_cache(latent, w, seq_lens, block_table=None, page_size: int = 0) -> np.ndarray:
    """The per-group cache that the GQA execution reads: entry [b, g, j] is
    w[g] @ c_j, for every sequence b, group g and visible position j < seq_lens[b].
    Returned contiguous, [B, G, max L, d_h], float64; positions past L are zero."""
    w = np.asarray(w, dtype=np.float64)                 # [G, d_h, d_c]
    G, d_h, _ = w.shape
    B = len(seq_lens)
    cap = int(np.max(np.asarray(seq_lens)))
    out = np.zeros((B, G, cap, d_h), dtype=np.float64)
    for b in range(B):
        L = int(seq_lens[b])
        C = latent_rows(latent, b, L, block_table, page_size)   # [L, d_c]
        for g in range(G):
            out[b, g, :L] = C @ w[g].T
    return out


def gqla_decode(q, latent, w_uk, w_uv, seq_lens, scale: float, block_table=None,
                page_size: int = 0, causal: bool = True):
    """Attention output for every (sequence, new token, query head) of a GQLA layer.

    q        [B, q_len, H, d_h]
    latent   [B, cap, d_c] contiguous, or [num_pages, page_size, d_c] paged
    w_uk     [G, d_h, d_c]; w_uv the same
    seq_lens [B] visible tokens per sequence, counting the q_len new ones
    returns  out [B, q_len, H, d_h] float64
    """
    w_uk = np.asarray(w_uk, dtype=np.float64)
    w_uv = np.asarray(w_uv, dtype=np.float64)
    assert w_uk.shape == w_uv.shape and w_uk.ndim == 3
    G = w_uk.shape[0]
    k = expand_cache(latent, w_uk, seq_lens, block_table, page_size)
    v = expand_cache(latent, w_uv, seq_lens, block_table, page_size)
    return gqa_decode(q, k, v, seq_lens, scale, G, causal=causal)


def append_latent(latent, new, seq_lens, block_table=None, page_size: int = 0) -> np.ndarray:
    """The latent cache after a step's new tokens are added to it, as a float64 copy.

    Every cached token keeps one joint latent vector (the GQLA abstract), so a decode
    step adds one row per new token. Reading (the same as for the plain GQA cache): the
    step's q_len new tokens are the last q_len of the seq_lens[b] positions, so row t of
    new[b] (new is [B, q_len, d_c]) becomes position seq_lens[b] - q_len + t of
    sequence b -- latent[b, pos] when contiguous, or slot pos % page_size of page
    block_table[b, pos // page_size] when paged. No other row changes.
    """
    out = np.array(latent, dtype=np.float64, copy=True)
    new = np.asarray(new, dtype=np.float64)
    B, q_len, _ = new.shape
    for b in range(B):
        L = int(seq_lens[b])
        assert q_len <= L, "every new token must be in the cache"
        for t in range(q_len):
            pos = L - q_len + t
            if block_table is None:
                out[b, pos] = new[b, t]
            else:
                out[int(block_table[b, pos // page_size]), pos % page_size] = new[b, t]
    return out


def latent_bytes(d_c: int, itemsize: int, seq_lens) -> int:
    """Latent-cache bytes one absorbed decode step must read: each visible token's
    latent once, d_c * itemsize * sum_b L_b (the expanded cache would need
    2 * G * d_h * itemsize per token)."""
    return d_c * itemsize * int(np.sum(np.asarray(seq_lens, dtype=np.int64)))
