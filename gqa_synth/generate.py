"""Seeded generation of decode inputs (queries, KV caches, lengths, block tables).

Recipe (stated once here, used by every test and the benchmark):

* sequence lengths L_b: fixed, or integers uniform in [len_lo, len_hi] (both ends
  inclusive) from numpy PCG64 with entropy (seed, 3);
* q, K, V values: N(0, 1) fp32 draws from a torch generator seeded from
  (seed, stream, b) with stream q=0, k=1, v=2; bf16 inputs are the RNE rounding of
  those fp32 draws;
* key-norm variation: K of KV head g is multiplied by s_g = 1 + std * z_g, z_g from
  PCG64 entropy (seed, 5), in fp32 before rounding;
* contiguous caches are [B, G, cap, d_h] with cap = max_b L_b; slots at or past L_b
  hold NaN so that any read of them shows up in the output;
* paged pools are [num_pages, G, page_size, d_h]: sequence b owns ceil(L_b / P)
  pages, taken in order from one seeded permutation of all page ids (entropy
  (seed, 4)); the block table is [B, ceil(len_hi / P)] int32 with -1 in unused
  entries; unused page slots and extra pages hold NaN.
* GQLA layers (d_c > 0): q as above; the latent of sequence b is N(0, 1) fp32 draws
  [L_b, d_c] seeded from (seed, 6, b), rounded to bf16, in a contiguous [B, cap, d_c]
  cache or a paged pool [num_pages, page_size, d_c] laid out as above; W_UK and W_UV
  are N(0, 1) / sqrt(d_c) draws [G, d_h, d_c] seeded from (seed, 7) and (seed, 8)
  (unit-variance keys and values), rounded to bf16.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

from .workloads import Workload

STREAM_Q, STREAM_K, STREAM_V, STREAM_LENS, STREAM_PERM, STREAM_KNORM, STREAM_LAT, STREAM_WUK, STREAM_WUV = range(9)


def _rng(*entropy: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(entropy))))


def _torch_seed(*entropy: int) -> int:
    st = np.random.SeedSequence(list(entropy)).generate_state(2, dtype=np.uint32)
    return int(st[0]) | (int(st[1] & 0x7FFFFFFF) << 32)


def draw_lengths(wl: Workload) -> np.ndarray:
    if wl.len_lo == wl.len_hi:
        return np.full(wl.B, wl.len_lo, dtype=np.int32)
    return _rng(wl.seed, STREAM_LENS).integers(
        wl.len_lo, wl.len_hi + 1, size=wl.B, dtype=np.int64).astype(np.int32)


def draw_key_scales(wl: Workload) -> np.ndarray:
    if wl.key_norm_std <= 0.0:
        return np.ones(wl.G, dtype=np.float32)
    z = _rng(wl.seed, STREAM_KNORM).standard_normal(wl.G)
    return (1.0 + wl.key_norm_std * z).astype(np.float32)


def draw_block_table(wl: Workload, lens: np.ndarray, extra_pages: Optional[int] = None):
    """Deal a seeded permutation of page ids to the sequences in order.

    Returns (table [B, max_blocks] int32, num_pages). Entry k of row b is the pool
    page that holds tokens [k*P, (k+1)*P) of sequence b; unused entries are -1.
    """
    P = wl.page_size
    extra = wl.extra_pages if extra_pages is None else extra_pages
    need = [-(-int(L) // P) for L in lens]
    num_pages = int(sum(need)) + int(extra)
    perm = _rng(wl.seed, STREAM_PERM).permutation(num_pages).astype(np.int32)
    max_blocks = max(wl.max_blocks_per_seq, max(need) if need else 0)
    table = np.full((wl.B, max_blocks), -1, dtype=np.int32)
    pos = 0
    for b, n in enumerate(need):
        table[b, :n] = perm[pos:pos + n]
        pos += n
    return table, num_pages


@dataclass
class DecodeInputs:
    wl: Workload
    q: "object"                 # torch.Tensor [B, q_len, H, d]
    k_cache: "object"           # contiguous [B,G,cap,d] or paged [pages,G,P,d]
    v_cache: "object"
    seq_lens: "object"          # torch int32 [B] on the same device
    block_table: "object"       # torch int32 [B, max_blocks] or None
    lens: np.ndarray            # host copy of seq_lens
    table: Optional[np.ndarray]  # host copy of the block table
    capacity: int
    num_pages: int
    key_scales: np.ndarray

    @property
    def kv_bytes(self) -> int:
        """K and V bytes the step must read: 2 * G * d_h * itemsize * sum_b L_b."""
        wl = self.wl
        return 2 * wl.G * wl.d_h * wl.itemsize * int(self.lens.astype(np.int64).sum())


def _torch_dtype(torch, name):
    return {"float32": torch.float32, "bfloat16": torch.bfloat16}[name]


def _normal(torch, shape, seed, device):
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32)


def make_inputs(wl: Workload, device="cpu", lens: Optional[np.ndarray] = None,
                nan_fill: bool = True) -> DecodeInputs:
    """Materialise a workload on `device` (torch tensors)."""
    import torch

    dt = _torch_dtype(torch, wl.dtype)
    lens = draw_lengths(wl) if lens is None else np.asarray(lens, dtype=np.int32)
    assert lens.shape == (wl.B,)
    ks = draw_key_scales(wl)
    d, G = wl.d_h, wl.G
    fill = float("nan") if nan_fill else 0.0

    q = _normal(torch, (wl.B, wl.q_len, wl.H, d), _torch_seed(wl.seed, STREAM_Q), device).to(dt)

    table = None
    if wl.layout == "paged":
        table, num_pages = draw_block_table(wl, lens)
        P = wl.page_size
        k_cache = torch.full((num_pages, G, P, d), fill, dtype=dt, device=device)
        v_cache = torch.full((num_pages, G, P, d), fill, dtype=dt, device=device)
        capacity = table.shape[1] * P
    else:
        num_pages = 0
        capacity = int(lens.max()) if wl.len_lo != wl.len_hi else wl.len_hi
        capacity = max(capacity, int(lens.max()))
        k_cache = torch.full((wl.B, G, capacity, d), fill, dtype=dt, device=device)
        v_cache = torch.full((wl.B, G, capacity, d), fill, dtype=dt, device=device)

    ks_t = torch.as_tensor(ks, device=device).view(G, 1, 1)
    for b in range(wl.B):
        L = int(lens[b])
        kb = _normal(torch, (G, L, d), _torch_seed(wl.seed, STREAM_K, b), device)
        kb = (kb * ks_t).to(dt)
        vb = _normal(torch, (G, L, d), _torch_seed(wl.seed, STREAM_V, b), device).to(dt)
        if table is None:
            k_cache[b, :, :L] = kb
            v_cache[b, :, :L] = vb
        else:
            _scatter_pages(torch, k_cache, kb, table[b], wl.page_size, device)
            _scatter_pages(torch, v_cache, vb, table[b], wl.page_size, device)
        del kb, vb

    seq_lens = torch.as_tensor(lens, dtype=torch.int32, device=device)
    bt = None if table is None else torch.as_tensor(table, dtype=torch.int32, device=device)
    return DecodeInputs(wl, q, k_cache, v_cache, seq_lens, bt, lens, table,
                        capacity, num_pages, ks)


def _scatter_pages(torch, pool, rows, table_row, P, device):
    """Write rows [G, L, d] of one sequence into its pages of pool [pages, G, P, d]."""
    G, L, d = rows.shape
    n_full = L // P
    if n_full:
        pages = torch.as_tensor(table_row[:n_full].astype(np.int64), device=device)
        pool[pages] = rows[:, :n_full * P].reshape(G, n_full, P, d).transpose(0, 1)
    tail = L - n_full * P
    if tail:
        pg = int(table_row[n_full])
        pool[pg, :, :tail] = rows[:, n_full * P:]


def paginate(torch, k_contig, lens, page_size, seed, extra_pages=0, fill=float("nan")):
    """Re-pack a contiguous cache [B,G,cap,d] into a permuted paged pool.

    Returns (pool [pages,G,P,d], table [B, ceil(cap/P)] int32 numpy, num_pages).
    The token order inside every sequence is unchanged; only storage moves.
    """
    B, G, cap, d = k_contig.shape
    P = page_size
    need = [-(-int(L) // P) for L in lens]
    num_pages = int(sum(need)) + int(extra_pages)
    perm = _rng(seed, STREAM_PERM).permutation(num_pages).astype(np.int32)
    max_blocks = -(-cap // P)
    table = np.full((B, max_blocks), -1, dtype=np.int32)
    pool = torch.full((num_pages, G, P, d), fill, dtype=k_contig.dtype, device=k_contig.device)
    pos = 0
    for b in range(B):
        n = need[b]
        table[b, :n] = perm[pos:pos + n]
        pos += n
        _scatter_pages(torch, pool, k_contig[b, :, :int(lens[b])], table[b], P, k_contig.device)
    return pool, table, num_pages


@dataclass
class LatentInputs:
    wl: Workload
    q: "object"                 # torch.Tensor [B, q_len, H, d_h]
    latent: "object"            # contiguous [B, cap, d_c] or paged [pages, P, d_c]
    w_uk: "object"              # [G, d_h, d_c]
    w_uv: "object"
    seq_lens: "object"          # torch int32 [B]
    block_table: "object"       # torch int32 [B, max_blocks] or None
    lens: np.ndarray
    table: Optional[np.ndarray]
    capacity: int
    num_pages: int

    @property
    def latent_bytes(self) -> int:
        """Latent bytes the absorbed step must read: d_c * itemsize * sum_b L_b."""
        return self.wl.d_c * self.wl.itemsize * int(self.lens.astype(np.int64).sum())


def make_latent_inputs(wl: Workload, device="cpu", lens: Optional[np.ndarray] = None,
                       nan_fill: bool = True) -> LatentInputs:
    """Materialise a GQLA workload (d_c > 0) on `device`."""
    import torch

    assert wl.d_c > 0, "not a GQLA workload"
    dt = _torch_dtype(torch, wl.dtype)
    lens = draw_lengths(wl) if lens is None else np.asarray(lens, dtype=np.int32)
    assert lens.shape == (wl.B,)
    d_c = wl.d_c
    fill = float("nan") if nan_fill else 0.0
    q = _normal(torch, (wl.B, wl.q_len, wl.H, wl.d_h), _torch_seed(wl.seed, STREAM_Q), device).to(dt)
    w_uk = (_normal(torch, (wl.G, wl.d_h, d_c), _torch_seed(wl.seed, STREAM_WUK), device) / np.sqrt(d_c)).to(dt)
    w_uv = (_normal(torch, (wl.G, wl.d_h, d_c), _torch_seed(wl.seed, STREAM_WUV), device) / np.sqrt(d_c)).to(dt)
    table = None
    if wl.layout == "paged":
        table, num_pages = draw_block_table(wl, lens)
        P = wl.page_size
        latent = torch.full((num_pages, P, d_c), fill, dtype=dt, device=device)
        capacity = table.shape[1] * P
    else:
        num_pages = 0
        capacity = max(wl.len_hi, int(lens.max()))
        latent = torch.full((wl.B, capacity, d_c), fill, dtype=dt, device=device)
    for b in range(wl.B):
        L = int(lens[b])
        cb = _normal(torch, (L, d_c), _torch_seed(wl.seed, STREAM_LAT, b), device).to(dt)
        if table is None:
            latent[b, :L] = cb
        else:
            P = wl.page_size
            n_full = L // P
            if n_full:
                pages = torch.as_tensor(table[b, :n_full].astype(np.int64), device=device)
                latent[pages] = cb[:n_full * P].reshape(n_full, P, d_c)
            if L - n_full * P:
                latent[int(table[b, n_full]), :L - n_full * P] = cb[n_full * P:]
        del cb
    seq_lens = torch.as_tensor(lens, dtype=torch.int32, device=device)
    bt = None if table is None else torch.as_tensor(table, dtype=torch.int32, device=device)
    return LatentInputs(wl, q, latent, w_uk, w_uv, seq_lens, bt, lens, table, capacity, num_pages)
