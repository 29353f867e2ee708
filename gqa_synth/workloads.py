"""Decode workloads: head counts, lengths, layout, dtype and seeds.

Head counts follow the adoption table on the llms.blog page (section "Adoption in
Modern LLMs": Llama-3 8B is 32 query heads over 8 KV heads, Llama-2 70B is 64 over
8); the paged block size of 16 tokens is one of the two sizes the same page gives
for PagedAttention; the 8K-64K length range mirrors the GQLA abstract on the
thelatestinai.com page. Everything is synthetic: values are N(0, 1) draws.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    B: int                 # sequences in the batch
    H: int                 # query heads
    G: int                 # KV heads (groups)
    d_h: int               # head dimension (d_k = d_v)
    q_len: int             # new query tokens per sequence in this step
    dtype: str             # "float32" | "bfloat16" (q, caches and out share it)
    len_lo: int            # sequence lengths L_b (visible keys incl. the new tokens)
    len_hi: int            #   fixed when len_lo == len_hi, else uniform integers
    layout: str = "contiguous"   # "contiguous" [B,G,cap,d] | "paged" [pages,G,P,d]
    page_size: int = 0
    key_norm_std: float = 0.0    # >0: K of KV head g scaled by 1 + std * z_g
    causal: bool = True
    seed: int = 0
    extra_pages: int = 0         # unused pool pages (NaN-filled) for paged layouts
    d_c: int = 0                 # >0: a GQLA layer -- one latent of d_c per token, G groups
                                 #     of up-projections [G, d_h, d_c] (absorbed execution)
    description: str = field(default="", compare=False)

    @property
    def heads_per_group(self) -> int:
        return self.H // self.G

    @property
    def R(self) -> int:
        """Query rows that share one KV head in one step: (H/G) * q_len; for a GQLA
        layer in its absorbed form every head reads the one latent: H * q_len."""
        if self.d_c:
            return self.H * self.q_len
        return self.heads_per_group * self.q_len

    @property
    def itemsize(self) -> int:
        return 4 if self.dtype == "float32" else 2

    @property
    def scale(self) -> float:
        """1/sqrt(d_h) rounded to fp32: the value actually passed to the kernel."""
        return float(np.float32(1.0 / math.sqrt(self.d_h)))

    @property
    def capacity(self) -> int:
        """Token capacity per sequence: contiguous row stride, or blocks * page size."""
        if self.layout == "paged":
            return self.max_blocks_per_seq * self.page_size
        return self.len_hi

    @property
    def max_blocks_per_seq(self) -> int:
        if self.layout != "paged":
            return 0
        return -(-self.len_hi // self.page_size)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


def _c5(G: int) -> Workload:
    return Workload(
        name=f"causal4_bf16_B8_H32_G{G}_d128_n131072p4",
        B=8, H=32, G=G, d_h=128, q_len=4, dtype="bfloat16",
        len_lo=131072 + 4, len_hi=131072 + 4,
        key_norm_std=0.25, causal=True, seed=1005,
        description=f"group sweep G={G}: 131072 cached + 4 new tokens, causal among the new ones",
    )


WORKLOADS: dict[str, Workload] = {}
for _w in [
    Workload(
        name="decode_fp32_B1_H8_G2_d64_n128",
        B=1, H=8, G=2, d_h=64, q_len=1, dtype="float32",
        len_lo=128, len_hi=128, seed=1001,
        description="single-token fp32 decode, contiguous cache",
    ),
    Workload(
        name="llama3_8b_decode_bf16_B16_H32_G8_d128_n4096",
        B=16, H=32, G=8, d_h=128, q_len=1, dtype="bfloat16",
        len_lo=4096, len_hi=4096, seed=1002,
        description="Llama-3-8B-like layer, every sequence 4096 tokens",
    ),
    Workload(
        name="llama2_70b_ragged_bf16_B32_H64_G8_d128_n1k_32k",
        B=32, H=64, G=8, d_h=128, q_len=1, dtype="bfloat16",
        len_lo=1024, len_hi=32768, seed=1003,
        description="Llama-2-70B-like layer, ragged lengths U[1024, 32768], padded to max",
    ),
    Workload(
        name="paged16_bf16_B64_H32_G4_d128_n8k_64k",
        B=64, H=32, G=4, d_h=128, q_len=1, dtype="bfloat16",
        len_lo=8192, len_hi=65536, layout="paged", page_size=16, seed=1004,
        description="paged cache, 16-token pages, permuted block table, lengths U[8192, 65536]",
    ),
    _c5(1), _c5(2), _c5(4), _c5(8), _c5(32),
    # verification of 16 drafted tokens against the cache, in 32-token pages: the
    # MQA case packs 16 x 32 = 512 query rows per KV group
    Workload(
        name="spec16_paged32_bf16_B8_H32_G1_d128_n32k",
        B=8, H=32, G=1, d_h=128, q_len=16, dtype="bfloat16",
        len_lo=32768 + 16, len_hi=32768 + 16, layout="paged", page_size=32, seed=1006,
        description="16 new tokens (causal among them), MQA, 32-token pages",
    ),
    # GQLA (thelatestinai page for 2604.07766): the abstract measures the absorbed and
    # the expanded execution on eight GPUs with tensor parallelism over 8K-64K inputs;
    # one GPU's share at TP 8 of a layer with 128 query heads in groups of eight holds
    # 16 heads in 2 groups and the whole latent (absorption replicates it). The
    # second workload is the same share run as plain GQA over the expanded cache, which
    # holds 2 x 2 x 128 = 512 numbers per token, as many as the latent.
    Workload(
        name="gqla_absorb_tp8_bf16_B16_H16_G2_d128_c512_n8k_64k",
        B=16, H=16, G=2, d_h=128, q_len=1, dtype="bfloat16",
        len_lo=8192, len_hi=65536, layout="paged", page_size=16, seed=1008, d_c=512,
        description="GQLA absorbed: 16 heads over one 512-wide latent, 16-token pages",
    ),
    Workload(
        name="gqla_expanded_tp8_bf16_B16_H16_G2_d128_n8k_64k",
        B=16, H=16, G=2, d_h=128, q_len=1, dtype="bfloat16",
        len_lo=8192, len_hi=65536, layout="paged", page_size=16, seed=1008,
        description="the same GQLA share run as GQA over the expanded per-group cache",
    ),
    Workload(
        name="spec16_paged32_bf16_B8_H32_G4_d128_n32k",
        B=8, H=32, G=4, d_h=128, q_len=16, dtype="bfloat16",
        len_lo=32768 + 16, len_hi=32768 + 16, layout="paged", page_size=32, seed=1007,
        description="16 new tokens (causal among them), G=4, 32-token pages",
    ),
]:
    WORKLOADS[_w.name] = _w

# The single-GPU benchmark's default line: the largest configuration that fits one GPU,
# the group sweep's MHA end (G = 32, 17.2 GB of K/V).
BENCH_DEFAULT = "causal4_bf16_B8_H32_G32_d128_n131072p4"

# The long-context configurations the benchmark also reports in its default run, each
# with its step time, KV GB/s and decode-kernel roofline fraction.
BENCH_PER_CONFIG = (
    "llama2_70b_ragged_bf16_B32_H64_G8_d128_n1k_32k",
    "paged16_bf16_B64_H32_G4_d128_n8k_64k",
    "causal4_bf16_B8_H32_G1_d128_n131072p4",
    "causal4_bf16_B8_H32_G2_d128_n131072p4",
    "causal4_bf16_B8_H32_G4_d128_n131072p4",
    "causal4_bf16_B8_H32_G8_d128_n131072p4",
)


def workload(name: str) -> Workload:
    try:
        return WORKLOADS[name]
    except KeyError:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(WORKLOADS)}") from None
