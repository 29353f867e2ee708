"""Shared helpers for the GPU parity tests: seeded inputs -> HIP path vs. CPU oracle."""
from __future__ import annotations

import numpy as np

import oracle
from gqa_synth import Workload, make_inputs

# Graded tolerance: fp32 inputs max-abs 1e-5; bf16 inputs |d| <= 2e-2 + 1e-2 |ref|.
# A stricter reported gate for bf16: relative L2 error <= 1e-2.
FP32_ATOL = 1e-5
BF16_ATOL, BF16_RTOL, BF16_RELL2 = 2e-2, 1e-2, 1e-2


def host64(t) -> np.ndarray:
    return t.detach().to("cpu").double().numpy()


def oracle_for(inp, rows_b=None, causal=True):
    """fp64 oracle output for the sequences in rows_b (all by default) of a DecodeInputs."""
    wl = inp.wl
    bs = list(range(wl.B)) if rows_b is None else list(rows_b)
    q = host64(inp.q[bs])
    lens = inp.lens[bs]
    if inp.block_table is None:
        cap = int(lens.max())
        k = host64(inp.k_cache[bs, :, :cap])
        v = host64(inp.v_cache[bs, :, :cap])
        return oracle.gqa_decode(q, k, v, lens, wl.scale, wl.G, causal=causal)
    # paged: hand the oracle a pool holding just these sequences' pages, with a
    # remapped table; the oracle does its own block-table gather
    import torch
    tbl = inp.table[bs]
    used = sorted({int(p) for b in range(len(bs)) for p in tbl[b, :-(-int(lens[b]) // wl.page_size)]})
    remap = {p: i for i, p in enumerate(used)}
    idx = torch.as_tensor(used, dtype=torch.long, device=inp.k_cache.device)
    k = host64(inp.k_cache[idx])
    v = host64(inp.v_cache[idx])
    t2 = np.full(tbl.shape, -1, dtype=np.int64)
    for b in range(len(bs)):
        n = -(-int(lens[b]) // wl.page_size)
        t2[b, :n] = [remap[int(p)] for p in tbl[b, :n]]
    return oracle.gqa_decode(q, k, v, lens, wl.scale, wl.G, block_table=t2,
                             page_size=wl.page_size, causal=causal)


def errors(got: np.ndarray, ref: np.ndarray) -> dict:
    d = np.abs(got - ref)
    big = np.abs(ref) > 1e-3
    return {
        "max_abs": float(d.max()) if d.size else 0.0,
        "max_rel": float((d[big] / np.abs(ref[big])).max()) if big.any() else 0.0,
        "rel_l2": float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300)),
        "worst": tuple(int(i) for i in np.unravel_index(np.argmax(d), d.shape)) if d.size else (),
    }


def assert_parity(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = "") -> dict:
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    e = errors(got, ref)
    if dtype == "float32":
        assert e["max_abs"] <= FP32_ATOL, f"{what}: {e}"
    else:
        bad = np.abs(got - ref) > BF16_ATOL + BF16_RTOL * np.abs(ref)
        assert not bad.any(), f"{what}: {int(bad.sum())} elements outside tolerance, {e}"
        assert e["rel_l2"] <= BF16_RELL2, f"{what}: rel-L2 {e}"
    return e


def small_workload(B, H, G, d, q_len, lens, dtype="bfloat16", paged=0, seed=7, causal=True,
                   key_norm_std=0.0, extra_pages=3):
    lo, hi = min(lens), max(lens)
    wl = Workload(name=f"t_B{B}_H{H}_G{G}_d{d}_q{q_len}", B=B, H=H, G=G, d_h=d, q_len=q_len,
                  dtype=dtype, len_lo=lo, len_hi=hi, layout="paged" if paged else "contiguous",
                  page_size=paged, causal=causal, seed=seed, key_norm_std=key_norm_std,
                  extra_pages=extra_pages if paged else 0)
    return wl, np.asarray(lens, dtype=np.int32)


def make(wl, lens, device="cuda"):
    return make_inputs(wl, device=device, lens=lens)


def host_workers() -> int:
    """Host threads for oracle work: the CPUs this process may use, at most 16."""
    import os
    try:
        n = len(os.sched_getaffinity(0))
    except Exception:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def sequence_kv_host(inp, b):
    """K and V of sequence b as host tensors [G, L_b, d] in the input dtype (the paged
    pool gathered through the block table on the device first)."""
    import torch
    wl = inp.wl
    L = int(inp.lens[b])
    if inp.block_table is None:
        return inp.k_cache[b, :, :L].cpu(), inp.v_cache[b, :, :L].cpu()
    P = wl.page_size
    n = -(-L // P)
    pages = torch.as_tensor(inp.table[b, :n].astype(np.int64), device=inp.k_cache.device)
    k = inp.k_cache[pages].transpose(0, 1).reshape(wl.G, n * P, wl.d_h)[:, :L]
    v = inp.v_cache[pages].transpose(0, 1).reshape(wl.G, n * P, wl.d_h)[:, :L]
    return k.cpu(), v.cpu()


def all_units_parity(inp, out, what: str, log=print) -> dict:
    """Compare every output element of a decode call with the fp64 oracle, one
    (sequence, KV group) unit at a time, units spread over host threads.

    out is the device output [B, q_len, H, d]. Each unit hands the oracle exactly the
    rows its group reads (K and V of that sequence and group, the group's query heads)
    and checks the group's output slice with assert_parity. Returns the worst errors.
    """
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    wl = inp.wl
    hpg = wl.H // wl.G
    got_all = out.cpu()
    q_all = inp.q.cpu()
    worst = {"max_abs": 0.0, "max_rel": 0.0, "rel_l2": 0.0, "units": 0}

    def one(b, g, k_b, v_b):
        lens = inp.lens[b:b + 1]
        q = q_all[b:b + 1, :, g * hpg:(g + 1) * hpg].double().numpy()
        k = k_b[g].double().numpy()[None, None]
        v = v_b[g].double().numpy()[None, None]
        ref = oracle.gqa_decode(q, k, v, lens, wl.scale, 1, causal=wl.causal)[0]
        got = got_all[b, :, g * hpg:(g + 1) * hpg].double().numpy()
        return assert_parity(got, ref, wl.dtype, f"{what} unit (b={b}, g={g}, L={int(lens[0])})")

    workers = host_workers()
    with threadpool_limits(limits=1, user_api="blas"), ThreadPoolExecutor(max_workers=workers) as ex:
        pending = []
        for b in range(wl.B):
            k_b, v_b = sequence_kv_host(inp, b)
            pending += [ex.submit(one, b, g, k_b, v_b) for g in range(wl.G)]
            # bound the host copies held at once: drain when two sequences' units are queued
            while len(pending) > max(2 * wl.G, workers):
                e = pending.pop(0).result()
                for key in ("max_abs", "max_rel", "rel_l2"):
                    worst[key] = max(worst[key], e[key])
                worst["units"] += 1
            del k_b, v_b
        for f in pending:
            e = f.result()
            for key in ("max_abs", "max_rel", "rel_l2"):
                worst[key] = max(worst[key], e[key])
            worst["units"] += 1
    log(f"[parity] {what}: {worst['units']} units, max_abs {worst['max_abs']:.2e} "
        f"max_rel {worst['max_rel']:.2e} rel_l2 {worst['rel_l2']:.2e} ({workers} host threads)")
    return worst
