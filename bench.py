#!/usr/bin/env python3
"""Single-GPU benchmark of one GQA decode step (the decode kernel + LSE merge).

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--append]

With no --workload the step runs on the largest configuration that fits one GPU (the
group sweep at G = 32: 8 sequences of 131072 + 4 tokens, 17.2 GB of K/V), and the line
also carries `per_config`: the same measurement on the other long-context
configurations (ragged, paged, and the group sweep at G = 1, 2, 4, 8).

A step is one gqa_decode call (gqa_decode_append with --append; gqla_absorb_decode for
a GQLA workload, gqla_absorb_decode_append with --append) over the whole batch of the
workload, inputs resident in HBM. Several
copies of the cache are rotated so that every step reads cold data (the 256 MiB
Infinity Cache cannot serve a step from the previous one). Prints one JSON line:

  value      KV GB/s = 2 * G * d_h * itemsize * sum(seq_lens) / (time per step); for a
             GQLA workload the latent's d_c * itemsize * sum(seq_lens)
  roofline   the decode kernel's algorithmic bytes over its own duration (HIP events
             that its launch stamps) against MI355X's 8 TB/s HBM peak, or its matrix
             work against the 2.5 PFLOP/s bf16 peak when that bounds it
  cpu_baseline  the fp64 CPU oracle on a bounded sample of the same workload
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GQA decode KV GB/s (% of MI355X HBM peak) and tokens/s at 1 GPU"
HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16 matrix-core peak (no sparsity)
KERNEL_SOURCES = ("decode_mfma.hip", "decode_valu.hip", "gqa_internal.h", "mfma_common.h")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "gqa_kv_cache_03_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str):
    """HBM bytes per decode launch from the committed rocprofv3 counter summary,
    if it was taken on the current kernel sources (else null)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # enough warm-up for the clocks to settle: a fresh process's first few steps run slow
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--num-splits", type=int, default=0)
    ap.add_argument("--chunk", type=int, default=0)
    ap.add_argument("--policy", default="auto", choices=["auto", "valu", "mfma"])
    ap.add_argument("--head-map", action="store_true",
                    help="non-uniform grouping: a seeded head->KV-head map with groups of up to 2*H/G heads")
    ap.add_argument("--active-frac", type=float, default=0.0,
                    help="per-(token, head) active mask with this fraction of pairs active (0: no mask)")
    ap.add_argument("--append", action="store_true",
                    help="time the fused append: the step also writes the new tokens' K/V (or latents) "
                         "into the cache")
    ap.add_argument("--copies", type=int, default=0, help="KV cache copies rotated (0: enough for >= 1 GiB)")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true")
    ap.add_argument("--no-per-config", action="store_true",
                    help="default run only: skip the other long-context configurations")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (counter calibration)")
    return ap.parse_args()


def calibrate_copy(mib: int) -> None:
    """A plain device-to-device copy of known size, for scaling HBM byte counters."""
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": n, "launches": 3}), flush=True)


def cpu_baseline(inp, budget_s: float):
    """Time the oracle, as it is, on (sequence, KV group) units in order until the
    budget is spent -- starting over from the first unit when a pass over the whole
    workload ends sooner -- and report KV GB/s over the sample."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
    except Exception:  # pragma: no cover
        threadpool_info = lambda: []
    wl = inp.wl
    hpg = wl.H // wl.G
    n_units = wl.B * wl.G
    # host fp32 copies are made outside the timer; kept across passes when they fit
    keep = 2 * 4 * wl.d_h * int(sum(int(L) for L in inp.lens)) * wl.G <= (4 << 30)
    cache = {}

    def unit(b, g):
        if (b, g) in cache:
            return cache[(b, g)]
        L = int(inp.lens[b])
        q = inp.q[b:b + 1, :, g * hpg:(g + 1) * hpg].float().cpu().numpy()
        if inp.block_table is None:
            k = inp.k_cache[b:b + 1, g:g + 1, :L].float().cpu().numpy()
            v = inp.v_cache[b:b + 1, g:g + 1, :L].float().cpu().numpy()
            tbl, P = None, 0
        else:
            import torch
            P = wl.page_size
            n = -(-L // P)
            pages = torch.as_tensor(inp.table[b, :n].astype(np.int64), device=inp.k_cache.device)
            k = inp.k_cache[pages][:, g:g + 1].float().cpu().numpy()
            v = inp.v_cache[pages][:, g:g + 1].float().cpu().numpy()
            tbl = np.arange(n, dtype=np.int64)[None, :]
        args = (q, k, v, tbl, P)
        if keep:
            cache[(b, g)] = args
        return args

    done_bytes, elapsed, units = 0, 0.0, 0
    while units == 0 or elapsed < budget_s:
        for i in range(n_units):
            b, g = divmod(i, wl.G)
            q, k, v, tbl, P = unit(b, g)
            t0 = time.perf_counter()
            oracle.gqa_decode(q, k, v, inp.lens[b:b + 1], wl.scale, 1, block_table=tbl, page_size=P,
                              causal=wl.causal)
            elapsed += time.perf_counter() - t0
            done_bytes += 2 * wl.d_h * wl.itemsize * int(inp.lens[b])
            units += 1
            if elapsed >= budget_s:
                break
    threads = 0
    for info in threadpool_info():
        if info.get("user_api") == "blas":
            threads = max(threads, int(info.get("num_threads", 0)))
    try:
        avail = len(os.sched_getaffinity(0))
    except Exception:  # pragma: no cover
        avail = os.cpu_count()
    return {
        "value": round(done_bytes / elapsed / 1e9, 4),
        "unit": "GB/s",
        "cores": threads or avail,
        "kind": "oracle",
        "sample": (f"{units} (sequence, KV group) units in order ({units / n_units:.2f} passes over the "
                   f"workload's {n_units}), {elapsed:.1f} s of fp64 numpy oracle time; "
                   f"{done_bytes / 1e6:.1f} MB of KV; host fp32 copies of the inputs, upcast inside the "
                   f"timed region; {avail} cores visible"),
        "tokens_per_s_equiv": round(units / n_units * wl.B * wl.q_len / elapsed, 3),
    }


def cpu_baseline_latent(inp, budget_s: float):
    """The GQLA oracle, as it is, on whole sequences in order (starting over when a
    pass ends sooner) until the budget is spent; KV GB/s counts the latent bytes."""
    import numpy as np
    import oracle
    wl = inp.wl
    wk = inp.w_uk.float().cpu().numpy()
    wv = inp.w_uv.float().cpu().numpy()
    done_bytes, elapsed, units = 0, 0.0, 0
    while units == 0 or elapsed < budget_s:
        for b in range(wl.B):
            L = int(inp.lens[b])
            q = inp.q[b:b + 1].float().cpu().numpy()
            if inp.block_table is None:
                lat = inp.latent[b:b + 1, :L].float().cpu().numpy()
            else:
                import torch
                n = -(-L // wl.page_size)
                pages = torch.as_tensor(inp.table[b, :n].astype(np.int64), device=inp.latent.device)
                lat = inp.latent[pages].reshape(1, n * wl.page_size, wl.d_c)[:, :L].float().cpu().numpy()
            t0 = time.perf_counter()
            oracle.gqla_decode(q, lat, wk, wv, inp.lens[b:b + 1], wl.scale, causal=wl.causal)
            elapsed += time.perf_counter() - t0
            done_bytes += wl.d_c * wl.itemsize * L
            units += 1
            if elapsed >= budget_s:
                break
    try:
        avail = len(os.sched_getaffinity(0))
    except Exception:  # pragma: no cover
        avail = os.cpu_count()
    return {
        "value": round(done_bytes / elapsed / 1e9, 4),
        "unit": "GB/s",
        "cores": avail,
        "kind": "oracle",
        "sample": (f"{units} sequences in order ({units / wl.B:.2f} passes over the workload's {wl.B}), "
                   f"{elapsed:.1f} s of fp64 numpy oracle time (expanding the latent, then attention); "
                   f"{done_bytes / 1e6:.1f} MB of latent; host fp32 copies of the inputs; {avail} cores visible"),
        "tokens_per_s_equiv": round(units / wl.B * wl.B * wl.q_len / elapsed, 3),
    }


def measure(name, args, dev, variant_opts=True, ceiling=False):
    """Generate workload `name` on `dev`, run args.warmup untimed steps, then time
    exactly args.steps back-to-back steps; then time the decode and merge kernels with
    the events their launches stamp over a second pass of the same steps. Returns the
    measurements, the inputs and the plan."""
    import numpy as np
    import torch

    from gqa_kv_cache_03_amd import (gqa_decode, gqa_decode_append, gqla_absorb_decode, gqla_absorb_decode_append,
                                     gqla_plan, plan, read_stream)
    from gqa_synth import make_inputs, make_latent_inputs, workload

    wl = workload(name)
    latent = bool(wl.d_c)   # a GQLA layer, run in its absorbed form
    use_append = args.append and variant_opts
    head_map = args.head_map and variant_opts
    active_frac = args.active_frac if variant_opts else 0.0
    if latent and (head_map or active_frac > 0 or args.policy == "valu"):
        sys.exit("the GQLA absorbed path takes no --head-map, --active-frac or valu policy")
    print(f"[bench] generating {name}", file=sys.stderr, flush=True)
    if latent:
        inp = make_latent_inputs(wl, device=dev)
        kv_bytes = inp.latent_bytes
        caches = [inp.latent]
    else:
        inp = make_inputs(wl, device=dev)
        kv_bytes = inp.kv_bytes
        caches = [inp.k_cache, inp.v_cache]
    alloc_bytes = sum(c.numel() * c.element_size() for c in caches)
    copies = args.copies or max(1, min(8, math.ceil((1 << 30) / alloc_bytes)))
    # ks[i] / vs[i]: the i-th rotated copy of the cache (the latent: ks only)
    ks = [caches[0]] + [caches[0].clone() for _ in range(copies - 1)]
    vs = [] if latent else [caches[1]] + [caches[1].clone() for _ in range(copies - 1)]
    out = torch.empty_like(inp.q)
    variant = {}
    if head_map:
        # every KV head keeps at least one query head; the rest are dealt at random with
        # at most twice the uniform group size per KV head
        rng = np.random.default_rng(wl.seed + 7)
        hpg = wl.H // wl.G
        while True:
            m = np.concatenate([np.arange(wl.G), rng.integers(0, wl.G, wl.H - wl.G)])
            rng.shuffle(m)
            if np.bincount(m, minlength=wl.G).max() <= 2 * hpg:
                break
        variant["head_group"] = torch.as_tensor(m.astype(np.int32), device=dev)
        variant["max_group_heads"] = 2 * hpg
    if active_frac > 0:
        rng = np.random.default_rng(wl.seed + 8)
        act = (rng.random((wl.B, wl.q_len, wl.H)) < active_frac).astype(np.uint8)
        variant["head_active"] = torch.as_tensor(act, device=dev)
    if latent:
        kw = dict(scale=wl.scale, causal=wl.causal, num_splits=args.num_splits, policy=args.policy)
        pl = gqla_plan(inp.q, inp.latent, inp.w_uk, inp.block_table, causal=wl.causal,
                       num_splits=args.num_splits, policy=args.policy)
    else:
        kw = dict(scale=wl.scale, causal=wl.causal, num_splits=args.num_splits, chunk_tokens=args.chunk,
                  policy=args.policy, **variant)
        pl = plan(inp.q, inp.k_cache, inp.block_table, causal=wl.causal, num_splits=args.num_splits,
                  chunk_tokens=args.chunk, policy=args.policy, **variant)
    ws = torch.empty(max(pl["workspace_bytes"], 256), dtype=torch.uint8, device=dev)

    new_bytes = 0
    if use_append and latent:
        # the new tokens' latents, as the down-projection would hand them over: [B, q_len, d_c]
        c_new = torch.empty((wl.B, wl.q_len, wl.d_c), dtype=inp.q.dtype, device=dev)
        for b in range(wl.B):
            for t in range(wl.q_len):
                pos = int(inp.lens[b]) - wl.q_len + t
                if inp.block_table is None:
                    c_new[b, t] = inp.latent[b, pos]
                else:
                    c_new[b, t] = inp.latent[int(inp.table[b, pos // wl.page_size]), pos % wl.page_size]
        new_bytes = c_new.numel() * c_new.element_size()
    elif use_append:
        # the new tokens' rows, as the projections would hand them over: [B, q_len, G, d_h]
        k_new = torch.empty((wl.B, wl.q_len, wl.G, wl.d_h), dtype=inp.q.dtype, device=dev)
        v_new = torch.empty_like(k_new)
        for b in range(wl.B):
            for t in range(wl.q_len):
                pos = int(inp.lens[b]) - wl.q_len + t
                if inp.block_table is None:
                    k_new[b, t], v_new[b, t] = inp.k_cache[b, :, pos], inp.v_cache[b, :, pos]
                else:
                    pg, sl = int(inp.table[b, pos // wl.page_size]), pos % wl.page_size
                    k_new[b, t], v_new[b, t] = inp.k_cache[pg, :, sl], inp.v_cache[pg, :, sl]
        new_bytes = 2 * k_new.numel() * k_new.element_size()

    def step(i, events=None):
        if latent and use_append:
            gqla_absorb_decode_append(inp.q, c_new, ks[i % copies], inp.w_uk, inp.w_uv, inp.seq_lens,
                                      inp.block_table, out=out, workspace=ws, profile_events=events, **kw)
        elif latent:
            gqla_absorb_decode(inp.q, ks[i % copies], inp.w_uk, inp.w_uv, inp.seq_lens, inp.block_table,
                               out=out, workspace=ws, profile_events=events, **kw)
        elif use_append:
            gqa_decode_append(inp.q, k_new, v_new, ks[i % copies], vs[i % copies], inp.seq_lens,
                              inp.block_table, out=out, workspace=ws, profile_events=events, **kw)
        else:
            gqa_decode(inp.q, ks[i % copies], vs[i % copies], inp.seq_lens, inp.block_table, out=out,
                       workspace=ws, profile_events=events, **kw)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region: K back-to-back steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    e0.record()
    for i in range(args.steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms = e0.elapsed_time(e1) / args.steps
    print(f"[bench] {name}: {args.steps} steps, {ms * 1e3:.1f} us/step (wall {wall * 1e6 / args.steps:.1f} us)",
          file=sys.stderr, flush=True)

    # per-kernel durations: the library's launches stamp these events with each kernel's own
    # begin and end times, so they time the kernels alone, as a kernel trace does
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for trio in evs:
        for ev in trio:
            ev.record()
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(i, events=[int(ev.cuda_event) for ev in evs[i]])
    torch.cuda.synchronize()
    dec = [evs[i][0].elapsed_time(evs[i][1]) for i in range(args.steps)]
    mrg = [evs[i][1].elapsed_time(evs[i][2]) for i in range(args.steps)]
    dec_ms = statistics.mean(dec)
    mrg_ms = statistics.mean(mrg)

    # the queries the decode kernel reads (the latent path: the absorbed, d_c-wide ones)
    q_bytes = inp.q.numel() * inp.q.element_size() * (wl.d_c // wl.d_h if latent else 1)
    tbl_bytes = 0 if inp.table is None else 4 * int(sum(-(-int(L) // wl.page_size) for L in inp.lens))
    # with the append, the new rows are read from k_new/v_new instead of the cache (same
    # count) and written to the cache once
    dec_alg_bytes = kv_bytes + q_bytes + tbl_bytes + new_bytes
    achieved = dec_alg_bytes / (dec_ms * 1e-3) / 1e9

    ceilings = {}
    if ceiling:
        # streaming-read ceiling over the same cache copies: wide register loads, and the
        # decode kernel's own direct-to-LDS pattern without its compute; the best counts
        buf = ks[0].view(torch.uint8).reshape(-1)
        if buf.numel() < (1 << 30) and len(ks) > 1:
            buf = torch.cat([k.view(torch.uint8).reshape(-1) for k in ks])
        nbytes = buf.numel() // 16 * 16
        sink = torch.empty(8192, dtype=torch.int32, device=dev)
        # the direct-to-LDS method in the decode kernel's own step: a K + V tile, or a
        # tile of the 512-wide latent
        step_bytes = 32768 if latent else 16384
        for label, fn in (("register_loads", lambda: read_stream(buf[:nbytes], sink)),
                          ("lds_double_buffer", lambda: read_stream(buf[:nbytes], step_bytes=step_bytes))):
            fn()
            torch.cuda.synchronize()
            c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            # one launch ahead of the first event keeps the device busy while the host
            # queues the rest, so the host's launch latency stays out of the timing
            fn()
            c0.record()
            for _ in range(10):
                fn()
            c1.record()
            torch.cuda.synchronize()
            ceilings[label] = round(nbytes / (c0.elapsed_time(c1) / 10 * 1e-3) / 1e9, 1)
        del buf

    # useful matrix work of the decode kernel: QK^T and PV, 2 * 2 * d_h flop per
    # (query row, visible key) -- counted over all L keys (the causal triangle among
    # the q_len new tokens is a negligible correction)
    width = wl.d_c if latent else wl.d_h   # the attention's head width (the latent's for GQLA)
    flops = 4 * wl.H * wl.q_len * width * int(sum(int(L) for L in inp.lens))
    tflops = flops / (dec_ms * 1e-3) / 1e12
    intensity = flops / dec_alg_bytes
    ridge = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9)
    mfma_bound = pl["policy"] == "mfma" and intensity > ridge
    del ks, vs, ws, out
    return dict(wl=wl, inp=inp, pl=pl, latent=latent, variant=variant, copies=copies, ms=ms, wall=wall,
                dec=dec, dec_ms=dec_ms, mrg_ms=mrg_ms, kv_bytes=kv_bytes, dec_alg_bytes=dec_alg_bytes,
                achieved=achieved, flops=flops, tflops=tflops, intensity=intensity, mfma_bound=mfma_bound,
                ceilings=ceilings)


def decode_kernel_name(pl) -> str:
    """The decode kernel a plan launches: the matrix-core kernel (its re-reading form
    when the group's rows are split into row blocks) or the vector-ALU kernel."""
    if pl["policy"] != "mfma":
        return "decode_valu_kernel"
    return "decode_mfma_reread_kernel" if pl["row_blocks"] > 1 else "decode_mfma_kernel"


def roofline_of(m, traffic_key):
    """The dominant (decode) kernel against the roofline that bounds it."""
    mb = m["mfma_bound"]
    return {
        "bound": "mfma" if mb else "hbm",
        "achieved": round(m["tflops"], 2) if mb else round(m["achieved"], 2),
        "peak": MFMA_BF16_PEAK_TFLOPS if mb else HBM_PEAK_GBPS,
        "unit": "TFLOP/s" if mb else "GB/s",
        "frac": round(m["tflops"] / MFMA_BF16_PEAK_TFLOPS if mb else m["achieved"] / HBM_PEAK_GBPS, 4),
        "traffic": load_traffic(traffic_key) if not m["variant"] else None,
        "kernel": decode_kernel_name(m["pl"]),
        "algorithmic_bytes_per_launch": int(m["dec_alg_bytes"]),
        "flops_per_launch": int(m["flops"]),
        "flop_per_byte": round(m["intensity"], 2),
        "hbm_gbps": round(m["achieved"], 2),
    }


def per_config_entry(line: dict) -> dict:
    """One long-context configuration's entry in the default run, from the JSON line that
    `bench.py --workload NAME` printed for it."""
    r = line["roofline"]
    return {
        "step_us": round(line["ms_per_step"] * 1e3, 2),
        "kv_gbps": round(line["value"], 1),
        "pct_of_hbm_peak": line["pct_of_hbm_peak"],
        "tokens_per_s": line["tokens_per_s"],
        "decode_us": round(line["kernel_ms"]["split_decode"] * 1e3, 2),
        "merge_us": round(line["kernel_ms"]["lse_merge"] * 1e3, 2),
        "decode_roofline_frac": r["frac"],
        "roofline_bound": r["bound"],
        "traffic": r["traffic"],
    }


def measure_in_child(name: str, warmup: int, steps: int) -> dict:
    """`bench.py --workload NAME` in a process of its own (the parent waits for it), so that
    every configuration starts from a fresh device context and allocator, as a
    stand-alone run of it does; returns the child's JSON line."""
    import subprocess
    cmd = [sys.executable, os.path.abspath(__file__), "--workload", name, "--warmup", str(warmup),
           "--steps", str(steps), "--no-cpu-baseline", "--no-ceiling"]
    print(f"[bench] per-config: {name}", file=sys.stderr, flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=sys.stderr, text=True, timeout=600)
    if r.returncode != 0:
        raise RuntimeError(f"per-config run of {name} failed with status {r.returncode}")
    lines = [x for x in r.stdout.strip().splitlines() if x.startswith("{")]
    return json.loads(lines[-1])


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the decode step has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy_mib:
        calibrate_copy(args.calibrate_copy_mib)
        return
    import numpy as np
    import torch

    from gqa_synth import BENCH_DEFAULT, BENCH_PER_CONFIG

    name = args.workload or BENCH_DEFAULT
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    m = measure(name, args, dev, ceiling=not args.no_ceiling)
    wl, inp, pl = m["wl"], m["inp"], m["pl"]
    latent = m["latent"]
    ms = m["ms"]
    value = m["kv_bytes"] / (ms * 1e-3) / 1e9
    ceiling = max(m["ceilings"].values()) if m["ceilings"] else None
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bfloat16" else "f32",
        "data": ("synthetic (seeded N(0,1) q and latent, N(0,1/d_c) up-projections, seeded lengths and "
                 "block tables)" if latent else "synthetic (seeded N(0,1) q/K/V, seeded lengths and block tables)"),
        "config": {
            "workload": name + (" +append" if args.append else "") + (" +head_map" if args.head_map else "")
            + (f" +active{args.active_frac:g}" if args.active_frac > 0 else ""),
            "B": wl.B, "H": wl.H, "G": wl.G, "d_h": wl.d_h, "q_len": wl.q_len, "d_c": wl.d_c or None,
            "layout": wl.layout, "page_size": wl.page_size or None,
            "lengths": [wl.len_lo, wl.len_hi], "sum_seq_lens": int(inp.lens.sum()),
            "kv_bytes": int(m["kv_bytes"]), "kv_copies_rotated": m["copies"], "plan": pl,
        },
        "tokens_per_s": round(wl.B * wl.q_len / (ms * 1e-3), 1),
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "read_ceiling_gbps": None if ceiling is None else round(ceiling, 1),
        "read_ceiling_by_method": m["ceilings"] or None,
        "kernel_ms": {"split_decode": round(m["dec_ms"], 6), "lse_merge": round(m["mrg_ms"], 6)},
        # spread of the event-timed decode kernel over the K steps
        "decode_ms_p10_p50_p90": [round(float(x), 6) for x in np.percentile(m["dec"], [10, 50, 90])],
        "roofline": roofline_of(m, name + ("_append" if args.append else "")),
        "mfma_util": None if pl["policy"] != "mfma" else round(m["tflops"] / MFMA_BF16_PEAK_TFLOPS, 4),
        "cpu_baseline": None,
        "per_config": None,
        "wall_ms_per_step": round(m["wall"] * 1e3 / args.steps, 6),
    }
    del m
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline_latent(inp, args.cpu_budget) if latent else cpu_baseline(inp, args.cpu_budget)
    del inp
    torch.cuda.empty_cache()
    if args.workload is None and not args.no_per_config:
        # the default run also measures every other long-context configuration with plain
        # calls (no append or grouping variant), each in a child process of its own
        # (at least 50 warm-up and 100 timed steps each, so that short runs still report
        # settled clocks for these shorter steps)
        res["per_config"] = {}
        warm, steps = max(args.warmup, 50), max(args.steps, 100)
        res["per_config_protocol"] = {"warmup": warm, "steps": steps, "process": "one child process per configuration"}
        for other in BENCH_PER_CONFIG:
            res["per_config"][other] = per_config_entry(measure_in_child(other, warm, steps))
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
