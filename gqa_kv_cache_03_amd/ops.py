"""Python binding of the decode library: torch tensors in, the C ABI call, status out.

torch supplies device memory and the current stream only; every step of the decode
runs in the library's HIP kernels.
"""
from __future__ import annotations

import ctypes
import math
from typing import Optional

from . import _lib
from ._lib import DecodeOpts, GqaError, Plan

_POLICIES = {"auto": _lib.GQA_POLICY_AUTO, "valu": _lib.GQA_POLICY_VALU, "mfma": _lib.GQA_POLICY_MFMA}


def _dtype_code(torch, dt) -> int:
    if dt == torch.float32:
        return _lib.GQA_DTYPE_F32
    if dt == torch.bfloat16:
        return _lib.GQA_DTYPE_BF16
    raise TypeError(f"unsupported dtype {dt}; float32 or bfloat16")


def make_opts(*, dtype_code: int, causal: bool, capacity: int, page_size: int = 0,
              max_blocks: int = 0, num_pages: int = 0, num_splits: int = 0,
              chunk_tokens: int = 0, policy: str = "auto", head_group=None, max_group_heads: int = 0,
              head_active=None) -> DecodeOpts:
    o = _lib.default_opts()
    o.dtype = dtype_code
    o.causal = 1 if causal else 0
    o.cache_capacity = capacity
    o.page_size = page_size
    o.max_blocks_per_seq = max_blocks
    o.num_pages = num_pages
    o.num_splits = num_splits
    o.chunk_tokens = chunk_tokens
    o.policy = _POLICIES[policy]
    o.head_group = None if head_group is None else head_group.data_ptr()
    o.max_group_heads = max_group_heads
    o.head_active = None if head_active is None else head_active.data_ptr()
    return o


def _geometry(q, k_cache, block_table):
    B, q_len, H, d = q.shape
    if block_table is None:
        if k_cache.dim() != 4 or k_cache.shape[0] != B or k_cache.shape[3] != d:
            raise ValueError("contiguous cache must be [B, G, capacity, d_h]")
        G, cap = k_cache.shape[1], k_cache.shape[2]
        return B, q_len, H, d, G, dict(capacity=cap)
    if k_cache.dim() != 4 or k_cache.shape[3] != d:
        raise ValueError("paged pool must be [num_pages, G, page_size, d_h]")
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B, max_blocks_per_seq]")
    num_pages, G, P = k_cache.shape[0], k_cache.shape[1], k_cache.shape[2]
    return B, q_len, H, d, G, dict(capacity=0, page_size=P, max_blocks=block_table.shape[1],
                                   num_pages=num_pages)


def plan(q, k_cache, block_table=None, *, causal=True, num_splits=0, chunk_tokens=0,
         policy="auto", head_group=None, max_group_heads: int = 0, head_active=None) -> dict:
    """What gqa_decode would launch for these tensors (no device work)."""
    import torch
    B, q_len, H, d, G, geo = _geometry(q, k_cache, block_table)
    o = make_opts(dtype_code=_dtype_code(torch, q.dtype), causal=causal, num_splits=num_splits,
                  chunk_tokens=chunk_tokens, policy=policy, head_group=head_group,
                  max_group_heads=max_group_heads, head_active=head_active, **geo)
    pl = Plan()
    st = _lib.lib().gqa_decode_plan(B, H, G, d, q_len, ctypes.byref(o), ctypes.byref(pl))
    if st != _lib.GQA_OK:
        raise GqaError(st, "gqa_decode_plan")
    return pl.as_dict()


def check_inputs(seq_lens, block_table=None, *, q_len: int, capacity: int = 0, page_size: int = 0,
                 num_pages: int = 0) -> dict:
    """Device-side check of a decode call's device-resident preconditions
    (gqa_decode_check_inputs): every length in [q_len, capacity] and every block-table
    entry the step reads in [0, num_pages). Contiguous caches give `capacity`; paged ones
    `page_size` and `num_pages` (the table gives max_blocks_per_seq). Waits for the result
    on the current stream and returns the counts and the first offenders (None if none)."""
    import torch
    B = seq_lens.shape[0]
    o = make_opts(dtype_code=_lib.GQA_DTYPE_BF16, causal=True, capacity=capacity if block_table is None else 0,
                  page_size=page_size if block_table is not None else 0,
                  max_blocks=block_table.shape[1] if block_table is not None else 0, num_pages=num_pages)
    report = torch.empty(4, dtype=torch.int32, device=seq_lens.device)
    st = _lib.lib().gqa_decode_check_inputs(
        seq_lens.data_ptr(), None if block_table is None else block_table.data_ptr(), B, q_len,
        torch.cuda.current_stream(seq_lens.device).cuda_stream, ctypes.byref(o), report.data_ptr())
    if st != _lib.GQA_OK:
        raise GqaError(st, "gqa_decode_check_inputs")
    r = [int(x) for x in report.cpu()]
    none = 2 ** 31 - 1
    return {"bad_lengths": r[0], "bad_entries": r[1], "first_bad_sequence": None if r[2] == none else r[2],
            "first_bad_entry": None if r[3] == none else r[3]}


def gqa_decode(q, k_cache, v_cache, seq_lens, block_table=None, *, scale: Optional[float] = None,
               out=None, causal: bool = True, num_splits: int = 0, chunk_tokens: int = 0,
               policy: str = "auto", workspace=None, profile_events=None, head_group=None,
               max_group_heads: int = 0, head_active=None):
    """One GQA decode step on the current HIP stream; returns `out`.

    q [B, q_len, H, d_h]; k_cache/v_cache [B, G, cap, d_h] (contiguous) or
    [num_pages, G, page_size, d_h] with block_table int32 [B, max_blocks];
    seq_lens int32 [B] counting the q_len new tokens. scale defaults to 1/sqrt(d_h).
    num_splits: MFMA policy -- persistent workgroups (0: what the device holds);
    VALU policy -- maximum context splits per sequence (0: heuristic).
    head_group: int32 [H] device tensor, the KV head of each query head (non-uniform
    groups; max_group_heads bounds any group's size, 0 = H). head_active: uint8
    [B, q_len, H] device tensor, 0 = that (token, head) is inactive and outputs 0.
    """
    return _call(q, None, None, k_cache, v_cache, seq_lens, block_table, scale=scale, out=out,
                 causal=causal, num_splits=num_splits, chunk_tokens=chunk_tokens, policy=policy,
                 workspace=workspace, profile_events=profile_events, head_group=head_group,
                 max_group_heads=max_group_heads, head_active=head_active)


def gqa_decode_noalloc(q, k_cache, v_cache, seq_lens, block_table=None, *, scale: Optional[float] = None,
                       out=None, causal: bool = True, num_splits: int = 0, chunk_tokens: int = 0,
                       policy: str = "auto", profile_events=None, head_group=None,
                       max_group_heads: int = 0, head_active=None):
    """gqa_decode through the no-allocation entry point: the split partials go to the
    library's fixed per-device scratch array, not to a workspace. `out` must be given
    by a caller that may not allocate (it is allocated here only when None). Calls
    that overlap on one GPU race on the scratch."""
    return _call(q, None, None, k_cache, v_cache, seq_lens, block_table, scale=scale, out=out,
                 causal=causal, num_splits=num_splits, chunk_tokens=chunk_tokens, policy=policy,
                 workspace=None, profile_events=profile_events, head_group=head_group,
                 max_group_heads=max_group_heads, head_active=head_active, noalloc=True)


def gqa_decode_append(q, k_new, v_new, k_cache, v_cache, seq_lens, block_table=None, *,
                      scale: Optional[float] = None, out=None, causal: bool = True, num_splits: int = 0,
                      chunk_tokens: int = 0, policy: str = "auto", workspace=None, profile_events=None,
                      head_group=None, max_group_heads: int = 0, head_active=None):
    """gqa_decode fused with writing the new tokens' K/V into the cache.

    k_new/v_new [B, q_len, G, d_h]: row t of sequence b is written at cache position
    seq_lens[b] - q_len + t (paged: through block_table, pages already allocated);
    the step then attends over the updated cache. Returns `out`.
    """
    return _call(q, k_new, v_new, k_cache, v_cache, seq_lens, block_table, scale=scale, out=out,
                 causal=causal, num_splits=num_splits, chunk_tokens=chunk_tokens, policy=policy,
                 workspace=workspace, profile_events=profile_events, head_group=head_group,
                 max_group_heads=max_group_heads, head_active=head_active)


def _call(q, k_new, v_new, k_cache, v_cache, seq_lens, block_table, *, scale, out, causal, num_splits,
          chunk_tokens, policy, workspace, profile_events, head_group=None, max_group_heads=0,
          head_active=None, noalloc=False):
    import torch
    tensors = [("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("seq_lens", seq_lens)]
    if k_new is not None or v_new is not None:
        tensors += [("k_new", k_new), ("v_new", v_new)]
    for name, t in tensors:
        if t is None:
            raise ValueError(f"{name} is required")
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise TypeError("q, k_cache and v_cache must share one dtype")
    if v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache must have the same shape")
    if seq_lens.dtype != torch.int32:
        raise TypeError("seq_lens must be int32")
    if block_table is not None and (block_table.dtype != torch.int32 or not block_table.is_contiguous()
                                    or not block_table.is_cuda):
        raise TypeError("block_table must be a contiguous int32 device tensor")
    B, q_len, H, d, G, geo = _geometry(q, k_cache, block_table)
    if seq_lens.numel() != B:
        raise ValueError("seq_lens must have B entries")
    if k_new is not None:
        for name, t in (("k_new", k_new), ("v_new", v_new)):
            if tuple(t.shape) != (B, q_len, G, d) or t.dtype != q.dtype:
                raise ValueError(f"{name} must be [B, q_len, G, d_h] = {(B, q_len, G, d)} in q's dtype")
    if head_group is not None and (head_group.dtype != torch.int32 or tuple(head_group.shape) != (H,)
                                   or not head_group.is_cuda or not head_group.is_contiguous()):
        raise ValueError("head_group must be a contiguous int32 device tensor of H entries")
    if head_active is not None and (head_active.dtype != torch.uint8 or not head_active.is_cuda
                                    or tuple(head_active.shape) != (B, q_len, H)
                                    or not head_active.is_contiguous()):
        raise ValueError("head_active must be a contiguous uint8 device tensor [B, q_len, H]")
    code = _dtype_code(torch, q.dtype)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = make_opts(dtype_code=code, causal=causal, num_splits=num_splits, chunk_tokens=chunk_tokens,
                  policy=policy, head_group=head_group, max_group_heads=max_group_heads,
                  head_active=head_active, **geo)
    L = _lib.lib()
    need = ctypes.c_size_t(0)
    if not noalloc:
        st = L.gqa_decode_workspace_size(B, H, G, d, q_len, ctypes.byref(o), ctypes.byref(need))
        if st != _lib.GQA_OK:
            raise GqaError(st, "gqa_decode_workspace_size")
    if need.value:
        if workspace is None or workspace.numel() * workspace.element_size() < need.value:
            workspace = torch.empty(need.value, dtype=torch.uint8, device=q.device)
        o.workspace = workspace.data_ptr()
        o.workspace_bytes = workspace.numel() * workspace.element_size()
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor shaped and typed like q")
    if profile_events is not None:
        for i, ev in enumerate(profile_events):
            o.profile_events[i] = ev
    stream = torch.cuda.current_stream(q.device).cuda_stream
    bt = None if block_table is None else block_table.data_ptr()
    if noalloc:
        st = L.gqa_decode_noalloc(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), seq_lens.data_ptr(),
                                  bt, out.data_ptr(), B, H, G, d, q_len, ctypes.c_float(scale), stream,
                                  ctypes.byref(o))
        if st != _lib.GQA_OK:
            raise GqaError(st, "gqa_decode_noalloc")
        return out
    if k_new is None:
        st = L.gqa_decode(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), seq_lens.data_ptr(), bt,
                          out.data_ptr(), B, H, G, d, q_len, ctypes.c_float(scale), stream, ctypes.byref(o))
    else:
        st = L.gqa_decode_append(q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), k_cache.data_ptr(),
                                 v_cache.data_ptr(), seq_lens.data_ptr(), bt, out.data_ptr(), B, H, G, d,
                                 q_len, ctypes.c_float(scale), stream, ctypes.byref(o))
    if st != _lib.GQA_OK:
        raise GqaError(st, "gqa_decode" if k_new is None else "gqa_decode_append")
    return out


def workspace_bytes(q, k_cache, block_table=None, **kw) -> int:
    return plan(q, k_cache, block_table, **kw)["workspace_bytes"]


def read_stream(buf, sink=None, workgroups: int = 0, step_bytes: int = 16384) -> None:
    """Measurement helper: stream-read `buf` (a device tensor) once.

    With `sink` (int32 device tensor of >= 8192 entries): wide nontemporal loads into
    registers. Without: the decode kernel's pattern, `workgroups` persistent workgroups
    (0: two per CU) reading through direct-to-LDS double-buffered steps of `step_bytes`
    (16384 or 32768).
    """
    import torch
    L = _lib.lib()
    stream = torch.cuda.current_stream(buf.device).cuda_stream
    nbytes = buf.numel() * buf.element_size()
    if sink is not None:
        st = L.gqa_bench_read_stream(buf.data_ptr(), nbytes, sink.data_ptr(), stream)
    else:
        if workgroups <= 0:
            workgroups = 2 * torch.cuda.get_device_properties(buf.device).multi_processor_count
        st = L.gqa_bench_read_stream_lds(buf.data_ptr(), nbytes, workgroups, step_bytes, stream)
    if st != _lib.GQA_OK:
        raise GqaError(st, "gqa_bench_read_stream")


def _latent_geometry(q, latent_cache, w_uk, block_table):
    B, q_len, H, d_h = q.shape
    if w_uk.dim() != 3 or w_uk.shape[1] != d_h:
        raise ValueError("w_uk must be [G, d_h, d_c]")
    G, d_c = w_uk.shape[0], w_uk.shape[2]
    if block_table is None:
        if latent_cache.dim() != 3 or latent_cache.shape[0] != B or latent_cache.shape[2] != d_c:
            raise ValueError("contiguous latent cache must be [B, capacity, d_c]")
        return B, q_len, H, d_h, G, d_c, dict(capacity=latent_cache.shape[1])
    if latent_cache.dim() != 3 or latent_cache.shape[2] != d_c:
        raise ValueError("paged latent pool must be [num_pages, page_size, d_c]")
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B, max_blocks_per_seq]")
    return B, q_len, H, d_h, G, d_c, dict(capacity=0, page_size=latent_cache.shape[1],
                                          max_blocks=block_table.shape[1], num_pages=latent_cache.shape[0])


def gqla_plan(q, latent_cache, w_uk, block_table=None, *, causal=True, num_splits=0, policy="auto") -> dict:
    """What gqla_absorb_decode would launch for these tensors (no device work)."""
    import torch
    B, q_len, H, d_h, G, d_c, geo = _latent_geometry(q, latent_cache, w_uk, block_table)
    o = make_opts(dtype_code=_dtype_code(torch, q.dtype), causal=causal, num_splits=num_splits, policy=policy,
                  **geo)
    pl = Plan()
    st = _lib.lib().gqla_absorb_plan(B, H, G, d_h, d_c, q_len, ctypes.byref(o), ctypes.byref(pl))
    if st != _lib.GQA_OK:
        raise GqaError(st, "gqla_absorb_plan")
    return pl.as_dict()


def gqla_absorb_decode(q, latent_cache, w_uk, w_uv, seq_lens, block_table=None, *,
                       scale: Optional[float] = None, out=None, causal: bool = True, num_splits: int = 0,
                       policy: str = "auto", workspace=None, profile_events=None):
    """One decode step of a GQLA layer in its absorbed (MQA) form.

    q [B, q_len, H, d_h] bf16; latent_cache [B, capacity, d_c] (or a paged pool
    [num_pages, page_size, d_c] with block_table [B, max_blocks]); w_uk, w_uv
    [G, d_h, d_c]; seq_lens int32 [B]. Returns out [B, q_len, H, d_h]: attention of
    each head over its group's expanded cache W c_j, computed against the latent.
    """
    return _latent_call(q, None, latent_cache, w_uk, w_uv, seq_lens, block_table, scale=scale, out=out,
                        causal=causal, num_splits=num_splits, policy=policy, workspace=workspace,
                        profile_events=profile_events)


def gqla_absorb_decode_append(q, c_new, latent_cache, w_uk, w_uv, seq_lens, block_table=None, *,
                              scale: Optional[float] = None, out=None, causal: bool = True, num_splits: int = 0,
                              policy: str = "auto", workspace=None, profile_events=None):
    """gqla_absorb_decode fused with writing the new tokens' latents c_new [B, q_len, d_c]
    into latent_cache at positions seq_lens[b] - q_len + t (the cache is modified)."""
    return _latent_call(q, c_new, latent_cache, w_uk, w_uv, seq_lens, block_table, scale=scale, out=out,
                        causal=causal, num_splits=num_splits, policy=policy, workspace=workspace,
                        profile_events=profile_events)


def _latent_call(q, c_new, latent_cache, w_uk, w_uv, seq_lens, block_table, *, scale, out, causal, num_splits,
                 policy, workspace, profile_events):
    import torch
    tensors = [("q", q), ("latent_cache", latent_cache), ("w_uk", w_uk), ("w_uv", w_uv), ("seq_lens", seq_lens)]
    if c_new is not None:
        tensors.append(("c_new", c_new))
    for name, t in tensors:
        if t is None:
            raise ValueError(f"{name} is required")
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    for name, t in tensors[1:4] + tensors[5:]:
        if t.dtype != q.dtype:
            raise TypeError(f"{name} must have q's dtype")
    if w_uv.shape != w_uk.shape:
        raise ValueError("w_uk and w_uv must have the same shape")
    if seq_lens.dtype != torch.int32:
        raise TypeError("seq_lens must be int32")
    if block_table is not None and (block_table.dtype != torch.int32 or not block_table.is_contiguous()
                                    or not block_table.is_cuda):
        raise TypeError("block_table must be a contiguous int32 device tensor")
    B, q_len, H, d_h, G, d_c, geo = _latent_geometry(q, latent_cache, w_uk, block_table)
    if seq_lens.numel() != B:
        raise ValueError("seq_lens must have B entries")
    if c_new is not None and tuple(c_new.shape) != (B, q_len, d_c):
        raise ValueError("c_new must be [B, q_len, d_c]")
    if scale is None:
        scale = 1.0 / math.sqrt(d_h)
    o = make_opts(dtype_code=_dtype_code(torch, q.dtype), causal=causal, num_splits=num_splits, policy=policy,
                  **geo)
    L = _lib.lib()
    need = ctypes.c_size_t(0)
    st = L.gqla_absorb_workspace_size(B, H, G, d_h, d_c, q_len, ctypes.byref(o), ctypes.byref(need))
    if st != _lib.GQA_OK:
        raise GqaError(st, "gqla_absorb_workspace_size")
    if workspace is None or workspace.numel() * workspace.element_size() < need.value:
        workspace = torch.empty(need.value, dtype=torch.uint8, device=q.device)
    o.workspace = workspace.data_ptr()
    o.workspace_bytes = workspace.numel() * workspace.element_size()
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor shaped and typed like q")
    if profile_events is not None:
        for i, ev in enumerate(profile_events):
            o.profile_events[i] = ev
    stream = torch.cuda.current_stream(q.device).cuda_stream
    bt = None if block_table is None else block_table.data_ptr()
    if c_new is None:
        st = L.gqla_absorb_decode(q.data_ptr(), latent_cache.data_ptr(), w_uk.data_ptr(), w_uv.data_ptr(),
                                  seq_lens.data_ptr(), bt, out.data_ptr(), B, H, G, d_h, d_c, q_len,
                                  ctypes.c_float(scale), stream, ctypes.byref(o))
        what = "gqla_absorb_decode"
    else:
        st = L.gqla_absorb_decode_append(q.data_ptr(), c_new.data_ptr(), w_uk.data_ptr(), w_uv.data_ptr(),
                                         latent_cache.data_ptr(), seq_lens.data_ptr(), bt, out.data_ptr(), B, H,
                                         G, d_h, d_c, q_len, ctypes.c_float(scale), stream, ctypes.byref(o))
        what = "gqla_absorb_decode_append"
    if st != _lib.GQA_OK:
        raise GqaError(st, what)
    return out
