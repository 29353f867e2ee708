"""ctypes view of libgqa_decode.so (the C ABI declared in include/gqa_decode.h).

Argument marshalling only. Loading fails loudly if the library was not built: there
is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgqa_decode.so")

GQA_OK = 0
GQA_ERR_INVALID_ARGUMENT = 1
GQA_ERR_UNSUPPORTED = 2
GQA_ERR_WORKSPACE = 3
GQA_ERR_HIP = 4
GQA_ERR_SCRATCH = 5

# fixed per-device scratch behind gqa_decode_noalloc (GQA_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 65 << 20

GQA_DTYPE_F32 = 0
GQA_DTYPE_BF16 = 1

GQA_POLICY_AUTO = 0
GQA_POLICY_VALU = 1
GQA_POLICY_MFMA = 2

# Every symbol the public headers declare.
EXPORTED = (
    "gqa_decode_opts_init",
    "gqa_decode",
    "gqa_decode_append",
    "gqa_decode_noalloc",
    "gqa_decode_check_inputs",
    "gqa_decode_plan",
    "gqa_decode_workspace_size",
    "gqa_status_string",
    "gqa_abi_version",
    "gqa_bench_read_stream",
    "gqa_bench_read_stream_lds",
    "gqla_absorb_decode",
    "gqla_absorb_decode_append",
    "gqla_absorb_plan",
    "gqla_absorb_workspace_size",
)


class DecodeOpts(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("dtype", ctypes.c_int32),
        ("causal", ctypes.c_int32),
        ("cache_capacity", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("num_splits", ctypes.c_int32),
        ("chunk_tokens", ctypes.c_int32),
        ("policy", ctypes.c_int32),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("profile_events", ctypes.c_void_p * 3),
        ("head_group", ctypes.c_void_p),
        ("max_group_heads", ctypes.c_int32),
        ("reserved0", ctypes.c_int32),
        ("head_active", ctypes.c_void_p),
    ]


class Plan(ctypes.Structure):
    _fields_ = [
        ("policy", ctypes.c_int32),
        ("schedule", ctypes.c_int32),
        ("rows", ctypes.c_int32),
        ("row_blocks", ctypes.c_int32),
        ("tile_tokens", ctypes.c_int32),
        ("chunk_tokens", ctypes.c_int32),
        ("max_splits", ctypes.c_int32),
        ("workgroups", ctypes.c_int32),
        ("capacity", ctypes.c_int32),
        ("grid", ctypes.c_int32 * 3),
        ("block_threads", ctypes.c_int32),
        ("lds_bytes", ctypes.c_int32),
        ("workspace_bytes", ctypes.c_size_t),
    ]

    def as_dict(self) -> dict:
        return {
            "policy": {1: "valu", 2: "mfma"}.get(self.policy, str(self.policy)),
            "schedule": {0: "split-k grid", 1: "persistent balanced"}.get(self.schedule, str(self.schedule)),
            "rows": self.rows,
            "row_blocks": self.row_blocks,
            "tile_tokens": self.tile_tokens,
            "chunk_tokens": self.chunk_tokens,
            "max_splits": self.max_splits,
            "workgroups": self.workgroups,
            "capacity": self.capacity,
            "grid": list(self.grid),
            "block_threads": self.block_threads,
            "lds_bytes": self.lds_bytes,
            "workspace_bytes": self.workspace_bytes,
        }


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m gqa_kv_cache_03_amd.build` "
            "(or __graft_entry__.build()); there is no fallback implementation")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    L.gqa_decode_opts_init.argtypes = [ctypes.POINTER(DecodeOpts)]
    L.gqa_decode_opts_init.restype = None
    L.gqa_decode.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, ctypes.c_float,
                             vp, ctypes.POINTER(DecodeOpts)]
    L.gqa_decode.restype = i32
    L.gqa_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, ctypes.c_float,
                                     vp, ctypes.POINTER(DecodeOpts)]
    L.gqa_decode_noalloc.restype = i32
    L.gqa_decode_append.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, ctypes.c_float,
                                    vp, ctypes.POINTER(DecodeOpts)]
    L.gqa_decode_append.restype = i32
    L.gqa_decode_check_inputs.argtypes = [vp, vp, i32, i32, vp, ctypes.POINTER(DecodeOpts), vp]
    L.gqa_decode_check_inputs.restype = i32
    L.gqa_decode_plan.argtypes = [i32, i32, i32, i32, i32, ctypes.POINTER(DecodeOpts), ctypes.POINTER(Plan)]
    L.gqa_decode_plan.restype = i32
    L.gqa_decode_workspace_size.argtypes = [i32, i32, i32, i32, i32, ctypes.POINTER(DecodeOpts),
                                            ctypes.POINTER(sz)]
    L.gqa_decode_workspace_size.restype = i32
    L.gqa_status_string.argtypes = [i32]
    L.gqa_status_string.restype = ctypes.c_char_p
    L.gqa_abi_version.argtypes = []
    L.gqa_abi_version.restype = i32
    L.gqa_bench_read_stream.argtypes = [vp, sz, vp, vp]
    L.gqa_bench_read_stream.restype = i32
    L.gqa_bench_read_stream_lds.argtypes = [vp, sz, i32, i32, vp]
    L.gqa_bench_read_stream_lds.restype = i32
    L.gqla_absorb_decode.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, ctypes.c_float,
                                     vp, ctypes.POINTER(DecodeOpts)]
    L.gqla_absorb_decode.restype = i32
    L.gqla_absorb_decode_append.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                            ctypes.c_float, vp, ctypes.POINTER(DecodeOpts)]
    L.gqla_absorb_decode_append.restype = i32
    L.gqla_absorb_plan.argtypes = [i32, i32, i32, i32, i32, i32, ctypes.POINTER(DecodeOpts), ctypes.POINTER(Plan)]
    L.gqla_absorb_plan.restype = i32
    L.gqla_absorb_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, ctypes.POINTER(DecodeOpts),
                                             ctypes.POINTER(sz)]
    L.gqla_absorb_workspace_size.restype = i32
    _lib = L
    return L


def default_opts() -> DecodeOpts:
    o = DecodeOpts()
    lib().gqa_decode_opts_init(ctypes.byref(o))
    return o


def status_string(st: int) -> str:
    return lib().gqa_status_string(st).decode()


class GqaError(RuntimeError):
    def __init__(self, status: int, what: str = "gqa_decode"):
        self.status = status
        super().__init__(f"{what} failed: status {status} ({status_string(status)})")
