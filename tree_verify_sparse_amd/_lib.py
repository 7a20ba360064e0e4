"""ctypes view of libsv.so (the C ABI declared in include/sv.h)."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsv.so")

SV_OK, SV_E_INVALID, SV_E_UNSUPPORTED, SV_E_WORKSPACE, SV_E_HIP = range(5)
SV_F32, SV_BF16 = 0, 1

# every symbol include/sv.h declares
EXPORTS = (
    "sv_abi_version", "sv_last_error",
    "sv_verify_workspace_size", "sv_verify_attn",
    "sv_topk_workspace_size", "sv_topk_select",
    "sv_sparse_workspace_size", "sv_sparse_draft_attn",
    "sv_verify_attn_per_head", "sv_sparse_draft_attn_per_head", "sv_select_sink_window",
    "sv_compact_kv", "sv_dense_draft_workspace_size", "sv_dense_draft_attn", "sv_build_tree",
    "sv_accept_commit",
    "sv_validate_kv", "sv_validate_tree", "sv_validate_index",
    "sv_set_verify_timing_events", "sv_verify_attn_noalloc",
    "sv_verify_select_workspace_size", "sv_verify_select",
)


class SvKvCache(ctypes.Structure):
    _fields_ = [
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("page_table", ctypes.c_void_p),
        ("page_size", ctypes.c_int32),
        ("max_pages", ctypes.c_int32),
        ("seq_stride", ctypes.c_int64),
        ("num_slots", ctypes.c_int64),
    ]


class SvError(RuntimeError):
    def __init__(self, status: int, msg: str):
        names = {1: "SV_E_INVALID", 2: "SV_E_UNSUPPORTED", 3: "SV_E_WORKSPACE", 4: "SV_E_HIP"}
        super().__init__(f"{names.get(status, status)}: {msg}")
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Load libsv.so from the package directory; fail loudly if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run `python -m tree_verify_sparse_amd.build` "
                          "(hipcc for gfx950); there is no fallback implementation")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, sz, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_float
    kvp = ctypes.POINTER(SvKvCache)
    lib.sv_validate_kv.restype = i32
    lib.sv_validate_kv.argtypes = [i32, i32, kvp, vp, i32, vp, vp]
    lib.sv_validate_tree.restype = i32
    lib.sv_validate_tree.argtypes = [i32, i32, vp, vp, vp]
    lib.sv_validate_index.restype = i32
    lib.sv_validate_index.argtypes = [i32, i32, kvp, vp, i32, vp, i32, vp, vp]
    lib.sv_abi_version.restype = i32
    lib.sv_abi_version.argtypes = []
    lib.sv_last_error.restype = ctypes.c_char_p
    lib.sv_last_error.argtypes = []
    lib.sv_verify_workspace_size.restype = sz
    lib.sv_verify_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32, i32, i32]
    lib.sv_verify_attn.restype = i32
    lib.sv_verify_attn.argtypes = [vp, i32, i32, i32, i32, i32, i32, kvp, vp, i32, vp, vp, i32, f32,
                                   vp, vp, vp, sz, vp]
    lib.sv_topk_workspace_size.restype = sz
    lib.sv_topk_workspace_size.argtypes = [i32, i32]
    lib.sv_topk_select.restype = i32
    lib.sv_topk_select.argtypes = [vp, i32, i32, vp, vp, i32, vp, vp, vp, sz, vp]
    lib.sv_sparse_workspace_size.restype = sz
    lib.sv_sparse_workspace_size.argtypes = [i32, i32, i32, i32, i32]
    lib.sv_sparse_draft_attn.restype = i32
    lib.sv_sparse_draft_attn.argtypes = [vp, i32, i32, i32, i32, i32, kvp, vp, i32, vp, i32, f32, vp, vp, sz, vp]
    lib.sv_verify_attn_per_head.restype = i32
    lib.sv_verify_attn_per_head.argtypes = lib.sv_verify_attn.argtypes
    lib.sv_sparse_draft_attn_per_head.restype = i32
    lib.sv_sparse_draft_attn_per_head.argtypes = lib.sv_sparse_draft_attn.argtypes
    lib.sv_select_sink_window.restype = i32
    lib.sv_select_sink_window.argtypes = [i32, i32, vp, i32, i32, i32, vp, vp, vp]
    lib.sv_compact_kv.restype = i32
    lib.sv_compact_kv.argtypes = [i32, i32, i32, i32, kvp, vp, i32, vp, i32, vp, vp, i32, vp]
    lib.sv_dense_draft_workspace_size.restype = sz
    lib.sv_dense_draft_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.sv_dense_draft_attn.restype = i32
    lib.sv_dense_draft_attn.argtypes = [vp, i32, i32, i32, i32, i32, vp, vp, i32, vp, f32, vp, vp, sz, vp]
    lib.sv_build_tree.restype = i32
    lib.sv_build_tree.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp, vp]
    lib.sv_accept_commit.restype = i32
    lib.sv_accept_commit.argtypes = [i32, i32, i32, i32, i32, kvp, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.sv_verify_select_workspace_size.restype = sz
    lib.sv_verify_select_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32, i32, i32]
    lib.sv_verify_select.restype = i32
    lib.sv_verify_select.argtypes = [vp, i32, i32, i32, i32, i32, i32, kvp, vp, i32, vp, vp, i32, f32,
                                     vp, i32, vp, vp, vp, vp, vp, sz, vp]
    lib.sv_verify_attn_noalloc.restype = i32
    lib.sv_verify_attn_noalloc.argtypes = [vp, i32, i32, i32, i32, i32, i32, kvp, vp, i32, vp, vp, i32, f32,
                                           vp, vp, vp]
    lib.sv_set_verify_timing_events.restype = i32
    lib.sv_set_verify_timing_events.argtypes = [vp, vp]
    _lib = lib
    return lib


def check(status: int) -> None:
    if status != SV_OK:
        raise SvError(status, load().sv_last_error().decode())
