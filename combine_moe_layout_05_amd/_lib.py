"""ctypes declarations of the C ABI in include/moe.h and the library loader.

The library is loaded after torch so that both resolve the same HIP runtime
(libamdhip64.so.7, matched by soname): device pointers and streams from torch
are then valid inside the library. Loading fails loudly when the built
library is missing; there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os
import threading

from ._paths import LIB_PATH

MOE_OK = 0
MOE_ERR_INVALID_ARG = -1
MOE_ERR_CAPACITY = -2
MOE_ERR_WORKSPACE = -3
MOE_ERR_HIP = -4
MOE_ERR_STATE = -5
MOE_ERR_UNSUPPORTED = -6
MOE_ERR_SCRATCH = -7
MOE_NOALLOC_SCRATCH_BYTES = 4 << 20

MOE_FLAG_BACKWARD = 1

MOE_F32 = 0
MOE_BF16 = 1
MOE_WEIGHTS_ROW_MAJOR = 0
MOE_WEIGHTS_TILED = 1

MOE_MAX_EXPERTS = 1024
MOE_MAX_TOPK = 16
MOE_WORKSPACE_ALIGN = 256

# Entry points declared in include/moe.h: name -> (restype, argtypes).
_i32, _i64, _vp, _int = C.c_int32, C.c_int64, C.c_void_p, C.c_int


class MoeConfig(C.Structure):
    _fields_ = [("num_max_tokens_per_rank", _i32), ("hidden", _i32),
                ("num_experts", _i32), ("topk", _i32), ("dtype", _i32), ("flags", _i32)]


class MoeBuffersDesc(C.Structure):
    _fields_ = [(n, _i64) for n in (
        "workspace_bytes", "nmax4", "max_rows", "row_bytes", "max_tiles", "tile_slots",
        "counts", "offsets", "row_map", "src_map", "s_e", "x_e", "y",
        "block_hist", "map_ids", "map_scores", "map_n_experts", "g_e", "g_s", "g_x")]


class MoeTuning(C.Structure):
    _fields_ = [("dispatch_segments", _i32), ("combine_segments", _i32),
                ("dispatch_nontemporal", _i32), ("combine_nontemporal", _i32),
                ("dispatch_block_waves", _i32), ("combine_block_waves", _i32),
                ("combine_store_nontemporal", _i32), ("layout_launches", _i32),
                ("dispatch_store_burst", _i32), ("combine_backward_store", _i32),
                ("dispatch_x_nontemporal", _i32)]


SIGNATURES = {
    "moe_workspace_bytes": (_int, [C.POINTER(MoeConfig), C.POINTER(C.c_size_t)]),
    "moe_create": (_int, [C.POINTER(MoeConfig), _vp, C.c_size_t, C.POINTER(_vp)]),
    "moe_destroy": (_int, [_vp]),
    "moe_workspace_offsets": (_int, [_vp, C.POINTER(MoeBuffersDesc)]),
    "moe_layout": (_int, [_vp, _vp, _i32, _i32, _vp]),
    "moe_layout_noalloc": (_int, [_vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp]),
    "moe_dispatch": (_int, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _vp]),
    "moe_combine": (_int, [_vp, _vp, _vp, _vp, _i32, _i32, _vp, C.POINTER(_vp)]),
    "moe_dispatch_scaled": (_int, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _vp]),
    "moe_layout_dispatch": (_int, [_vp, _vp, _vp, _vp, _i32, _i32, _vp]),
    "moe_topk_from_routing_map": (_int, [_vp, _vp, _vp, _i32, _vp, C.POINTER(_vp),
                                         C.POINTER(_vp), C.POINTER(_vp)]),
    "moe_combine_backward": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _vp,
                                    C.POINTER(_vp), C.POINTER(_vp)]),
    "moe_dispatch_backward": (_int, [_vp, _vp, _vp, _i32, _i32, _vp, C.POINTER(_vp)]),
    "moe_grouped_gemm": (_int, [_vp, _vp, _vp, _i32, _i64, _i32, _i32, _vp, _i32, _i32, _vp]),
    "moe_tiled_weights_bytes": (_i64, [_i32, _i32, _i32]),
    "moe_tile_expert_weights": (_int, [_vp, _i32, _i32, _i32, _vp, _vp]),
    "moe_set_tuning": (_int, [_vp, C.POINTER(MoeTuning)]),
    "moe_get_tuning": (_int, [_vp, C.POINTER(MoeTuning)]),
    "moe_ceil_div": (_i64, [_i64, _i64]),
    "moe_round_up4": (_i64, [_i64]),
    "moe_num_max_tokens_pretrain": (_i64, [_i64, _i64, _i64, _i64]),
    "moe_num_max_tokens_infer": (_i64, [_i64, _i64, _i64]),
    "moe_validate_num_max": (_int, [_i64, _i64]),
    "moe_check_capacity": (_int, [_i64, _i64, _i64]),
    "moe_strerror": (C.c_char_p, [_int]),
}

_lock = threading.Lock()
_lib = None


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        msg = "?"
        if _lib is not None:
            msg = _lib.moe_strerror(status).decode()
        super().__init__(f"{what}: status {status} ({msg})")


def _hip_runtimes_mapped() -> set:
    paths = set()
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    paths.add(os.path.realpath(line.split()[-1]))
    except OSError:
        pass
    return paths


def load(path: str = LIB_PATH):
    """Load libmoe_layout.so once and declare its entry points."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise RuntimeError(
                f"{path} is not built; run `python combine_moe_layout_05_amd/build.py`")
        import torch  # noqa: F401  (loads torch's HIP runtime first)
        lib = C.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        runtimes = _hip_runtimes_mapped()
        if len(runtimes) > 1:
            raise RuntimeError(f"two HIP runtimes are mapped: {sorted(runtimes)}")
        _lib = lib
        return lib


def check(status: int, what: str) -> None:
    if status != MOE_OK:
        raise MoeError(status, what)
