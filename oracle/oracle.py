"""ctypes/NumPy wrapper of the C oracle in moe_oracle.c (test infrastructure).

The wrapper only marshals arrays; every value is computed by the C code.
Arrays follow the layout the C functions document:
  ids      int32 [T, K]             scores   float32 [T, K]
  x        float32 [T, D] or uint16 [T, D] (bf16 bits)
  row_map  int32 [round_up4(ntpr), K], -1 = no expert
  src      int32 [total]            counts int32 [E], offsets int32 [E+1]
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "liborc.so")
_lock = threading.Lock()
_lib = None

GCC_FLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC",
             "-shared", "-std=c11", "-Wall", "-Wextra"]


def lib_path() -> str:
    return _LIB


def build_oracle(force: bool = True) -> str:
    """Compile moe_oracle.c with gcc into liborc.so next to it."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", *GCC_FLAGS, _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build_oracle()
        L = C.CDLL(_LIB)
        i64, i32, vp, p64 = C.c_int64, C.c_int32, C.c_void_p, C.POINTER(C.c_int64)
        L.orc_ceil_div.argtypes = [i64, i64]; L.orc_ceil_div.restype = i64
        L.orc_round_up4.argtypes = [i64]; L.orc_round_up4.restype = i64
        L.orc_num_max_pretrain.argtypes = [i64, i64, i64, i64]; L.orc_num_max_pretrain.restype = i64
        L.orc_num_max_infer.argtypes = [i64, i64, i64]; L.orc_num_max_infer.restype = i64
        L.orc_validate_num_max.argtypes = [i64, i64]; L.orc_validate_num_max.restype = C.c_int
        L.orc_check_capacity.argtypes = [i64, i64, i64]; L.orc_check_capacity.restype = C.c_int
        L.orc_layout.argtypes = [vp, i64, i64, i32, i32, vp, vp, vp, vp]; L.orc_layout.restype = i64
        L.orc_dispatch.argtypes = [vp, i64, vp, i32, vp, i64, vp, vp, C.c_int]; L.orc_dispatch.restype = None
        L.orc_dispatch_rows.argtypes = [vp, i64, vp, i32, vp, vp, i64, vp, vp]; L.orc_dispatch_rows.restype = None
        L.orc_combine.argtypes = [vp, C.c_int, i64, vp, vp, i64, i32, vp, C.c_int]; L.orc_combine.restype = None
        L.orc_combine_tokens.argtypes = [vp, C.c_int, i64, vp, vp, i32, vp, i64, vp]; L.orc_combine_tokens.restype = None
        L.orc_f32_to_bf16.argtypes = [C.c_float]; L.orc_f32_to_bf16.restype = C.c_uint16
        L.orc_combine_backward.argtypes = [vp, vp, C.c_int, i64, vp, vp, i64, i32, vp, vp, C.c_int]
        L.orc_combine_backward.restype = None
        L.orc_dispatch_backward.argtypes = [vp, C.c_int, i64, vp, i64, i32, vp, C.c_int]
        L.orc_dispatch_backward.restype = None
        L.orc_topk_from_routing_map.argtypes = [vp, vp, i64, i32, i32, vp, vp, vp]
        L.orc_topk_from_routing_map.restype = None
        L.orc_dispatch_scaled.argtypes = [vp, C.c_int, i64, vp, i32, vp, i64, vp, C.c_int]
        L.orc_dispatch_scaled.restype = None
        L.orc_grouped_gemm.argtypes = [vp, vp, vp, i32, i64, i64, vp, C.c_int]
        L.orc_grouped_gemm.restype = None
        L.orc_grouped_gemm_at.argtypes = [vp, vp, vp, i32, i64, i64, vp, vp, i64, vp, C.c_int]
        L.orc_grouped_gemm_at.restype = None
        L.orc_f64_to_bf16_n.argtypes = [vp, i64, vp]
        L.orc_f64_to_bf16_n.restype = None
        _lib = L
        return L


def _ptr(a: np.ndarray):
    assert a.flags.c_contiguous
    return a.ctypes.data_as(C.c_void_p)


def _dtype_code(x: np.ndarray) -> int:
    if x.dtype == np.float32:
        return 0
    if x.dtype == np.uint16:
        return 1
    raise TypeError(f"x must be float32 or uint16 (bf16 bits), got {x.dtype}")


def ceil_div(a: int, b: int) -> int:
    return int(_load().orc_ceil_div(a, b))


def round_up4(n: int) -> int:
    return int(_load().orc_round_up4(n))


def num_max_pretrain(local_batch: int, seq_len: int, cp: int, tp: int) -> int:
    return int(_load().orc_num_max_pretrain(local_batch, seq_len, cp, tp))


def num_max_infer(max_num_batched_tokens: int, cp: int, tp: int) -> int:
    return int(_load().orc_num_max_infer(max_num_batched_tokens, cp, tp))


def validate_num_max(configured: int, derived: int) -> int:
    return int(_load().orc_validate_num_max(configured, derived))


def check_capacity(T: int, ntpr: int, nmax: int) -> int:
    return int(_load().orc_check_capacity(T, ntpr, nmax))


def layout(ids: np.ndarray, T: int, ntpr: int, E: int, K: int) -> dict:
    """Counts, offsets, row_map [round_up4(ntpr), K] and src [total]."""
    L = _load()
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    if ids.size < T * K:
        raise ValueError("ids must hold T*K entries")
    n4 = round_up4(ntpr)
    if n4 < 0:
        raise ValueError("num_tokens_per_rank must be >= 0")
    counts = np.zeros(E, np.int32)
    offsets = np.zeros(E + 1, np.int32)
    row_map = np.empty((n4, K), np.int32)
    src = np.empty(max(n4 * K, 1), np.int32)
    ids_arg = ids if ids.size else np.zeros(1, np.int32)
    total = L.orc_layout(_ptr(ids_arg), T, ntpr, E, K, _ptr(counts), _ptr(offsets),
                         _ptr(row_map), _ptr(src))
    if total < 0:
        raise ValueError("oracle layout rejected its arguments")
    return {"counts": counts, "offsets": offsets, "row_map": row_map,
            "src": src[:total].copy(), "total": int(total)}


def dispatch(x: np.ndarray, scores: np.ndarray, K: int, src: np.ndarray,
             nthreads: int = 1):
    """x_e [total, D] and s_e [total] (bit copies)."""
    L = _load()
    x = np.ascontiguousarray(x)
    scores = np.ascontiguousarray(scores, dtype=np.float32)
    src = np.ascontiguousarray(src, dtype=np.int32)
    total = src.size
    D = x.shape[1]
    row_bytes = D * x.itemsize
    x_e = np.empty((total, D), x.dtype)
    s_e = np.empty(total, np.float32)
    if total:
        L.orc_dispatch(_ptr(x), row_bytes, _ptr(scores), K, _ptr(src), total,
                       _ptr(x_e), _ptr(s_e), nthreads)
    return x_e, s_e


def dispatch_rows(x: np.ndarray, scores: np.ndarray, K: int, src: np.ndarray,
                  rows: np.ndarray):
    L = _load()
    x = np.ascontiguousarray(x)
    scores = np.ascontiguousarray(scores, dtype=np.float32)
    src = np.ascontiguousarray(src, dtype=np.int32)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    if rows.size and (rows.min() < 0 or rows.max() >= src.size):
        raise IndexError("row outside [0,total)")
    out_x = np.empty((rows.size, x.shape[1]), x.dtype)
    out_s = np.empty(rows.size, np.float32)
    if rows.size:
        L.orc_dispatch_rows(_ptr(x), x.shape[1] * x.itemsize, _ptr(scores), K,
                            _ptr(src), _ptr(rows), rows.size, _ptr(out_x), _ptr(out_s))
    return out_x, out_s


def combine(y_e: np.ndarray, row_map: np.ndarray, scores: np.ndarray, T: int,
            K: int, nthreads: int = 1) -> np.ndarray:
    """y [T, D] in y_e's dtype (float32, or uint16 bf16 bits)."""
    L = _load()
    y_e = np.ascontiguousarray(y_e)
    row_map = np.ascontiguousarray(row_map, dtype=np.int32)
    scores = np.ascontiguousarray(scores, dtype=np.float32)
    D = y_e.shape[1]
    y = np.empty((T, D), y_e.dtype)
    if T:
        ye_arg = y_e if y_e.size else np.zeros((1, D), y_e.dtype)
        L.orc_combine(_ptr(ye_arg), _dtype_code(y_e), D, _ptr(row_map), _ptr(scores),
                      T, K, _ptr(y), nthreads)
    return y


def combine_tokens(y_e: np.ndarray, row_map: np.ndarray, scores: np.ndarray,
                   K: int, tokens: np.ndarray) -> np.ndarray:
    L = _load()
    y_e = np.ascontiguousarray(y_e)
    row_map = np.ascontiguousarray(row_map, dtype=np.int32)
    scores = np.ascontiguousarray(scores, dtype=np.float32)
    tokens = np.ascontiguousarray(tokens, dtype=np.int64)
    D = y_e.shape[1]
    out = np.empty((tokens.size, D), y_e.dtype)
    if tokens.size:
        L.orc_combine_tokens(_ptr(y_e), _dtype_code(y_e), D, _ptr(row_map), _ptr(scores),
                             K, _ptr(tokens), tokens.size, _ptr(out))
    return out


def f32_to_bf16(values) -> np.ndarray:
    """Elementwise oracle rounding of float32 values to bf16 bits."""
    L = _load()
    v = np.asarray(values, dtype=np.float32).ravel()
    return np.array([L.orc_f32_to_bf16(float(f)) for f in v], dtype=np.uint16)


def run_pipeline(x: np.ndarray, ids: np.ndarray, scores: np.ndarray, T: int,
                 ntpr: int, E: int, K: int, nthreads: int = 1) -> dict:
    """Layout, dispatch, identity expert (y_e = x_e) and combine of tokens
    [0,T); x, ids and scores hold at least T rows."""
    lay = layout(ids[:T], T, ntpr, E, K)
    x_e, s_e = dispatch(x[:T], scores[:T], K, lay["src"], nthreads)
    y = combine(x_e, lay["row_map"], scores[:T], T, K, nthreads)
    lay.update(x_e=x_e, s_e=s_e, y=y)
    return lay


def combine_backward(g: np.ndarray, y_e: np.ndarray, row_map: np.ndarray,
                     scores: np.ndarray, T: int, K: int, nthreads: int = 1):
    """(g_e [rows, D] with rows r(t,k) written and the rest zero,
    grad_s [T, K] float64) for dL/dy = g [T, D]."""
    L = _load()
    g = np.ascontiguousarray(g)
    y_e = np.ascontiguousarray(y_e)
    if g.dtype != y_e.dtype:
        raise TypeError("g and y_e need the same element dtype")
    row_map = np.ascontiguousarray(row_map, dtype=np.int32)
    scores = np.ascontiguousarray(scores, dtype=np.float32)
    D = y_e.shape[1]
    g_e = np.zeros_like(y_e)
    grad_s = np.zeros((T, K), np.float64)
    if T:
        L.orc_combine_backward(_ptr(g), _ptr(y_e), _dtype_code(y_e), D, _ptr(row_map),
                               _ptr(scores), T, K, _ptr(g_e), _ptr(grad_s), nthreads)
    return g_e, grad_s


def dispatch_backward(h: np.ndarray, row_map: np.ndarray, T: int, K: int,
                      nthreads: int = 1) -> np.ndarray:
    """gx [T, D] = sum over each token's slots of h rows (fp32, k order)."""
    L = _load()
    h = np.ascontiguousarray(h)
    row_map = np.ascontiguousarray(row_map, dtype=np.int32)
    D = h.shape[1]
    gx = np.empty((T, D), h.dtype)
    if T:
        h_arg = h if h.size else np.zeros((1, D), h.dtype)
        L.orc_dispatch_backward(_ptr(h_arg), _dtype_code(h), D, _ptr(row_map), T, K,
                                _ptr(gx), nthreads)
    return gx


def topk_from_routing_map(routing_map: np.ndarray, probs: np.ndarray, K: int):
    """(ids [T, K] int32, scores [T, K] float32, n_experts [T] int32)."""
    L = _load()
    m = np.ascontiguousarray(routing_map).astype(np.uint8, copy=False)
    m = np.ascontiguousarray(m)
    probs = np.ascontiguousarray(probs, dtype=np.float32)
    T, E = m.shape
    ids = np.empty((T, K), np.int32)
    scores = np.empty((T, K), np.float32)
    n = np.empty(T, np.int32)
    if T:
        L.orc_topk_from_routing_map(_ptr(m), _ptr(probs), T, E, K, _ptr(ids), _ptr(scores),
                                    _ptr(n))
    return ids, scores, n


def dispatch_scaled(x: np.ndarray, scores: np.ndarray, K: int, src: np.ndarray,
                    nthreads: int = 1) -> np.ndarray:
    """x_e [total, D]: row r = scores[slot] * x[slot // K], rounded."""
    L = _load()
    x = np.ascontiguousarray(x)
    scores = np.ascontiguousarray(scores, dtype=np.float32)
    src = np.ascontiguousarray(src, dtype=np.int32)
    D = x.shape[1]
    x_e = np.empty((src.size, D), x.dtype)
    if src.size:
        L.orc_dispatch_scaled(_ptr(x), _dtype_code(x), D, _ptr(scores), K, _ptr(src), src.size,
                              _ptr(x_e), nthreads)
    return x_e


def _gemm_args(x_e, w, offsets):
    x_e = np.ascontiguousarray(x_e)
    w = np.ascontiguousarray(w)
    if x_e.dtype != np.uint16 or w.dtype != np.uint16:
        raise TypeError("the expert step takes bf16 bits (uint16) for x_e and w")
    offsets = np.ascontiguousarray(offsets, dtype=np.int32)
    E, N, Kd = w.shape
    if offsets.shape != (E + 1,) or x_e.shape[1] != Kd:
        raise ValueError("shapes: x_e [rows, Kd], w [E, N, Kd], offsets [E+1]")
    if offsets[0] < 0 or np.any(np.diff(offsets) < 0) or offsets[-1] > x_e.shape[0]:
        raise ValueError("offsets must be a non-decreasing prefix sum within x_e's rows")
    return x_e, w, offsets, E, N, Kd


def grouped_gemm(x_e: np.ndarray, w: np.ndarray, offsets: np.ndarray,
                 nthreads: int = 1) -> np.ndarray:
    """out [rows, N] float64: row r of expert e's segment is x_e[r] @ w[e].T
    (w [E, N, Kd] bf16 bits); rows outside every segment stay NaN."""
    L = _load()
    x_e, w, offsets, E, N, Kd = _gemm_args(x_e, w, offsets)
    out = np.full((x_e.shape[0], N), np.nan)
    if out.size and offsets[-1] > 0:
        L.orc_grouped_gemm(_ptr(x_e), _ptr(w), _ptr(offsets), E, Kd, N, _ptr(out), nthreads)
    return out


def grouped_gemm_at(x_e: np.ndarray, w: np.ndarray, offsets: np.ndarray, rows, cols,
                    nthreads: int = 1) -> np.ndarray:
    """The grouped_gemm values at positions (rows[i], cols[i]) only."""
    L = _load()
    x_e, w, offsets, E, N, Kd = _gemm_args(x_e, w, offsets)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    if rows.shape != cols.shape or np.any(cols < 0) or np.any(cols >= N):
        raise ValueError("rows and cols: same shape, cols within [0, N)")
    out = np.empty(rows.shape, np.float64)
    if rows.size:
        L.orc_grouped_gemm_at(_ptr(x_e), _ptr(w), _ptr(offsets), E, Kd, N, _ptr(rows),
                              _ptr(cols), rows.size, _ptr(out), nthreads)
    return out


def f64_to_bf16(values) -> np.ndarray:
    """Elementwise oracle rounding of float64 values to bf16 bits (one rounding)."""
    L = _load()
    v = np.ascontiguousarray(values, dtype=np.float64)
    out = np.empty(v.shape, np.uint16)
    if v.size:
        L.orc_f64_to_bf16_n(_ptr(v), v.size, _ptr(out))
    return out


def run_layer(x: np.ndarray, ids: np.ndarray, scores: np.ndarray, w: np.ndarray, T: int,
              ntpr: int, E: int, K: int, nthreads: int = 1) -> dict:
    """Layout, dispatch, the expert step (w [E, D, D] bf16 bits; its output
    rounded once to bf16) and combine of tokens [0,T)."""
    lay = layout(ids[:T], T, ntpr, E, K)
    x_e, s_e = dispatch(x[:T], scores[:T], K, lay["src"], nthreads)
    h = grouped_gemm(x_e, w, lay["offsets"], nthreads)
    y_e = f64_to_bf16(h)
    y = combine(y_e, lay["row_map"], scores[:T], T, K, nthreads)
    lay.update(x_e=x_e, s_e=s_e, h=h, y_e=y_e, y=y)
    return lay
