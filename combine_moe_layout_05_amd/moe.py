"""Python binding of the MoE layout / dispatch / combine / expert-step C ABI.

Argument marshalling only: this module checks tensor placement, dtype and
shape, passes raw device pointers and torch's current HIP stream to
libmoe_layout.so, and returns torch views of the library's persistent buffers.
Every step of the path runs in the library's HIP kernels.

The API follows "Unify expert parallel token dispatcher API" (section "API
design"): the lifetime maximum num_max_tokens_per_rank sizes the storage once;
each dispatch takes the current capacity num_tokens_per_rank, with
x_TD.shape[0] <= num_tokens_per_rank <= num_max_tokens_per_rank. Capacities
are padded up to a multiple of 4 tokens; padded rows route to no expert and
combine slices them off ("fix(moe): equalize and align per-rank token counts
for HybridEP dispatch", section "Fix").
"""
from __future__ import annotations

import ctypes as C
from typing import NamedTuple, Optional

import torch

from . import _lib as L

_DTYPES = {torch.float32: L.MOE_F32, torch.bfloat16: L.MOE_BF16}


class Layout(NamedTuple):
    counts: torch.Tensor     # int32 [E], device
    offsets: torch.Tensor    # int32 [E+1], offsets[E] = total, device
    row_map: torch.Tensor    # int32 [round_up4(ntpr), K], -1 = no expert


class Dispatched(NamedTuple):
    x_e: torch.Tensor        # [round_up4(ntpr) * K, D] view; rows [0, total) valid
    s_e: torch.Tensor        # float32 [round_up4(ntpr) * K]; rows [0, total) valid


# torch's current HIP stream of a device as a raw handle. The private getter
# returns the handle without building a Python stream object (about 0.1 us
# against 2 us per call); the public API serves when it is absent.
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(device: torch.device) -> int:
    if _raw_stream is not None:
        return _raw_stream(device.index)
    return torch.cuda.current_stream(device).cuda_stream


def ceil_div(a: int, b: int) -> int:
    return int(L.load().moe_ceil_div(a, b))


_round_up4_cache: dict = {}


def round_up4(n: int) -> int:
    """moe_round_up4 of the library, remembered per argument (the calls take
    a capacity that rarely changes, and a ctypes call per use costs more than
    the launch it sizes)."""
    r = _round_up4_cache.get(n)
    if r is None:
        r = int(L.load().moe_round_up4(n))
        if len(_round_up4_cache) < 4096:
            _round_up4_cache[n] = r
    return r


def num_max_tokens_pretrain(local_batch: int, seq_len: int, cp: int = 1, tp: int = 1) -> int:
    return int(L.load().moe_num_max_tokens_pretrain(local_batch, seq_len, cp, tp))


def num_max_tokens_infer(max_num_batched_tokens: int, cp: int = 1, tp: int = 1) -> int:
    return int(L.load().moe_num_max_tokens_infer(max_num_batched_tokens, cp, tp))


def validate_num_max(configured: int, derived: int) -> None:
    L.check(L.load().moe_validate_num_max(configured, derived), "validate_num_max")


class TiledExpertWeights(NamedTuple):
    """Expert weights in the matrix-core tile order (moe_tile_expert_weights)."""
    data: torch.Tensor       # uint8 [moe_tiled_weights_bytes], device
    num_experts: int
    n_out: int
    k_in: int


def tile_expert_weights(weights: torch.Tensor) -> TiledExpertWeights:
    """One-time rewrite of bf16 [E, n_out, k_in] expert weights into the tile
    order the expert step reads fastest (moe_tile_expert_weights)."""
    if weights.dtype != torch.bfloat16 or weights.dim() != 3 or not weights.is_contiguous():
        raise ValueError("weights must be a contiguous bf16 [E, n_out, k_in] tensor")
    E, n_out, k_in = weights.shape
    lib = L.load()
    nbytes = int(lib.moe_tiled_weights_bytes(E, n_out, k_in))
    if nbytes < 0:
        raise ValueError(f"unsupported expert weight shape {tuple(weights.shape)}")
    data = torch.empty(nbytes, dtype=torch.uint8, device=weights.device)
    L.check(lib.moe_tile_expert_weights(weights.data_ptr(), E, n_out, k_in, data.data_ptr(),
                                        _stream(weights.device)), "moe_tile_expert_weights")
    return TiledExpertWeights(data, E, n_out, k_in)


def grouped_gemm(x_expert: torch.Tensor, weights, offsets: torch.Tensor,
                 out: Optional[torch.Tensor] = None, *, row_tile: int = 0) -> torch.Tensor:
    """Expert step between dispatch and combine (moe_grouped_gemm): for each
    expert e, rows r in [offsets[e], offsets[e+1]) get
    out[r] = x_expert[r] @ W[e].T (fp32 accumulation, one rounding to bf16).
    offsets stays on the device (e.g. Layout.offsets); rows outside every
    segment keep what `out` held.

    x_expert bf16 [R, k_in]; weights bf16 [E, n_out, k_in] or the
    TiledExpertWeights of them (same results, faster); offsets int32 [E+1];
    out bf16 [R, n_out] (allocated with torch.empty if None)."""
    dev = x_expert.device
    if isinstance(weights, TiledExpertWeights):
        E, n_out, k_in = weights.num_experts, weights.n_out, weights.k_in
        w_t, layout = weights.data, L.MOE_WEIGHTS_TILED
        if w_t.device != dev:
            raise ValueError(f"weights must be on {dev}, got {w_t.device}")
        # the kernel trusts the tiled buffer's size: check it here
        need = int(L.load().moe_tiled_weights_bytes(E, n_out, k_in))
        if (w_t.dtype != torch.uint8 or w_t.dim() != 1 or not w_t.is_contiguous()
                or w_t.numel() != need):
            raise ValueError(f"tiled weights must be a contiguous uint8 tensor of {need} bytes "
                             f"(moe_tiled_weights_bytes({E}, {n_out}, {k_in}))")
    else:
        if weights.device != dev:
            raise ValueError(f"weights must be on {dev}, got {weights.device}")
        if weights.dtype != torch.bfloat16:
            raise TypeError(f"weights must be torch.bfloat16, got {weights.dtype}")
        if weights.dim() != 3 or not weights.is_contiguous():
            raise ValueError("weights must be a contiguous 3-d tensor")
        E, n_out, k_in = weights.shape
        w_t, layout = weights, L.MOE_WEIGHTS_ROW_MAJOR
    for name, t, dt, dim in (("x_expert", x_expert, torch.bfloat16, 2),
                             ("offsets", offsets, torch.int32, 1)):
        if t.device != dev:
            raise ValueError(f"{name} must be on {dev}, got {t.device}")
        if t.dtype != dt:
            raise TypeError(f"{name} must be {dt}, got {t.dtype}")
        if t.dim() != dim or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {dim}-d tensor")
    R = x_expert.shape[0]
    if x_expert.shape[1] != k_in or offsets.shape[0] != E + 1:
        raise ValueError("shapes: x_expert [R, k_in], weights [E, n_out, k_in], offsets [E+1]")
    if out is None:
        out = torch.empty((R, n_out), dtype=torch.bfloat16, device=dev)
    elif (out.device != dev or out.dtype != torch.bfloat16 or tuple(out.shape) != (R, n_out)
          or not out.is_contiguous()):
        raise ValueError(f"out must be a contiguous bf16 [{R}, {n_out}] tensor on {dev}")
    L.check(L.load().moe_grouped_gemm(x_expert.data_ptr(), w_t.data_ptr(), offsets.data_ptr(),
                                      E, R, k_in, n_out, out.data_ptr(), int(row_tile), layout,
                                      _stream(dev)), "moe_grouped_gemm")
    return out


def layout_noalloc(topk_ids: torch.Tensor, num_experts: int, counts: torch.Tensor,
                   offsets: torch.Tensor, row_map: torch.Tensor, src_map: torch.Tensor, *,
                   num_tokens_per_rank: Optional[int] = None) -> None:
    """moe_layout for callers that cannot allocate (moe_layout_noalloc): no
    context, no workspace; the per-tile histograms live in the library's
    static device scratch. Fills the caller's counts int32 [E], offsets
    int32 [E+1], row_map int32 [round_up4(ntpr), K] and src_map int32
    [>= T*K] (rows [0, total) written) from ids int32 [T, K], on the current
    stream. Calls on one device must not overlap (they share the scratch)."""
    dev = topk_ids.device
    if topk_ids.dim() != 2:
        raise ValueError("topk_ids must be [T, K]")
    T, K = topk_ids.shape
    ntpr = T if num_tokens_per_rank is None else int(num_tokens_per_rank)
    n4 = round_up4(ntpr) if ntpr >= 0 else -1
    want = (("topk_ids", topk_ids, None), ("counts", counts, (num_experts,)),
            ("offsets", offsets, (num_experts + 1,)), ("row_map", row_map, (n4, K)),
            ("src_map", src_map, None))
    for name, t, shape in want:
        if t.device != dev or t.dtype != torch.int32 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous int32 tensor on {dev}")
        if shape is not None and tuple(t.shape) != shape:
            raise ValueError(f"{name} must have shape {shape}, got {tuple(t.shape)}")
    if src_map.numel() < T * K:
        raise ValueError("src_map needs at least T * K entries")
    L.check(L.load().moe_layout_noalloc(topk_ids.data_ptr(), T, ntpr, num_experts, K,
                                        counts.data_ptr(), offsets.data_ptr(), row_map.data_ptr(),
                                        src_map.data_ptr(), _stream(dev)), "moe_layout_noalloc")


class MoeDispatcher:
    """One persistent workspace for MoE token layout, dispatch and combine.

    The workspace (a uint8 device tensor) is allocated once here, at the
    lifetime maximum, and carved by the library into fixed-address buffers;
    no later call allocates, grows, synchronizes or reads back.

    The views the calls return (Layout, Dispatched, combine's y[:T]) are
    made once per extent and shared by every call with that extent: they
    always show the buffers' current contents, and their metadata (shape,
    requires_grad) should not be changed; take a view or a copy for that.

    x_e_generation counts the calls that rewrote x_e (dispatch,
    dispatch_scaled, layout_dispatch), so a holder of an x_e view can tell
    whether the rows it saw are still there. close() (also run when the
    object is collected) waits for the device's queued work before the
    library context is destroyed, since that work may still use the context's
    buffers and counter slot.
    """

    def __init__(self, num_max_tokens_per_rank: int, hidden: int, num_experts: int,
                 topk: int, dtype: torch.dtype = torch.bfloat16,
                 device: Optional[torch.device] = None, backward: bool = False):
        if dtype not in _DTYPES:
            raise TypeError(f"dtype must be one of {list(_DTYPES)}")
        lib = L.load()
        self.device = torch.device(device if device is not None else "cuda")
        if self.device.type != "cuda":
            raise ValueError("the HIP library needs a GPU device")
        if self.device.index is None:
            self.device = torch.device("cuda", torch.cuda.current_device())
        self.dtype = dtype
        self.hidden, self.num_experts, self.topk = hidden, num_experts, topk
        self.num_max_tokens_per_rank = num_max_tokens_per_rank
        self.backward_enabled = bool(backward)
        self.x_e_generation = 0
        self._dev_index = self.device.index
        self._views: dict = {}
        self._out = C.c_void_p()
        self._out_ref = C.byref(self._out)
        self._cfg = L.MoeConfig(num_max_tokens_per_rank, hidden, num_experts, topk,
                                _DTYPES[dtype], L.MOE_FLAG_BACKWARD if backward else 0)
        nbytes = C.c_size_t(0)
        L.check(lib.moe_workspace_bytes(C.byref(self._cfg), C.byref(nbytes)),
                "moe_workspace_bytes")
        self.workspace = torch.empty(nbytes.value, dtype=torch.uint8, device=self.device)
        ctx = C.c_void_p()
        L.check(lib.moe_create(C.byref(self._cfg), self.workspace.data_ptr(), nbytes.value,
                               C.byref(ctx)), "moe_create")
        self._ctx = ctx
        self._lib = lib
        d = L.MoeBuffersDesc()
        L.check(lib.moe_workspace_offsets(ctx, C.byref(d)), "moe_workspace_offsets")
        self.desc = d
        E, K, D = num_experts, topk, hidden
        self.nmax4 = int(d.nmax4)
        self.counts = self._view(d.counts, E, torch.int32)
        self.offsets = self._view(d.offsets, E + 1, torch.int32)
        self.row_map = self._view(d.row_map, d.max_rows, torch.int32).view(self.nmax4, K)
        self.src_map = self._view(d.src_map, d.max_rows, torch.int32)
        self.s_e = self._view(d.s_e, d.max_rows, torch.float32)
        self.x_e = self._view(d.x_e, d.max_rows * D, dtype).view(d.max_rows, D)
        self.y = self._view(d.y, self.nmax4 * D, dtype).view(self.nmax4, D)
        self.map_ids = self._view(d.map_ids, d.max_rows, torch.int32).view(self.nmax4, K)
        self.map_scores = self._view(d.map_scores, d.max_rows, torch.float32).view(self.nmax4, K)
        self.map_n_experts = self._view(d.map_n_experts, self.nmax4, torch.int32)
        if backward:
            self.g_e = self._view(d.g_e, d.max_rows * D, dtype).view(d.max_rows, D)
            self.g_s = self._view(d.g_s, d.max_rows, torch.float32).view(self.nmax4, K)
            self.g_x = self._view(d.g_x, self.nmax4 * D, dtype).view(self.nmax4, D)

    def _view(self, off: int, n: int, dtype: torch.dtype) -> torch.Tensor:
        nbytes = int(n) * torch.empty(0, dtype=dtype).element_size()
        return self.workspace[int(off):int(off) + nbytes].view(dtype)

    def rows_for(self, num_tokens_per_rank: int) -> int:
        """Rows of the expert-major buffers a call with this capacity uses."""
        return round_up4(int(num_tokens_per_rank)) * self.topk

    def close(self) -> None:
        """Destroy the library context after the device has finished every
        queued kernel (they may still read its buffers or hold its counter
        slot). The workspace tensor is released with this object."""
        ctx = getattr(self, "_ctx", None)
        if ctx is not None and ctx.value:
            if torch.cuda.is_current_stream_capturing():
                # A wait is not allowed while a graph is being captured, and
                # the captured work may use this context: keep it alive.
                return
            torch.cuda.synchronize(self.device)
            self._lib.moe_destroy(ctx)
            self._ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:  # interpreter shutdown: the runtime may be gone
            pass

    # -- argument checks (marshalling) -------------------------------------
    def _dev(self, t: torch.Tensor, name: str, dtype: torch.dtype, cols: int) -> torch.Tensor:
        if t.dtype != dtype:
            raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
        if not t.is_cuda or t.get_device() != self._dev_index:
            raise ValueError(f"{name} must be on {self.device}, got {t.device}")
        if t.dim() != 2 or t.shape[1] != cols:
            raise ValueError(f"{name} must be [T, {cols}], got {tuple(t.shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        return t

    def _cached(self, key, make):
        """A view of a persistent buffer, made once per (buffer, extent)."""
        v = self._views.get(key)
        if v is None:
            v = make()
            if len(self._views) < 1024:
                self._views[key] = v
        return v

    def _ntpr(self, T: int, num_tokens_per_rank: Optional[int]) -> int:
        return T if num_tokens_per_rank is None else int(num_tokens_per_rank)

    # -- the three calls ---------------------------------------------------
    def layout(self, topk_ids: torch.Tensor, num_tokens_per_rank: Optional[int] = None) -> Layout:
        """Per-expert counts, offsets and the row map of ids [T, K]."""
        ids = self._dev(topk_ids, "topk_ids", torch.int32, self.topk)
        T = ids.shape[0]
        ntpr = self._ntpr(T, num_tokens_per_rank)
        L.check(self._lib.moe_layout(self._ctx, ids.data_ptr(), T, ntpr, _stream(self.device)),
                "moe_layout")
        n4 = round_up4(ntpr)
        return self._cached(("layout", n4),
                            lambda: Layout(self.counts, self.offsets, self.row_map[:n4]))

    def dispatch(self, x_TD: torch.Tensor, topk_scores_TK: torch.Tensor,
                 topk_expert_ids_TK: torch.Tensor, num_local_tokens_per_expert_E: torch.Tensor,
                 *, num_tokens_per_rank: Optional[int] = None) -> Dispatched:
        """Permute x rows and scores into the expert-major buffers using the
        row map of the preceding layout() on the same ids."""
        return self._dispatch(self._lib.moe_dispatch, "moe_dispatch", x_TD, topk_scores_TK,
                              topk_expert_ids_TK, num_local_tokens_per_expert_E,
                              num_tokens_per_rank)

    def dispatch_scaled(self, x_TD: torch.Tensor, topk_scores_TK: torch.Tensor,
                        topk_expert_ids_TK: torch.Tensor,
                        num_local_tokens_per_expert_E: torch.Tensor, *,
                        num_tokens_per_rank: Optional[int] = None) -> Dispatched:
        """dispatch() with each copy scaled by its slot's score (one fp32
        product, rounded); pair with combine(topk_scores_TK=None)."""
        return self._dispatch(self._lib.moe_dispatch_scaled, "moe_dispatch_scaled", x_TD,
                              topk_scores_TK, topk_expert_ids_TK,
                              num_local_tokens_per_expert_E, num_tokens_per_rank)

    def _dispatch(self, fn, what, x_TD, topk_scores_TK, topk_expert_ids_TK, counts,
                  num_tokens_per_rank) -> Dispatched:
        x = self._dev(x_TD, "x_TD", self.dtype, self.hidden)
        T = x.shape[0]
        s = self._dev(topk_scores_TK, "topk_scores_TK", torch.float32, self.topk)
        ids = self._dev(topk_expert_ids_TK, "topk_expert_ids_TK", torch.int32, self.topk)
        if s.shape[0] != T or ids.shape[0] != T:
            raise ValueError("x_TD, topk_scores_TK and topk_expert_ids_TK need the same T")
        ntpr = self._ntpr(T, num_tokens_per_rank)
        L.check(fn(self._ctx, x.data_ptr(), s.data_ptr(), ids.data_ptr(), counts.data_ptr(), T,
                   ntpr, _stream(self.device)), what)
        self.x_e_generation += 1
        rows = round_up4(ntpr) * self.topk
        return self._cached(("dispatched", rows),
                            lambda: Dispatched(self.x_e[:rows], self.s_e[:rows]))

    def layout_dispatch(self, x_TD: torch.Tensor, topk_scores_TK: torch.Tensor,
                        topk_expert_ids_TK: torch.Tensor, *,
                        num_tokens_per_rank: Optional[int] = None):
        """layout() then dispatch() in two launches (moe_layout_dispatch; the
        separate calls take three above 32768 slots); same results bit for
        bit. Returns (Layout, Dispatched)."""
        x = self._dev(x_TD, "x_TD", self.dtype, self.hidden)
        T = x.shape[0]
        s = self._dev(topk_scores_TK, "topk_scores_TK", torch.float32, self.topk)
        ids = self._dev(topk_expert_ids_TK, "topk_expert_ids_TK", torch.int32, self.topk)
        if s.shape[0] != T or ids.shape[0] != T:
            raise ValueError("x_TD, topk_scores_TK and topk_expert_ids_TK need the same T")
        ntpr = self._ntpr(T, num_tokens_per_rank)
        L.check(self._lib.moe_layout_dispatch(self._ctx, x.data_ptr(), s.data_ptr(),
                                              ids.data_ptr(), T, ntpr, _stream(self.device)),
                "moe_layout_dispatch")
        self.x_e_generation += 1
        n4 = round_up4(ntpr)
        rows = n4 * self.topk
        return (Layout(self.counts, self.offsets, self.row_map[:n4]),
                Dispatched(self.x_e[:rows], self.s_e[:rows]))

    def topk_from_routing_map(self, routing_map_TE: torch.Tensor, probs_TE: torch.Tensor):
        """(ids [T, K], scores [T, K], n_experts [T]) views: the top-k form of
        a boolean routing map with probabilities (experts in ascending order,
        -1 / 0 past a token's experts)."""
        m = routing_map_TE
        if m.dtype == torch.bool:
            m = m.view(torch.uint8)
        m = self._dev(m, "routing_map_TE", torch.uint8, self.num_experts)
        p = self._dev(probs_TE, "probs_TE", torch.float32, self.num_experts)
        T = m.shape[0]
        if p.shape[0] != T:
            raise ValueError("routing_map_TE and probs_TE need the same T")
        o_ids, o_s, o_n = C.c_void_p(), C.c_void_p(), C.c_void_p()
        L.check(self._lib.moe_topk_from_routing_map(self._ctx, m.data_ptr(), p.data_ptr(), T,
                                                    _stream(self.device), C.byref(o_ids),
                                                    C.byref(o_s), C.byref(o_n)),
                "moe_topk_from_routing_map")
        return self.map_ids[:T], self.map_scores[:T], self.map_n_experts[:T]

    def combine(self, y_expert: torch.Tensor, row_map: torch.Tensor,
                topk_scores_TK: Optional[torch.Tensor], *,
                num_tokens_per_rank: Optional[int] = None, T: Optional[int] = None) -> torch.Tensor:
        """Score-weighted sum of expert outputs back to token order; returns
        y[:T] (a view of the persistent output buffer). topk_scores_TK=None
        gives unit weights (then T is required)."""
        if topk_scores_TK is None:
            if T is None:
                raise ValueError("T is required when topk_scores_TK is None")
            s_ptr = 0
        else:
            s = self._dev(topk_scores_TK, "topk_scores_TK", torch.float32, self.topk)
            if T is not None and T != s.shape[0]:
                raise ValueError("T differs from topk_scores_TK.shape[0]")
            T = s.shape[0]
            s_ptr = s.data_ptr()
        if (y_expert.dtype != self.dtype or not y_expert.is_cuda
                or y_expert.get_device() != self._dev_index):
            raise TypeError("y_expert must match the dispatcher's device and dtype")
        if y_expert.dim() != 2 or y_expert.shape[1] != self.hidden or not y_expert.is_contiguous():
            raise ValueError(f"y_expert must be a contiguous [rows, {self.hidden}] tensor")
        rm = self._row_map(row_map, T)
        ntpr = self._ntpr(T, num_tokens_per_rank)
        if y_expert.shape[0] < round_up4(ntpr) * self.topk:
            raise ValueError("y_expert needs round_up4(num_tokens_per_rank) * topk rows")
        L.check(self._lib.moe_combine(self._ctx, y_expert.data_ptr(), rm.data_ptr(), s_ptr,
                                      T, ntpr, _stream(self.device), self._out_ref),
                "moe_combine")
        return self._cached(("y", T), lambda: self.y[:T])

    # -- backward ----------------------------------------------------------
    def _expert_rows(self, t: torch.Tensor, name: str, ntpr: int) -> torch.Tensor:
        if t.device != self.device or t.dtype != self.dtype:
            raise TypeError(f"{name} must match the dispatcher's device and dtype")
        if t.dim() != 2 or t.shape[1] != self.hidden or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [rows, {self.hidden}] tensor")
        if t.shape[0] < round_up4(ntpr) * self.topk:
            raise ValueError(f"{name} needs round_up4(num_tokens_per_rank) * topk rows")
        return t

    def _row_map(self, rm: torch.Tensor, T: int) -> torch.Tensor:
        if (rm.dtype != torch.int32 or not rm.is_cuda or rm.get_device() != self._dev_index
                or not rm.is_contiguous()):
            raise ValueError("row_map must be a contiguous int32 tensor on the device")
        if rm.dim() != 2 or rm.shape[1] != self.topk or rm.shape[0] < T:
            raise ValueError(f"row_map must be [>= T, {self.topk}]")
        return rm

    def combine_backward(self, grad_y: torch.Tensor, y_expert: torch.Tensor,
                         row_map: torch.Tensor, topk_scores_TK: torch.Tensor, *,
                         num_tokens_per_rank: Optional[int] = None,
                         total: Optional[torch.Tensor] = None):
        """(dL/dy_expert [round_up4(ntpr)*K, D] view; dL/dscores [T, K] view)
        for dL/dy = grad_y [T, D]. Rows [0, total) of dL/dy_expert are the
        slots' rows. With `total` (a one-element int32 device tensor holding
        the layout's offsets[E], e.g. Layout.offsets[-1:]) the library also
        writes +0.0 into the rows from *total on, which no slot reaches;
        otherwise those rows keep what the buffer held."""
        s = self._dev(topk_scores_TK, "topk_scores_TK", torch.float32, self.topk)
        T = s.shape[0]
        g = self._dev(grad_y, "grad_y", self.dtype, self.hidden)
        if g.shape[0] != T:
            raise ValueError("grad_y and topk_scores_TK need the same T")
        ntpr = self._ntpr(T, num_tokens_per_rank)
        ye = self._expert_rows(y_expert, "y_expert", ntpr)
        rm = self._row_map(row_map, T)
        tot_ptr = 0
        if total is not None:
            if (total.device != self.device or total.dtype != torch.int32
                    or total.numel() != 1 or not total.is_contiguous()):
                raise ValueError("total must be a one-element int32 tensor on the device")
            tot_ptr = total.data_ptr()
        out_e, out_s = C.c_void_p(), C.c_void_p()
        L.check(self._lib.moe_combine_backward(self._ctx, g.data_ptr(), ye.data_ptr(),
                                               rm.data_ptr(), s.data_ptr(), tot_ptr, T, ntpr,
                                               _stream(self.device), C.byref(out_e),
                                               C.byref(out_s)), "moe_combine_backward")
        return self.g_e[:round_up4(ntpr) * self.topk], self.g_s[:T]

    def dispatch_backward(self, grad_x_expert: torch.Tensor, row_map: torch.Tensor, T: int, *,
                          num_tokens_per_rank: Optional[int] = None) -> torch.Tensor:
        """dL/dx [T, D] (a view) for dL/dx_expert = grad_x_expert."""
        ntpr = self._ntpr(T, num_tokens_per_rank)
        h = self._expert_rows(grad_x_expert, "grad_x_expert", ntpr)
        rm = self._row_map(row_map, T)
        out = C.c_void_p()
        L.check(self._lib.moe_dispatch_backward(self._ctx, h.data_ptr(), rm.data_ptr(), T, ntpr,
                                                _stream(self.device), C.byref(out)),
                "moe_dispatch_backward")
        return self.g_x[:T]

    # -- tuning ------------------------------------------------------------
    def set_tuning(self, dispatch_segments: int = 0, combine_segments: int = 0,
                   dispatch_nontemporal: Optional[bool] = None,
                   combine_nontemporal: Optional[bool] = None,
                   dispatch_block_waves: int = 0, combine_block_waves: int = 0,
                   combine_store_nontemporal: Optional[bool] = None,
                   layout_launches: int = 0, dispatch_store_burst: int = 0,
                   combine_backward_store: int = 0, dispatch_x_nontemporal: int = 0) -> None:
        """Launch shape only; results never depend on it. 0 / None keep the
        current value; layout_launches 1 or 2 forces one or two layout
        launches (-1 chooses by size); dispatch_store_burst 1 or 2 selects
        back-to-back or paced dispatch stores; combine_backward_store 1 or 2
        selects streaming or ordinary stores of dL/dy_e; dispatch_x_nontemporal
        1 or 2 selects streaming or ordinary loads of x in dispatch."""
        cur = self.get_tuning()
        dnt = cur["dispatch_nontemporal"] if dispatch_nontemporal is None else dispatch_nontemporal
        cnt = cur["combine_nontemporal"] if combine_nontemporal is None else combine_nontemporal
        snt = -1 if combine_store_nontemporal is None else int(combine_store_nontemporal)
        t = L.MoeTuning(dispatch_segments, combine_segments, int(dnt), int(cnt),
                        dispatch_block_waves, combine_block_waves, snt, layout_launches,
                        dispatch_store_burst, combine_backward_store, dispatch_x_nontemporal)
        L.check(self._lib.moe_set_tuning(self._ctx, C.byref(t)), "moe_set_tuning")

    def get_tuning(self) -> dict:
        t = L.MoeTuning()
        L.check(self._lib.moe_get_tuning(self._ctx, C.byref(t)), "moe_get_tuning")
        return {"dispatch_segments": t.dispatch_segments, "combine_segments": t.combine_segments,
                "dispatch_nontemporal": bool(t.dispatch_nontemporal),
                "combine_nontemporal": bool(t.combine_nontemporal),
                "dispatch_block_waves": t.dispatch_block_waves,
                "combine_block_waves": t.combine_block_waves,
                "combine_store_nontemporal": bool(t.combine_store_nontemporal),
                "layout_launches": t.layout_launches,
                "dispatch_store_burst": t.dispatch_store_burst,
                "combine_backward_store": t.combine_backward_store,
                "dispatch_x_nontemporal": t.dispatch_x_nontemporal}
