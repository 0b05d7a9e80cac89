"""CPU tests of the C-ABI library's host side: it loads, exports every entry
point include/moe.h declares, and its pure-host logic (capacity helpers,
configuration checks, workspace carve-up, argument validation) behaves as the
pages state. No call here launches a kernel."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import oracle
from combine_moe_layout_05_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


@pytest.fixture(scope="module")
def lib():
    return L.load()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = _declared_functions()
    assert "moe_layout" in names and "moe_dispatch" in names and "moe_combine" in names
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(L.SIGNATURES), "binding and header disagree"


def test_capacity_helpers_agree_with_oracle(lib):
    rng = np.random.default_rng(0)
    for a, b in zip(rng.integers(-3, 10**7, 300), rng.integers(-1, 5000, 300)):
        assert lib.moe_ceil_div(int(a), int(b)) == oracle.ceil_div(int(a), int(b))
    for n in range(-3, 3000):
        assert lib.moe_round_up4(n) == oracle.round_up4(n)
    cases = [(8, 4096, 1, 1), (8, 4097, 2, 4), (1, 32768, 1, 1), (3, 100, 3, 3),
             (0, 5, 1, 1), (2, 5, 0, 1), (-1, 5, 1, 1)]
    for c in cases:
        assert lib.moe_num_max_tokens_pretrain(*c) == oracle.num_max_pretrain(*c)
    for c in [(8192, 2, 2), (8193, 2, 2), (1, 8, 1), (10, 0, 1)]:
        assert lib.moe_num_max_tokens_infer(*c) == oracle.num_max_infer(*c)
    for conf, der in [(0, 1), (-4, -8), (4103, 4104), (4104, 4104), (8192, 4104)]:
        assert (lib.moe_validate_num_max(conf, der) == 0) == (oracle.validate_num_max(conf, der) == 0)
    for T in range(-1, 12):
        for ntpr in range(-1, 12):
            for nmax in range(-1, 12):
                assert (lib.moe_check_capacity(T, ntpr, nmax) == 0) == \
                       (oracle.check_capacity(T, ntpr, nmax) == 0)


def _cfg(nmax=4096, D=7168, E=256, K=8, dtype=L.MOE_BF16, flags=0):
    return L.MoeConfig(nmax, D, E, K, dtype, flags)


def _bytes(lib, cfg):
    n = C.c_size_t(0)
    st = lib.moe_workspace_bytes(C.byref(cfg), C.byref(n))
    return st, n.value


def test_config_validation(lib):
    assert _bytes(lib, _cfg())[0] == L.MOE_OK
    assert _bytes(lib, _cfg(nmax=0))[0] == L.MOE_ERR_CAPACITY
    assert _bytes(lib, _cfg(D=7))[0] == L.MOE_ERR_INVALID_ARG       # 14 B rows
    assert _bytes(lib, _cfg(D=4, dtype=L.MOE_F32))[0] == L.MOE_OK   # 16 B rows
    assert _bytes(lib, _cfg(D=4))[0] == L.MOE_ERR_INVALID_ARG       # 8 B bf16 rows
    assert _bytes(lib, _cfg(E=0))[0] == L.MOE_ERR_INVALID_ARG
    assert _bytes(lib, _cfg(E=L.MOE_MAX_EXPERTS + 1))[0] == L.MOE_ERR_INVALID_ARG
    assert _bytes(lib, _cfg(K=0))[0] == L.MOE_ERR_INVALID_ARG
    assert _bytes(lib, _cfg(K=L.MOE_MAX_TOPK + 1))[0] == L.MOE_ERR_INVALID_ARG
    assert _bytes(lib, _cfg(dtype=7))[0] == L.MOE_ERR_INVALID_ARG
    assert _bytes(lib, _cfg(nmax=2**31 - 1, K=16))[0] == L.MOE_ERR_INVALID_ARG  # int32 rows
    assert _bytes(lib, _cfg(flags=2))[0] == L.MOE_ERR_INVALID_ARG              # unknown flag
    assert _bytes(lib, _cfg(flags=L.MOE_FLAG_BACKWARD))[0] == L.MOE_OK
    assert lib.moe_workspace_bytes(None, None) == L.MOE_ERR_INVALID_ARG


@pytest.mark.parametrize("flags", [0, L.MOE_FLAG_BACKWARD])
@pytest.mark.parametrize("nmax,D,E,K,dtype", [
    (4096, 7168, 256, 8, L.MOE_BF16), (64, 128, 8, 2, L.MOE_F32),
    (4097, 2048, 128, 8, L.MOE_BF16), (32768, 7168, 256, 8, L.MOE_BF16),
    (1, 8, 1, 1, L.MOE_BF16), (8192, 4096, 1024, 16, L.MOE_BF16)])
def test_workspace_carve_up(lib, nmax, D, E, K, dtype, flags):
    cfg = _cfg(nmax, D, E, K, dtype, flags)
    st, nbytes = _bytes(lib, cfg)
    assert st == L.MOE_OK
    fake = 1 << 40                                   # never dereferenced on the host
    ctx = C.c_void_p()
    assert lib.moe_create(C.byref(cfg), fake, nbytes, C.byref(ctx)) == L.MOE_OK
    d = L.MoeBuffersDesc()
    assert lib.moe_workspace_offsets(ctx, C.byref(d)) == L.MOE_OK
    eb = 4 if dtype == L.MOE_F32 else 2
    n4 = oracle.round_up4(nmax)
    assert d.nmax4 == n4 and d.max_rows == n4 * K and d.row_bytes == D * eb
    sizes = {"counts": E * 4, "offsets": (E + 1) * 4, "row_map": n4 * K * 4,
             "src_map": n4 * K * 4, "s_e": n4 * K * 4, "x_e": n4 * K * D * eb,
             "y": n4 * D * eb, "block_hist": d.max_tiles * oracle.round_up4(E) * 4,
             "map_ids": n4 * K * 4, "map_scores": n4 * K * 4, "map_n_experts": n4 * 4}
    if flags & L.MOE_FLAG_BACKWARD:
        sizes.update(g_e=n4 * K * D * eb, g_s=n4 * K * 4, g_x=n4 * D * eb)
    else:
        assert d.g_e == d.g_s == d.g_x == -1
    assert d.max_tiles * d.tile_slots >= n4 * K
    spans = sorted((getattr(d, k), getattr(d, k) + v, k) for k, v in sizes.items())
    for (a0, a1, ka), (b0, b1, kb) in zip(spans, spans[1:]):
        assert a1 <= b0, (ka, kb)                    # no overlap
    for off, _, k in spans:
        assert off % L.MOE_WORKSPACE_ALIGN == 0, k
    assert spans[-1][1] <= d.workspace_bytes == nbytes
    assert lib.moe_destroy(ctx) == L.MOE_OK


def _ctx(lib, cfg):
    st, nbytes = _bytes(lib, cfg)
    ctx = C.c_void_p()
    assert lib.moe_create(C.byref(cfg), 1 << 40, nbytes, C.byref(ctx)) == L.MOE_OK
    d = L.MoeBuffersDesc()
    lib.moe_workspace_offsets(ctx, C.byref(d))
    return ctx, d, nbytes


def test_create_rejects_bad_workspace(lib):
    cfg = _cfg(64, 128, 8, 2, L.MOE_F32)
    st, nbytes = _bytes(lib, cfg)
    ctx = C.c_void_p()
    assert lib.moe_create(C.byref(cfg), 1 << 40, nbytes - 1, C.byref(ctx)) == L.MOE_ERR_WORKSPACE
    assert lib.moe_create(C.byref(cfg), (1 << 40) + 16, nbytes, C.byref(ctx)) == L.MOE_ERR_WORKSPACE
    assert lib.moe_create(C.byref(cfg), None, nbytes, C.byref(ctx)) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_create(C.byref(cfg), 1 << 40, nbytes, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_destroy(None) == L.MOE_OK


def test_calls_reject_bad_arguments_before_enqueueing(lib):
    # Every case below fails a host check, so no kernel is launched.
    cfg = _cfg(4096, 2048, 128, 8, L.MOE_BF16)
    ctx, d, _ = _ctx(lib, cfg)
    base = 1 << 40
    counts = base + d.counts
    row_map = base + d.row_map
    ids = x = s = 1 << 41
    out = C.c_void_p()
    # capacity relation T <= ntpr <= nmax
    assert lib.moe_layout(ctx, ids, 2049, 2048, None) == L.MOE_ERR_CAPACITY
    assert lib.moe_layout(ctx, ids, 10, 4097, None) == L.MOE_ERR_CAPACITY
    assert lib.moe_layout(ctx, ids, -1, 8, None) == L.MOE_ERR_CAPACITY
    assert lib.moe_layout(ctx, None, 5, 8, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_layout(None, ids, 5, 8, None) == L.MOE_ERR_INVALID_ARG
    # dispatch / combine before any layout on this context
    assert lib.moe_dispatch(ctx, x, s, ids, counts, 5, 8, None) == L.MOE_ERR_STATE
    assert lib.moe_combine(ctx, base + d.x_e, row_map, s, 5, 8, None, C.byref(out)) == L.MOE_ERR_STATE
    # counts must be the context's own buffer
    assert lib.moe_dispatch(ctx, x, s, ids, counts + 256, 5, 8, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_dispatch(ctx, None, s, ids, counts, 5, 8, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_dispatch(ctx, x, s, ids, counts, 4097, 4097, None) == L.MOE_ERR_CAPACITY
    assert lib.moe_combine(ctx, None, row_map, s, 5, 8, None, C.byref(out)) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_combine(ctx, base + d.x_e, row_map, s, 5, 8, None, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_combine(ctx, base + d.x_e, row_map, s, 9, 8, None, C.byref(out)) == L.MOE_ERR_CAPACITY
    # alignment: 16 bytes for hidden-state rows, 4 for int32 / float32 arrays
    assert lib.moe_layout(ctx, ids + 2, 5, 8, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_dispatch(ctx, x + 8, s, ids, counts, 5, 8, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_dispatch(ctx, x, s + 2, ids, counts, 5, 8, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_dispatch(ctx, x, s, ids + 1, counts, 5, 8, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_combine(ctx, base + d.x_e + 4, row_map, s, 5, 8, None,
                           C.byref(out)) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_combine(ctx, base + d.x_e, row_map + 2, s, 5, 8, None,
                           C.byref(out)) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_combine(ctx, base + d.x_e, row_map, s + 1, 5, 8, None,
                           C.byref(out)) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_layout_dispatch(ctx, x + 8, s, ids, 5, 8, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_layout_dispatch(ctx, x, s, ids + 2, 5, 8, None) == L.MOE_ERR_INVALID_ARG
    lib.moe_destroy(ctx)


def test_backward_calls_need_the_flag_and_a_matching_layout(lib):
    out_e, out_s, out_x = C.c_void_p(), C.c_void_p(), C.c_void_p()
    p = 1 << 41
    ctx, d, _ = _ctx(lib, _cfg(4096, 2048, 128, 8, L.MOE_BF16))
    assert lib.moe_combine_backward(ctx, p, p, p, p, None, 5, 8, None, C.byref(out_e),
                                    C.byref(out_s)) == L.MOE_ERR_UNSUPPORTED
    assert lib.moe_dispatch_backward(ctx, p, p, 5, 8, None, C.byref(out_x)) == L.MOE_ERR_UNSUPPORTED
    lib.moe_destroy(ctx)
    ctx, d, _ = _ctx(lib, _cfg(4096, 2048, 128, 8, L.MOE_BF16, L.MOE_FLAG_BACKWARD))
    rm = (1 << 40) + d.row_map
    assert lib.moe_combine_backward(ctx, p, p, rm, p, p, 5, 8, None, C.byref(out_e),
                                    C.byref(out_s)) == L.MOE_ERR_STATE
    assert lib.moe_dispatch_backward(ctx, p, rm, 5, 8, None, C.byref(out_x)) == L.MOE_ERR_STATE
    assert lib.moe_combine_backward(ctx, p, p, p, p, p, 9, 8, None, C.byref(out_e),
                                    C.byref(out_s)) == L.MOE_ERR_CAPACITY
    assert lib.moe_combine_backward(ctx, None, p, p, p, p, 5, 8, None, C.byref(out_e),
                                    C.byref(out_s)) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_combine_backward(ctx, p, p, p, p, None, 5, 8, None, None,
                                    C.byref(out_s)) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_dispatch_backward(ctx, None, p, 5, 8, None, C.byref(out_x)) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_dispatch_backward(ctx, p, p, 5, 4097, None, C.byref(out_x)) == L.MOE_ERR_CAPACITY
    # alignment (checked before the layout state)
    for args in [(p + 8, p, rm, p, p), (p, p + 8, rm, p, p), (p, p, rm + 2, p, p),
                 (p, p, rm, p + 2, p), (p, p, rm, p, p + 1)]:
        assert lib.moe_combine_backward(ctx, *args, 5, 8, None, C.byref(out_e),
                                        C.byref(out_s)) == L.MOE_ERR_INVALID_ARG, args
    assert lib.moe_dispatch_backward(ctx, p + 4, rm, 5, 8, None, C.byref(out_x)) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_dispatch_backward(ctx, p, rm + 2, 5, 8, None, C.byref(out_x)) == L.MOE_ERR_INVALID_ARG
    lib.moe_destroy(ctx)


def test_variant_calls_reject_bad_arguments(lib):
    ctx, d, _ = _ctx(lib, _cfg(4096, 2048, 128, 8, L.MOE_BF16))
    p = 1 << 41
    o1, o2, o3 = C.c_void_p(), C.c_void_p(), C.c_void_p()
    assert lib.moe_topk_from_routing_map(ctx, p, p, 4097, None, C.byref(o1), C.byref(o2),
                                         C.byref(o3)) == L.MOE_ERR_CAPACITY
    assert lib.moe_topk_from_routing_map(ctx, p, p, -1, None, C.byref(o1), C.byref(o2),
                                         C.byref(o3)) == L.MOE_ERR_CAPACITY
    assert lib.moe_topk_from_routing_map(ctx, None, p, 5, None, C.byref(o1), C.byref(o2),
                                         C.byref(o3)) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_topk_from_routing_map(ctx, p, p, 5, None, None, C.byref(o2),
                                         C.byref(o3)) == L.MOE_ERR_INVALID_ARG
    counts = (1 << 40) + d.counts
    assert lib.moe_dispatch_scaled(ctx, p, p, p, counts, 5, 8, None) == L.MOE_ERR_STATE
    assert lib.moe_dispatch_scaled(ctx, p, p, p, counts + 4, 5, 8, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_dispatch_scaled(ctx, p, None, p, counts, 5, 8, None) == L.MOE_ERR_INVALID_ARG
    lib.moe_destroy(ctx)


def test_fused_layout_dispatch_rejects_bad_arguments(lib):
    ctx, d, _ = _ctx(lib, _cfg(4096, 2048, 128, 8, L.MOE_BF16))
    p = 1 << 41
    assert lib.moe_layout_dispatch(ctx, p, p, p, 4097, 4097, None) == L.MOE_ERR_CAPACITY
    assert lib.moe_layout_dispatch(ctx, p, p, p, 9, 8, None) == L.MOE_ERR_CAPACITY
    assert lib.moe_layout_dispatch(ctx, p, p, p, -1, 8, None) == L.MOE_ERR_CAPACITY
    for bad in ((None, p, p), (p, None, p), (p, p, None)):
        assert lib.moe_layout_dispatch(ctx, *bad, 5, 8, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_layout_dispatch(None, p, p, p, 5, 8, None) == L.MOE_ERR_INVALID_ARG
    lib.moe_destroy(ctx)


def test_fused_counter_slots_run_out_and_come_back(lib):
    # Each context holds one of 1024 completion-counter slots from create to
    # destroy. The slot is checked before the pointers, so a call with a NULL
    # x tells the two cases apart without enqueueing anything: no slot gives
    # MOE_ERR_UNSUPPORTED, a slot MOE_ERR_INVALID_ARG.
    p = 1 << 41
    cfg = _cfg(64, 128, 8, 2, L.MOE_F32)
    made = []
    try:
        for _ in range(1100):
            c, _, _ = _ctx(lib, cfg)
            made.append(c)
            if lib.moe_layout_dispatch(c, None, p, p, 5, 8, None) == L.MOE_ERR_UNSUPPORTED:
                break
        else:
            pytest.fail("contexts never ran out of counter slots")
        assert len(made) <= 1025
        first = made.pop(0)
        assert lib.moe_layout_dispatch(first, None, p, p, 5, 8, None) == L.MOE_ERR_INVALID_ARG
        lib.moe_destroy(first)                      # its slot becomes free again
        c, _, _ = _ctx(lib, cfg)
        made.append(c)
        assert lib.moe_layout_dispatch(c, None, p, p, 5, 8, None) == L.MOE_ERR_INVALID_ARG
    finally:
        for c in made:
            lib.moe_destroy(c)


def test_grouped_gemm_rejects_bad_arguments(lib):
    p = 1 << 41                                   # 16-byte aligned, never dereferenced
    ok = dict(x=p, w=p, off=p, E=256, rows=32768, k=7168, n=4096, out=p, tile=0, lay=0)

    def call(**kw):
        a = dict(ok, **kw)
        return lib.moe_grouped_gemm(a["x"], a["w"], a["off"], a["E"], a["rows"], a["k"], a["n"],
                                    a["out"], a["tile"], a["lay"], None)

    bad = L.MOE_ERR_INVALID_ARG
    for kw in (dict(E=0), dict(E=1025), dict(rows=-1), dict(rows=1 << 31), dict(k=0), dict(k=12),
               dict(n=4), dict(n=4100), dict(tile=32), dict(tile=96), dict(lay=2), dict(lay=-1),
               dict(x=None), dict(w=None), dict(off=None), dict(out=None), dict(x=p + 8),
               dict(w=p + 4), dict(out=p + 2), dict(off=p + 2),
               # more workgroups than one launch may have
               dict(rows=(1 << 31) - 1, n=1 << 14, tile=64)):
        assert call(**kw) == bad, kw
    # nothing to do: accepted without touching the (null) buffers
    assert call(rows=0, x=None, w=None, off=None, out=None) == L.MOE_OK
    assert call(rows=0, x=None, w=None, off=None, out=None, lay=1) == L.MOE_OK


def test_tiled_weight_size_and_argument_checks(lib):
    # E * ceil(n/32)*32 * ceil(k/64)*64 * 2 bytes (zero padded)
    for E, n, k in ((256, 4096, 7168), (5, 200, 72), (1, 8, 8), (1024, 8, 64)):
        assert lib.moe_tiled_weights_bytes(E, n, k) == E * (-(-n // 32) * 32) * (-(-k // 64) * 64) * 2
    for E, n, k in ((0, 8, 8), (1025, 8, 8), (1, 4, 8), (1, 8, 12), (1, 8, 0)):
        assert lib.moe_tiled_weights_bytes(E, n, k) == -1
    p = 1 << 41
    bad = L.MOE_ERR_INVALID_ARG
    assert lib.moe_tile_expert_weights(None, 4, 64, 64, p, None) == bad
    assert lib.moe_tile_expert_weights(p, 4, 64, 64, None, None) == bad
    assert lib.moe_tile_expert_weights(p + 8, 4, 64, 64, p, None) == bad
    assert lib.moe_tile_expert_weights(p, 4, 60, 64, p, None) == bad
    assert lib.moe_tile_expert_weights(p, 0, 64, 64, p, None) == bad


def test_tuning_roundtrip_and_limits(lib):
    ctx, _, _ = _ctx(lib, _cfg())
    t = L.MoeTuning()
    assert lib.moe_get_tuning(ctx, C.byref(t)) == L.MOE_OK
    assert 1 <= t.dispatch_segments <= 16 and 1 <= t.combine_segments <= 16
    assert 1 <= t.dispatch_block_waves <= 16 and 1 <= t.combine_block_waves <= 16
    # 7168 bf16 = 896 chunks: 14 one-chunk segments; a dispatch workgroup per token row
    assert (t.dispatch_segments, t.dispatch_block_waves, t.combine_block_waves) == (14, 14, 16)
    assert t.combine_store_nontemporal == 0          # 58.7 MB output: stays cacheable
    assert t.layout_launches == -1                   # layout launches chosen by size
    assert t.dispatch_store_burst == 2               # dispatch stores paced by default
    assert t.combine_backward_store == 2             # 470 MB of dL/dy_e: ordinary stores
    assert t.dispatch_x_nontemporal == 1             # 470 MB expert buffer: x streamed
    assert lib.moe_set_tuning(ctx, C.byref(L.MoeTuning(4, 3, 1, 1, 2, 16, 1, 2))) == L.MOE_OK
    assert lib.moe_get_tuning(ctx, C.byref(t)) == L.MOE_OK and t.layout_launches == 2
    assert lib.moe_set_tuning(ctx, C.byref(L.MoeTuning(4, 3, 1, 1, 2, 16, 1, 1))) == L.MOE_OK
    assert lib.moe_get_tuning(ctx, C.byref(t)) == L.MOE_OK and t.layout_launches == 1
    assert lib.moe_set_tuning(ctx, C.byref(L.MoeTuning(4, 3, 1, 1, 2, 16, 1, 0, 2))) == L.MOE_OK
    assert lib.moe_get_tuning(ctx, C.byref(t)) == L.MOE_OK
    assert (t.layout_launches, t.dispatch_store_burst) == (1, 2)
    assert lib.moe_get_tuning(ctx, C.byref(t)) == L.MOE_OK
    assert (t.dispatch_segments, t.combine_segments, t.dispatch_nontemporal, t.combine_nontemporal,
            t.dispatch_block_waves, t.combine_block_waves, t.combine_store_nontemporal) == \
        (4, 3, 1, 1, 2, 16, 1)
    assert lib.moe_set_tuning(ctx, C.byref(L.MoeTuning(0, 0, 0, 0, 0, 0, -1))) == L.MOE_OK
    assert lib.moe_get_tuning(ctx, C.byref(t)) == L.MOE_OK
    assert (t.dispatch_segments, t.combine_segments, t.dispatch_nontemporal, t.combine_nontemporal,
            t.dispatch_block_waves, t.combine_block_waves, t.combine_store_nontemporal) == \
        (4, 3, 0, 0, 2, 16, 1)
    assert t.layout_launches == 1                    # 0 keeps the current value
    t.combine_backward_store = 1
    assert lib.moe_set_tuning(ctx, C.byref(t)) == L.MOE_OK
    t.combine_backward_store = 0                     # 0 keeps the current value
    assert lib.moe_set_tuning(ctx, C.byref(t)) == L.MOE_OK
    assert lib.moe_get_tuning(ctx, C.byref(t)) == L.MOE_OK and t.combine_backward_store == 1
    for v in (3, -1):
        t.combine_backward_store = v
        assert lib.moe_set_tuning(ctx, C.byref(t)) == L.MOE_ERR_INVALID_ARG
    t.combine_backward_store = 0
    t.dispatch_x_nontemporal = 2
    assert lib.moe_set_tuning(ctx, C.byref(t)) == L.MOE_OK
    t.dispatch_x_nontemporal = 0                     # 0 keeps the current value
    assert lib.moe_set_tuning(ctx, C.byref(t)) == L.MOE_OK
    assert lib.moe_get_tuning(ctx, C.byref(t)) == L.MOE_OK and t.dispatch_x_nontemporal == 2
    for v in (3, -1):
        t.dispatch_x_nontemporal = v
        assert lib.moe_set_tuning(ctx, C.byref(t)) == L.MOE_ERR_INVALID_ARG
    lib.moe_destroy(ctx)
    ctx, _, _ = _ctx(lib, _cfg(nmax=256, D=1024))    # 4 MB of dL/dy_e: cached
    assert lib.moe_get_tuning(ctx, C.byref(t)) == L.MOE_OK and t.combine_backward_store == 2
    assert t.dispatch_x_nontemporal == 2             # 4 MB expert buffer: x cached
    assert t.dispatch_block_waves == 16              # one-chunk rows: 16-wavefront workgroups
    lib.moe_destroy(ctx)
    ctx, _, _ = _ctx(lib, _cfg(nmax=4096, D=2048, E=128))   # 128 MiB expert buffer, 4 KiB rows
    assert lib.moe_get_tuning(ctx, C.byref(t)) == L.MOE_OK
    assert (t.dispatch_segments, t.dispatch_block_waves) == (4, 16)
    assert t.combine_block_waves == 16               # y cached: 16-wavefront combine workgroups
    lib.moe_destroy(ctx)
    ctx, _, _ = _ctx(lib, _cfg(nmax=8192, D=2048, E=128))   # 256 MiB: one token row
    assert lib.moe_get_tuning(ctx, C.byref(t)) == L.MOE_OK
    assert (t.dispatch_segments, t.dispatch_block_waves) == (4, 4)
    lib.moe_destroy(ctx)
    ctx, _, _ = _ctx(lib, _cfg(nmax=32768))         # 470 MB output: streamed
    assert lib.moe_get_tuning(ctx, C.byref(t)) == L.MOE_OK and t.combine_store_nontemporal == 1
    assert t.combine_backward_store == 1             # 3.76 GB of dL/dy_e: streamed
    assert t.dispatch_x_nontemporal == 2             # 3.76 GB expert buffer: x cached
    assert t.dispatch_block_waves == 4               # and 4-wavefront dispatch workgroups
    assert t.combine_block_waves == 14               # y streamed: a combine workgroup per row
    for bad in ((17, 1, 0, 0, 0, 0, 0), (-1, 1, 0, 0, 0, 0, 0), (1, 1, 0, 0, 17, 0, 0),
                (1, 1, 0, 0, 0, -2, 0), (1, 1, 0, 0, 0, 0, 0, 3), (1, 1, 0, 0, 0, 0, 0, -2),
                (1, 1, 0, 0, 0, 0, 0, 0, 3), (1, 1, 0, 0, 0, 0, 0, 0, -1)):
        assert lib.moe_set_tuning(ctx, C.byref(L.MoeTuning(*bad))) == L.MOE_ERR_INVALID_ARG
    lib.moe_destroy(ctx)


def test_strerror_covers_every_status(lib):
    for st in (0, -1, -2, -3, -4, -5, -6):
        msg = lib.moe_strerror(st).decode()
        assert msg and msg != "unknown status"
    assert lib.moe_strerror(-99).decode() == "unknown status"


def test_product_path_does_not_import_the_oracle():
    pkg = os.path.join(ROOT, "combine_moe_layout_05_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "moe_oracle" not in text and "liborc" not in text, f


def test_layout_noalloc_rejects_bad_arguments_before_any_launch(lib):
    """moe_layout_noalloc checks everything on the host first, so these calls
    return without touching a device (the pointers are never dereferenced):
    sizes, the capacity relation, null pointers, and inputs whose per-tile
    histograms would not fit the static scratch."""
    p = C.c_void_p(1 << 40)
    f = lib.moe_layout_noalloc
    assert f(p, 5, 8, 0, 8, p, p, p, p, None) == L.MOE_ERR_INVALID_ARG        # E = 0
    assert f(p, 5, 8, 1025, 8, p, p, p, p, None) == L.MOE_ERR_INVALID_ARG     # E > max
    assert f(p, 5, 8, 16, 17, p, p, p, p, None) == L.MOE_ERR_INVALID_ARG      # K > max
    assert f(p, 9, 8, 16, 2, p, p, p, p, None) == L.MOE_ERR_CAPACITY          # T > ntpr
    assert f(p, -1, 8, 16, 2, p, p, p, p, None) == L.MOE_ERR_CAPACITY
    assert f(None, 5, 8, 16, 2, p, p, p, p, None) == L.MOE_ERR_INVALID_ARG    # ids, T > 0
    for i in range(4):
        outs = [p, p, p, p]
        outs[i] = None
        assert f(p, 5, 8, 16, 2, *outs, None) == L.MOE_ERR_INVALID_ARG
    assert f(p, 0, (2**31 - 512) // 16 + 4, 16, 16, p, p, p, p, None) == L.MOE_ERR_INVALID_ARG
    odd = (1 << 40) + 2                                                      # not 4-byte aligned
    assert f(odd, 5, 8, 16, 2, p, p, p, p, None) == L.MOE_ERR_INVALID_ARG
    for i in range(4):
        outs = [p, p, p, p]
        outs[i] = odd
        assert f(p, 5, 8, 16, 2, *outs, None) == L.MOE_ERR_INVALID_ARG
    # Scratch: 1024-slot tiles above 65536 slots, one row of round_up4(E)
    # int32 per tile, 4 MiB in all.
    assert L.MOE_NOALLOC_SCRATCH_BYTES == 4 << 20
    assert f(p, 0, 131076, 1024, 8, p, p, p, p, None) == L.MOE_ERR_SCRATCH    # 1025 tiles x 4 KiB
    assert f(p, 0, 524292, 256, 8, p, p, p, p, None) == L.MOE_ERR_SCRATCH     # 4097 tiles x 1 KiB
    assert f(p, 131076, 131076, 1024, 8, p, p, p, p, None) == L.MOE_ERR_SCRATCH
    assert b"static scratch" in lib.moe_strerror(L.MOE_ERR_SCRATCH)
