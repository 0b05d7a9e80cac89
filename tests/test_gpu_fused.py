"""GPU parity of moe_layout_dispatch, the layout fused into dispatch (two
launches): every buffer it writes equals, bit for bit, what moe_layout
followed by moe_dispatch writes on the same inputs, and the oracle's layout
and dispatch. Covers the workload shapes, padding, edge cases, launch shapes,
repeated calls (the completion counter returns to zero), graph replays with
fresh routing and a poisoned workspace."""
import gc

import numpy as np
import pytest
import torch

import oracle
import workloads
from combine_moe_layout_05_amd import MoeDispatcher, round_up4

from gpu_util import (DEV, ORACLE_THREADS, assert_dispatch_equal, assert_layout_equal, f32_dev,
                      i32_dev, note, sync_or_fail, torch_dtype, x_to_dev, x_to_np)

pytestmark = pytest.mark.gpu


def _free():
    gc.collect()
    torch.cuda.empty_cache()


def _read(disp, ntpr, copy_x_e=True):
    sync_or_fail()
    total = int(disp.offsets[-1].item())
    n4 = round_up4(ntpr)
    out = {"counts": disp.counts.cpu().numpy(), "offsets": disp.offsets.cpu().numpy(),
           "row_map": disp.row_map[:n4].cpu().numpy(), "src": disp.src_map[:total].cpu().numpy(),
           "s_e": disp.s_e[:total].cpu().numpy(), "total": total}
    if copy_x_e:
        out["x_e"] = x_to_np(disp.x_e[:total])
    return out


def _both(disp_a, disp_b, x, ids, scores, T, ntpr, copy_x_e=True):
    """(separate calls on disp_a, fused call on disp_b) read back."""
    x_d = x_to_dev(x[:T]) if T else torch.empty((0, disp_a.hidden), dtype=disp_a.dtype, device=DEV)
    ids_d = i32_dev(ids[:T].reshape(T, disp_a.topk))
    s_d = f32_dev(scores[:T].reshape(T, disp_a.topk))
    lay = disp_a.layout(ids_d, ntpr)
    disp_a.dispatch(x_d, s_d, ids_d, lay.counts, num_tokens_per_rank=ntpr)
    sep = _read(disp_a, ntpr, copy_x_e)
    disp_b.layout_dispatch(x_d, s_d, ids_d, num_tokens_per_rank=ntpr)
    fused = _read(disp_b, ntpr, copy_x_e)
    return sep, fused


def _assert_same(sep, fused):
    assert sep.keys() == fused.keys()
    for k in sep:
        if k == "total":
            assert sep[k] == fused[k]
            continue
        assert sep[k].shape == fused[k].shape, k
        assert np.array_equal(sep[k].view(np.uint8), fused[k].view(np.uint8)), k


def _check(x, ids, scores, T, ntpr, nmax, D, E, K, dtype, tuning=None, copy_x_e=True):
    dt = torch_dtype(x)
    a = MoeDispatcher(nmax, D, E, K, dtype=dt, device=DEV)
    b = MoeDispatcher(nmax, D, E, K, dtype=dt, device=DEV)
    if tuning:
        a.set_tuning(**tuning)
        b.set_tuning(**tuning)
    note(f"fused T={T} ntpr={ntpr} nmax={nmax} D={D} E={E} K={K} {dtype} tuning={tuning}")
    sep, fused = _both(a, b, x, ids, scores, T, ntpr, copy_x_e)
    _assert_same(sep, fused)
    o = oracle.layout(ids, T, ntpr, E, K)
    assert_layout_equal(fused, o, T)
    if copy_x_e:
        x_e, s_e = oracle.dispatch(x[:T], scores[:T].reshape(T, K), K, o["src"],
                                   nthreads=ORACLE_THREADS)
        assert_dispatch_equal(fused, {"x_e": x_e, "s_e": s_e})
    del a, b
    _free()
    return fused


def _x(rng, T, D, dtype):
    xf = rng.standard_normal((max(T, 1), D)).astype(np.float32)
    if dtype == "bf16":
        return torch.from_numpy(xf).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return xf


@pytest.mark.parametrize("name", ["tiny", "padded", "dsv3", "graph"])
def test_workload_shapes(name):
    w = workloads.WORKLOADS[name]
    b = workloads.make_batch(w, T=w.nmax if name == "graph" else None)
    _check(b["x"], b["ids"], b["scores"], w.T, w.ntpr, w.nmax, w.D, w.E, w.K, w.dtype)


@pytest.mark.parametrize("T", workloads.PADDED_T_VALUES)
def test_padded_prefixes(T):
    w = workloads.WORKLOADS["padded"]
    b = workloads.make_batch(w)
    _check(b["x"], b["ids"], b["scores"], T, w.ntpr, w.nmax, w.D, w.E, w.K, w.dtype)


def test_prefill_layout_and_sampled_rows():
    # 262144 slots: the 1024-slot tiles; x_e (3.76 GB) compared on sampled rows
    w = workloads.WORKLOADS["prefill32k_zipf"]
    b = workloads.make_batch(w)
    a = MoeDispatcher(w.nmax, w.D, w.E, w.K, dtype=torch.bfloat16, device=DEV)
    note("fused prefill32k_zipf: separate path")
    x_d = x_to_dev(b["x"])
    ids_d = i32_dev(b["ids"])
    s_d = f32_dev(b["scores"])
    lay = a.layout(ids_d, w.ntpr)
    a.dispatch(x_d, s_d, ids_d, lay.counts, num_tokens_per_rank=w.ntpr)
    sep = _read(a, w.ntpr, copy_x_e=False)
    rng = np.random.default_rng(7)
    rows = np.sort(rng.choice(sep["total"], size=4096, replace=False))
    sep_rows = x_to_np(a.x_e[torch.from_numpy(rows).to(DEV)])
    a.x_e[:sep["total"]].view(torch.int16).fill_(-1)
    a.row_map.fill_(-7)
    note("fused prefill32k_zipf: fused path on the same context")
    a.layout_dispatch(x_d, s_d, ids_d, num_tokens_per_rank=w.ntpr)
    fused = _read(a, w.ntpr, copy_x_e=False)
    _assert_same(sep, fused)
    assert np.array_equal(x_to_np(a.x_e[torch.from_numpy(rows).to(DEV)]).view(np.uint8),
                          sep_rows.view(np.uint8))
    o = oracle.layout(b["ids"], w.T, w.ntpr, w.E, w.K)
    assert_layout_equal(fused, o, w.T)
    src = o["src"][rows]
    assert np.array_equal(sep_rows.view(np.uint8), b["x"][src // w.K].view(np.uint8))
    del a
    _free()


def test_rows_past_4_gib():
    """40960 tokens of 14 KiB rows (327680 slots, 4.70 GB of x_e): the
    ranking dispatch writes rows past byte offset 2^32. Layout, row map,
    source map and scores against the separate calls and the oracle; sampled
    rows, most of them past 4 GiB, bit for bit against x."""
    w = workloads.Workload("past_4_gib", T=40960, ntpr=40960, nmax=40960, D=7168, E=256, K=8,
                           dtype="bf16", routing="zipf", zipf_s=1.2, scores="sigmoid_norm",
                           seed=3)
    b = workloads.make_batch(w)
    a = MoeDispatcher(w.nmax, w.D, w.E, w.K, dtype=torch.bfloat16, device=DEV)
    x_d, ids_d, s_d = x_to_dev(b["x"]), i32_dev(b["ids"]), f32_dev(b["scores"])
    note("fused past 4 GiB: separate path")
    lay = a.layout(ids_d, w.ntpr)
    a.dispatch(x_d, s_d, ids_d, lay.counts, num_tokens_per_rank=w.ntpr)
    sep = _read(a, w.ntpr, copy_x_e=False)
    row_bytes = w.D * 2
    assert sep["total"] * row_bytes > 1 << 32
    far = (1 << 32) // row_bytes
    rng = np.random.default_rng(9)
    rows = np.unique(np.concatenate([rng.integers(far, sep["total"], 3000),
                                     rng.integers(0, far, 500), [far, sep["total"] - 1]]))
    a.x_e[:sep["total"]].view(torch.int16).fill_(-1)
    a.row_map.fill_(-7)
    note("fused past 4 GiB: fused path on the same context")
    a.layout_dispatch(x_d, s_d, ids_d, num_tokens_per_rank=w.ntpr)
    fused = _read(a, w.ntpr, copy_x_e=False)
    _assert_same(sep, fused)
    o = oracle.layout(b["ids"], w.T, w.ntpr, w.E, w.K)
    assert_layout_equal(fused, o, w.T)
    got = x_to_np(a.x_e[torch.from_numpy(rows).to(DEV)])
    assert np.array_equal(got.view(np.uint8), b["x"][o["src"][rows] // w.K].view(np.uint8))
    del a
    _free()


def test_empty_batch():
    K = 4
    ids = np.zeros((0, K), np.int32)
    for ntpr in (0, 6):
        f = _check(_x(np.random.default_rng(0), 0, 64, "bf16"), ids, np.zeros((0, K), np.float32),
                   0, ntpr, 16, 64, 8, K, "bf16")
        assert f["total"] == 0 and (f["counts"] == 0).all() and (f["offsets"] == 0).all()
        assert (f["row_map"] == -1).all()


def test_no_slot_reaches_an_expert():
    T, K = 37, 4
    ids = np.full((T, K), -1, np.int32)
    f = _check(_x(np.random.default_rng(1), T, 128, "bf16"), ids,
               np.full((T, K), np.nan, np.float32), T, T, 40, 128, 8, K, "bf16")
    assert f["total"] == 0 and (f["row_map"] == -1).all()


def test_out_of_range_and_duplicate_ids():
    rng = np.random.default_rng(3)
    T, E, K = 513, 16, 6
    ids = rng.integers(0, E, size=(T, K)).astype(np.int32)
    m = rng.random((T, K)) < 0.1
    ids[m] = rng.choice(np.array([-1, -7, E, E + 3, 2**31 - 1], np.int32), size=int(m.sum()))
    scores = rng.standard_normal((T, K)).astype(np.float32)
    _check(_x(rng, T, 256, "bf16"), ids, scores, T, 600, 1000, 256, E, K, "bf16")
    _check(_x(rng, T, 64, "f32"), ids, scores, T, T, T, 64, E, K, "f32")


def test_max_experts_and_topk_with_a_hot_expert():
    rng = np.random.default_rng(5)
    T, E, K = 300, 1024, 16
    ids = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    ids[::3, 0] = 7                                  # one expert in a third of the tokens
    _check(_x(rng, T, 64, "bf16"), ids, rng.random((T, K)).astype(np.float32),
           T, T, 300, 64, E, K, "bf16")


def test_single_expert_skewed_tiles():
    # every slot of a long batch on one expert: ranks run across many tiles
    rng = np.random.default_rng(6)
    T, E, K = 5000, 4, 8
    ids = np.zeros((T, K), np.int32)
    ids[rng.random((T, K)) < 0.05] = 3
    _check(_x(rng, T, 64, "bf16"), ids, rng.random((T, K)).astype(np.float32),
           T, T, 5000, 64, E, K, "bf16")


@pytest.mark.parametrize("tuning", [dict(dispatch_segments=1, dispatch_block_waves=1),
                                    dict(dispatch_segments=2, dispatch_block_waves=16),
                                    dict(dispatch_segments=16, dispatch_block_waves=7),
                                    dict(dispatch_segments=3, dispatch_block_waves=5,
                                         dispatch_nontemporal=True)])
def test_launch_shapes(tuning):
    # several tokens per workgroup and tokens split over workgroups
    rng = np.random.default_rng(8)
    T, E, K, D = 777, 64, 8, 1000
    ids = rng.integers(0, E, size=(T, K)).astype(np.int32)
    _check(_x(rng, T, D, "bf16"), ids, rng.random((T, K)).astype(np.float32),
           T, 781, 800, D, E, K, "bf16", tuning=tuning)


def test_repeated_calls_reset_the_counter():
    # many fused calls of different sizes in a row on one context: each one
    # must find its last workgroup, so the counter is back at zero each time
    w = workloads.WORKLOADS["padded"]
    b = workloads.make_batch(w)
    a = MoeDispatcher(w.nmax, w.D, w.E, w.K, dtype=torch.bfloat16, device=DEV)
    f = MoeDispatcher(w.nmax, w.D, w.E, w.K, dtype=torch.bfloat16, device=DEV)
    for T, ntpr in ((2047, 2048), (3, 2048), (614, 4096), (0, 8), (2048, 2048), (13, 13)):
        note(f"fused repeat T={T} ntpr={ntpr}")
        sep, fused = _both(a, f, b["x"], b["ids"], b["scores"], T, ntpr)
        _assert_same(sep, fused)
    del a, f
    _free()


def test_graph_replays_with_fresh_routing():
    # layout+dispatch fused, captured with combine; every replay equals the
    # eager separate path on the same inputs
    rng = np.random.default_rng(11)
    N, D, E, K = 2048, 512, 32, 4
    disp = MoeDispatcher(N, D, E, K, dtype=torch.bfloat16, device=DEV)
    ref = MoeDispatcher(N, D, E, K, dtype=torch.bfloat16, device=DEV)
    x_d = torch.zeros((N, D), dtype=torch.bfloat16, device=DEV)
    ids_d = torch.zeros((N, K), dtype=torch.int32, device=DEV)
    s_d = torch.zeros((N, K), dtype=torch.float32, device=DEV)

    def fill(T):
        x = _x(rng, N, D, "bf16")
        ids = np.stack([rng.permutation(E)[:K] for _ in range(N)]).astype(np.int32)
        ids[T:] = -1
        s = rng.random((N, K)).astype(np.float32)
        s[T:] = 0.0
        x_d.copy_(x_to_dev(x))
        ids_d.copy_(i32_dev(ids))
        s_d.copy_(f32_dev(s))

    fill(N)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        lay, dsp = disp.layout_dispatch(x_d, s_d, ids_d)
        disp.combine(dsp.x_e, lay.row_map, s_d)
    torch.cuda.current_stream().wait_stream(s)
    sync_or_fail()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lay, dsp = disp.layout_dispatch(x_d, s_d, ids_d)
        y = disp.combine(dsp.x_e, lay.row_map, s_d)
    for i, T in enumerate((N, 41, 1000, 2047, 7, N)):
        note(f"fused graph replay {i} T={T}")
        fill(T)
        g.replay()
        sync_or_fail()
        got = _read(disp, N)
        y_got = x_to_np(y)
        rl = ref.layout(ids_d, N)
        ref.dispatch(x_d, s_d, ids_d, rl.counts)
        want = _read(ref, N)
        y_want = x_to_np(ref.combine(ref.x_e, rl.row_map, s_d))
        _assert_same(want, got)
        assert np.array_equal(y_got.view(np.uint8), y_want.view(np.uint8))
    del g, disp, ref
    _free()


def test_poisoned_workspace():
    # only the documented regions are written: rows [0,total) of x_e / s_e /
    # src_map and row_map rows [0, round_up4(ntpr))
    w = workloads.WORKLOADS["padded"]
    b = workloads.make_batch(w)
    T, ntpr = 614, 1001
    d = MoeDispatcher(w.nmax, w.D, w.E, w.K, dtype=torch.bfloat16, device=DEV)
    d.workspace.fill_(0xFF)
    d.layout_dispatch(x_to_dev(b["x"][:T]), f32_dev(b["scores"][:T]), i32_dev(b["ids"][:T]),
                      num_tokens_per_rank=ntpr)
    got = _read(d, ntpr)
    o = oracle.layout(b["ids"], T, ntpr, w.E, w.K)
    assert_layout_equal(got, o, T)
    total, n4 = o["total"], round_up4(ntpr)
    assert bool((d.x_e[total:].view(torch.int16) == -1).all())
    assert bool((d.s_e[total:].view(torch.int32) == -1).all())
    assert bool((d.src_map[total:] == -1).all())
    assert bool((d.row_map[n4:] == -1).all())
    del d
    _free()


def test_two_contexts_interleaved():
    # different counter slots: alternating fused calls on two contexts
    rng = np.random.default_rng(12)
    T, E, K, D = 900, 16, 4, 256
    c1 = MoeDispatcher(T, D, E, K, dtype=torch.bfloat16, device=DEV)
    c2 = MoeDispatcher(T, D, E, K, dtype=torch.bfloat16, device=DEV)
    outs = []
    for c in (c1, c2, c1, c2):
        ids = rng.integers(0, E, size=(T, K)).astype(np.int32)
        x = _x(rng, T, D, "bf16")
        c.layout_dispatch(x_to_dev(x), f32_dev(rng.random((T, K)).astype(np.float32)),
                          i32_dev(ids))
        outs.append((c, ids))
        got = _read(c, T, copy_x_e=False)
        assert_layout_equal(got, oracle.layout(ids, T, T, E, K), T)
    del c1, c2, outs
    _free()


@pytest.mark.parametrize("E", [1, 3, 130])
def test_expert_counts_off_the_quad_grid(E):
    # E not a multiple of 4 (padded histogram rows) and E = 1 (one quad of
    # experts, so the last workgroup's scan splits the tiles into 16 slices)
    rng = np.random.default_rng(20 + E)
    T, K = 3001, 8
    ids = rng.integers(0, E, size=(T, K)).astype(np.int32)
    ids[rng.random((T, K)) < 0.03] = -1
    _check(_x(rng, T, 64, "bf16"), ids, rng.random((T, K)).astype(np.float32),
           T, T, T, 64, E, K, "bf16")


def test_dropping_a_dispatcher_waits_for_its_queued_work():
    """A fused call enqueued on a side stream, the dispatcher dropped right
    after, a new dispatcher created (it takes the lowest free completion-
    counter slot, the one just given back) and a fused call on the main
    stream. Dropping waits for the queued work, so the two launches never
    share a live counter: the side-stream results read before the drop and
    the main-stream results both equal the oracle."""
    w = workloads.WORKLOADS["graph"]
    b = workloads.make_batch(w)
    T = w.T
    ids_d, s_d, x_d = i32_dev(b["ids"]), f32_dev(b["scores"]), x_to_dev(b["x"])
    o = oracle.layout(b["ids"], T, w.ntpr, w.E, w.K)
    side = torch.cuda.Stream(device=DEV)
    side.wait_stream(torch.cuda.current_stream(DEV))
    first = MoeDispatcher(w.nmax, w.D, w.E, w.K, dtype=torch.bfloat16, device=DEV)
    note("fused call on a side stream, then the dispatcher is dropped")
    with torch.cuda.stream(side):
        first.layout_dispatch(x_d, s_d, ids_d)
        row_map_1 = first.row_map[:w.ntpr].clone()
        offsets_1 = first.offsets.clone()
    torch.cuda.current_stream(DEV).wait_stream(side)
    del first
    gc.collect()
    second = MoeDispatcher(w.nmax, w.D, w.E, w.K, dtype=torch.bfloat16, device=DEV)
    note("fused call on the main stream with a new dispatcher")
    second.layout_dispatch(x_d, s_d, ids_d)
    got = _read(second, w.ntpr, copy_x_e=False)
    np.testing.assert_array_equal(row_map_1.cpu().numpy(), o["row_map"])
    np.testing.assert_array_equal(offsets_1.cpu().numpy(), o["offsets"])
    assert_layout_equal(got, o, T)
    second.close()
    with pytest.raises(Exception):
        second.layout(ids_d)                   # a closed dispatcher has no context
    del second
    _free()
