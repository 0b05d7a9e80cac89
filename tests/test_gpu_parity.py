"""GPU parity of the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs: layout and dispatched data bit-exact, combine within the
stated bar (and, by design, bitwise equal), across the workload shapes, the
unequal/unaligned token counts, padding, edge cases and a poisoned workspace."""
import gc

import numpy as np
import pytest
import torch

import oracle
import workloads
from combine_moe_layout_05_amd import MoeDispatcher, MoeError, round_up4

from gpu_util import (DEV, ORACLE_THREADS, assert_combine_within_bar, assert_dispatch_equal,
                      assert_layout_equal, f32_dev, i32_dev, note, run_gpu, sync_or_fail,
                      torch_dtype, x_to_dev, x_to_np)

pytestmark = pytest.mark.gpu


def _dispatcher(w: workloads.Workload, dtype=None, nmax=None):
    dt = dtype or (torch.bfloat16 if w.dtype == "bf16" else torch.float32)
    return MoeDispatcher(nmax or w.nmax, w.D, w.E, w.K, dtype=dt, device=DEV)


def _free():
    gc.collect()
    torch.cuda.empty_cache()


def _full_check(disp, b, T, ntpr, E, K):
    note(f"T={T} ntpr={ntpr} D={disp.hidden} E={E} K={K} dtype={disp.dtype}")
    g = run_gpu(disp, b["x"], b["ids"], b["scores"], T, ntpr)
    o = oracle.run_pipeline(b["x"], b["ids"], b["scores"], T, ntpr, E, K, nthreads=ORACLE_THREADS)
    assert_layout_equal(g, o, T)
    assert_dispatch_equal(g, o)
    assert_combine_within_bar(g["y"], o["y"])
    assert np.array_equal(g["y"], o["y"]), "combine differs from the oracle bitwise"
    return g, o


# ---------------------------------------------------------------------------
# The workload shapes

def test_tiny_fp32_parity():
    w = workloads.WORKLOADS["tiny"]
    b = workloads.make_batch(w)
    disp = _dispatcher(w)
    _full_check(disp, b, w.T, w.ntpr, w.E, w.K)


@pytest.fixture(scope="module")
def padded():
    w = workloads.WORKLOADS["padded"]
    b = workloads.make_batch(w)
    disp = _dispatcher(w)
    yield w, b, disp
    del disp
    _free()


@pytest.mark.parametrize("T", workloads.PADDED_T_VALUES)
def test_padded_unaligned_parity(padded, T):
    w, b, disp = padded
    _full_check(disp, b, T, w.ntpr, w.E, w.K)


def test_dsv3_parity():
    w = workloads.WORKLOADS["dsv3"]
    b = workloads.make_batch(w)
    disp = _dispatcher(w)
    g, o = _full_check(disp, b, w.T, w.ntpr, w.E, w.K)
    assert g["counts"].argmax() == 0 and g["total"] == w.T * w.K
    del disp
    _free()


@pytest.mark.parametrize("name", ["prefill32k_uniform", "prefill32k_zipf"])
def test_prefill32k_parity(name):
    w = workloads.WORKLOADS[name]
    note(f"{name}: drawing inputs")
    b = workloads.make_batch(w)
    disp = _dispatcher(w)
    note(f"{name}: GPU pipeline")
    g = run_gpu(disp, b["x"], b["ids"], b["scores"], w.T, w.ntpr, copy_x_e=False)
    note(f"{name}: oracle")
    o = oracle.run_pipeline(b["x"], b["ids"], b["scores"], w.T, w.ntpr, w.E, w.K,
                            nthreads=ORACLE_THREADS)
    assert_layout_equal(g, o, w.T)
    assert np.array_equal(g["s_e"].view(np.uint32), o["s_e"].view(np.uint32))
    # x_e is 3.76 GB: compare it in slices of rows.
    step = 1 << 15
    for r0 in range(0, o["total"], step):
        r1 = min(r0 + step, o["total"])
        assert np.array_equal(x_to_np(disp.x_e[r0:r1]), o["x_e"][r0:r1]), (r0, r1)
    assert_combine_within_bar(g["y"], o["y"])
    assert np.array_equal(g["y"], o["y"])
    del disp, o
    _free()


def test_expert_buffer_past_4_gib():
    """40960 tokens of 14 KiB rows (327680 dispatched rows, 4.70 GB of x_e):
    rows past byte offset 2^32 are written by dispatch and read by combine
    (64-bit addressing), and the layout runs its two-launch form at 327680
    slots. Layout, s_e, every x_e row (in slices) and y against the oracle."""
    w = workloads.Workload("past_4_gib", T=40960, ntpr=40960, nmax=40960, D=7168, E=256, K=8,
                           dtype="bf16", routing="zipf", zipf_s=1.2, scores="sigmoid_norm",
                           seed=3)
    note("past 4 GiB: drawing inputs")
    b = workloads.make_batch(w)
    disp = _dispatcher(w)
    assert disp.desc.max_rows * w.D * 2 > 1 << 32
    note("past 4 GiB: GPU pipeline")
    g = run_gpu(disp, b["x"], b["ids"], b["scores"], w.T, w.ntpr, copy_x_e=False)
    note("past 4 GiB: oracle")
    o = oracle.run_pipeline(b["x"], b["ids"], b["scores"], w.T, w.ntpr, w.E, w.K,
                            nthreads=ORACLE_THREADS)
    assert o["total"] == w.T * w.K and o["total"] * w.D * 2 > 1 << 32
    assert_layout_equal(g, o, w.T)
    assert np.array_equal(g["s_e"].view(np.uint32), o["s_e"].view(np.uint32))
    step = 1 << 15
    for r0 in range(0, o["total"], step):
        r1 = min(r0 + step, o["total"])
        assert np.array_equal(x_to_np(disp.x_e[r0:r1]), o["x_e"][r0:r1]), (r0, r1)
    assert np.array_equal(g["y"], o["y"])
    del disp, o
    _free()


def test_graph_shape_full_capacity_parity():
    w = workloads.WORKLOADS["graph"]
    b = workloads.make_batch(w, T=w.nmax, seed=w.seed + 1)
    disp = _dispatcher(w)
    _full_check(disp, b, w.T, w.ntpr, w.E, w.K)
    del disp
    _free()


# ---------------------------------------------------------------------------
# Properties that hold at any size

def test_identity_expert_closed_form_dsv3():
    """With identity experts y = (sum_k s_k) x up to fp32 summation error plus
    the final bf16 rounding, independently of the oracle."""
    w = workloads.WORKLOADS["dsv3"]
    b = workloads.make_batch(w)
    disp = _dispatcher(w)
    note("dsv3 closed form")
    g = run_gpu(disp, b["x"], b["ids"], b["scores"], w.T, w.ntpr, copy_x_e=False)
    x = (b["x"].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    s = b["scores"].astype(np.float64)
    y = (g["y"].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    exact = s.sum(axis=1)[:, None] * x
    u = 2.0 ** -24
    bound = (w.K * u / (1 - w.K * u)) * (np.abs(s).sum(axis=1)[:, None] * np.abs(x))
    bound = bound + np.abs(exact) * 2.0 ** -8 * (1 + 1e-6) + 2.0 ** -133
    assert np.all(np.abs(y - exact) <= bound)
    del disp
    _free()


def test_repeat_calls_are_bitwise_identical():
    w = workloads.WORKLOADS["dsv3"]
    b = workloads.make_batch(w)
    disp = _dispatcher(w)
    note("dsv3 determinism")
    a = run_gpu(disp, b["x"], b["ids"], b["scores"], w.T, w.ntpr)
    c = run_gpu(disp, b["x"], b["ids"], b["scores"], w.T, w.ntpr)
    for k in ("counts", "offsets", "row_map", "src", "s_e", "x_e", "y"):
        assert np.array_equal(a[k], c[k]), k
    del disp
    _free()


# ---------------------------------------------------------------------------
# Padding: unequal/unaligned counts reproduce the equal-count run

def test_unequal_counts_reproduce_equal_count_run(padded):
    w, b, disp = padded
    note("padding invariance, full 2048-row run")
    full = run_gpu(disp, b["x"], b["ids"], b["scores"], 2048, 2048, copy_x_e=False)
    for T in workloads.PADDED_T_VALUES:
        note(f"padding invariance T={T}")
        g = run_gpu(disp, b["x"], b["ids"], b["scores"], T, 2048, copy_x_e=False)
        assert np.array_equal(g["y"], full["y"][:T]), T
    for a, c in workloads.PADDED_PAIRS:
        ntpr = round_up4(max(a, c))
        note(f"pair {a}&{c} ntpr={ntpr}")
        ya = run_gpu(disp, b["x"], b["ids"], b["scores"], a, ntpr, copy_x_e=False)["y"]
        yc = run_gpu(disp, b["x"][a:], b["ids"][a:], b["scores"][a:], c, ntpr, copy_x_e=False)["y"]
        assert np.array_equal(ya, full["y"][:a])
        assert np.array_equal(yc, full["y"][a:a + c])


def test_virtual_padding_equals_materialized_padding(padded):
    w, b, disp = padded
    for T in (3, 5, 13, 614):
        n4 = round_up4(2047)
        note(f"virtual vs materialized T={T}")
        virt = run_gpu(disp, b["x"], b["ids"], b["scores"], T, 2047)
        xm = b["x"][:n4].copy()
        xm[T:] = 0
        idm = b["ids"][:n4].copy()
        idm[T:] = -1
        sm = b["scores"][:n4].copy()
        sm[T:] = 0.0
        mat = run_gpu(disp, xm, idm, sm, n4, n4)
        for key in ("counts", "offsets", "src", "row_map", "x_e", "s_e"):
            assert np.array_equal(virt[key], mat[key]), key
        assert np.array_equal(virt["y"], mat["y"][:T])
        assert (mat["y"][T:] == 0).all()


# ---------------------------------------------------------------------------
# Poisoned workspace: nothing reads an unwritten row; nothing writes padding

@pytest.mark.parametrize("name,T", [("tiny", 61), ("padded", 614), ("padded", 5)])
def test_poisoned_workspace(name, T):
    w = workloads.WORKLOADS[name]
    b = workloads.make_batch(w)
    disp = _dispatcher(w)
    disp.workspace.fill_(0xFF)                 # NaN for floats, -1 for int32
    sync_or_fail()
    ntpr = w.ntpr
    note(f"poison {name} T={T}")
    g = run_gpu(disp, b["x"], b["ids"], b["scores"], T, ntpr)
    o = oracle.run_pipeline(b["x"], b["ids"], b["scores"], T, ntpr, w.E, w.K)
    assert_layout_equal(g, o, T)
    assert_dispatch_equal(g, o)
    assert np.array_equal(g["y"], o["y"])
    n4 = round_up4(ntpr)
    total = o["total"]
    # rows past the true total and padding outputs were never written
    tail = disp.x_e[total:n4 * w.K].view(torch.int16) if disp.dtype == torch.bfloat16 \
        else disp.x_e[total:n4 * w.K].view(torch.int32)
    assert bool((tail == -1).all())
    assert bool((disp.s_e[total:].view(torch.int32) == -1).all())
    ytail = disp.y[T:].view(torch.int16) if disp.dtype == torch.bfloat16 else disp.y[T:].view(torch.int32)
    assert bool((ytail == -1).all())
    assert bool((disp.row_map[n4:] == -1).all())      # beyond the current capacity: untouched
    assert bool((disp.src_map[total:] == -1).all())
    del disp
    _free()


# ---------------------------------------------------------------------------
# Edge cases

def _edge(T, ntpr, nmax, D, E, K, dtype, ids, scores=None, seed=0, segments=None, tuning=None):
    rng = np.random.default_rng(seed)
    xf = rng.standard_normal((max(T, 1), D)).astype(np.float32)
    if dtype == "bf16":
        x = torch.from_numpy(xf).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    else:
        x = xf
    if scores is None:
        scores = rng.random((max(T, 1), K)).astype(np.float32)
    disp = MoeDispatcher(nmax, D, E, K, dtype=torch_dtype(x), device=DEV)
    if segments:
        disp.set_tuning(dispatch_segments=segments[0], combine_segments=segments[1],
                        dispatch_nontemporal=bool(segments[2]),
                        combine_nontemporal=bool(segments[2]),
                        dispatch_block_waves=segments[3], combine_block_waves=segments[4],
                        combine_store_nontemporal=bool(segments[2]))
    if tuning:
        disp.set_tuning(**tuning)
    note(f"edge T={T} ntpr={ntpr} nmax={nmax} D={D} E={E} K={K} {dtype} seg={segments} "
         f"tuning={tuning}")
    g = run_gpu(disp, x, ids, scores, T, ntpr)
    o = oracle.run_pipeline(x, ids, scores, T, ntpr, E, K)
    assert_layout_equal(g, o, T)
    assert_dispatch_equal(g, o)
    assert_combine_within_bar(g["y"], o["y"])
    assert np.array_equal(g["y"], o["y"])
    return g, disp


def test_empty_batch():
    K = 4
    ids = np.zeros((0, K), np.int32)
    for ntpr in (0, 6):
        g, disp = _edge(0, ntpr, 16, 64, 8, K, "bf16", ids)
        assert g["total"] == 0 and (g["counts"] == 0).all() and (g["offsets"] == 0).all()
        assert g["row_map"].shape == (round_up4(ntpr), K) and (g["row_map"] == -1).all()
        assert g["y"].shape == (0, 64)


def test_all_slots_without_expert_give_positive_zero():
    T, K = 37, 4
    ids = np.full((T, K), -1, np.int32)
    g, _ = _edge(T, T, 40, 128, 8, K, "bf16", ids, scores=np.full((T, K), np.nan, np.float32))
    assert g["total"] == 0 and (g["y"] == 0).all()


def test_out_of_range_and_duplicate_ids():
    rng = np.random.default_rng(3)
    T, E, K = 513, 16, 6
    ids = rng.integers(0, E, size=(T, K)).astype(np.int32)      # duplicates allowed
    m = rng.random((T, K)) < 0.1
    ids[m] = rng.choice(np.array([-1, -7, E, E + 3, 2**31 - 1], np.int32), size=int(m.sum()))
    scores = rng.standard_normal((T, K)).astype(np.float32)
    scores[ids < 0] = np.nan                   # never read
    _edge(T, 600, 1000, 256, E, K, "bf16", ids, scores=scores)
    _edge(T, T, T, 64, E, K, "f32", ids, scores=scores)


def test_max_experts_and_topk():
    rng = np.random.default_rng(4)
    T, E, K = 300, 1024, 16
    ids = np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int32)
    _edge(T, T, T, 64, E, K, "bf16", ids)


def test_single_expert_single_slot_smallest_row():
    ids = np.zeros((5, 1), np.int32)
    _edge(5, 5, 5, 8, 1, 1, "bf16", ids)        # 16-byte rows
    _edge(5, 7, 9, 4, 1, 1, "f32", ids)


@pytest.mark.parametrize("segments", [(1, 1, 0, 1, 1), (2, 3, 1, 16, 3), (16, 16, 0, 7, 16),
                                      (5, 2, 1, 4, 4), (14, 14, 0, 14, 4)])
def test_ragged_row_and_launch_shapes(segments):
    rng = np.random.default_rng(5)
    T, E, K = 1001, 64, 8
    ids = np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int32)
    ids[rng.random((T, K)) < 0.05] = -1
    _edge(T, 1003, 2048, 200, E, K, "bf16", ids, segments=segments)   # 25 chunks per row
    _edge(T, T, T, 7168, E, K, "bf16", ids, segments=segments)        # 896 chunks per row
    _edge(T, T, T, 36, E, K, "f32", ids, segments=segments)           # 9 chunks per row


@pytest.mark.parametrize("burst", [1, 2])
@pytest.mark.parametrize("name,T", [("tiny", 61), ("padded", 614), ("padded", 2047),
                                    ("dsv3", 4096)])
def test_dispatch_store_schedules(name, T, burst):
    """Both store schedules of the one-chunk dispatch (a wavefront's K row
    stores back to back, or each after the previous one) give the oracle's
    buffers bit for bit."""
    w = workloads.WORKLOADS[name]
    b = workloads.make_batch(w)
    disp = _dispatcher(w)
    disp.set_tuning(dispatch_store_burst=burst)
    assert disp.get_tuning()["dispatch_store_burst"] == burst
    _full_check(disp, b, T, w.ntpr, w.E, w.K)
    del disp
    _free()


@pytest.mark.parametrize("xnt", [1, 2])
@pytest.mark.parametrize("name,T", [("padded", 2047), ("dsv3", 4096), ("graph", 8192)])
def test_dispatch_x_loads(name, T, xnt):
    """Streaming (xnt=1) and ordinary (xnt=2) loads of x in dispatch give the
    oracle's buffers bit for bit."""
    w = workloads.WORKLOADS[name]
    b = workloads.make_batch(w)
    disp = _dispatcher(w)
    default = disp.get_tuning()["dispatch_x_nontemporal"]
    # expert buffer 134 MB (padded): ordinary; 470 / 537 MB: streaming
    assert default == (2 if name == "padded" else 1)
    disp.set_tuning(dispatch_x_nontemporal=xnt)
    assert disp.get_tuning()["dispatch_x_nontemporal"] == xnt
    _full_check(disp, b, T, w.ntpr, w.E, w.K)
    del disp
    _free()


@pytest.mark.parametrize("xnt", [1, 2])
def test_dispatch_x_loads_every_launch_shape(xnt):
    """Both load forms on the multi-chunk copy (rows split into segments of
    several chunks per lane) and the one-chunk copy."""
    rng = np.random.default_rng(10)
    T, E, K = 1001, 64, 8
    ids = np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int32)
    ids[rng.random((T, K)) < 0.05] = -1
    for seg in ((2, 3, 0, 16, 3), (14, 14, 0, 14, 16)):
        _edge(T, 1003, 2048, 200, E, K, "bf16", ids, segments=seg,
              tuning={"dispatch_x_nontemporal": xnt})
        _edge(T, T, T, 7168, E, K, "bf16", ids, segments=seg,
              tuning={"dispatch_x_nontemporal": xnt})
    _edge(T, T, T, 36, E, K, "f32", ids, tuning={"dispatch_x_nontemporal": xnt})


@pytest.mark.parametrize("burst", [1, 2])
def test_dispatch_store_schedules_with_no_expert_slots(burst):
    rng = np.random.default_rng(8)
    T, E, K = 777, 64, 8
    ids = np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int32)
    ids[rng.random((T, K)) < 0.2] = -1
    ids[::5] = -1                                                     # whole tokens with no expert
    _edge(T, 779, 1024, 2048, E, K, "bf16", ids, tuning={"dispatch_store_burst": burst})
    _edge(T, T, T, 7168, E, K, "bf16", ids, tuning={"dispatch_store_burst": burst})


def test_unaligned_capacity_rounds_up():
    rng = np.random.default_rng(6)
    T, E, K = 5, 8, 2
    ids = np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int32)
    g, disp = _edge(T, 5, 4097, 128, E, K, "bf16", ids)
    assert g["row_map"].shape == (8, K) and (g["row_map"][T:] == -1).all()
    assert disp.nmax4 == 4100


def test_non_identity_expert_output():
    """combine reads the caller's expert output, not the dispatched copy."""
    w = workloads.WORKLOADS["padded"]
    b = workloads.make_batch(w)
    disp = _dispatcher(w)
    T, ntpr = 2047, 2048
    x2 = (torch.from_numpy(b["x"][:T].view(np.int16)).view(torch.bfloat16) * 2)
    x2 = x2.view(torch.int16).numpy().view(np.uint16)        # exact doubling
    note("non-identity expert")
    ids_d, s_d = i32_dev(b["ids"][:T]), f32_dev(b["scores"][:T])
    lay = disp.layout(ids_d, ntpr)
    dsp = disp.dispatch(x_to_dev(b["x"][:T]), s_d, ids_d, lay.counts, num_tokens_per_rank=ntpr)
    y_expert = dsp.x_e * 2
    y = disp.combine(y_expert, lay.row_map, s_d, num_tokens_per_rank=ntpr)
    sync_or_fail()
    o = oracle.run_pipeline(x2, b["ids"], b["scores"], T, ntpr, w.E, w.K)
    assert np.array_equal(x_to_np(y), o["y"])
    del disp
    _free()


def test_call_order_and_counts_are_enforced():
    w = workloads.WORKLOADS["tiny"]
    b = workloads.make_batch(w)
    disp = _dispatcher(w)
    ids_d, s_d, x_d = i32_dev(b["ids"]), f32_dev(b["scores"]), x_to_dev(b["x"])
    lay = disp.layout(ids_d[:60], 64)
    with pytest.raises(MoeError):            # T differs from the layout's
        disp.dispatch(x_d, s_d, ids_d, lay.counts, num_tokens_per_rank=64)
    with pytest.raises(MoeError):            # counts not from this context
        disp.dispatch(x_d[:60], s_d[:60], ids_d[:60], lay.counts.clone(), num_tokens_per_rank=64)
    with pytest.raises(MoeError):            # capacity above the lifetime maximum
        disp.layout(ids_d, 65)
    disp.dispatch(x_d[:60], s_d[:60], ids_d[:60], lay.counts, num_tokens_per_rank=64)
    y = disp.combine(disp.x_e, lay.row_map, s_d[:60], num_tokens_per_rank=64)
    sync_or_fail()
    o = oracle.run_pipeline(b["x"], b["ids"], b["scores"], 60, 64, w.E, w.K)
    assert np.array_equal(x_to_np(y), o["y"])


def test_misaligned_rows_are_rejected_and_nothing_runs():
    """Hidden-state rows move as 16-byte vectors: x or expert outputs that start
    at an element offset (a view into a larger buffer) are refused before any
    launch, and the context's previous results stay as they were."""
    w = workloads.WORKLOADS["padded"]
    b = workloads.make_batch(w)
    T = 614
    disp = _dispatcher(w)
    ids_d, s_d, x_d = i32_dev(b["ids"][:T]), f32_dev(b["scores"][:T]), x_to_dev(b["x"][:T])
    lay = disp.layout(ids_d, w.ntpr)
    disp.dispatch(x_d, s_d, ids_d, lay.counts, num_tokens_per_rank=w.ntpr)
    y = disp.combine(disp.x_e, lay.row_map, s_d, num_tokens_per_rank=w.ntpr)
    sync_or_fail()
    # bit patterns: rows of x_e past the total hold whatever the workspace
    # held before, NaN patterns included, which compare unequal as values
    x_e_before, y_before = disp.x_e.view(torch.int16).clone(), y.view(torch.int16).clone()
    big = torch.empty((T * w.D + 8,), dtype=x_d.dtype, device=DEV)
    x_off = big[1:1 + T * w.D].view(T, w.D)          # 2 bytes past a 16-byte boundary
    x_off.copy_(x_d)
    with pytest.raises(MoeError):
        disp.dispatch(x_off, s_d, ids_d, lay.counts, num_tokens_per_rank=w.ntpr)
    rows = disp.x_e.shape[0]
    ye = torch.empty((rows * w.D + 8,), dtype=x_d.dtype, device=DEV)[4:4 + rows * w.D].view(rows, w.D)
    with pytest.raises(MoeError):
        disp.combine(ye, lay.row_map, s_d, num_tokens_per_rank=w.ntpr)
    sync_or_fail()
    assert torch.equal(disp.x_e.view(torch.int16), x_e_before)
    assert torch.equal(y.view(torch.int16), y_before)
