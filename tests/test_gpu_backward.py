"""GPU parity of the backward entry points (moe_combine_backward,
moe_dispatch_backward) against the CPU oracle on the same seeded inputs, and
the pages' bitwise reproduction of the equal-count run in the backward pass.

Bars: the scaled copy dL/dy_e and the gather-sum dL/dx are compared bitwise
(one fp32 product / an fp32 sum in k order, then the element rounding: the
same operations on both sides). dL/dscores is a length-D dot product whose
fp32 evaluation order on the GPU (lane-local, butterfly over lanes, then
wavefronts) is not the oracle's; it is compared with the oracle's exact fp64
value within the fp32 summation bound gamma_D * sum_d |g_d * y_d|,
gamma_D = D u / (1 - D u), u = 2^-24."""
import gc

import numpy as np
import pytest
import torch

import oracle
import workloads
from combine_moe_layout_05_amd import MoeDispatcher, MoeError, round_up4

from gpu_util import (DEV, ORACLE_THREADS, f32_dev, i32_dev, note, sync_or_fail, x_to_dev,
                      x_to_np)

pytestmark = pytest.mark.gpu
U32 = 2.0 ** -24


def _free():
    gc.collect()
    torch.cuda.empty_cache()


def _grad_y(T, D, dtype, seed):
    g = np.random.default_rng(seed).standard_normal((T, D)).astype(np.float32)
    if dtype == "f32":
        return g
    return torch.from_numpy(g).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _f64(a):
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def gpu_backward(disp, x, ids, scores, g, T, ntpr):
    """Forward layout + dispatch, identity expert, then both backward calls."""
    ids_d, s_d = i32_dev(ids[:T]), f32_dev(scores[:T])
    lay = disp.layout(ids_d, ntpr)
    dsp = disp.dispatch(x_to_dev(x[:T]), s_d, ids_d, lay.counts, num_tokens_per_rank=ntpr)
    g_e, g_s = disp.combine_backward(x_to_dev(g[:T]), dsp.x_e, lay.row_map, s_d,
                                     num_tokens_per_rank=ntpr)
    g_x = disp.dispatch_backward(g_e, lay.row_map, T, num_tokens_per_rank=ntpr)
    sync_or_fail()
    total = int(lay.offsets[-1].item())
    return {"g_e": x_to_np(g_e[:total]), "g_s": g_s.cpu().numpy(), "g_x": x_to_np(g_x),
            "row_map": lay.row_map.cpu().numpy(), "total": total}


def oracle_backward(x, ids, scores, g, T, ntpr, E, K):
    lay = oracle.layout(ids[:T], T, ntpr, E, K)
    x_e, _ = oracle.dispatch(x[:T], scores[:T], K, lay["src"], ORACLE_THREADS)
    g_e, g_s = oracle.combine_backward(g[:T], x_e, lay["row_map"], scores[:T], T, K,
                                       ORACLE_THREADS)
    g_x = oracle.dispatch_backward(g_e, lay["row_map"], T, K, ORACLE_THREADS)
    return {"g_e": g_e, "g_s": g_s, "g_x": g_x, "row_map": lay["row_map"],
            "total": lay["total"], "x_e": x_e}


def assert_backward_parity(gb, ob, g, T, K):
    assert gb["total"] == ob["total"]
    np.testing.assert_array_equal(gb["row_map"], ob["row_map"])
    assert np.array_equal(gb["g_e"].view(np.uint8), ob["g_e"].view(np.uint8)), "dL/dy_e"
    assert np.array_equal(gb["g_x"].view(np.uint8), ob["g_x"].view(np.uint8)), "dL/dx"
    # dL/dscores within the fp32 dot-product bound of the exact value
    D = g.shape[1]
    gamma = D * U32 / (1 - D * U32)
    G = _f64(g[:T])
    rm = ob["row_map"][:T]
    got = gb["g_s"].astype(np.float64)
    for t0 in range(0, T, 256):
        t1 = min(T, t0 + 256)
        for k in range(K):
            r = rm[t0:t1, k]
            ok = r >= 0
            mag = np.zeros(t1 - t0)
            if ok.any():
                Y = _f64(ob["x_e"][r[ok]])
                mag[ok] = np.sum(np.abs(G[t0:t1][ok] * Y), axis=1)
            err = np.abs(got[t0:t1, k] - ob["g_s"][t0:t1, k])
            assert np.all(err <= gamma * mag + 1e-30), (t0, k, float(err.max()))
            # no-expert slots: exactly +0.0
            assert np.all(gb["g_s"][t0:t1, k][~ok].view(np.uint32) == 0)


def _case(name, T=None):
    w = workloads.WORKLOADS[name]
    b = workloads.make_batch(w, T=T)
    g = _grad_y(b["ids"].shape[0], w.D, w.dtype, 77)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    disp = MoeDispatcher(w.nmax, w.D, w.E, w.K, dtype=dt, device=DEV, backward=True)
    return w, b, g, disp


def test_backward_tiny_fp32():
    w, b, g, disp = _case("tiny")
    for T in (w.T, 61, 1):
        note(f"backward tiny T={T}")
        gb = gpu_backward(disp, b["x"], b["ids"], b["scores"], g, T, w.ntpr)
        ob = oracle_backward(b["x"], b["ids"], b["scores"], g, T, w.ntpr, w.E, w.K)
        assert_backward_parity(gb, ob, g, T, w.K)


@pytest.mark.parametrize("T", [5, 614, 2047])
def test_backward_padded(T):
    w, b, g, disp = _case("padded")
    note(f"backward padded T={T}")
    gb = gpu_backward(disp, b["x"], b["ids"], b["scores"], g, T, w.ntpr)
    ob = oracle_backward(b["x"], b["ids"], b["scores"], g, T, w.ntpr, w.E, w.K)
    assert_backward_parity(gb, ob, g, T, w.K)
    del disp
    _free()


@pytest.mark.parametrize("name", ["dsv3", "graph"])
def test_backward_full_shapes(name):
    w, b, g, disp = _case(name)
    # dL/dy_e of 470 / 537 MB: ordinary stores by default
    assert disp.get_tuning()["combine_backward_store"] == 2
    note(f"backward {name} T={w.T}")
    gb = gpu_backward(disp, b["x"], b["ids"], b["scores"], g, w.T, w.ntpr)
    ob = oracle_backward(b["x"], b["ids"], b["scores"], g, w.T, w.ntpr, w.E, w.K)
    assert_backward_parity(gb, ob, g, w.T, w.K)
    note(f"backward {name} repeat")
    gb2 = gpu_backward(disp, b["x"], b["ids"], b["scores"], g, w.T, w.ntpr)
    for k in ("g_e", "g_s", "g_x"):
        assert np.array_equal(gb[k], gb2[k]), k          # deterministic
    del disp, ob
    _free()


def test_backward_past_4_gib():
    """40960 tokens of 14 KiB rows (327680 rows, 4.70 GB of dL/dy_e):
    combine_backward writes and reads rows past byte offset 2^32 and
    dispatch_backward gathers them (64-bit addressing). dL/dy_e and dL/dx
    bitwise; dL/dscores within the fp32 dot-product bound on the tokens that
    have a row past 4 GiB."""
    w = workloads.Workload("past_4_gib", T=40960, ntpr=40960, nmax=40960, D=7168, E=256, K=8,
                           dtype="bf16", routing="zipf", zipf_s=1.2, scores="sigmoid_norm",
                           seed=3)
    note("backward past 4 GiB: drawing inputs")
    b = workloads.make_batch(w)
    g = _grad_y(w.T, w.D, w.dtype, 77)
    disp = MoeDispatcher(w.nmax, w.D, w.E, w.K, dtype=torch.bfloat16, device=DEV, backward=True)
    assert disp.get_tuning()["combine_backward_store"] == 1     # 4.70 GB: streaming stores
    note("backward past 4 GiB: GPU")
    gb = gpu_backward(disp, b["x"], b["ids"], b["scores"], g, w.T, w.ntpr)
    del disp
    _free()
    note("backward past 4 GiB: oracle")
    ob = oracle_backward(b["x"], b["ids"], b["scores"], g, w.T, w.ntpr, w.E, w.K)
    row_bytes = w.D * 2
    assert gb["total"] == ob["total"] and ob["total"] * row_bytes > 1 << 32
    np.testing.assert_array_equal(gb["row_map"], ob["row_map"])
    assert np.array_equal(gb["g_e"].view(np.uint8), ob["g_e"].view(np.uint8)), "dL/dy_e"
    assert np.array_equal(gb["g_x"].view(np.uint8), ob["g_x"].view(np.uint8)), "dL/dx"
    rm = ob["row_map"][:w.T].astype(np.int64)
    far = np.nonzero((rm * row_bytes >= 1 << 32).any(axis=1))[0]
    assert far.size > 0
    tokens = far[:: max(1, far.size // 1024)]
    gamma = w.D * U32 / (1 - w.D * U32)
    G = _f64(g[tokens])
    for k in range(w.K):
        r = rm[tokens, k]
        ok = r >= 0
        mag = np.zeros(tokens.size)
        mag[ok] = np.sum(np.abs(G[ok] * _f64(ob["x_e"][r[ok]])), axis=1)
        err = np.abs(gb["g_s"][tokens, k].astype(np.float64) - ob["g_s"][tokens, k])
        assert np.all(err <= gamma * mag + 1e-30), (k, float(err.max()))
    del ob, gb
    _free()


def test_backward_unequal_counts_reproduce_equal_count_run():
    w, b, g, disp = _case("padded")
    note("backward padding invariance, full run")
    full = gpu_backward(disp, b["x"], b["ids"], b["scores"], g, 2048, 2048)
    frm = full["row_map"][:2048]
    for T in workloads.PADDED_T_VALUES:
        note(f"backward padding invariance T={T}")
        gb = gpu_backward(disp, b["x"], b["ids"], b["scores"], g, T, 2048)
        assert np.array_equal(gb["g_s"].view(np.uint32), full["g_s"][:T].view(np.uint32))
        assert np.array_equal(gb["g_x"], full["g_x"][:T])
        rm = gb["row_map"][:T].ravel()
        rf = frm[:T].ravel()
        assert np.array_equal(gb["g_e"][rm[rm >= 0]], full["g_e"][rf[rf >= 0]])
    for a, c in workloads.PADDED_PAIRS:
        ntpr = round_up4(max(a, c))
        note(f"backward pair {a}&{c}")
        ga = gpu_backward(disp, b["x"], b["ids"], b["scores"], g, a, ntpr)
        gc_ = gpu_backward(disp, b["x"][a:], b["ids"][a:], b["scores"][a:], g[a:], c, ntpr)
        assert np.array_equal(ga["g_x"], full["g_x"][:a])
        assert np.array_equal(gc_["g_x"], full["g_x"][a:a + c])
        assert np.array_equal(ga["g_s"], full["g_s"][:a])
        assert np.array_equal(gc_["g_s"], full["g_s"][a:a + c])
    del disp
    _free()


def test_backward_edge_cases():
    rng = np.random.default_rng(9)
    cases = [  # T, ntpr, nmax, D, E, K, dtype, duplicates/oob
        (513, 600, 1000, 256, 16, 6, "bf16", True),
        (300, 300, 300, 64, 1024, 16, "bf16", False),
        (77, 80, 80, 36, 8, 3, "f32", True),
        (123, 123, 130, 200, 32, 8, "bf16", False),
        (9, 9, 9, 8, 1, 1, "bf16", False),
    ]
    for T, ntpr, nmax, D, E, K, dtype, messy in cases:
        if messy:
            ids = rng.integers(0, E, size=(T, K)).astype(np.int32)
            m = rng.random((T, K)) < 0.1
            ids[m] = rng.choice(np.array([-1, E, -3], np.int32), size=int(m.sum()))
        else:
            ids = np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int32)
        ids[0, :] = -1                                   # one token without an expert
        scores = rng.standard_normal((T, K)).astype(np.float32)
        xf = rng.standard_normal((T, D)).astype(np.float32)
        x = xf if dtype == "f32" else \
            torch.from_numpy(xf).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        g = _grad_y(T, D, dtype, 6)
        disp = MoeDispatcher(nmax, D, E, K, dtype=torch.bfloat16 if dtype == "bf16" else torch.float32,
                             device=DEV, backward=True)
        note(f"backward edge T={T} ntpr={ntpr} D={D} E={E} K={K} {dtype}")
        gb = gpu_backward(disp, x, ids, scores, g, T, ntpr)
        ob = oracle_backward(x, ids, scores, g, T, ntpr, E, K)
        assert_backward_parity(gb, ob, g, T, K)
        assert (gb["g_x"][0].view(np.uint8) == 0).all()       # +0.0
        assert (gb["g_s"][0].view(np.uint32) == 0).all()


def test_backward_poisoned_workspace_and_flag():
    w = workloads.WORKLOADS["padded"]
    b = workloads.make_batch(w)
    g = _grad_y(2048, w.D, "bf16", 8)
    disp = MoeDispatcher(w.nmax, w.D, w.E, w.K, dtype=torch.bfloat16, device=DEV, backward=True)
    disp.workspace.fill_(0xFF)
    sync_or_fail()
    T = 614
    note("backward poison T=614")
    gb = gpu_backward(disp, b["x"], b["ids"], b["scores"], g, T, w.ntpr)
    ob = oracle_backward(b["x"], b["ids"], b["scores"], g, T, w.ntpr, w.E, w.K)
    assert_backward_parity(gb, ob, g, T, w.K)
    assert bool((disp.g_e[ob["total"]:].view(torch.int16) == -1).all())   # not written
    assert bool((disp.g_x[T:].view(torch.int16) == -1).all())
    del disp
    plain = MoeDispatcher(64, 128, 8, 2, dtype=torch.float32, device=DEV)
    ids = i32_dev(np.zeros((4, 2), np.int32))
    s = f32_dev(np.ones((4, 2), np.float32))
    lay = plain.layout(ids, 4)
    with pytest.raises(AttributeError):
        plain.g_e
    with pytest.raises(MoeError):
        plain.dispatch_backward(plain.x_e, lay.row_map, 4)
    sync_or_fail()
    _free()


@pytest.mark.parametrize("store", [1, 2])
@pytest.mark.parametrize("T", [614, 2047, 0])
def test_backward_total_zeroes_the_rows_no_slot_reaches(T, store):
    """With the device-side total, moe_combine_backward writes +0.0 into the
    dL/dy_e rows [total, round_up4(ntpr) * K), which no slot reaches, and
    leaves the rows past the current capacity alone (a poisoned workspace
    shows both). The slots' rows stay bitwise equal to the oracle, with
    streaming (store=1) and ordinary (store=2) stores of dL/dy_e."""
    w = workloads.WORKLOADS["padded"]
    b = workloads.make_batch(w)
    g = _grad_y(2048, w.D, "bf16", 8)
    disp = MoeDispatcher(w.nmax, w.D, w.E, w.K, dtype=torch.bfloat16, device=DEV, backward=True)
    assert disp.get_tuning()["combine_backward_store"] == 2     # 134 MB of dL/dy_e: cached
    disp.set_tuning(combine_backward_store=store)
    assert disp.get_tuning()["combine_backward_store"] == store
    disp.workspace.fill_(0xFF)
    sync_or_fail()
    note(f"backward with total, poisoned workspace, T={T}, store={store}")
    ids_d, s_d = i32_dev(b["ids"][:T]), f32_dev(b["scores"][:T])
    x_d = x_to_dev(b["x"][:T]) if T else torch.empty((0, w.D), dtype=torch.bfloat16, device=DEV)
    g_d = x_to_dev(g[:T]) if T else torch.empty((0, w.D), dtype=torch.bfloat16, device=DEV)
    lay = disp.layout(ids_d, w.ntpr)
    dsp = disp.dispatch(x_d, s_d, ids_d, lay.counts, num_tokens_per_rank=w.ntpr)
    total_d = lay.offsets[-1:].clone()
    g_e, _ = disp.combine_backward(g_d, dsp.x_e, lay.row_map, s_d, num_tokens_per_rank=w.ntpr,
                                   total=total_d)
    sync_or_fail()
    rows = round_up4(w.ntpr) * w.K
    total = int(total_d.item())
    assert g_e.shape[0] == rows
    ob = oracle_backward(b["x"], b["ids"], b["scores"], g, T, w.ntpr, w.E, w.K) if T else None
    if T:
        assert total == ob["total"]
        assert np.array_equal(x_to_np(g_e[:total]).view(np.uint8), ob["g_e"].view(np.uint8))
    else:
        assert total == 0
    tail = g_e[total:rows].view(torch.int16)
    assert bool((tail == 0).all()), "rows past the total must be exactly +0.0"
    assert bool((disp.g_e[rows:].view(torch.int16) == -1).all()), "rows past the capacity"
    with pytest.raises(ValueError):
        disp.combine_backward(g_d, dsp.x_e, lay.row_map, s_d, num_tokens_per_rank=w.ntpr,
                              total=lay.offsets)              # not a one-element tensor
    del disp
    _free()
