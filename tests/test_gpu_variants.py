"""GPU parity of the input/weighting variants against the oracle: the
routing-map input format (boolean map [T][E] + probabilities, HybridEP's
convention) converted on the device to the top-k form, and dispatch with the
scores applied followed by a unit-weight combine."""
import gc

import numpy as np
import pytest
import torch

import oracle
import workloads
from combine_moe_layout_05_amd import MoeDispatcher

from gpu_util import DEV, ORACLE_THREADS, f32_dev, i32_dev, note, sync_or_fail, x_to_dev, x_to_np

pytestmark = pytest.mark.gpu


def _free():
    gc.collect()
    torch.cuda.empty_cache()


def _map_from_topk(ids, scores, E):
    T, K = ids.shape
    m = np.zeros((T, E), np.uint8)
    p = np.zeros((T, E), np.float32)
    rows = np.repeat(np.arange(T), K)
    flat = ids.ravel()
    ok = flat >= 0
    m[rows[ok], flat[ok]] = 1
    p[rows[ok], flat[ok]] = scores.ravel()[ok]
    return m, p


@pytest.mark.parametrize("T,E,K,extra", [(4096, 256, 8, 0), (1000, 100, 6, 3), (300, 1024, 16, 0),
                                         (77, 8, 2, 1)])
def test_routing_map_conversion_parity(T, E, K, extra):
    rng = np.random.default_rng(T + E)
    ids = np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int32)
    ids[rng.random((T, K)) < 0.05] = -1
    ids[-5:] = -1                                       # padded rows: all-False, zero probs
    scores = rng.random((T, K)).astype(np.float32)
    m, p = _map_from_topk(ids, scores, E)
    if extra:                                           # rows with more than K experts
        for t in range(0, T, 97):
            m[t, rng.choice(E, size=min(E, K + extra), replace=False)] = 1
    p += (m > 0) * rng.random((T, E)).astype(np.float32) * (p == 0)
    disp = MoeDispatcher(T, 128, E, K, dtype=torch.bfloat16, device=DEV)
    note(f"routing map T={T} E={E} K={K}")
    gi, gs, gn = disp.topk_from_routing_map(torch.from_numpy(m.astype(bool)).to(DEV), f32_dev(p))
    sync_or_fail()
    oi, os_, on = oracle.topk_from_routing_map(m, p, K)
    np.testing.assert_array_equal(gi.cpu().numpy(), oi)
    assert np.array_equal(gs.cpu().numpy().view(np.uint32), os_.view(np.uint32))
    np.testing.assert_array_equal(gn.cpu().numpy(), on)
    del disp
    _free()


@pytest.mark.parametrize("name", ["padded", "dsv3"])
def test_routing_map_end_to_end(name):
    w = workloads.WORKLOADS[name]
    b = workloads.make_batch(w)
    T = w.T - 3
    m, p = _map_from_topk(b["ids"][:T], b["scores"][:T], w.E)
    disp = MoeDispatcher(w.nmax, w.D, w.E, w.K, dtype=torch.bfloat16, device=DEV)
    note(f"routing map end to end {name} T={T}")
    ids_d, s_d, n_d = disp.topk_from_routing_map(torch.from_numpy(m).to(DEV), f32_dev(p))
    lay = disp.layout(ids_d, w.ntpr)
    dsp = disp.dispatch(x_to_dev(b["x"][:T]), s_d, ids_d, lay.counts, num_tokens_per_rank=w.ntpr)
    y = disp.combine(dsp.x_e, lay.row_map, s_d, num_tokens_per_rank=w.ntpr)
    sync_or_fail()
    oi, os_, on = oracle.topk_from_routing_map(m, p, w.K)
    o = oracle.run_pipeline(b["x"], oi, os_, T, w.ntpr, w.E, w.K, nthreads=ORACLE_THREADS)
    np.testing.assert_array_equal(lay.counts.cpu().numpy(), o["counts"])
    np.testing.assert_array_equal(lay.row_map.cpu().numpy(), o["row_map"])
    assert np.array_equal(x_to_np(y), o["y"])
    assert (n_d.cpu().numpy() == w.K).all()
    del disp
    _free()


@pytest.mark.parametrize("name,dtype", [("padded", "bf16"), ("dsv3", "bf16"), ("tiny", "f32")])
def test_scaled_dispatch_and_unit_combine(name, dtype):
    w = workloads.WORKLOADS[name]
    b = workloads.make_batch(w)
    T = w.T - 1
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    disp = MoeDispatcher(w.nmax, w.D, w.E, w.K, dtype=dt, device=DEV)
    note(f"scaled dispatch {name} T={T}")
    ids_d, s_d = i32_dev(b["ids"][:T]), f32_dev(b["scores"][:T])
    lay = disp.layout(ids_d, w.ntpr)
    dsp = disp.dispatch_scaled(x_to_dev(b["x"][:T]), s_d, ids_d, lay.counts,
                               num_tokens_per_rank=w.ntpr)
    y = disp.combine(dsp.x_e, lay.row_map, None, num_tokens_per_rank=w.ntpr, T=T)
    sync_or_fail()
    total = int(lay.offsets[-1].item())
    lo = oracle.layout(b["ids"][:T], T, w.ntpr, w.E, w.K)
    xs = oracle.dispatch_scaled(b["x"][:T], b["scores"][:T], w.K, lo["src"], ORACLE_THREADS)
    assert np.array_equal(x_to_np(dsp.x_e[:total]).view(np.uint8), xs.view(np.uint8))
    assert np.array_equal(disp.s_e[:total].cpu().numpy(), b["scores"][:T].ravel()[lo["src"]])
    yo = oracle.combine(xs, lo["row_map"], np.ones((T, w.K), np.float32), T, w.K, ORACLE_THREADS)
    assert np.array_equal(x_to_np(y), yo)
    del disp
    _free()
