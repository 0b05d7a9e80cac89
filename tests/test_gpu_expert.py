"""GPU parity of the expert step (moe_grouped_gemm) against the CPU oracle.

Bar. Each output is a k_in-long bf16 dot product accumulated in fp32 on the
matrix cores (order not specified) and rounded once to bf16, so against the
oracle's fp64 value v:
    |gpu - v| <= gamma_k * sum_d |x_d * w_d| + 2^-8 * |gpu|
gamma_k = k u / (1 - k u), u = 2^-24 (the fp32 summation bound, any order),
plus the final rounding (unit roundoff 2^-8 of an 8-bit significand). With
scaled identity experts every sum is exact, so the whole layer (layout,
dispatch, expert, combine) is compared bit for bit with the oracle's layer:
the analytic check the uccl page's graph test makes ("Tests").
"""
import gc

import numpy as np
import pytest
import torch

import oracle
import workloads
from combine_moe_layout_05_amd import (MoeDispatcher, MoeError, grouped_gemm, round_up4,
                                       tile_expert_weights)

from gpu_util import DEV, ORACLE_THREADS, f32_dev, i32_dev, note, sync_or_fail, x_to_dev, x_to_np

pytestmark = pytest.mark.gpu
U32 = 2.0 ** -24
POISON = 0xFFFF            # a NaN pattern the kernel never writes (int16 -1)


def _free():
    gc.collect()
    torch.cuda.empty_cache()


def _f64(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _gamma(k):
    return k * U32 / (1 - k * U32)


def _offsets(counts):
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)


def _assert_within_bound(got_bits, exact, mag, k_in, what):
    got = _f64(got_bits)
    assert np.isfinite(got).all(), what
    bound = _gamma(k_in) * mag + 2.0 ** -8 * np.abs(got) + 1e-300
    err = np.abs(got - exact)
    bad = err > bound
    assert not bad.any(), (what, int(bad.sum()), float((err / bound).max()))
    return float(np.mean(got_bits == oracle.f64_to_bf16(exact)))


def _run(x_e, w, off, max_rows, row_tile, out_fill=-1, tiled=False):
    xd, wd = x_to_dev(x_e), x_to_dev(w)
    if tiled:
        wd = tile_expert_weights(wd)
    out = torch.full((max_rows, w.shape[1]), out_fill, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    grouped_gemm(xd, wd, i32_dev(off), out, row_tile=row_tile)
    sync_or_fail()
    return x_to_np(out)


SMALL = [  # E, counts (None = random), k_in, n_out
    (8, None, 256, 384),                    # whole steps, whole feature tiles
    (5, [0, 65, 1, 130, 7], 72, 200),       # ragged k (9 chunks) and features (200)
    (1, [3], 8, 8),                         # one chunk, one partial tile
    (16, [0] * 7 + [300] + [0] * 8, 520, 136),  # one expert with every row
    (300, None, 64, 128),                   # more experts than lanes
    (4, [900, 0, 1300, 300], 200, 72),      # >= 512 rows per expert: tiles dealt in chunks
    (3, [40, 0, 200], 128, 1000),           # a second, partial 512-feature tile
]


@pytest.mark.parametrize("tiled", [False, True])
@pytest.mark.parametrize("row_tile", [64, 128, 0])
@pytest.mark.parametrize("case", range(len(SMALL)))
def test_grouped_gemm_small_shapes(case, row_tile, tiled):
    E, counts, k_in, n_out = SMALL[case]
    rng = np.random.default_rng(100 + case)
    if counts is None:
        counts = rng.integers(0, 90, E)
        counts[rng.random(E) < 0.2] = 0
    off = _offsets(counts)
    total = int(off[-1])
    max_rows = total + 37                    # rows past the total must stay untouched
    x = workloads.expert_rows(max_rows, k_in, 7 + case)
    w = workloads.expert_weights(E, n_out, k_in, 11 + case)
    note(f"grouped_gemm E={E} k_in={k_in} n_out={n_out} total={total} row_tile={row_tile} "
         f"tiled={tiled}")
    got = _run(x, w, off, max_rows, row_tile, tiled=tiled)
    exact = oracle.grouped_gemm(x, w, off, ORACLE_THREADS)
    mag = np.zeros_like(exact)
    ax, aw = np.abs(_f64(x)), np.abs(_f64(w))
    for e in range(E):
        seg = slice(off[e], off[e + 1])
        mag[seg] = ax[seg] @ aw[e].T
    exact_frac = _assert_within_bound(got[:total], exact[:total], mag[:total], k_in, "values")
    assert (got[total:] == POISON).all()
    assert exact_frac > 0.9, exact_frac      # most outputs are the correctly rounded value


def test_grouped_gemm_row_tiles_agree_bitwise_and_repeat():
    E, k_in, n_out = 12, 192, 256
    rng = np.random.default_rng(5)
    off = _offsets(rng.integers(0, 200, E))
    x = workloads.expert_rows(int(off[-1]), k_in, 1)
    w = workloads.expert_weights(E, n_out, k_in, 2)
    note("grouped_gemm row tiles 64 vs 128, row-major vs tiled weights")
    a = _run(x, w, off, int(off[-1]), 64)
    b = _run(x, w, off, int(off[-1]), 128)
    c = _run(x, w, off, int(off[-1]), 64, out_fill=0)
    d = _run(x, w, off, int(off[-1]), 128, tiled=True)
    f = _run(x, w, off, int(off[-1]), 64, tiled=True)
    for other in (b, c, d, f):
        assert np.array_equal(a, other)


@pytest.mark.parametrize("E,n_out,k_in", [(3, 200, 72), (2, 64, 128), (1, 8, 8)])
def test_tiled_weight_layout(E, n_out, k_in):
    """The tiled form against the layout's definition, built with numpy:
    chunk (((e*NB + b)*S + t)*4 + s)*64 + l = w[e][32b + l%32][64t + 32(l//32)
    + 8s : +8], zero past n_out / k_in."""
    w = workloads.expert_weights(E, n_out, k_in, 9)
    NB, S = -(-n_out // 32), -(-k_in // 64)
    pad = np.zeros((E, NB * 32, S * 64), np.uint16)
    pad[:, :n_out, :k_in] = w
    ref = pad.reshape(E, NB, 32, S, 2, 4, 8).transpose(0, 1, 3, 5, 4, 2, 6).reshape(-1)
    note(f"tile layout E={E} n_out={n_out} k_in={k_in}")
    t = tile_expert_weights(x_to_dev(w))
    sync_or_fail()
    got = t.data.cpu().numpy().view(np.uint16)
    assert got.size == ref.size
    assert np.array_equal(got, ref)


def test_grouped_gemm_edge_offsets():
    rng = np.random.default_rng(6)
    E, k_in, n_out = 4, 64, 64
    x = workloads.expert_rows(64, k_in, 3)
    w = workloads.expert_weights(E, n_out, k_in, 4)
    note("grouped_gemm all-empty segments")
    got = _run(x, w, np.zeros(E + 1, np.int32), 64, 0)
    assert (got == POISON).all()
    note("grouped_gemm segments ending at max_rows")
    off = np.array([0, 10, 10, 40, 64], np.int32)
    got = _run(x, w, off, 64, 0)
    exact = oracle.grouped_gemm(x, w, off)
    mag = np.concatenate([np.abs(_f64(x[off[e]:off[e + 1]])) @ np.abs(_f64(w[e])).T
                          for e in range(E)])
    _assert_within_bound(got, exact, mag, k_in, "edge")
    # offsets past max_rows are clamped on the device: nothing outside the
    # buffers is touched (rows written are then unspecified, so not checked)
    note("grouped_gemm offsets past max_rows (clamped)")
    bad = np.array([0, 30, 20, 1000, 70000], np.int32)
    _ = _run(x, w, bad, 64, 0)
    del rng


def test_grouped_gemm_rejects_bad_tensors():
    x = torch.zeros((8, 64), dtype=torch.bfloat16, device=DEV)
    w = torch.zeros((2, 64, 64), dtype=torch.bfloat16, device=DEV)
    off = torch.zeros(3, dtype=torch.int32, device=DEV)
    with pytest.raises(TypeError):
        grouped_gemm(x.float(), w, off)
    with pytest.raises(ValueError):
        grouped_gemm(x, w, off[:2])
    with pytest.raises(MoeError):
        grouped_gemm(x[:, :60].contiguous(), w[:, :, :60].contiguous(), off)   # k_in % 8
    t = tile_expert_weights(w)
    bad = t._replace(data=t.data[:-16])                  # a tiled buffer of the wrong size
    with pytest.raises(ValueError):
        grouped_gemm(x, bad, off)
    with pytest.raises(ValueError):
        grouped_gemm(x, t._replace(n_out=128), off)


def test_grouped_gemm_dsv3_full_size_sampled():
    """The launch the benchmark times: dsv3 routing (T=4096, E=256, K=8,
    hidden 7168) dispatched on the GPU, experts 7168 -> 4096; sampled outputs
    against the oracle's dispatch and dot products."""
    sh = workloads.EXPERT_SHAPES["dsv3"]
    wl = workloads.WORKLOADS[sh["workload"]]
    b = workloads.make_batch(wl)
    k_in, n_out = sh["k_in"], sh["n_out"]
    note("dsv3 expert weights")
    w = workloads.expert_weights(wl.E, n_out, k_in, sh["seed"])
    wd = x_to_dev(w)
    wt = tile_expert_weights(wd)
    disp = MoeDispatcher(wl.nmax, wl.D, wl.E, wl.K, dtype=torch.bfloat16, device=DEV)
    ids_d, s_d = i32_dev(b["ids"]), f32_dev(b["scores"])
    note("dsv3 layout + dispatch + grouped_gemm")
    lay = disp.layout(ids_d, wl.ntpr)
    dsp = disp.dispatch(x_to_dev(b["x"]), s_d, ids_d, lay.counts, num_tokens_per_rank=wl.ntpr)
    max_rows = round_up4(wl.ntpr) * wl.K
    out = torch.full((max_rows, n_out), -1, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    grouped_gemm(dsp.x_e, wt, lay.offsets, out)
    out_rm = torch.full_like(out, 0)
    grouped_gemm(dsp.x_e, wd, lay.offsets, out_rm)
    sync_or_fail(120)
    total = int(lay.offsets[-1].item())
    ov = out.view(torch.int16)
    assert not bool((ov[:total] == -1).any()), "a row of the segments was not written"
    assert bool((ov[total:] == -1).all()), "a row past the total was written"
    # the two weight layouts run the same products in the same order
    assert bool(torch.equal(ov[:total], out_rm.view(torch.int16)[:total]))
    del out_rm
    got_off = lay.offsets.cpu().numpy()

    lo = oracle.layout(b["ids"], wl.T, wl.ntpr, wl.E, wl.K)
    x_e, _ = oracle.dispatch(b["x"], b["scores"], wl.K, lo["src"], ORACLE_THREADS)
    assert np.array_equal(got_off, lo["offsets"])
    rng = np.random.default_rng(3)
    off = lo["offsets"]
    firsts = off[:-1][np.diff(off) > 0]
    lasts = off[1:][np.diff(off) > 0] - 1
    rows = np.concatenate([firsts, lasts, rng.integers(0, total, 3000)]).astype(np.int64)
    cols = np.concatenate([np.zeros(firsts.size), np.full(lasts.size, n_out - 1),
                           rng.integers(0, n_out, 3000)]).astype(np.int64)
    note(f"dsv3 oracle at {rows.size} positions")
    exact = oracle.grouped_gemm_at(x_e, w, off, rows, cols, ORACLE_THREADS)
    owner = np.searchsorted(off, rows, side="right") - 1
    ax = np.abs(_f64(x_e[rows]))
    aw = np.abs(_f64(w[owner, cols]))
    mag = np.sum(ax * aw, axis=1)
    got = x_to_np(out[torch.from_numpy(rows).to(DEV), torch.from_numpy(cols).to(DEV)])
    _assert_within_bound(got, exact, mag, k_in, "dsv3 samples")
    del disp, wd, wt, out, dsp
    _free()


def test_grouped_gemm_dsv3_every_output_against_an_fp32_matmul():
    """Every one of the 134M outputs at the benchmark's shape (DSV3 routing,
    256 experts, 7168 -> 4096, tiled weights), checked against an
    independent fp32 matrix product of each expert's segment (torch on the
    GPU, full fp32 precision). bf16 products are exact in fp32, so both sums
    are within gamma_k * sum|x w| of the exact value; with the final bf16
    rounding: |gpu - ref| <= 2 gamma_k * sum|x w| + 2^-8 |gpu|. The sampled
    oracle test above pins exact values; this one covers every position."""
    sh = workloads.EXPERT_SHAPES["dsv3"]
    wl = workloads.WORKLOADS[sh["workload"]]
    b = workloads.make_batch(wl)
    k_in, n_out = sh["k_in"], sh["n_out"]
    note("dsv3 expert weights (full-size check)")
    wd = x_to_dev(workloads.expert_weights(wl.E, n_out, k_in, sh["seed"]))
    wt = tile_expert_weights(wd)
    disp = MoeDispatcher(wl.nmax, wl.D, wl.E, wl.K, dtype=torch.bfloat16, device=DEV)
    ids_d, s_d = i32_dev(b["ids"]), f32_dev(b["scores"])
    lay = disp.layout(ids_d, wl.ntpr)
    dsp = disp.dispatch(x_to_dev(b["x"]), s_d, ids_d, lay.counts, num_tokens_per_rank=wl.ntpr)
    out = torch.empty((round_up4(wl.ntpr) * wl.K, n_out), dtype=torch.bfloat16, device=DEV)
    note("dsv3 grouped_gemm (full-size check)")
    grouped_gemm(dsp.x_e, wt, lay.offsets, out)
    sync_or_fail(120)
    off = lay.offsets.cpu().numpy()
    gamma = _gamma(k_in)
    prec = torch.get_float32_matmul_precision()
    torch.set_float32_matmul_precision("highest")
    try:
        worst = 0.0
        for e in range(wl.E):
            s0, s1 = int(off[e]), int(off[e + 1])
            if s1 == s0:
                continue
            x = dsp.x_e[s0:s1].float()
            w = wd[e].float()
            ref = x @ w.t()
            mag = x.abs() @ w.abs().t()
            got = out[s0:s1].float()
            err = (got - ref).abs()
            bound = 2 * gamma * mag + 2.0 ** -8 * got.abs()
            ratio = float((err / bound.clamp_min(1e-30)).max())
            worst = max(worst, ratio)
            assert bool((err <= bound).all()), f"expert {e}: error beyond the fp32 bound ({ratio:.3f})"
        sync_or_fail(120)
    finally:
        torch.set_float32_matmul_precision(prec)
    note(f"dsv3 full-size check: worst error / bound = {worst:.3f}")
    del disp, wd, wt, out, dsp
    _free()


def test_grouped_gemm_rows_past_4_gib():
    """40960 tokens dispatched (327680 rows, 4.70 GB of x_e), experts
    7168 -> 4096 with tiled weights: rows past byte offset 2^32 are read, and
    output rows past 2^31 bytes written (64-bit addressing). Rows outside the
    segments untouched; sampled outputs, most of them in rows past 4 GiB of
    x_e, against the oracle's dot products within the fp32 bound."""
    sh = workloads.EXPERT_SHAPES["dsv3"]
    k_in, n_out = sh["k_in"], sh["n_out"]
    wl = workloads.Workload("past_4_gib", T=40960, ntpr=40960, nmax=40960, D=k_in, E=256, K=8,
                            dtype="bf16", routing="zipf", zipf_s=1.2, scores="sigmoid_norm",
                            seed=3)
    b = workloads.make_batch(wl)
    note("past 4 GiB: expert weights")
    w = workloads.expert_weights(wl.E, n_out, k_in, sh["seed"])
    wt = tile_expert_weights(x_to_dev(w))
    disp = MoeDispatcher(wl.nmax, wl.D, wl.E, wl.K, dtype=torch.bfloat16, device=DEV)
    ids_d, s_d = i32_dev(b["ids"]), f32_dev(b["scores"])
    note("past 4 GiB: layout + dispatch + grouped_gemm")
    lay = disp.layout(ids_d, wl.ntpr)
    dsp = disp.dispatch(x_to_dev(b["x"]), s_d, ids_d, lay.counts, num_tokens_per_rank=wl.ntpr)
    max_rows = round_up4(wl.ntpr) * wl.K
    out = torch.full((max_rows, n_out), -1, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    grouped_gemm(dsp.x_e, wt, lay.offsets, out)
    sync_or_fail(120)
    total = int(lay.offsets[-1].item())
    row_bytes = k_in * 2
    assert total * row_bytes > 1 << 32
    ov = out.view(torch.int16)
    assert not bool((ov[:total] == -1).any()), "a row of the segments was not written"
    assert bool((ov[total:] == -1).all()), "a row past the total was written"
    got_off = lay.offsets.cpu().numpy()
    del wt
    lo = oracle.layout(b["ids"], wl.T, wl.ntpr, wl.E, wl.K)
    x_e, _ = oracle.dispatch(b["x"], b["scores"], wl.K, lo["src"], ORACLE_THREADS)
    off = lo["offsets"]
    assert np.array_equal(got_off, off)
    rng = np.random.default_rng(4)
    far = (1 << 32) // row_bytes                       # first row past 4 GiB of x_e
    rows = np.concatenate([rng.integers(far, total, 3000), rng.integers(0, far, 500),
                           [far, total - 1]]).astype(np.int64)
    cols = np.concatenate([rng.integers(0, n_out, 3500), [0, n_out - 1]]).astype(np.int64)
    note(f"past 4 GiB: oracle at {rows.size} positions")
    exact = oracle.grouped_gemm_at(x_e, w, off, rows, cols, ORACLE_THREADS)
    owner = np.searchsorted(off, rows, side="right") - 1
    mag = np.sum(np.abs(_f64(x_e[rows])) * np.abs(_f64(w[owner, cols])), axis=1)
    got = x_to_np(out[torch.from_numpy(rows).to(DEV), torch.from_numpy(cols).to(DEV)])
    _assert_within_bound(got, exact, mag, k_in, "rows past 4 GiB")
    del disp, out, dsp
    _free()


def _identity_experts(E, D):
    c = 2.0 ** (np.arange(E) % 5 - 2)
    w = np.zeros((E, D, D), np.uint16)
    for e in range(E):
        w[e][np.arange(D), np.arange(D)] = oracle.f64_to_bf16(np.array([c[e]]))[0]
    return w


def _dyadic_batch(T, D, E, K, seed):
    rng = np.random.default_rng(seed)
    ids = np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int32)
    ids[rng.random((T, K)) < 0.1] = -1
    x = oracle.f64_to_bf16(rng.integers(-128, 129, (T, D)) / 16.0)
    scores = (2.0 ** -rng.integers(0, 3, (T, K)) * rng.choice([-1, 1], (T, K))).astype(np.float32)
    return x, ids, scores


def _gpu_layer(disp, x, ids, scores, wd, T, ntpr, h):
    ids_d, s_d = i32_dev(ids[:T]), f32_dev(scores[:T])
    lay = disp.layout(ids_d, ntpr)
    dsp = disp.dispatch(x_to_dev(x[:T]), s_d, ids_d, lay.counts, num_tokens_per_rank=ntpr)
    n = round_up4(ntpr) * disp.topk
    grouped_gemm(dsp.x_e[:n], wd, lay.offsets, h[:n])
    return disp.combine(h[:n], lay.row_map, s_d, num_tokens_per_rank=ntpr)


@pytest.mark.parametrize("tiled", [False, True])
@pytest.mark.parametrize("T,ntpr", [(614, 2048), (2047, 2048), (5, 8)])
def test_layer_with_scaled_identity_experts_is_exact(T, ntpr, tiled):
    nmax, D, E, K = 2048, 512, 64, 8
    x, ids, scores = _dyadic_batch(nmax, D, E, K, 21)
    w = _identity_experts(E, D)
    wd = x_to_dev(w)
    if tiled:
        wd = tile_expert_weights(wd)
    disp = MoeDispatcher(nmax, D, E, K, dtype=torch.bfloat16, device=DEV)
    h = torch.empty((round_up4(nmax) * K, D), dtype=torch.bfloat16, device=DEV)
    note(f"layer scaled identity T={T} ntpr={ntpr} tiled={tiled}")
    y = x_to_np(_gpu_layer(disp, x, ids, scores, wd, T, ntpr, h))
    ref = oracle.run_layer(x, ids, scores, w, T, ntpr, E, K, ORACLE_THREADS)
    assert np.array_equal(y, ref["y"])
    del disp, wd, h
    _free()


def test_layer_graph_replays_with_fresh_routing():
    """layout -> dispatch -> expert -> combine captured once and replayed with
    new routing and token counts; every replay is checked bitwise against the
    oracle's layer, with eager calls on the same buffers in between."""
    nmax, D, E, K = 512, 256, 32, 4
    w = _identity_experts(E, D)
    wd = tile_expert_weights(x_to_dev(w))
    disp = MoeDispatcher(nmax, D, E, K, dtype=torch.bfloat16, device=DEV)
    n = round_up4(nmax) * K
    h = torch.empty((n, D), dtype=torch.bfloat16, device=DEV)
    x_in = torch.zeros((nmax, D), dtype=torch.bfloat16, device=DEV)
    ids_in = torch.full((nmax, K), -1, dtype=torch.int32, device=DEV)
    s_in = torch.zeros((nmax, K), dtype=torch.float32, device=DEV)

    def step():
        lay = disp.layout(ids_in, nmax)
        dsp = disp.dispatch(x_in, s_in, ids_in, lay.counts, num_tokens_per_rank=nmax)
        grouped_gemm(dsp.x_e, wd, lay.offsets, h)
        return disp.combine(h, lay.row_map, s_in, num_tokens_per_rank=nmax)

    note("layer graph warmup + capture")
    side = torch.cuda.Stream(DEV)
    side.wait_stream(torch.cuda.current_stream(DEV))
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream(DEV).wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        y_graph = step()
    for i in range(12):
        T = [nmax, 1, 300, 77, 512, 4][i % 6]
        x, ids, scores = _dyadic_batch(nmax, D, E, K, 500 + i)
        ids[T:] = -1                        # tokens past T route nowhere
        scores[T:] = 0.0
        x_in.copy_(x_to_dev(x))
        ids_in.copy_(i32_dev(ids))
        s_in.copy_(f32_dev(scores))
        note(f"layer graph replay {i} T={T}")
        g.replay()
        sync_or_fail()
        ref = oracle.run_layer(x, ids, scores, w, nmax, nmax, E, K, ORACLE_THREADS)
        assert np.array_equal(x_to_np(y_graph), ref["y"]), i
        if i % 3 == 2:                      # an eager layer on the same buffers
            xe, ie, se = _dyadic_batch(nmax, D, E, K, 900 + i)
            note(f"layer eager between replays {i}")
            ye = x_to_np(_gpu_layer(disp, xe, ie, se, wd, 37, 40, h))
            refe = oracle.run_layer(xe, ie, se, w, 37, 40, E, K, ORACLE_THREADS)
            assert np.array_equal(ye, refe["y"])
    del g, disp, wd, h
    _free()
