"""Pins of the oracle's expert step (a grouped GEMM over the expert-major rows,
driven by the per-expert offsets) and of its one-step fp64 -> bf16 rounding.

Each test checks the oracle against something fixed outside it: numpy's
float64 matrix product, exactly representable special cases (scaled identity
and selection weights), brute-force loops on tiny integer inputs, the
midpoints between consecutive bf16 values, torch's fp32 -> bf16 conversion,
and the analytic expected output of a whole layer with scaled identity
experts (the oracle the uccl page's graph test validates against, "Tests").
Runs on the CPU only.
"""
import numpy as np
import pytest
import torch

import oracle

U32 = 2.0 ** -24


def _bits_to_f64(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _torch_bf16_bits(f32):
    t = torch.from_numpy(np.ascontiguousarray(f32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _rand_bf16(shape, rng, scale=1.0):
    return _torch_bf16_bits(rng.standard_normal(shape).astype(np.float32) * scale)


def _offsets(counts):
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)


# ---------------------------------------------------------------- rounding

def test_f64_to_bf16_agrees_with_torch_on_fp32_values():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
                        [0.0, -0.0, 1.0, -1.0, np.inf, -np.inf]]).astype(np.float32)
    v = v[np.isfinite(v) | np.isinf(v)]
    assert np.array_equal(oracle.f64_to_bf16(v.astype(np.float64)), _torch_bf16_bits(v))


def test_f64_to_bf16_rounds_midpoints_to_even_and_others_to_nearest():
    # every pair of consecutive positive finite bf16 values (a, b)
    bits = np.arange(0x0000, 0x7F7F, dtype=np.uint16)
    a = _bits_to_f64(bits)
    b = _bits_to_f64(bits + 1)
    mid = (a + b) / 2                                  # exact in fp64
    below = np.nextafter(mid, 0.0)
    above = np.nextafter(mid, np.inf)
    assert np.array_equal(oracle.f64_to_bf16(below), bits)
    assert np.array_equal(oracle.f64_to_bf16(above), bits + 1)
    even = np.where(bits % 2 == 0, bits, bits + 1).astype(np.uint16)
    assert np.array_equal(oracle.f64_to_bf16(mid), even)
    assert np.array_equal(oracle.f64_to_bf16(-mid), even | np.uint16(0x8000))


def test_f64_to_bf16_special_values():
    big = float.fromhex("0x1.FEp127")
    cases = {
        1.0 + 2.0 ** -8 + 2.0 ** -40: 0x3F81,   # through fp32 this would tie down to 0x3F80
        1.0 + 2.0 ** -8: 0x3F80,
        big: 0x7F7F,                             # largest finite
        big + 2.0 ** 118: 0x7F7F,                # below the overflow midpoint
        big + 2.0 ** 119: 0x7F80,                # the midpoint (spacing 2^120): to even = inf
        2.0 ** -133: 0x0001,
        2.0 ** -134: 0x0000,                     # midpoint to even zero
        3 * 2.0 ** -134: 0x0002,
        -0.0: 0x8000,
        float("nan"): 0x7FC0,
        float("-inf"): 0xFF80,
    }
    got = oracle.f64_to_bf16(np.array(list(cases.keys())))
    assert [int(g) for g in got] == list(cases.values())


# ------------------------------------------------------------ expert step

def test_grouped_gemm_one_expert_is_the_matrix_product():
    rng = np.random.default_rng(1)
    x = _rand_bf16((37, 72), rng)
    w = _rand_bf16((1, 40, 72), rng)
    out = oracle.grouped_gemm(x, w, np.array([0, 37], np.int32))
    ref = _bits_to_f64(x) @ _bits_to_f64(w[0]).T
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_grouped_gemm_segments_use_their_own_weight_and_leave_other_rows():
    rng = np.random.default_rng(2)
    counts = [3, 0, 7, 1, 0]
    off = _offsets(counts)
    rows = int(off[-1]) + 3
    x = _rand_bf16((rows, 48), rng)
    w = _rand_bf16((5, 24, 48), rng)
    out = oracle.grouped_gemm(x, w, off, nthreads=4)
    for e in range(5):
        seg = slice(off[e], off[e + 1])
        ref = _bits_to_f64(x[seg]) @ _bits_to_f64(w[e]).T
        np.testing.assert_allclose(out[seg], ref, rtol=1e-12, atol=1e-12)
    assert np.isnan(out[off[-1]:]).all()


def test_grouped_gemm_scaled_identity_experts_are_exact():
    rng = np.random.default_rng(3)
    E, D = 6, 64
    counts = rng.integers(0, 9, E)
    off = _offsets(counts)
    x = _rand_bf16((int(off[-1]), D), rng)
    c = 2.0 ** (np.arange(E) % 5 - 2)
    w = np.stack([_torch_bf16_bits(np.eye(D, dtype=np.float32) * c[e]) for e in range(E)])
    out = oracle.grouped_gemm(x, w, off)
    for e in range(E):
        seg = slice(off[e], off[e + 1])
        assert np.array_equal(out[seg], c[e] * _bits_to_f64(x[seg]))


def test_grouped_gemm_selection_weights_pick_input_columns():
    # non-square weights: output column n of expert e is input column (3n + e) % Kd
    rng = np.random.default_rng(4)
    E, Kd, N = 3, 20, 12
    off = _offsets([4, 5, 2])
    x = _rand_bf16((11, Kd), rng)
    w = np.zeros((E, N, Kd), np.float32)
    for e in range(E):
        for n in range(N):
            w[e, n, (3 * n + e) % Kd] = 1.0
    out = oracle.grouped_gemm(x, _torch_bf16_bits(w), off)
    xf = _bits_to_f64(x)
    for e in range(E):
        for r in range(off[e], off[e + 1]):
            assert np.array_equal(out[r], xf[r, [(3 * n + e) % Kd for n in range(N)]])


def test_grouped_gemm_bruteforce_tiny_integers():
    rng = np.random.default_rng(5)
    E, Kd, N = 3, 5, 4
    counts = [2, 0, 3]
    off = _offsets(counts)
    xi = rng.integers(-9, 10, (5, Kd))
    wi = rng.integers(-9, 10, (E, N, Kd))
    out = oracle.grouped_gemm(_torch_bf16_bits(xi), _torch_bf16_bits(wi), off)
    for e in range(E):
        for r in range(off[e], off[e + 1]):
            for n in range(N):
                s = 0
                for d in range(Kd):
                    s += int(xi[r, d]) * int(wi[e, n, d])
                assert out[r, n] == s


def test_grouped_gemm_at_chosen_positions():
    rng = np.random.default_rng(6)
    off = _offsets([5, 0, 9, 3])
    x = _rand_bf16((20, 40), rng)
    w = _rand_bf16((4, 16, 40), rng)
    rows = np.array([0, 4, 5, 13, 16, 17, 19])
    cols = np.array([0, 15, 3, 7, 1, 2, 5])
    got = oracle.grouped_gemm_at(x, w, off, rows, cols)
    owner = [0, 0, 2, 2, 3, None, None]
    xf = _bits_to_f64(x)
    for i, e in enumerate(owner):
        if e is None:
            assert np.isnan(got[i])
        else:
            ref = float(np.dot(xf[rows[i]], _bits_to_f64(w[e, cols[i]])))
            assert abs(got[i] - ref) <= 1e-12 * max(1.0, abs(ref))


def test_grouped_gemm_rejects_inconsistent_offsets():
    x = np.zeros((4, 8), np.uint16)
    w = np.zeros((2, 8, 8), np.uint16)
    for off in ([0, 3, 2], [0, 2, 5], [-1, 1, 2]):
        with pytest.raises(ValueError):
            oracle.grouped_gemm(x, w, np.array(off, np.int32))


# ------------------------------------------------------------- whole layer

def _layer_batch(T, D, E, K, seed):
    rng = np.random.default_rng(seed)
    ids = np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int32)
    ids[rng.random((T, K)) < 0.1] = -1
    ids[1, :] = -1                                   # a token with no expert
    # dyadic values: every sum below is exact in fp32
    x = _torch_bf16_bits(rng.integers(-128, 129, (T, D)).astype(np.float32) / 16)
    scores = (2.0 ** -rng.integers(0, 3, (T, K)) * rng.choice([-1, 1], (T, K))).astype(np.float32)
    return x, ids, scores


def test_layer_with_scaled_identity_experts_matches_the_analytic_output():
    T, D, E, K = 50, 32, 8, 4
    x, ids, scores = _layer_batch(T, D, E, K, 7)
    c = 2.0 ** (np.arange(E) % 5 - 2)
    w = np.stack([_torch_bf16_bits(np.eye(D, dtype=np.float32) * c[e]) for e in range(E)])
    got = oracle.run_layer(x, ids, scores, w, T, T, E, K)["y"]
    xf = _bits_to_f64(x)
    expect = np.zeros((T, D))
    for t in range(T):
        for k in range(K):
            if ids[t, k] >= 0:
                expect[t] += float(scores[t, k]) * c[ids[t, k]] * xf[t]
    assert np.array_equal(got, oracle.f64_to_bf16(expect))
    assert (got[1] == 0).all()                       # +0.0 for the token without expert


def test_layer_random_weights_against_independent_composition():
    T, D, E, K = 40, 24, 5, 3
    rng = np.random.default_rng(8)
    x, ids, scores = _layer_batch(T, D, E, K, 9)
    w = _rand_bf16((E, D, D), rng, 0.25)
    got = _bits_to_f64(oracle.run_layer(x, ids, scores, w, T, T, E, K)["y"])
    # each slot's expert output, built from numpy products, rounded once to bf16
    xf, wf = _bits_to_f64(x), _bits_to_f64(w)
    expect = np.zeros((T, D))
    mag = np.zeros((T, D))
    for t in range(T):
        for k in range(K):
            e = ids[t, k]
            if e < 0:
                continue
            h = _bits_to_f64(oracle.f64_to_bf16(xf[t] @ wf[e].T))
            expect[t] += float(scores[t, k]) * h
            mag[t] += np.abs(float(scores[t, k]) * h)
    # fp32 fused multiply-adds over K slots, then one bf16 rounding
    bound = K * U32 * mag * 1.01 + 2.0 ** -8 * np.abs(got) + 1e-300
    assert np.all(np.abs(got - expect) <= bound)


def test_layer_token_output_depends_only_on_its_routing():
    # NeMo Automodel page, "Testing": split runs reproduce the full run
    T, D, E, K = 24, 16, 6, 2
    rng = np.random.default_rng(10)
    x, ids, scores = _layer_batch(T, D, E, K, 11)
    w = _rand_bf16((E, D, D), rng, 0.3)
    full = oracle.run_layer(x, ids, scores, w, T, T, E, K)["y"]
    for a in (3, 8, 13):
        first = oracle.run_layer(x, ids, scores, w, a, 16, E, K)["y"]
        rest = oracle.run_layer(x[a:], ids[a:], scores[a:], w, T - a, T - a, E, K)["y"]
        assert np.array_equal(first, full[:a])
        assert np.array_equal(rest, full[a:])
