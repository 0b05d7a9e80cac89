"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each test checks the oracle against one of: values the pages print (golden
files with their citation), closed forms, library routines (numpy bincount,
cumsum, stable argsort, torch's bf16 conversion), brute-force enumeration on
tiny inputs, exactly representable special cases, or the standard error
bound of recursive fp32 summation. Runs on the CPU only.
"""
import itertools
import json
import os

import numpy as np
import pytest
import torch

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
U32 = 2.0 ** -24  # unit roundoff of fp32


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _bf16_to_f64(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _torch_bf16_bits(f32):
    t = torch.from_numpy(np.ascontiguousarray(f32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _routing(T, E, K, seed, none_frac=0.0, oob_frac=0.0, distinct=True):
    rng = np.random.default_rng(seed)
    if distinct:
        ids = np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int32)
    else:
        ids = rng.integers(0, E, size=(T, K)).astype(np.int32)
    if none_frac:
        ids[rng.random((T, K)) < none_frac] = -1
    if oob_frac:
        m = rng.random((T, K)) < oob_frac
        ids[m] = rng.choice(np.array([E, E + 7, -5, 2**31 - 1], np.int32), size=int(m.sum()))
    return ids


# --------------------------------------------------------------------------
# Capacity: closed forms and the pages' printed values

def test_ceil_div_defining_inequality():
    rng = np.random.default_rng(1)
    for a, b in zip(rng.integers(0, 10**9, 500), rng.integers(1, 10**5, 500)):
        q = oracle.ceil_div(int(a), int(b))
        assert q * b >= a and (q - 1) * b < a          # smallest q with q*b >= a
    assert oracle.ceil_div(0, 7) == 0
    assert oracle.ceil_div(-1, 2) == -1 and oracle.ceil_div(3, 0) == -1


def test_capacity_derivations_closed_form():
    # Pretraining: local_batch * ceil_div(seq_len, cp*tp).
    assert oracle.num_max_pretrain(8, 4096, 1, 1) == 32768
    # seq_len not divisible by the shard degree: floor would give 8*512.
    assert oracle.num_max_pretrain(8, 4097, 2, 4) == 8 * 513
    assert oracle.num_max_pretrain(1, 32768, 1, 1) == 32768   # 32k prefill, degree 1
    # vLLM inference: ceil_div(max_num_batched_tokens, cp*tp).
    assert oracle.num_max_infer(8192, 2, 2) == 2048
    assert oracle.num_max_infer(8193, 2, 2) == 2049
    assert oracle.num_max_infer(8192, 0, 1) == -1


def test_validate_num_max():
    assert oracle.validate_num_max(0, 1) != 0            # must be positive
    assert oracle.validate_num_max(-4, -8) != 0
    assert oracle.validate_num_max(4103, 4104) != 0      # smaller than derived
    assert oracle.validate_num_max(4104, 4104) == 0
    assert oracle.validate_num_max(8192, 4104) == 0


def test_round_up4_against_pages_alignment_matrix():
    g = _golden("alignment_matrix.json")
    bpt, mult = g["bytes_per_token"], g["extent_multiple_bytes"]
    # The unpadded counts reproduce the pages' pass/abort matrix ...
    for n in g["abort_counts"]:
        assert (n * bpt) % mult != 0
    for n in g["pass_counts"]:
        assert (n * bpt) % mult == 0
        assert oracle.round_up4(n) == n                  # aligned: no padding
    # ... and every rounded count passes, by the least padding possible.
    for n in list(range(0, 2000)) + g["abort_counts"]:
        r = oracle.round_up4(n)
        assert (r * bpt) % mult == 0 and n <= r < n + 4


def test_capacity_relation_cases():
    g = _golden("token_counts_from_pages.json")
    for a, b in g["unequal_pairs"]:
        ntpr = oracle.round_up4(max(a, b))
        assert oracle.check_capacity(a, ntpr, 4096) == 0
        assert oracle.check_capacity(b, ntpr, 4096) == 0
    assert oracle.check_capacity(2047, 2047, 2048) == 0
    assert oracle.check_capacity(2048, 2047, 2048) != 0   # T above the capacity
    assert oracle.check_capacity(2049, 2048, 4096) != 0
    assert oracle.check_capacity(0, 4097, 4096) != 0      # capacity above the max
    assert oracle.check_capacity(0, 0, 0) != 0            # nmax must be >= 1
    assert oracle.check_capacity(0, 0, 1) == 0            # T = 0 is a legal no-op
    assert oracle.check_capacity(-1, 0, 1) != 0
    # The relation implies the rounded capacities stay ordered.
    for ntpr in range(0, 40):
        for nmax in range(max(ntpr, 1), 40):
            assert oracle.round_up4(ntpr) <= oracle.round_up4(nmax)
    lens = g["dynamic_lengths"]
    nmax = max(lens)
    for T in lens:
        assert oracle.check_capacity(T, T, nmax) == 0
    a, b = g["activation_recompute_extents"]
    assert oracle.round_up4(a) == a and oracle.round_up4(b) == b


def test_layout_rejects_more_tokens_than_the_capacity():
    """The page's relation is T <= num_tokens_per_rank; rounding the capacity
    up to 4 adds padding rows, not room for tokens. So the layout must reject
    ntpr < T <= round_up4(ntpr) as check_capacity does, at its C entry point
    and through the wrapper, and still accept T == ntpr."""
    import ctypes as C
    E, K = 8, 2
    from oracle.oracle import _load
    lib = _load()
    for ntpr in (1, 2, 3, 5, 6, 7, 2045, 2046, 2047):
        n4 = oracle.round_up4(ntpr)
        for T in range(ntpr + 1, n4 + 1):
            assert oracle.check_capacity(T, ntpr, 4096) != 0
            ids = _routing(T, E, K, seed=T)
            counts = np.zeros(E, np.int32)
            offsets = np.zeros(E + 1, np.int32)
            row_map = np.empty(n4 * K, np.int32)
            src = np.empty(n4 * K, np.int32)
            p = lambda a: a.ctypes.data_as(C.c_void_p)  # noqa: E731
            assert lib.orc_layout(p(ids), T, ntpr, E, K, p(counts), p(offsets), p(row_map),
                                  p(src)) == -1
            with pytest.raises(ValueError):
                oracle.layout(ids, T, ntpr, E, K)
        ids = _routing(ntpr, E, K, seed=ntpr)
        assert oracle.layout(ids, ntpr, ntpr, E, K)["total"] == ntpr * K


# --------------------------------------------------------------------------
# Layout

def test_layout_hand_worked_example():
    # ids [[2,0],[0,2],[1,-1]], E=4, K=2. Slots in flattened order:
    # 0->e2, 1->e0, 2->e0, 3->e2, 4->e1, 5->none. Expert 0 gets slots 1,2
    # (rows 0,1), expert 1 slot 4 (row 2), expert 2 slots 0,3 (rows 3,4).
    ids = np.array([[2, 0], [0, 2], [1, -1]], np.int32)
    r = oracle.layout(ids, T=3, ntpr=3, E=4, K=2)
    assert r["counts"].tolist() == [2, 1, 2, 0]
    assert r["offsets"].tolist() == [0, 2, 3, 5, 5]
    assert r["row_map"].tolist() == [[3, 0], [1, 4], [2, -1], [-1, -1]]
    assert r["src"].tolist() == [1, 2, 4, 0, 3]
    assert r["total"] == 5


def _brute_rows(flat_e, E):
    """row of slot i = #slots with a smaller expert + #earlier slots with the
    same expert; direct O(n^2) counting, no sort."""
    n = len(flat_e)
    rows = []
    for i in range(n):
        e = flat_e[i]
        if e is None:
            rows.append(-1)
            continue
        smaller = sum(1 for j in range(n) if flat_e[j] is not None and flat_e[j] < e)
        earlier = sum(1 for j in range(i) if flat_e[j] == e)
        rows.append(smaller + earlier)
    return rows


def test_layout_bruteforce_exhaustive_tiny():
    E, K = 4, 2
    choices = [-1, 0, 1, 2, 3]
    pairs = [p for p in itertools.product(choices, repeat=2)
             if p[0] != p[1] or p[0] == -1]
    assert len(pairs) == 21
    checked = 0
    for T in (1, 2, 3):
        for routing in itertools.product(pairs, repeat=T):
            ids = np.array(routing, np.int32).reshape(T, K)
            ntpr = T + (checked % 3)          # vary the padded capacity too
            r = oracle.layout(ids, T, ntpr, E, K)
            flat = [None if v < 0 else int(v) for v in ids.ravel()]
            want = _brute_rows(flat, E)
            n4 = oracle.round_up4(ntpr)
            got = r["row_map"]
            assert got.shape == (n4, K)
            assert got[:T].ravel().tolist() == want
            assert (got[T:] == -1).all()
            cnt = [sum(1 for v in flat if v == e) for e in range(E)]
            assert r["counts"].tolist() == cnt
            assert r["total"] == sum(cnt)
            for i, row in enumerate(want):
                if row >= 0:
                    assert r["src"][row] == i
            checked += 1
    assert checked == 21 + 21**2 + 21**3


@pytest.mark.parametrize("T,E,K,none_frac,oob_frac,distinct,seed", [
    (64, 8, 2, 0.0, 0.0, True, 0),
    (1000, 128, 8, 0.1, 0.0, True, 1),
    (777, 256, 8, 0.0, 0.05, True, 2),
    (513, 16, 6, 0.2, 0.02, False, 3),   # duplicates allowed
    (300, 1, 1, 0.3, 0.0, True, 4),
    (5, 1024, 16, 0.0, 0.0, True, 5),
])
def test_layout_matches_library_routines(T, E, K, none_frac, oob_frac, distinct, seed):
    ids = _routing(T, E, K, seed, none_frac, oob_frac, distinct)
    ntpr = T + 3
    r = oracle.layout(ids, T, ntpr, E, K)
    flat = ids.ravel().astype(np.int64)
    valid = (flat >= 0) & (flat < E)
    # counts: bincount of the valid ids
    np.testing.assert_array_equal(r["counts"], np.bincount(flat[valid], minlength=E))
    # offsets: exclusive cumulative sum
    np.testing.assert_array_equal(r["offsets"], np.concatenate([[0], np.cumsum(r["counts"])]))
    # src: stable argsort of the valid slots by expert
    key = np.where(valid, flat, E)
    order = np.argsort(key, kind="stable")[: int(valid.sum())]
    np.testing.assert_array_equal(r["src"], order)
    # row_map is the inverse permutation on valid slots, -1 elsewhere
    want = np.full(oracle.round_up4(ntpr) * K, -1, np.int64)
    want[order] = np.arange(order.size)
    np.testing.assert_array_equal(r["row_map"].ravel(), want)


def _check_layout_invariants(r, ids, T, ntpr, E, K):
    n4 = oracle.round_up4(ntpr)
    rm = r["row_map"]
    assert rm.shape == (n4, K)
    assert (rm[T:] == -1).all()                       # padding reaches no expert
    total = r["total"]
    used = rm[rm >= 0]
    assert used.size == total
    assert np.array_equal(np.sort(used), np.arange(total))   # bijection
    src, off = r["src"], r["offsets"]
    for e in range(E):
        seg = src[off[e]:off[e + 1]]
        assert (np.diff(seg) > 0).all()                # stable order within expert
        assert (ids.ravel()[seg] == e).all()           # segment holds expert e
    flat_rm = rm[:T].ravel()
    assert (flat_rm[src] == np.arange(total)).all()


@pytest.mark.parametrize("name", ["tiny", "padded", "dsv3"])
def test_layout_invariants_on_workloads(name):
    w = workloads.WORKLOADS[name]
    b = workloads.make_batch(w, with_x=False)
    r = oracle.layout(b["ids"], w.T, w.ntpr, w.E, w.K)
    _check_layout_invariants(r, b["ids"], w.T, w.ntpr, w.E, w.K)
    assert r["total"] == w.T * w.K


def test_layout_skew_of_zipf_routing():
    # Zipf(1.1) over 256 experts, top-8 without replacement: expert 0 is the
    # hottest and carries most tokens; every token still has 8 distinct ids.
    w = workloads.WORKLOADS["dsv3"]
    b = workloads.make_batch(w, with_x=False)
    r = oracle.layout(b["ids"], w.T, w.ntpr, w.E, w.K)
    c = r["counts"]
    assert c.argmax() == 0 and c[0] > 0.8 * w.T
    assert all(len(set(row)) == w.K for row in b["ids"].tolist())


def test_layout_padding_invariance():
    w = workloads.WORKLOADS["padded"]
    b = workloads.make_batch(w, with_x=False)
    for T in workloads.PADDED_T_VALUES:
        ref = oracle.layout(b["ids"][:T], T, oracle.round_up4(T), w.E, w.K)
        for ntpr in (T, 2048, 4096):
            r = oracle.layout(b["ids"][:T], T, ntpr, w.E, w.K)
            for key in ("counts", "offsets", "src"):
                np.testing.assert_array_equal(r[key], ref[key])
            np.testing.assert_array_equal(r["row_map"][:T], ref["row_map"][:T])
            assert (r["row_map"][T:] == -1).all()


def test_layout_empty_and_all_none():
    r = oracle.layout(np.zeros((0, 8), np.int32), 0, 0, 16, 8)
    assert r["total"] == 0 and r["row_map"].shape == (0, 8)
    assert (r["counts"] == 0).all() and (r["offsets"] == 0).all()
    r = oracle.layout(np.zeros((0, 8), np.int32), 0, 5, 16, 8)
    assert r["row_map"].shape == (8, 8) and (r["row_map"] == -1).all()
    ids = np.full((7, 4), -1, np.int32)
    r = oracle.layout(ids, 7, 7, 16, 4)
    assert r["total"] == 0 and (r["row_map"] == -1).all()


# --------------------------------------------------------------------------
# Dispatch

@pytest.mark.parametrize("name", ["tiny", "padded"])
def test_dispatch_is_the_row_gather(name):
    w = workloads.WORKLOADS[name]
    b = workloads.make_batch(w)
    T = w.T - 5
    r = oracle.layout(b["ids"][:T], T, w.ntpr, w.E, w.K)
    x_e, s_e = oracle.dispatch(b["x"][:T], b["scores"][:T], w.K, r["src"])
    # numpy fancy-index gather: row r of x_e is token src[r] // K.
    assert np.array_equal(x_e.view(np.uint8), b["x"][r["src"] // w.K].view(np.uint8))
    want_s = b["scores"][:T].ravel()[r["src"]]
    assert np.array_equal(s_e.view(np.uint32), want_s.view(np.uint32))
    rows = np.array([0, r["total"] - 1, r["total"] // 2], np.int64)
    xr, sr = oracle.dispatch_rows(b["x"][:T], b["scores"][:T], w.K, r["src"], rows)
    assert np.array_equal(xr, x_e[rows]) and np.array_equal(sr, s_e[rows])


def test_dispatch_threads_equal_serial():
    w = workloads.WORKLOADS["padded"]
    b = workloads.make_batch(w)
    r = oracle.layout(b["ids"], w.T, w.ntpr, w.E, w.K)
    a = oracle.dispatch(b["x"], b["scores"], w.K, r["src"], nthreads=1)
    c = oracle.dispatch(b["x"], b["scores"], w.K, r["src"], nthreads=4)
    assert np.array_equal(a[0], c[0]) and np.array_equal(a[1], c[1])


# --------------------------------------------------------------------------
# Combine

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_combine_k1_unit_score_identity_is_exact(dtype):
    w = workloads.Workload("k1", T=50, ntpr=52, nmax=64, D=96, E=5, K=1,
                           dtype=dtype, routing="uniform", seed=3)
    b = workloads.make_batch(w)
    scores = np.ones((w.T, 1), np.float32)
    out = oracle.run_pipeline(b["x"], b["ids"], scores, w.T, w.ntpr, w.E, w.K)
    assert np.array_equal(out["y"].view(np.uint8), b["x"].view(np.uint8))


def _dyadic_inputs(T, D, seed):
    rng = np.random.default_rng(seed)
    # x with at most 8 significant bits (exact in bf16), moderate exponents.
    mant = rng.integers(128, 256, size=(T, D)).astype(np.float64)
    expo = rng.integers(-20, 10, size=(T, D))
    sign = rng.choice([-1.0, 1.0], size=(T, D))
    x = (sign * mant * np.exp2(expo - 7)).astype(np.float32)
    base = np.array([0.5, 0.25, 0.125, 0.0625], np.float32)
    scores = np.stack([rng.permutation(base) for _ in range(T)]).astype(np.float32)
    ids = np.argsort(rng.random((T, 8)), axis=1)[:, :4].astype(np.int32)
    ids[rng.random((T, 4)) < 0.25] = -1
    return x, ids, scores


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_combine_dyadic_scores_are_exact(dtype):
    T, D, E, K = 40, 64, 8, 4
    x, ids, scores = _dyadic_inputs(T, D, 7)
    xin = x if dtype == "f32" else _torch_bf16_bits(x)
    assert np.array_equal(_bf16_to_f64(_torch_bf16_bits(x)), x.astype(np.float64))
    out = oracle.run_pipeline(xin, ids, scores, T, T, E, K)
    ssum = np.where(ids >= 0, scores, 0).astype(np.float64).sum(axis=1)
    exact = ssum[:, None] * x.astype(np.float64)       # every product and sum is exact
    assert np.array_equal(exact.astype(np.float32).astype(np.float64), exact)
    if dtype == "f32":
        assert np.array_equal(out["y"], exact.astype(np.float32))
    else:
        assert np.array_equal(out["y"], _torch_bf16_bits(exact.astype(np.float32)))


def test_combine_all_none_token_is_positive_zero():
    x = np.full((3, 16), -2.5, np.float32)
    ids = np.array([[-1, -1], [1, -1], [-1, -1]], np.int32)
    scores = np.array([[np.nan, -1.0], [2.0, np.nan], [0.0, 0.0]], np.float32)
    for xin in (x, _torch_bf16_bits(x)):
        out = oracle.run_pipeline(xin, ids, scores, 3, 3, 4, 2)
        y = out["y"].view(np.uint32 if xin.dtype == np.float32 else np.uint16)
        assert (y[0] == 0).all() and (y[2] == 0).all()   # +0.0, sign bit clear
        got = out["y"][1] if xin.dtype == np.float32 else _bf16_to_f64(out["y"][1])
        assert np.all(np.asarray(got, np.float64) == -5.0)  # NaN score on a none slot ignored


def _exact_combine(y_e64, row_map, scores, T, K):
    y = np.zeros((T, y_e64.shape[1]))
    mag = np.zeros_like(y)
    for k in range(K):
        r = row_map[:T, k]
        m = r >= 0
        term = scores[:T, k].astype(np.float64)[m, None] * y_e64[r[m]]
        y[m] += term
        mag[m] += np.abs(term)
    return y, mag


@pytest.mark.parametrize("dtype,K", [("f32", 8), ("bf16", 8), ("f32", 3), ("bf16", 16)])
def test_combine_general_expert_output_within_summation_bound(dtype, K):
    # Non-identity expert outputs: wrong rows, dropped terms or wrong signs
    # break the bound by orders of magnitude.
    rng = np.random.default_rng(11 + K)
    T, E, D = 200, 32, 48
    ids = _routing(T, E, K, 12 + K, none_frac=0.1)
    scores = rng.standard_normal((T, K)).astype(np.float32)
    r = oracle.layout(ids, T, T, E, K)
    ye = rng.standard_normal((r["total"], D)).astype(np.float32)
    if dtype == "bf16":
        ye_in = _torch_bf16_bits(ye)
        ye64 = _bf16_to_f64(ye_in)
    else:
        ye_in, ye64 = ye, ye.astype(np.float64)
    y = oracle.combine(ye_in, r["row_map"], scores, T, K)
    exact, mag = _exact_combine(ye64, r["row_map"], scores, T, K)
    gamma = K * U32 / (1 - K * U32)
    bound = gamma * mag
    if dtype == "bf16":
        got = _bf16_to_f64(y)
        bound = bound + np.abs(exact) * 2.0 ** -8 + 2.0 ** -133   # half a bf16 ulp
    else:
        got = y.astype(np.float64)
    assert np.all(np.abs(got - exact) <= bound)


def test_combine_identity_expert_closed_form_bound_tiny_workload():
    w = workloads.WORKLOADS["tiny"]
    b = workloads.make_batch(w)
    out = oracle.run_pipeline(b["x"], b["ids"], b["scores"], w.T, w.ntpr, w.E, w.K)
    s = b["scores"].astype(np.float64)
    x = b["x"].astype(np.float64)
    exact = s.sum(axis=1)[:, None] * x
    bound = (w.K * U32 / (1 - w.K * U32)) * (np.abs(s).sum(axis=1)[:, None] * np.abs(x))
    assert np.all(np.abs(out["y"].astype(np.float64) - exact) <= bound)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(5)
    bits = rng.integers(0, 2**32, size=20000, dtype=np.uint64).astype(np.uint32)
    # ties: low half exactly 0x8000 with even and odd kept parts
    ties = (rng.integers(0, 2**16, size=2000, dtype=np.uint64).astype(np.uint32) << 16) | 0x8000
    special = np.array([0, 0x80000000, 0x7F800000, 0xFF800000, 0x00000001, 0x807FFFFF,
                        0x7F7FFFFF, 0x7F7F8000, 0x3F808000, 0x3F818000], np.uint32)
    allb = np.concatenate([bits, ties, special])
    f = allb.view(np.float32)
    got = oracle.f32_to_bf16(f)
    nan = np.isnan(f)
    assert (got[nan] == 0x7FC0).all()
    np.testing.assert_array_equal(got[~nan], _torch_bf16_bits(f[~nan]))


def test_combine_duplicate_ids_get_own_rows_and_sum():
    x = np.arange(8, dtype=np.float32).reshape(2, 4)
    ids = np.array([[1, 1], [0, 1]], np.int32)
    scores = np.array([[0.25, 0.5], [1.0, 2.0]], np.float32)
    out = oracle.run_pipeline(x, ids, scores, 2, 2, 2, 2)
    assert out["row_map"].tolist()[:2] == [[1, 2], [0, 3]]
    np.testing.assert_array_equal(out["y"][0], 0.75 * x[0])
    np.testing.assert_array_equal(out["y"][1], 3.0 * x[1])


def test_combine_threads_equal_serial():
    w = workloads.WORKLOADS["padded"]
    b = workloads.make_batch(w)
    a = oracle.run_pipeline(b["x"], b["ids"], b["scores"], 600, 2048, w.E, w.K, nthreads=1)
    c = oracle.run_pipeline(b["x"], b["ids"], b["scores"], 600, 2048, w.E, w.K, nthreads=4)
    assert np.array_equal(a["y"], c["y"])
    toks = np.array([0, 17, 599], np.int64)
    yt = oracle.combine_tokens(a["x_e"], a["row_map"], b["scores"][:600], w.K, toks)
    assert np.array_equal(yt, a["y"][toks])


# --------------------------------------------------------------------------
# Padding: unequal/unaligned counts reproduce the equal-count run

def _small_padded_batch():
    w = workloads.WORKLOADS["padded"]
    w = workloads.Workload("padded_small", T=2048, ntpr=2048, nmax=4096, D=64,
                           E=w.E, K=w.K, dtype="bf16", routing="uniform", seed=0)
    return w, workloads.make_batch(w)


def test_unequal_counts_reproduce_equal_count_run():
    w, b = _small_padded_batch()
    full = oracle.run_pipeline(b["x"], b["ids"], b["scores"], 2048, 2048, w.E, w.K)
    for T in workloads.PADDED_T_VALUES:
        out = oracle.run_pipeline(b["x"], b["ids"], b["scores"], T, 2048, w.E, w.K)
        assert np.array_equal(out["y"], full["y"][:T])
    for a, c in workloads.PADDED_PAIRS:        # two "ranks" sharing one capacity
        ntpr = oracle.round_up4(max(a, c))
        ya = oracle.run_pipeline(b["x"], b["ids"], b["scores"], a, ntpr, w.E, w.K)["y"]
        yc = oracle.run_pipeline(b["x"][a:], b["ids"][a:], b["scores"][a:], c, ntpr, w.E, w.K)["y"]
        assert np.array_equal(ya, full["y"][:a])
        assert np.array_equal(yc, full["y"][a:a + c])


def test_virtual_padding_equals_materialized_padding():
    w, b = _small_padded_batch()
    for T in (3, 5, 13, 614):
        n4 = oracle.round_up4(2047)
        virt = oracle.run_pipeline(b["x"], b["ids"], b["scores"], T, 2047, w.E, w.K)
        xm = b["x"][:n4].copy()
        xm[T:] = 0
        idm = b["ids"][:n4].copy()
        idm[T:] = -1                     # all-False routing
        sm = b["scores"][:n4].copy()
        sm[T:] = 0.0                     # zero probability
        mat = oracle.run_pipeline(xm, idm, sm, n4, n4, w.E, w.K)
        for key in ("counts", "offsets", "src", "row_map", "x_e", "s_e"):
            assert np.array_equal(virt[key], mat[key]), key
        assert np.array_equal(virt["y"], mat["y"][:T])
        assert (mat["y"][T:] == 0).all()  # padded rows are +0.0, then sliced off


# --------------------------------------------------------------------------
# Backward: pinned by the adjoint identities and by finite differences of the
# forward definitions, with inputs chosen so that every fp32/bf16 operation
# is exact (small integers, dyadic scores): then the identities hold exactly.

def _exact_case(T, E, K, dtype, seed, none_frac=0.15):
    rng = np.random.default_rng(seed)
    ids = np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int32)
    ids[rng.random((T, K)) < none_frac] = -1
    scores = rng.choice(np.array([0.5, 0.25, 0.125, 0.0625, -0.5, 1.0], np.float32), size=(T, K))
    lay = oracle.layout(ids, T, T, E, K)
    def ints(shape):
        v = rng.integers(-8, 9, size=shape).astype(np.float32)
        return v if dtype == "f32" else _torch_bf16_bits(v)
    return ids, scores, lay, ints


def _f64(a):
    return a.astype(np.float64) if a.dtype == np.float32 else _bf16_to_f64(a)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_dispatch_backward_is_the_adjoint_of_dispatch(dtype):
    T, E, K, D = 37, 12, 4, 24
    ids, scores, lay, ints = _exact_case(T, E, K, dtype, 21)
    x = ints((T, D))
    x_e, _ = oracle.dispatch(x, scores, K, lay["src"])
    h = ints((lay["total"], D))
    gx = oracle.dispatch_backward(h, lay["row_map"], T, K)
    lhs = float(np.sum(_f64(x_e) * _f64(h)))       # <dispatch(x), h>
    rhs = float(np.sum(_f64(x) * _f64(gx)))        # <x, dispatch^T h>
    assert lhs == rhs
    # brute force: gx[t] = sum over the token's slots of h rows
    want = np.zeros((T, D))
    for t in range(T):
        for k in range(K):
            r = lay["row_map"][t, k]
            if r >= 0:
                want[t] += _f64(h[r:r + 1])[0]
    assert np.array_equal(_f64(gx), want)


def test_dispatch_backward_equals_unit_score_combine():
    w = workloads.WORKLOADS["padded"]
    b = workloads.make_batch(w)
    T = 300
    lay = oracle.layout(b["ids"][:T], T, T, w.E, w.K)
    rng = np.random.default_rng(3)
    h = _torch_bf16_bits(rng.standard_normal((lay["total"], 40)).astype(np.float32))
    gx = oracle.dispatch_backward(h, lay["row_map"], T, w.K)
    ones = np.ones((T, w.K), np.float32)
    assert np.array_equal(gx, oracle.combine(h, lay["row_map"], ones, T, w.K))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_combine_backward_is_the_adjoint_in_expert_outputs(dtype):
    T, E, K, D = 41, 10, 4, 20
    ids, scores, lay, ints = _exact_case(T, E, K, dtype, 22)
    y_e = ints((lay["total"], D))
    g = ints((T, D))
    y = oracle.combine(y_e, lay["row_map"], scores, T, K)
    g_e, grad_s = oracle.combine_backward(g, y_e, lay["row_map"], scores, T, K)
    lhs = float(np.sum(_f64(y) * _f64(g)))          # <combine(y_e), g>
    rhs = float(np.sum(_f64(y_e) * _f64(g_e)))      # <y_e, combine^T g>
    assert lhs == rhs
    # brute force of both outputs
    for t in range(T):
        for k in range(K):
            r = lay["row_map"][t, k]
            if r < 0:
                assert grad_s[t, k] == 0.0
                continue
            assert np.array_equal(_f64(g_e[r:r + 1])[0], float(scores[t, k]) * _f64(g[t:t + 1])[0])
            assert grad_s[t, k] == float(np.dot(_f64(g[t:t + 1])[0], _f64(y_e[r:r + 1])[0]))


def test_combine_backward_score_gradient_by_finite_differences():
    # L(s) = sum_t <g[t], y[t]> is linear in s, so (L(s + d e_tk) - L(s)) / d
    # is exactly dL/ds[t,k]; every forward operation is exact here.
    T, E, K, D = 9, 8, 4, 16
    ids, scores, lay, ints = _exact_case(T, E, K, "f32", 23, none_frac=0.2)
    y_e = ints((lay["total"], D))
    g = ints((T, D))
    _, grad_s = oracle.combine_backward(g, y_e, lay["row_map"], scores, T, K)
    base = float(np.sum(oracle.combine(y_e, lay["row_map"], scores, T, K).astype(np.float64) * g))
    delta = np.float32(1.0 / 32)
    for t in range(T):
        for k in range(K):
            s2 = scores.copy()
            s2[t, k] += delta
            Lp = float(np.sum(oracle.combine(y_e, lay["row_map"], s2, T, K).astype(np.float64) * g))
            fd = (Lp - base) / float(delta)
            assert fd == grad_s[t, k], (t, k)


def test_combine_backward_general_values_within_bounds():
    rng = np.random.default_rng(24)
    T, E, K, D = 120, 32, 8, 64
    ids = np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int32)
    ids[rng.random((T, K)) < 0.1] = -1
    scores = rng.standard_normal((T, K)).astype(np.float32)
    lay = oracle.layout(ids, T, T, E, K)
    y_e = _torch_bf16_bits(rng.standard_normal((lay["total"], D)).astype(np.float32))
    g = _torch_bf16_bits(rng.standard_normal((T, D)).astype(np.float32))
    g_e, grad_s = oracle.combine_backward(g, y_e, lay["row_map"], scores, T, K)
    G, Y = _f64(g), _f64(y_e)
    for t in range(T):
        for k in range(K):
            r = lay["row_map"][t, k]
            if r < 0:
                continue
            exact = scores[t, k] * G[t]
            got = _f64(g_e[r:r + 1])[0]
            # one fp32 product, then one bf16 rounding
            assert np.all(np.abs(got - exact) <= np.abs(exact) * (2.0 ** -8 + 2.0 ** -24) + 2.0 ** -133)
            assert abs(grad_s[t, k] - np.dot(G[t], Y[r])) <= 1e-12 * np.sum(np.abs(G[t] * Y[r]))


def test_backward_unequal_counts_reproduce_equal_count_run():
    w, b = _small_padded_batch()
    rng = np.random.default_rng(25)
    D = w.D
    g_full = _torch_bf16_bits(rng.standard_normal((2048, D)).astype(np.float32))
    lay_f = oracle.layout(b["ids"], 2048, 2048, w.E, w.K)
    x_e_f, _ = oracle.dispatch(b["x"], b["scores"], w.K, lay_f["src"])
    ge_f, gs_f = oracle.combine_backward(g_full, x_e_f, lay_f["row_map"], b["scores"], 2048, w.K)
    gx_f = oracle.dispatch_backward(ge_f, lay_f["row_map"], 2048, w.K)
    for T in workloads.PADDED_T_VALUES:
        lay = oracle.layout(b["ids"][:T], T, 2048, w.E, w.K)
        x_e, _ = oracle.dispatch(b["x"][:T], b["scores"][:T], w.K, lay["src"])
        ge, gs = oracle.combine_backward(g_full[:T], x_e, lay["row_map"], b["scores"][:T], T, w.K)
        gx = oracle.dispatch_backward(ge, lay["row_map"], T, w.K)
        assert np.array_equal(gs, gs_f[:T])
        assert np.array_equal(gx, gx_f[:T])
        rm, rmf = lay["row_map"][:T].ravel(), lay_f["row_map"][:T].ravel()
        assert np.array_equal(ge[rm[rm >= 0]], ge_f[rmf[rmf >= 0]])   # per slot


# --------------------------------------------------------------------------
# Routing-map input format and scores applied on dispatch

def _map_from_topk(ids, probs_src, E):
    T, K = ids.shape
    m = np.zeros((T, E), np.uint8)
    p = np.zeros((T, E), np.float32)
    rows = np.repeat(np.arange(T), K)
    flat = ids.ravel()
    ok = flat >= 0
    m[rows[ok], flat[ok]] = 1
    p[rows[ok], flat[ok]] = probs_src.ravel()[ok]
    return m, p


def test_routing_map_round_trip_and_padding_rows():
    rng = np.random.default_rng(41)
    T, E, K = 200, 64, 8
    ids = np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int32)
    ids[rng.random((T, K)) < 0.1] = -1
    ids[-7:] = -1                                   # padded rows: all-False, zero probs
    scores = rng.random((T, K)).astype(np.float32)
    m, p = _map_from_topk(ids, scores, E)
    got_ids, got_s, n = oracle.topk_from_routing_map(m, p, K)
    for t in range(T):
        valid = np.sort(ids[t][ids[t] >= 0])
        assert n[t] == valid.size
        assert got_ids[t, :valid.size].tolist() == valid.tolist()       # ascending experts
        assert (got_ids[t, valid.size:] == -1).all()
        assert np.array_equal(got_s[t, :valid.size], p[t, valid])
        assert (got_s[t, valid.size:] == 0).all()
    assert (n[-7:] == 0).all() and (got_ids[-7:] == -1).all()


def test_routing_map_row_with_more_than_k_experts_keeps_the_lowest():
    m = np.zeros((2, 10), np.uint8)
    m[0, [1, 3, 4, 7, 9]] = 1
    p = np.arange(20, dtype=np.float32).reshape(2, 10) / 8
    ids, s, n = oracle.topk_from_routing_map(m, p, 3)
    assert ids.tolist() == [[1, 3, 4], [-1, -1, -1]]
    assert s[0].tolist() == [p[0, 1], p[0, 3], p[0, 4]] and n.tolist() == [5, 0]


def test_routing_map_layout_matches_topk_layout_per_expert():
    # Both formats put the same tokens in each expert's segment, in token order.
    w = workloads.WORKLOADS["padded"]
    b = workloads.make_batch(w, with_x=False)
    T = 777
    m, p = _map_from_topk(b["ids"][:T], b["scores"][:T], w.E)
    ids2, s2, n = oracle.topk_from_routing_map(m, p, w.K)
    a = oracle.layout(b["ids"][:T], T, T, w.E, w.K)
    c = oracle.layout(ids2, T, T, w.E, w.K)
    np.testing.assert_array_equal(a["counts"], c["counts"])
    np.testing.assert_array_equal(a["offsets"], c["offsets"])
    np.testing.assert_array_equal(a["src"] // w.K, c["src"] // w.K)
    # and the slot scores travel with their experts
    sa = b["scores"][:T].ravel()[a["src"]]
    sc = s2.ravel()[c["src"]]
    assert np.array_equal(sa, sc)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_dispatch_scaled_is_one_rounded_product(dtype):
    w = workloads.Workload("sc", T=300, ntpr=300, nmax=300, D=48, E=32, K=4, dtype=dtype,
                           routing="uniform", seed=4)
    b = workloads.make_batch(w)
    lay = oracle.layout(b["ids"], w.T, w.ntpr, w.E, w.K)
    x_e = oracle.dispatch_scaled(b["x"], b["scores"], w.K, lay["src"])
    t = lay["src"] // w.K
    s = b["scores"].ravel()[lay["src"]]
    xf = b["x"].astype(np.float32) if dtype == "f32" else \
        (b["x"].astype(np.uint32) << 16).view(np.float32)
    prod = (s[:, None].astype(np.float32) * xf[t]).astype(np.float32)   # fp32 product
    want = prod if dtype == "f32" else _torch_bf16_bits(prod)
    assert np.array_equal(x_e, want)


def test_scaled_dispatch_with_unit_combine_matches_weighted_combine_when_exact():
    T, D, E, K = 40, 64, 8, 4
    x, ids, scores = _dyadic_inputs(T, D, 9)
    lay = oracle.layout(ids, T, T, E, K)
    xs = oracle.dispatch_scaled(x, scores, K, lay["src"])
    y_unit = oracle.combine(xs, lay["row_map"], np.ones((T, K), np.float32), T, K)
    x_e, _ = oracle.dispatch(x, scores, K, lay["src"])
    y_w = oracle.combine(x_e, lay["row_map"], scores, T, K)
    assert np.array_equal(y_unit, y_w)
