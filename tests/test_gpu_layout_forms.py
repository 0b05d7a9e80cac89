"""The routing layout in its two launch forms against each other and against
the oracle: one launch (every workgroup counts the whole batch into LDS, then
ranks its own tile) and two (per-tile counts, then offsets and ranks). Counts,
offsets, row map and source map must be bit-identical between the forms, the
automatic choice and the oracle, across the workload shapes, the tile-size
switches of both forms, batches past the one-launch limit, invalid and
duplicate ids, and empty batches."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from combine_moe_layout_05_amd import MoeDispatcher, round_up4

from gpu_util import DEV, i32_dev, note, sync_or_fail

pytestmark = pytest.mark.gpu

# (name, T, ntpr, nmax, E, K, routing, zipf_s, seed)
CASES = [
    ("tiny", 64, 64, 64, 8, 2, "uniform", 0.0, 0),
    ("padded_T614", 614, 2048, 4096, 128, 8, "uniform", 0.0, 1),
    ("dsv3", 4096, 4096, 4096, 256, 8, "zipf", 1.1, 0),
    ("just_past_32768_slots", 4097, 4097, 4100, 256, 8, "zipf", 1.1, 2),
    ("graph", 8192, 8192, 8192, 128, 8, "uniform", 0.0, 3),
    ("prefill32k_zipf", 32768, 32768, 32768, 256, 8, "zipf", 1.2, 1),
    ("E1024_K16", 3000, 3001, 4096, 1024, 16, "zipf", 1.1, 4),
    ("E1_K1", 777, 778, 800, 1, 1, "uniform", 0.0, 5),
    ("E3_K2_ragged", 1001, 1003, 1100, 3, 2, "uniform", 0.0, 6),
    ("past_one_launch_limit", 40000, 40000, 40000, 64, 16, "zipf", 1.2, 7),
]


def _ids(T, E, K, routing, s, seed, bad=False, dup=False):
    rng = np.random.default_rng(seed)
    ids = workloads._draw_ids(rng, T, E, K, routing, s) if T else np.zeros((0, K), np.int32)
    if bad and T:
        flat = ids.reshape(-1)
        pick = rng.choice(flat.size, size=max(1, flat.size // 17), replace=False)
        flat[pick] = rng.choice(np.array([-1, E, E + 7, -2**31, 2**31 - 1], np.int32), pick.size)
    if dup and T and K > 1:
        ids[::3, 1] = ids[::3, 0]
    return np.ascontiguousarray(ids, dtype=np.int32)


def _run(disp, ids_np, T, ntpr, launches):
    disp.set_tuning(layout_launches=launches)
    lay = disp.layout(i32_dev(ids_np), ntpr)
    sync_or_fail()
    total = int(lay.offsets[-1].item())
    return {"counts": lay.counts.cpu().numpy().copy(), "offsets": lay.offsets.cpu().numpy().copy(),
            "row_map": lay.row_map.cpu().numpy().copy(),
            "src": disp.src_map[:total].cpu().numpy().copy(), "total": total}


def _check(name, T, ntpr, nmax, E, K, ids_np):
    # D = 64 bf16 (128-byte rows): the layout does not depend on D, and the
    # expert buffer stays small at the largest slot counts.
    disp = MoeDispatcher(nmax, 64, E, K, dtype=torch.bfloat16, device=DEV)
    slots = round_up4(ntpr) * K
    res = {}
    for launches in (1, 2, -1):
        note(f"layout form {launches}: {name} T={T} ntpr={ntpr} E={E} K={K} slots={slots}")
        res[launches] = _run(disp, ids_np, T, ntpr, launches)
    o = oracle.layout(ids_np, T, ntpr, E, K)
    for launches, g in res.items():
        assert g["total"] == o["total"], (launches, g["total"], o["total"])
        assert np.array_equal(g["counts"], o["counts"]), f"counts, form {launches}"
        assert np.array_equal(g["offsets"], o["offsets"]), f"offsets, form {launches}"
        assert np.array_equal(g["row_map"].reshape(-1), o["row_map"].reshape(-1)), \
            f"row_map, form {launches}"
        assert np.array_equal(g["src"], o["src"]), f"src_map, form {launches}"
    del disp


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_layout_forms_match_each_other_and_the_oracle(case):
    name, T, ntpr, nmax, E, K, routing, s, seed = case
    _check(name, T, ntpr, nmax, E, K, _ids(T, E, K, routing, s, seed))


def test_layout_forms_with_invalid_and_duplicate_ids():
    T, ntpr, nmax, E, K = 5000, 5003, 5004, 256, 8
    ids = _ids(T, E, K, "zipf", 1.1, 11, bad=True, dup=True)
    _check("bad_and_duplicate_ids", T, ntpr, nmax, E, K, ids)


@pytest.mark.parametrize("ntpr", [0, 8])
def test_layout_forms_empty_batch(ntpr):
    _check("empty", 0, ntpr, 16, 32, 4, np.zeros((0, 4), np.int32))


def test_layout_forms_all_slots_without_expert():
    T, E, K = 300, 16, 4
    _check("no_expert", T, T, T, E, K, np.full((T, K), -1, np.int32))


def test_layout_forms_alternate_on_one_context():
    """Switching forms between calls on one context leaves no state behind."""
    T, ntpr, nmax, E, K = 2048, 2048, 2048, 128, 8
    disp = MoeDispatcher(nmax, 64, E, K, dtype=torch.bfloat16, device=DEV)
    a = _ids(T, E, K, "zipf", 1.1, 21)
    b = _ids(T, E, K, "uniform", 0.0, 22)
    ref = {"a": oracle.layout(a, T, ntpr, E, K), "b": oracle.layout(b, T, ntpr, E, K)}
    for i, (key, launches) in enumerate([("a", 1), ("b", 2), ("a", 2), ("b", 1), ("a", 1)]):
        note(f"alternating layout forms, call {i}: batch {key}, form {launches}")
        g = _run(disp, a if key == "a" else b, T, ntpr, launches)
        assert np.array_equal(g["row_map"].reshape(-1), ref[key]["row_map"].reshape(-1))
        assert np.array_equal(g["src"], ref[key]["src"])
        assert np.array_equal(g["offsets"], ref[key]["offsets"])
    del disp


@pytest.mark.parametrize("shift", [1, 2, 3])
@pytest.mark.parametrize("shape", [(4096, 4096, 256, 8), (1001, 1003, 3, 3), (5, 8, 16, 2)],
                         ids=["dsv3", "ragged_K3", "tiny_T5"])
def test_layout_forms_ids_off_16_byte_alignment(shift, shape):
    """Ids whose device address is 4, 8 or 12 bytes past a 16-byte boundary (a
    view into a larger buffer): the one-launch count reads the slots before
    the first boundary and after the last whole quad one by one, and decides
    per slot which side of the tile start each falls on."""
    T, ntpr, E, K = shape
    ids = _ids(T, E, K, "zipf" if E > 8 else "uniform", 1.1, 30 + shift, bad=True)
    buf = torch.full((T * K + 8,), -1, dtype=torch.int32, device=DEV)
    view = buf[shift:shift + T * K].view(T, K)
    view.copy_(i32_dev(ids))
    assert view.data_ptr() % 16 == 4 * shift
    disp = MoeDispatcher(ntpr + 1, 64, E, K, dtype=torch.bfloat16, device=DEV)
    o = oracle.layout(ids, T, ntpr, E, K)
    for launches in (1, 2):
        note(f"layout form {launches}: ids shifted by {4 * shift} bytes, T={T} E={E} K={K}")
        disp.set_tuning(layout_launches=launches)
        lay = disp.layout(view, ntpr)
        sync_or_fail()
        total = int(lay.offsets[-1].item())
        assert total == o["total"]
        assert np.array_equal(lay.counts.cpu().numpy(), o["counts"])
        assert np.array_equal(lay.offsets.cpu().numpy(), o["offsets"])
        assert np.array_equal(lay.row_map.cpu().numpy().reshape(-1), o["row_map"].reshape(-1))
        assert np.array_equal(disp.src_map[:total].cpu().numpy(), o["src"])
    del disp
