"""GPU tests of moe_layout_noalloc, the layout entry point that allocates
nothing (its per-tile histograms live in the library's static device
scratch). Called through the C ABI and compared bit for bit with moe_layout
on a context (and with the oracle): two calls in a row, the second smaller,
then more sizes on the same scratch, the largest input the scratch admits,
and a rejected one that writes nothing."""
import ctypes as C

import numpy as np
import pytest
import torch

import oracle
from combine_moe_layout_05_amd import MoeDispatcher, layout_noalloc, round_up4
from combine_moe_layout_05_amd import _lib as L

from gpu_util import DEV, i32_dev, note, sync_or_fail

pytestmark = pytest.mark.gpu


def _ids(T, E, K, seed, zipf=0.0):
    """K distinct ids per token (Gumbel-top-K over E, Zipf-skewed when
    zipf > 0); for large T*E, independent uniform ids (repeats within a
    token are allowed: each slot gets its own row)."""
    rng = np.random.default_rng(seed)
    if T * E > 1 << 24:
        return np.ascontiguousarray(rng.integers(0, E, size=(T, K)).astype(np.int32))
    logp = -zipf * np.log(np.arange(1, E + 1)) if zipf else np.zeros(E)
    g = logp[None, :] + rng.gumbel(size=(T, E))
    return np.ascontiguousarray(np.argsort(-g, axis=1)[:, :K].astype(np.int32))


def _outputs(E, K, ntpr, T):
    """Output buffers filled with a poison value (0x5A5A5A5A)."""
    n4 = round_up4(ntpr)
    fill = 0x5A5A5A5A
    return {"counts": torch.full((E,), fill, dtype=torch.int32, device=DEV),
            "offsets": torch.full((E + 1,), fill, dtype=torch.int32, device=DEV),
            "row_map": torch.full((n4, K), fill, dtype=torch.int32, device=DEV),
            "src_map": torch.full((max(T * K, 1),), fill, dtype=torch.int32, device=DEV)}


def _call_abi(ids_d, T, ntpr, E, K, out):
    """moe_layout_noalloc through ctypes, on torch's current stream."""
    lib = L.load()
    stream = torch.cuda.current_stream(DEV).cuda_stream
    return lib.moe_layout_noalloc(C.c_void_p(ids_d.data_ptr() if T else 0), T, ntpr, E, K,
                                  out["counts"].data_ptr(), out["offsets"].data_ptr(),
                                  out["row_map"].data_ptr(), out["src_map"].data_ptr(),
                                  C.c_void_p(stream))


def _reference(disp, ids_d, ntpr):
    lay = disp.layout(ids_d, ntpr)
    sync_or_fail()
    total = int(lay.offsets[-1].item())
    return {"counts": lay.counts.cpu().numpy(), "offsets": lay.offsets.cpu().numpy(),
            "row_map": lay.row_map.cpu().numpy(), "src_map": disp.src_map[:total].cpu().numpy(),
            "total": total}


def _check(out, ref, T, K):
    sync_or_fail()
    total = ref["total"]
    np.testing.assert_array_equal(out["counts"].cpu().numpy(), ref["counts"])
    np.testing.assert_array_equal(out["offsets"].cpu().numpy(), ref["offsets"])
    np.testing.assert_array_equal(out["row_map"].cpu().numpy(), ref["row_map"])
    src = out["src_map"].cpu().numpy()
    np.testing.assert_array_equal(src[:total], ref["src_map"])
    # rows past the total are not written
    assert (src[total:] == 0x5A5A5A5A).all()


def test_two_calls_in_a_row_then_smaller_and_larger():
    E, K = 128, 8
    nmax = 40000
    disp = MoeDispatcher(nmax, 16, E, K, dtype=torch.bfloat16, device=DEV)
    # 65536 slots (two launches, 128 tiles), then 40000 (two launches, 79
    # tiles: a smaller input on the same scratch), then 1000 tokens (one
    # launch, no scratch), then 32768 tokens (256 tiles) and 8192 again.
    for i, (T, ntpr, zipf) in enumerate([(8192, 8192, 0.0), (4998, 5000, 1.1), (1000, 1003, 0.0),
                                         (32768, 32768, 1.2), (8192, 8192, 0.0)]):
        ids = _ids(T, E, K, seed=100 + i, zipf=zipf)
        ids_d = i32_dev(ids)
        out = _outputs(E, K, ntpr, T)
        note(f"layout_noalloc call {i}: T={T} ntpr={ntpr} E={E} K={K} "
             f"({round_up4(ntpr) * K} slots)")
        assert _call_abi(ids_d, T, ntpr, E, K, out) == L.MOE_OK
        ref = _reference(disp, ids_d, ntpr)
        _check(out, ref, T, K)
        o = oracle.layout(ids, T, ntpr, E, K)
        np.testing.assert_array_equal(ref["row_map"], o["row_map"])
        np.testing.assert_array_equal(ref["src_map"], o["src"])
    del disp
    torch.cuda.empty_cache()


def test_largest_input_the_scratch_admits_and_a_rejected_one():
    """1024 experts, 131072 tokens of 8 slots: 1024 tiles of 1024 slots, one
    4 KiB histogram row each = the whole 4 MiB scratch. Four more tokens
    need one more tile: MOE_ERR_SCRATCH, and nothing is written."""
    E, K, T = 1024, 8, 131072
    assert 1024 * 1024 * 4 == L.MOE_NOALLOC_SCRATCH_BYTES
    ids = _ids(T, E, K, seed=7)
    ids[::97, 3] = -1                          # some slots without an expert
    ids_d = i32_dev(ids)
    out = _outputs(E, K, T, T)
    note(f"layout_noalloc full scratch: T={T} E={E} K={K}")
    assert _call_abi(ids_d, T, T, E, K, out) == L.MOE_OK
    disp = MoeDispatcher(T + 4, 16, E, K, dtype=torch.bfloat16, device=DEV)
    ref = _reference(disp, ids_d, T)
    _check(out, ref, T, K)
    o = oracle.layout(ids, T, T, E, K)
    np.testing.assert_array_equal(ref["row_map"], o["row_map"])

    note("layout_noalloc over the scratch limit is rejected on the host")
    big = _outputs(E, K, T + 4, T)
    assert _call_abi(ids_d, T, T + 4, E, K, big) == L.MOE_ERR_SCRATCH
    sync_or_fail()
    for name, t in big.items():
        assert bool((t == 0x5A5A5A5A).all()), name
    with pytest.raises(L.MoeError):
        layout_noalloc(ids_d, E, big["counts"], big["offsets"], big["row_map"], big["src_map"],
                       num_tokens_per_rank=T + 4)
    del disp
    torch.cuda.empty_cache()


def test_binding_and_empty_batch():
    """The binding passes the same arguments; T = 0 writes zero counts,
    offsets and an all -1 row map."""
    E, K = 8, 2
    for T, ntpr in ((61, 64), (0, 6)):
        ids = _ids(T, E, K, seed=3) if T else np.zeros((0, K), np.int32)
        ids_d = i32_dev(ids) if T else torch.zeros((0, K), dtype=torch.int32, device=DEV)
        out = _outputs(E, K, ntpr, T)
        note(f"layout_noalloc binding T={T} ntpr={ntpr}")
        layout_noalloc(ids_d, E, out["counts"], out["offsets"], out["row_map"], out["src_map"],
                       num_tokens_per_rank=ntpr)
        sync_or_fail()
        o = oracle.layout(ids, T, ntpr, E, K)
        np.testing.assert_array_equal(out["counts"].cpu().numpy(), o["counts"])
        np.testing.assert_array_equal(out["offsets"].cpu().numpy(), o["offsets"])
        np.testing.assert_array_equal(out["row_map"].cpu().numpy(), o["row_map"])
        np.testing.assert_array_equal(out["src_map"].cpu().numpy()[:o["total"]], o["src"])
