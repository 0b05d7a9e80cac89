"""The benchmark's traffic reference kernels move the bytes they claim: the
gather-copy stores, for every token, the XOR of the K expert-major rows its
row map names (no-expert slots skipped), over the combine's launch shape;
the sequential mix stores the XOR of each 8 KiB block. Checked against torch
bit operations on the same buffers."""
import ctypes

import numpy as np
import pytest
import torch

from combine_moe_layout_05_amd._paths import PROBE_LIB_PATH

from gpu_util import DEV, note, sync_or_fail

pytestmark = pytest.mark.gpu


def _lib():
    lib = ctypes.CDLL(PROBE_LIB_PATH)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.probe_gather_copy.argtypes = [vp, vp, i32, i32, i32, i64, vp, vp, ctypes.c_int, vp]
    lib.probe_stream.argtypes = [ctypes.c_int, vp, vp, i64, vp, vp]
    return lib


def _stream():
    return torch.cuda.current_stream(DEV).cuda_stream


@pytest.mark.parametrize("T,K,chunks,rows", [(37, 8, 896, 300), (300, 3, 5, 1000), (64, 1, 64, 64)])
def test_gather_copy_stores_the_xor_of_each_tokens_rows(T, K, chunks, rows):
    lib = _lib()
    g = torch.Generator(device="cpu").manual_seed(T)
    src = torch.randint(-2**31, 2**31 - 1, (rows, chunks * 4), dtype=torch.int32, generator=g)
    rm = torch.randint(0, rows, (T, K), dtype=torch.int32, generator=g)
    rm[::5, 0] = -1                       # no expert
    rm[1::7, -1] = rows + 3               # outside the row limit: skipped too
    src_d, rm_d = src.to(DEV), rm.to(DEV)
    out = torch.full((T, chunks * 4), 7, dtype=torch.int32, device=DEV)
    sink = torch.full((4,), 0x7FC17FC1, dtype=torch.int32, device=DEV)
    note(f"probe gather_copy T={T} K={K} chunks={chunks}")
    assert lib.probe_gather_copy(src_d.data_ptr(), rm_d.data_ptr(), T, K, chunks, rows,
                                 out.data_ptr(), sink.data_ptr(), 1, _stream()) == 0
    assert lib.probe_gather_copy(src_d.data_ptr(), rm_d.data_ptr(), T, K, chunks, rows,
                                 out.data_ptr(), sink.data_ptr(), 0, _stream()) == 0
    sync_or_fail()
    want = torch.zeros((T, chunks * 4), dtype=torch.int32)
    for t in range(T):
        for k in range(K):
            r = int(rm[t, k])
            if 0 <= r < rows:
                want[t] ^= src[r]
    assert torch.equal(out.cpu(), want)
    assert int(sink[0].item()) == 0x7FC17FC1   # the read-only pass stored nothing


def test_sequential_mix_and_streams():
    lib = _lib()
    n = 1 << 20                                # bytes read
    a = torch.randint(-2**31, 2**31 - 1, (n // 4,), dtype=torch.int32, device=DEV)
    b = torch.zeros((n // 32,), dtype=torch.int32, device=DEV)
    sink = torch.full((4,), 0x7FC17FC1, dtype=torch.int32, device=DEV)
    note("probe streams")
    assert lib.probe_stream(2, a.data_ptr(), b.data_ptr(), n, sink.data_ptr(), _stream()) == 0
    assert lib.probe_stream(0, a.data_ptr(), None, n, sink.data_ptr(), _stream()) == 0
    sync_or_fail()
    # wavefront w reads 8 consecutive KiB (256 int32 each) and writes 1 KiB:
    # lane l's 16 bytes are the XOR of the same lane's 16 bytes of each KiB
    blocks = a.view(-1, 8, 256).cpu()
    want = blocks[:, 0]
    for i in range(1, 8):
        want = want ^ blocks[:, i]
    assert torch.equal(b.cpu(), want.reshape(-1))
    c = torch.zeros((n // 4,), dtype=torch.int32, device=DEV)
    assert lib.probe_stream(1, None, c.data_ptr(), n, sink.data_ptr(), _stream()) == 0
    sync_or_fail()
    idx = torch.arange(n // 16, dtype=torch.int32)
    want_w = torch.stack([idx, torch.ones_like(idx), 2 * torch.ones_like(idx),
                          3 * torch.ones_like(idx)], dim=1).reshape(-1)
    assert torch.equal(c.cpu(), want_w)
    assert lib.probe_stream(2, a.data_ptr(), b.data_ptr(), n + 16, sink.data_ptr(), _stream()) != 0
    # kind 3: each KiB of a written to eight consecutive KiB of d
    m = 1 << 16
    d = torch.zeros((8 * m // 4,), dtype=torch.int32, device=DEV)
    assert lib.probe_stream(3, a.data_ptr(), d.data_ptr(), m, sink.data_ptr(), _stream()) == 0
    sync_or_fail()
    src = a[: m // 4].view(-1, 256).cpu()
    assert torch.equal(d.view(-1, 8, 256).cpu(), src[:, None, :].expand(-1, 8, -1))
    assert lib.probe_stream(3, a.data_ptr(), d.data_ptr(), m + 16, sink.data_ptr(), _stream()) != 0
