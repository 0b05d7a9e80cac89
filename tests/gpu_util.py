"""Helpers for the GPU parity tests: move seeded NumPy inputs to the device,
run the HIP path through the binding, and compare with the oracle to the bar
the tests state (bit-exact for integer and copied data; fp32 combine within
1e-5 relative; bf16 combine within 1 ulp)."""
import os
import sys

import numpy as np
import torch

DEV = torch.device("cuda", 0)
ORACLE_THREADS = max(1, min(16, len(os.sched_getaffinity(0))))


def note(msg: str) -> None:
    """Name the case on stdout before each GPU step."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def sync_or_fail(timeout_s: float = 30.0, stream=None) -> None:
    """Wait for the stream by polling it against a deadline, so a hang turns
    into a test failure instead of a blocked process."""
    import time
    s = stream if stream is not None else torch.cuda.current_stream(DEV)
    deadline = time.monotonic() + timeout_s
    while not s.query():
        if time.monotonic() > deadline:
            raise TimeoutError(f"GPU work did not finish within {timeout_s} s")
        time.sleep(0.0005)
    torch.cuda.synchronize()


def x_to_dev(x: np.ndarray) -> torch.Tensor:
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def x_to_np(t: torch.Tensor) -> np.ndarray:
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def i32_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def f32_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def torch_dtype(x: np.ndarray) -> torch.dtype:
    return torch.bfloat16 if x.dtype == np.uint16 else torch.float32


def run_gpu(disp, x, ids, scores, T, ntpr, y_expert=None, copy_x_e=True):
    """layout -> dispatch -> (identity expert unless y_expert) -> combine on
    the first T rows; returns host copies of every output."""
    x_d = x_to_dev(x[:T]) if T else torch.empty((0, disp.hidden), dtype=disp.dtype, device=DEV)
    ids_d = i32_dev(ids[:T].reshape(T, disp.topk))
    s_d = f32_dev(scores[:T].reshape(T, disp.topk))
    lay = disp.layout(ids_d, ntpr)
    dsp = disp.dispatch(x_d, s_d, ids_d, lay.counts, num_tokens_per_rank=ntpr)
    ye = dsp.x_e if y_expert is None else y_expert
    y = disp.combine(ye, lay.row_map, s_d, num_tokens_per_rank=ntpr)
    sync_or_fail()
    total = int(lay.offsets[-1].item())
    out = {
        "counts": lay.counts.cpu().numpy(),
        "offsets": lay.offsets.cpu().numpy(),
        "row_map": lay.row_map.cpu().numpy(),
        "src": disp.src_map[:total].cpu().numpy(),
        "s_e": disp.s_e[:total].cpu().numpy(),
        "y": x_to_np(y),
        "total": total,
    }
    if copy_x_e:
        out["x_e"] = x_to_np(disp.x_e[:total])
    return out


def bf16_ulp_distance(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    def key(u):
        u = u.astype(np.int32)
        mag = u & 0x7FFF
        return np.where(u & 0x8000, -mag, mag)
    return np.abs(key(a) - key(b))


def assert_combine_within_bar(y_gpu: np.ndarray, y_orc: np.ndarray) -> None:
    """fp32: |gpu - oracle| <= 1e-5 |oracle|; bf16: at most 1 ulp apart."""
    assert y_gpu.shape == y_orc.shape and y_gpu.dtype == y_orc.dtype
    if y_gpu.dtype == np.uint16:
        assert not np.any((y_orc & 0x7FFF) > 0x7F80), "oracle produced NaN"
        d = bf16_ulp_distance(y_gpu, y_orc)
        assert d.max(initial=0) <= 1, f"max bf16 ulp distance {d.max()}"
    else:
        a = y_gpu.astype(np.float64)
        b = y_orc.astype(np.float64)
        assert np.all(np.isfinite(b))
        assert np.all(np.abs(a - b) <= 1e-5 * np.abs(b)), "fp32 combine beyond 1e-5 relative"


def assert_layout_equal(g: dict, o: dict, T: int) -> None:
    np.testing.assert_array_equal(g["counts"], o["counts"])
    np.testing.assert_array_equal(g["offsets"], o["offsets"])
    assert g["total"] == o["total"]
    np.testing.assert_array_equal(g["row_map"], o["row_map"])
    np.testing.assert_array_equal(g["src"], o["src"])


def assert_dispatch_equal(g: dict, o: dict) -> None:
    assert g["x_e"].shape == o["x_e"].shape
    assert np.array_equal(g["x_e"].view(np.uint8), o["x_e"].view(np.uint8))
    assert np.array_equal(g["s_e"].view(np.uint32), o["s_e"].view(np.uint32))
