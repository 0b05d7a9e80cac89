"""Seeded synthetic inputs for MoE token layout, dispatch and combine.

This module only draws random inputs: hidden states, top-k expert ids and
top-k scores, shaped like the MoE workloads of the source pages. It holds no
layout, dispatch or combine arithmetic, so both the CPU oracle's tests and the
HIP path's tests, the smoke check and the benchmark can take their inputs from
here without sharing any of the method.

Representation (all NumPy, C-contiguous):
  x       float32 [T, D] for fp32 workloads, uint16 [T, D] bf16 bit patterns
          for bf16 workloads (N(0,1) draws rounded to bf16 by torch's CPU
          conversion, which rounds to nearest even)
  ids     int32   [T, K] expert ids, K distinct ids per token
  scores  float32 [T, K]

Routing draws use Gumbel-top-k (Kool, van Hoof & Welling 2019): adding
independent Gumbel noise to log-probabilities and keeping the K largest gives
K distinct ids sampled without replacement; the slots keep the sampling order
(largest perturbed logit first).
"""
from __future__ import annotations

import dataclasses
import os
from typing import Optional

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "make_batch", "replay_T", "replay_batch",
    "x_to_torch_dtype_name", "EXPERT_SHAPES", "expert_weights", "expert_rows",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload shape.

    T: materialized tokens, ntpr: num_tokens_per_rank for a call, nmax:
    num_max_tokens_per_rank the buffers are sized for.
    """
    name: str
    T: int
    ntpr: int
    nmax: int
    D: int
    E: int
    K: int
    dtype: str            # "f32" or "bf16"
    routing: str          # "uniform" or "zipf"
    zipf_s: float = 0.0
    scores: str = "softmax"   # "softmax" or "sigmoid_norm"
    seed: int = 0


# Shapes of the pages' MoE workloads, restated as synthetic configurations.
WORKLOADS = {
    # Tiny fp32 case the oracle finishes instantly.
    "tiny": Workload("tiny", T=64, ntpr=64, nmax=64, D=128, E=8, K=2,
                     dtype="f32", routing="uniform", scores="softmax", seed=0),
    # Unequal/unaligned token counts (the pages' 3,5,7,13 and 614,2047) as
    # prefixes of one 2048-row batch; capacity 2048, lifetime max 4096.
    "padded": Workload("padded", T=2048, ntpr=2048, nmax=4096, D=2048, E=128,
                       K=8, dtype="bf16", routing="uniform", scores="softmax",
                       seed=0),
    # DeepSeek-V3-shaped layer: 4096 tokens, hidden 7168, 256 experts, top-8.
    "dsv3": Workload("dsv3", T=4096, ntpr=4096, nmax=4096, D=7168, E=256, K=8,
                     dtype="bf16", routing="zipf", zipf_s=1.1,
                     scores="sigmoid_norm", seed=0),
    # 32k-token prefill with the same dims, uniform and skewed routing.
    "prefill32k_uniform": Workload("prefill32k_uniform", T=32768, ntpr=32768,
                                   nmax=32768, D=7168, E=256, K=8, dtype="bf16",
                                   routing="uniform", scores="sigmoid_norm",
                                   seed=0),
    "prefill32k_zipf": Workload("prefill32k_zipf", T=32768, ntpr=32768,
                                nmax=32768, D=7168, E=256, K=8, dtype="bf16",
                                routing="zipf", zipf_s=1.2,
                                scores="sigmoid_norm", seed=1),
    # Worst-token graph capture: buffers for 8192 tokens, T varies per replay.
    "graph": Workload("graph", T=8192, ntpr=8192, nmax=8192, D=4096, E=128,
                      K=8, dtype="bf16", routing="uniform", scores="softmax",
                      seed=1000),
}

PADDED_T_VALUES = (3, 5, 7, 13, 614, 2047)
PADDED_PAIRS = ((8, 3), (6, 6), (5, 3), (13, 7))
GRAPH_REPLAYS = 100
GRAPH_T_MIN = 41


def x_to_torch_dtype_name(dtype: str) -> str:
    return {"f32": "float32", "bf16": "bfloat16"}[dtype]


def _draw_x(rng: np.random.Generator, T: int, D: int, dtype: str) -> np.ndarray:
    x = rng.standard_normal((T, D), dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype != "bf16":
        raise ValueError(f"unknown dtype {dtype!r}")
    import torch  # CPU conversion only: float32 -> bfloat16, round to nearest even
    xb = torch.from_numpy(x).to(torch.bfloat16)
    return xb.view(torch.int16).numpy().view(np.uint16).copy()


def _draw_ids(rng: np.random.Generator, T: int, E: int, K: int,
              routing: str, zipf_s: float) -> np.ndarray:
    if K > E:
        raise ValueError("K distinct experts need K <= E")
    if routing == "uniform":
        logp = np.zeros(E, dtype=np.float64)
    elif routing == "zipf":
        logp = -zipf_s * np.log(np.arange(1, E + 1, dtype=np.float64))
    else:
        raise ValueError(f"unknown routing {routing!r}")
    g = logp[None, :] + rng.gumbel(size=(T, E))
    top = np.argpartition(-g, K - 1, axis=1)[:, :K]
    order = np.argsort(-np.take_along_axis(g, top, axis=1), axis=1, kind="stable")
    return np.ascontiguousarray(np.take_along_axis(top, order, axis=1).astype(np.int32))


def _draw_scores(rng: np.random.Generator, T: int, K: int, kind: str) -> np.ndarray:
    logits = rng.standard_normal((T, K))
    if kind == "softmax":
        z = np.exp(logits - logits.max(axis=1, keepdims=True))
        s = z / z.sum(axis=1, keepdims=True)
    elif kind == "sigmoid_norm":
        sig = 1.0 / (1.0 + np.exp(-logits))
        s = sig / sig.sum(axis=1, keepdims=True)
    else:
        raise ValueError(f"unknown score kind {kind!r}")
    return np.ascontiguousarray(s.astype(np.float32))


def make_batch(w: Workload, T: Optional[int] = None, seed: Optional[int] = None,
               with_x: bool = True) -> dict:
    """Draw one batch of T rows (default w.T) for workload w.

    x, ids and scores come from three independent child streams of
    SeedSequence(seed), so the routing of a batch does not depend on whether
    x was drawn, and a shorter T is not a prefix of a longer one (take
    prefixes explicitly where the prefix property is wanted).
    """
    T = w.T if T is None else T
    seed = w.seed if seed is None else seed
    sx, si, ss = np.random.SeedSequence(seed).spawn(3)
    out = {
        "ids": _draw_ids(np.random.default_rng(si), T, w.E, w.K, w.routing, w.zipf_s),
        "scores": _draw_scores(np.random.default_rng(ss), T, w.K, w.scores),
    }
    if with_x:
        out["x"] = _draw_x(np.random.default_rng(sx), T, w.D, w.dtype)
    return out


def replay_T(i: int, nmax: int = 8192, t_min: int = GRAPH_T_MIN) -> int:
    """Token count of graph replay i: 41 first, then the full 8192, then
    uniform in [41, nmax] from seed 1000+i."""
    if i == 0:
        return t_min
    if i == 1:
        return nmax
    return int(np.random.default_rng(1000 + i).integers(t_min, nmax + 1))


def replay_batch(i: int, w: Workload = WORKLOADS["graph"]) -> dict:
    """Fresh routing and hidden states for graph replay i (seed 1000+i)."""
    T = replay_T(i, w.nmax)
    b = make_batch(w, T=T, seed=w.seed + i)
    b["T"] = T
    return b


# Expert step (one linear map per expert between dispatch and combine). The
# pages fix no expert width; "dsv3" uses DeepSeek-V3's routed-expert width
# 2048, with gate and up projections fused: k_in = hidden 7168 -> n_out 4096.
EXPERT_SHAPES = {
    "dsv3": dict(workload="dsv3", k_in=7168, n_out=4096, seed=2024),
    "prefill32k_zipf": dict(workload="prefill32k_zipf", k_in=7168, n_out=4096, seed=2024),
    "prefill32k_uniform": dict(workload="prefill32k_uniform", k_in=7168, n_out=4096, seed=2024),
}


def expert_weights(E: int, n_out: int, k_in: int, seed: int) -> np.ndarray:
    """uint16 [E, n_out, k_in] bf16 bit patterns: uniform random sign and
    7-bit mantissa, exponent uniform over 2^-11 .. 2^-4 (magnitudes of a
    k_in-wide linear layer's weights). Expert e draws raw 64-bit words from
    its own stream (SeedSequence(seed).spawn(E)[e]), four 16-bit fields per
    word, on a thread pool, so the 15 GB of the dsv3 shape take seconds."""
    from concurrent.futures import ThreadPoolExecutor

    out = np.empty((E, n_out, k_in), np.uint16)
    n = n_out * k_in
    words = (n + 3) // 4
    keep = np.uint64(0x807F807F807F807F)      # sign and mantissa of 4 fields
    low3 = np.uint64(0x0007000700070007)
    bias = np.uint64(0x0074007400740074)      # 116 in every field
    streams = np.random.SeedSequence(seed).spawn(E)

    def fill(e):
        rng = np.random.default_rng(streams[e])
        w = rng.integers(0, 2 ** 64 - 1, size=words, dtype=np.uint64, endpoint=True)
        w = (w & keep) | ((((w >> np.uint64(7)) & low3) + bias) << np.uint64(7))
        out[e] = w.view(np.uint16)[:n].reshape(n_out, k_in)

    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(fill, range(E)))
    return out


def expert_rows(rows: int, k_in: int, seed: int) -> np.ndarray:
    """uint16 [rows, k_in] bf16 bits of N(0,1) draws (expert input rows)."""
    rng = np.random.default_rng(seed)
    return _draw_x(rng, rows, k_in, "bf16")
