"""Host-side pieces of bench.py, on the CPU: the algorithmic byte counts
behind every reported rate, the counter-digest guard, and the refusal of
multi-GPU runs (this path has one GPU)."""
import json
import os
import subprocess
import sys

import numpy as np

import bench
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_dsv3_bytes_per_token_match_the_method():
    # T=4096, D=7168 bf16, K=8: dispatch reads x (14336 B), row_map and scores
    # (4K + 4K) and writes 8 rows and s_e (4K); combine reads 8 rows, row_map,
    # scores and writes one row.
    w = workloads.WORKLOADS["dsv3"]
    row = 7168 * 2
    assert bench.bytes_per_token(w, "dispatch") == row * 9 + 32 + 32 + 32 == 129120
    assert bench.bytes_per_token(w, "combine") == row * 9 + 32 + 32 == 129088
    assert bench.bytes_per_token(w, "layout") == 96
    # dispatch + combine per token, and over the batch (1.058 GB)
    both = bench.bytes_per_token(w, "dispatch") + bench.bytes_per_token(w, "combine")
    assert both == 258208 and both * w.T == 1057619968


def test_bytes_per_token_follow_dtype_and_topk():
    tiny = workloads.WORKLOADS["tiny"]               # fp32, D=128, K=2
    assert bench.bytes_per_token(tiny, "dispatch") == 128 * 4 * 3 + 24
    assert bench.bytes_per_token(tiny, "combine") == 128 * 4 * 3 + 16
    g = workloads.WORKLOADS["graph"]                 # bf16, D=4096, K=8
    assert bench.bytes_per_token(g, "combine_backward") == 4096 * 2 * 17 + 96
    assert bench.bytes_per_token(g, "dispatch_backward") == 4096 * 2 * 9 + 32


def test_expert_bytes_count_each_used_expert_once():
    counts = np.array([3, 0, 5, 1], np.int32)        # expert 1 has no rows
    k_in, n_out = 64, 32
    weights = 3 * n_out * k_in * 2                   # three experts with rows
    rows = 9 * (k_in + n_out) * 2                    # rows in and out
    assert bench.expert_algorithmic_bytes(counts, k_in, n_out) == weights + rows + 5 * 4


def test_counter_traffic_is_dropped_when_the_kernel_changed(tmp_path, monkeypatch):
    rec = {"kernel_source_sha256": bench.source_digest("combine"),
           "hbm_bytes_per_launch": 123}
    (tmp_path / "combine_dsv3_counters.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.counter_traffic("combine", "dsv3") == 123
    rec["kernel_source_sha256"] = "0" * 64
    (tmp_path / "combine_dsv3_counters.json").write_text(json.dumps(rec))
    assert bench.counter_traffic("combine", "dsv3") is None
    assert bench.counter_traffic("dispatch", "dsv3") is None       # no summary at all


def test_more_than_one_gpu_is_refused():
    for argv, env in ((["--gpus", "2"], {}), ([], {"WORLD_SIZE": "4"})):
        p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv],
                           capture_output=True, text=True, timeout=120,
                           env=dict(os.environ, **env))
        assert p.returncode == 2, p.stderr
        assert "one GPU only" in p.stderr and p.stdout == ""


def test_configs_cover_the_five_configurations_of_the_metric():
    """tiny; padded at T=3 and T=2047; both 32k prefills; the graph shape at
    T=8192, eager and replayed (the DSV3 shape is the line's top level)."""
    keys = [c[0] for c in bench.CONFIGS]
    assert keys == ["tiny", "padded_T3", "padded_T2047", "prefill32k_uniform",
                    "prefill32k_zipf", "graph_T8192"]
    for key, wname, T, graph, meaningful in bench.CONFIGS:
        w = workloads.WORKLOADS[wname]
        assert T is None or 0 < T <= w.ntpr <= w.nmax
        assert graph == (key == "graph_T8192")
        assert meaningful == (key not in ("tiny", "padded_T3"))


def test_host_cores_report_the_affinity():
    rec = bench.host_cores()
    assert rec["affinity"] == len(os.sched_getaffinity(0)) >= 1
    assert rec["cgroup_quota_cpus"] is None or rec["cgroup_quota_cpus"] > 0


def test_traffic_probe_library_is_built_apart_from_the_product():
    """bench.py's traffic reference kernels live in their own library; the
    product library exports none of them."""
    import ctypes

    from combine_moe_layout_05_amd import _lib
    from combine_moe_layout_05_amd._paths import PROBE_LIB_PATH
    probe = ctypes.CDLL(PROBE_LIB_PATH)
    assert hasattr(probe, "probe_gather_copy") and hasattr(probe, "probe_stream")
    product = _lib.load()
    assert not hasattr(product, "probe_gather_copy")
