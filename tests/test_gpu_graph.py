"""hipGraph capture and replay of layout -> dispatch -> expert -> combine.

Worst-token mode ("ep: graph-safe worst-token HT dispatch+combine", sections
"Summary" and "Tests"): the graph is captured once at the lifetime maximum
(8192 tokens); before each replay fresh routing is written into the captured
input tensors with rows past the replay's T set to id -1 and score 0. Every
replay is checked against the oracle on its own T, some against an eager run
of the same inputs bitwise, and eager calls on the same context are
interleaved with the replays."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from combine_moe_layout_05_amd import MoeDispatcher

from gpu_util import (DEV, ORACLE_THREADS, assert_combine_within_bar, f32_dev, i32_dev,
                      note, sync_or_fail, x_to_dev, x_to_np)

pytestmark = pytest.mark.gpu

W = workloads.WORKLOADS["graph"]
CHUNKS = 4
PER_CHUNK = workloads.GRAPH_REPLAYS // CHUNKS


def _double_bf16(x_bits: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).view(torch.bfloat16) * 2
    return t.view(torch.int16).numpy().view(np.uint16)


class Captured:
    """Static inputs, the dispatcher and one captured graph."""

    def __init__(self, tuning=None):
        N, D, K = W.nmax, W.D, W.K
        self.disp = MoeDispatcher(N, D, W.E, K, dtype=torch.bfloat16, device=DEV)
        if tuning:
            self.disp.set_tuning(**tuning)
        self.x = torch.zeros((N, D), dtype=torch.bfloat16, device=DEV)
        self.ids = torch.full((N, K), -1, dtype=torch.int32, device=DEV)
        self.s = torch.zeros((N, K), dtype=torch.float32, device=DEV)
        self.y_e = torch.zeros((self.disp.desc.max_rows, D), dtype=torch.bfloat16, device=DEV)
        side = torch.cuda.Stream(device=DEV)
        side.wait_stream(torch.cuda.current_stream(DEV))
        with torch.cuda.stream(side):          # warm-up outside the capture
            self._body()
        torch.cuda.current_stream(DEV).wait_stream(side)
        sync_or_fail()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self.y = self._body()
        sync_or_fail()
        self.eager_calls = 0

    def _body(self):
        d = self.disp
        lay = d.layout(self.ids, W.nmax)
        d.dispatch(self.x, self.s, self.ids, lay.counts, num_tokens_per_rank=W.nmax)
        torch.mul(d.x_e, 2, out=self.y_e)      # the expert: exact doubling in bf16
        return d.combine(self.y_e, lay.row_map, self.s, num_tokens_per_rank=W.nmax)

    def load(self, b):
        T = b["T"]
        self.x[:T].copy_(x_to_dev(b["x"]))
        self.x[T:].zero_()
        self.ids[:T].copy_(i32_dev(b["ids"]))
        self.ids[T:].fill_(-1)
        self.s[:T].copy_(f32_dev(b["scores"]))
        self.s[T:].zero_()

    def eager(self, x, ids, scores, T, ntpr):
        d = self.disp
        ids_d, s_d = i32_dev(ids[:T]), f32_dev(scores[:T])
        lay = d.layout(ids_d, ntpr)
        d.dispatch(x_to_dev(x[:T]), s_d, ids_d, lay.counts, num_tokens_per_rank=ntpr)
        ye = d.x_e[: lay.row_map.shape[0] * W.K] * 2
        y = d.combine(ye, lay.row_map, s_d, num_tokens_per_rank=ntpr)
        sync_or_fail()
        self.eager_calls += 1
        return x_to_np(y), lay.counts.cpu().numpy(), lay.offsets.cpu().numpy()


@pytest.fixture(scope="module")
def cap():
    note("graph: capture at 8192 tokens")
    c = Captured()
    yield c
    del c
    torch.cuda.empty_cache()


def _oracle(b, T, ntpr):
    return oracle.run_pipeline(_double_bf16(b["x"][:T]), b["ids"], b["scores"], T, ntpr,
                               W.E, W.K, nthreads=ORACLE_THREADS)


@pytest.mark.parametrize("chunk", range(CHUNKS))
def test_graph_replays_with_fresh_routing(cap, chunk):
    for i in range(chunk * PER_CHUNK, (chunk + 1) * PER_CHUNK):
        b = workloads.replay_batch(i)
        T = b["T"]
        note(f"graph replay {i} T={T}")
        cap.load(b)
        if i % 10 == 7:
            # poison every persistent buffer between replays: the replay must
            # rebuild everything it reads (no state carries over)
            cap.disp.workspace.fill_(0xFF)
            cap.y_e.fill_(0xFF)
        cap.graph.replay()
        sync_or_fail()
        y = x_to_np(cap.y)
        o = _oracle(b, T, T)
        np.testing.assert_array_equal(cap.disp.counts.cpu().numpy(), o["counts"])
        assert int(cap.disp.offsets[-1].item()) == o["total"] == T * W.K
        assert_combine_within_bar(y[:T], o["y"])
        assert np.array_equal(y[:T], o["y"])
        assert (y[T:] == 0).all()               # sentinel rows: +0.0, sliced off
        if i % 10 == 5:
            # replay == eager run of the same inputs, bitwise
            ye, ce, _ = cap.eager(b["x"], b["ids"], b["scores"], T, T)
            assert np.array_equal(ye, y[:T])
            np.testing.assert_array_equal(ce, o["counts"])
        if i % 10 == 9:
            # an unrelated eager batch on the same context between replays
            w2 = workloads.Workload("interleave", T=777 + i, ntpr=800 + i, nmax=W.nmax, D=W.D,
                                    E=W.E, K=W.K, dtype="bf16", routing="zipf", zipf_s=1.1,
                                    seed=5000 + i)
            b2 = workloads.make_batch(w2)
            note(f"eager interleave after replay {i}: T={w2.T} ntpr={w2.ntpr}")
            ye, ce, oe = cap.eager(b2["x"], b2["ids"], b2["scores"], w2.T, w2.ntpr)
            o2 = _oracle(b2, w2.T, w2.ntpr)
            np.testing.assert_array_equal(ce, o2["counts"])
            np.testing.assert_array_equal(oe, o2["offsets"])
            assert np.array_equal(ye, o2["y"])


@pytest.fixture(scope="module")
def cap_other_forms():
    # The one-launch layout (forced at 65536 slots: 2048-slot tiles) and
    # back-to-back dispatch stores, the forms the defaults do not take here.
    note("graph: capture at 8192 tokens, one-launch layout, back-to-back stores")
    c = Captured(tuning={"layout_launches": 1, "dispatch_store_burst": 1})
    yield c
    del c
    torch.cuda.empty_cache()


def test_graph_replays_other_launch_forms(cap_other_forms):
    c = cap_other_forms
    for i in list(range(0, 12)) + [17, 27, 37, 45, 59]:
        b = workloads.replay_batch(i)
        T = b["T"]
        note(f"graph replay (other forms) {i} T={T}")
        c.load(b)
        if i % 10 == 7:
            c.disp.workspace.fill_(0xFF)
            c.y_e.fill_(0xFF)
        c.graph.replay()
        sync_or_fail()
        y = x_to_np(c.y)
        o = _oracle(b, T, T)
        np.testing.assert_array_equal(c.disp.counts.cpu().numpy(), o["counts"])
        np.testing.assert_array_equal(c.disp.offsets.cpu().numpy(), o["offsets"])
        assert np.array_equal(y[:T], o["y"])
        assert (y[T:] == 0).all()
        if i % 10 == 5:
            ye, ce, _ = c.eager(b["x"], b["ids"], b["scores"], T, T)
            assert np.array_equal(ye, y[:T])


def test_graph_buckets_with_different_capacities_share_one_context():
    """Two graphs captured on one context at capacities 2048 and 8192 ("Unify
    expert parallel token dispatcher API", section "API design": different
    graph buckets may use different current capacities over the same
    storage), each holding forward and backward; replays alternate with fresh
    routing and every replay matches the oracle."""
    N, D, E, K = 8192, 1024, 64, 8
    disp = MoeDispatcher(N, D, E, K, dtype=torch.bfloat16, device=DEV, backward=True)
    w = workloads.Workload("buckets", T=N, ntpr=N, nmax=N, D=D, E=E, K=K, dtype="bf16",
                           routing="zipf", zipf_s=1.1, seed=0)
    graphs = {}
    for n in (2048, 8192):
        st = {"x": torch.zeros((n, D), dtype=torch.bfloat16, device=DEV),
              "ids": torch.full((n, K), -1, dtype=torch.int32, device=DEV),
              "s": torch.zeros((n, K), dtype=torch.float32, device=DEV),
              "gy": torch.zeros((n, D), dtype=torch.bfloat16, device=DEV)}

        def body(st=st, n=n):
            lay = disp.layout(st["ids"], n)
            disp.dispatch(st["x"], st["s"], st["ids"], lay.counts, num_tokens_per_rank=n)
            y = disp.combine(disp.x_e, lay.row_map, st["s"], num_tokens_per_rank=n)
            g_e, g_s = disp.combine_backward(st["gy"], disp.x_e, lay.row_map, st["s"],
                                             num_tokens_per_rank=n)
            g_x = disp.dispatch_backward(g_e, lay.row_map, n, num_tokens_per_rank=n)
            return y, g_s, g_x

        side = torch.cuda.Stream(device=DEV)
        side.wait_stream(torch.cuda.current_stream(DEV))
        with torch.cuda.stream(side):
            body()
        torch.cuda.current_stream(DEV).wait_stream(side)
        sync_or_fail()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            outs = body()
        sync_or_fail()
        graphs[n] = (g, st, outs)

    rng = np.random.default_rng(31)
    for i in range(10):
        n = (2048, 8192)[i % 2]
        g, st, (y, g_s, g_x) = graphs[n]
        T = int(rng.integers(1, n + 1))
        b = workloads.make_batch(w, T=T, seed=700 + i)
        gy = torch.from_numpy(rng.standard_normal((T, D)).astype(np.float32)).to(torch.bfloat16)
        gy_bits = gy.view(torch.int16).numpy().view(np.uint16)
        st["x"][:T].copy_(x_to_dev(b["x"]))
        st["x"][T:].zero_()
        st["ids"][:T].copy_(i32_dev(b["ids"]))
        st["ids"][T:].fill_(-1)
        st["s"][:T].copy_(f32_dev(b["scores"]))
        st["s"][T:].zero_()
        st["gy"][:T].copy_(x_to_dev(gy_bits))
        st["gy"][T:].zero_()
        note(f"bucket {n} replay {i} T={T}")
        g.replay()
        sync_or_fail()
        o = oracle.run_pipeline(b["x"], b["ids"], b["scores"], T, T, E, K, nthreads=ORACLE_THREADS)
        assert np.array_equal(x_to_np(y)[:T], o["y"])
        assert (x_to_np(y)[T:] == 0).all()
        ge_o, gs_o = oracle.combine_backward(gy_bits, o["x_e"], o["row_map"], b["scores"], T, K)
        gx_o = oracle.dispatch_backward(ge_o, o["row_map"], T, K)
        assert np.array_equal(x_to_np(g_x)[:T], gx_o)
        got = g_s.cpu().numpy()[:T].astype(np.float64)
        G = (gy_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        Y = (o["x_e"].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        rm = o["row_map"][:T]
        gamma = D * 2.0 ** -24 / (1 - D * 2.0 ** -24)
        for k in range(K):
            mag = np.sum(np.abs(G * Y[rm[:, k]]), axis=1)
            assert np.all(np.abs(got[:, k] - gs_o[:, k]) <= gamma * mag + 1e-30)
    del graphs, disp
    torch.cuda.empty_cache()
