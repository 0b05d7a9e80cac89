"""The autograd layer routes gradients through the library's backward
kernels: loss = <y, G> with y = combine(expert(dispatch(x))) gives dL/dx,
dL/dscores and dL/dy_e that match the oracle's backward definitions."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from combine_moe_layout_05_amd import MoeDispatcher, MoeTokenDispatcher

from gpu_util import (DEV, ORACLE_THREADS, f32_dev, i32_dev, note, sync_or_fail, x_to_dev,
                      x_to_np)

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("name,T", [("padded", 2047), ("padded", 13), ("dsv3", 4096)])
def test_autograd_matches_oracle_backward(name, T):
    w = workloads.WORKLOADS[name]
    b = workloads.make_batch(w)
    rng = np.random.default_rng(3)
    G = torch.from_numpy(rng.standard_normal((T, w.D)).astype(np.float32)).to(torch.bfloat16)
    layer = MoeTokenDispatcher(MoeDispatcher(w.nmax, w.D, w.E, w.K, dtype=torch.bfloat16,
                                             device=DEV, backward=True))
    x = x_to_dev(b["x"][:T]).requires_grad_(True)
    s = f32_dev(b["scores"][:T]).requires_grad_(True)
    ids = i32_dev(b["ids"][:T])
    note(f"autograd {name} T={T}")
    x_e = layer.dispatch(x, s, ids, num_tokens_per_rank=w.ntpr)
    y_e = x_e * 2                                  # expert: exact doubling in bf16
    y_e.retain_grad()
    y = layer.combine(y_e, s)
    # Poison the library's dL/dy_e buffer: the rows past the true total must
    # come back +0.0 from the library itself.
    layer.disp.g_e.view(torch.int16).fill_(0x7F7F)
    (y.float() * G.to(DEV).float()).sum().backward()
    sync_or_fail()

    lay = oracle.layout(b["ids"][:T], T, w.ntpr, w.E, w.K)
    xe_o, _ = oracle.dispatch(b["x"][:T], b["scores"][:T], w.K, lay["src"], ORACLE_THREADS)
    ye_o = (torch.from_numpy(xe_o.view(np.int16)).view(torch.bfloat16) * 2)
    ye_o = ye_o.view(torch.int16).numpy().view(np.uint16)
    y_o = oracle.combine(ye_o, lay["row_map"], b["scores"][:T], T, w.K, ORACLE_THREADS)
    assert np.array_equal(_bits(y), y_o)
    g_bits = G.view(torch.int16).numpy().view(np.uint16)
    ge_o, gs_o = oracle.combine_backward(g_bits, ye_o, lay["row_map"], b["scores"][:T], T, w.K,
                                         ORACLE_THREADS)
    total = lay["total"]
    # dL/dy_e: the scaled copies on live rows, zero past the true total
    gye = _bits(y_e.grad)
    assert np.array_equal(gye[:total], ge_o)
    assert (gye[total:] == 0).all()
    # dL/dx: the expert doubles its input, so dL/dx_e = 2 dL/dy_e
    gxe = (torch.from_numpy(ge_o.view(np.int16)).view(torch.bfloat16) * 2)
    gxe = gxe.view(torch.int16).numpy().view(np.uint16)
    gx_o = oracle.dispatch_backward(gxe, lay["row_map"], T, w.K, ORACLE_THREADS)
    assert np.array_equal(_bits(x.grad), gx_o)
    # dL/dscores within the fp32 dot-product bound
    D = w.D
    gamma = D * 2.0 ** -24 / (1 - D * 2.0 ** -24)
    Gf = (g_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    Yf = (ye_o.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    rm = lay["row_map"][:T]
    got = s.grad.cpu().numpy().astype(np.float64)
    for k in range(w.K):
        mag = np.sum(np.abs(Gf * Yf[rm[:, k]]), axis=1)
        assert np.all(np.abs(got[:, k] - gs_o[:, k]) <= gamma * mag + 1e-30)
    del layer
    torch.cuda.empty_cache()


def test_two_layers_keep_their_own_state():
    w = workloads.WORKLOADS["padded"]
    b = workloads.make_batch(w)
    T = 1000
    mk = lambda: MoeTokenDispatcher(MoeDispatcher(w.nmax, w.D, w.E, w.K, dtype=torch.bfloat16,
                                                  device=DEV, backward=True))
    l1, l2 = mk(), mk()
    x = x_to_dev(b["x"][:T]).requires_grad_(True)
    s1 = f32_dev(b["scores"][:T]).requires_grad_(True)
    ids1 = i32_dev(b["ids"][:T])
    ids2 = i32_dev(np.roll(b["ids"][:T], 1, axis=0))
    s2 = f32_dev(np.roll(b["scores"][:T], 1, axis=0)).requires_grad_(True)
    note("autograd two layers")
    h = l1.combine(l1.dispatch(x, s1, ids1) * 1, s1)
    y = l2.combine(l2.dispatch(h, s2, ids2) * 1, s2)
    y.float().sum().backward()
    sync_or_fail()
    assert torch.isfinite(x.grad.float()).all() and torch.isfinite(s1.grad).all()
    # the same through a plain fp32 torch reference of dispatch/combine
    def ref(xf, sf, idx):
        return (xf[:, None, :] * sf[:, :, None]).sum(dim=1)   # identity experts
    xr = x.detach().float().requires_grad_(True)
    s1r = s1.detach().clone().requires_grad_(True)
    s2r = s2.detach().clone().requires_grad_(True)
    yr = ref(ref(xr, s1r, None), s2r, None)
    yr.sum().backward()
    assert torch.allclose(x.grad.float(), xr.grad, rtol=3e-2, atol=3e-2)
    assert torch.allclose(s2.grad, s2r.grad, rtol=3e-2, atol=5e-1)


def _oracle_grads(b, w, T, G):
    """dL/dx and dL/dy_e of loss = <combine(2 * dispatch(x)), G> by the oracle."""
    lay = oracle.layout(b["ids"][:T], T, w.ntpr, w.E, w.K)
    xe_o, _ = oracle.dispatch(b["x"][:T], b["scores"][:T], w.K, lay["src"], ORACLE_THREADS)
    ye_o = (torch.from_numpy(xe_o.view(np.int16)).view(torch.bfloat16) * 2)
    ye_o = ye_o.view(torch.int16).numpy().view(np.uint16)
    g_bits = G.view(torch.int16).numpy().view(np.uint16)
    ge_o, _ = oracle.combine_backward(g_bits, ye_o, lay["row_map"], b["scores"][:T], T, w.K,
                                      ORACLE_THREADS)
    gxe = (torch.from_numpy(ge_o.view(np.int16)).view(torch.bfloat16) * 2)
    gxe = gxe.view(torch.int16).numpy().view(np.uint16)
    gx_o = oracle.dispatch_backward(gxe, lay["row_map"], T, w.K, ORACLE_THREADS)
    return gx_o, ge_o, lay["total"]


class _SavingExpert(torch.autograd.Function):
    """y = 2 x that saves its input, as a weight-gradient expert would."""
    @staticmethod
    def forward(ctx, x):
        ctx.save_for_backward(x)
        return x * 2

    @staticmethod
    def backward(ctx, g):
        ctx.saved_tensors                         # what a weight gradient would read
        return g * 2


def test_second_forward_before_backward_is_detected():
    """Two forwards on one layer before the first backward: the first
    micro-batch's expert input (a view of x_e) was rewritten, so the
    backward raises instead of using the newer rows."""
    w = workloads.WORKLOADS["padded"]
    b = workloads.make_batch(w)
    layer = MoeTokenDispatcher(MoeDispatcher(w.nmax, w.D, w.E, w.K, dtype=torch.bfloat16,
                                             device=DEV, backward=True))
    T = 600
    note("autograd two forwards in flight, shared x_e")
    xa = x_to_dev(b["x"][:T]).requires_grad_(True)
    sa = f32_dev(b["scores"][:T]).requires_grad_(True)
    ya = layer.combine(_SavingExpert.apply(layer.dispatch(xa, sa, i32_dev(b["ids"][:T]),
                                                          num_tokens_per_rank=w.ntpr)), sa)
    xb = x_to_dev(b["x"][T:2 * T]).requires_grad_(True)
    sb = f32_dev(b["scores"][T:2 * T]).requires_grad_(True)
    yb = layer.combine(_SavingExpert.apply(layer.dispatch(xb, sb, i32_dev(b["ids"][T:2 * T]),
                                                          num_tokens_per_rank=w.ntpr)), sb)
    with pytest.raises(RuntimeError, match="clone_x_e"):
        ya.float().sum().backward()
    yb.float().sum().backward()                   # the latest forward is still intact
    sync_or_fail()
    assert torch.isfinite(xb.grad.float()).all()
    del layer
    torch.cuda.empty_cache()


def test_clone_x_e_keeps_forwards_in_flight_independent():
    """With clone_x_e=True, forward(A), forward(B), backward(A), backward(B)
    give each micro-batch the oracle's gradients bit for bit."""
    w = workloads.WORKLOADS["padded"]
    b = workloads.make_batch(w)
    layer = MoeTokenDispatcher(MoeDispatcher(w.nmax, w.D, w.E, w.K, dtype=torch.bfloat16,
                                             device=DEV, backward=True), clone_x_e=True)
    rng = np.random.default_rng(4)
    T = 600
    runs = []
    for lo in (0, T):
        bb = {k: b[k][lo:lo + T] for k in ("x", "ids", "scores")}
        G = torch.from_numpy(rng.standard_normal((T, w.D)).astype(np.float32)).to(torch.bfloat16)
        x = x_to_dev(bb["x"]).requires_grad_(True)
        s = f32_dev(bb["scores"]).requires_grad_(True)
        note(f"autograd clone_x_e forward rows {lo}..{lo + T}")
        x_e = layer.dispatch(x, s, i32_dev(bb["ids"]), num_tokens_per_rank=w.ntpr)
        y_e = _SavingExpert.apply(x_e)
        y_e.retain_grad()
        y = layer.combine(y_e, s)
        runs.append((bb, G, x, y_e, y))
    for bb, G, x, y_e, y in runs:
        note("autograd clone_x_e backward")
        (y.float() * G.to(DEV).float()).sum().backward()
        sync_or_fail()
        gx_o, ge_o, total = _oracle_grads(bb, w, T, G)
        assert np.array_equal(_bits(x.grad), gx_o)
        gye = _bits(y_e.grad)
        assert np.array_equal(gye[:total], ge_o)
        assert (gye[total:] == 0).all()
    del layer
    torch.cuda.empty_cache()
