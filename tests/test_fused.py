"""q, k, v read in place from one projection tensor, and one fused gradient
(FLAT page, "FLAT: Flash Linear Attention on TPUs": the data-movement paragraph
of Gated Linear Attention, and Full Linear Attention Layer).

The kernels do the same arithmetic whatever the row strides of q, k, v, dq, dk,
dv, so every output with q, k, v as views of one [B, T, W] tensor must equal,
bit for bit, the output from packed copies of the same values; the packed path
is held to the oracle by test_parity.py, and one case here is also checked
against the oracle directly.  Padding columns after the three views are NaN in
the inputs (a read of them would poison the results) and hold a sentinel in the
gradient buffer (a write would change it).
"""
import numpy as np
import pytest
import torch

import oracle
from ssm_recurrence_amd import binding as gb
from ssm_recurrence_amd.inputs import small_case, workload

pytestmark = pytest.mark.gpu

SENTINEL = 12345.0


def strided_views(X, H_qk, d_k, H, d_v):
    """q, k, v as views of the first 2*H_qk*d_k + H*d_v columns of X [B, T, >= that]."""
    wq = H_qk * d_k
    return (X[..., :wq].unflatten(-1, (H_qk, d_k)), X[..., wq:2 * wq].unflatten(-1, (H_qk, d_k)),
            X[..., 2 * wq:2 * wq + H * d_v].unflatten(-1, (H, d_v)))


def fuse(case, pad, dev="cuda"):
    """The projection tensor [B, T, W + pad] holding q | k | v, padding NaN."""
    B, T = case.q.shape[:2]
    W = 2 * case.H_qk * case.d_k + case.H * case.d_v
    X = torch.full((B, T, W + pad), float("nan"), dtype=case.dtype, device=dev)
    for view, src in zip(strided_views(X, case.H_qk, case.d_k, case.H, case.d_v),
                         (case.q, case.k, case.v)):
        view.copy_(src)
    return X, W


def run_packed(c, split):
    o, hT = gb.fwd(c.q, c.k, c.v, c.g, c.h0, c.segment_ids, gate=c.gate, split=split)
    dq, dk, dv, dg, dh0 = gb.bwd(c.q, c.k, c.v, c.g, c.dO, c.h0, c.segment_ids, c.dhT,
                                 gate=c.gate, split=split)
    return dict(o=o, hT=hT, dq=dq, dk=dk, dv=dv, dg=dg, dh0=dh0)


def run_fused(c, X, W, split):
    """Inputs read from X; gradients written into one buffer dX shaped like X."""
    H_qk, d_k, H, d_v = c.H_qk, c.d_k, c.H, c.d_v
    q, k, v = strided_views(X, H_qk, d_k, H, d_v)
    o, hT = gb.fwd(q, k, v, c.g, c.h0, c.segment_ids, gate=c.gate, split=split)
    dX = torch.full(X.shape, SENTINEL, dtype=X.dtype, device=X.device)
    grads = strided_views(dX, H_qk, d_k, H, d_v)
    dq, dk, dv, dg, dh0 = gb.bwd(q, k, v, c.g, c.dO, c.h0, c.segment_ids, c.dhT, gate=c.gate,
                                 split=split, grads=grads)
    assert dq.data_ptr() == grads[0].data_ptr() and dv.data_ptr() == grads[2].data_ptr()
    return dict(o=o, hT=hT, dq=dq, dk=dk, dv=dv, dg=dg, dh0=dh0), dX


def assert_same(a, b, what):
    for n in a:
        if a[n] is None:
            assert b[n] is None, n
            continue
        assert torch.equal(a[n], b[n]), "%s: %s differs (max %g)" % (
            what, n, float((a[n].float() - b[n].float()).abs().max()))


CASES = [
    # (T, d_k, d_v, gate, dtype, H, H_qk, lengths, split, pad)
    (300, 128, 128, "scalar", torch.bfloat16, 4, 4, [100, 200], 0, 0),
    (300, 128, 128, "scalar", torch.bfloat16, 4, 2, None, 3, 64),
    (257, 128, 128, "vector", torch.bfloat16, 4, 4, [57, 200], 0, 0),
    (257, 128, 128, "vector", torch.bfloat16, 2, 2, None, 2, 8),
    (200, 128, 128, "scalar", torch.float32, 4, 2, [64, 136], 0, 4),
    (200, 128, 128, "scalar", torch.float32, 4, 4, None, 2, 0),
    (190, 64, 64, "vector", torch.bfloat16, 2, 1, [5, 185], 0, 8),
    (130, 64, 128, "vector", torch.float32, 4, 2, None, 0, 4),
    (100, 128, 64, "scalar", torch.float32, 2, 2, None, 0, 0),
]


@pytest.mark.parametrize("T,dk,dv,gate,dtype,H,Hqk,lens,split,pad", CASES,
                         ids=["T%d-%d-%d-%s-%s-H%d-%d-s%d-pad%d" % (c[0], c[1], c[2], c[3],
                              str(c[4])[6:], c[5], c[6], c[8], c[9]) for c in CASES])
def test_fused_equals_packed(T, dk, dv, gate, dtype, H, Hqk, lens, split, pad):
    case = small_case(seed=T + H + dk, B=2, T=T, H=H, H_qk=Hqk, d=dk, d_v=dv, gate=gate,
                      dtype=dtype, lengths=lens).to("cuda")
    print("fused", T, dk, dv, gate, dtype, H, Hqk, split, pad, flush=True)
    ref = run_packed(case, split)
    X, W = fuse(case, pad)
    got, dX = run_fused(case, X, W, split)
    torch.cuda.synchronize()
    assert_same(got, ref, "fused")
    if pad:
        assert torch.all(dX[..., W:] == SENTINEL), "a padding column of the gradient was written"


def test_fused_layout_helpers_and_oracle():
    """fused_views / bwd's own fused gradient / GLAFusedFunction, checked against
    the oracle (vector gate, bf16, heads sharing q/k)."""
    case = small_case(seed=9, B=2, T=150, H=4, H_qk=2, d=128, gate="vector", dtype=torch.bfloat16,
                      lengths=[70, 80])
    c = case.to("cuda")
    X, W = fuse(c, 0)
    q, k, v = gb.fused_views(X, c.H_qk, c.d_k, c.H, c.d_v)
    o, hT = gb.fwd(q, k, v, c.g, c.h0, c.segment_ids, gate=c.gate)
    dq, dk, dv, dg, dh0 = gb.bwd(q, k, v, c.g, c.dO, c.h0, c.segment_ids, c.dhT, gate=c.gate)
    dX = gb.fused_grad(dq)
    assert dX.shape == X.shape and dX.is_contiguous()
    wq = c.H_qk * c.d_k
    assert dk.data_ptr() == dX.data_ptr() + wq * 2 and dv.data_ptr() == dX.data_ptr() + 2 * wq * 2

    Xa = X.clone().requires_grad_(True)
    g = c.g.clone().requires_grad_(True)
    oa, hTa = gb.GLAFusedFunction.apply(Xa, g, c.h0, c.segment_ids, c.H_qk, c.d_k, c.gate)
    loss = (oa.float() * c.dO.float()).sum() + (hTa * c.dhT).sum()
    loss.backward()
    torch.cuda.synchronize()
    assert torch.equal(oa, o) and torch.equal(Xa.grad, dX) and torch.equal(g.grad, dg)

    ref_o, ref_hT = oracle.fwd(case.q, case.k, case.v, case.g, case.h0, case.segment_ids, gate=case.gate)
    rq, rk, rv, rg, rh0 = oracle.bwd(case.q, case.k, case.v, case.g, case.dO, case.h0,
                                     case.segment_ids, case.dhT, gate=case.gate)
    ref_dX = np.concatenate([rq.reshape(2, 150, -1), rk.reshape(2, 150, -1), rv.reshape(2, 150, -1)], -1)
    for name, a, b in (("o", o, ref_o), ("hT", hT, ref_hT), ("dX", dX, ref_dX), ("dg", dg, rg),
                       ("dh0", dh0, rh0)):
        a = a.detach().float().cpu().numpy().astype(np.float64)
        err = np.max(np.abs(a - b)) / np.max(np.abs(b))
        print(name, "%.2e" % err, flush=True)
        assert err <= 2e-2, (name, err)


def test_fused_full_size_c3():
    """GLA vector gate, bf16, B=4 T=4096 H=16 d=128, from one [4, 4096, 6144]
    projection, in the launch configuration bench.py times: equal to the packed run."""
    c = workload("c3").to("cuda")
    print("fused c3", flush=True)
    ref = run_packed(c, 0)
    X, W = fuse(c, 0)
    got, _ = run_fused(c, X, W, 0)
    torch.cuda.synchronize()
    assert_same(got, ref, "fused c3")
