"""GPU parity of the output norm and gate (gla_norm_gate_fwd / gla_norm_gate_bwd)
against the fp64 oracle (oracle/norm_gate.py), element by element.

Tolerance per output tensor, as for the recurrence: max|a - b| / max|b| <= 1e-4
for fp32 activations, 2e-2 for bf16 activations (sums in fp32).  The oracle
reads the same cast inputs.  Cases cover both head widths, row counts that leave
a wave's row groups partly empty, a single row, eps = 0 and a large eps, and the
layer shape of the FLAT page's benchmarks (B=8, T=4096, H=16, d=128), whose
per-row outputs are compared on sampled rows and whose dgamma is compared whole.
"""
import numpy as np
import pytest
import torch

import oracle.norm_gate as on
from ssm_recurrence_amd import binding as gb
from ssm_recurrence_amd.inputs import norm_gate_case, norm_gate_workload

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def rel(a, b):
    assert np.all(np.isfinite(a)), "non-finite values in GPU output"
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-30))


def to_np(t):
    return t.detach().to("cpu", torch.float64).numpy()


def run_gpu(case):
    c = case.to("cuda")
    y = gb.norm_gate_fwd(c.o, c.z, c.gamma, c.eps)
    d_o, dz, dgamma = gb.norm_gate_bwd(c.o, c.z, c.gamma, c.dy, c.eps)
    torch.cuda.synchronize()
    return dict(y=y, d_o=d_o, dz=dz, dgamma=dgamma)


def check(case, got=None):
    got = got or run_gpu(case)
    ref = dict(y=on.norm_gate_fwd(case.o, case.z, case.gamma, case.eps))
    ref["d_o"], ref["dz"], ref["dgamma"] = on.norm_gate_bwd(case.o, case.z, case.gamma, case.dy, case.eps)
    tol = TOL[case.dtype]
    errs = {n: rel(to_np(got[n]), r) if r.size else 0.0 for n, r in ref.items()}
    print(case.name, tuple(case.o.shape), case.dtype, case.eps, {n: "%.2e" % e for n, e in errs.items()},
          flush=True)
    bad = {n: e for n, e in errs.items() if not e <= tol}
    assert not bad, "parity failed: %s (tol %g)" % (bad, tol)


CASES = [
    # (B, T, H, d, dtype, eps)
    (2, 100, 4, 128, torch.float32, 1e-5),
    (1, 1, 1, 64, torch.float32, 1e-5),
    (2, 3, 2, 64, torch.bfloat16, 1e-5),
    (3, 257, 5, 128, torch.bfloat16, 1e-5),
    (1, 300, 16, 128, torch.float32, 0.0),
    (2, 513, 16, 128, torch.bfloat16, 1e-2),
    (2, 1000, 3, 64, torch.bfloat16, 1e-6),
    (4, 2048, 16, 64, torch.float32, 1e-5),
]


@pytest.mark.parametrize("B,T,H,d,dtype,eps", CASES,
                         ids=["B%d-T%d-H%d-d%d-%s-eps%g" % (c[0], c[1], c[2], c[3], str(c[4])[6:], c[5])
                              for c in CASES])
def test_norm_gate_parity(B, T, H, d, dtype, eps):
    check(norm_gate_case("small", B=B, T=T, H=H, d=d, dtype=dtype, seed=B * 100 + T + H + d, eps=eps))


def test_norm_gate_empty_rows():
    """T = 0: no rows; dgamma is zero."""
    case = norm_gate_case("empty", B=2, T=0, H=3, d=128, dtype=torch.float32, seed=1).to("cuda")
    y = gb.norm_gate_fwd(case.o, case.z, case.gamma, case.eps)
    d_o, dz, dgamma = gb.norm_gate_bwd(case.o, case.z, case.gamma, case.dy, case.eps)
    torch.cuda.synchronize()
    assert y.numel() == 0 and d_o.numel() == 0 and dz.numel() == 0
    assert torch.all(dgamma == 0)


def test_norm_gate_deterministic():
    case = norm_gate_case("det", B=2, T=700, H=16, d=128, dtype=torch.bfloat16, seed=5)
    a, b = run_gpu(case), run_gpu(case)
    for n in a:
        assert torch.equal(a[n], b[n]), n


def test_norm_gate_autograd():
    """NormGateFunction gives the library's own gradients under autograd."""
    case = norm_gate_case("ag", B=1, T=50, H=2, d=64, dtype=torch.float32, seed=7).to("cuda")
    o = case.o.clone().requires_grad_(True)
    z = case.z.clone().requires_grad_(True)
    g = case.gamma.clone().requires_grad_(True)
    y = gb.NormGateFunction.apply(o, z, g, case.eps)
    (y * case.dy).sum().backward()
    d_o, dz, dgamma = gb.norm_gate_bwd(case.o, case.z, case.gamma, case.dy, case.eps)
    torch.cuda.synchronize()
    assert torch.equal(o.grad, d_o) and torch.equal(z.grad, dz) and torch.equal(g.grad, dgamma)


def test_norm_gate_full_size_sampled():
    """The benchmark shape, in the launch configuration bench.py times: every
    output on every 61st time step of every row and head, dgamma whole (the
    oracle's sum taken one batch row at a time)."""
    case = norm_gate_workload()
    print("full-size norm gate", tuple(case.o.shape), flush=True)
    got = run_gpu(case)
    ts = slice(0, None, 61)
    sub = lambda t: t[:, ts]
    y = on.norm_gate_fwd(sub(case.o), sub(case.z), case.gamma, case.eps)
    d_o, dz, _ = on.norm_gate_bwd(sub(case.o), sub(case.z), case.gamma, sub(case.dy), case.eps)
    dgamma = sum(on.norm_gate_bwd(case.o[b], case.z[b], case.gamma, case.dy[b], case.eps)[2]
                 for b in range(case.o.shape[0]))
    errs = dict(y=rel(to_np(sub(got["y"])), y), d_o=rel(to_np(sub(got["d_o"])), d_o),
                dz=rel(to_np(sub(got["dz"])), dz), dgamma=rel(to_np(got["dgamma"]), dgamma))
    print({n: "%.2e" % e for n, e in errs.items()}, flush=True)
    assert all(e <= TOL[case.dtype] for e in errs.values()), errs
