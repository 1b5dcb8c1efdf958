"""GPU parity of the short depthwise causal convolution (gla_conv_fwd / gla_conv_bwd)
against the fp64 oracle (oracle/conv.py), element by element.

Tolerance per output tensor, as for the recurrence: max|a - b| / max|b| <= 1e-4 for
fp32 activations, 2e-2 for bf16 activations (sums in fp32).  The oracle reads the
same cast inputs.  Cases cover ragged rows (T not a multiple of the 64-step strips
or of the 256-step workgroups), channel counts that leave lanes idle, rows shorter
than the filter, no bias, and the page's full shape (B=8, T=4096, 2048 channels),
checked whole on sampled channel ranges (the convolution is per channel).
"""
import numpy as np
import pytest
import torch

import oracle.conv as oc
from ssm_recurrence_amd import binding as gb
from ssm_recurrence_amd.inputs import conv_case, conv_workload

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-30))


def to_np(t):
    return t.detach().to("cpu", torch.float64).numpy()


def run_gpu(case):
    c = case.to("cuda")
    y = gb.conv_fwd(c.x, c.w, c.bias)
    dx, dw, db = gb.conv_bwd(c.x, c.w, c.bias, c.dy)
    torch.cuda.synchronize()
    return dict(y=y, dx=dx, dw=dw, db=db)


def check(case, got=None, chans=None):
    got = got or run_gpu(case)
    sl = slice(None) if chans is None else chans
    x, dy = case.x[:, :, sl], case.dy[:, :, sl]
    w = case.w[:, sl]
    b = None if case.bias is None else case.bias[sl]
    ref = dict(y=oc.conv_fwd(x, w, b))
    ref["dx"], ref["dw"], ref["db"] = oc.conv_bwd(x, w, b, dy)
    tol = TOL[case.dtype]
    errs = {}
    for n, r in ref.items():
        g = got[n]
        g = g[:, sl] if n == "dw" else (g[sl] if n == "db" else g[:, :, sl])
        errs[n] = rel(to_np(g), r) if r.size else 0.0
    print(case.name, tuple(case.x.shape), case.dtype, {n: "%.2e" % e for n, e in errs.items()}, flush=True)
    bad = {n: e for n, e in errs.items() if not e <= tol}
    assert not bad, "parity failed: %s (tol %g)" % (bad, tol)


CASES = [
    # (B, T, C, dtype, bias)
    (2, 100, 64, torch.float32, True),
    (1, 1, 8, torch.float32, True),
    (2, 3, 16, torch.bfloat16, False),
    (3, 257, 520, torch.bfloat16, True),
    (1, 300, 1032, torch.float32, False),
    (2, 513, 2048, torch.bfloat16, True),
    (1, 64, 512, torch.float32, True),
    (2, 1000, 24, torch.bfloat16, True),
]


@pytest.mark.parametrize("B,T,C,dtype,bias", CASES,
                         ids=["B%d-T%d-C%d-%s-%s" % (c[0], c[1], c[2], str(c[3])[6:], "bias" if c[4] else "nobias")
                              for c in CASES])
def test_conv_parity(B, T, C, dtype, bias):
    check(conv_case("small", B=B, T=T, C=C, dtype=dtype, seed=B * 1000 + T + C, bias=bias))


def test_conv_empty_row():
    """T = 0: no output rows; dw and db are zero."""
    case = conv_case("empty", B=2, T=0, C=16, dtype=torch.float32, seed=1).to("cuda")
    y = gb.conv_fwd(case.x, case.w, case.bias)
    dx, dw, db = gb.conv_bwd(case.x, case.w, case.bias, case.dy)
    torch.cuda.synchronize()
    assert y.numel() == 0 and dx.numel() == 0
    assert torch.all(dw == 0) and torch.all(db == 0)


def test_conv_deterministic():
    case = conv_case("det", B=3, T=700, C=1024, dtype=torch.bfloat16, seed=5)
    a, b = run_gpu(case), run_gpu(case)
    for n in a:
        assert torch.equal(a[n], b[n]), n


def test_conv_full_size_sampled():
    """The page's benchmark shape, in the launch configuration bench.py times;
    whole outputs compared on two channel ranges."""
    case = conv_workload()
    print("full-size conv", tuple(case.x.shape), flush=True)
    got = run_gpu(case)
    for chans in (slice(0, 128), slice(1920, 2048)):
        check(case, got=got, chans=chans)
