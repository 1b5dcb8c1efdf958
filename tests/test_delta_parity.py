"""GPU parity of the gated delta rule (gla_delta_fwd / gla_delta_bwd) against the
fp64 oracle (oracle/delta.py), element by element.

Tolerance per output tensor, as for the recurrence: max|a - b| / max|b| <= 1e-4
for fp32 inputs, 2e-2 for bf16 inputs (every product and sum in fp32).  The
oracle reads the same cast inputs.  Cases cover both head widths (and unequal
d_k, d_v), ragged chunk tails, one-token rows, documents starting on and inside
chunks (one of one token), rows without h0, and the benchmark layout (B=4,
T=4096, H=8, d=128, bf16), compared whole on a sampled (batch row, heads) slice.
"""
import numpy as np
import pytest
import torch

import oracle.delta as od
from ssm_recurrence_amd import binding as gb
from ssm_recurrence_amd.inputs import delta_case, delta_workload

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}
NAMES = ("dq", "dk", "dv", "dg", "dbeta", "dh0")


def rel(a, b):
    assert np.all(np.isfinite(a)), "non-finite values in GPU output"
    m = np.max(np.abs(b)) if b.size else 0.0
    return float(np.max(np.abs(a - b)) / m) if m > 0 else float(np.max(np.abs(a - b), initial=0.0))


def to_np(t):
    return t.detach().to("cpu", torch.float64).numpy()


def run_gpu(c):
    o, hT = gb.delta_fwd(c.q, c.k, c.v, c.g, c.beta, c.h0, c.segment_ids)
    grads = gb.delta_bwd(c.q, c.k, c.v, c.g, c.beta, c.dO, c.h0, c.segment_ids, c.dhT,
                         want_dh0=c.h0 is not None)
    torch.cuda.synchronize()
    out = dict(o=o, hT=hT)
    out.update(zip(NAMES, grads))
    return out


def run_oracle(c):
    o, hT = od.delta_fwd(c.q, c.k, c.v, c.g, c.beta, c.h0, c.segment_ids)
    ref = dict(o=o, hT=hT)
    ref.update(zip(NAMES, od.delta_bwd(c.q, c.k, c.v, c.g, c.beta, c.dO, c.h0, c.segment_ids, c.dhT)))
    if c.h0 is None:
        ref.pop("dh0")
    return ref


def compare(got, ref, dtype, label):
    errs = {n: rel(to_np(got[n]), r) for n, r in ref.items()}
    print(label, {n: "%.2e" % e for n, e in errs.items()}, flush=True)
    bad = {n: e for n, e in errs.items() if not e <= TOL[dtype]}
    assert not bad, "parity failed: %s (tol %g)" % (bad, TOL[dtype])


CASES = [
    # (B, T, H, d_k, d_v, dtype, lengths, h0)
    (2, 100, 2, 64, 64, torch.float32, None, True),
    (1, 1, 1, 64, 64, torch.float32, None, True),
    (2, 64, 2, 128, 128, torch.float32, None, True),
    (1, 200, 2, 128, 64, torch.float32, [50, 1, 100, 49], True),
    (2, 130, 2, 64, 128, torch.bfloat16, None, True),
    (1, 300, 4, 128, 128, torch.bfloat16, [64, 64, 1, 171], True),
    (2, 65, 3, 64, 64, torch.float32, [1, 64], False),
    (1, 513, 2, 128, 128, torch.float32, None, True),
]


@pytest.mark.parametrize("B,T,H,dk,dv,dtype,lens,h0", CASES,
                         ids=["B%d-T%d-H%d-%d-%d-%s-%s-%s" % (c[0], c[1], c[2], c[3], c[4], str(c[5])[6:],
                              "seg" if c[6] else "noseg", "h0" if c[7] else "noh0") for c in CASES])
def test_delta_parity(B, T, H, dk, dv, dtype, lens, h0):
    case = delta_case("small", B=B, T=T, H=H, d_k=dk, d_v=dv, dtype=dtype, seed=B * 100 + T + H + dk,
                      lengths=lens, with_h0=h0, with_dhT=h0)
    print("delta", B, T, H, dk, dv, dtype, lens, h0, flush=True)
    got = run_gpu(case.to("cuda"))
    compare(got, run_oracle(case), dtype, "delta small")


REUSE_CASES = [
    (1, 200, 2, 128, 64, torch.float32, [50, 1, 100, 49]),
    (1, 300, 4, 128, 128, torch.bfloat16, [64, 64, 1, 171]),
    (2, 130, 2, 64, 128, torch.bfloat16, None),
]


@pytest.mark.parametrize("B,T,H,dk,dv,dtype,lens", REUSE_CASES,
                         ids=["B%d-T%d-%s" % (c[0], c[1], str(c[5])[6:]) for c in REUSE_CASES])
def test_delta_bwd_reuses_forward_workspace(B, T, H, dk, dv, dtype, lens):
    """GLA_DELTA_WS_FROM_FWD on both calls: the backward handed the forward's
    workspace skips recomputing the per-chunk factors and the states entering the
    chunks (the forward stored them); its gradients equal, bit for bit, those of a
    backward that recomputes them (the same products in the same order), match the
    oracle, and a second backward on the same workspace gives them again."""
    case = delta_case("reuse", B=B, T=T, H=H, d_k=dk, d_v=dv, dtype=dtype, seed=7 + T, lengths=lens,
                      with_h0=True, with_dhT=True)
    c = case.to("cuda")
    print("delta reuse", B, T, H, dk, dv, dtype, lens, flush=True)
    ws = torch.empty(gb.delta_workspace_size(gb.delta_problem(c.q, c.v, gb.GLA_DELTA_WS_FROM_FWD)),
                     dtype=torch.uint8, device="cuda")
    o, hT = gb.delta_fwd(c.q, c.k, c.v, c.g, c.beta, c.h0, c.segment_ids, ws=ws, ws_from_fwd=True)
    args = (c.q, c.k, c.v, c.g, c.beta, c.dO, c.h0, c.segment_ids, c.dhT)
    reused = gb.delta_bwd(*args, ws=ws, ws_from_fwd=True)
    again = gb.delta_bwd(*args, ws=ws, ws_from_fwd=True)
    fresh = gb.delta_bwd(*args)
    torch.cuda.synchronize()
    for n, x, y, z in zip(NAMES, reused, again, fresh):
        assert torch.equal(x, z), n
        assert torch.equal(x, y), n
    got = dict(o=o, hT=hT)
    got.update(zip(NAMES, reused))
    compare(got, run_oracle(case), dtype, "delta reuse")


def test_delta_ws_stamp_guards_reuse():
    """GLA_DELTA_WS_FROM_FWD reuses ws only when its stamp (sizes, flags, input
    pointers, generation) is this call's: a workspace from other inputs, from the
    same buffers changed in place under a new generation, left by a backward that
    recomputed for other inputs, or written by a forward without the flag (which
    stores no states) is recomputed, so every gradient equals the recomputing
    backward's, bit for bit."""
    mk = lambda seed: delta_case("stamp", B=1, T=200, H=2, d_k=64, d_v=64, dtype=torch.bfloat16, seed=seed,
                                 lengths=[120, 80], with_h0=True, with_dhT=True).to("cuda")
    a, b = mk(11), mk(12)
    args = lambda c: (c.q, c.k, c.v, c.g, c.beta, c.dO, c.h0, c.segment_ids, c.dhT)
    fresh_a, fresh_b = gb.delta_bwd(*args(a)), gb.delta_bwd(*args(b))
    ws = torch.empty(gb.delta_workspace_size(gb.delta_problem(a.q, a.v, gb.GLA_DELTA_WS_FROM_FWD)),
                     dtype=torch.uint8, device="cuda")
    ws.fill_(255)
    gb.delta_fwd(a.q, a.k, a.v, a.g, a.beta, a.h0, a.segment_ids, ws=ws, ws_from_fwd=True, generation=1)
    # other inputs, same generation: their own factors
    got_b = gb.delta_bwd(*args(b), ws=ws, ws_from_fwd=True, generation=1)
    # the backward recomputed for b: ws now holds b's factors, stamped so; a again
    got_a = gb.delta_bwd(*args(a), ws=ws, ws_from_fwd=True, generation=1)
    # a's forward, then a's q changed in place under a new generation
    gb.delta_fwd(a.q, a.k, a.v, a.g, a.beta, a.h0, a.segment_ids, ws=ws, ws_from_fwd=True, generation=2)
    q_old = a.q.clone()
    a.q.copy_(b.q)
    got_a2 = gb.delta_bwd(*args(a), ws=ws, ws_from_fwd=True, generation=3)
    fresh_a2 = gb.delta_bwd(*args(a))
    a.q.copy_(q_old)
    # a forward without the flag stores factors only: a flagged backward on a fresh
    # workspace (no states in it) recomputes everything
    ws2 = torch.empty_like(ws).fill_(255)
    gb.delta_fwd(b.q, b.k, b.v, b.g, b.beta, b.h0, b.segment_ids, ws=ws2, generation=4)
    got_b2 = gb.delta_bwd(*args(b), ws=ws2, ws_from_fwd=True, generation=4)
    torch.cuda.synchronize()
    for n, x, y in zip(NAMES, got_b2, fresh_b):
        assert torch.equal(x, y), "forward without the flag: " + n
    for n, x, y in zip(NAMES, got_b, fresh_b):
        assert torch.equal(x, y), "other inputs: " + n
    for n, x, y in zip(NAMES, got_a, fresh_a):
        assert torch.equal(x, y), "after a recomputing backward: " + n
    for n, x, y in zip(NAMES, got_a2, fresh_a2):
        assert torch.equal(x, y), "inputs changed in place: " + n


def test_delta_autograd_matches_bwd():
    """DeltaFunction keeps the forward's workspace for its backward."""
    case = delta_case("autograd", B=1, T=150, H=2, d_k=64, d_v=64, dtype=torch.float32, seed=3,
                      lengths=[70, 80], with_h0=True, with_dhT=True)
    c = case.to("cuda")
    leaves = [x.clone().requires_grad_(True) for x in (c.q, c.k, c.v, c.g, c.beta, c.h0)]
    o, hT = gb.DeltaFunction.apply(*leaves, c.segment_ids)
    torch.autograd.backward([o, hT], [c.dO, c.dhT])
    ref = gb.delta_bwd(c.q, c.k, c.v, c.g, c.beta, c.dO, c.h0, c.segment_ids, c.dhT)
    for n, leaf, r in zip(NAMES, leaves, ref):
        assert torch.equal(leaf.grad, r), n


def test_delta_empty_rows():
    case = delta_case("empty", B=2, T=0, H=2, d_k=64, dtype=torch.float32, seed=1).to("cuda")
    got = run_gpu(case)
    assert got["o"].numel() == 0
    assert torch.equal(got["hT"], case.h0) and torch.equal(got["dh0"], case.dhT)


def test_delta_deterministic():
    case = delta_case("det", B=1, T=300, H=2, d_k=128, dtype=torch.bfloat16, seed=5).to("cuda")
    a, b = run_gpu(case), run_gpu(case)
    for n in a:
        assert torch.equal(a[n], b[n]), n


def test_delta_full_size_sampled():
    """The benchmark layout, in the launch configuration bench.py times; batch row 0,
    heads 0 and 5 compared whole against the oracle run on that slice."""
    case = delta_workload()
    print("full-size delta", tuple(case.q.shape), flush=True)
    c = case.to("cuda")
    got = run_gpu(c)
    # the benchmark's backward reuses the forward's factors: bit for bit the same
    ws = torch.empty(gb.delta_workspace_size(gb.delta_problem(c.q, c.v, gb.GLA_DELTA_WS_FROM_FWD)),
                     dtype=torch.uint8, device="cuda")
    gb.delta_fwd(c.q, c.k, c.v, c.g, c.beta, c.h0, c.segment_ids, ws=ws, ws_from_fwd=True, generation=1)
    reused = gb.delta_bwd(c.q, c.k, c.v, c.g, c.beta, c.dO, c.h0, c.segment_ids, c.dhT, ws=ws,
                          ws_from_fwd=True, generation=1)
    torch.cuda.synchronize()
    for n, x in zip(NAMES, reused):
        assert torch.equal(x, got[n]), "full-size reuse: " + n
    del c, ws, reused
    heads = [0, 5]
    sub = head_slice(case, heads)
    ref = run_oracle(sub)
    pick = {n: (got[n][0:1][:, heads] if n in ("hT", "dh0") else got[n][0:1][:, :, heads]) for n in ref}
    compare(pick, ref, case.dtype, "delta full size (b=0, h=0,5)")


def head_slice(case, heads):
    """Batch row 0 and the given heads of a case (the rule is per (b, h))."""
    import dataclasses
    s4 = lambda x: x[0:1][:, :, heads].contiguous()
    sh = lambda x: None if x is None else x[0:1][:, heads].contiguous()
    return dataclasses.replace(case, q=s4(case.q), k=s4(case.k), v=s4(case.v), g=s4(case.g),
                               beta=s4(case.beta), dO=s4(case.dO), h0=sh(case.h0), dhT=sh(case.dhT),
                               segment_ids=None if case.segment_ids is None else case.segment_ids[0:1])
