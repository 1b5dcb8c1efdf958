"""GPU parity: the HIP library against the fp64 oracle, element by element.

Tolerance (per tensor): max|gpu - oracle| / max|oracle| <= 1e-4 for fp32
inputs and <= 2e-2 for bf16 inputs (fp32 accumulation), for o, hT and every
gradient.  The oracle reads exactly the values the GPU reads (bf16 inputs are
rounded once, when drawn).  Outputs and workspace are poisoned with NaN before
each call, so any element a kernel fails to write shows up.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from ssm_recurrence_amd import binding as gb
from ssm_recurrence_amd.inputs import small_case, workload

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


@pytest.fixture(autouse=True)
def nan_poison(monkeypatch):
    """torch.empty / empty_like return NaN-filled (or 0xFF-filled) memory."""
    real_empty, real_like = torch.empty, torch.empty_like

    def poison(t):
        if t.is_floating_point():
            t.fill_(float("nan"))
        elif t.dtype == torch.uint8:
            t.fill_(255)
        return t

    monkeypatch.setattr(torch, "empty", lambda *a, **k: poison(real_empty(*a, **k)))
    monkeypatch.setattr(torch, "empty_like", lambda *a, **k: poison(real_like(*a, **k)))
    yield


def rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if a.size == 0:
        return 0.0
    assert np.all(np.isfinite(a)), "non-finite values in GPU output"
    m = np.max(np.abs(b))
    d = np.max(np.abs(a - b))
    return d / m if m > 0 else d


def to_np(t):
    return None if t is None else t.detach().float().cpu().numpy().astype(np.float64)


def run_gpu(case, dev="cuda", split=0):
    c = case.to(dev)
    o, hT = gb.fwd(c.q, c.k, c.v, c.g, c.h0, c.segment_ids, gate=c.gate, split=split)
    dq, dk, dv, dg, dh0 = gb.bwd(c.q, c.k, c.v, c.g, c.dO, c.h0, c.segment_ids, c.dhT, gate=c.gate,
                                 split=split)
    torch.cuda.synchronize()
    return dict(o=o, hT=hT, dq=dq, dk=dk, dv=dv, dg=dg, dh0=dh0)


def run_oracle(case):
    o, hT = oracle.fwd(case.q, case.k, case.v, case.g, case.h0, case.segment_ids, gate=case.gate)
    dq, dk, dv, dg, dh0 = oracle.bwd(case.q, case.k, case.v, case.g, case.dO, case.h0,
                                     case.segment_ids, case.dhT, gate=case.gate)
    return dict(o=o, hT=hT, dq=dq, dk=dk, dv=dv, dg=dg, dh0=dh0)


def check(case, got=None, ref=None):
    got = got or run_gpu(case)
    ref = ref or run_oracle(case)
    tol = TOL[case.dtype]
    errs = {n: rel(to_np(got[n]), ref[n]) for n in ref}
    print(case.name, case.gate, case.dtype, tuple(case.q.shape), tuple(case.v.shape),
          {n: "%.2e" % e for n, e in errs.items()}, flush=True)
    bad = {n: e for n, e in errs.items() if not e <= tol}
    assert not bad, "parity failed: %s (tol %g)" % (bad, tol)
    return got, ref


SMALL = [
    # (T, d_k, d_v, gate, dtype, H, H_qk, lengths, h0/dhT)
    (1, 64, 64, "scalar", torch.float32, 2, 2, None, True),
    (63, 64, 64, "scalar", torch.float32, 2, 2, None, True),
    (64, 64, 64, "vector", torch.float32, 2, 2, None, True),
    (100, 128, 128, "scalar", torch.float32, 2, 1, None, True),
    (100, 128, 128, "vector", torch.float32, 2, 2, None, True),
    (130, 64, 128, "vector", torch.float32, 4, 2, None, False),
    (200, 128, 64, "scalar", torch.float32, 4, 1, [64, 1, 50, 3, 82], True),
    (1, 128, 128, "vector", torch.bfloat16, 2, 2, None, True),
    (63, 128, 128, "scalar", torch.bfloat16, 2, 2, None, True),
    (100, 128, 128, "vector", torch.bfloat16, 4, 4, None, True),
    (256, 128, 128, "vector", torch.bfloat16, 2, 2, [100, 28, 128], True),
    (256, 128, 128, "scalar", torch.bfloat16, 4, 2, [64, 64, 1, 1, 1, 60, 65], True),
    (190, 64, 64, "vector", torch.bfloat16, 2, 1, [5, 7, 1, 100, 77], False),
    (300, 64, 128, "scalar", torch.bfloat16, 8, 2, None, True),
    # one- and two-token rows with segment ids (a reset on the second token)
    (1, 128, 128, "scalar", torch.bfloat16, 2, 2, [1], True),
    (2, 128, 128, "scalar", torch.float32, 2, 2, [1, 1], True),
    (2, 128, 128, "vector", torch.bfloat16, 2, 2, [1, 1], True),
]


@pytest.mark.parametrize("T,dk,dv,gate,dtype,H,Hqk,lens,hs", SMALL,
                         ids=["T%d-%d-%d-%s-%s-H%d-%d-%s-%s" % (c[0], c[1], c[2], c[3],
                              str(c[4])[6:], c[5], c[6], "seg" if c[7] else "noseg",
                              "h0" if c[8] else "noh0") for c in SMALL])
def test_small_parity(T, dk, dv, gate, dtype, H, Hqk, lens, hs):
    case = small_case(seed=T * 7 + dk + H, B=2, T=T, H=H, H_qk=Hqk, d=dk, d_v=dv, gate=gate,
                      dtype=dtype, with_h0=hs, with_dhT=hs, lengths=lens)
    check(case)


def test_workload_c1():
    """Scalar-decay fp32, B=1 H=2 T=256 d=64, chunk 64 (the small oracle-sized workload)."""
    check(workload("c1"))


# Sequence split forced on small rows: pieces of whole chunks, documents that
# start inside a piece, on a piece boundary and cross several pieces, ragged tails.
SPLIT = [
    # (T, d_k, d_v, gate, dtype, H, H_qk, lengths, h0/dhT, split)
    (640, 64, 64, "scalar", torch.float32, 2, 2, [200, 300, 140], True, 3),
    (700, 128, 128, "vector", torch.float32, 2, 2, None, True, 4),
    (1000, 128, 128, "vector", torch.bfloat16, 2, 2, [300, 700], True, 5),
    (513, 128, 128, "scalar", torch.bfloat16, 4, 2, None, True, 2),
    (640, 128, 128, "scalar", torch.bfloat16, 2, 2, [256, 384], False, 100),
    (448, 64, 128, "vector", torch.bfloat16, 4, 1, [10, 50, 4, 300, 84], True, 7),
    (300, 128, 128, "scalar", torch.float32, 4, 2, [100, 50, 150], True, 2),
    (200, 128, 128, "scalar", torch.float32, 2, 2, None, False, 1),
    # enough pieces for the state passes' wide blocks (64 key channels x all columns)
    (4096, 128, 128, "vector", torch.bfloat16, 4, 4, [1000, 3096], True, 32),
    (4096, 128, 128, "scalar", torch.float32, 4, 2, [2500, 1596], True, 32),
    # bf16 scalar gate, more walking pieces (288) than workgroups (256): some
    # workgroups walk two pieces in turn; heads share q/k
    (1100, 128, 128, "scalar", torch.bfloat16, 16, 8, [500, 600], True, 12),
    # longer rows in a few pieces: documents crossing pieces, a ragged tail, a
    # last piece shorter than the others (76 chunks: 4 x 16 + 12)
    (2048, 128, 128, "scalar", torch.bfloat16, 2, 2, [700, 1348], True, 2),
    (1950, 128, 128, "vector", torch.bfloat16, 2, 2, [37, 1000, 913], True, 2),
    (1024, 128, 128, "scalar", torch.bfloat16, 2, 1, [300, 724], False, 2),
    (4850, 128, 128, "scalar", torch.bfloat16, 2, 2, [2000, 2850], True, 5),
    (1536, 64, 128, "vector", torch.bfloat16, 4, 2, None, True, 3),
    # fp32 state passes with a whole head per workgroup (256 workgroups) over
    # pieces of three chunks, the last one ragged
    (3062, 128, 128, "scalar", torch.float32, 8, 2, [1000, 2062], True, 16),
    # the most pieces whose summaries the forward kernel and the backward's state
    # passes chain themselves (8: 24 chunks in pieces of 3), and one more piece,
    # where the combine runs instead (27 chunks)
    (1500, 128, 128, "vector", torch.bfloat16, 2, 2, [400, 1100], True, 8),
    (1700, 128, 128, "vector", torch.bfloat16, 2, 2, [400, 1300], True, 9),
    (1500, 128, 128, "scalar", torch.float32, 2, 2, [700, 800], True, 8),
]


@pytest.mark.parametrize("T,dk,dv,gate,dtype,H,Hqk,lens,hs,split", SPLIT,
                         ids=["T%d-%d-%d-%s-%s-H%d-%d-%s-%s-P%d" % (c[0], c[1], c[2], c[3],
                              str(c[4])[6:], c[5], c[6], "seg" if c[7] else "noseg",
                              "h0" if c[8] else "noh0", c[9]) for c in SPLIT])
def test_split_parity(T, dk, dv, gate, dtype, H, Hqk, lens, hs, split):
    case = small_case(seed=T + split, B=2, T=T, H=H, H_qk=Hqk, d=dk, d_v=dv, gate=gate,
                      dtype=dtype, with_h0=hs, with_dhT=hs, lengths=lens)
    check(case, got=run_gpu(case, split=split))


def subcase(case, b, qh):
    """Batch row b and q/k head qh (with the heads that read it) of a case."""
    G = case.H // case.H_qk
    hs = slice(qh * G, (qh + 1) * G)
    pick = lambda x, h: None if x is None else x[b:b + 1, :, h].contiguous()
    st = lambda x: None if x is None else x[b:b + 1, hs].contiguous()
    return dataclasses.replace(
        case, q=pick(case.q, slice(qh, qh + 1)), k=pick(case.k, slice(qh, qh + 1)),
        v=pick(case.v, hs), g=pick(case.g, hs), dO=pick(case.dO, hs), h0=st(case.h0),
        dhT=st(case.dhT),
        segment_ids=None if case.segment_ids is None else case.segment_ids[b:b + 1].contiguous())


def sub_outputs(got, case, b, qh):
    G = case.H // case.H_qk
    hs = slice(qh * G, (qh + 1) * G)
    qs = slice(qh, qh + 1)
    out = {}
    for n, t in got.items():
        if t is None:
            out[n] = None
        elif n in ("hT", "dh0"):
            out[n] = t[b:b + 1, hs]
        elif n in ("dq", "dk"):
            out[n] = t[b:b + 1, :, qs]
        else:
            out[n] = t[b:b + 1, :, hs]
    return out


# Full workload sizes in the launch configuration the benchmark times (the
# library's own split choice); outputs compared on sampled (batch row, q/k head
# group) pairs, each checked whole against the oracle run on that slice alone.
FULL = {"c2": [(0, 0), (3, 1)], "c3": [(0, 0), (3, 15)], "c4": [(0, 0), (0, 9), (0, 15)],
        "c5a": [(0, 0), (0, 15)], "c5b": [(0, 3), (7, 15)]}


@pytest.mark.parametrize("name", list(FULL))
def test_full_size_sampled(name):
    case = workload(name)
    print("full-size", name, tuple(case.q.shape), tuple(case.v.shape), flush=True)
    got = run_gpu(case)
    for b, qh in FULL[name]:
        sub = subcase(case, b, qh)
        check(sub, got=sub_outputs(got, case, b, qh))


def test_packed_documents_match_separate_runs():
    """The packed-document workload (B=1, T=65536, H=16, scalar gate, bf16): for
    sampled heads, every document of the GPU's packed run matches a separate
    oracle run of that document alone, from h0 for the first document and from
    zero for the others; hT is the last document's final state and dh0 the first
    document's initial-state gradient."""
    case = workload("c4")
    lens = case.doc_lengths
    assert lens is not None and len(lens) > 1
    got = run_gpu(case)
    tol = TOL[case.dtype]
    for qh in (0, 11 % case.H_qk):
        sub = subcase(case, 0, qh)
        g_sub = {n: to_np(t) for n, t in sub_outputs(got, case, 0, qh).items()}
        t0 = 0
        for i, n in enumerate(lens):
            ts = slice(t0, t0 + n)
            cut = lambda x: x[:, ts].contiguous()
            h0 = sub.h0 if i == 0 else None
            o, hT = oracle.fwd(cut(sub.q), cut(sub.k), cut(sub.v), cut(sub.g), h0, None,
                               gate=sub.gate)
            dq, dk, dv, dg, dh0 = oracle.bwd(cut(sub.q), cut(sub.k), cut(sub.v), cut(sub.g),
                                             cut(sub.dO), h0, None, None, gate=sub.gate)
            ref = dict(o=o, dq=dq, dk=dk, dv=dv, dg=dg)
            errs = {k: rel(g_sub[k][:, ts], v) for k, v in ref.items()}
            if i == len(lens) - 1:
                errs["hT"] = rel(g_sub["hT"], hT)
            if i == 0:
                errs["dh0"] = rel(g_sub["dh0"], dh0)
            bad = {k: e for k, e in errs.items() if not e <= tol}
            assert not bad, "head %d document %d [%d, %d): %s" % (qh, i, t0, t0 + n, bad)
            t0 += n
        print("head", qh, len(lens), "documents match", flush=True)


@pytest.mark.parametrize("gate,dtype,states", [("vector", torch.bfloat16, True),
                                                ("scalar", torch.float32, True),
                                                ("vector", torch.float32, False),
                                                ("scalar", torch.bfloat16, False)])
def test_empty_sequence(gate, dtype, states):
    """T = 0: the state passes straight through, hT = h0 and dh0 = dhT (zeros when
    absent), every output written (the outputs start as NaN)."""
    B, H, d, dev = 2, 4, 128, "cuda"
    mk = lambda *shape, dt=dtype: torch.empty(shape, dtype=dt, device=dev)
    q, k, v, dO = mk(B, 0, H, d), mk(B, 0, H, d), mk(B, 0, H, d), mk(B, 0, H, d)
    g = mk(B, 0, H, d) if gate == "vector" else mk(B, 0, H)
    gen = torch.Generator().manual_seed(7)
    h0 = torch.randn((B, H, d, d), generator=gen).to(dev) if states else None
    dhT = torch.randn((B, H, d, d), generator=gen).to(dev) if states else None
    o, hT = gb.fwd(q, k, v, g, h0, None, gate=gate)
    dq, dk, dv, dg, dh0 = gb.bwd(q, k, v, g, dO, h0, None, dhT, gate=gate)
    torch.cuda.synchronize()
    zeros = torch.zeros((B, H, d, d), device=dev)
    assert tuple(o.shape) == (B, 0, H, d) and tuple(dg.shape) == tuple(g.shape)
    assert torch.equal(hT, h0 if states else zeros)
    assert torch.equal(dh0, dhT if states else zeros)


def test_deterministic():
    case = small_case(seed=3, B=1, T=200, H=4, H_qk=2, d=128, gate="vector", dtype=torch.bfloat16,
                      lengths=[70, 130])
    a = run_gpu(case)
    b = run_gpu(case)
    for n in a:
        assert torch.equal(a[n], b[n]), n


def test_strong_decay_stays_finite():
    """Gates 10x stronger than the GLA workload's: no inf or NaN, parity holds."""
    case = small_case(seed=11, B=1, T=192, H=2, d=128, gate="vector", dtype=torch.bfloat16,
                      gate_kind="gla", gate_mult=10.0)
    check(case)


# Log gates far beyond the range of the chunk-local factored form (every |g| above
# 1.875 in some chunk): -3 and -8 per token on every channel, channels alternating
# between -8 and -0.01, elements drawn from {-8, -0.01}, and rows whose first half
# is at -3 while the second half has the GLA workload's gates (strong and ordinary
# chunks in one walk).  Both dtypes, both d_k kernels families (128: the
# whole-head kernels; 64: the sliced ones), documents inside chunks, forced splits.
STRONG = [
    # (gate_kind, mult, dtype, d, T, lengths, split)
    ("unit", 3.0, torch.bfloat16, 128, 256, [100, 28, 128], 0),
    ("unit", 8.0, torch.bfloat16, 128, 256, [100, 28, 128], 0),
    ("mix_channels", 8.0, torch.bfloat16, 128, 256, [100, 28, 128], 0),
    ("mix_random", 8.0, torch.bfloat16, 128, 256, [7, 121, 128], 0),
    ("half_unit", 3.0, torch.bfloat16, 128, 512, [300, 212], 2),
    ("unit", 3.0, torch.float32, 128, 256, [100, 28, 128], 0),
    ("unit", 8.0, torch.float32, 128, 256, [100, 28, 128], 0),
    ("mix_channels", 8.0, torch.float32, 128, 256, [100, 28, 128], 0),
    ("mix_random", 8.0, torch.float32, 128, 200, None, 2),
    ("unit", 8.0, torch.bfloat16, 64, 256, [100, 28, 128], 0),
    ("mix_random", 8.0, torch.bfloat16, 64, 190, [5, 7, 1, 100, 77], 0),
    ("mix_channels", 8.0, torch.float32, 64, 256, [100, 28, 128], 3),
]


@pytest.mark.parametrize("kind,mult,dtype,d,T,lens,split", STRONG,
                         ids=["%s-x%g-%s-d%d-T%d-%s-P%d" % (c[0], c[1], str(c[2])[6:], c[3], c[4],
                              "seg" if c[5] else "noseg", c[6]) for c in STRONG])
def test_strong_gate_parity(kind, mult, dtype, d, T, lens, split):
    case = small_case(seed=T + d + int(mult), B=2, T=T, H=2, d=d, gate="vector", dtype=dtype,
                      gate_kind=kind, gate_mult=mult, lengths=lens)
    check(case, got=run_gpu(case, split=split))
