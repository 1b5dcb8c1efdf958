"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Every check here is independent of the oracle's code: numpy brute force of the
quadratic (attention-like) form, closed forms through library matmuls, central
finite differences of the oracle's own forward, the gate-gradient suffix-sum
identity, the backward-as-reversed-forward identity and invariants (document
resets, split and resume, head sharing, scalar = vector gate).  None needs a GPU.

Sources: the recurrence and its gate forms are on the FLAT page ("FLAT: Flash
Linear Attention on TPUs", Linear Attention > Forward Recurrence and the table
of gated forms: RetNet's constant gate (L_f)_{mn} = f^{m-n}); the backward
statements (state gradient as linear attention run in reverse, grad of log f
as a suffix sum of q*dq - k*dk plus a boundary term) are in Linear Attention >
Backward Recurrence on the same page; document resets are on the JLA page
("JLA: JAX Linear Attention", segment_ids paragraph).
"""
import json
import os

import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_inputs(rng, B=2, T=11, H=2, Hqk=None, dk=3, dv=4, gate="scalar", h0=True,
                dhT=True, gscale=0.3):
    Hqk = H if Hqk is None else Hqk
    q = rng.standard_normal((B, T, Hqk, dk))
    k = rng.standard_normal((B, T, Hqk, dk))
    v = rng.standard_normal((B, T, H, dv))
    gs = (B, T, H, dk) if gate == "vector" else (B, T, H)
    g = -gscale * np.abs(rng.standard_normal(gs)) + 0.05 * rng.standard_normal(gs)
    dO = rng.standard_normal((B, T, H, dv))
    H0 = rng.standard_normal((B, H, dk, dv)) * 0.5 if h0 else None
    DHT = rng.standard_normal((B, H, dk, dv)) if dhT else None
    return q, k, v, g, dO, H0, DHT


def seg_from_lengths(B, lens):
    ids = np.concatenate([np.full(n, i) for i, n in enumerate(lens)]).astype(np.int32)
    return np.tile(ids, (B, 1))


def gate_vec(g, gate, dk):
    """Per-channel log gate [B,T,H,dk] from either gate form."""
    return g if gate == "vector" else np.repeat(g[..., None], dk, axis=-1)


def brute_force(q, k, v, g, h0, seg, gate):
    """Quadratic form: o_t = sum_{s<=t, same doc} ((q_t*e^{b_t-b_s}).k_s) v_s
    + [t in first doc] h0^T (q_t * e^{b_t}), with b the row's cumulative log gate."""
    B, T, Hqk, dk = q.shape
    H, dv = v.shape[2], v.shape[3]
    G = H // Hqk
    gv = gate_vec(g, gate, dk)
    o = np.zeros((B, T, H, dv))
    hT = np.zeros((B, H, dk, dv))
    for b in range(B):
        sid = seg[b] if seg is not None else np.zeros(T, dtype=np.int32)
        first = sid[0]
        for h in range(H):
            cum = np.cumsum(gv[b, :, h, :], axis=0)  # b_t, [T, dk]
            for t in range(T):
                acc = np.zeros(dv)
                for s in range(t + 1):
                    if sid[s] != sid[t]:
                        continue
                    # same document: no reset in (s, t]
                    if np.any(sid[s:t + 1] != sid[t]):
                        continue
                    w = np.dot(q[b, t, h // G] * np.exp(cum[t] - cum[s]), k[b, s, h // G])
                    acc += w * v[b, s, h]
                if h0 is not None and np.all(sid[:t + 1] == first):
                    acc += h0[b, h].T @ (q[b, t, h // G] * np.exp(cum[t]))
                o[b, t, h] = acc
            # final state: the last document's keys, plus h0 if one document
            last = sid[T - 1]
            start = T - 1
            while start > 0 and sid[start - 1] == last:
                start -= 1
            for s in range(start, T):
                hT[b, h] += np.outer(np.exp(cum[T - 1] - cum[s]) * k[b, s, h // G], v[b, s, h])
            if h0 is not None and start == 0:
                hT[b, h] += np.exp(cum[T - 1])[:, None] * h0[b, h]
    return o, hT


def loss(o, hT, dO, dhT):
    return float(np.sum(o * dO) + (np.sum(hT * dhT) if dhT is not None else 0.0))


def rel(a, b):
    d = np.max(np.abs(a - b)) if a.size else 0.0
    m = np.max(np.abs(b)) if b.size else 0.0
    return d / m if m > 0 else d


# ---------------------------------------------------------------- P0: worked example


def test_hand_worked_example():
    """Values worked out by hand from the recurrence (tests/golden/hand_example.json)."""
    with open(os.path.join(GOLDEN, "hand_example.json")) as f:
        ex = json.load(f)
    for case in ex["cases"]:
        a = {kk: np.array(vv, dtype=np.float64) for kk, vv in case["inputs"].items()
             if vv is not None}
        seg = np.array(case["segment_ids"], dtype=np.int32) if case.get("segment_ids") else None
        o, hT = oracle.fwd(a["q"], a["k"], a["v"], a["g"], h0=a.get("h0"), segment_ids=seg,
                           gate=case["gate"], threads=1)
        np.testing.assert_allclose(o, np.array(case["o"]), rtol=1e-14, atol=1e-14)
        np.testing.assert_allclose(hT, np.array(case["hT"]), rtol=1e-14, atol=1e-14)
        if "dq" in case:
            dq, dk, dv, dg, dh0 = oracle.bwd(a["q"], a["k"], a["v"], a["g"], a["dO"],
                                             h0=a.get("h0"), segment_ids=seg,
                                             dhT=a.get("dhT"), gate=case["gate"], threads=1)
            for name, got in (("dq", dq), ("dk", dk), ("dv", dv), ("dg", dg), ("dh0", dh0)):
                np.testing.assert_allclose(got, np.array(case[name]), rtol=1e-13, atol=1e-14,
                                           err_msg=name)


# ---------------------------------------------------------------- P1: brute force


@pytest.mark.parametrize("gate", ["scalar", "vector"])
@pytest.mark.parametrize("segs", [None, [3, 1, 5, 2], [1, 10]])
@pytest.mark.parametrize("Hqk", [2, 1])
def test_forward_matches_quadratic_form(gate, segs, Hqk):
    rng = np.random.default_rng(11)
    q, k, v, g, dO, h0, dhT = rand_inputs(rng, B=2, T=11, H=2, Hqk=Hqk, gate=gate)
    seg = seg_from_lengths(2, segs) if segs else None
    o, hT = oracle.fwd(q, k, v, g, h0=h0, segment_ids=seg, gate=gate, threads=2)
    o_ref, hT_ref = brute_force(q, k, v, g, h0, seg, gate)
    assert rel(o, o_ref) < 1e-12
    assert rel(hT, hT_ref) < 1e-12


def test_forward_unsorted_segment_ids():
    """A reset happens wherever the id changes, whether ids increase or not."""
    rng = np.random.default_rng(5)
    q, k, v, g, dO, h0, dhT = rand_inputs(rng, B=1, T=9, H=1)
    seg = np.array([[7, 7, 2, 2, 2, 7, 7, 0, 0]], dtype=np.int32)
    o, hT = oracle.fwd(q, k, v, g, h0=h0, segment_ids=seg, threads=1)
    o_ref, hT_ref = brute_force(q, k, v, g, h0, seg, "scalar")
    assert rel(o, o_ref) < 1e-12 and rel(hT, hT_ref) < 1e-12


# ---------------------------------------------------------------- P2: closed forms


def test_alpha_one_closed_form_and_gradients():
    """alpha = 1 is plain causal linear attention: o = tril(QK^T)V + Q h0, hT = K^T V + h0,
    and the gradients of L = <o,dO> + <hT,dhT> follow by matrix calculus."""
    rng = np.random.default_rng(3)
    T, dk, dv = 17, 5, 6
    Q, K, V = (rng.standard_normal((T, dk)), rng.standard_normal((T, dk)),
               rng.standard_normal((T, dv)))
    dO, h0, dhT = rng.standard_normal((T, dv)), rng.standard_normal((dk, dv)), \
        rng.standard_normal((dk, dv))
    P = np.tril(Q @ K.T)
    o_ref = P @ V + Q @ h0
    hT_ref = K.T @ V + h0
    dP = np.tril(dO @ V.T)
    dV_ref = P.T @ dO + K @ dhT
    dQ_ref = dP @ K + dO @ h0.T
    dK_ref = dP.T @ Q + V @ dhT.T
    dh0_ref = Q.T @ dO + dhT
    sh = lambda x: x[None, :, None, :]
    g = np.zeros((1, T, 1))
    o, hT = oracle.fwd(sh(Q), sh(K), sh(V), g, h0=h0[None, None], threads=1)
    assert rel(o[0, :, 0], o_ref) < 1e-13 and rel(hT[0, 0], hT_ref) < 1e-13
    dq, dk_, dv_, dg, dh0 = oracle.bwd(sh(Q), sh(K), sh(V), g, sh(dO), h0=h0[None, None],
                                       dhT=dhT[None, None], threads=1)
    assert rel(dq[0, :, 0], dQ_ref) < 1e-13
    assert rel(dk_[0, :, 0], dK_ref) < 1e-13
    assert rel(dv_[0, :, 0], dV_ref) < 1e-13
    assert rel(dh0[0, 0], dh0_ref) < 1e-13
    # gate gradient at alpha = 1: d/dg_t of L equals sum over entries of dS_t * S_{t-1}
    S = [h0]
    for t in range(T):
        S.append(S[-1] + np.outer(K[t], V[t]))
    dS = dhT.copy()
    dg_ref = np.zeros(T)
    for t in range(T - 1, -1, -1):
        dS = dS + np.outer(Q[t], dO[t])
        dg_ref[t] = np.sum(dS * S[t])
    assert rel(dg[0, :, 0], dg_ref) < 1e-12


def test_constant_gate_retnet_closed_form():
    """Constant scalar gate gamma (RetNet): o = ((QK^T) * L_gamma) V + diag(gamma^{t+1}) Q h0
    with (L_gamma)_{mn} = gamma^{m-n} for m >= n."""
    rng = np.random.default_rng(4)
    T, dk, dv, gamma = 23, 4, 3, 0.83
    Q, K, V = (rng.standard_normal((T, dk)), rng.standard_normal((T, dk)),
               rng.standard_normal((T, dv)))
    h0 = rng.standard_normal((dk, dv))
    m = np.arange(T)
    L = np.where(m[:, None] >= m[None, :], gamma ** (m[:, None] - m[None, :]).astype(float), 0.0)
    o_ref = ((Q @ K.T) * L) @ V + (gamma ** (m + 1.0))[:, None] * (Q @ h0)
    hT_ref = (K * (gamma ** (T - 1.0 - m))[:, None]).T @ V + gamma ** T * h0
    sh = lambda x: x[None, :, None, :]
    g = np.full((1, T, 1), np.log(gamma))
    o, hT = oracle.fwd(sh(Q), sh(K), sh(V), g, h0=h0[None, None], threads=1)
    assert rel(o[0, :, 0], o_ref) < 1e-12 and rel(hT[0, 0], hT_ref) < 1e-12


# ---------------------------------------------------------------- P3: finite differences


def _fd_grad(f, x, eps=1e-6):
    gr = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        old = x[i]
        x[i] = old + eps
        fp = f()
        x[i] = old - eps
        fm = f()
        x[i] = old
        gr[i] = (fp - fm) / (2 * eps)
    return gr


@pytest.mark.parametrize("gate,Hqk,segs", [("scalar", 2, None), ("vector", 2, None),
                                           ("scalar", 1, [4, 1, 3]), ("vector", 1, [2, 6]),
                                           ("vector", 2, [1, 1, 6])])
def test_backward_matches_finite_differences(gate, Hqk, segs):
    rng = np.random.default_rng(7)
    q, k, v, g, dO, h0, dhT = rand_inputs(rng, B=1, T=8, H=2, Hqk=Hqk, dk=3, dv=2, gate=gate)
    seg = seg_from_lengths(1, segs) if segs else None

    def L():
        o, hT = oracle.fwd(q, k, v, g, h0=h0, segment_ids=seg, gate=gate, threads=1)
        return loss(o, hT, dO, dhT)

    dq, dk_, dv_, dg, dh0 = oracle.bwd(q, k, v, g, dO, h0=h0, segment_ids=seg, dhT=dhT,
                                       gate=gate, threads=1)
    for name, x, got in (("q", q, dq), ("k", k, dk_), ("v", v, dv_), ("g", g, dg),
                         ("h0", h0, dh0)):
        num = _fd_grad(L, x)
        err = np.max(np.abs(num - got)) / max(np.max(np.abs(num)), 1e-30)
        assert err < 1e-6, (name, err)


# ---------------------------------------------------------------- P4: gate-gradient identity


@pytest.mark.parametrize("gate", ["scalar", "vector"])
@pytest.mark.parametrize("segs", [None, [5, 1, 7, 3]])
def test_gate_gradient_suffix_sum_identity(gate, segs):
    """dg_t = sum_{t'>=t, same doc} (q*dq - k*dk)_{t'} + [t in last doc] rowsum(dhT*hT),
    with per-head dq, dk (summed over channels for the scalar gate)."""
    rng = np.random.default_rng(9)
    B, T, H, Hqk, dk = 2, 16, 4, 2, 3
    q, k, v, g, dO, h0, dhT = rand_inputs(rng, B=B, T=T, H=H, Hqk=Hqk, dk=dk, dv=5, gate=gate)
    seg = seg_from_lengths(B, segs) if segs else None
    _, hT = oracle.fwd(q, k, v, g, h0=h0, segment_ids=seg, gate=gate, threads=2)
    _, _, _, dg, _ = oracle.bwd(q, k, v, g, dO, h0=h0, segment_ids=seg, dhT=dhT, gate=gate,
                                threads=2)
    dqh, dkh = oracle.bwd_per_head(q, k, v, g, dO, h0=h0, segment_ids=seg, dhT=dhT, gate=gate,
                                   threads=2)
    G = H // Hqk
    ref = np.zeros_like(dg)
    for b in range(B):
        sid = seg[b] if seg is not None else np.zeros(T, dtype=np.int32)
        for h in range(H):
            x = q[b, :, h // G] * dqh[b, :, h] - k[b, :, h // G] * dkh[b, :, h]  # [T, dk]
            bnd = np.sum(dhT[b, h] * hT[b, h], axis=1)  # [dk]
            if gate == "scalar":
                x, bnd = x.sum(-1), bnd.sum()
            run = bnd
            for t in range(T - 1, -1, -1):
                if t < T - 1 and sid[t + 1] != sid[t]:
                    run = 0.0 * run  # leaving the next document: no boundary term, restart
                run = run + x[t]
                is_reset = t > 0 and sid[t] != sid[t - 1]
                ref[b, t, h] = 0.0 if is_reset else run
    assert rel(dg, ref) < 1e-10
    # corollary: dg at the first token of a document that starts from zero is exactly 0
    if segs:
        starts = np.cumsum([0] + segs[:-1])[1:]
        assert np.all(dg[:, starts] == 0.0)


# ---------------------------------------------------------------- P5: backward = reversed forward


def test_backward_is_forward_in_reverse():
    """For a scalar gate, each input gradient is the oracle's own forward run on permuted
    arguments: reversed time with gates shifted by one for dv and dk, original time for dq."""
    rng = np.random.default_rng(13)
    B, T, H, dk, dv = 2, 19, 3, 4, 5
    q, k, v, g, dO, h0, dhT = rand_inputs(rng, B=B, T=T, H=H, dk=dk, dv=dv)
    dq, dk_, dv_, dg, dh0 = oracle.bwd(q, k, v, g, dO, h0=h0, dhT=dhT, threads=2)
    rev = lambda x: x[:, ::-1].copy()
    gs = np.concatenate([g[:, 1:], np.zeros((B, 1, H))], axis=1)  # g'_t = g_{t+1}, last 0
    gr = rev(gs)
    o_dv, h_dv = oracle.fwd(rev(k), rev(q), rev(dO), gr, h0=dhT, threads=2)
    assert rel(rev(o_dv), dv_) < 1e-12
    # the reversed run ends on the gradient of S_0; one more decay by alpha_0 gives dh0
    assert rel(np.exp(g[:, 0])[:, :, None, None] * h_dv, dh0) < 1e-12
    o_dk, _ = oracle.fwd(rev(v), rev(dO), rev(q), gr, h0=np.swapaxes(dhT, 2, 3).copy(),
                         threads=2)
    assert rel(rev(o_dk), dk_) < 1e-12
    o_dq, _ = oracle.fwd(dO, v, k, g, h0=np.swapaxes(h0, 2, 3).copy(), threads=2)
    assert rel(o_dq, dq) < 1e-12


# ---------------------------------------------------------------- P6: invariants


@pytest.mark.parametrize("gate", ["scalar", "vector"])
def test_packed_documents_equal_separate_runs(gate):
    rng = np.random.default_rng(21)
    lens = [4, 1, 9, 2, 6]
    T = sum(lens)
    q, k, v, g, dO, h0, dhT = rand_inputs(rng, B=1, T=T, H=2, gate=gate)
    seg = seg_from_lengths(1, lens)
    o, hT = oracle.fwd(q, k, v, g, h0=h0, segment_ids=seg, gate=gate, threads=1)
    grads = oracle.bwd(q, k, v, g, dO, h0=h0, segment_ids=seg, dhT=dhT, gate=gate, threads=1)
    s = 0
    for i, n in enumerate(lens):
        sl = slice(s, s + n)
        first, last = i == 0, i == len(lens) - 1
        hh = h0 if first else None
        dd = dhT if last else None
        oi, hTi = oracle.fwd(q[:, sl], k[:, sl], v[:, sl], g[:, sl], h0=hh, gate=gate, threads=1)
        gi = oracle.bwd(q[:, sl], k[:, sl], v[:, sl], g[:, sl], dO[:, sl], h0=hh, dhT=dd,
                        gate=gate, threads=1)
        assert rel(o[:, sl], oi) < 1e-12
        for i_g, (a, b_) in enumerate(zip(grads[:4], gi[:4])):
            ref = b_.copy()
            if i_g == 3 and not first:
                ref[:, 0] = 0.0  # a reset token's gate is unused
            assert rel(a[:, sl], ref) < 1e-12 or np.max(np.abs(a[:, sl] - ref)) < 1e-13
        if first:
            assert rel(grads[4], gi[4]) < 1e-12
        if last:
            assert rel(hT, hTi) < 1e-12
        s += n


def test_split_and_resume_equals_one_run():
    rng = np.random.default_rng(22)
    q, k, v, g, dO, h0, dhT = rand_inputs(rng, B=2, T=20, H=2, gate="vector")
    o, hT = oracle.fwd(q, k, v, g, h0=h0, gate="vector", threads=2)
    o1, h1 = oracle.fwd(q[:, :7], k[:, :7], v[:, :7], g[:, :7], h0=h0, gate="vector", threads=2)
    o2, h2 = oracle.fwd(q[:, 7:], k[:, 7:], v[:, 7:], g[:, 7:], h0=h1, gate="vector", threads=2)
    assert rel(np.concatenate([o1, o2], axis=1), o) < 1e-12 and rel(h2, hT) < 1e-12
    # backward: the second piece's dh0 is the first piece's dhT
    full = oracle.bwd(q, k, v, g, dO, h0=h0, dhT=dhT, gate="vector", threads=2)
    b2 = oracle.bwd(q[:, 7:], k[:, 7:], v[:, 7:], g[:, 7:], dO[:, 7:], h0=h1, dhT=dhT,
                    gate="vector", threads=2)
    b1 = oracle.bwd(q[:, :7], k[:, :7], v[:, :7], g[:, :7], dO[:, :7], h0=h0, dhT=b2[4],
                    gate="vector", threads=2)
    for i in range(4):
        assert rel(np.concatenate([b1[i], b2[i]], axis=1), full[i]) < 1e-12
    assert rel(b1[4], full[4]) < 1e-12


def test_head_sharing_equals_repeat_and_sum():
    rng = np.random.default_rng(23)
    G = 3
    q, k, v, g, dO, h0, dhT = rand_inputs(rng, B=2, T=9, H=6, Hqk=2, gate="vector")
    o, hT = oracle.fwd(q, k, v, g, h0=h0, gate="vector", threads=2)
    qr, kr = np.repeat(q, G, axis=2), np.repeat(k, G, axis=2)
    o2, hT2 = oracle.fwd(qr, kr, v, g, h0=h0, gate="vector", threads=2)
    assert rel(o, o2) < 1e-13 and rel(hT, hT2) < 1e-13
    a = oracle.bwd(q, k, v, g, dO, h0=h0, dhT=dhT, gate="vector", threads=2)
    b = oracle.bwd(qr, kr, v, g, dO, h0=h0, dhT=dhT, gate="vector", threads=2)
    B, T = q.shape[:2]
    assert rel(a[0], b[0].reshape(B, T, 2, G, -1).sum(3)) < 1e-12
    assert rel(a[1], b[1].reshape(B, T, 2, G, -1).sum(3)) < 1e-12
    for i in (2, 3, 4):
        assert rel(a[i], b[i]) < 1e-12


def test_scalar_gate_equals_vector_gate_with_equal_channels():
    rng = np.random.default_rng(24)
    dk = 4
    q, k, v, g, dO, h0, dhT = rand_inputs(rng, B=1, T=13, H=2, dk=dk, gate="scalar")
    seg = seg_from_lengths(1, [6, 7])
    gv = np.repeat(g[..., None], dk, axis=-1)
    o1, h1 = oracle.fwd(q, k, v, g, h0=h0, segment_ids=seg, gate="scalar", threads=1)
    o2, h2 = oracle.fwd(q, k, v, gv, h0=h0, segment_ids=seg, gate="vector", threads=1)
    assert rel(o1, o2) < 1e-13 and rel(h1, h2) < 1e-13
    a = oracle.bwd(q, k, v, g, dO, h0=h0, segment_ids=seg, dhT=dhT, gate="scalar", threads=1)
    b = oracle.bwd(q, k, v, gv, dO, h0=h0, segment_ids=seg, dhT=dhT, gate="vector", threads=1)
    for i in (0, 1, 2, 4):
        assert rel(a[i], b[i]) < 1e-13
    assert rel(a[3], b[3].sum(-1)) < 1e-12


def test_thread_count_does_not_change_results():
    rng = np.random.default_rng(25)
    q, k, v, g, dO, h0, dhT = rand_inputs(rng, B=1, T=70, H=2, dk=8, dv=64, gate="vector")
    a = oracle.bwd(q, k, v, g, dO, h0=h0, dhT=dhT, gate="vector", threads=1)
    b = oracle.bwd(q, k, v, g, dO, h0=h0, dhT=dhT, gate="vector", threads=8)
    for x, y in zip(a, b):
        assert np.array_equal(x, y) or rel(x, y) < 1e-14


def test_empty_sequence():
    rng = np.random.default_rng(26)
    q, k, v, g, dO, h0, dhT = rand_inputs(rng, B=1, T=0, H=2)
    o, hT = oracle.fwd(q, k, v, g, h0=h0, threads=1)
    assert o.shape == (1, 0, 2, 4)
    assert np.array_equal(hT, h0)
    dq, dk_, dv_, dg, dh0 = oracle.bwd(q, k, v, g, dO, h0=h0, dhT=dhT, threads=1)
    assert np.array_equal(dh0, dhT)
