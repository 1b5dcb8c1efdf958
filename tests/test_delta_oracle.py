"""Pins for the fp64 gated delta rule oracle (oracle/delta.py), on the CPU.

Each pin checks the oracle against something other than itself:
  - the delta rule's defining property: with beta = 1 and unit keys, the new
    state maps k_t to v_t exactly, whatever the gate and the earlier state, so
    reading with q_t = k_t returns v_t;
  - beta = 0: nothing is written or erased, the state is h0 decayed by the
    product of the gates;
  - keys that are distinct basis vectors (h0 = 0): nothing is ever erased, and
    the rule is the scalar-gated linear attention with keys beta_t k_t, checked
    against the gated linear attention oracle (pinned on its own);
  - document resets: a packed row equals its documents run one by one;
  - the backward: torch autograd through a torch transcription of the update
    (an independent derivative), and central finite differences.
A planted mistake in a copy of the oracle (the erase taken before the decay,
beta missing from the erase, dbeta of the wrong sign, dk without its X term,
dg without the gate factor) fails at least one pin.
"""
import numpy as np
import pytest
import torch

import oracle
import oracle.delta as od


def rand_case(seed, B=2, T=40, H=2, d=8, dv=6, h0=True, unit_keys=False):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, H, d)) / np.sqrt(d)
    k = rng.standard_normal((B, T, H, d))
    k = k / np.linalg.norm(k, axis=-1, keepdims=True) if unit_keys else k / np.sqrt(d)
    v = rng.standard_normal((B, T, H, dv))
    g = -rng.uniform(0.01, 0.5, (B, T, H))
    beta = rng.uniform(0.1, 0.9, (B, T, H))
    hh = rng.standard_normal((B, H, d, dv)) * 0.5 if h0 else None
    dO = rng.standard_normal((B, T, H, dv))
    dhT = rng.standard_normal((B, H, d, dv))
    return q, k, v, g, beta, hh, dO, dhT


def close(a, b, tol=1e-10):
    a, b = np.asarray(a), np.asarray(b)
    return np.max(np.abs(a - b)) <= tol * max(1.0, np.max(np.abs(b)))


def pin_exact_write(fwd, seed=1):
    q, k, v, g, beta, h0, _, _ = rand_case(seed, unit_keys=True)
    o, _ = fwd(k, k, v, g, np.ones_like(beta), h0)
    return close(o, v, 1e-9)


def pin_no_write(fwd, seed=2):
    q, k, v, g, beta, h0, _, _ = rand_case(seed)
    o, hT = fwd(q, k, v, g, np.zeros_like(beta), h0)
    gam = np.exp(np.cumsum(g, axis=1))                              # [B, T, H]
    ref = gam[..., None] * np.einsum("bthk,bhkv->bthv", q, h0)
    return close(o, ref) and close(hT, gam[:, -1][..., None, None] * h0)


def pin_orthogonal_keys_is_gla(fwd, seed=3):
    """Distinct basis keys and h0 = 0: no erase ever happens (k_t^T S_{t-1} = 0),
    so the rule is the gated linear attention with keys beta_t k_t."""
    B, T, H, d, dv = 2, 24, 2, 32, 5
    rng = np.random.default_rng(seed)
    idx = np.stack([rng.permutation(d)[:T] for _ in range(B * H)]).reshape(B, H, T).transpose(0, 2, 1)
    k = np.zeros((B, T, H, d))
    np.put_along_axis(k, idx[..., None], 1.0, axis=-1)
    q = rng.standard_normal((B, T, H, d))
    v = rng.standard_normal((B, T, H, dv))
    g = -rng.uniform(0.01, 0.5, (B, T, H))
    beta = rng.uniform(0.1, 0.9, (B, T, H))
    o, hT = fwd(q, k, v, g, beta)
    o2, hT2 = oracle.fwd(q, k * beta[..., None], v, g, gate="scalar")
    return close(o, o2) and close(hT, hT2)


def pin_resets(fwd, seed=4):
    q, k, v, g, beta, h0, _, _ = rand_case(seed, B=1, T=30)
    lens = [7, 1, 12, 10]
    seg = np.repeat(np.arange(len(lens)), lens)[None].astype(np.int32)
    o, hT = fwd(q, k, v, g, beta, h0, torch.tensor(seg))
    parts, t0, S = [], 0, None
    for i, n in enumerate(lens):
        sl = slice(t0, t0 + n)
        oi, S = fwd(q[:, sl], k[:, sl], v[:, sl], g[:, sl], beta[:, sl], h0 if i == 0 else None)
        parts.append(oi)
        t0 += n
    return close(o, np.concatenate(parts, axis=1)) and close(hT, S)


def torch_grads(q, k, v, g, beta, h0, dO, dhT, seg=None):
    ts = [torch.tensor(x, requires_grad=True) for x in (q, k, v, g, beta, h0)]
    tq, tk, tv, tg, tb, th = ts
    B, T, H, d = q.shape
    S = th
    outs = []
    for t in range(T):
        a = torch.exp(tg[:, t])
        if seg is not None and t > 0:
            a = torch.where(torch.tensor(seg[:, t] != seg[:, t - 1])[:, None], torch.zeros_like(a), a)
        kt, vt, bt = tk[:, t], tv[:, t], tb[:, t]
        # S <- alpha (I - beta k k^T) S + beta k v^T, one term at a time
        P = torch.eye(d, dtype=torch.float64) - bt[..., None, None] * kt[..., :, None] * kt[..., None, :]
        S = a[..., None, None] * (P @ S) + bt[..., None, None] * kt[..., :, None] * vt[..., None, :]
        outs.append(torch.einsum("bhk,bhkv->bhv", tq[:, t], S))
    o = torch.stack(outs, dim=1)
    ((o * torch.tensor(dO)).sum() + (S * torch.tensor(dhT)).sum()).backward()
    return [t.grad.numpy() for t in ts]


def pin_autograd(bwd, seed=5, seg=None):
    q, k, v, g, beta, h0, dO, dhT = rand_case(seed, T=70)  # two checkpoint stretches
    want = torch_grads(q, k, v, g, beta, h0, dO, dhT, seg)
    got = bwd(q, k, v, g, beta, dO, h0, None if seg is None else torch.tensor(seg), dhT)
    # want: dq, dk, dv, dg, dbeta, dh0 in the same order
    return all(close(a, b, 1e-9) for a, b in zip(got, want))


def pin_finite_differences(fwd, bwd, seed=6, h=1e-6):
    q, k, v, g, beta, h0, dO, dhT = rand_case(seed, B=1, T=6, H=1, d=3, dv=2)
    seg = torch.tensor([[0, 0, 0, 1, 1, 1]], dtype=torch.int32)

    def L(*a):
        o, hT = fwd(*a, seg)
        return float(np.sum(o * dO) + np.sum(hT * dhT))
    args = [q, k, v, g, beta, h0]
    got = bwd(q, k, v, g, beta, dO, h0, seg, dhT)
    order = [0, 1, 2, 3, 4, 5]  # bwd returns dq, dk, dv, dg, dbeta, dh0
    for i, gi in zip(order, got):
        for idx in np.ndindex(args[i].shape):
            p = [a.copy() for a in args]
            m = [a.copy() for a in args]
            p[i][idx] += h
            m[i][idx] -= h
            num = (L(*p) - L(*m)) / (2 * h)
            if abs(num - gi[idx]) > 1e-6 * max(1.0, abs(num)):
                return False
    return True


def all_pins(fwd, bwd):
    seg = np.repeat(np.arange(4), [20, 1, 30, 19])[None].repeat(2, 0).astype(np.int32)
    return {
        "exact write": pin_exact_write(fwd),
        "no write": pin_no_write(fwd),
        "orthogonal keys = gated linear attention": pin_orthogonal_keys_is_gla(fwd),
        "resets": pin_resets(fwd),
        "autograd": pin_autograd(bwd),
        "autograd with resets": pin_autograd(bwd, seed=7, seg=seg),
        "finite differences": pin_finite_differences(fwd, bwd),
    }


def test_oracle_passes_every_pin():
    res = all_pins(od.delta_fwd, od.delta_bwd)
    assert all(res.values()), res


def test_backward_checkpoint_interval_does_not_matter(monkeypatch):
    q, k, v, g, beta, h0, dO, dhT = rand_case(8, T=50)
    a = od.delta_bwd(q, k, v, g, beta, dO, h0, None, dhT)
    monkeypatch.setattr(od, "CH", 7)
    b = od.delta_bwd(q, k, v, g, beta, dO, h0, None, dhT)
    assert all(close(x, y, 1e-12) for x, y in zip(a, b))


# ---- planted mistakes
def _mut_fwd(erase_first=False, no_beta_erase=False):
    def fwd(q, k, v, g, beta, h0=None, segment_ids=None):
        q, k, v, g, beta, S, reset = od._inputs(q, k, v, g, beta, h0, segment_ids)
        o = np.zeros(q.shape[:3] + (v.shape[3],))
        for t in range(q.shape[1]):
            a, b, kt = od._alpha(g, reset, t), beta[:, t], k[:, t]
            be = np.ones_like(b) if no_beta_erase else b
            if erase_first:   # alpha applied to the write term as well
                kS = np.einsum("bhk,bhkv->bhv", kt, S)
                S = a[..., None, None] * (S + kt[..., :, None] * (b[..., None] * v[:, t] - be[..., None] * kS)[..., None, :])
            else:
                X = a[..., None, None] * S
                kX = np.einsum("bhk,bhkv->bhv", kt, X)
                S = X + kt[..., :, None] * (b[..., None] * v[:, t] - be[..., None] * kX)[..., None, :]
            o[:, t] = np.einsum("bhk,bhkv->bhv", q[:, t], S)
        return o, S
    return fwd


def _dk_without_x_term(q, k, v, g, beta, dO, h0, segment_ids, dhT):
    """dk as the oracle's backward forms it, but without -beta X dS^T k."""
    q, k, v, g, beta, S, reset = od._inputs(q, k, v, g, beta, h0, segment_ids)
    dO = od._f64(dO)
    T = q.shape[1]
    prev = []
    for t in range(T):
        prev.append(S)
        _, S = od._step(S, k[:, t], v[:, t], od._alpha(g, reset, t), beta[:, t])
    dk = np.zeros_like(k)
    dS = np.zeros_like(S) if dhT is None else od._f64(dhT).copy()
    for t in range(T - 1, -1, -1):
        a_t, b_t, k_t, v_t = od._alpha(g, reset, t), beta[:, t], k[:, t], v[:, t]
        X, _ = od._step(prev[t], k_t, v_t, a_t, b_t)
        dS = dS + q[:, t][..., :, None] * dO[:, t][..., None, :]
        r = v_t - np.einsum("bhk,bhkv->bhv", k_t, X)
        dSk = np.einsum("bhkv,bhk->bhv", dS, k_t)
        dk[:, t] = b_t[..., None] * np.einsum("bhkv,bhv->bhk", dS, r)
        dX = dS - b_t[..., None, None] * k_t[..., :, None] * dSk[..., None, :]
        dS = a_t[..., None, None] * dX
    return dk


def _mut_bwd(which):
    def bwd(q, k, v, g, beta, dO, h0=None, segment_ids=None, dhT=None):
        dq, dk, dv, dg, dbeta, dh0 = od.delta_bwd(q, k, v, g, beta, dO, h0, segment_ids, dhT)
        if which == "dbeta sign":
            dbeta = -dbeta
        if which == "dk no X term":
            dk = _dk_without_x_term(q, k, v, g, beta, dO, h0, segment_ids, dhT)
        if which == "dg no gate factor":
            dg = dg / np.exp(np.asarray(g))
        return dq, dk, dv, dg, dbeta, dh0
    return bwd


@pytest.mark.parametrize("fwd,bwd,name", [
    (_mut_fwd(erase_first=True), od.delta_bwd, "erase before the decay, write decayed"),
    (_mut_fwd(no_beta_erase=True), od.delta_bwd, "beta missing from the erase"),
    (od.delta_fwd, _mut_bwd("dbeta sign"), "dbeta of the wrong sign"),
    (od.delta_fwd, _mut_bwd("dk no X term"), "dk without its X term"),
    (od.delta_fwd, _mut_bwd("dg no gate factor"), "dg without the gate factor"),
])
def test_pins_catch_planted_mistakes(fwd, bwd, name):
    res = all_pins(fwd, bwd)
    assert not all(res.values()), "%s passed every pin" % name
