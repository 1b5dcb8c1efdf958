"""fp64 CPU oracle for the gated delta rule (test infrastructure).

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module; the HIP library never does, and nothing
here comes from it.

The pages name the variant (FLAT page, "FLAT: Flash Linear Attention on TPUs",
Conclusion, future work 1: DeltaNet, Gated DeltaNet and Kimi Delta Attention,
whose state update is not a plain sum of outer products; probjax page, "GPU
kernels", section Gated DeltaNet: a token-by-token recurrence as the reference
and a chunked WY/UT form whose backward keeps only chunk-boundary states) but
do not write the update out.  The reading taken here is the published Gated
DeltaNet update, in this library's state orientation (S is d_k x d_v and
o = S^T q, as for the gated linear attention):

    S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,   o_t = S_t^T q_t,

with alpha_t = exp(g_t) a scalar gate per (b, t, h) and beta_t a scalar write
strength per (b, t, h).  Document resets follow the gated linear attention
(JLA page, "JLA: JAX Linear Attention", segment_ids): where segment_ids changes
the carried state is dropped (alpha_t unused), h0 seeds the row's first
document and hT is the state after the last token.

This module is that recurrence token by token, vectorised over (b, h).  The
backward is reverse-mode differentiation of the same steps, written out: with
X = alpha_t S_{t-1} (zero after a reset) and dS the gradient of S_t,

    dq_t = S_t do_t            (after dS += q_t do_t^T)
    dv_t = beta_t dS^T k_t
    dbeta_t = k_t^T dS (v_t - X^T k_t)
    dk_t = beta_t dS (v_t - X^T k_t) - beta_t X dS^T k_t
    dX = (I - beta_t k_t k_t^T) dS,   dg_t = <dX, X>,   dS_{t-1} = alpha_t dX

(dg_t and the carry are zero at reset tokens); dh0 is the carry past t = 0.
States are kept at every CH-th token and recomputed in between.
"""
from __future__ import annotations

import numpy as np

CH = 64  # checkpoint interval of the backward (any value gives the same result)


def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):  # a torch tensor: take its exact values
        import torch
        x = x.detach().to("cpu").to(torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _inputs(q, k, v, g, beta, h0, segment_ids):
    q, k, v, g, beta, h0 = map(_f64, (q, k, v, g, beta, h0))
    B, T, H, dk = q.shape
    dv = v.shape[3]
    if k.shape != q.shape or v.shape[:3] != (B, T, H) or g.shape != (B, T, H) or beta.shape != (B, T, H):
        raise ValueError("bad shapes")
    if h0 is None:
        h0 = np.zeros((B, H, dk, dv))
    reset = np.zeros((B, T), dtype=bool)
    if segment_ids is not None:
        seg = np.asarray(segment_ids.cpu() if hasattr(segment_ids, "cpu") else segment_ids)
        reset[:, 1:] = seg[:, 1:] != seg[:, :-1]
    return q, k, v, g, beta, h0, reset


def _step(S, k_t, v_t, a_t, b_t):
    """One update on [B, H, dk, dv] states; returns (X, S_t)."""
    X = a_t[..., None, None] * S
    kX = np.einsum("bhk,bhkv->bhv", k_t, X)
    S_t = X + b_t[..., None, None] * k_t[..., :, None] * (v_t - kX)[..., None, :]
    return X, S_t


def _alpha(g, reset, t):
    return np.where(reset[:, t][:, None], 0.0, np.exp(g[:, t]))


def delta_fwd(q, k, v, g, beta, h0=None, segment_ids=None):
    """(o [B,T,H,dv], hT [B,H,dk,dv]) as float64."""
    q, k, v, g, beta, S, reset = _inputs(q, k, v, g, beta, h0, segment_ids)
    B, T, H, _ = q.shape
    o = np.zeros((B, T, H, v.shape[3]))
    for t in range(T):
        _, S = _step(S, k[:, t], v[:, t], _alpha(g, reset, t), beta[:, t])
        o[:, t] = np.einsum("bhk,bhkv->bhv", q[:, t], S)
    return o, S


def delta_bwd(q, k, v, g, beta, dO, h0=None, segment_ids=None, dhT=None):
    """(dq, dk, dv, dg, dbeta, dh0) as float64, given dO = dL/do and dhT = dL/dhT."""
    q, k, v, g, beta, S, reset = _inputs(q, k, v, g, beta, h0, segment_ids)
    dO = _f64(dO)
    B, T, H, dk = q.shape
    dv_ = v.shape[3]
    # states entering every CH-th token
    ckpt = {}
    for t in range(T):
        if t % CH == 0:
            ckpt[t] = S.copy()
        _, S = _step(S, k[:, t], v[:, t], _alpha(g, reset, t), beta[:, t])
    dq, dk_, dv, dg, dbeta = (np.zeros_like(q), np.zeros_like(k), np.zeros_like(v),
                              np.zeros((B, T, H)), np.zeros((B, T, H)))
    dS = np.zeros((B, H, dk, dv_)) if dhT is None else _f64(dhT).copy()
    for c0 in range(((T - 1) // CH) * CH if T else 0, -1, -CH):
        c1 = min(c0 + CH, T)
        # recompute the states of this stretch: prev[t - c0] = S_{t-1}
        prev, S = [], ckpt[c0]
        for t in range(c0, c1):
            prev.append(S)
            _, S = _step(S, k[:, t], v[:, t], _alpha(g, reset, t), beta[:, t])
        for t in range(c1 - 1, c0 - 1, -1):
            a_t, b_t, k_t, v_t = _alpha(g, reset, t), beta[:, t], k[:, t], v[:, t]
            X, S_t = _step(prev[t - c0], k_t, v_t, a_t, b_t)
            dS = dS + q[:, t][..., :, None] * dO[:, t][..., None, :]
            dq[:, t] = np.einsum("bhkv,bhv->bhk", S_t, dO[:, t])
            r = v_t - np.einsum("bhk,bhkv->bhv", k_t, X)          # v - X^T k
            dSk = np.einsum("bhkv,bhk->bhv", dS, k_t)               # dS^T k
            dv[:, t] = b_t[..., None] * dSk
            dbeta[:, t] = np.einsum("bhv,bhv->bh", dSk, r)
            dk_[:, t] = b_t[..., None] * (np.einsum("bhkv,bhv->bhk", dS, r)
                                          - np.einsum("bhkv,bhv->bhk", X, dSk))
            dX = dS - b_t[..., None, None] * k_t[..., :, None] * dSk[..., None, :]
            dg[:, t] = np.where(reset[:, t][:, None], 0.0, np.einsum("bhkv,bhkv->bh", dX, X))
            dS = a_t[..., None, None] * dX
    return dq, dk_, dv, dg, dbeta, dS
