"""fp64 CPU oracle for the short depthwise causal convolution (test infrastructure).

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module; the HIP library never does, and nothing
here comes from it.

What it computes (FLAT page, "FLAT: Flash Linear Attention on TPUs", section
Depthwise Causal Short Convolution, Forward and Backward): for each batch row,
time step t and channel c, with K taps W[k, c] and a bias b[c],

    z_t = b + sum_{k=0}^{K-1} W_k * x_{t-(K-1-k)}      (tap K-1 reads x_t;
                                                         x before t = 0 is zero)
    y_t = SiLU(z_t) = z_t * sigmoid(z_t)

and the backward given dy:

    dz_t = dy_t * SiLU'(z_t),  SiLU'(z) = s * (1 + z * (1 - s)),  s = sigmoid(z)
    dx_t = sum_k W_k * dz_{t+(K-1-k)}                   (dz past the end is zero)
    dW_k = sum over every (b, t) of x_{t-(K-1-k)} * dz_t
    db   = sum over every (b, t) of dz_t

written, as the page describes the kernel, as a sum of K shifted copies of x
(and of dz for the input gradient).  There are no document resets: the page's
convolution has none, and the plainest reading is that it runs over each row
as given.
"""
from __future__ import annotations

import numpy as np


def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):  # a torch tensor: take its exact values
        import torch
        x = x.detach().to("cpu").to(torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def conv_z(x, w, b=None):
    """Pre-activation z [B, T, C] from x [B, T, C], taps w [K, C], bias b [C] (or None)."""
    x, w, b = _f64(x), _f64(w), _f64(b)
    B, T, C = x.shape
    K = w.shape[0]
    if w.shape != (K, C) or (b is not None and b.shape != (C,)):
        raise ValueError("bad shapes")
    z = np.zeros((B, T, C))
    if b is not None:
        z += b
    for k in range(K):
        s = K - 1 - k  # tap k reads the input s steps back
        if s < T:
            z[:, s:, :] += w[k] * x[:, :T - s, :]
    return z


def conv_fwd(x, w, b=None):
    """y = SiLU(z), float64 [B, T, C]."""
    z = conv_z(x, w, b)
    return z * _sigmoid(z)


def conv_bwd(x, w, b, dy):
    """(dx [B, T, C], dw [K, C], db [C]) as float64, given dy = dL/dy."""
    x, w, dy = _f64(x), _f64(w), _f64(dy)
    B, T, C = x.shape
    K = w.shape[0]
    z = conv_z(x, w, b)
    s = _sigmoid(z)
    dz = dy * s * (1.0 + z * (1.0 - s))
    dx = np.zeros((B, T, C))
    dw = np.zeros((K, C))
    for k in range(K):
        sh = K - 1 - k
        if sh < T:
            dx[:, :T - sh, :] += w[k] * dz[:, sh:, :]
            dw[k] = np.sum(x[:, :T - sh, :] * dz[:, sh:, :], axis=(0, 1))
    db = dz.sum(axis=(0, 1))
    return dx, dw, db
