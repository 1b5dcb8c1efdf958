"""fp64 CPU oracle for the output norm and gate (test infrastructure).

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module; the HIP library never does, and nothing
here comes from it.

What it computes (FLAT page, "FLAT: Flash Linear Attention on TPUs", section
Full Linear Attention Layer: the layer output is a per-head RMSNorm of the
recurrence output multiplied by a swish output gate).  The page names the op and
nothing more; the plainest reading, taken here, is for each batch row b, step
t and head h, over the head's d channels j:

    r     = 1 / sqrt(mean_j o_j^2 + eps)
    n_j   = o_j * r                              (RMSNorm of the head's output)
    y_j   = gamma_j * n_j * swish(z_j),  swish(z) = z * sigmoid(z)

with one scale vector gamma [d] shared by every head (one norm applied to each
head) and z [B, T, H, d] the gate's pre-activation.  The backward given dy:

    dz_j     = dy_j * gamma_j * n_j * swish'(z_j),  swish'(z) = s (1 + z (1 - s))
    dn_j     = dy_j * gamma_j * swish(z_j)
    do_j     = r * (dn_j - n_j * mean_i(dn_i * n_i))
    dgamma_j = sum over every (b, t, h) of dy_j * n_j * swish(z_j)

(the RMSNorm gradient: r depends on o through the mean of squares).
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


def norm_gate_fwd(o, z, gamma, eps):
    """y [..., d] from o, z [..., d] (any leading shape) and gamma [d]."""
    o, z, gamma = _f64(o), _f64(z), _f64(gamma)
    if o.shape != z.shape or gamma.shape != (o.shape[-1],):
        raise ValueError("bad shapes")
    r = 1.0 / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    n = o * r
    return gamma * n * (z * _sigmoid(z))


def norm_gate_bwd(o, z, gamma, dy, eps):
    """(do, dz, dgamma) as float64, given dy = dL/dy."""
    o, z, gamma, dy = _f64(o), _f64(z), _f64(gamma), _f64(dy)
    d = o.shape[-1]
    r = 1.0 / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    n = o * r
    s = _sigmoid(z)
    sw = z * s
    dz = dy * gamma * n * s * (1.0 + z * (1.0 - s))
    dn = dy * gamma * sw
    do = r * (dn - n * np.sum(dn * n, axis=-1, keepdims=True) / d)
    dgamma = np.sum((dy * n * sw).reshape(-1, d), axis=0)
    return do, dz, dgamma
