"""Pins for the fp64 output norm-and-gate oracle (oracle/norm_gate.py), on the CPU.

Each pin checks the oracle against something other than itself:
  - torch's own rms_norm and silu in float64, with autograd for every gradient
    (a library forward and an independent backward);
  - central finite differences of L = <y, dy> on a tiny case;
  - closed forms: with one channel and eps = 0 the norm is sign(o), so
    y = gamma * sign(o) * swish(z); with eps = 0 the output does not change when
    a head's o is scaled by c > 0, so the input gradient is orthogonal to o;
  - the bias-free swish limit: for large z, swish(z) -> z.
A planted mistake in a copy of the oracle (eps outside the square root, a sum
instead of the mean, a sigmoid gate instead of swish, the RMSNorm gradient
without its projection term, dgamma without the normalised output) fails at
least one pin.
"""
import numpy as np
import pytest
import torch

import oracle.norm_gate as on

EPS = 1e-3


def rand_case(seed, shape=(2, 3, 2, 8), scale=1.0):
    rng = np.random.default_rng(seed)
    o = rng.standard_normal(shape) * scale
    z = rng.standard_normal(shape) * 2
    gamma = rng.uniform(0.5, 1.5, shape[-1])
    dy = rng.standard_normal(shape)
    return o, z, gamma, dy


def close(a, b, tol=1e-10):
    a, b = np.asarray(a), np.asarray(b)
    return np.max(np.abs(a - b)) <= tol * max(1.0, np.max(np.abs(b)))


def pin_torch(fwd, bwd, o, z, gamma, dy, eps=EPS):
    ot = torch.tensor(o, requires_grad=True)
    zt = torch.tensor(z, requires_grad=True)
    gt = torch.tensor(gamma, requires_grad=True)
    y = torch.nn.functional.rms_norm(ot, (o.shape[-1],), weight=gt, eps=eps) * \
        torch.nn.functional.silu(zt)
    (y * torch.tensor(dy)).sum().backward()
    do, dz, dg = bwd(o, z, gamma, dy, eps)
    return (close(fwd(o, z, gamma, eps), y.detach().numpy()) and close(do, ot.grad.numpy())
            and close(dz, zt.grad.numpy()) and close(dg, gt.grad.numpy()))


def pin_finite_differences(fwd, bwd, o, z, gamma, dy, eps=EPS, h=1e-6):
    L = lambda o_, z_, g_: float(np.sum(fwd(o_, z_, g_, eps) * dy))
    grads = bwd(o, z, gamma, dy, eps)
    for i, (arr, g) in enumerate(zip((o, z, gamma), grads)):
        for idx in list(np.ndindex(arr.shape))[::2]:
            p, m = arr.copy(), arr.copy()
            p[idx] += h
            m[idx] -= h
            args_p = [p if j == i else a for j, a in enumerate((o, z, gamma))]
            args_m = [m if j == i else a for j, a in enumerate((o, z, gamma))]
            num = (L(*args_p) - L(*args_m)) / (2 * h)
            if abs(num - g[idx]) > 1e-6 * max(1.0, abs(num)):
                return False
    return True


def pin_one_channel(fwd, seed=3):
    o, z, gamma, _ = rand_case(seed, shape=(4, 5, 1))
    sw = z / (1 + np.exp(-z))
    return close(fwd(o, z, gamma, 0.0), gamma * np.sign(o) * sw)


def pin_scale_invariance(fwd, bwd, seed=4):
    o, z, gamma, dy = rand_case(seed)
    c = np.exp(np.random.default_rng(seed).standard_normal(o.shape[:-1] + (1,)))
    do = bwd(o, z, gamma, dy, 0.0)[0]
    return (close(fwd(c * o, z, gamma, 0.0), fwd(o, z, gamma, 0.0))
            and np.max(np.abs(np.sum(do * o, axis=-1))) <= 1e-12 * np.max(np.abs(do)) * np.max(np.abs(o)) * o.shape[-1])


def pin_large_gate(fwd, seed=5):
    o, _, gamma, _ = rand_case(seed)
    z = np.full(o.shape, 40.0)
    n = o / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + EPS)
    return close(fwd(o, z, gamma, EPS), gamma * n * 40.0, tol=1e-12)


def all_pins(fwd, bwd):
    res = {}
    o, z, gamma, dy = rand_case(1)
    res["torch rms_norm + silu, autograd"] = pin_torch(fwd, bwd, o, z, gamma, dy)
    o2, z2, g2, dy2 = rand_case(2, shape=(1, 2, 2, 4), scale=0.05)  # eps matters at this scale
    res["torch, small o"] = pin_torch(fwd, bwd, o2, z2, g2, dy2)
    res["finite differences"] = pin_finite_differences(fwd, bwd, o2, z2, g2, dy2)
    res["one channel"] = pin_one_channel(fwd)
    res["scale invariance"] = pin_scale_invariance(fwd, bwd)
    res["large gate"] = pin_large_gate(fwd)
    return res


def test_oracle_passes_every_pin():
    res = all_pins(on.norm_gate_fwd, on.norm_gate_bwd)
    assert all(res.values()), res


# ---- planted mistakes: each fails at least one pin
def _sig(z):
    return 1 / (1 + np.exp(-z))


def mut_eps_outside_fwd(o, z, gamma, eps):
    n = o / (np.sqrt(np.mean(o * o, axis=-1, keepdims=True)) + eps)
    return gamma * n * z * _sig(z)


def mut_sum_fwd(o, z, gamma, eps):
    n = o / np.sqrt(np.sum(o * o, axis=-1, keepdims=True) + eps)
    return gamma * n * z * _sig(z)


def mut_sigmoid_gate_fwd(o, z, gamma, eps):
    return on.norm_gate_fwd(o, z, gamma, eps) / np.where(z == 0, 1, z)


def mut_no_projection_bwd(o, z, gamma, dy, eps):
    do, dz, dg = on.norm_gate_bwd(o, z, gamma, dy, eps)
    r = 1 / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    return r * dy * gamma * z * _sig(z), dz, dg


def mut_dgamma_bwd(o, z, gamma, dy, eps):
    do, dz, _ = on.norm_gate_bwd(o, z, gamma, dy, eps)
    return do, dz, np.sum((dy * z * _sig(z)).reshape(-1, o.shape[-1]), axis=0)


@pytest.mark.parametrize("fwd,bwd,name", [
    (mut_eps_outside_fwd, on.norm_gate_bwd, "eps outside the square root"),
    (mut_sum_fwd, on.norm_gate_bwd, "sum instead of mean"),
    (mut_sigmoid_gate_fwd, on.norm_gate_bwd, "sigmoid gate"),
    (on.norm_gate_fwd, mut_no_projection_bwd, "RMSNorm gradient without projection"),
    (on.norm_gate_fwd, mut_dgamma_bwd, "dgamma without the normalised output"),
])
def test_pins_catch_planted_mistakes(fwd, bwd, name):
    res = all_pins(fwd, bwd)
    assert not all(res.values()), "%s passed every pin" % name
