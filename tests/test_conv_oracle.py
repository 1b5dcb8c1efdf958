"""Pins for the fp64 convolution oracle (oracle/conv.py), all on the CPU.

Each pin checks the oracle against something other than itself:
  - numpy.convolve per channel (a library convolution, no shifted copies);
  - torch's grouped conv1d and SiLU in float64, with autograd for every gradient
    (an independent backward);
  - central finite differences of L = <y, dy> on a tiny case;
  - K = 1, where the convolution is an elementwise affine map;
  - causality: a change of x at step t0 moves y only at t0 .. t0 + K - 1.
A planted mistake in a copy of the oracle (reversed taps, a dropped SiLU'
term, the input gradient shifted the wrong way, the bias gradient averaged)
fails at least one pin.
"""
import numpy as np
import pytest
import torch

import oracle.conv as oc


def rand_case(seed, B=2, T=37, C=5, K=4, bias=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, T, C))
    w = rng.uniform(-1, 1, (K, C))
    b = rng.uniform(-1, 1, C) if bias else None
    dy = rng.standard_normal((B, T, C))
    return x, w, b, dy


def close(a, b, tol=1e-10):
    a, b = np.asarray(a), np.asarray(b)
    return np.max(np.abs(a - b)) <= tol * max(1.0, np.max(np.abs(b)))


def pin_numpy_convolve(fwd, x, w, b):
    B, T, C = x.shape
    z = np.zeros_like(x)
    for bb in range(B):
        for c in range(C):
            z[bb, :, c] = np.convolve(x[bb, :, c], w[::-1, c])[:T] + (0.0 if b is None else b[c])
    y = z / (1 + np.exp(-z))
    return close(fwd(x, w, b), y)


def torch_ref(x, w, b, dy):
    K, C = w.shape
    xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    wt = torch.tensor(w, dtype=torch.float64, requires_grad=True)
    bt = torch.tensor(b if b is not None else np.zeros(C), dtype=torch.float64, requires_grad=True)
    # conv1d is a cross-correlation: weight[c, 0, j] multiplies input[t - (K - 1) + j],
    # which is tap j here; left padding K - 1 makes it causal
    inp = torch.nn.functional.pad(xt.permute(0, 2, 1), (K - 1, 0))
    z = torch.nn.functional.conv1d(inp, wt.t().unsqueeze(1), bt, groups=C)
    y = torch.nn.functional.silu(z).permute(0, 2, 1)
    (y * torch.tensor(dy)).sum().backward()
    return y.detach().numpy(), xt.grad.numpy(), wt.grad.numpy(), bt.grad.numpy()


def pin_torch(fwd, bwd, x, w, b, dy):
    y, dx, dw, db = torch_ref(x, w, b, dy)
    gx, gw, gb = bwd(x, w, b, dy)
    ok = close(fwd(x, w, b), y) and close(gx, dx) and close(gw, dw)
    return ok and (b is None or close(gb, db))


def pin_finite_differences(fwd, bwd, x, w, b, dy, h=1e-6):
    L = lambda x_, w_, b_: float(np.sum(fwd(x_, w_, b_) * dy))
    gx, gw, gb = bwd(x, w, b, dy)
    for arr, g in ((x, gx), (w, gw), (b, gb)):
        for idx in list(np.ndindex(arr.shape))[::3]:
            p, m = arr.copy(), arr.copy()
            p[idx] += h
            m[idx] -= h
            args_p = [p if a is arr else a for a in (x, w, b)]
            args_m = [m if a is arr else a for a in (x, w, b)]
            num = (L(*args_p) - L(*args_m)) / (2 * h)
            if abs(num - g[idx]) > 1e-6 * max(1.0, abs(num)):
                return False
    return True


def pin_k1(fwd, seed=3):
    x, w, b, _ = rand_case(seed, K=1)
    z = w[0] * x + b
    return close(fwd(x, w, b), z / (1 + np.exp(-z)))


def pin_causal(fwd, seed=4):
    x, w, b, _ = rand_case(seed, T=20, K=4)
    y0 = fwd(x, w, b)
    x2 = x.copy()
    x2[:, 9, :] += 1.0
    d = np.abs(fwd(x2, w, b) - y0).max(axis=(0, 2))
    return bool(np.all(d[:9] == 0) and np.all(d[9:13] > 0) and np.all(d[13:] == 0))


def all_pins(fwd, bwd):
    results = {}
    x, w, b, dy = rand_case(1)
    results["numpy.convolve"] = pin_numpy_convolve(fwd, x, w, b)
    results["torch autograd"] = pin_torch(fwd, bwd, x, w, b, dy)
    xs, ws, bs, dys = rand_case(2, B=1, T=7, C=2)
    results["finite differences"] = pin_finite_differences(fwd, bwd, xs, ws, bs, dys)
    results["K = 1"] = pin_k1(fwd)
    results["causality"] = pin_causal(fwd)
    return results


def test_oracle_passes_every_pin():
    res = all_pins(oc.conv_fwd, oc.conv_bwd)
    assert all(res.values()), res


def test_no_bias_and_short_rows():
    for T in (1, 2, 3, 5):
        x, w, _, dy = rand_case(5 + T, T=T, bias=False)
        assert pin_numpy_convolve(oc.conv_fwd, x, w, None)
        assert pin_torch(oc.conv_fwd, oc.conv_bwd, x, w, None, dy)


# ---- planted mistakes: each is caught by at least one pin
def _sig(z):
    return 1 / (1 + np.exp(-z))


def mut_reversed_taps_fwd(x, w, b=None):
    return oc.conv_fwd(x, w[::-1].copy(), b)


def mut_reversed_taps_bwd(x, w, b, dy):
    return oc.conv_bwd(x, w[::-1].copy(), b, dy)


def mut_dropped_term_bwd(x, w, b, dy):
    z = oc.conv_z(x, w, b)
    K, T = w.shape[0], x.shape[1]
    dz = dy * _sig(z)  # SiLU' without the z (1 - s) term
    dx = np.zeros_like(x)
    dw = np.zeros_like(w)
    for k in range(K):
        s = K - 1 - k
        dx[:, :T - s] += w[k] * dz[:, s:]
        dw[k] = np.sum(x[:, :T - s] * dz[:, s:], axis=(0, 1))
    return dx, dw, dz.sum(axis=(0, 1))


def mut_wrong_shift_bwd(x, w, b, dy):
    dx, dw, db = oc.conv_bwd(x, w, b, dy)
    z = oc.conv_z(x, w, b)
    s_ = _sig(z)
    dz = dy * s_ * (1 + z * (1 - s_))
    K, T = w.shape[0], x.shape[1]
    dx = np.zeros_like(x)
    for k in range(K):
        s = K - 1 - k
        dx[:, s:] += w[k] * dz[:, :T - s]  # causal instead of anti-causal
    return dx, dw, db


def mut_mean_bias_bwd(x, w, b, dy):
    dx, dw, db = oc.conv_bwd(x, w, b, dy)
    return dx, dw, db / (x.shape[0] * x.shape[1])


@pytest.mark.parametrize("fwd,bwd,name", [
    (mut_reversed_taps_fwd, mut_reversed_taps_bwd, "reversed taps"),
    (oc.conv_fwd, mut_dropped_term_bwd, "dropped SiLU' term"),
    (oc.conv_fwd, mut_wrong_shift_bwd, "input gradient shifted the wrong way"),
    (oc.conv_fwd, mut_mean_bias_bwd, "bias gradient averaged"),
])
def test_pins_catch_planted_mistakes(fwd, bwd, name):
    res = all_pins(fwd, bwd)
    assert not all(res.values()), "%s passed every pin" % name
