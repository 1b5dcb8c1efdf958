"""fp64 CPU oracle for the gated linear-attention recurrence (test infrastructure).

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library never does, and this
package imports nothing from it.  The arithmetic lives in ``gla_oracle.c``
(plain C, one token at a time, double precision); this file only compiles it
with gcc and marshals numpy arrays through ctypes.

What it computes is stated in the header of ``gla_oracle.c``: the recurrence
S_t = diag(alpha_t) S_{t-1} + k_t v_t^T, o_t = S_t^T q_t written on the FLAT
page ("FLAT: Flash Linear Attention on TPUs", Linear Attention > Forward and
Backward Recurrence), with the document resets of the JLA page ("JLA: JAX
Linear Attention", segment_ids paragraph).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gla_oracle.c")
_BUILD = os.path.join(_HERE, "_build")
_LIB_PATH = os.path.join(_BUILD, "libgla_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into oracle/_build/libgla_oracle.so."""
    global _lib
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    os.makedirs(_BUILD, exist_ok=True)
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c99", "-Wall", "-Wextra", "-shared", "-fPIC", "-pthread",
           "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    _lib = None
    return _LIB_PATH


def _load(path=None):
    global _lib
    if _lib is None or path is not None:
        if path is None and not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(path or _LIB_PATH)
        i64, i32, dp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        lib.gla_oracle_fwd.argtypes = [i64] * 6 + [i32] + [dp] * 8 + [i32]
        lib.gla_oracle_fwd.restype = i32
        lib.gla_oracle_bwd.argtypes = [i64] * 6 + [i32] + [dp] * 13 + [i32]
        lib.gla_oracle_bwd.restype = i32
        lib.gla_oracle_bwd_per_head.argtypes = [i64] * 6 + [i32] + [dp] * 10 + [i32]
        lib.gla_oracle_bwd_per_head.restype = i32
        _lib = lib
    return _lib


def use_library(path=None):
    """Point this module at another build of gla_oracle.c (None: the default one).

    Used by the test that plants mistakes in a copy of the oracle."""
    global _lib
    _lib = None
    if path is not None:
        _load(path)


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):  # a torch tensor: take its exact values
        x = x.detach().to("cpu")
        import torch
        x = x.to(torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _seg(x):
    if x is None:
        return None
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dims(q, v, g, gate):
    B, T, Hqk, dk = q.shape
    H, dv = v.shape[2], v.shape[3]
    if v.shape[:2] != (B, T) or H % Hqk:
        raise ValueError("bad shapes")
    want_g = (B, T, H, dk) if gate == "vector" else (B, T, H)
    if tuple(g.shape) != want_g:
        raise ValueError("gate shape %s, expected %s" % (tuple(g.shape), want_g))
    return B, T, H, Hqk, dk, dv


def fwd(q, k, v, g, h0=None, segment_ids=None, gate="scalar", threads=None):
    """Forward: returns (o [B,T,H,dv], hT [B,H,dk,dv]) as float64 numpy arrays."""
    q, k, v, g, h0 = _f64(q), _f64(k), _f64(v), _f64(g), _f64(h0)
    seg = _seg(segment_ids)
    B, T, H, Hqk, dk, dv = _dims(q, v, g, gate)
    o = np.zeros((B, T, H, dv))
    hT = np.zeros((B, H, dk, dv))
    rc = _load().gla_oracle_fwd(B, T, H, Hqk, dk, dv, int(gate == "vector"), _ptr(q), _ptr(k),
                                _ptr(v), _ptr(g), _ptr(h0), _ptr(seg), _ptr(o), _ptr(hT),
                                threads or default_threads())
    if rc:
        raise RuntimeError("gla_oracle_fwd failed: %d" % rc)
    return o, hT


def bwd(q, k, v, g, dO, h0=None, segment_ids=None, dhT=None, gate="scalar", threads=None):
    """Backward: returns (dq, dk, dv, dg, dh0) as float64 numpy arrays.

    dq and dk are summed over the heads that share a q/k head.
    """
    q, k, v, g, dO, h0, dhT = map(_f64, (q, k, v, g, dO, h0, dhT))
    seg = _seg(segment_ids)
    B, T, H, Hqk, dk, dv = _dims(q, v, g, gate)
    dq = np.zeros((B, T, Hqk, dk))
    dkk = np.zeros((B, T, Hqk, dk))
    dvv = np.zeros((B, T, H, dv))
    dg = np.zeros(g.shape)
    dh0 = np.zeros((B, H, dk, dv))
    rc = _load().gla_oracle_bwd(B, T, H, Hqk, dk, dv, int(gate == "vector"), _ptr(q), _ptr(k),
                                _ptr(v), _ptr(g), _ptr(h0), _ptr(seg), _ptr(dO), _ptr(dhT),
                                _ptr(dq), _ptr(dkk), _ptr(dvv), _ptr(dg), _ptr(dh0),
                                threads or default_threads())
    if rc:
        raise RuntimeError("gla_oracle_bwd failed: %d" % rc)
    return dq, dkk, dvv, dg, dh0


def bwd_per_head(q, k, v, g, dO, h0=None, segment_ids=None, dhT=None, gate="scalar",
                 threads=None):
    """Per-head dq, dk ([B,T,H,dk]) before the sum over heads sharing q/k."""
    q, k, v, g, dO, h0, dhT = map(_f64, (q, k, v, g, dO, h0, dhT))
    seg = _seg(segment_ids)
    B, T, H, Hqk, dk, dv = _dims(q, v, g, gate)
    dq = np.zeros((B, T, H, dk))
    dkk = np.zeros((B, T, H, dk))
    rc = _load().gla_oracle_bwd_per_head(B, T, H, Hqk, dk, dv, int(gate == "vector"), _ptr(q),
                                         _ptr(k), _ptr(v), _ptr(g), _ptr(h0), _ptr(seg),
                                         _ptr(dO), _ptr(dhT), _ptr(dq), _ptr(dkk),
                                         threads or default_threads())
    if rc:
        raise RuntimeError("gla_oracle_bwd_per_head failed: %d" % rc)
    return dq, dkk
