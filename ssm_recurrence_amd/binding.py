"""ctypes binding of the C ABI in include/gla.h (argument marshalling only).

torch supplies device memory and the current HIP stream; every step of the
computation runs in the HIP library.  There is no fallback: if the library is
not built, or the device is not a gfx950, calls raise.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_lib", "libgla.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "gla.h")

GLA_F32, GLA_BF16 = 0, 1
GLA_GATE_SCALAR, GLA_GATE_VECTOR = 0, 1
GLA_SAVE_STATES = 1
STATUS = {0: "GLA_OK", -1: "GLA_E_NULL", -2: "GLA_E_SHAPE", -3: "GLA_E_DTYPE",
          -4: "GLA_E_UNSUPPORTED", -5: "GLA_E_ALIGN", -6: "GLA_E_WORKSPACE",
          -7: "GLA_E_DEVICE", -8: "GLA_E_LAUNCH", -9: "GLA_E_SCRATCH"}


class Problem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("T", ctypes.c_int64), ("H", ctypes.c_int64),
                ("H_qk", ctypes.c_int64), ("d_k", ctypes.c_int64), ("d_v", ctypes.c_int64),
                ("chunk", ctypes.c_int32), ("gate", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("split", ctypes.c_int32), ("ld_qk", ctypes.c_int64), ("ld_v", ctypes.c_int64),
                ("ld_dqk", ctypes.c_int64), ("ld_dv", ctypes.c_int64), ("flags", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("generation", ctypes.c_int64)]


class ConvProblem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("T", ctypes.c_int64), ("C", ctypes.c_int64),
                ("K", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class NormGateProblem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("T", ctypes.c_int64), ("H", ctypes.c_int64),
                ("d", ctypes.c_int64), ("eps", ctypes.c_float), ("dtype", ctypes.c_int32)]


class DeltaProblem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("T", ctypes.c_int64), ("H", ctypes.c_int64),
                ("d_k", ctypes.c_int64), ("d_v", ctypes.c_int64), ("dtype", ctypes.c_int32),
                ("flags", ctypes.c_int32), ("generation", ctypes.c_int64)]


class GlaError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        msg = "%s failed: %s (%d)" % (what, STATUS.get(status, "?"), status)
        try:
            msg += ": " + load().gla_status_str(status).decode()
        except Exception:  # pragma: no cover
            pass
        super().__init__(msg)


_lib = None


def load():
    """Load libgla.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("HIP library not built: %s (run ssm_recurrence_amd.build)" % LIB_PATH)
        lib = ctypes.CDLL(LIB_PATH)
        P, vp, sz = ctypes.POINTER(Problem), ctypes.c_void_p, ctypes.c_size_t
        lib.gla_workspace_size.argtypes = [P, ctypes.c_int, ctypes.POINTER(sz)]
        lib.gla_workspace_size.restype = ctypes.c_int
        lib.gla_fwd.argtypes = [P] + [vp] * 9 + [sz, vp]
        lib.gla_fwd.restype = ctypes.c_int
        lib.gla_fwd_noalloc.argtypes = [P] + [vp] * 9
        lib.gla_fwd_noalloc.restype = ctypes.c_int
        lib.gla_fwd_noalloc_max_scratch.argtypes = []
        lib.gla_fwd_noalloc_max_scratch.restype = sz
        lib.gla_bwd.argtypes = [P] + [vp] * 14 + [sz, vp]
        lib.gla_bwd.restype = ctypes.c_int
        CP = ctypes.POINTER(ConvProblem)
        lib.gla_conv_workspace_size.argtypes = [CP, ctypes.POINTER(sz)]
        lib.gla_conv_workspace_size.restype = ctypes.c_int
        lib.gla_conv_fwd.argtypes = [CP] + [vp] * 5
        lib.gla_conv_fwd.restype = ctypes.c_int
        lib.gla_conv_bwd.argtypes = [CP] + [vp] * 8 + [sz, vp]
        lib.gla_conv_bwd.restype = ctypes.c_int
        NP = ctypes.POINTER(NormGateProblem)
        lib.gla_norm_gate_workspace_size.argtypes = [NP, ctypes.POINTER(sz)]
        lib.gla_norm_gate_workspace_size.restype = ctypes.c_int
        lib.gla_norm_gate_fwd.argtypes = [NP] + [vp] * 5
        lib.gla_norm_gate_fwd.restype = ctypes.c_int
        lib.gla_norm_gate_bwd.argtypes = [NP] + [vp] * 8 + [sz, vp]
        lib.gla_norm_gate_bwd.restype = ctypes.c_int
        DP = ctypes.POINTER(DeltaProblem)
        lib.gla_delta_workspace_size.argtypes = [DP, ctypes.c_int, ctypes.POINTER(sz)]
        lib.gla_delta_workspace_size.restype = ctypes.c_int
        lib.gla_delta_fwd.argtypes = [DP] + [vp] * 10 + [sz, vp]
        lib.gla_delta_fwd.restype = ctypes.c_int
        lib.gla_delta_bwd.argtypes = [DP] + [vp] * 16 + [sz, vp, sz, vp]
        lib.gla_delta_bwd.restype = ctypes.c_int
        lib.gla_status_str.argtypes = [ctypes.c_int]
        lib.gla_status_str.restype = ctypes.c_char_p
        lib.gla_version.argtypes = []
        lib.gla_version.restype = ctypes.c_int
        _lib = lib
    return _lib


def header_functions():
    """Names of the functions include/gla.h declares."""
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(gla_[a-z_0-9]+)\s*\(", txt)))


def make_problem(B, T, H, H_qk, d_k, d_v, gate="scalar", dtype=torch.bfloat16, chunk=64, split=0,
                 ld_qk=0, ld_v=0, ld_dqk=0, ld_dv=0, flags=0, generation=0):
    """gla_problem; split = sequence pieces per (b, h), 0 = chosen by the library;
    ld_* = row strides of q/k, v, dq/dk, dv in elements (0 = packed); flags = 0
    or GLA_SAVE_STATES, with the caller's input generation."""
    return Problem(B, T, H, H_qk, d_k, d_v, chunk,
                   GLA_GATE_VECTOR if gate == "vector" else GLA_GATE_SCALAR,
                   GLA_BF16 if dtype == torch.bfloat16 else GLA_F32, split,
                   ld_qk, ld_v, ld_dqk, ld_dv, flags, 0, generation)


def workspace_size(prob: Problem, backward: bool) -> int:
    n = ctypes.c_size_t(0)
    rc = load().gla_workspace_size(ctypes.byref(prob), int(bool(backward)), ctypes.byref(n))
    if rc:
        raise GlaError(rc, "gla_workspace_size")
    return n.value


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(t, name, dtype=None, strided=False):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if not strided and not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))


def row_stride(t, name):
    """Elements between consecutive tokens of a [B, T, heads, d] tensor whose heads
    of one token are packed (0 when the whole tensor is packed); raises for any
    other layout."""
    if t.is_contiguous():
        return 0
    B, T, nh, d = t.shape
    s0, s1, s2, s3 = t.stride()
    ld = s1 if T > 1 else s0
    ok = (s3 == 1 or d == 1) and (s2 == d or nh == 1) and (T == 1 or s1 == ld) and (B == 1 or s0 == T * ld)
    if not ok or ld < nh * d:
        raise ValueError("%s: token rows must hold packed heads, rows ld elements apart "
                         "(strides %s)" % (name, t.stride()))
    return ld


def problem_of(q, v, g, gate, chunk=64, split=0, k=None, save_states=False, generation=0):
    B, T, H_qk, d_k = q.shape
    H, d_v = v.shape[2], v.shape[3]
    want = (B, T, H, d_k) if gate == "vector" else (B, T, H)
    if tuple(g.shape) != want:
        raise ValueError("g has shape %s, expected %s" % (tuple(g.shape), want))
    ld_qk, ld_v = row_stride(q, "q"), row_stride(v, "v")
    if k is not None and row_stride(k, "k") != ld_qk:
        raise ValueError("q and k must have the same row stride")
    return make_problem(B, T, H, H_qk, d_k, d_v, gate, q.dtype, chunk, split, ld_qk, ld_v,
                        flags=GLA_SAVE_STATES if save_states else 0, generation=generation)


def states_workspace(q, k, v, g, *, gate="scalar", chunk=64, split=0):
    """A workspace for a fwd / bwd pair with save_states=True (one size serves both)."""
    prob = problem_of(q, v, g, gate, chunk, split, k, save_states=True)
    n = workspace_size(prob, True)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=q.device)


def _workspace(prob, backward, device, ws, keep=False):
    """(ws, bytes): the given workspace, or a new one if it is missing or too small
    (keep: the caller's workspace is required, as it carries saved states)."""
    n = workspace_size(prob, backward)
    if n == 0 and not keep:
        return None, 0
    if ws is None or ws.numel() < n:
        if keep:
            raise ValueError("workspace of %d bytes, %d needed" % (0 if ws is None else ws.numel(), n))
        ws = torch.empty(n, dtype=torch.uint8, device=device)
    return ws, ws.numel()


def fwd(q, k, v, g, h0=None, segment_ids=None, *, gate="scalar", chunk=64, want_hT=True,
        out=None, ws=None, split=0, save_states=False, generation=0):
    """o [B,T,H,d_v] (input dtype) and hT [B,H,d_k,d_v] fp32 (None if not wanted).

    save_states=True (GLA_SAVE_STATES): also store the per-chunk states in `ws`
    (states_workspace() makes one), stamped with these inputs and `generation`,
    for a bwd(..., save_states=True, ws=ws) of the same inputs."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, n, q.dtype, strided=True)
    _check(g, "g", q.dtype)
    _check(h0, "h0", torch.float32)
    _check(segment_ids, "segment_ids", torch.int32)
    prob = problem_of(q, v, g, gate, chunk, split, k, save_states, generation)
    if save_states and ws is None:
        raise ValueError("save_states: pass the workspace the backward will be given")
    B, T, H, d_v, d_k = prob.B, prob.T, prob.H, prob.d_v, prob.d_k
    o = out if out is not None else torch.empty((B, T, H, d_v), dtype=q.dtype, device=q.device)
    hT = torch.empty((B, H, d_k, d_v), dtype=torch.float32, device=q.device) if want_hT else None
    ws, nws = _workspace(prob, False, q.device, ws, keep=save_states)
    rc = load().gla_fwd(ctypes.byref(prob), _p(q), _p(k), _p(v), _p(g), _p(h0), _p(segment_ids),
                        _p(o), _p(hT), _p(ws), nws, _stream())
    if rc:
        raise GlaError(rc, "gla_fwd")
    return o, hT


def fwd_noalloc(q, k, v, g, h0=None, segment_ids=None, *, gate="scalar", chunk=64, want_hT=True,
                out=None, split=0):
    """As fwd(), through gla_fwd_noalloc: no workspace (the library's fixed scratch);
    o and hT are allocated here unless `out` is given and want_hT is False."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, n, q.dtype, strided=True)
    _check(g, "g", q.dtype)
    _check(h0, "h0", torch.float32)
    _check(segment_ids, "segment_ids", torch.int32)
    prob = problem_of(q, v, g, gate, chunk, split, k)
    B, T, H, d_v, d_k = prob.B, prob.T, prob.H, prob.d_v, prob.d_k
    o = out if out is not None else torch.empty((B, T, H, d_v), dtype=q.dtype, device=q.device)
    hT = torch.empty((B, H, d_k, d_v), dtype=torch.float32, device=q.device) if want_hT else None
    rc = load().gla_fwd_noalloc(ctypes.byref(prob), _p(q), _p(k), _p(v), _p(g), _p(h0),
                                _p(segment_ids), _p(o), _p(hT), _stream())
    if rc:
        raise GlaError(rc, "gla_fwd_noalloc")
    return o, hT


def fused_views(X, H_qk, d_k, H, d_v):
    """q [B,T,H_qk,d_k], k, v [B,T,H,d_v] as views of a fused projection X of shape
    [B, T, 2*H_qk*d_k + H*d_v] holding q | k | v along its last axis."""
    B, T, W = X.shape
    wq = H_qk * d_k
    if W != 2 * wq + H * d_v:
        raise ValueError("fused width %d, expected %d" % (W, 2 * wq + H * d_v))
    return (X[..., :wq].unflatten(-1, (H_qk, d_k)), X[..., wq:2 * wq].unflatten(-1, (H_qk, d_k)),
            X[..., 2 * wq:].unflatten(-1, (H, d_v)))


def _fused_base(q, k, v):
    """(B, T, W) when q, k, v are the three views fused_views makes of one tensor."""
    B, T, H_qk, d_k = q.shape
    H, d_v = v.shape[2], v.shape[3]
    wq, W, es = H_qk * d_k, 2 * H_qk * d_k + H * d_v, q.element_size()
    if T == 0 or q.untyped_storage().data_ptr() != v.untyped_storage().data_ptr():
        return None
    try:
        lds = (row_stride(q, "q"), row_stride(k, "k"), row_stride(v, "v"))
    except ValueError:
        return None
    if lds != (W, W, W) or k.data_ptr() != q.data_ptr() + wq * es or v.data_ptr() != q.data_ptr() + 2 * wq * es:
        return None
    return B, T, W


def bwd(q, k, v, g, dO, h0=None, segment_ids=None, dhT=None, *, gate="scalar", chunk=64,
        want_dh0=True, ws=None, split=0, grads=None, save_states=False, generation=0):
    """dq, dk [B,T,H_qk,d_k], dv [B,T,H,d_v], dg (shape of g), dh0 fp32 (or None).

    grads = (dq, dk, dv) writes the gradients into those tensors (token rows may
    be strided, as q, k, v may be).  Otherwise, when q, k, v are the views
    fused_views makes of one projection tensor, dq, dk, dv are returned as the
    same views of one fused gradient tensor (fused_grad() of the result gives
    it); else they are packed.

    save_states=True: `ws` is the workspace a fwd(..., save_states=True) of these
    inputs was given; its states are used when its stamp matches these inputs and
    `generation`, else recomputed."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, n, q.dtype, strided=True)
    for t, n in ((g, "g"), (dO, "dO")):
        _check(t, n, q.dtype)
    _check(h0, "h0", torch.float32)
    _check(dhT, "dhT", torch.float32)
    _check(segment_ids, "segment_ids", torch.int32)
    prob = problem_of(q, v, g, gate, chunk, split, k, save_states, generation)
    if save_states and ws is None:
        raise ValueError("save_states: pass the workspace the forward was given")
    if grads is not None:
        dq, dk, dv = grads
        for t, ref, n in ((dq, q, "dq"), (dk, k, "dk"), (dv, v, "dv")):
            _check(t, n, q.dtype, strided=True)
            if t.shape != ref.shape:
                raise ValueError("%s has shape %s, expected %s" % (n, tuple(t.shape), tuple(ref.shape)))
        prob.ld_dqk, prob.ld_dv = row_stride(dq, "dq"), row_stride(dv, "dv")
        if row_stride(dk, "dk") != prob.ld_dqk:
            raise ValueError("dq and dk must have the same row stride")
    elif _fused_base(q, k, v) is not None:
        dX = torch.empty(_fused_base(q, k, v), dtype=q.dtype, device=q.device)
        dq, dk, dv = fused_views(dX, prob.H_qk, prob.d_k, prob.H, prob.d_v)
        prob.ld_dqk = prob.ld_dv = dX.shape[2]
    else:
        dq = torch.empty(q.shape, dtype=q.dtype, device=q.device)
        dk = torch.empty(k.shape, dtype=q.dtype, device=q.device)
        dv = torch.empty(v.shape, dtype=q.dtype, device=q.device)
    dg = torch.empty_like(g)
    dh0 = (torch.empty((prob.B, prob.H, prob.d_k, prob.d_v), dtype=torch.float32, device=q.device)
           if want_dh0 else None)
    ws, nws = _workspace(prob, True, q.device, ws, keep=save_states)
    rc = load().gla_bwd(ctypes.byref(prob), _p(q), _p(k), _p(v), _p(g), _p(h0), _p(segment_ids),
                        _p(dO), _p(dhT), _p(dq), _p(dk), _p(dv), _p(dg), _p(dh0), _p(ws), nws,
                        _stream())
    if rc:
        raise GlaError(rc, "gla_bwd")
    return dq, dk, dv, dg, dh0


def fused_grad(dq):
    """The fused gradient tensor [B, T, W] whose first view is dq (as bwd returns it
    for fused inputs)."""
    B, T = dq.shape[:2]
    ld = row_stride(dq, "dq")
    return dq.as_strided((B, T, ld), (T * ld, ld, 1), dq.storage_offset())


_gla_generation = [0]


class GLAFunction(torch.autograd.Function):
    """Autograd wrapper: forward and backward both run the HIP library.
    save_states=True keeps the forward's workspace, with the per-chunk states the
    forward stored, for the backward (memory held from forward to backward in
    exchange for the backward's state passes); the workspace is stamped with a
    generation of its own (autograd itself rejects inputs changed in between)."""

    @staticmethod
    def forward(ctx, q, k, v, g, h0, segment_ids, gate, save_states=False):
        ws, gen = None, 0
        if save_states:
            _gla_generation[0] += 1
            gen = _gla_generation[0]
            ws = states_workspace(q, k, v, g, gate=gate)
        o, hT = fwd(q, k, v, g, h0, segment_ids, gate=gate, ws=ws, save_states=save_states,
                    generation=gen)
        ctx.save_for_backward(q, k, v, g, h0, segment_ids)
        ctx.gate, ctx.ws, ctx.gen, ctx.saved = gate, ws, gen, save_states
        return o, hT

    @staticmethod
    def backward(ctx, dO, dhT):
        q, k, v, g, h0, seg = ctx.saved_tensors
        dO = dO.contiguous() if dO is not None else torch.zeros(v.shape, dtype=v.dtype, device=v.device)
        dhT = dhT.contiguous().float() if dhT is not None else None
        dq, dk, dv, dg, dh0 = bwd(q, k, v, g, dO, h0, seg, dhT, gate=ctx.gate,
                                  want_dh0=h0 is not None, ws=ctx.ws, save_states=ctx.saved,
                                  generation=ctx.gen)
        ctx.ws = None
        return dq, dk, dv, dg, dh0, None, None, None


class GLAFusedFunction(torch.autograd.Function):
    """Autograd wrapper over a fused projection X [B, T, 2*H_qk*d_k + H*d_v]
    (q | k | v): the kernels read q, k, v in place and the backward writes one
    fused gradient dX; no split, copy or concatenation runs around them."""

    @staticmethod
    def forward(ctx, X, g, h0, segment_ids, H_qk, d_k, gate):
        H = g.shape[2]
        d_v = (X.shape[2] - 2 * H_qk * d_k) // H
        q, k, v = fused_views(X, H_qk, d_k, H, d_v)
        o, hT = fwd(q, k, v, g, h0, segment_ids, gate=gate)
        ctx.save_for_backward(X, g, h0, segment_ids)
        ctx.shape = (H_qk, d_k, H, d_v)
        ctx.gate = gate
        return o, hT

    @staticmethod
    def backward(ctx, dO, dhT):
        X, g, h0, seg = ctx.saved_tensors
        H_qk, d_k, H, d_v = ctx.shape
        q, k, v = fused_views(X, H_qk, d_k, H, d_v)
        dO = dO.contiguous() if dO is not None else torch.zeros(v.shape, dtype=v.dtype, device=v.device)
        dhT = dhT.contiguous().float() if dhT is not None else None
        dX = torch.empty_like(X)
        dq, dk, dv = fused_views(dX, H_qk, d_k, H, d_v)
        _, _, _, dg, dh0 = bwd(q, k, v, g, dO, h0, seg, dhT, gate=ctx.gate,
                               want_dh0=h0 is not None, grads=(dq, dk, dv))
        return dX, dg, dh0, None, None, None, None


def fwd_into(prob, q, k, v, g, h0, seg, o, hT, ws, nws, stream=None):
    """gla_fwd on preallocated buffers (no allocation); raises on a non-zero status."""
    rc = load().gla_fwd(ctypes.byref(prob), _p(q), _p(k), _p(v), _p(g), _p(h0), _p(seg), _p(o),
                        _p(hT), _p(ws), nws, stream if stream is not None else _stream())
    if rc:
        raise GlaError(rc, "gla_fwd")


def bwd_into(prob, q, k, v, g, h0, seg, dO, dhT, dq, dk, dv, dg, dh0, ws, nws, stream=None):
    """gla_bwd on preallocated buffers (no allocation); raises on a non-zero status."""
    rc = load().gla_bwd(ctypes.byref(prob), _p(q), _p(k), _p(v), _p(g), _p(h0), _p(seg), _p(dO),
                        _p(dhT), _p(dq), _p(dk), _p(dv), _p(dg), _p(dh0), _p(ws), nws,
                        stream if stream is not None else _stream())
    if rc:
        raise GlaError(rc, "gla_bwd")


# ---- short depthwise causal convolution (gla_conv_* in include/gla.h)
def conv_problem(x, K=4):
    B, T, C = x.shape
    return ConvProblem(B, T, C, K, GLA_BF16 if x.dtype == torch.bfloat16 else GLA_F32)


def conv_workspace_size(prob: ConvProblem) -> int:
    n = ctypes.c_size_t(0)
    rc = load().gla_conv_workspace_size(ctypes.byref(prob), ctypes.byref(n))
    if rc:
        raise GlaError(rc, "gla_conv_workspace_size")
    return n.value


def conv_fwd(x, w, bias=None, out=None):
    """y [B,T,C] (dtype of x) = SiLU(causal depthwise conv of x with w [K,C] fp32, + bias [C] fp32)."""
    _check(x, "x")
    _check(w, "w", torch.float32)
    _check(bias, "bias", torch.float32)
    prob = conv_problem(x, w.shape[0])
    y = torch.empty_like(x) if out is None else out
    rc = load().gla_conv_fwd(ctypes.byref(prob), _p(x), _p(w), _p(bias), _p(y), _stream())
    if rc:
        raise GlaError(rc, "gla_conv_fwd")
    return y


def conv_bwd(x, w, bias, dy, ws=None, want_db=True):
    """(dx [B,T,C], dw [K,C] fp32, db [C] fp32 or None) given dy = dL/dy."""
    for t, n in ((x, "x"), (dy, "dy")):
        _check(t, n, x.dtype)
    _check(w, "w", torch.float32)
    _check(bias, "bias", torch.float32)
    prob = conv_problem(x, w.shape[0])
    dx = torch.empty_like(x)
    dw = torch.empty_like(w)
    db = torch.empty(x.shape[2], dtype=torch.float32, device=x.device) if want_db else None
    n = conv_workspace_size(prob)
    if ws is None or ws.numel() < n:
        ws = torch.empty(max(n, 1), dtype=torch.uint8, device=x.device)
    rc = load().gla_conv_bwd(ctypes.byref(prob), _p(x), _p(w), _p(bias), _p(dy), _p(dx), _p(dw),
                             _p(db), _p(ws), ws.numel(), _stream())
    if rc:
        raise GlaError(rc, "gla_conv_bwd")
    return dx, dw, db


# ---- output norm and gate (gla_norm_gate_* in include/gla.h)
def norm_gate_problem(o, eps=1e-5):
    B, T, H, d = o.shape
    return NormGateProblem(B, T, H, d, eps, GLA_BF16 if o.dtype == torch.bfloat16 else GLA_F32)


def norm_gate_workspace_size(prob: NormGateProblem) -> int:
    n = ctypes.c_size_t(0)
    rc = load().gla_norm_gate_workspace_size(ctypes.byref(prob), ctypes.byref(n))
    if rc:
        raise GlaError(rc, "gla_norm_gate_workspace_size")
    return n.value


def norm_gate_fwd(o, z, gamma, eps=1e-5, out=None):
    """y [B,T,H,d] (dtype of o) = gamma * RMSNorm(o) per head * swish(z)."""
    _check(o, "o")
    _check(z, "z", o.dtype)
    _check(gamma, "gamma", torch.float32)
    if z.shape != o.shape or gamma.shape != (o.shape[3],):
        raise ValueError("z must be shaped like o and gamma [d]")
    prob = norm_gate_problem(o, eps)
    y = torch.empty_like(o) if out is None else out
    rc = load().gla_norm_gate_fwd(ctypes.byref(prob), _p(o), _p(z), _p(gamma), _p(y), _stream())
    if rc:
        raise GlaError(rc, "gla_norm_gate_fwd")
    return y


def norm_gate_bwd(o, z, gamma, dy, eps=1e-5, ws=None):
    """(do, dz [B,T,H,d], dgamma [d] fp32) given dy = dL/dy."""
    for t, n in ((o, "o"), (z, "z"), (dy, "dy")):
        _check(t, n, o.dtype)
    _check(gamma, "gamma", torch.float32)
    if z.shape != o.shape or dy.shape != o.shape or gamma.shape != (o.shape[3],):
        raise ValueError("z and dy must be shaped like o and gamma [d]")
    prob = norm_gate_problem(o, eps)
    d_o, dz = torch.empty_like(o), torch.empty_like(o)
    dgamma = torch.empty_like(gamma)
    n = norm_gate_workspace_size(prob)
    if ws is None or ws.numel() < n:
        ws = torch.empty(max(n, 1), dtype=torch.uint8, device=o.device)
    rc = load().gla_norm_gate_bwd(ctypes.byref(prob), _p(o), _p(z), _p(gamma), _p(dy), _p(d_o), _p(dz),
                                  _p(dgamma), _p(ws), ws.numel(), _stream())
    if rc:
        raise GlaError(rc, "gla_norm_gate_bwd")
    return d_o, dz, dgamma


class NormGateFunction(torch.autograd.Function):
    """Autograd wrapper: y = gamma * RMSNorm(o) * swish(z), both passes in the HIP library."""

    @staticmethod
    def forward(ctx, o, z, gamma, eps):
        ctx.save_for_backward(o, z, gamma)
        ctx.eps = eps
        return norm_gate_fwd(o, z, gamma, eps)

    @staticmethod
    def backward(ctx, dy):
        o, z, gamma = ctx.saved_tensors
        d_o, dz, dgamma = norm_gate_bwd(o, z, gamma, dy.contiguous(), ctx.eps)
        return d_o, dz, dgamma, None


# ---- gated delta rule (gla_delta_* in include/gla.h)
GLA_DELTA_WS_FROM_FWD = 1


def delta_problem(q, v, flags=0, generation=0):
    B, T, H, d_k = q.shape
    return DeltaProblem(B, T, H, d_k, v.shape[3], GLA_BF16 if q.dtype == torch.bfloat16 else GLA_F32, flags,
                        generation)


def delta_workspace_size(prob: DeltaProblem, backward: bool = False) -> int:
    """Bytes of ws (both calls; backward=False) or of the backward's scratch."""
    n = ctypes.c_size_t(0)
    rc = load().gla_delta_workspace_size(ctypes.byref(prob), int(bool(backward)), ctypes.byref(n))
    if rc:
        raise GlaError(rc, "gla_delta_workspace_size")
    return n.value


def _delta_checks(q, k, v, g, beta):
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (g, "g"), (beta, "beta")):
        _check(t, n, q.dtype)
    B, T, H, _ = q.shape
    if k.shape != q.shape or v.shape[:3] != (B, T, H) or g.shape != (B, T, H) or beta.shape != (B, T, H):
        raise ValueError("delta rule: q, k [B,T,H,d_k], v [B,T,H,d_v], g, beta [B,T,H]")


def _buffer(n, device, buf=None):
    if buf is None or buf.numel() < n:
        buf = torch.empty(max(n, 1), dtype=torch.uint8, device=device)
    return buf


def delta_fwd(q, k, v, g, beta, h0=None, segment_ids=None, *, want_hT=True, ws=None, ws_from_fwd=False,
              generation=0):
    """o [B,T,H,d_v] (input dtype) and hT [B,H,d_k,d_v] fp32 (None if not wanted).
    ws (allocated here when None or too small) receives the per-chunk factors,
    stamped with these inputs and `generation`; with ws_from_fwd
    (GLA_DELTA_WS_FROM_FWD, for a delta_bwd(..., ws_from_fwd=True) given this ws)
    also the states entering the chunks, which that backward then need not
    recompute."""
    _delta_checks(q, k, v, g, beta)
    _check(h0, "h0", torch.float32)
    _check(segment_ids, "segment_ids", torch.int32)
    prob = delta_problem(q, v, GLA_DELTA_WS_FROM_FWD if ws_from_fwd else 0, generation)
    B, T, H, d_k = q.shape
    o = torch.empty(v.shape, dtype=q.dtype, device=q.device)
    hT = torch.empty((B, H, d_k, v.shape[3]), dtype=torch.float32, device=q.device) if want_hT else None
    ws = _buffer(delta_workspace_size(prob), q.device, ws)
    rc = load().gla_delta_fwd(ctypes.byref(prob), _p(q), _p(k), _p(v), _p(g), _p(beta), _p(h0),
                              _p(segment_ids), _p(o), _p(hT), _p(ws), ws.numel(), _stream())
    if rc:
        raise GlaError(rc, "gla_delta_fwd")
    return o, hT


def delta_bwd(q, k, v, g, beta, dO, h0=None, segment_ids=None, dhT=None, *, want_dh0=True, ws=None,
              ws_from_fwd=False, generation=0, scratch=None):
    """dq, dk, dv, dg, dbeta (input dtype) and dh0 fp32 (or None).  ws_from_fwd: ws may
    hold the factors and states a delta_fwd(..., ws_from_fwd=True) computed for these
    inputs and `generation`; the library reuses them only when the workspace's stamp
    says so, and recomputes otherwise (GLA_DELTA_WS_FROM_FWD).  scratch: the
    backward's own workspace (allocated here when None or too small)."""
    _delta_checks(q, k, v, g, beta)
    _check(dO, "dO", q.dtype)
    _check(h0, "h0", torch.float32)
    _check(dhT, "dhT", torch.float32)
    _check(segment_ids, "segment_ids", torch.int32)
    prob = delta_problem(q, v, GLA_DELTA_WS_FROM_FWD if ws_from_fwd else 0, generation)
    B, T, H, d_k = q.shape
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dg, dbeta = torch.empty_like(g), torch.empty_like(beta)
    dh0 = (torch.empty((B, H, d_k, v.shape[3]), dtype=torch.float32, device=q.device)
           if want_dh0 else None)
    ws = _buffer(delta_workspace_size(prob), q.device, ws)
    scratch = _buffer(delta_workspace_size(prob, True), q.device, scratch)
    rc = load().gla_delta_bwd(ctypes.byref(prob), _p(q), _p(k), _p(v), _p(g), _p(beta), _p(h0),
                              _p(segment_ids), _p(dO), _p(dhT), _p(dq), _p(dk), _p(dv), _p(dg),
                              _p(dbeta), _p(dh0), _p(ws), ws.numel(), _p(scratch), scratch.numel(),
                              _stream())
    if rc:
        raise GlaError(rc, "gla_delta_bwd")
    return dq, dk, dv, dg, dbeta, dh0


_delta_generation = [0]


class DeltaFunction(torch.autograd.Function):
    """Autograd wrapper of the gated delta rule: both passes run the HIP library.
    The forward's workspace (its per-chunk factors and states) is kept for the backward,
    stamped with a generation of its own (autograd itself rejects inputs changed
    in place in between); the backward's scratch is allocated in the backward."""

    @staticmethod
    def forward(ctx, q, k, v, g, beta, h0, segment_ids):
        _delta_generation[0] += 1
        gen = _delta_generation[0]
        ws = _buffer(delta_workspace_size(delta_problem(q, v, GLA_DELTA_WS_FROM_FWD)), q.device)
        o, hT = delta_fwd(q, k, v, g, beta, h0, segment_ids, ws=ws, ws_from_fwd=True, generation=gen)
        ctx.save_for_backward(q, k, v, g, beta, h0, segment_ids)
        ctx.ws, ctx.gen = ws, gen
        return o, hT

    @staticmethod
    def backward(ctx, dO, dhT):
        q, k, v, g, beta, h0, seg = ctx.saved_tensors
        dO = dO.contiguous() if dO is not None else torch.zeros(v.shape, dtype=v.dtype, device=v.device)
        dhT = dhT.contiguous().float() if dhT is not None else None
        dq, dk, dv, dg, dbeta, dh0 = delta_bwd(q, k, v, g, beta, dO, h0, seg, dhT, want_dh0=h0 is not None,
                                               ws=ctx.ws, ws_from_fwd=True, generation=ctx.gen)
        return dq, dk, dv, dg, dbeta, dh0, None
