"""The C-ABI library: it loads, exports every function include/gla.h declares,
and rejects bad arguments on the host before touching a device (no GPU needed)."""
import ctypes

import pytest
import torch

from ssm_recurrence_amd import binding as gb


@pytest.fixture(scope="module")
def lib():
    return gb.load()


def test_exports_every_declared_function(lib):
    names = gb.header_functions()
    assert set(names) >= {"gla_fwd", "gla_bwd", "gla_workspace_size", "gla_status_str", "gla_version"}
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for s in range(0, -10, -1):
        assert lib.gla_status_str(s)
    assert lib.gla_version() >= 100


FAKE = 0x10000  # 16-byte aligned, never dereferenced: every call here fails validation first


def call_fwd(lib, prob, ptrs=None, ws_bytes=0):
    p = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, h0=None, seg=None, o=FAKE, hT=None, ws=None)
    p.update(ptrs or {})
    c = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.gla_fwd(None if prob is None else ctypes.byref(prob), c(p["q"]), c(p["k"]),
                       c(p["v"]), c(p["g"]), c(p["h0"]), c(p["seg"]), c(p["o"]), c(p["hT"]),
                       c(p["ws"]), ws_bytes, None)


def call_bwd(lib, prob, ptrs=None, ws_bytes=0):
    names = ["q", "k", "v", "g", "h0", "seg", "dO", "dhT", "dq", "dk", "dv", "dg", "dh0", "ws"]
    p = {n: FAKE for n in names}
    p.update(h0=None, seg=None, dhT=None, dh0=None, ws=None)
    p.update(ptrs or {})
    c = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.gla_bwd(ctypes.byref(prob), *[c(p[n]) for n in names], ws_bytes, None)


def prob(**kw):
    d = dict(B=2, T=100, H=4, H_qk=2, d_k=128, d_v=64, gate="vector", dtype=torch.bfloat16)
    d.update(kw)
    return gb.make_problem(**d)


def test_null_problem_and_pointers(lib):
    assert call_fwd(lib, None) == -1
    assert call_fwd(lib, prob(), {"q": None}) == -1
    assert call_fwd(lib, prob(), {"o": None}) == -1
    assert call_bwd(lib, prob(), {"dg": None}) == -1
    n = ctypes.c_size_t()
    assert lib.gla_workspace_size(ctypes.byref(prob()), 1, None) == -1


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), -2), (dict(T=-1), -2), (dict(H=3, H_qk=2), -2), (dict(H_qk=5, H=4), -2),
    (dict(d_k=0), -2), (dict(d_k=96), -4), (dict(d_v=32), -4), (dict(chunk=32), -4),
    (dict(chunk=0), -2),
])
def test_shape_errors(lib, kw, code):
    assert call_fwd(lib, prob(**kw)) == code
    assert call_bwd(lib, prob(**kw)) == code


def test_dtype_and_gate_errors(lib):
    p = prob()
    p.dtype = 7
    assert call_fwd(lib, p) == -3
    p = prob()
    p.gate = 2
    assert call_bwd(lib, p) == -3
    p = prob()
    p.split = -1
    assert call_fwd(lib, p) == -2
    assert call_bwd(lib, p) == -2


def test_alignment_errors(lib):
    assert call_fwd(lib, prob(), {"v": FAKE + 4}) == -5
    assert call_fwd(lib, prob(), {"h0": FAKE + 8}) == -5
    assert call_bwd(lib, prob(), {"dh0": FAKE + 2}) == -5


def test_workspace_errors_and_size(lib):
    p = prob()
    n = ctypes.c_size_t()
    assert lib.gla_workspace_size(ctypes.byref(p), 1, ctypes.byref(n)) == 0
    assert n.value > 0
    assert call_bwd(lib, p, {"ws": None}, ws_bytes=n.value) == -6
    assert call_bwd(lib, p, {"ws": FAKE}, ws_bytes=n.value - 1) == -6
    assert lib.gla_workspace_size(ctypes.byref(p), 0, ctypes.byref(n)) == 0


def _ws(lib, p, backward):
    n = ctypes.c_size_t()
    assert lib.gla_workspace_size(ctypes.byref(p), int(backward), ctypes.byref(n)) == 0
    return n.value


def test_saved_states_flags_and_workspace(lib):
    """GLA_SAVE_STATES: other flag bits and a non-zero reserved word are refused;
    with the flag one workspace size serves both calls; where the forward stores
    states (scalar gate, 128 x 128) it holds the stamp (256 bytes) and the
    state entering every chunk plus the final one, in the input dtype, besides
    everything the backward alone needs; elsewhere it is the backward's own."""
    for kw in (dict(flags=2), dict(flags=gb.GLA_SAVE_STATES | 4)):
        p = prob(**kw)
        assert call_fwd(lib, p) == -4
        assert call_bwd(lib, p) == -4
        assert lib.gla_workspace_size(ctypes.byref(p), 1, ctypes.byref(ctypes.c_size_t())) == -4
    p = prob()
    p.reserved = 1
    assert call_fwd(lib, p) == -4
    for dtype, es in ((torch.bfloat16, 2), (torch.float32, 4)):
        for gate in ("scalar", "vector"):
            for d_k, d_v in ((128, 128), (64, 128), (64, 64)):
                for T, split in ((100, 0), (64 * 40, 4), (1, 0)):
                    kw = dict(B=2, T=T, H=4, H_qk=2, d_k=d_k, d_v=d_v, gate=gate, dtype=dtype, split=split)
                    plain = prob(**kw)
                    saved = prob(flags=gb.GLA_SAVE_STATES, generation=7, **kw)
                    nc = (T + 63) // 64
                    states = 2 * 4 * (nc + 1) * d_k * d_v * es
                    assert _ws(lib, saved, False) == _ws(lib, saved, True)
                    assert _ws(lib, saved, False) >= max(_ws(lib, plain, False), _ws(lib, plain, True))
                    if gate == "scalar" and d_k == d_v == 128:
                        # (where the forward stores them)
                        assert _ws(lib, saved, True) >= _ws(lib, plain, True) + 256
                        assert _ws(lib, saved, False) >= 256 + states
                    else:
                        assert _ws(lib, saved, True) == _ws(lib, plain, True)
    assert call_fwd_noalloc(lib, prob(flags=gb.GLA_SAVE_STATES)) == -4


def test_split_workspace(lib):
    """The sequence split needs piece summaries and entry states: two fp32
    [B, H, P, d_k, d_v] buffers plus the decay products, in both passes."""
    B, H, T, d = 1, 2, 64 * 16, 64
    base = prob(B=B, T=T, H=H, H_qk=H, d_k=d, d_v=d)
    base.split = 1
    assert _ws(lib, base, False) == 0
    bwd1 = _ws(lib, base, True)
    for P in (2, 4, 16):
        p = prob(B=B, T=T, H=H, H_qk=H, d_k=d, d_v=d)
        p.split = P
        need = 2 * B * H * P * d * d * 4 + B * H * P * d * 4
        assert _ws(lib, p, False) >= need
        assert _ws(lib, p, True) >= bwd1 + need
    # more pieces than chunks: capped at one chunk per piece
    p = prob(B=B, T=T, H=H, H_qk=H, d_k=d, d_v=d)
    p.split = 1000
    q = prob(B=B, T=T, H=H, H_qk=H, d_k=d, d_v=d)
    q.split = 16
    assert _ws(lib, p, True) == _ws(lib, q, True)


def test_auto_split_only_when_short_of_workgroups(lib):
    """split = 0: long rows at small B*H are split, large B*H is not."""
    small_bh = prob(B=1, T=65536, H=16, H_qk=16, d_k=128, d_v=128)
    large_bh = prob(B=16, T=2048, H=16, H_qk=16, d_k=128, d_v=128)  # one workgroup per head fills the device
    assert _ws(lib, small_bh, False) > 0
    assert _ws(lib, large_bh, False) == 0
    one = prob(B=1, T=65536, H=16, H_qk=16, d_k=128, d_v=128)
    one.split = 1
    assert _ws(lib, small_bh, True) > _ws(lib, one, True)


@pytest.mark.parametrize("kw,code", [
    (dict(ld_qk=255), -2),                          # below the packed width (2 x 128)
    (dict(ld_qk=260), -2),                          # not whole 16-byte units in bf16
    (dict(ld_v=100), -2), (dict(ld_dqk=-8), -2), (dict(ld_dv=1 << 40), -2),
    (dict(ld_qk=264, ld_v=264, ld_dqk=264, ld_dv=264), -7),   # valid (no device here)
    (dict(ld_qk=260, dtype=torch.float32), -7),     # 16-byte units of fp32
    (dict(ld_qk=258, dtype=torch.float32), -2),
])
@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-device path")
def test_row_stride_checks(lib, kw, code):
    """Row strides of q/k, v, dq/dk, dv: 0 (packed) or at least the packed width in
    whole 16-byte units; valid ones get past the stride checks (to the device
    check, or the backward's missing workspace)."""
    assert call_fwd(lib, prob(**kw)) == code
    assert call_bwd(lib, prob(**kw)) == (-6 if code == -7 else code)


def test_row_strides_leave_workspace_unchanged(lib):
    a, b = ctypes.c_size_t(), ctypes.c_size_t()
    assert lib.gla_workspace_size(ctypes.byref(prob()), 1, ctypes.byref(a)) == 0
    assert lib.gla_workspace_size(ctypes.byref(prob(ld_qk=1024, ld_v=1024, ld_dqk=512, ld_dv=4096)), 1,
                                  ctypes.byref(b)) == 0
    assert a.value == b.value


def test_binding_row_stride_and_fused_views():
    """Host logic of the binding: row strides read from tensor strides, the fused
    projection's views, and the fused gradient recovered from dq (CPU tensors)."""
    B, T, H_qk, d_k, H, d_v = 2, 5, 2, 64, 4, 32
    W = 2 * H_qk * d_k + H * d_v
    X = torch.arange(B * T * W, dtype=torch.float32).reshape(B, T, W)
    q, k, v = gb.fused_views(X, H_qk, d_k, H, d_v)
    assert q.shape == (B, T, H_qk, d_k) and v.shape == (B, T, H, d_v)
    assert [gb.row_stride(t, "t") for t in (q, k, v)] == [W, W, W]
    assert gb.row_stride(X[..., :W].reshape(B, T, 8, W // 8), "x") == 0
    assert torch.equal(q[1, 3, 1], X[1, 3, d_k:2 * d_k]) and torch.equal(v[0, 4, 3], X[0, 4, -d_v:])
    assert gb._fused_base(q, k, v) == (B, T, W)
    assert gb._fused_base(q.contiguous(), k, v) is None
    assert gb.fused_grad(q).data_ptr() == X.data_ptr() and gb.fused_grad(q).shape == X.shape
    with pytest.raises(ValueError):
        gb.row_stride(torch.zeros(B, H, T, d_k).transpose(1, 2), "q")   # heads not packed in a row
    with pytest.raises(ValueError):
        gb.fused_views(X[..., 1:], H_qk, d_k, H, d_v)


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-device path")
def test_valid_call_without_gpu_reports_device_error(lib):
    """No silent fallback: with no usable device a valid call returns GLA_E_DEVICE."""
    assert call_fwd(lib, prob(H_qk=4, d_v=128)) == -7


def call_fwd_noalloc(lib, prob, ptrs=None):
    p = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, h0=None, seg=None, o=FAKE, hT=None)
    p.update(ptrs or {})
    c = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.gla_fwd_noalloc(None if prob is None else ctypes.byref(prob), c(p["q"]), c(p["k"]),
                               c(p["v"]), c(p["g"]), c(p["h0"]), c(p["seg"]), c(p["o"]), c(p["hT"]), None)


def test_noalloc_forward_host_checks(lib):
    """gla_fwd_noalloc: the forward's argument checks, and a problem whose forward
    workspace exceeds the fixed scratch rejected with GLA_E_SCRATCH before any
    device is touched (every pointer here is fake: nothing may run)."""
    assert lib.gla_fwd_noalloc_max_scratch() == 64 << 20
    assert call_fwd_noalloc(lib, None) == -1
    assert call_fwd_noalloc(lib, prob(), {"o": None}) == -1
    assert call_fwd_noalloc(lib, prob(), {"q": FAKE + 4}) == -5
    assert call_fwd_noalloc(lib, prob(d_k=96)) == -4
    # 64 heads x 16 pieces of 128 x 128 fp32 summaries and entry states: 128 MiB
    big = gb.make_problem(B=1, T=65536, H=64, H_qk=64, d_k=128, d_v=128, gate="vector",
                          dtype=torch.bfloat16, split=16)
    assert gb.workspace_size(big, False) > lib.gla_fwd_noalloc_max_scratch()
    assert call_fwd_noalloc(lib, big) == -9
    assert b"scratch" in lib.gla_status_str(-9)


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-device path")
def test_noalloc_without_gpu_reports_device_error(lib):
    assert call_fwd_noalloc(lib, prob(H_qk=4, d_v=128)) == -7


# ---- the short depthwise causal convolution (gla_conv_*): host-side validation
def conv_prob(**kw):
    d = dict(B=2, T=100, C=64, K=4, dtype=1)
    d.update(kw)
    return gb.ConvProblem(d["B"], d["T"], d["C"], d["K"], d["dtype"])


def call_conv_fwd(lib, p, ptrs=None):
    q = dict(x=FAKE, w=FAKE, bias=None, y=FAKE)
    q.update(ptrs or {})
    c = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.gla_conv_fwd(None if p is None else ctypes.byref(p), c(q["x"]), c(q["w"]),
                            c(q["bias"]), c(q["y"]), None)


def call_conv_bwd(lib, p, ptrs=None, ws_bytes=0):
    names = ["x", "w", "bias", "dy", "dx", "dw", "db", "ws"]
    q = {n: FAKE for n in names}
    q.update(bias=None, db=None, ws=None)
    q.update(ptrs or {})
    c = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.gla_conv_bwd(ctypes.byref(p), *[c(q[n]) for n in names], ws_bytes, None)


def test_conv_argument_errors(lib):
    assert call_conv_fwd(lib, None) == -1
    assert call_conv_fwd(lib, conv_prob(), {"x": None}) == -1
    assert call_conv_bwd(lib, conv_prob(), {"dw": None}) == -1
    assert call_conv_fwd(lib, conv_prob(B=0)) == -2
    assert call_conv_fwd(lib, conv_prob(T=-1)) == -2
    assert call_conv_fwd(lib, conv_prob(K=3)) == -4
    assert call_conv_fwd(lib, conv_prob(C=12)) == -4
    assert call_conv_fwd(lib, conv_prob(dtype=5)) == -3
    assert call_conv_fwd(lib, conv_prob(), {"y": FAKE + 4}) == -5
    assert call_conv_bwd(lib, conv_prob(), {"db": FAKE + 8}) == -5


def test_conv_workspace(lib):
    p = conv_prob(B=3, T=1000, C=64)
    n = ctypes.c_size_t()
    assert lib.gla_conv_workspace_size(ctypes.byref(p), ctypes.byref(n)) == 0
    # one partial [K + 1][C] fp32 per (batch row, 256 time steps)
    assert n.value == 3 * 4 * 5 * 64 * 4
    assert call_conv_bwd(lib, p, {"ws": None}, ws_bytes=n.value) == -6
    assert call_conv_bwd(lib, p, {"ws": FAKE}, ws_bytes=n.value - 1) == -6
    assert lib.gla_conv_workspace_size(ctypes.byref(p), None) == -1


# ---- the output norm and gate (gla_norm_gate_*): host-side validation
def norm_prob(**kw):
    d = dict(B=2, T=100, H=4, d=128, eps=1e-5, dtype=1)
    d.update(kw)
    return gb.NormGateProblem(d["B"], d["T"], d["H"], d["d"], d["eps"], d["dtype"])


def call_norm_fwd(lib, p, ptrs=None):
    q = dict(o=FAKE, z=FAKE, gamma=FAKE, y=FAKE)
    q.update(ptrs or {})
    c = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.gla_norm_gate_fwd(None if p is None else ctypes.byref(p), c(q["o"]), c(q["z"]),
                                 c(q["gamma"]), c(q["y"]), None)


def call_norm_bwd(lib, p, ptrs=None, ws_bytes=0):
    names = ["o", "z", "gamma", "dy", "d_o", "dz", "dgamma", "ws"]
    q = {n: FAKE for n in names}
    q.update(ws=None)
    q.update(ptrs or {})
    c = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.gla_norm_gate_bwd(ctypes.byref(p), *[c(q[n]) for n in names], ws_bytes, None)


def test_norm_gate_argument_errors(lib):
    assert call_norm_fwd(lib, None) == -1
    assert call_norm_fwd(lib, norm_prob(), {"z": None}) == -1
    assert call_norm_bwd(lib, norm_prob(), {"dgamma": None}) == -1
    assert call_norm_fwd(lib, norm_prob(B=0)) == -2
    assert call_norm_fwd(lib, norm_prob(T=-1)) == -2
    assert call_norm_fwd(lib, norm_prob(eps=-1.0)) == -2
    assert call_norm_fwd(lib, norm_prob(eps=float("nan"))) == -2
    assert call_norm_fwd(lib, norm_prob(eps=float("inf"))) == -2
    assert call_norm_fwd(lib, norm_prob(d=96)) == -4
    assert call_norm_fwd(lib, norm_prob(dtype=3)) == -3
    assert call_norm_fwd(lib, norm_prob(), {"o": FAKE + 8}) == -5
    assert call_norm_bwd(lib, norm_prob(), {"dz": FAKE + 4}) == -5


def test_norm_gate_workspace(lib):
    n = ctypes.c_size_t()
    assert lib.gla_norm_gate_workspace_size(ctypes.byref(norm_prob()), ctypes.byref(n)) == 0
    assert n.value > 0 and n.value % (128 * 4) == 0
    assert call_norm_bwd(lib, norm_prob(), ws_bytes=n.value) == -6
    assert call_norm_bwd(lib, norm_prob(), {"ws": FAKE}, ws_bytes=n.value - 1) == -6
    assert lib.gla_norm_gate_workspace_size(ctypes.byref(norm_prob(T=0)), ctypes.byref(n)) == 0
    assert n.value == 0
    # at most 768 partials of d floats, however many rows
    assert lib.gla_norm_gate_workspace_size(ctypes.byref(norm_prob(B=64, T=65536, H=64)), ctypes.byref(n)) == 0
    assert n.value == 768 * 128 * 4


# ---- the gated delta rule (gla_delta_*): host-side validation
def delta_prob(**kw):
    d = dict(B=2, T=100, H=4, d_k=128, d_v=64, dtype=1)
    d.update(kw)
    return gb.DeltaProblem(d["B"], d["T"], d["H"], d["d_k"], d["d_v"], d["dtype"], 0, 0)


def call_delta_fwd(lib, p, ptrs=None, ws_bytes=0):
    names = ["q", "k", "v", "g", "beta", "h0", "seg", "o", "hT", "ws"]
    q = {n: FAKE for n in names}
    q.update(h0=None, seg=None, hT=None, ws=None)
    q.update(ptrs or {})
    c = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.gla_delta_fwd(None if p is None else ctypes.byref(p), *[c(q[n]) for n in names], ws_bytes, None)


def call_delta_bwd(lib, p, ptrs=None, ws_bytes=0, scratch_bytes=0):
    names = ["q", "k", "v", "g", "beta", "h0", "seg", "dO", "dhT", "dq", "dk", "dv", "dg", "dbeta", "dh0", "ws"]
    q = {n: FAKE for n in names}
    q.update(h0=None, seg=None, dhT=None, dh0=None, ws=None, scratch=None)
    q.update(ptrs or {})
    c = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.gla_delta_bwd(ctypes.byref(p), *[c(q[n]) for n in names], ws_bytes, c(q["scratch"]),
                             scratch_bytes, None)


def test_delta_argument_errors(lib):
    assert call_delta_fwd(lib, None) == -1
    assert call_delta_fwd(lib, delta_prob(), {"beta": None}) == -1
    assert call_delta_bwd(lib, delta_prob(), {"dbeta": None}) == -1
    assert call_delta_fwd(lib, delta_prob(B=0)) == -2
    assert call_delta_bwd(lib, delta_prob(T=-1)) == -2
    assert call_delta_fwd(lib, delta_prob(d_k=96)) == -4
    assert call_delta_bwd(lib, delta_prob(d_v=32)) == -4
    assert call_delta_fwd(lib, delta_prob(dtype=5)) == -3
    unknown_flag = delta_prob()
    unknown_flag.flags = 2  # only GLA_DELTA_WS_FROM_FWD (1) is defined
    assert call_delta_fwd(lib, unknown_flag) == -4
    assert call_delta_bwd(lib, unknown_flag) == -4
    assert call_delta_fwd(lib, delta_prob(), {"g": FAKE + 4}) == -5
    assert call_delta_bwd(lib, delta_prob(), {"dh0": FAKE + 8}) == -5


def delta_sizes(lib, p):
    n, m = ctypes.c_size_t(), ctypes.c_size_t()
    assert lib.gla_delta_workspace_size(ctypes.byref(p), 0, ctypes.byref(n)) == 0
    assert lib.gla_delta_workspace_size(ctypes.byref(p), 1, ctypes.byref(m)) == 0
    return n.value, m.value


def test_delta_workspace(lib):
    """ws: a 256-byte stamp and the forward's per-chunk factors (T, P: 64 x 64;
    U: 64 x d_v; W, gamma Q, decayed K: 64 x d_k; the carry: 4 floats); the
    backward's scratch: 2 d_k x d_v + 64 (2 d_v + 3 d_k) floats per chunk."""
    p = delta_prob()  # 2 chunks x 8 heads, d_k 128, d_v 64
    n, m = delta_sizes(lib, p)
    per_f = 2 * 64 * 64 + 64 * (64 + 3 * 128) + 4
    per_b = 2 * 128 * 64 + 64 * (2 * 64 + 3 * 128)
    assert n == 256 + 2 * 8 * per_f * 4 and m == 2 * 8 * per_b * 4
    assert call_delta_fwd(lib, p, ws_bytes=n) == -6                       # ws NULL
    assert call_delta_fwd(lib, p, {"ws": FAKE}, ws_bytes=n - 1) == -6
    assert call_delta_bwd(lib, p, {"ws": FAKE}, ws_bytes=n - 1, scratch_bytes=m) == -6
    assert call_delta_bwd(lib, p, {"ws": FAKE}, ws_bytes=n, scratch_bytes=m) == -6   # scratch NULL
    assert call_delta_bwd(lib, p, {"ws": FAKE, "scratch": FAKE}, ws_bytes=n, scratch_bytes=m - 1) == -6
    assert call_delta_bwd(lib, p, {"ws": FAKE, "scratch": FAKE + 8}, ws_bytes=n, scratch_bytes=m) == -5
    n2, m2 = delta_sizes(lib, delta_prob(T=200))
    assert n2 - 256 == 2 * (n - 256) and m2 == 2 * m  # 4 chunks against 2
    # GLA_DELTA_WS_FROM_FWD: the state entering each chunk (d_k x d_v) and the
    # effective writes (64 x d_v) move from the scratch into ws
    f = delta_prob()
    f.flags = 1
    nf, mf = delta_sizes(lib, f)
    moved = 128 * 64 + 64 * 64
    assert nf == n + 2 * 8 * moved * 4 and mf == m - 2 * 8 * moved * 4
