"""Seeded synthetic inputs for the gated linear-attention path.

This module holds no arithmetic of the method: it only draws random tensors
with the shapes and distributions of the workloads and casts them to the
storage dtype.  Both the HIP path and the CPU oracle take their inputs from
here; neither imports the other.

Recipe (every workload): a ``torch.Generator`` seeded with the workload's seed
draws, on the CPU in float32 and in this order, q, k, v, g, h0, dO, dhT (a
tensor that the workload does not use is not drawn).  Then every tensor except
the fp32 states (h0, dhT) is cast to the storage dtype with round-to-nearest-
even.  Document lengths for packed rows come from ``numpy.random.default_rng``
with the same seed: integers drawn uniformly from the inclusive range until
they cover T, the last one truncated to fit.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch


@dataclasses.dataclass
class Case:
    name: str
    gate: str                     # "scalar" or "vector"
    dtype: torch.dtype            # storage dtype of q, k, v, g, o and the gradients
    q: torch.Tensor               # [B, T, H_qk, d_k]
    k: torch.Tensor               # [B, T, H_qk, d_k]
    v: torch.Tensor               # [B, T, H, d_v]
    g: torch.Tensor               # [B, T, H] or [B, T, H, d_k], natural-log gate
    dO: torch.Tensor              # [B, T, H, d_v]
    h0: Optional[torch.Tensor] = None          # [B, H, d_k, d_v] fp32
    dhT: Optional[torch.Tensor] = None         # [B, H, d_k, d_v] fp32
    segment_ids: Optional[torch.Tensor] = None  # [B, T] int32
    chunk: int = 64
    doc_lengths: Optional[list] = None

    @property
    def B(self): return self.q.shape[0]
    @property
    def T(self): return self.q.shape[1]
    @property
    def H_qk(self): return self.q.shape[2]
    @property
    def d_k(self): return self.q.shape[3]
    @property
    def H(self): return self.v.shape[2]
    @property
    def d_v(self): return self.v.shape[3]

    def tensors(self):
        return dict(q=self.q, k=self.k, v=self.v, g=self.g, dO=self.dO, h0=self.h0,
                    dhT=self.dhT, segment_ids=self.segment_ids)

    def to(self, device):
        kw = {}
        for f in ("q", "k", "v", "g", "dO", "h0", "dhT", "segment_ids"):
            x = getattr(self, f)
            kw[f] = None if x is None else x.to(device)
        return dataclasses.replace(self, **kw)


def doc_lengths(T: int, lo: int, hi: int, seed: int):
    """Document lengths drawn from U[lo, hi] (inclusive) until they cover T."""
    rng = np.random.default_rng(seed)
    out, tot = [], 0
    while tot < T:
        n = int(rng.integers(lo, hi + 1))
        n = min(n, T - tot)
        out.append(n)
        tot += n
    return out


def segment_ids_from_lengths(lengths, T: int) -> torch.Tensor:
    ids = np.concatenate([np.full(n, i, dtype=np.int32) for i, n in enumerate(lengths)])
    assert ids.shape[0] == T
    return torch.from_numpy(ids)


def _gate(gen, shape, kind: str):
    x = torch.randn(shape, generator=gen)
    if kind == "ssd_mild":       # -0.1 * softplus(N(0,1))
        return -0.1 * torch.nn.functional.softplus(x)
    if kind == "ssd_mamba":      # -exp(U(-4,0)) * softplus(N(0,1)); U drawn after N
        u = torch.rand(shape, generator=gen) * 4.0 - 4.0
        return -torch.exp(u) * torch.nn.functional.softplus(x)
    if kind == "gla":            # logsigmoid(N(0,1)) / 16
        return torch.nn.functional.logsigmoid(x) / 16.0
    # Strong decays (scaled by gate_mult): every channel -1; channels alternating
    # between -1 and -1/800 (so that x8 gives -8 and -0.01); each element -1 or
    # -1/800 at random; -1 in the first half of the sequence and the GLA
    # distribution in the second, so strong and ordinary chunks alternate in a row.
    if kind == "unit":
        return -torch.ones(shape)
    if kind == "mix_channels":
        alt = (torch.arange(shape[-1]) % 2 == 0).to(torch.float32)
        return -(alt + (1.0 - alt) / 800.0).expand(shape).clone()
    if kind == "mix_random":
        pick = (torch.rand(shape, generator=gen) < 0.5).to(torch.float32)
        return -(pick + (1.0 - pick) / 800.0)
    if kind == "half_unit":
        g = torch.nn.functional.logsigmoid(x) / 16.0
        g[:, : shape[1] // 2] = -1.0
        return g
    raise ValueError(kind)


def make_case(name, *, B, T, H, H_qk, d_k, d_v, gate, dtype, seed, gate_kind,
              qk_scale=None, with_h0=False, with_dhT=False, lengths=None,
              chunk=64, gate_mult=1.0) -> Case:
    gen = torch.Generator().manual_seed(seed)
    s = (1.0 / math.sqrt(d_k)) if qk_scale is None else qk_scale
    q = torch.randn((B, T, H_qk, d_k), generator=gen) * s
    k = torch.randn((B, T, H_qk, d_k), generator=gen) * s
    v = torch.randn((B, T, H, d_v), generator=gen)
    gshape = (B, T, H, d_k) if gate == "vector" else (B, T, H)
    g = _gate(gen, gshape, gate_kind) * gate_mult
    h0 = torch.randn((B, H, d_k, d_v), generator=gen) * 0.1 if with_h0 else None
    dO = torch.randn((B, T, H, d_v), generator=gen)
    dhT = torch.randn((B, H, d_k, d_v), generator=gen) if with_dhT else None
    seg = None
    if lengths is not None:
        seg = segment_ids_from_lengths(lengths, T).reshape(1, T).repeat(B, 1).contiguous()
    cast = lambda x: x.to(dtype).contiguous()
    return Case(name=name, gate=gate, dtype=dtype, q=cast(q), k=cast(k), v=cast(v),
                g=cast(g), dO=cast(dO), h0=h0, dhT=dhT, segment_ids=seg, chunk=chunk,
                doc_lengths=lengths)


# The five workloads (c5 has two layouts of the same 16,384 tokens per step).
WORKLOADS = {
    "c1": "SSD scalar gate, fp32, B=1 H=2 T=256 d=64, chunk 64",
    "c2": "SSD scalar gate, fp32, B=4 T=8192 H=8 (2 q/k groups of 4) d=128, chunk 64",
    "c3": "GLA vector gate, bf16, B=4 T=4096 H=16 d=128, chunk 64, h0 and dhT",
    "c4": "SSD scalar gate, bf16, packed documents, B=1 T=65536 H=16 d=128, chunk 64, h0",
    "c5a": "GLA vector gate, bf16, B=1 T=16384 H=16 d=128, chunk 64, h0 and dhT",
    "c5b": "GLA vector gate, bf16, B=8 T=2048 H=16 d=128, chunk 64, h0 and dhT",
}


def workload(name: str) -> Case:
    if name == "c1":
        return make_case(name, B=1, T=256, H=2, H_qk=2, d_k=64, d_v=64, gate="scalar",
                         dtype=torch.float32, seed=1, gate_kind="ssd_mild")
    if name == "c2":
        return make_case(name, B=4, T=8192, H=8, H_qk=2, d_k=128, d_v=128, gate="scalar",
                         dtype=torch.float32, seed=2, gate_kind="ssd_mamba")
    if name == "c3":
        return make_case(name, B=4, T=4096, H=16, H_qk=16, d_k=128, d_v=128, gate="vector",
                         dtype=torch.bfloat16, seed=3, gate_kind="gla", with_h0=True,
                         with_dhT=True)
    if name == "c4":
        T = 65536
        lens = doc_lengths(T, 512, 8192, seed=4)
        return make_case(name, B=1, T=T, H=16, H_qk=16, d_k=128, d_v=128, gate="scalar",
                         dtype=torch.bfloat16, seed=4, gate_kind="ssd_mamba", with_h0=True,
                         lengths=lens)
    if name == "c5a":
        return make_case(name, B=1, T=16384, H=16, H_qk=16, d_k=128, d_v=128, gate="vector",
                         dtype=torch.bfloat16, seed=5, gate_kind="gla", with_h0=True,
                         with_dhT=True)
    if name == "c5b":
        return make_case(name, B=8, T=2048, H=16, H_qk=16, d_k=128, d_v=128, gate="vector",
                         dtype=torch.bfloat16, seed=5, gate_kind="gla", with_h0=True,
                         with_dhT=True)
    raise KeyError(name)


def small_case(seed=0, *, B=1, T=100, H=2, H_qk=None, d=64, d_v=None, gate="scalar",
               dtype=torch.float32, with_h0=True, with_dhT=True, lengths=None,
               gate_kind=None, gate_mult=1.0) -> Case:
    """A small case for parity sweeps (same distributions as the workloads)."""
    H_qk = H if H_qk is None else H_qk
    d_v = d if d_v is None else d_v
    gk = gate_kind or ("gla" if gate == "vector" else "ssd_mamba")
    return make_case("small", B=B, T=T, H=H, H_qk=H_qk, d_k=d, d_v=d_v, gate=gate,
                     dtype=dtype, seed=seed, gate_kind=gk, with_h0=with_h0,
                     with_dhT=with_dhT, lengths=lengths, gate_mult=gate_mult)


# ---- the short depthwise causal convolution
@dataclasses.dataclass
class ConvCase:
    name: str
    dtype: torch.dtype
    x: torch.Tensor      # [B, T, C], storage dtype
    w: torch.Tensor      # [K, C] fp32
    bias: Optional[torch.Tensor]  # [C] fp32
    dy: torch.Tensor     # [B, T, C], storage dtype

    def to(self, device):
        return dataclasses.replace(self, x=self.x.to(device), w=self.w.to(device),
                                   bias=None if self.bias is None else self.bias.to(device),
                                   dy=self.dy.to(device))


def conv_case(name="conv", *, B, T, C, K=4, dtype=torch.bfloat16, seed=0, bias=True):
    """Seeded inputs for the convolution: a torch.Generator draws, on the CPU in
    float32 and in this order, x ~ N(0, 1), w ~ U(-1/sqrt(K), 1/sqrt(K)), bias ~ the
    same uniform, dy ~ N(0, 1) (the bound is PyTorch's default for a depthwise
    convolution, fan-in K); x and dy are then cast to the storage dtype."""
    gen = torch.Generator().manual_seed(seed)
    bound = 1.0 / math.sqrt(K)
    x = torch.randn(B, T, C, generator=gen)
    w = (torch.rand(K, C, generator=gen) * 2 - 1) * bound
    bb = (torch.rand(C, generator=gen) * 2 - 1) * bound if bias else None
    dy = torch.randn(B, T, C, generator=gen)
    return ConvCase(name, dtype, x.to(dtype), w, bb, dy.to(dtype))


def conv_workload():
    """The page's convolution benchmark shape: B=8, S=4096, 2048 channels, K=4,
    bias and SiLU, bf16 activations."""
    return conv_case("conv", B=8, T=4096, C=2048, K=4, dtype=torch.bfloat16, seed=11)


# ---- the output norm and gate
@dataclasses.dataclass
class NormGateCase:
    name: str
    dtype: torch.dtype
    o: torch.Tensor               # [B, T, H, d] recurrence output
    z: torch.Tensor               # [B, T, H, d] gate pre-activation
    gamma: torch.Tensor           # [d] fp32
    dy: torch.Tensor              # [B, T, H, d]
    eps: float = 1e-5

    def to(self, device):
        return dataclasses.replace(self, o=self.o.to(device), z=self.z.to(device),
                                   gamma=self.gamma.to(device), dy=self.dy.to(device))


def norm_gate_case(name="norm_gate", *, B, T, H, d=128, dtype=torch.bfloat16, seed=0, eps=1e-5):
    """o, z, dy ~ N(0, 1), gamma ~ U(0.5, 1.5); bf16 values are rounded once, when drawn."""
    gen = torch.Generator().manual_seed(seed)
    o = torch.randn((B, T, H, d), generator=gen).to(dtype)
    z = torch.randn((B, T, H, d), generator=gen).to(dtype)
    gamma = torch.rand(d, generator=gen) + 0.5
    dy = torch.randn((B, T, H, d), generator=gen).to(dtype)
    return NormGateCase(name, dtype, o, z, gamma, dy, eps)


def norm_gate_workload():
    """The layer shape of the FLAT page's benchmarks: B=8, T=4096, H=16, d=128, bf16."""
    return norm_gate_case("norm_gate", B=8, T=4096, H=16, d=128, dtype=torch.bfloat16, seed=13)


# ---- the gated delta rule
@dataclasses.dataclass
class DeltaCase:
    name: str
    dtype: torch.dtype
    q: torch.Tensor               # [B, T, H, d_k], unit norm per row
    k: torch.Tensor               # [B, T, H, d_k], unit norm per row
    v: torch.Tensor               # [B, T, H, d_v]
    g: torch.Tensor               # [B, T, H] natural-log gate
    beta: torch.Tensor            # [B, T, H] write strength in (0, 1)
    dO: torch.Tensor              # [B, T, H, d_v]
    h0: Optional[torch.Tensor] = None
    dhT: Optional[torch.Tensor] = None
    segment_ids: Optional[torch.Tensor] = None

    def to(self, device):
        mv = lambda x: None if x is None else x.to(device)
        return dataclasses.replace(self, q=mv(self.q), k=mv(self.k), v=mv(self.v), g=mv(self.g),
                                   beta=mv(self.beta), dO=mv(self.dO), h0=mv(self.h0), dhT=mv(self.dhT),
                                   segment_ids=mv(self.segment_ids))


def delta_case(name="delta", *, B, T, H, d_k=128, d_v=None, dtype=torch.bfloat16, seed=0,
               lengths=None, with_h0=True, with_dhT=True):
    """q, k: N(0, 1) rows scaled to unit L2 norm (the delta rule's keys are normalised
    in its layers); v, dO ~ N(0, 1); g = log sigmoid of N(3, 1) (gates near 0.95);
    beta = sigmoid of N(0, 1); h0 ~ 0.1 N(0, 1), dhT ~ N(0, 1).  bf16 values are
    rounded once, when drawn."""
    d_v = d_k if d_v is None else d_v
    gen = torch.Generator().manual_seed(seed)
    unit = lambda x: x / x.norm(dim=-1, keepdim=True)
    q = unit(torch.randn((B, T, H, d_k), generator=gen))
    k = unit(torch.randn((B, T, H, d_k), generator=gen))
    v = torch.randn((B, T, H, d_v), generator=gen)
    g = torch.nn.functional.logsigmoid(torch.randn((B, T, H), generator=gen) + 3.0)
    beta = torch.sigmoid(torch.randn((B, T, H), generator=gen))
    dO = torch.randn((B, T, H, d_v), generator=gen)
    h0 = torch.randn((B, H, d_k, d_v), generator=gen) * 0.1 if with_h0 else None
    dhT = torch.randn((B, H, d_k, d_v), generator=gen) if with_dhT else None
    seg = None
    if lengths is not None:
        seg = segment_ids_from_lengths(lengths, T).reshape(1, T).repeat(B, 1).contiguous()
    cast = lambda x: x.to(dtype).contiguous()
    return DeltaCase(name, dtype, cast(q), cast(k), cast(v), cast(g), cast(beta), cast(dO), h0, dhT, seg)


def delta_workload():
    """The pages' Gated DeltaNet benchmark layout: bf16, batch 4, 8 heads, chunk 64,
    d_k = d_v = 128, here at T = 4096."""
    return delta_case("delta", B=4, T=4096, H=8, d_k=128, dtype=torch.bfloat16, seed=17)
