"""bench.py's host logic, without a GPU: the refusal of more than one GPU, the
algorithmic bytes and FLOPs its rooflines divide by, the choice of the bound a
path faces, the roofline fields, the reading of committed profile summaries
(stale ones give no traffic), and the states note in its config."""
import os
import subprocess
import sys
import types

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def case(B, T, H, H_qk, d, gate, dtype, h0=True, dhT=True, seg=False):
    """The fields bench's helpers read (no tensors are allocated)."""
    return types.SimpleNamespace(B=B, T=T, H=H, H_qk=H_qk, d_k=d, d_v=d, chunk=64, gate=gate, dtype=dtype,
                                 h0=object() if h0 else None, dhT=object() if dhT else None,
                                 segment_ids=object() if seg else None)


C2 = case(4, 8192, 8, 2, 128, "scalar", torch.float32, h0=False, dhT=False)
C3 = case(4, 4096, 16, 16, 128, "vector", torch.bfloat16)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_algorithmic_bytes_per_token_head():
    """bf16 GLA, d = 128, q/k per head: the backward reads q, k, v, g, dO (5 x 256
    bytes per token-head) and writes dq, dk, dv, dg (4 x 256): 2,304 bytes, plus
    h0, dhT read and dh0 written (fp32 128 x 128 per head)."""
    alg = bench.algorithmic(C3)
    th = C3.B * C3.T * C3.H
    st = C3.B * C3.H * 128 * 128 * 4
    assert alg["bwd_bytes"] == 2304 * th + 3 * st
    # forward: q, k, v, g read, o written (1,280 per token-head), h0 read, hT written
    assert alg["fwd_bytes"] == 1280 * th + 2 * st
    # FLOPs: causal half of the chunk products plus the state terms, per token-head
    assert alg["bwd_flops"] == th * (4 * 64 * 128 + 8 * 128 * 128) == th * 163840
    assert alg["fwd_flops"] == th * 81920


def test_algorithmic_bytes_with_shared_qk():
    """fp32 SSD with four heads per q/k head: q, k (and dq, dk) count once per group."""
    alg = bench.algorithmic(C2)
    tq = C2.B * C2.T * C2.H_qk * 128 * 4
    tv = C2.B * C2.T * C2.H * 128 * 4
    tg = C2.B * C2.T * C2.H * 4
    assert alg["bwd_bytes"] == 2 * tq + tv + tg + tv + 2 * tq + tv + tg
    assert abs(alg["bwd_bytes"] / 1e6 - 539.0) < 0.5


def test_bound_is_the_one_the_path_faces():
    # split-bf16 fp32 (three bf16 products): HBM binds c2
    a2 = bench.algorithmic(C2)
    kind, t = bench.bound_time(C2, a2["bwd_bytes"], a2["bwd_flops"])
    assert kind == "hbm" and t == pytest.approx(a2["bwd_bytes"] / 8e12)
    assert 3 * a2["bwd_flops"] / 2.5e15 < t
    # bf16 GLA: HBM
    a3 = bench.algorithmic(C3)
    assert bench.bound_time(C3, a3["bwd_bytes"], a3["bwd_flops"])[0] == "hbm"
    # fp32 vector gate runs on the fp32 matrix cores: they bind
    c = case(4, 4096, 16, 16, 128, "vector", torch.float32)
    a = bench.algorithmic(c)
    kind, t = bench.bound_time(c, a["bwd_bytes"], a["bwd_flops"])
    assert kind == "mfma" and t == pytest.approx(a["bwd_flops"] / 157.3e12)


def test_roofline_fields():
    a2 = bench.algorithmic(C2)
    r = bench.gla_roofline(C2, 200.0, 650.0, copy_gbs=5000.0)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert r["achieved"] == pytest.approx(a2["bwd_bytes"] / 650e-6 / 1e9, rel=1e-3)
    assert r["frac"] == pytest.approx(r["achieved"] / r["peak"], rel=1e-3)
    assert r["copy_frac"] == pytest.approx(r["achieved"] / 5000.0, rel=1e-3)
    assert 0 < r["step_frac"] < 1
    assert r["fp32_mfma_frac"] == pytest.approx(a2["bwd_flops"] / 650e-6 / 157.3e12, rel=1e-3)
    assert "three bf16 products" in r["products"]
    assert "fp32_mfma_frac" not in bench.gla_roofline(C3, 170.0, 440.0)


def test_profile_summary_traffic_needs_matching_sources(tmp_path, monkeypatch):
    (tmp_path / "profiles").mkdir()
    (tmp_path / "ssm_recurrence_amd" / "csrc").mkdir(parents=True)
    (tmp_path / "ssm_recurrence_amd" / "csrc" / "k.hip").write_text("// kernel\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    f = tmp_path / "profiles" / bench.PROFILE["c3"]
    assert bench.measured_traffic("c3") is None  # no summary
    f.write_text("traffic_bytes_per_gla_bwd: 1234.5\nsource_hash: %s\n" % bench.source_hash())
    assert bench.measured_traffic("c3") == 1234.5
    (tmp_path / "ssm_recurrence_amd" / "csrc" / "k.hip").write_text("// kernel, changed\n")
    assert bench.measured_traffic("c3") is None  # stale: the sources changed since
    assert bench.measured_traffic("no_such_workload") is None


def test_committed_summaries_name_the_current_sources_or_none():
    """Every committed summary carries its sources' hash; bench reports traffic only
    while it matches (this checks the parsing of the real files, not a match)."""
    for w, name in bench.PROFILE.items():
        p = os.path.join(ROOT, "profiles", name)
        assert os.path.exists(p), name
        text = open(p).read()
        assert "source_hash:" in text and "rocprofv3" in text
        v = bench.measured_traffic(w, "traffic_bytes_per_gla_bwd" if w not in ("conv", "norm_gate", "delta")
                                   else "traffic_bytes_per_gla_%s_bwd" % w)
        assert v is None or v > 0


def test_states_note():
    c4 = case(1, 65536, 16, 16, 128, "scalar", torch.bfloat16, dhT=False, seg=True)
    assert "stored by the forward" in bench.states_note(c4, True)
    assert "stored by the forward" in bench.states_note(C2, True)
    assert "stores none" in bench.states_note(C3, True)
    assert "recomputed" in bench.states_note(c4, False)
