"""Host-side logic of bench.py (no GPU): the workload accounting the
benchmark reports against, and the token shard that `--shard P` times."""
import pytest

import bench
from video_audio_diffusion_amd import inputs

C3 = inputs.CONFIGS[3]


@pytest.mark.parametrize("P", [1, 2, 4, 7, 8])
def test_shard_covers_its_share(P):
    s = bench.shard_config(C3, P)
    assert s.n_tok == -(-C3.n_tok // P)
    assert (s.dim, s.heads, s.head_dim, s.ffn) == (C3.dim, C3.heads, C3.head_dim, C3.ffn)
    starts = [seg.start for seg in s.segments]
    assert starts[0] == 0 and all(a.start + a.length == b.start for a, b in zip(s.segments, s.segments[1:]))
    assert sum(seg.length for seg in s.segments) == s.n_tok
    assert s.segments[0].kind == "text" and s.segments[0].length == C3.segments[0].length


def test_step_flops_match_the_workload():
    """Per-token work at the 15 s 768p shape: the projections' 2·(5376·21504
    + 7168·5376 + 5376·28672 + 14336·5376) flops and attention's 4·N·7168."""
    f = bench.step_flops(C3)
    N = C3.n_tok
    gemm = f["gemm_qkv"] + f["gemm_o"] + f["gemm_gu"] + f["gemm_d"]
    assert gemm / N == 2 * (5376 * 21504 + 7168 * 5376 + 5376 * 28672 + 14336 * 5376)
    assert f["attention"] == 4 * N * N * 56 * 128
    assert f["gemm_o_gate"] == f["gemm_o"] and f["gemm_gu_swiglu"] == f["gemm_gu"]
    assert f["gemm_qkv_rope"] == f["gemm_qkv"]


def test_step_bytes_of_the_streaming_passes():
    b = bench.step_bytes(C3)
    N, D, I, F = C3.n_tok, C3.dim, C3.inner, C3.ffn
    assert b["adaln_attn"] == 2 * N * D * 2 and b["qknorm_rope"] == 4 * N * I * 2
    assert b["swiglu"] == 3 * N * F * 2 and b["gate_ffn"] == 3 * N * D * 2


def test_traffic_is_dropped_when_the_sources_change(tmp_path, monkeypatch):
    """Counter bytes are reported only for the kernel sources they were taken on."""
    import json
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "traffic.json").write_text(json.dumps({"source_hash": "not-the-current-hash",
                                                   "kernels": {"attention": {"bytes_per_launch": 1.0}}}))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "current")
    assert bench.measured_traffic("attention") is None
    (prof / "traffic.json").write_text(json.dumps({"source_hash": "current",
                                                   "kernels": {"attention": {"bytes_per_launch": 1.0}}}))
    assert bench.measured_traffic("attention") == 1.0
