"""Host logic of bench.py (CPU only): the one-GPU guard, the traffic lookup tied to
the kernel source, and the FLOP counts of the workload configurations."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402


def _run(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, capture_output=True,
                          text=True, env=env, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = _run(["--gpus", "2"])
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_world_size_above_one_is_refused():
    r = _run([], {"WORLD_SIZE": "4"})
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_traffic_lookup_follows_the_kernel_source(tmp_path, monkeypatch):
    good = bench.kernel_source_hash()
    f = tmp_path / "traffic.md"
    f.write_text("| kind | a | b |\n|---|---|---|\n"
                 "| `gemm_fwd_NT_128x128_bf16` | 12 | 3.0002e+08 |\n\n"
                 "kernel source sha256: %s (gemm.hip, then common.h)\n" % good)
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic("gemm_fwd_NT_128x128_bf16") == 3.0002e8
    assert bench.measured_traffic("gemm_dgrad_NT_128x128_bf16") is None      # no row
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 64)      # kernel changed
    assert bench.measured_traffic("gemm_fwd_NT_128x128_bf16") is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.md"))
    assert bench.measured_traffic("gemm_fwd_NT_128x128_bf16") is None


def test_committed_traffic_matches_committed_kernels():
    """The committed profile was taken on the committed GEMM source (else the bench reports null)."""
    for kind in ("gemm_fwd_NT_128x128_bf16", "gemm_dgrad_NT_128x128_bf16", "gemm_wgrad_NT_1x128_f32"):
        assert bench.measured_traffic(kind) is not None, kind


def test_kernel_hash_covers_gemm_and_common():
    names = [os.path.basename(p) for p in bench.KERNEL_SOURCES]
    assert names == ["gemm.hip", "common.h"]


def test_workload_flop_counts():
    T = synth.TOKENS
    fwd = sum(2.0 * T * n * k for _, n, k in synth.FUSED_GEMMS)
    assert round(fwd / 1e9, 1) == 824.6                 # layer forward
    assert round(2 * fwd / 1e9, 1) == 1649.3             # layer backward
    step = 3 * sum(2.0 * T * n * k for _, n, k, _ in synth.LAYER_GEMMS) * synth.LAYERS
    assert round(step / 1e12, 2) == 69.27                # 28-layer stack, three passes
    assert abs(3 * 2.0 * 16384 * 2048 * 6144 / 1e9 - 1236.95) < 0.01   # outlier stress
