"""Host logic of bench.py, on the CPU: the one-GPU refusal, the algorithmic
flop and byte counts the roofline divides by, and the rule that a committed
HBM-traffic summary counts only for the kernel source it was taken on."""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from jagged_hstu_attention_attn_amd.inputs import make_inputs  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""   # no JSON line for a run that did not happen


def test_algorithmic_counts_tiny_workload():
    """Lengths [10, 100, 1000], causal only: the valid pairs are the
    triangular numbers L (L + 1) / 2; one head, d = 8, fp32, a 1024-entry
    position table and no time bias."""
    inp = make_inputs("tiny", seed=0)
    pairs = sum(L * (L + 1) // 2 for L in (10, 100, 1000))
    flops, byts = bench.algorithmic(inp, pairs)
    assert flops == 2.0 * (8 + 8) * 1 * pairs
    n = 1110
    want = n * 1 * (2 * 8 + 3 * 8) * 4      # q, k read; v, u read; out written (fp32)
    want += 4 * (3 + 1)                     # offsets
    want += 4 * 1024                        # position table
    assert inp.timestamps is None and inp.time_table is None and inp.num_targets is None
    assert byts == want


def test_algorithmic_counts_scale_with_heads_and_dtype():
    inp = make_inputs("ranking", seed=1234)
    f1, b1 = bench.algorithmic(inp, 1000)
    assert f1 == 2.0 * (inp.d_qk + inp.d_v) * inp.num_heads * 1000
    N, H = inp.total_tokens, inp.num_heads
    tensors = N * H * (2 * inp.d_qk + 3 * inp.d_v) * 2          # bf16
    meta = 8 * N + 4 * (inp.num_seqs + 1) + 4 * inp.num_seqs     # timestamps, offsets, targets
    tables = 4 * (inp.pos_table.shape[0] + inp.time_table.shape[0])
    assert b1 == tensors + meta + tables


def _write_summary(root, workload, kernel, sha, nbytes):
    os.makedirs(os.path.join(root, "profiles"), exist_ok=True)
    with open(os.path.join(root, "profiles", f"attn_fwd_{workload}_traffic.md"), "w") as f:
        f.write(f"# summary\n\nkernel: {kernel}\nkernel_source_sha: {sha}\n"
                f"hbm_bytes_per_launch: {nbytes}\n")


def test_traffic_summary_counts_only_for_its_kernel_source(tmp_path, monkeypatch):
    k = "hstu_attn_fwd_w16_kernel"
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda kernel: "0123abcd")
    assert bench.traffic_from_profile("windowed", k) is None          # no summary
    _write_summary(str(tmp_path), "windowed", k, "0123abcd", "5.5e+08")
    assert bench.traffic_from_profile("windowed", k) == pytest.approx(5.5e8)
    assert bench.traffic_from_profile("windowed", "hstu_attn_fwd_kernel") is None   # other kernel
    _write_summary(str(tmp_path), "windowed", k, "ffff0000", "5.5e+08")
    assert bench.traffic_from_profile("windowed", k) is None          # source changed since


def test_kernel_source_hash_follows_the_sources():
    h = bench.kernel_source_hash("hstu_attn_fwd_w16_kernel")
    assert len(h) == 16 and int(h, 16) >= 0
    assert h == bench.kernel_source_hash("hstu_attn_fwd_w16_kernel")
    assert h != bench.kernel_source_hash("hstu_attn_fwd_kernel")
    for kernel, files in bench.KERNEL_SOURCES.items():
        for rel in files:
            assert os.path.exists(os.path.join(ROOT, bench._CSRC + rel)), (kernel, rel)
