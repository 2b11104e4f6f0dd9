"""Host-side checks of bench.py: its byte accounting (the roofline's
algorithmic bytes) and its one-GPU contract.  No GPU needed."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from synth import WORKLOADS  # noqa: E402


def test_expert_bytes_match_the_format_definitions():
    # one expert = W_gate, W_up [f][d] and W_down [d][f] = 3*d*f weights
    d, f = 6144, 2816
    n = 3 * d * f
    assert bench._expert_bytes(WORKLOADS["decode_bf16"])["total"] == 2 * n == 103_809_024
    # MX-FP4: half a byte per weight plus one E8M0 byte per 32 weights
    assert bench._expert_bytes(WORKLOADS["decode_mxfp4"])["total"] == n // 2 + n // 32 == 27_574_272
    # NVFP4: half a byte per weight plus one E4M3 byte per 16 (the fp32 matrix
    # scales are 12 bytes per expert and left out)
    assert bench._expert_bytes(WORKLOADS["decode_nvfp4"])["total"] == n // 2 + n // 16
    eb = bench._expert_bytes(WORKLOADS["decode_bf16"])
    assert eb["gate_up"] == 2 * eb["down"]


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""
