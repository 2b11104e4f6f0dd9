"""The Python binding fails loudly instead of computing anywhere but in the
HIP library: host tensors are refused before any library call, and a missing
library raises ImportError on first use.  No GPU needed (no call here
reaches a kernel)."""

import os
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import expert_ffn_layer_softmax_amd as moe  # noqa: E402


def _host_inputs(T=4, d=64, E=8, k=2, f=64):
    x = torch.zeros(T, d, dtype=torch.bfloat16)
    w = dict(w_gate=torch.zeros(E, f, d, dtype=torch.bfloat16), w_up=torch.zeros(E, f, d, dtype=torch.bfloat16),
             w_down=torch.zeros(E, d, f, dtype=torch.bfloat16))
    logits = torch.zeros(T, E, dtype=torch.float32)
    return x, w, logits, k


def _refuses(call):
    with pytest.raises(ValueError, match="no CPU path"):
        call()


def test_every_entry_point_refuses_host_tensors():
    x, w, logits, k = _host_inputs()
    idx = torch.zeros(4, k, dtype=torch.int32)
    tw = torch.zeros(4, k, dtype=torch.float32)
    _refuses(lambda: moe.moe_route(logits, k))
    _refuses(lambda: moe.moe_permute(idx, 8))
    _refuses(lambda: moe.moe_layer_forward(x, w, k, logits=logits))
    _refuses(lambda: moe.moe_layer_forward_noalloc(x, w, k, logits=logits))
    _refuses(lambda: moe.moe_quantize_mxfp8(torch.zeros(4, 64, dtype=torch.bfloat16)))
    offsets = torch.zeros(9, dtype=torch.int32)
    sorted_src = torch.zeros(8, dtype=torch.int32)
    _refuses(lambda: moe.moe_expert_ffn(x, offsets, sorted_src, k, w))
    _refuses(lambda: moe.moe_combine(torch.zeros(8, 64), sorted_src, tw, torch.bfloat16))


def test_missing_library_raises_import_error(tmp_path):
    """With the library absent the first use raises ImportError (the package
    itself still imports, so that the build command can run from a fresh
    checkout)."""
    missing = str(tmp_path / "libmoe_mi355x.so")
    code = ("import expert_ffn_layer_softmax_amd as m\n"
            "try:\n"
            "    m.load()\n"
            "except ImportError as e:\n"
            "    print('IMPORT_ERROR', e)\n"
            "else:\n"
            "    print('LOADED')\n")
    env = dict(os.environ, MOE_MI355X_LIB=missing)
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    assert "IMPORT_ERROR" in r.stdout and "LOADED" not in r.stdout
