"""The planner's choices for the benchmarked shards, read from its plan log
(TP_PLAN_LOG=1) on a host with no GPU: the calls validate their arguments and
plan every launch before enqueueing anything, then fail at the first launch.
Runs only where no GPU is visible (the placeholder device addresses would
otherwise reach a kernel)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SCRIPT = r"""
import sys
sys.path.insert(0, {root!r})
from megatron_tensor_layer_tp_amd import tpshard as T
L = T.lib()
A = 1 << 20                      # a placeholder address, 16-byte aligned, never dereferenced
BF = T.TP_DT_BF16
s, h, ft = {s}, {h}, {ft}
nb = T.tp_mlp_bwd_workspace(BF, s, h, ft)
st = L.tp_mlp_bwd(T.TP_ACT_GELU, BF, s, h, ft, *([A] * 9), A, nb, None)
print("status", st)
"""


def no_gpu():
    try:
        import torch
        return torch.cuda.device_count() == 0
    except Exception:
        return True


def plan_lines(s, h, ft):
    env = dict(os.environ, TP_PLAN_LOG="1")
    env.pop("TP_GEMM_PAIR", None)
    env.pop("TP_GEMM_VARIANT", None)
    r = subprocess.run([sys.executable, "-c", SCRIPT.format(root=ROOT, s=s, h=h, ft=ft)], capture_output=True,
                       text=True, timeout=120, env=env)
    return [l for l in (r.stdout + r.stderr).splitlines() if l.startswith("[tp plan]")]


@pytest.mark.skipif(not no_gpu(), reason="placeholder addresses must not reach a real GPU")
def test_gpt3_mlp_backward_pairs_activation_gradient_first():
    # s = 2048 tokens against h = 12288: the weight gradients' K is the short one, so the
    # first pass pairs dZ (first) with dW2 (second), both as 256x256 8-wave tiles
    lines = plan_lines(2048, 12288, 6144)
    dz = [l for l in lines if "dZ GEMM" in l]
    dw2 = [l for l in lines if "dW2 GEMM" in l]
    assert dz and dw2, lines
    assert "(paired, first)" in dz[0] and "(paired, second)" in dw2[0], lines
    assert "256x256:waves8" in dz[0] and "256x256:waves8" in dw2[0], lines


@pytest.mark.skipif(not no_gpu(), reason="placeholder addresses must not reach a real GPU")
def test_gpt2_mlp_backward_keeps_weight_gradient_first():
    # s = 8192 tokens against h = 768: the weight gradients have the long K and go first, split
    lines = plan_lines(8192, 768, 1536)
    dw2 = [l for l in lines if "dW2 GEMM" in l]
    assert dw2 and "(paired, first)" in dw2[0] and "splits=1" not in dw2[0], lines
