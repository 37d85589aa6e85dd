"""Host-side parts of bench.py (no GPU): the one-GPU rule, and the algorithmic
bytes per call that the roofline's `traffic` ratio divides by, checked against
figures worked out by hand (the V=128256 t=8 shard's CE statistics read
525.34 MB of fp32 logits, which the LM head writes)."""
import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def bench_module():
    spec = importlib.util.spec_from_file_location("bench_host", os.path.join(ROOT, "bench.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stdout + r.stderr


def test_algorithmic_bytes_of_every_row():
    b = bench_module()
    for row in b.ROW_NAMES:
        assert b.alg_bytes(row) > 0, row
    s5, Vs, h5 = 8192, 128256 // 8, 8192
    # CE statistics: the fp32 logits once, targets in, three fp32 scalars out per position
    assert b.alg_bytes("vocab_ce") == 4.0 * s5 * Vs + 20.0 * s5
    assert abs(4.0 * s5 * Vs - 525.34e6) < 0.01e6
    # LM head: H and the weight shard read once (bf16), fp32 logits written once
    assert b.alg_bytes("lm_head_fwd") == 2.0 * (s5 * h5 + h5 * Vs) + 4.0 * s5 * Vs
    # the fused LM head + CE drops the logits' write and read
    assert b.alg_bytes("lm_head_ce_fused") < b.alg_bytes("lm_head_fwd") - 4.0 * s5 * Vs + 1e6
    # GPT-3-175B t=8 MLP forward: X, W1, W2 read; Z, H, Y written (bf16)
    s, h, ft = 2048, 12288, 6144
    assert b.alg_bytes("mlp_fwd_gpt3") == 2.0 * (s * h + 2 * h * ft + 2 * s * ft + s * h)
