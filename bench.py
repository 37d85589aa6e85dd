#!/usr/bin/env python3
"""Benchmark of the tensor-parallel shard path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--rows all|mlp] [--no-cpu-baseline]

A step is one pass over every step of the shard path on seeded synthetic
inputs already resident in HBM:
  * MLP shard forward + backward (column GEMM + GeLU, row GEMM, and the dZ /
    dW2 / dX / dW1 GEMMs) at the GPT-3-175B t=8 shard: s=2048, h=12288,
    f/t=6144 -- the workload the headline metric is quoted on -- and at the
    GPT-2-small t=2 shard (s=8*1024, h=768, f/t=1536);
  * SwiGLU shard and attention projections, forward + backward, at the
    Llama-3-70B t=8 shard (s=8192, h=8192, f/t=3584, dq=1024, dkv=128);
  * vocab shard at V=128256, t=8: LM-head GEMM (fp32 logits [8192,16032]),
    cross-entropy statistics on those logits, and the embedding gather of
    8192 ids from a [16032,8192] table.
Each library call is bracketed by HIP events on the stream it runs on.  One
JSON line is printed: the headline is the GPT-3-175B MLP shard's
forward+backward TFLOP/s; every row's time and throughput is listed under
"rows"; "roofline" covers the longest single-kernel call (the LM-head GEMM)
and "roofline_ce" the cross-entropy kernel; "cpu_baseline" times the fp64
oracle on a bounded sample of the headline workload, with "rows" beside it
for the other rows.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--rows", choices=["all", "mlp"], default="all")
    p.add_argument("--only", default=None,
                   help="time a single row (e.g. lm_head_fwd) -- for profiling runs")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="only run a 1 GiB device-to-device copy (HBM counter calibration)")
    p.add_argument("--counter-summary", default=None, metavar="DIR",
                   help="reduce the rocprofv3 counter passes under DIR (DIR/<row>/<fetch|write|sq>, DIR/copy/"
                        "<fetch|write>) to profiles/hbm_traffic.json and print a markdown table")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="target CPU time of the oracle sample")
    return p.parse_args()


def src_hash(*names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "megatron_tensor_layer_tp_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


class Row:
    """One library call of the step, with its algorithmic work per call."""

    def __init__(self, name, config, fn, flops=0.0, bytes_=0.0):
        self.name, self.config, self.fn = name, config, fn
        self.flops, self.bytes = flops, bytes_
        self.events = []

    def run(self, torch, record):
        if record:
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            self.fn()
            b.record()
            self.events.append((a, b))
        else:
            self.fn()

    def times(self):
        return sorted(a.elapsed_time(b) for a, b in self.events)

    def ms(self):
        return sum(a.elapsed_time(b) for a, b in self.events) / max(1, len(self.events))

    def pct(self, q):
        t = self.times()
        return t[min(len(t) - 1, int(q * (len(t) - 1) + 0.5))] if t else 0.0


class GpuSampler:
    """Best-effort shader clock, power and temperatures of the GPU during the
    timed steps, read (read-only) from the amdgpu sysfs files: the current
    level of pp_dpm_sclk and the hwmon power and temperature inputs.  Empty
    when the files are not there."""

    def __init__(self):
        import glob
        import threading
        self.files = {}
        for dev in sorted(glob.glob("/sys/class/drm/*/device")):
            if not os.path.exists(os.path.join(dev, "pp_dpm_sclk")):
                continue
            self.files["sclk_mhz"] = (os.path.join(dev, "pp_dpm_sclk"), None)
            for hw in sorted(glob.glob(os.path.join(dev, "hwmon", "hwmon*"))):
                if os.path.exists(os.path.join(hw, "power1_input")):
                    self.files["power_w"] = (os.path.join(hw, "power1_input"), 1e-6)
                for t in sorted(glob.glob(os.path.join(hw, "temp*_input"))):
                    lab = t.replace("_input", "_label")
                    name = open(lab).read().strip() if os.path.exists(lab) else os.path.basename(t)[:-6]
                    self.files[f"temp_{name}_c"] = (t, 1e-3)
            break
        self.samples = {k: [] for k in self.files}
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    @staticmethod
    def _read(f, scale):
        with open(f) as fh:
            txt = fh.read()
        if scale is not None:
            return float(txt) * scale
        for line in txt.splitlines():  # "1: 2100Mhz *" marks the current level
            if line.strip().endswith("*"):
                return float(line.split(":")[1].strip().split("M")[0])
        raise ValueError("no current level")

    def _run(self):
        while not self._stop.is_set():
            for k, (f, scale) in self.files.items():
                try:
                    self.samples[k].append(self._read(f, scale))
                except (OSError, ValueError, IndexError):
                    pass
            self._stop.wait(0.01)

    def __enter__(self):
        if self.files:
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self.files:
            self._thread.join()

    def summary(self):
        out = {}
        for k, v in self.samples.items():
            if v:
                out[k] = {"mean": round(sum(v) / len(v), 1), "max": round(max(v), 1), "n": len(v)}
        return out or None


def build_rows(torch, which, only=None):
    import numpy as np

    from megatron_tensor_layer_tp_amd import inputs as I
    from megatron_tensor_layer_tp_amd import tpshard as T

    dev = "cuda:0"

    def up(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(a).to(dev)

    def bf(shape):
        return torch.empty(shape, dtype=torch.int16, device=dev)

    BF = T.TP_DT_BF16
    rows = []

    def want(*names):
        return only is None or only in names

    # ---- MLP shard: GPT-3-175B t=8 (the headline workload) and GPT-2-small t=2
    if want("mlp_fwd_gpt3", "mlp_bwd_gpt3"):
        rows += mlp_rows(torch, up, bf, I, T, 3, "gpt3")
        progress(f"inputs: {rows[-1].config} ready")
    if want("mlp_fwd_gpt2", "mlp_bwd_gpt2"):
        rows += mlp_rows(torch, up, bf, I, T, 2, "gpt2")
        progress(f"inputs: {rows[-1].config} ready")
    if which == "mlp":
        return rows
    if want("swiglu_fwd", "swiglu_bwd", "attn_proj_fwd", "attn_proj_bwd", "attn_core_fwd", "attn_core_bwd",
            "sp_ln_fwd", "sp_ln_bwd"):
        rows += layer_rows(torch, up, bf, I, T, want)
        progress(f"inputs: {rows[-1].config} ready")
    if want("lm_head_fwd", "vocab_ce", "vocab_embed", "vocab_ce_bwd", "lm_head_ce_fused"):
        rows += vocab_rows(torch, up, bf, I, T)
        progress(f"inputs: {rows[-1].config} ready")
    return rows


def mlp_rows(torch, up, bf, I, T, cfg, tag):
    """MLP shard forward and backward (GeLU) of one workload, shard 0."""
    dev = "cuda:0"
    BF = T.TP_DT_BF16
    rows = []
    d = I.mlp_inputs(cfg, shards=[0])
    s, h, ft = d["s"], d["h"], d["ft"]
    X, W1, W2, dY = up(d["X"]), up(d["W1"][0]), up(d["W2"][0]), up(d["dY"])
    Z, H, Y = bf((s, ft)), bf((s, ft)), bf((s, h))
    dX, dW1, dW2 = bf((s, h)), bf((h, ft)), bf((ft, h))
    nb = T.tp_mlp_bwd_workspace(BF, s, h, ft)
    ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=dev)
    del d
    gf = 2.0 * s * h * ft
    name = I.CONFIGS[cfg]["name"]
    rows.append(Row(f"mlp_fwd_{tag}", name, lambda: T.tp_mlp_fwd(T.TP_ACT_GELU, BF, s, h, ft, X, W1, W2, Z, H, Y),
                    flops=2 * gf))
    rows.append(Row(f"mlp_bwd_{tag}", name, lambda: T.tp_mlp_bwd(T.TP_ACT_GELU, BF, s, h, ft, X, W1, W2, Z, H, dY,
                                                                 dX, dW1, dW2, ws, nb), flops=4 * gf))
    return rows


def layer_rows(torch, up, bf, I, T, want):
    """SwiGLU shard and attention projections, Llama-3-70B t=8."""
    dev = "cuda:0"
    BF = T.TP_DT_BF16
    rows = []
    c4 = I.CONFIGS[4]["name"]
    sw = I.swiglu_inputs(4)
    s4, h4, f4 = sw["s"], sw["h"], sw["ft"]
    X4, dY4 = up(sw["X"]), up(sw["dY"])
    Wg, Wu, Wd = up(sw["Wg"][0]), up(sw["Wu"][0]), up(sw["Wd"][0])
    del sw
    G, U, A = bf((s4, f4)), bf((s4, f4)), bf((s4, f4))
    Y4, dX4 = bf((s4, h4)), bf((s4, h4))
    dWg, dWu, dWd = bf((h4, f4)), bf((h4, f4)), bf((f4, h4))
    nb4 = T.tp_swiglu_bwd_workspace(BF, s4, h4, f4)
    ws4 = torch.empty(max(nb4, 256), dtype=torch.uint8, device=dev)
    g4 = 2.0 * s4 * h4 * f4
    rows.append(Row("swiglu_fwd", c4, lambda: T.tp_swiglu_fwd(BF, s4, h4, f4, X4, Wg, Wu, Wd, G, U, A, Y4),
                    flops=3 * g4))
    rows.append(Row("swiglu_bwd", c4, lambda: T.tp_swiglu_bwd(BF, s4, h4, f4, X4, Wg, Wu, Wd, G, U, A, dY4,
                                                              dX4, dWg, dWu, dWd, ws4, nb4), flops=6 * g4))
    at = I.attn_inputs(4)
    dq, dkv = at["dq"], at["dkv"]
    Wq, Wk, Wv, Wo = (up(at[n][0]) for n in ("Wq", "Wk", "Wv", "Wo"))
    O, dQ, dK, dV = (up(at[n][0]) for n in ("O", "dQ", "dK", "dV"))
    del at
    Q, K, V = bf((s4, dq)), bf((s4, dkv)), bf((s4, dkv))
    dWq, dWk, dWv, dO, dWo = bf((h4, dq)), bf((h4, dkv)), bf((h4, dkv)), bf((s4, dq)), bf((dq, h4))
    Ya = bf((s4, h4))
    # attention core between the projections: causal, 8 query heads on 1 KV head, d = 128
    ac = I.attn_core_inputs(4)
    Qc, Kc, Vc = up(ac["Q"][0]), up(ac["K"][0]), up(ac["V"][0])
    nqc, nkvc = ac["nq"], ac["nkv"]
    Oc = bf((s4, dq))
    lsec = torch.empty((nqc, s4), dtype=torch.float32, device=dev)
    del ac
    causal = s4 * (s4 + 1) / 2.0
    rows.append(Row("attn_core_fwd", c4, lambda: T.tp_attn_core_fwd(BF, s4, nqc, nkvc, 128, Qc, Kc, Vc, Oc, lsec),
                    flops=2.0 * 2.0 * causal * 128 * nqc))
    # its backward on the forward's O and lse: five products over the visible half
    # (the recomputed scores, dP, dV, dK, dQ; the dQ pass's second recompute of the
    # scores and dP is not counted)
    dOc = up(I.normal_bf16((s4, nqc * 128), 1.0, 4, I.T_ADO, 0))
    dQc, dKc, dVc = bf((s4, nqc * 128)), bf((s4, nkvc * 128)), bf((s4, nkvc * 128))
    nbc = T.tp_attn_core_bwd_workspace(BF, s4, nqc, nkvc, 128)
    wsc = torch.empty(max(nbc, 256), dtype=torch.uint8, device=dev)
    rows.append(Row("attn_core_bwd", c4, lambda: T.tp_attn_core_bwd(BF, s4, nqc, nkvc, 128, Qc, Kc, Vc, Oc, dOc, lsec,
                                                                    dQc, dKc, dVc, wsc, nbc),
                    flops=5.0 * 2.0 * causal * 128 * nqc))
    # sequence-parallel region on this shard's s/t = 1024 positions: residual + dropout + LayerNorm
    sp = I.sp_inputs(4)
    n_sp, p_sp = sp["n"], sp["p"]
    spy, spx, spm, spg, spb, spdz, spdun = (up(sp[k]) for k in ("y", "x", "mask", "gamma", "beta", "dz", "dun"))
    del sp
    spu, spz, spdx, spdy = bf((n_sp, h4)), bf((n_sp, h4)), bf((n_sp, h4)), bf((n_sp, h4))
    spdg, spdb = bf((h4,)), bf((h4,))
    spmean, sprstd = (torch.empty(n_sp, dtype=torch.float32, device=dev) for _ in range(2))
    nbs = T.tp_sp_ln_bwd_workspace(BF, n_sp, h4)
    wss = torch.empty(max(nbs, 256), dtype=torch.uint8, device=dev)
    el = float(n_sp * h4)
    rows.append(Row("sp_ln_fwd", c4, lambda: T.tp_sp_ln_fwd(BF, n_sp, h4, p_sp, 1e-5, spy, spx, spm, spg, spb,
                                                            spu, spz, spmean, sprstd),
                    bytes_=9.0 * el + 4.0 * h4 + 8.0 * n_sp))
    rows.append(Row("sp_ln_bwd", c4, lambda: T.tp_sp_ln_bwd(BF, n_sp, h4, p_sp, spdz, spdun, spu, spmean, sprstd,
                                                            spg, spm, spdx, spdy, spdg, spdb, wss, nbs),
                    bytes_=11.0 * el + 6.0 * h4 + 8.0 * n_sp))
    nba = T.tp_attn_proj_bwd_workspace(BF, s4, h4, dq, dkv)
    wsa = torch.empty(max(nba, 256), dtype=torch.uint8, device=dev)
    qkv = 2.0 * s4 * h4 * (dq + 2 * dkv)
    og = 2.0 * s4 * dq * h4
    rows.append(Row("attn_proj_fwd", c4, lambda: T.tp_attn_proj_fwd(BF, s4, h4, dq, dkv, X4, Wq, Wk, Wv, O, Wo,
                                                                    Q, K, V, Ya), flops=qkv + og))
    rows.append(Row("attn_proj_bwd", c4, lambda: T.tp_attn_proj_bwd(BF, s4, h4, dq, dkv, X4, Wq, Wk, Wv, O, Wo,
                                                                    dQ, dK, dV, dY4, dX4, dWq, dWk, dWv, dO,
                                                                    dWo, wsa, nba), flops=2 * qkv + 2 * og))
    return rows


def vocab_rows(torch, up, bf, I, T):
    """Vocab shard 0 of V=128256, t=8: LM head, CE statistics, embedding."""
    dev = "cuda:0"
    BF = T.TP_DT_BF16
    rows = []
    c5 = I.CONFIGS[5]["name"]
    vd = I.vocab_inputs(5, with_logits=False)
    s5, h5, Vs = vd["s"], vd["h"], vd["Vs"]
    Hf, Wlm, table = up(vd["Hf"]), up(vd["Wlm"][0]), up(vd["table"][0])
    tgt, ids = up(vd["targets"]), up(vd["ids"])
    n_in = int(((vd["ids"] >= 0) & (vd["ids"] < Vs)).sum())
    del vd
    logits = torch.empty((s5, Vs), dtype=torch.float32, device=dev)
    m, se, tl = (torch.empty(s5, dtype=torch.float32, device=dev) for _ in range(3))
    emb = bf((s5, h5))
    rows.append(Row("lm_head_fwd", c5, lambda: T.tp_lm_head_fwd(BF, s5, h5, Vs, Hf, Wlm, logits),
                    flops=2.0 * s5 * h5 * Vs))
    rows.append(Row("vocab_ce", c5, lambda: T.tp_vocab_ce(s5, Vs, 0, logits, tgt, m, se, tl),
                    bytes_=4.0 * s5 * Vs + 8.0 * s5 + 12.0 * s5))
    rows.append(Row("vocab_embed", c5, lambda: T.tp_vocab_embed(BF, s5, Vs, h5, 0, ids, table, emb),
                    bytes_=2.0 * s5 * h5 + 2.0 * n_in * h5 + 8.0 * s5))
    # CE backward on the shard's logits: (M, S) of this shard stand in for the
    # combined statistics; the gradient is stored bf16 for the LM head's backward
    dlg = bf((s5, Vs))
    gl = torch.full((s5,), 1.0 / s5, dtype=torch.float32, device=dev)
    rows.append(Row("vocab_ce_bwd", c5, lambda: T.tp_vocab_ce_bwd(BF, s5, Vs, 0, logits, tgt, m, se, gl, dlg),
                    bytes_=4.0 * s5 * Vs + 2.0 * s5 * Vs + 8.0 * s5 + 12.0 * s5))
    # the fused form: LM head with the CE statistics in its epilogue, logits never stored
    nbf = T.tp_lm_head_ce_workspace(BF, s5, h5, Vs)
    wsf = torch.empty(max(nbf, 256), dtype=torch.uint8, device=dev)
    fm, fse, ftl = (torch.empty(s5, dtype=torch.float32, device=dev) for _ in range(3))
    rows.append(Row("lm_head_ce_fused", c5,
                    lambda: T.tp_lm_head_ce_fwd(BF, s5, h5, Vs, 0, Hf, Wlm, tgt, fm, fse, ftl, wsf, nbf),
                    flops=2.0 * s5 * h5 * Vs))
    return rows


def progress(msg: str) -> None:
    """One line on stderr per finished stage (the JSON result goes to stdout)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _grow(run, work, lo, hi, budget):
    """Time run(R) for R = lo, 2 lo, ... (at most hi) until one call takes at
    least budget / 2 seconds; at R = hi whole calls repeat until they do.
    Returns (rate, R, seconds, calls) of the last timing, rate = calls *
    work(R) / seconds."""
    R = lo
    while True:
        t0 = time.perf_counter()
        run(R)
        el = time.perf_counter() - t0
        if el >= budget / 2:
            return work(R) / el, R, el, 1
        if R >= hi:
            break
        R = min(hi, R * 2)
    calls = 1
    while el < budget / 2:
        run(R)
        calls += 1
        el = time.perf_counter() - t0
    return calls * work(R) / el, R, el, calls


def cpu_baseline(seconds: float):
    """The fp64 oracle, as it stands, on bounded samples of the bench's
    workloads, on this host's cores.  The headline entry is the GPT-3-175B t=8
    MLP shard forward+backward on the first R of its 2048 rows (full shard
    weights; every product's work is linear in R, so the rate is that of the
    whole workload); "rows" holds the other rows the same way: the rate of a
    leading-row sample (labelled with its size), or of the whole input where it
    is small (embedding gather, sequence-parallel slice)."""
    import ctypes

    import numpy as np

    import oracle
    from megatron_tensor_layer_tp_amd import inputs as I

    oracle.build()
    f = I.bf16_bits_to_f64
    try:
        threads = ctypes.CDLL("libgomp.so.1").omp_get_max_threads()
    except OSError:
        threads = None
    out = {"cpu_model": cpu_model(), "rows": {}}
    rowb = max(1.0, seconds / 8)

    # headline: GPT-3-175B t=8 MLP shard
    d = I.mlp_inputs(3, shards=[0])
    X, dY, W1, W2 = f(d["X"]), f(d["dY"]), f(d["W1"][0]), f(d["W2"][0])
    s3, h3, f3 = d["s"], d["h"], d["ft"]
    del d

    def mlp_run(Xa, dYa, Wa, Wb):
        def run(R):
            oracle.mlp_fwd("gelu", Xa[:R], Wa, Wb)
            oracle.mlp_bwd("gelu", Xa[:R], Wa, Wb, dYa[:R])
        return run

    rate, R, el, n = _grow(mlp_run(X, dY, W1, W2), lambda R: 12.0 * R * h3 * f3, 8, s3, seconds / 2)
    out.update(value=rate / 1e12, unit="TFLOP/s", cores=threads, kind="oracle",
               sample=f"MLP shard fwd+bwd (GeLU), {n} call(s) on {R} of {s3} rows of the GPT-3-175B t=8 shard (h={h3}, "
                      f"f/t={f3}, full shard weights), fp64, {el:.2f} s; rate extrapolated linearly to all rows")
    del X, dY, W1, W2

    progress(f"cpu baseline: headline sample done ({el:.1f} s)")

    def add(name, unit, rate, desc):
        out["rows"][name] = {"value": rate, "unit": unit, "sample": desc}
        progress(f"cpu baseline: {name} done")

    d = I.mlp_inputs(2, shards=[0])
    X, dY, W1, W2 = f(d["X"]), f(d["dY"]), f(d["W1"][0]), f(d["W2"][0])
    rate, R, el, n = _grow(mlp_run(X, dY, W1, W2), lambda R: 12.0 * R * d["h"] * d["ft"], 64, d["s"], rowb)
    add("mlp_gpt2", "TFLOP/s", rate / 1e12, f"fwd+bwd, {n} call(s) on {R} of {d['s']} rows, {el:.2f} s (extrapolated)")
    del d, X, dY, W1, W2

    sw = I.swiglu_inputs(4)
    X, dY = f(sw["X"]), f(sw["dY"])
    Wg, Wu, Wd = f(sw["Wg"][0]), f(sw["Wu"][0]), f(sw["Wd"][0])
    h4, f4 = sw["h"], sw["ft"]
    del sw

    def sw_run(R):
        oracle.swiglu_fwd(X[:R], Wg, Wu, Wd)
        oracle.swiglu_bwd(X[:R], Wg, Wu, Wd, dY[:R])
    rate, R, el, n = _grow(sw_run, lambda R: 18.0 * R * h4 * f4, 8, 8192, rowb)
    add("swiglu", "TFLOP/s", rate / 1e12, f"fwd+bwd, {n} call(s) on {R} of 8192 rows, {el:.2f} s (extrapolated)")
    del Wg, Wu, Wd

    at = I.attn_inputs(4)
    Wq, Wk, Wv, Wo = (f(at[n][0]) for n in ("Wq", "Wk", "Wv", "Wo"))
    O, dQ, dK, dV = (f(at[n][0]) for n in ("O", "dQ", "dK", "dV"))
    dq, dkv = at["dq"], at["dkv"]
    del at

    def at_run(R):
        oracle.attn_fwd(X[:R], Wq, Wk, Wv, O[:R], Wo)
        oracle.attn_bwd(X[:R], Wq, Wk, Wv, O[:R], Wo, dQ[:R], dK[:R], dV[:R], dY[:R])
    rate, R, el, n = _grow(at_run, lambda R: 6.0 * R * h4 * (dq + 2 * dkv + dq), 8, 8192, rowb)
    add("attn_proj", "TFLOP/s", rate / 1e12, f"fwd+bwd, {n} call(s) on {R} of 8192 rows, {el:.2f} s (extrapolated)")
    del X, dY, Wq, Wk, Wv, Wo, O, dQ, dK, dV

    ac = I.attn_core_inputs(4)
    Qc, Kc, Vc = f(ac["Q"][0]), f(ac["K"][0]), f(ac["V"][0])
    nq, nkv, sc = ac["nq"], ac["nkv"], ac["s"]
    del ac

    def core_rows(R):  # R positions spread evenly over the sequence
        return np.linspace(0, sc - 1, R).astype(np.int64)

    rate, R, el, n = _grow(lambda R: oracle.attn_core_fwd(Qc, Kc, Vc, nq, nkv, rows=core_rows(R)),
                        lambda R: float(sum(4.0 * 128 * nq * (r + 1) for r in core_rows(R))), 8, sc, rowb)
    add("attn_core_fwd", "TFLOP/s", rate / 1e12, f"{R} of {sc} query positions spread over the sequence, "
        f"{el:.2f} s (causal FLOPs of those rows)")
    del Qc, Kc, Vc

    vd = I.vocab_inputs(5, with_table=True, with_logits=False)
    Hf, Wlm = f(vd["Hf"]), f(vd["Wlm"][0])
    Vs, h5, s5 = vd["Vs"], vd["h"], vd["s"]
    rate, R, el, n = _grow(lambda R: oracle.lm_head(Hf[:R], Wlm), lambda R: 2.0 * R * h5 * Vs, 4, s5, rowb)
    add("lm_head_fwd", "TFLOP/s", rate / 1e12, f"{n} call(s) on {R} of {s5} rows, {el:.2f} s (extrapolated)")
    del Hf, Wlm
    n_in = int(((vd["ids"] >= 0) & (vd["ids"] < Vs)).sum())
    ids, table, tg = vd["ids"], vd["table"][0], vd["targets"]
    del vd
    rate, R, el, n = _grow(lambda R: oracle.embed(ids[:R], table, 0),
                           lambda R: 2.0 * R * h5 + 2.0 * n_in * h5 * R / s5 + 8.0 * R, 1024, s5, rowb)
    add("vocab_embed", "GB/s", rate / 1e9, f"{n} call(s) over {R} of {s5} ids, {el:.2f} s")
    del table
    z = I.normal_f32((s5, Vs), 0.905, 5, I.T_LOGITS, 0).astype(np.float64)
    rate, R, el, n = _grow(lambda R: oracle.ce_stats(z[:R], tg[:R], 0), lambda R: (4.0 * Vs + 20.0) * R, 256, s5,
                           rowb)
    add("vocab_ce", "GB/s", rate / 1e9, f"{n} call(s) over {R} of {s5} positions of fp32 logits, {el:.2f} s")
    m, se, _ = oracle.ce_stats(z, tg, 0)
    g = np.full(s5, 1.0 / s5)
    rate, R, el, n = _grow(lambda R: oracle.ce_bwd(z[:R], tg[:R], 0, m[:R], se[:R], g[:R]),
                           lambda R: (6.0 * Vs + 20.0) * R, 256, s5, rowb)
    add("vocab_ce_bwd", "GB/s", rate / 1e9, f"{n} call(s) over {R} of {s5} positions, {el:.2f} s")
    del z

    sp = I.sp_inputs(4)
    y_, x_, gm, bt = f(sp["y"]), f(sp["x"]), f(sp["gamma"]), f(sp["beta"])
    n_sp, hs = sp["n"], sp["h"]
    mask, dz_, dun_ = sp["mask"], f(sp["dz"]), f(sp["dun"])
    rate, R, el, n = _grow(lambda R: oracle.sp_ln_fwd(y_[:R], x_[:R], mask[:R], gm, bt, sp["p"]),
                           lambda R: 9.0 * R * hs + 4.0 * hs + 8.0 * R, 64, n_sp, rowb)
    add("sp_ln_fwd", "GB/s", rate / 1e9, f"{n} call(s) over {R} of {n_sp} rows x {hs}, {el:.2f} s")
    u, zz, mu, rs = oracle.sp_ln_fwd(y_, x_, mask, gm, bt, sp["p"])
    rate, R, el, n = _grow(lambda R: oracle.sp_ln_bwd(dz_[:R], dun_[:R], u[:R], mu[:R], rs[:R], gm, mask[:R],
                                                      sp["p"]),
                           lambda R: 11.0 * R * hs + 6.0 * hs + 8.0 * R, 64, n_sp, rowb)
    add("sp_ln_bwd", "GB/s", rate / 1e9, f"{n} call(s) over {R} of {n_sp} rows x {hs}, {el:.2f} s")
    return out


# ---------------------------------------------------------------------------
# rocprofv3 counter passes -> per-row summaries
# ---------------------------------------------------------------------------
ROW_NAMES = ["mlp_fwd_gpt3", "mlp_bwd_gpt3", "mlp_fwd_gpt2", "mlp_bwd_gpt2", "swiglu_fwd", "swiglu_bwd",
             "attn_proj_fwd", "attn_proj_bwd", "attn_core_fwd", "attn_core_bwd", "sp_ln_fwd", "sp_ln_bwd",
             "lm_head_fwd", "vocab_ce", "vocab_embed", "vocab_ce_bwd", "lm_head_ce_fused"]
COUNTER_PASSES = {"fetch": ["FETCH_SIZE"], "write": ["WRITE_SIZE"],
                  "sq": ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CU_CYCLES", "SQ_INSTS_MFMA"]}


def alg_bytes(row: str) -> float:
    """Compulsory HBM bytes of one call of a bench row: every input read once,
    every output (and every intermediate a call must hand between its launches)
    written once -- the per-unit figures times the workload's sizes."""
    from megatron_tensor_layer_tp_amd import inputs as I
    b = 2.0
    if row.startswith("mlp_"):
        c = I.CONFIGS[3 if row.endswith("gpt3") else 2]
        s, h, ft = c["s"], c["h"], c["f"] // c["t"]
        if row.startswith("mlp_fwd"):
            return b * (s * h + 2 * h * ft + 2 * s * ft + s * h)
        # X, W1, W2, Z, H, dY read; dX, dW1, dW2 written; dZ written and read back
        return b * (2 * s * h + 2 * h * ft + 2 * s * ft) + b * (s * h + 2 * h * ft) + 2 * b * s * ft
    c = I.CONFIGS[4]
    s, h = c["s"], c["h"]
    ft = c["f"] // c["t"]
    dq, dkv = c["dq_full"] // c["t"], c["dkv_full"] // c["t"]
    nq = dq // 128
    c5 = I.CONFIGS[5]
    s5, h5, Vs = c5["s"], c5["h"], c5["V"] // c5["t"]
    n_sp = s // c["t"]
    table = {
        "swiglu_fwd": b * (s * h + 3 * h * ft + 3 * s * ft + s * h),
        "swiglu_bwd": b * (s * h + 3 * h * ft + 3 * s * ft + s * h) + b * (s * h + 3 * h * ft) + 2 * 2 * b * s * ft,
        "attn_proj_fwd": b * (s * h + h * (dq + 2 * dkv) + s * dq + dq * h + s * (dq + 2 * dkv) + s * h),
        "attn_proj_bwd": b * (s * h + h * (dq + 2 * dkv) + s * dq + dq * h + s * (dq + 2 * dkv) + s * h)
        + b * (s * h + h * (dq + 2 * dkv) + s * dq + dq * h),
        "attn_core_fwd": b * (s * dq + 2 * s * dkv + s * dq) + 4.0 * nq * s,
        "attn_core_bwd": b * (3 * s * dq + 2 * s * dkv) + 4.0 * nq * s + b * (s * dq + 2 * s * dkv),
        "sp_ln_fwd": 9.0 * n_sp * h + 4.0 * h + 8.0 * n_sp,
        "sp_ln_bwd": 11.0 * n_sp * h + 6.0 * h + 8.0 * n_sp,
        "lm_head_fwd": b * (s5 * h5 + h5 * Vs) + 4.0 * s5 * Vs,
        "lm_head_ce_fused": b * (s5 * h5 + h5 * Vs) + 8.0 * s5 + 12.0 * s5,
        "vocab_ce": 4.0 * s5 * Vs + 20.0 * s5,
        "vocab_ce_bwd": 6.0 * s5 * Vs + 20.0 * s5,
        "vocab_embed": 2.0 * s5 * h5 + 2.0 * h5 * s5 / 8 + 8.0 * s5,   # about 1/8 of the ids in the shard
    }
    return table[row]


def csrc_hash() -> str:
    names = sorted(n for n in os.listdir(os.path.join(ROOT, "megatron_tensor_layer_tp_amd", "csrc")))
    return src_hash(*names)


def traffic_for(key: str):
    """HBM bytes per launch of the row's dominant kernel from the committed
    counter summary, or None when any kernel source changed since the counters
    were taken."""
    p = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    if t.get("csrc_hash") != csrc_hash():
        return None
    e = t.get("rows", {}).get(key)
    return e["dominant_kernel"]["bytes"] if e else None


def summarize_counters(d: str):
    """Reduce rocprofv3 --pmc passes under d to profiles/hbm_traffic.json and a
    markdown table (printed).  Layout: d/<row>/<pass>/**/*counter_collection.csv
    for each row of ROW_NAMES and pass of COUNTER_PASSES (fetch, write, sq), and
    d/copy/fetch, d/copy/write for the 1 GiB copy that calibrates FETCH_SIZE and
    WRITE_SIZE (bytes per KiB reported).  Per (kernel, grid) the counters are
    averaged over the dispatches after the first (cold caches); kernels launched
    once per run (the inputs of vocab_ce / attn_core_bwd) are left out."""
    import csv
    import glob

    def dispatches(path):
        by = {}
        for f in glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True):
            with open(f) as fh:
                for r in csv.DictReader(fh):
                    e = by.setdefault(int(r["Dispatch_Id"]), {"kernel": r["Kernel_Name"], "grid": int(r["Grid_Size"]),
                                                             "us": (int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
                                                             / 1000.0})
                    e[r["Counter_Name"]] = e.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        return [by[k] for k in sorted(by)]

    def per_kernel(recs, counter, runtime=False):
        groups = {}
        for e in recs:
            groups.setdefault((e["kernel"], e["grid"]), []).append(e)
        out = {}
        for key, es in groups.items():
            if len(es) < 2 or (key[0].startswith("__amd_rocclr") and not runtime):  # the inputs' own copies
                continue
            es = es[1:]
            out[key] = {"n": len(es), "us": sum(x["us"] for x in es) / len(es),
                        counter: sum(x.get(counter, 0.0) for x in es) / len(es)}
        return out

    def short(name):
        name = name.replace("void ", "").replace("(anonymous namespace)::", "")
        return name.split("(GemmDesc")[0].split("((")[0].split("(")[0] if "<" not in name else name.split("(Gemm")[0]

    cf = per_kernel(dispatches(os.path.join(d, "copy", "fetch")), "FETCH_SIZE", runtime=True)
    cw = per_kernel(dispatches(os.path.join(d, "copy", "write")), "WRITE_SIZE", runtime=True)
    kf = next(v for k, v in cf.items() if "copyBuffer" in k[0])["FETCH_SIZE"]
    kw = next(v for k, v in cw.items() if "copyBuffer" in k[0])["WRITE_SIZE"]
    ff, wf = (1 << 30) / (kf * 1024), (1 << 30) / (kw * 1024)
    res = {"csrc_hash": csrc_hash(),
           "calibration": {"copy_bytes": 1 << 30, "fetch_size_kib": round(kf, 1), "write_size_kib": round(kw, 1),
                           "fetch_factor": round(ff, 4), "write_factor": round(wf, 4)},
           "rows": {}}
    lines = ["| row | kernel | grid | us | FETCH KiB | WRITE KiB | HBM bytes | MFMA busy |",
             "|---|---|---:|---:|---:|---:|---:|---:|"]
    for row in ROW_NAMES:
        rd = os.path.join(d, row)
        if not os.path.isdir(rd):
            continue
        f = per_kernel(dispatches(os.path.join(rd, "fetch")), "FETCH_SIZE")
        w = per_kernel(dispatches(os.path.join(rd, "write")), "WRITE_SIZE")
        sq = {}
        for k, v in per_kernel(dispatches(os.path.join(rd, "sq")), "SQ_VALU_MFMA_BUSY_CYCLES").items():
            sq[k] = v
        recs = dispatches(os.path.join(rd, "sq"))
        busy = {}
        for e in recs:
            busy.setdefault((e["kernel"], e["grid"]), []).append(e)
        kernels = []
        for key in f:
            if key not in w:
                continue
            by = f[key]["FETCH_SIZE"] * 1024 * ff + w[key]["WRITE_SIZE"] * 1024 * wf
            mf = None
            es = busy.get(key, [])[1:]
            if es:
                mb = sum(x.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) for x in es)
                cu = sum(x.get("SQ_BUSY_CU_CYCLES", 0.0) for x in es)
                mf = mb / (4.0 * cu) if cu > 0 else None
            kernels.append({"kernel": short(key[0]), "grid": key[1], "us": round(f[key]["us"], 2),
                            "fetch_kib": round(f[key]["FETCH_SIZE"], 1), "write_kib": round(w[key]["WRITE_SIZE"], 1),
                            "bytes": int(by), "mfma_busy": None if mf is None else round(mf, 4)})
        if not kernels:
            continue
        dom = max(kernels, key=lambda k: k["us"])
        total = sum(k["bytes"] for k in kernels)
        alg = alg_bytes(row)
        res["rows"][row] = {"kernels": kernels, "dominant_kernel": dom, "bytes_per_call": total,
                            "algorithmic_bytes": int(alg), "ratio": round(total / alg, 3)}
        for k in kernels:
            mfs = "" if k["mfma_busy"] is None else f"{100 * k['mfma_busy']:.1f}%"
            lines.append(f"| {row} | `{k['kernel']}` | {k['grid']} | {k['us']:.1f} | {k['fetch_kib']:.0f} | "
                         f"{k['write_kib']:.0f} | {k['bytes'] / 1e6:.1f} MB | {mfs} |")
        lines.append(f"| {row} | **call total** | | | | | {total / 1e6:.1f} MB "
                     f"(algorithmic {alg / 1e6:.1f} MB, x{total / alg:.2f}) | |")
    with open(os.path.join(ROOT, "profiles", "hbm_traffic.json"), "w") as fh:
        json.dump(res, fh, indent=1)
    print("\n".join(lines))


def main():
    args = parse()
    if args.counter_summary:
        summarize_counters(args.counter_summary)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    import torch

    from megatron_tensor_layer_tp_amd import tpshard as T

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    T.lib()  # fails loudly when libtpshard.so is missing
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        # a plain copy of known size: reads and writes exactly 1 GiB per launch
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": 1 << 30, "launches": 3}))
        return
    first = "lm_head_fwd" if args.only in ("vocab_ce", "vocab_ce_bwd") else \
        "attn_core_fwd" if args.only == "attn_core_bwd" else args.only
    rows = build_rows(torch, args.rows, first)
    progress(f"inputs resident, {len(rows)} rows")
    if args.only:
        keep = [r for r in rows if r.name == args.only]
        if not keep:
            print(f"no row named {args.only}; rows: {[r.name for r in rows]}", file=sys.stderr)
            sys.exit(2)
        if args.only in ("vocab_ce", "vocab_ce_bwd"):  # input: the LM head's output, computed once
            next(r for r in rows if r.name == "lm_head_fwd").fn()
            if args.only == "vocab_ce_bwd":
                next(r for r in rows if r.name == "vocab_ce").fn()
        if args.only == "attn_core_bwd":  # inputs: the forward's O and lse, computed once
            next(r for r in rows if r.name == "attn_core_fwd").fn()
        rows = keep
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        for r in rows:
            r.run(torch, False)
    torch.cuda.synchronize()
    progress("warm-up done")
    with GpuSampler() as sampler:
        t0 = time.perf_counter()
        for _ in range(args.steps):
            for r in rows:
                r.run(torch, True)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    progress(f"timed {args.steps} steps in {wall:.2f} s")

    by = {r.name: r for r in rows}
    if args.only:
        r = rows[0]
        ms = r.ms()
        print(json.dumps({"row": r.name, "config": r.config, "ms": ms,
                          "tflops": r.flops / (ms * 1e-3) / 1e12 if r.flops else None,
                          "gbs": r.bytes / (ms * 1e-3) / 1e9 if r.bytes else None}))
        return
    def mlp_rate(tag):
        ms = by[f"mlp_fwd_{tag}"].ms() + by[f"mlp_bwd_{tag}"].ms()
        return (by[f"mlp_fwd_{tag}"].flops + by[f"mlp_bwd_{tag}"].flops) / (ms * 1e-3) / 1e12

    value = mlp_rate("gpt3")
    other_mlp = {"gpt2-small-gelu-mlp-t2 (s=8192, h=768, f/t=1536) fwd+bwd TFLOP/s": round(mlp_rate("gpt2"), 2)}
    if "swiglu_fwd" in by:
        sw_ms = by["swiglu_fwd"].ms() + by["swiglu_bwd"].ms()
        other_mlp["llama3-70b-swiglu-t8 (s=8192, h=8192, f/t=3584) fwd+bwd TFLOP/s"] = round(
            (by["swiglu_fwd"].flops + by["swiglu_bwd"].flops) / (sw_ms * 1e-3) / 1e12, 2)
    out_rows = {}
    for r in rows:
        ms = r.ms()
        e = {"config": r.config, "ms": round(ms, 4), "ms_p10": round(r.pct(0.1), 4),
             "ms_median": round(r.pct(0.5), 4), "ms_p90": round(r.pct(0.9), 4)}
        if r.flops:
            tf = r.flops / (ms * 1e-3) / 1e12
            e.update(tflops=round(tf, 2), frac_mfma_peak=round(tf / PEAK_BF16_TFLOPS, 4))
        if r.bytes:
            gbs = r.bytes / (ms * 1e-3) / 1e9
            e.update(gbs=round(gbs, 1), frac_hbm_peak=round(gbs / PEAK_HBM_GBS, 4))
        out_rows[r.name] = e

    res = {
        "metric": "TP-shard MLP fwd+bwd TFLOP/s (bf16, % MFMA peak); vocab-CE GB/s",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,sigma) bf16 inputs, random-init weights)",
        "config": {"workload": "gpt3-175b-gelu-mlp-t8: s=2048 (b=1), h=12288, f/t=6144, GeLU, bf16",
                   "frac_mfma_peak": round(value / PEAK_BF16_TFLOPS, 4),
                   "other_mlp_workloads": other_mlp,
                   "step_rows": "mlp fwd+bwd (this workload, and gpt2-small t=2); swiglu + attention "
                                "projections + attention core fwd+bwd + sequence-parallel region "
                                "(llama3-70b t=8, s=8192); lm head + vocab CE (+ backward) + fused "
                                "lm head/CE + embedding (V=128256 t=8, s=8192)"
                                if args.rows == "all" else "mlp fwd+bwd only"},
        "rows": out_rows,
        "gpu_during_steps": sampler.summary(),
    }
    if "vocab_ce" in by:
        ce = by["vocab_ce"]
        res["vocab_ce_gbs"] = out_rows["vocab_ce"]["gbs"]
    if "lm_head_fwd" in by:
        r = by["lm_head_fwd"]
        ach = r.flops / (r.ms() * 1e-3) / 1e12
        res["roofline"] = {"kernel": "gemm_dma_kernel<256,256,NN,store fp32,8 waves> (tp_lm_head_fwd)",
                           "bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS,
                           "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                           "traffic": traffic_for("lm_head_fwd")}
        c = by["vocab_ce"]
        gbs = c.bytes / (c.ms() * 1e-3) / 1e9
        res["roofline_ce"] = {"kernel": "vocab_ce_kernel<4> (tp_vocab_ce)", "bound": "hbm",
                              "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                              "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic_for("vocab_ce")}
    else:
        r = by["mlp_bwd_gpt3"]
        ach = r.flops / (r.ms() * 1e-3) / 1e12
        res["roofline"] = {"kernel": "gemm_dma kernels (tp_mlp_bwd, 4 GEMMs)", "bound": "mfma",
                           "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                           "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": None}
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
