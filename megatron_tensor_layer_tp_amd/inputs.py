"""Seeded synthetic inputs for the tensor-parallel shard path.

This module is shared by the tests, the benchmark and the smoke check.  It
produces host arrays only (numpy) and holds none of the layer's arithmetic: no
products, activations or reductions.  Its one numeric conversion is the
round-to-nearest-even narrowing of fp32 samples to bfloat16 bit patterns, so
that the GPU library and the fp64 checker read the very same input values.

Every tensor draws from its own PCG64 stream, keyed by
``SeedSequence(entropy=ENTROPY, spawn_key=(config, tensor, shard))``.  A full
(unsharded) weight is the concatenation of its shards' draws, so a caller can
generate shard 0 alone (the benchmark) or all shards (the parity tests) and see
identical values for the shard they share.

Shard convention (two-card worked example in "7.3 模型并行与张量并行", §7.3.2):
shard i of t holds columns ``[i*f/t, (i+1)*f/t)`` of the column-split weight and
the same rows of the row-split weight; vocab shard i holds vocab rows
``[i*V/t, (i+1)*V/t)`` ("7.3.4" and the CMU 11-868 lecture 16 notes, §5.5).
"""
from __future__ import annotations

import numpy as np

ENTROPY = 20261202

# tensor ids used in the seed key; never renumber (stored values depend on them)
T_X, T_W1, T_W2, T_DY, T_WG, T_WU, T_WD, T_WQ, T_WK, T_WV, T_WO, T_O, T_DQ, T_DK, \
    T_DV, T_HF, T_WLM, T_TGT, T_TABLE, T_IDS, T_LOGITS = range(21)
T_AQ, T_AK, T_AV = 21, 22, 23   # attention-core inputs
T_SPY, T_SPX, T_SPMASK, T_SPG, T_SPB, T_SPDZ, T_SPDUN = range(24, 31)   # sequence-parallel region
T_ADO = 31   # gradient arriving at the attention core's output


def _rng(config: int, tensor: int, shard: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence(entropy=ENTROPY, spawn_key=(config, tensor, shard))))


# ---------------------------------------------------------------------------
# bfloat16 bit patterns
# ---------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bfloat16 (round to nearest, ties to even); uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    out = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to fp32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(b).astype(np.float64)


# ---------------------------------------------------------------------------
# primitive draws
# ---------------------------------------------------------------------------
def normal_bf16(shape, sigma: float, config: int, tensor: int, shard: int = 0) -> np.ndarray:
    """N(0, sigma^2) samples (sigma is the standard deviation), as bf16 bits."""
    g = _rng(config, tensor, shard)
    x = g.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return f32_to_bf16_bits(x)


def normal_f32(shape, sigma: float, config: int, tensor: int, shard: int = 0) -> np.ndarray:
    g = _rng(config, tensor, shard)
    x = g.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return x


def int_uniform_f32(shape, lo: int, hi: int, config: int, tensor: int, shard: int = 0) -> np.ndarray:
    """Integers uniform on the closed range [lo, hi], stored as fp32."""
    g = _rng(config, tensor, shard)
    return g.integers(lo, hi + 1, size=shape).astype(np.float32)


def ids_uniform(n: int, vocab: int, config: int, tensor: int, shard: int = 0) -> np.ndarray:
    """Token ids uniform over the whole vocabulary [0, vocab), int64."""
    g = _rng(config, tensor, shard)
    return g.integers(0, vocab, size=(n,), dtype=np.int64)


# ---------------------------------------------------------------------------
# workloads (sizes of the five shard configurations)
# ---------------------------------------------------------------------------
CONFIGS = {
    # tiny ReLU MLP, two emulated shards, fp32 holding integers in [-3, 3]
    1: dict(name="tiny-relu-mlp-t2", kind="mlp", act="relu", dtype="f32",
            s=8, h=16, f=64, t=2, int_range=(-3, 3)),
    # GPT-2-small sized GeLU MLP shard, t=2, b*s = 8*1024 rows
    2: dict(name="gpt2-small-gelu-mlp-t2", kind="mlp", act="gelu", dtype="bf16",
            s=8 * 1024, h=768, f=3072, t=2, sx=1.0, sw=0.02, sdy=1.0),
    # GPT-3-175B sized GeLU MLP shard, t=8, one sequence of 2048 tokens
    3: dict(name="gpt3-175b-gelu-mlp-t8", kind="mlp", act="gelu", dtype="bf16",
            s=2048, h=12288, f=49152, t=8, sx=1.0, sw=0.006, sdy=1.0),
    # Llama-3-70B sized layer shard, t=8, s=8192: SwiGLU + attention projections
    4: dict(name="llama3-70b-layer-t8", kind="layer", dtype="bf16",
            s=8192, h=8192, f=28672, t=8, dq_full=8192, dkv_full=1024,
            sx=1.0, sw=0.01, sdy=1.0),
    # vocab-parallel shard, V=128256, t=8: LM head, CE statistics, embedding gather
    5: dict(name="llama3-vocab-t8", kind="vocab", dtype="bf16",
            s=8192, h=8192, V=128256, t=8, sx=1.0, sw=0.01, slogit=None),
}


def shard_width(full: int, t: int) -> int:
    if full % t:
        raise ValueError(f"{full} does not split evenly over t={t}")
    return full // t


# ---------------------------------------------------------------------------
# per-config input sets
# ---------------------------------------------------------------------------
def mlp_inputs(cfg_id: int, shards=None, s=None):
    """Inputs of an MLP configuration.

    Returns a dict with X [s,h], dY [s,h] and per-shard W1 [h,f/t], W2 [f/t,h]
    (lists indexed by shard).  bf16 configs hold uint16 bit patterns; the fp32
    integer configuration holds float32 integers.  ``s`` may shrink the row
    count (rows are a prefix of the full draw's leading rows only when the
    generator is asked for the same s, so tests pass their own s explicitly).
    """
    c = CONFIGS[cfg_id]
    s = c["s"] if s is None else s
    h, t = c["h"], c["t"]
    ft = shard_width(c["f"], t)
    shards = range(t) if shards is None else shards
    out = {"s": s, "h": h, "ft": ft, "t": t, "act": c["act"], "dtype": c["dtype"]}
    if c["dtype"] == "f32":
        lo, hi = c["int_range"]
        out["X"] = int_uniform_f32((s, h), lo, hi, cfg_id, T_X)
        out["dY"] = int_uniform_f32((s, h), lo, hi, cfg_id, T_DY)
        out["W1"] = {i: int_uniform_f32((h, ft), lo, hi, cfg_id, T_W1, i) for i in shards}
        out["W2"] = {i: int_uniform_f32((ft, h), lo, hi, cfg_id, T_W2, i) for i in shards}
    else:
        out["X"] = normal_bf16((s, h), c["sx"], cfg_id, T_X)
        out["dY"] = normal_bf16((s, h), c["sdy"], cfg_id, T_DY)
        out["W1"] = {i: normal_bf16((h, ft), c["sw"], cfg_id, T_W1, i) for i in shards}
        out["W2"] = {i: normal_bf16((ft, h), c["sw"], cfg_id, T_W2, i) for i in shards}
    return out


def swiglu_inputs(cfg_id: int = 4, shards=(0,), s=None, h=None, ft=None):
    """SwiGLU shard inputs: X [s,h], dY [s,h], Wg/Wu [h,ft], Wd [ft,h] (bf16 bits)."""
    c = CONFIGS[cfg_id]
    s = c["s"] if s is None else s
    h = c["h"] if h is None else h
    ft = shard_width(c["f"], c["t"]) if ft is None else ft
    out = {"s": s, "h": h, "ft": ft,
           "X": normal_bf16((s, h), c["sx"], cfg_id, T_X),
           "dY": normal_bf16((s, h), c["sdy"], cfg_id, T_DY)}
    for name, tid, shp in (("Wg", T_WG, (h, ft)), ("Wu", T_WU, (h, ft)), ("Wd", T_WD, (ft, h))):
        out[name] = {i: normal_bf16(shp, c["sw"], cfg_id, tid, i) for i in shards}
    return out


def attn_inputs(cfg_id: int = 4, shards=(0,), s=None, h=None, dq=None, dkv=None):
    """Attention-projection shard inputs (bf16 bits).

    X [s,h]; Wq [h,dq], Wk/Wv [h,dkv], Wo [dq,h]; the attention-core output O
    [s,dq] and the gradients dQ [s,dq], dK/dV [s,dkv], dY [s,h] are synthetic
    N(0,1) draws (the attention core itself is not part of this path).
    """
    c = CONFIGS[cfg_id]
    s = c["s"] if s is None else s
    h = c["h"] if h is None else h
    dq = shard_width(c["dq_full"], c["t"]) if dq is None else dq
    dkv = shard_width(c["dkv_full"], c["t"]) if dkv is None else dkv
    out = {"s": s, "h": h, "dq": dq, "dkv": dkv,
           "X": normal_bf16((s, h), c["sx"], cfg_id, T_X),
           "dY": normal_bf16((s, h), c["sdy"], cfg_id, T_DY)}
    for name, tid, shp in (("Wq", T_WQ, (h, dq)), ("Wk", T_WK, (h, dkv)),
                           ("Wv", T_WV, (h, dkv)), ("Wo", T_WO, (dq, h))):
        out[name] = {i: normal_bf16(shp, c["sw"], cfg_id, tid, i) for i in shards}
    for name, tid, shp in (("O", T_O, (s, dq)), ("dQ", T_DQ, (s, dq)),
                           ("dK", T_DK, (s, dkv)), ("dV", T_DV, (s, dkv))):
        out[name] = {i: normal_bf16(shp, 1.0, cfg_id, tid, i) for i in shards}
    return out


def attn_core_inputs(cfg_id: int = 4, shards=(0,), s=None):
    """Attention-core shard inputs (bf16 bits): Q [s,dq] (dq / 128 query heads)
    and K, V [s,dkv] (dkv / 128 key/value heads), N(0,1) draws, so the scores
    Q.K/sqrt(128) have unit spread."""
    c = CONFIGS[cfg_id]
    s = c["s"] if s is None else s
    dq = shard_width(c["dq_full"], c["t"])
    dkv = shard_width(c["dkv_full"], c["t"])
    out = {"s": s, "dq": dq, "dkv": dkv, "nq": dq // 128, "nkv": dkv // 128}
    for name, tid, w in (("Q", T_AQ, dq), ("K", T_AK, dkv), ("V", T_AV, dkv)):
        out[name] = {i: normal_bf16((s, w), 1.0, cfg_id, tid, i) for i in shards}
    return out


def sp_inputs(cfg_id: int = 4, n=None, h=None, p: float = 0.1):
    """Sequence-parallel region inputs for one shard's n = s/t positions (bf16
    bits unless stated): y (sublayer output after the reduce-scatter) and x
    (residual stream) N(0,1); a dropout mask [n,h] uint8 with P(keep) = 1 - p;
    LayerNorm gamma ~ 1 + N(0, 0.1^2), beta ~ N(0, 0.1^2); and the backward's
    dz, dun ~ N(0,1)."""
    c = CONFIGS[cfg_id]
    n = c["s"] // c["t"] if n is None else n
    h = c["h"] if h is None else h
    keep = _rng(cfg_id, T_SPMASK).random((n, h)) >= p
    g = _rng(cfg_id, T_SPG).standard_normal(h).astype(np.float32)
    return {"n": n, "h": h, "p": p,
            "y": normal_bf16((n, h), 1.0, cfg_id, T_SPY), "x": normal_bf16((n, h), 1.0, cfg_id, T_SPX),
            "mask": keep.astype(np.uint8),
            "gamma": f32_to_bf16_bits(1.0 + 0.1 * g), "beta": normal_bf16((h,), 0.1, cfg_id, T_SPB),
            "dz": normal_bf16((n, h), 1.0, cfg_id, T_SPDZ), "dun": normal_bf16((n, h), 1.0, cfg_id, T_SPDUN)}


def vocab_inputs(cfg_id: int = 5, shards=(0,), s=None, h=None, V=None, t=None,
                 with_lm=True, with_table=True, with_logits=True, logit_sigma=0.905):
    """Vocab-parallel inputs.

    Hf [s,h] bf16 and per-shard Wlm [h,V/t] bf16 (LM head); targets [s] and ids
    [s] int64, uniform over [0,V); per-shard embedding tables [V/t,h] bf16; and
    per-shard fp32 logit slices [s,V/t] drawn N(0, logit_sigma^2), the spread an
    N(0,1) x N(0,0.01) product over h=8192 gives, so the CE statistics can be
    checked on inputs that do not come from any GEMM.
    """
    c = CONFIGS[cfg_id]
    s = c["s"] if s is None else s
    h = c["h"] if h is None else h
    V = c["V"] if V is None else V
    t = c["t"] if t is None else t
    Vs = shard_width(V, t)
    out = {"s": s, "h": h, "V": V, "t": t, "Vs": Vs,
           "targets": ids_uniform(s, V, cfg_id, T_TGT),
           "ids": ids_uniform(s, V, cfg_id, T_IDS)}
    if with_lm:
        out["Hf"] = normal_bf16((s, h), c["sx"], cfg_id, T_HF)
        out["Wlm"] = {i: normal_bf16((h, Vs), c["sw"], cfg_id, T_WLM, i) for i in shards}
    if with_table:
        out["table"] = {i: normal_bf16((Vs, h), 1.0, cfg_id, T_TABLE, i) for i in shards}
    if with_logits:
        out["logits"] = {i: normal_f32((s, Vs), logit_sigma, cfg_id, T_LOGITS, i) for i in shards}
    return out


def sample_rows(n: int, k: int, config: int, salt: int = 0, stratum: int = 64) -> np.ndarray:
    """Seeded, sorted, distinct indices in [0, n) for sampled parity checks.

    Stratified: one index drawn uniformly inside every run of ``stratum``
    consecutive indices (so every 64-row strip -- each wave's slice of a 128-
    or 256-row tile, each 128-row query block -- holds at least one), the
    first and the last index (edge tiles), then further distinct random
    indices until there are at least ``k``.  All of [0, n) when k >= n.
    """
    if k >= n:
        return np.arange(n, dtype=np.int64)
    g = _rng(config, 1000 + salt, 0)
    starts = np.arange(0, n, stratum, dtype=np.int64)
    widths = np.minimum(stratum, n - starts)
    picked = set((starts + (g.random(starts.shape[0]) * widths).astype(np.int64)).tolist())
    picked.update((0, n - 1))
    if len(picked) < k:
        rest = np.setdiff1d(np.arange(n, dtype=np.int64), np.fromiter(picked, dtype=np.int64))
        picked.update(g.choice(rest, size=k - len(picked), replace=False).tolist())
    return np.array(sorted(picked), dtype=np.int64)
