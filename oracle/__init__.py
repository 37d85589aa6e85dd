"""fp64 CPU oracle for one tensor-parallel shard of a transformer layer.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import this package.  The GPU library shares
no code with it: the oracle's arithmetic lives in ``oracle.c`` (plain C,
double precision, sums in increasing k order) and the definitions below only
compose those routines on numpy arrays.

Each function states the passage it follows.  Page names used below:
  [book]    "7.3 模型并行与张量并行：把一层切到多张卡上" (LLM internals book)
  [lec16]   CMU 11-868 lecture 16 notes, "5. 张量并行 · Tensor parallelism"

Parity pins (tests/test_oracle_*.py) tie every function here to something
other than itself: the book's two-card worked example (§7.3.2/§7.3.3), its
row-split-first counterexample, exact integer arithmetic in pure Python,
central finite differences of the forward pass, numpy / torch fp64 library
routines (matmul, gelu, silu, cross_entropy), and closed forms.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

RELU, GELU, SILU = 0, 1, 2
_ACT = {"relu": RELU, "gelu": GELU, "silu": SILU}


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc (-O2, OpenMP, no fast-math) into liboracle.so."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared",
                               "-fno-fast-math", "-ffp-contract=off", "-D_GNU_SOURCE",
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None
_d = ctypes.POINTER(ctypes.c_double)
_i64 = ctypes.c_int64


def _L():
    global _lib
    if _lib is None:
        # ORACLE_LIB: an alternative build of oracle.c (the sanitizer test's)
        lib = ctypes.CDLL(os.environ.get("ORACLE_LIB") or build())
        lib.or_gemm.argtypes = [_i64, _i64, _i64, _d, _d, _d]
        lib.or_act.argtypes = [ctypes.c_int, _i64, _d, _d]
        lib.or_act_grad.argtypes = [ctypes.c_int, _i64, _d, _d]
        lib.or_ce_stats.argtypes = [_i64, _i64, _i64, _d, ctypes.c_void_p, _d, _d, _d]
        lib.or_ce_combine.argtypes = [_i64, _i64, _d, _d, _d, _d]
        lib.or_ce_direct.argtypes = [_i64, _i64, _d, ctypes.c_void_p, _d]
        lib.or_ce_bwd.argtypes = [_i64, _i64, _i64, _d, ctypes.c_void_p, _d, _d, _d, _d]
        lib.or_sp_ln_fwd.argtypes = [_i64, _i64, ctypes.c_double, ctypes.c_double, _d, _d, ctypes.c_void_p,
                                     _d, _d, _d, _d, _d, _d]
        lib.or_sp_ln_bwd.argtypes = [_i64, _i64, ctypes.c_double, _d, _d, _d, _d, _d, _d, ctypes.c_void_p,
                                     _d, _d, _d, _d]
        lib.or_attn_fwd.argtypes = [_i64, _i64, _i64, _i64, ctypes.c_int, _d, _d, _d, _i64, ctypes.c_void_p,
                                    _d, _d]
        lib.or_attn_bwd.argtypes = [_i64, _i64, _i64, _i64, ctypes.c_int, _d, _d, _d, _d, _i64, ctypes.c_void_p,
                                    _i64, ctypes.c_void_p, _d, _d, _d]
        lib.or_embed_u16.argtypes = [_i64, _i64, _i64, _i64, ctypes.c_void_p,
                                     ctypes.c_void_p, ctypes.c_void_p]
        lib.or_embed_u32.argtypes = [_i64, _i64, _i64, _i64, ctypes.c_void_p,
                                     ctypes.c_void_p, ctypes.c_void_p]
        _lib = lib
    return _lib


def set_threads(n: int) -> None:
    """Number of OpenMP threads the oracle uses (libgomp reads OMP_NUM_THREADS once)."""
    gomp = ctypes.CDLL("libgomp.so.1")
    gomp.omp_set_num_threads(ctypes.c_int(int(n)))


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _p(a: np.ndarray):
    return a.ctypes.data_as(_d)


# ---------------------------------------------------------------------------
# primitives
# ---------------------------------------------------------------------------
def matmul(A, B, ta: bool = False, tb: bool = False) -> np.ndarray:
    """op(A) . op(B) in fp64, op = transpose when asked; every entry is one dot
    product summed over k in increasing order (oracle.c or_gemm)."""
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    Am = np.ascontiguousarray(A.T if ta else A)          # [M, K]
    Bt = np.ascontiguousarray(B if tb else B.T)          # [N, K]
    M, K = Am.shape
    N, K2 = Bt.shape
    if K != K2:
        raise ValueError(f"inner sizes differ: {K} vs {K2}")
    C = np.empty((M, N), dtype=np.float64)
    if M and N:
        if K == 0:
            C[...] = 0.0
        else:
            _L().or_gemm(M, N, K, _p(Am), _p(Bt), _p(C))
    return C


def act(kind, z) -> np.ndarray:
    """ReLU max(z,0); GeLU z*Phi(z) (erf form); SiLU z*sigmoid(z)."""
    kind = _ACT.get(kind, kind)
    z = _f64(z)
    out = np.empty_like(z)
    if z.size:
        _L().or_act(kind, z.size, _p(z), _p(out))
    return out


def act_grad(kind, z) -> np.ndarray:
    """ReLU' = [z>0] (0 at z=0); GeLU' = Phi(z) + z*phi(z); SiLU' = sg*(1+z*(1-sg))."""
    kind = _ACT.get(kind, kind)
    z = _f64(z)
    out = np.empty_like(z)
    if z.size:
        _L().or_act_grad(kind, z.size, _p(z), _p(out))
    return out


# ---------------------------------------------------------------------------
# MLP shard: column-parallel GEMM, element-wise activation, row-parallel GEMM
# [lec16] §5.2; [book] §7.3.2 (forward) and §7.3.3 (backward)
# ---------------------------------------------------------------------------
def mlp_fwd(actk, X, W1, W2):
    """Z = X.W1(i); H = act(Z); Y(i) = H.W2(i), the partial sum g reduces."""
    Z = matmul(X, W1)
    H = act(actk, Z)
    Y = matmul(H, W2)
    return Z, H, Y


def mlp_bwd(actk, X, W1, W2, dY):
    """dH = dY.W2(i)^T; dZ = dH * act'(Z); dX(i) = dZ.W1(i)^T (the partial sum f
    reduces); dW1(i) = X^T.dZ; dW2(i) = H^T.dY.  Z is recomputed from X.W1(i)."""
    Z = matmul(X, W1)
    H = act(actk, Z)
    dH = matmul(dY, W2, tb=True)
    dZ = dH * act_grad(actk, Z)
    dX = matmul(dZ, W1, tb=True)
    dW1 = matmul(X, dZ, ta=True)
    dW2 = matmul(H, dY, ta=True)
    return dX, dW1, dW2


def mlp_fwd_rows(actk, X, W1, W2, rows):
    """mlp_fwd restricted to the given output rows (each row depends on its own X row)."""
    return mlp_fwd(actk, _f64(X)[rows], W1, W2)


def mlp_bwd_sampled(actk, X, W1, W2, dY, rows, cols1, rows2):
    """Selected entries of mlp_bwd: dX[rows,:], dW1[:,cols1], dW2[rows2,:].

    dX row r needs only dZ[r,:]; dW1 column j needs dZ[:,j] = (dY.W2[j,:]^T) *
    act'(X.W1[:,j]); dW2 row j needs H[:,j] = act(X.W1[:,j]).
    """
    X = _f64(X)
    W1 = _f64(W1)
    W2 = _f64(W2)
    dY = _f64(dY)
    Zr = matmul(X[rows], W1)
    dZr = matmul(dY[rows], W2, tb=True) * act_grad(actk, Zr)
    dX = matmul(dZr, W1, tb=True)
    W1c = np.ascontiguousarray(W1[:, cols1])
    Zc = matmul(X, W1c)
    dZc = matmul(dY, np.ascontiguousarray(W2[cols1, :]), tb=True) * act_grad(actk, Zc)
    dW1 = matmul(X, dZc, ta=True)
    Hc = act(actk, matmul(X, np.ascontiguousarray(W1[:, rows2])))
    dW2 = matmul(Hc, dY, ta=True)
    return dX, dW1, dW2


# ---------------------------------------------------------------------------
# SwiGLU shard: gate and up column-split, element-wise product on the shard,
# down row-split.  [book] §7.3.4.  Reading: A = SiLU(X.Wg) * (X.Wu), beta = 1.
# ---------------------------------------------------------------------------
def swiglu_fwd(X, Wg, Wu, Wd):
    """G = X.Wg(i); U = X.Wu(i); A = SiLU(G)*U; Y(i) = A.Wd(i)."""
    G = matmul(X, Wg)
    U = matmul(X, Wu)
    A = act(SILU, G) * U
    Y = matmul(A, Wd)
    return G, U, A, Y


def swiglu_bwd(X, Wg, Wu, Wd, dY):
    """dA = dY.Wd^T; dG = dA*U*SiLU'(G); dU = dA*SiLU(G); dWd = A^T.dY;
    dX(i) = dG.Wg^T + dU.Wu^T; dWg = X^T.dG; dWu = X^T.dU."""
    G = matmul(X, Wg)
    U = matmul(X, Wu)
    sG = act(SILU, G)
    A = sG * U
    dA = matmul(dY, Wd, tb=True)
    dG = dA * U * act_grad(SILU, G)
    dU = dA * sG
    dX = matmul(dG, Wg, tb=True) + matmul(dU, Wu, tb=True)
    dWg = matmul(X, dG, ta=True)
    dWu = matmul(X, dU, ta=True)
    dWd = matmul(A, dY, ta=True)
    return dX, dWg, dWu, dWd


def swiglu_fwd_rows(X, Wg, Wu, Wd, rows):
    return swiglu_fwd(_f64(X)[rows], Wg, Wu, Wd)


def swiglu_bwd_sampled(X, Wg, Wu, Wd, dY, rows, cols, rows_d):
    """dX[rows,:], dWg[:,cols], dWu[:,cols], dWd[rows_d,:] of swiglu_bwd."""
    X = _f64(X)
    Wg = _f64(Wg)
    Wu = _f64(Wu)
    Wd = _f64(Wd)
    dY = _f64(dY)

    def grads_at(Xs, dYs, c):
        Wgc = np.ascontiguousarray(Wg[:, c])
        Wuc = np.ascontiguousarray(Wu[:, c])
        G = matmul(Xs, Wgc)
        U = matmul(Xs, Wuc)
        dA = matmul(dYs, np.ascontiguousarray(Wd[c, :]), tb=True)
        dG = dA * U * act_grad(SILU, G)
        dU = dA * act(SILU, G)
        return Wgc, Wuc, dG, dU

    allc = np.arange(Wg.shape[1])
    Wgc, Wuc, dGr, dUr = grads_at(X[rows], dY[rows], allc)
    dX = matmul(dGr, Wgc, tb=True) + matmul(dUr, Wuc, tb=True)
    _, _, dGc, dUc = grads_at(X, dY, cols)
    dWg = matmul(X, dGc, ta=True)
    dWu = matmul(X, dUc, ta=True)
    Ac = act(SILU, matmul(X, np.ascontiguousarray(Wg[:, rows_d]))) * \
        matmul(X, np.ascontiguousarray(Wu[:, rows_d]))
    dWd = matmul(Ac, dY, ta=True)
    return dX, dWg, dWu, dWd


# ---------------------------------------------------------------------------
# attention projections, head-split: Q/K/V column-split, W_O row-split
# [book] §7.3.4; [lec16] §5.3.  The attention core between them is not part of
# the path: O (its output) and dQ/dK/dV (its input gradients) are inputs.
# ---------------------------------------------------------------------------
def attn_fwd(X, Wq, Wk, Wv, O, Wo):
    """Q = X.Wq(i); K = X.Wk(i); V = X.Wv(i); Y(i) = O.Wo(i)."""
    return matmul(X, Wq), matmul(X, Wk), matmul(X, Wv), matmul(O, Wo)


def attn_bwd(X, Wq, Wk, Wv, O, Wo, dQ, dK, dV, dY):
    """dX(i) = dQ.Wq^T + dK.Wk^T + dV.Wv^T; dW{q,k,v} = X^T.d{Q,K,V};
    dO = dY.Wo^T; dWo = O^T.dY."""
    dX = matmul(dQ, Wq, tb=True) + matmul(dK, Wk, tb=True) + matmul(dV, Wv, tb=True)
    dWq = matmul(X, dQ, ta=True)
    dWk = matmul(X, dK, ta=True)
    dWv = matmul(X, dV, ta=True)
    dO = matmul(dY, Wo, tb=True)
    dWo = matmul(O, dY, ta=True)
    return dX, dWq, dWk, dWv, dO, dWo


def attn_fwd_rows(X, Wq, Wk, Wv, O, Wo, rows):
    return attn_fwd(_f64(X)[rows], Wq, Wk, Wv, _f64(O)[rows], Wo)


def attn_bwd_sampled(X, Wq, Wk, Wv, O, Wo, dQ, dK, dV, dY, rows, cq, ckv, rows_o):
    """dX[rows], dO[rows], dWq[:,cq], dWk[:,ckv], dWv[:,ckv], dWo[rows_o,:]."""
    X, O, dQ, dK, dV, dY = map(_f64, (X, O, dQ, dK, dV, dY))
    dX = (matmul(dQ[rows], Wq, tb=True) + matmul(dK[rows], Wk, tb=True)
          + matmul(dV[rows], Wv, tb=True))
    dO = matmul(dY[rows], Wo, tb=True)
    dWq = matmul(X, np.ascontiguousarray(dQ[:, cq]), ta=True)
    dWk = matmul(X, np.ascontiguousarray(dK[:, ckv]), ta=True)
    dWv = matmul(X, np.ascontiguousarray(dV[:, ckv]), ta=True)
    dWo = matmul(np.ascontiguousarray(O[:, rows_o]), dY, ta=True)
    return dX, dWq, dWk, dWv, dO, dWo


# ---------------------------------------------------------------------------
# vocab-parallel LM head, cross entropy and embedding
# [book] §7.3.4; [lec16] §5.5
# ---------------------------------------------------------------------------
def lm_head(Hf, Wlm):
    """logits(i) = Hf.Wlm(i): the shard's [s, V/t] slice of the output layer."""
    return matmul(Hf, Wlm)


def lm_head_rows(Hf, Wlm, rows):
    return matmul(_f64(Hf)[rows], Wlm)


def ce_stats(logits, targets, vocab_start: int):
    """Per-position (max, sum exp(z - max), target logit or 0) of one shard."""
    z = _f64(logits)
    s, Vs = z.shape
    tg = np.ascontiguousarray(targets, dtype=np.int64)
    m = np.empty(s)
    se = np.empty(s)
    tl = np.empty(s)
    if s:
        _L().or_ce_stats(s, Vs, int(vocab_start), _p(z), tg.ctypes.data, _p(m), _p(se), _p(tl))
    return m, se, tl


def ce_combine(ms, ses, tls):
    """loss = M + ln(sum_i se_i exp(m_i - M)) - sum_i tl_i with M = max_i m_i:
    what the three per-position reductions across shards deliver."""
    m = _f64(np.stack(ms))
    se = _f64(np.stack(ses))
    tl = _f64(np.stack(tls))
    t, s = m.shape
    loss = np.empty(s)
    if s:
        _L().or_ce_combine(t, s, _p(m), _p(se), _p(tl), _p(loss))
    return loss


def ce_global(ms, ses):
    """The combined (M, S) per position from the shards' (m_i, se_i):
    M = max_i m_i, S = sum_i se_i exp(m_i - M) (shards with no columns add 0)."""
    m = _f64(np.stack(ms))
    se = _f64(np.stack(ses))
    M = m.max(axis=0)
    w = np.where(se > 0, se * np.exp(np.where(se > 0, m - M, 0.0)), 0.0)
    return M, w.sum(axis=0)


def ce_bwd(logits, targets, vocab_start: int, M, S, g):
    """dz = g * (exp(z - M) / S - onehot(target)) on one shard's [s, Vs] slice,
    with M, S the combined statistics and g the incoming gradient per position."""
    z = _f64(logits)
    s, Vs = z.shape
    tg = np.ascontiguousarray(targets, dtype=np.int64)
    M, S, g = (_f64(np.asarray(a)) for a in (M, S, g))
    dz = np.empty((s, Vs))
    if s and Vs:
        _L().or_ce_bwd(s, Vs, int(vocab_start), _p(z), tg.ctypes.data, _p(M), _p(S), _p(g), _p(dz))
    return dz


def ce_direct(logits_full, targets):
    """loss_r = logsumexp(z_r) - z_r[y_r] over the whole vocabulary."""
    z = _f64(logits_full)
    s, V = z.shape
    tg = np.ascontiguousarray(targets, dtype=np.int64)
    loss = np.empty(s)
    if s:
        _L().or_ce_direct(s, V, _p(z), tg.ctypes.data, _p(loss))
    return loss


def embed(ids, table, vocab_start: int):
    """out[r] = table[id_r - start] if the id is in this shard, else zeros.
    ``table`` is a 2-D array of 2- or 4-byte elements; bits are copied."""
    ids = np.ascontiguousarray(ids, dtype=np.int64)
    table = np.ascontiguousarray(table)
    Vs, h = table.shape
    n = ids.shape[0]
    out = np.empty((n, h), dtype=table.dtype)
    if n and h:
        if table.itemsize == 2:
            _L().or_embed_u16(n, Vs, h, int(vocab_start), ids.ctypes.data,
                              table.ctypes.data, out.ctypes.data)
        elif table.itemsize == 4:
            _L().or_embed_u32(n, Vs, h, int(vocab_start), ids.ctypes.data,
                              table.ctypes.data, out.ctypes.data)
        else:
            raise TypeError("table elements must be 2 or 4 bytes")
    return out


# ---------------------------------------------------------------------------
# attention core on the shard's heads
# [book] §7.3.4 (each card runs attention on its own 8 query heads and 1 KV
# head, then concatenates them to [s, 1024]); the CS336 lecture-8 book's
# activation-memory section (FlashAttention recomputes the s x s scores)
# ---------------------------------------------------------------------------
def attn_core_fwd(Q, K, V, nq: int, nkv: int, causal: bool = True, rows=None):
    """O = softmax(Q_j K_g^T / sqrt(d) + causal mask) V_g for every query head j
    (KV head g = j // (nq // nkv)), and the per-head log-sum-exp of the scores.
    Q [s, nq*d], K and V [s, nkv*d]; returns O [len(rows), nq*d] and lse
    [nq, len(rows)] (all positions when rows is None)."""
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    s = Q.shape[0]
    d = Q.shape[1] // nq
    assert Q.shape[1] == nq * d and K.shape == (s, nkv * d) and V.shape == K.shape and nq % nkv == 0
    rows = np.arange(s, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    nr = rows.shape[0]
    O = np.empty((nr, nq * d))
    lse = np.empty((nq, nr))
    if nr and d:
        _L().or_attn_fwd(s, nq, nkv, d, int(bool(causal)), _p(Q), _p(K), _p(V), nr, rows.ctypes.data,
                         _p(O), _p(lse))
    return O, lse


def attn_core_bwd(Q, K, V, dO, nq: int, nkv: int, causal: bool = True, rows=None, cols=None):
    """Gradients of attn_core_fwd's O with respect to Q, K, V for the incoming
    gradient dO [s, nq*d]: with P the attention weights of head j (KV head g),
    dP = dO_j V_g^T, dS = P * (dP - rowsum(P * dP)), dQ_j = dS K_g / sqrt(d),
    dK_g = sum over the group's heads of dS^T Q_j / sqrt(d), dV_g = sum over
    the group's heads of P^T dO_j.  Returns dQ at positions ``rows`` [nr, nq*d]
    and dK, dV at key positions ``cols`` [nc, nkv*d] (all positions when None)."""
    Q, K, V, dO = _f64(Q), _f64(K), _f64(V), _f64(dO)
    s = Q.shape[0]
    d = Q.shape[1] // nq
    assert Q.shape == dO.shape and K.shape == (s, nkv * d) and V.shape == K.shape and nq % nkv == 0
    rows = np.arange(s, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.arange(s, dtype=np.int64) if cols is None else np.ascontiguousarray(cols, dtype=np.int64)
    nr, nc = rows.shape[0], cols.shape[0]
    dQ = np.zeros((nr, nq * d))
    dK = np.zeros((nc, nkv * d))
    dV = np.zeros((nc, nkv * d))
    if s and d and nq:
        _L().or_attn_bwd(s, nq, nkv, d, int(bool(causal)), _p(Q), _p(K), _p(V), _p(dO), nr, rows.ctypes.data,
                         nc, cols.ctypes.data, _p(dQ), _p(dK), _p(dV))
    return dQ, dK, dV


# ---------------------------------------------------------------------------
# sequence-parallel region: [book] §7.3.6 (LayerNorm and dropout act on each
# position independently, so each card keeps only s/t positions between the
# reduce-scatter that ends a sublayer and the all-gather that starts the next)
# ---------------------------------------------------------------------------
LN_EPS = 1e-5


def sp_ln_fwd(y, x, mask, gamma, beta, p: float, eps: float = LN_EPS):
    """u = x + y * mask / (1 - p);  z = LayerNorm(u) * gamma + beta.
    Returns u, z [n, h] and the per-position mean and 1/sqrt(var + eps)."""
    y, x, gamma, beta = (_f64(a) for a in (y, x, gamma, beta))
    mask = np.ascontiguousarray(mask, dtype=np.uint8)
    n, h = x.shape
    u, z = np.empty((n, h)), np.empty((n, h))
    mean, rstd = np.empty(n), np.empty(n)
    if n and h:
        _L().or_sp_ln_fwd(n, h, float(p), float(eps), _p(y), _p(x), mask.ctypes.data, _p(gamma), _p(beta),
                          _p(u), _p(z), _p(mean), _p(rstd))
    return u, z, mean, rstd


def sp_ln_bwd(dz, dun, u, mean, rstd, gamma, mask, p: float):
    """Gradients of sp_ln_fwd: dx (= du, the residual input), dy (through the
    dropout), and this slice's dgamma, dbeta."""
    dz, dun, u, mean, rstd, gamma = (_f64(a) for a in (dz, dun, u, mean, rstd, gamma))
    mask = np.ascontiguousarray(mask, dtype=np.uint8)
    n, h = dz.shape
    dx, dy = np.empty((n, h)), np.empty((n, h))
    dg, db = np.zeros(h), np.zeros(h)
    if h:
        _L().or_sp_ln_bwd(n, h, float(p), _p(dz), _p(dun), _p(u), _p(mean), _p(rstd), _p(gamma),
                          mask.ctypes.data, _p(dx), _p(dy), _p(dg), _p(db))
    return dx, dy, dg, db
