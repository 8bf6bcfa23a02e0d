"""ctypes front of the oracle's fp32 canonical score arithmetic (csa.c).

Test infrastructure only.  Pages followed: "SparseLoRA: Accelerating LLM
Fine-Tuning with Contextual Sparsity" -- paper-graph summary §3.4 "SVD
Sparsity Estimator" (Algorithm 1, runtime usage) and "Oracle Sparse Neuron
Selection Criteria"; Paper-Notes page, "SVD 稀疏估计器", "L2 Norm 准则",
"QK Norm 准则".
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None
_i64 = ctypes.c_int64
_fp = ctypes.POINTER(ctypes.c_float)
_ip = ctypes.POINTER(ctypes.c_int32)


def lib():
    global _lib
    if _lib is None:
        path = _build.OUT
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_build.SRC):
            _build.build()
        L = ctypes.CDLL(path)
        L.orc_exp_sl.restype = ctypes.c_float
        L.orc_exp_sl.argtypes = [ctypes.c_float]
        L.orc_silu_sl.restype = ctypes.c_float
        L.orc_silu_sl.argtypes = [ctypes.c_float]
        L.orc_exp_sl_vec.argtypes = [_fp, _fp, _i64]
        L.orc_silu_sl_vec.argtypes = [_fp, _fp, _i64]
        L.orc_get_exp_constants11.argtypes = [_fp]
        L.orc_exp_sweep.restype = ctypes.c_double
        L.orc_exp_sweep.argtypes = [ctypes.c_uint32, ctypes.c_float, ctypes.c_float,
                                    ctypes.POINTER(_i64)]
        L.orc_r64.restype = ctypes.c_float
        L.orc_r64.argtypes = [_fp, _i64, _fp, _i64, _i64]
        L.orc_stage1.argtypes = [_fp, _i64, _ip, _i64, _i64, _fp, _i64, _fp]
        L.orc_ssq.argtypes = [ctypes.c_int, _fp, _i64, _i64, _i64, _fp, _i64, _fp, _i64, _i64, _fp]
        L.orc_qk_combine.argtypes = [_fp, _fp, _i64, _i64, _i64, _fp]
        L.orc_key.restype = ctypes.c_uint32
        L.orc_key.argtypes = [ctypes.c_float]
        L.orc_select.restype = _i64
        L.orc_select.argtypes = [_fp, _i64, _i64, _ip]
        _lib = L
    return _lib


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _p(a, t=_fp):
    return a.ctypes.data_as(t)


def exp_constants():
    """(LOG2E, LN2_HI, LN2_LO, C0..C7) as derived by the oracle."""
    out = np.zeros(11, np.float32)
    lib().orc_get_exp_constants11(_p(out))
    return out


def exp_sl(z):
    z = _f32(z)
    out = np.empty_like(z)
    lib().orc_exp_sl_vec(_p(z), _p(out), z.size)
    return out


def silu_sl(z):
    z = _f32(z)
    out = np.empty_like(z)
    lib().orc_silu_sl_vec(_p(z), _p(out), z.size)
    return out


def exp_sweep(stride=61, lo=-104.0, hi=89.0):
    cnt = _i64(0)
    worst = lib().orc_exp_sweep(stride, lo, hi, ctypes.byref(cnt))
    return worst, cnt.value


def r64(a, b):
    a, b = _f32(a), _f32(b)
    assert a.shape == b.shape and a.ndim == 1
    return np.float32(lib().orc_r64(_p(a), 1, _p(b), 1, a.size))


def stage1(x, ctx_rows, WA_t):
    """Estimator stage 1: xa[m, j] = R64_i(x[ctx_rows[m], i], W_A[i, j]).

    x: [T, D_in] values (bf16 values widened exactly, or fp32); WA_t: [k_tot, D_in].
    Returns xa [T_c, k_tot] fp32.  Pinned by tests/test_oracle_score.py."""
    x, WA_t = _f32(x), _f32(WA_t)
    rows = np.ascontiguousarray(ctx_rows, dtype=np.int32)
    T_c, D = rows.size, x.shape[1]
    k_tot = WA_t.shape[0]
    assert WA_t.shape[1] == D
    xa = np.zeros((T_c, k_tot), np.float32)
    lib().orc_stage1(_p(x), x.shape[1], _p(rows, _ip), T_c, D, _p(WA_t), k_tot, _p(xa))
    return xa


def ssq_l2(xa, WB, off=0):
    """Per-channel sum over context tokens of y_hat^2 (R64 order); y_hat from
    xa[:, off:off+k] and WB [k, C].  Pinned by tests/test_oracle_score.py."""
    xa, WB = _f32(xa), _f32(WB)
    k, C = WB.shape
    out = np.zeros(C, np.float32)
    lib().orc_ssq(0, _p(xa), xa.shape[1], xa.shape[0], off, _p(WB), 0, _p(WB), k, C, _p(out))
    return out


def ssq_swiglu(xa, WB_gate, WB_up, off_gate=0, off_up=None):
    """FFN criterion: per-channel sum over context tokens of
    (silu_sl(g_hat) * u_hat)^2 (R64 order).  Pinned by tests/test_oracle_score.py."""
    xa, WBg, WBu = _f32(xa), _f32(WB_gate), _f32(WB_up)
    k, C = WBg.shape
    if off_up is None:
        off_up = off_gate + k
    out = np.zeros(C, np.float32)
    lib().orc_ssq(1, _p(xa), xa.shape[1], xa.shape[0], off_gate, _p(WBg), off_up, _p(WBu),
                  k, C, _p(out))
    return out


def qk_combine(ssqQ, ssqK, n_kv_heads, n_rep, head_dim):
    """QK criterion in key/value channel space: (sum over the group's query heads
    of ssqQ) * ssqK.  Pinned by tests/test_oracle_score.py."""
    ssqQ, ssqK = _f32(ssqQ), _f32(ssqK)
    assert ssqQ.size == n_kv_heads * n_rep * head_dim and ssqK.size == n_kv_heads * head_dim
    out = np.zeros(ssqK.size, np.float32)
    lib().orc_qk_combine(_p(ssqQ), _p(ssqK), n_kv_heads, n_rep, head_dim, _p(out))
    return out


def keys(scores):
    s = _f32(scores)
    u = s.view(np.uint32).copy()
    u[np.isnan(s)] = 0x7FC00000
    return u


def select(scores, n):
    """Top-n channels by key (ties: lower index first), ascending.
    Pinned by tests/test_oracle_select.py."""
    s = _f32(scores)
    C = s.size
    n = int(n)
    if not 0 <= n <= C:
        raise ValueError(f"n_keep={n} outside [0, {C}]")
    idx = np.zeros(max(n, 1), np.int32)
    cnt = lib().orc_select(_p(s), C, n, _p(idx, _ip))
    assert cnt == n
    return idx[:n].copy()


def select_ffn(x, ctx_rows, WA_t_gu, WB_gate, WB_up, n):
    """FFN group selection: estimator on the context rows of the group input,
    SwiGLU-L2 scores, top-n (paper-graph summary §3.4, Algorithm 1 steps 1-3)."""
    k = WB_gate.shape[0]
    xa = stage1(x, ctx_rows, WA_t_gu)
    return select(ssq_swiglu(xa, WB_gate, WB_up, 0, k), n)


def select_attn(x, ctx_rows, WA_t_qkv, WB_q, WB_k, WB_v, n_kv_heads, n_rep, head_dim, n_qk, n_vo):
    """Attention group selections (QK criterion, VO criterion) from one
    estimator pass over the context rows of the group input."""
    k = WB_q.shape[0]
    xa = stage1(x, ctx_rows, WA_t_qkv)
    sq, sk = ssq_l2(xa, WB_q, off=0), ssq_l2(xa, WB_k, off=k)
    idx_qk = select(qk_combine(sq, sk, n_kv_heads, n_rep, head_dim), n_qk)
    idx_vo = select(ssq_l2(xa, WB_v, off=2 * k), n_vo)
    return idx_qk, idx_vo


# ---------------------------------------------------------------- criterion variants
# Paper-graph summary §3.4 "Oracle Sparse Neuron Selection Criteria" (the
# criteria on exact outputs, the oracle row of Table 7), "Why not head-level
# pruning for QK?" and the pruning-criterion ablation of Table 10 (random,
# head-level).


def dense_ssq(crit, Y0, Y1, rows):
    """Criterion on exact outputs: v = Y0[rows] ("l2") or
    silu_sl(Y0[rows]) * Y1[rows] ("swiglu", one fp32 rounding of the product);
    ssq[c] = R64 over the listed rows of (v[:, c], v[:, c])."""
    rows = np.asarray(rows, np.int64)
    v = _f32(np.asarray(Y0, np.float32)[rows])
    if crit == "swiglu":
        v = _f32(silu_sl(v) * np.asarray(Y1, np.float32)[rows])
    T_c, C = v.shape
    out = np.zeros(C, np.float32)
    for c in range(C):
        col = np.ascontiguousarray(v[:, c])
        out[c] = np.float32(lib().orc_r64(_p(col), 1, _p(col), 1, T_c))
    return out


def dense_scores(crit, Y0, Y1, rows, n_kv_heads=1, n_rep=1, head_dim=1):
    """Scores of the exact ("oracle") criterion: L2 and SwiGLU-L2 as dense_ssq;
    QK from Q = Y0 and K = Y1 through qk_combine."""
    if crit == "qk":
        return qk_combine(dense_ssq("l2", Y0, None, rows), dense_ssq("l2", Y1, None, rows),
                          n_kv_heads, n_rep, head_dim)
    return dense_ssq(crit, Y0, Y1, rows)


def head_scores(scores, n_heads, head_dim):
    """hs[g] = sum over j < head_dim of scores[g head_dim + j], fp32 adds with j
    ascending from +0."""
    s = _f32(scores).reshape(n_heads, head_dim)
    hs = np.zeros(n_heads, np.float32)
    for j in range(head_dim):
        hs = (hs + s[:, j]).astype(np.float32)
    return hs


def select_heads(scores, n_heads, head_dim, heads_keep):
    """Head-level selection: the heads_keep heads with the largest head score
    (rule of ``select``) keep every channel; channels ascending."""
    heads = select(head_scores(scores, n_heads, head_dim), heads_keep)
    return (heads[:, None] * head_dim + np.arange(head_dim)[None, :]).reshape(-1).astype(np.int32)


_GAMMA = np.uint64(0x9E3779B97F4A7C15)


def random_scores(seed, C):
    """Uniform scores for the random-selection ablation: score[c] = top 24 bits
    of the (c + 1)-th SplitMix64 output from state ``seed`` (Steele, Lea and
    Flood, 2014), times 2^-24."""
    with np.errstate(over="ignore"):
        z = np.uint64(seed) + np.arange(1, C + 1, dtype=np.uint64) * _GAMMA
        z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
        z = z ^ (z >> np.uint64(31))
    return ((z >> np.uint64(40)).astype(np.float64) * 2.0 ** -24).astype(np.float32)
