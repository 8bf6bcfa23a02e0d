"""Seeded generators of the synthetic inputs.

Recipe (the same for every configuration):
  * numpy ``Generator(PCG64)``; one child stream per tensor, spawned from
    ``SeedSequence(cfg.seed)`` in the fixed order of ``_FFN_ORDER`` /
    ``_ATTN_ORDER`` / ``_LAYER_ORDER``;
  * frozen weights and LoRA factors ~ N(0, 0.02^2), rounded to the
    configuration's dtype (bf16 round-to-nearest-even, or fp32);
  * linear inputs: N(0, 1) per element, then each row scaled to unit RMS
    (x / sqrt(mean(x^2) + 1e-5)), then rounded to the dtype;
  * upstream gradient dy ~ N(0, 1) on every row, rounded to the dtype;
  * token roles: the last ``out_per_seq`` tokens of each sequence are output
    tokens (role 1), the rest are context tokens (role 0);
  * estimator factors: the rank-k truncated SVD of the dtype-rounded frozen
    weight, computed in fp64 and stored in fp32 (``svd_factor_pair``).  The
    pages compute these offline and load them with the weights; here they are
    part of the input set, produced once per weight.
No method arithmetic lives here.
"""
import numpy as np

from .configs import Config

_FFN_ORDER = ["x", "W_gate", "W_up", "W_down", "A_gate", "B_gate", "A_up", "B_up",
              "A_down", "B_down", "dy"]
_ATTN_ORDER = ["x", "W_q", "W_k", "W_v", "W_o", "A_q", "B_q", "A_k", "B_k", "A_v", "B_v",
               "A_o", "B_o", "x_o", "dy_q", "dy_k", "dy_v", "dy_o"]
_LAYER_ORDER = ["x", "W_q", "W_k", "W_v", "W_o", "W_gate", "W_up", "W_down",
                "A_q", "B_q", "A_k", "B_k", "A_v", "B_v", "A_o", "B_o",
                "A_gate", "B_gate", "A_up", "B_up", "A_down", "B_down", "dy"]


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even); returns uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    if np.isfinite(a).all():
        # finite bit patterns are at most 0xFF7FFFFF, so adding at most 0x8000
        # cannot wrap in 32 bits
        u = a.view(np.uint32)
        t = (u >> 16) & 1
        t += 0x7FFF
        t += u
        t >>= 16
        return t.astype(np.uint16)
    u = a.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32 values."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def round_dtype(a: np.ndarray, dtype: str) -> np.ndarray:
    """fp32 array whose values are representable in ``dtype``."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    if dtype == "bf16":
        return bf16_bits_to_f32(f32_to_bf16_bits(a))
    if dtype == "f32":
        return a
    raise ValueError(dtype)


def _streams(seed: int, names):
    kids = np.random.SeedSequence(seed).spawn(len(names))
    return {n: np.random.Generator(np.random.PCG64(s)) for n, s in zip(names, kids)}


def _normal(rng, shape, std, dtype):
    return round_dtype(rng.standard_normal(shape, dtype=np.float32) * np.float32(std), dtype)


def _rms_rows(rng, shape, dtype):
    x = rng.standard_normal(shape, dtype=np.float32)
    ms = np.mean(x.astype(np.float64) ** 2, axis=-1, keepdims=True)
    return round_dtype((x / np.sqrt(ms + 1e-5)).astype(np.float32), dtype)


def roles_for(cfg: Config) -> np.ndarray:
    """uint8[T]: 1 = output token (dense path), 0 = context token."""
    r = np.zeros((cfg.batch, cfg.seq), dtype=np.uint8)
    if cfg.out_per_seq:
        r[:, cfg.seq - cfg.out_per_seq:] = 1
    return r.reshape(-1)


def svd_factor_pair(W_lin: np.ndarray, k: int):
    """Rank-k estimator factors of a frozen weight given in nn.Linear layout
    [D_out, D_in] (so the math-layout weight is W = W_lin^T, y = x W).

    With W = U diag(s) V^T: W_A = U[:, :k] diag(sqrt(s_k)) and
    W_B = diag(sqrt(s_k)) V[:, :k]^T.  Returns (W_A^T [k, D_in], W_B [k, D_out]),
    both fp32.  Each singular pair is signed so that the largest-magnitude
    entry of its left vector is positive.
    """
    Wm = np.asarray(W_lin, dtype=np.float64).T          # [D_in, D_out]
    d_in, d_out = Wm.shape
    if min(d_in, d_out) <= 2048 or k > 64:
        U, s, Vt = np.linalg.svd(Wm, full_matrices=False)
        U, s, V = U[:, :k], s[:k], Vt[:k].T
    else:
        import scipy.linalg as sla
        if d_in <= d_out:
            w, U = sla.eigh(Wm @ Wm.T, subset_by_index=[d_in - k, d_in - 1])
            U, w = U[:, ::-1], w[::-1]
            s = np.sqrt(np.maximum(w, 0.0))
            V = (Wm.T @ U) / s
        else:
            w, V = sla.eigh(Wm.T @ Wm, subset_by_index=[d_out - k, d_out - 1])
            V, w = V[:, ::-1], w[::-1]
            s = np.sqrt(np.maximum(w, 0.0))
            U = (Wm @ V) / s
    sign = np.sign(U[np.argmax(np.abs(U), axis=0), np.arange(U.shape[1])])
    sign[sign == 0] = 1.0
    U, V = U * sign, V * sign
    rs = np.sqrt(s)
    WA_t = (U * rs).T.astype(np.float32)
    WB = (rs[:, None] * V.T).astype(np.float32)
    return np.ascontiguousarray(WA_t), np.ascontiguousarray(WB)


def make_ffn_inputs(cfg: Config, with_factors: bool = True) -> dict:
    """Inputs of one SwiGLU FFN block (gate/up/down) with LoRA on all three."""
    D, F, r, T, dt = cfg.hidden, cfg.inter, cfg.lora_rank, cfg.tokens, cfg.dtype
    g = _streams(cfg.seed, _FFN_ORDER)
    out = {
        "x": _rms_rows(g["x"], (T, D), dt),
        "W_gate": _normal(g["W_gate"], (F, D), 0.02, dt),
        "W_up": _normal(g["W_up"], (F, D), 0.02, dt),
        "W_down": _normal(g["W_down"], (D, F), 0.02, dt),
        "A_gate": _normal(g["A_gate"], (r, D), 0.02, dt),
        "B_gate": _normal(g["B_gate"], (F, r), 0.02, dt),
        "A_up": _normal(g["A_up"], (r, D), 0.02, dt),
        "B_up": _normal(g["B_up"], (F, r), 0.02, dt),
        "A_down": _normal(g["A_down"], (r, F), 0.02, dt),
        "B_down": _normal(g["B_down"], (D, r), 0.02, dt),
        "dy": _normal(g["dy"], (T, D), 1.0, dt),
        "roles": roles_for(cfg),
        "scale": cfg.lora_scale,
    }
    if with_factors:
        k = cfg.est_rank
        WA_g, WB_g = svd_factor_pair(out["W_gate"], k)
        WA_u, WB_u = svd_factor_pair(out["W_up"], k)
        out["WA_t_gu"] = np.ascontiguousarray(np.concatenate([WA_g, WA_u], axis=0))
        out["WB_gate"], out["WB_up"] = WB_g, WB_u
    return out


def make_attn_inputs(cfg: Config, with_factors: bool = True) -> dict:
    """Inputs of the q/k/v/o projections (GQA when n_kv_heads < n_q_heads).

    The o-projection's input ``x_o`` is an independent unit-RMS tensor (there
    is no attention core between the projections in this workload)."""
    D, r, T, dt = cfg.hidden, cfg.lora_rank, cfg.tokens, cfg.dtype
    Cq, Ckv = cfg.n_q_heads * cfg.head_dim, cfg.n_kv_heads * cfg.head_dim
    g = _streams(cfg.seed, _ATTN_ORDER)
    out = {
        "x": _rms_rows(g["x"], (T, D), dt),
        "W_q": _normal(g["W_q"], (Cq, D), 0.02, dt),
        "W_k": _normal(g["W_k"], (Ckv, D), 0.02, dt),
        "W_v": _normal(g["W_v"], (Ckv, D), 0.02, dt),
        "W_o": _normal(g["W_o"], (D, Cq), 0.02, dt),
        "x_o": _rms_rows(g["x_o"], (T, Cq), dt),
        "roles": roles_for(cfg),
        "scale": cfg.lora_scale,
    }
    for p, (cin, cout) in {"q": (D, Cq), "k": (D, Ckv), "v": (D, Ckv), "o": (Cq, D)}.items():
        out["A_" + p] = _normal(g["A_" + p], (r, cin), 0.02, dt)
        out["B_" + p] = _normal(g["B_" + p], (cout, r), 0.02, dt)
    out["dy_q"] = _normal(g["dy_q"], (T, Cq), 1.0, dt)
    out["dy_k"] = _normal(g["dy_k"], (T, Ckv), 1.0, dt)
    out["dy_v"] = _normal(g["dy_v"], (T, Ckv), 1.0, dt)
    out["dy_o"] = _normal(g["dy_o"], (T, D), 1.0, dt)
    if with_factors:
        k = cfg.est_rank
        fa = {p: svd_factor_pair(out["W_" + p], k) for p in ("q", "k", "v")}
        out["WA_t_qkv"] = np.ascontiguousarray(np.concatenate([fa[p][0] for p in "qkv"], axis=0))
        for p in "qkv":
            out["WB_" + p] = fa[p][1]
    return out


def make_layer_inputs(cfg: Config, with_factors: bool = True, seed: int = None) -> dict:
    """Inputs of one decoder layer: attention projections (GQA when
    n_kv_heads < n_q_heads) and a SwiGLU FFN, LoRA on all seven linears, the
    layer input x and the upstream gradient dy.  ``seed`` overrides
    ``cfg.seed`` (one seed per layer of a stack)."""
    D, F, r, T, dt = cfg.hidden, cfg.inter, cfg.lora_rank, cfg.tokens, cfg.dtype
    Cq, Ckv = cfg.n_q_heads * cfg.head_dim, cfg.n_kv_heads * cfg.head_dim
    g = _streams(cfg.seed if seed is None else seed, _LAYER_ORDER)
    shapes = {"W_q": (Cq, D), "W_k": (Ckv, D), "W_v": (Ckv, D), "W_o": (D, Cq),
              "W_gate": (F, D), "W_up": (F, D), "W_down": (D, F)}
    out = {"x": _rms_rows(g["x"], (T, D), dt), "roles": roles_for(cfg), "scale": cfg.lora_scale,
           "dy": _normal(g["dy"], (T, D), 1.0, dt)}
    for name, shp in shapes.items():
        out[name] = _normal(g[name], shp, 0.02, dt)
        p = name[2:]
        out["A_" + p] = _normal(g["A_" + p], (r, shp[1]), 0.02, dt)
        out["B_" + p] = _normal(g["B_" + p], (shp[0], r), 0.02, dt)
    if with_factors:
        k = cfg.est_rank
        fa = {p: svd_factor_pair(out["W_" + p], k) for p in ("q", "k", "v", "gate", "up")}
        out["WA_t_qkv"] = np.ascontiguousarray(np.concatenate([fa[p][0] for p in "qkv"], axis=0))
        out["WA_t_gu"] = np.ascontiguousarray(np.concatenate([fa["gate"][0], fa["up"][0]], axis=0))
        for p in ("q", "k", "v", "gate", "up"):
            out["WB_" + p] = fa[p][1]
    return out


# ---------------------------------------------------------------- 32-layer stack
#
# The stack has 32 layers of LLaMA3-8B shape (7 weights of up to 14336 x 4096
# per layer), too many for the exact fp64 SVD above in a test's time.  Its
# recipe differs in two documented ways:
#   * each layer's tensors come from child streams of SeedSequence((seed,
#     layer)) in ``_STACK_LAYER_ORDER`` and are drawn on a thread pool;
#   * its estimator factors are the rank-k truncated SVD from a seeded
#     randomized subspace iteration (``svd_factor_pair_subspace``), i.e. an
#     approximate, not the exact, top-k singular subspace.
# Stack input x: unit-RMS rows; upstream gradient at the top: N(0, 1) on
# output rows and 0 on context rows (the loss is taken on output tokens).

_STACK_LAYER_ORDER = _LAYER_ORDER[1:-1] + ["omega_q", "omega_k", "omega_v", "omega_gate", "omega_up"]


def svd_factor_pair_subspace(W_lin: np.ndarray, k: int, rng, oversample: int = 16, iters: int = 3):
    """Rank-k estimator factors from a randomized subspace iteration (Halko,
    Martinsson and Tropp 2011, Algorithms 4.4 and 5.1) on W = W_lin^T, in fp32:
    Q spans W Omega refined by ``iters`` power steps with re-orthonormalisation,
    then the SVD of the small matrix Q^T W.  Same output convention and sign
    rule as ``svd_factor_pair``."""
    Wm = np.asarray(W_lin, dtype=np.float32).T          # [D_in, D_out]
    d_in, d_out = Wm.shape
    p = min(k + oversample, d_in, d_out)
    Om = rng.standard_normal((d_out, p), dtype=np.float32)
    Q, _ = np.linalg.qr(Wm @ Om)
    for _ in range(iters):
        Z, _ = np.linalg.qr(Wm.T @ Q)
        Q, _ = np.linalg.qr(Wm @ Z)
    Ub, s, Vt = np.linalg.svd((Q.T @ Wm).astype(np.float64), full_matrices=False)
    U = Q.astype(np.float64) @ Ub[:, :k]
    s, V = s[:k], Vt[:k].T
    sign = np.sign(U[np.argmax(np.abs(U), axis=0), np.arange(U.shape[1])])
    sign[sign == 0] = 1.0
    U, V = U * sign, V * sign
    rs = np.sqrt(s)
    return (np.ascontiguousarray((U * rs).T.astype(np.float32)),
            np.ascontiguousarray((rs[:, None] * V.T).astype(np.float32)))


def make_stack_io(cfg: Config) -> dict:
    """Stack input x, top-of-stack upstream gradient dy, roles and scale."""
    D, T, dt = cfg.hidden, cfg.tokens, cfg.dtype
    g = _streams(cfg.seed, ["x", "dy"])
    roles = roles_for(cfg)
    dy = _normal(g["dy"], (T, D), 1.0, dt)
    dy[roles == 0] = 0.0
    return {"x": _rms_rows(g["x"], (T, D), dt), "dy": dy, "roles": roles, "scale": cfg.lora_scale}


def make_stack_layer(cfg: Config, layer: int, with_factors: bool = True, workers: int = 16) -> dict:
    """Weights, LoRA factors and estimator factors of one layer of the stack."""
    from concurrent.futures import ThreadPoolExecutor
    D, F, r, dt = cfg.hidden, cfg.inter, cfg.lora_rank, cfg.dtype
    Cq, Ckv = cfg.n_q_heads * cfg.head_dim, cfg.n_kv_heads * cfg.head_dim
    kids = np.random.SeedSequence((cfg.seed, layer)).spawn(len(_STACK_LAYER_ORDER))
    g = {n: np.random.Generator(np.random.PCG64(s)) for n, s in zip(_STACK_LAYER_ORDER, kids)}
    shapes = {"W_q": (Cq, D), "W_k": (Ckv, D), "W_v": (Ckv, D), "W_o": (D, Cq),
              "W_gate": (F, D), "W_up": (F, D), "W_down": (D, F)}
    jobs = {}
    for name, shp in shapes.items():
        p = name[2:]
        jobs[name] = shp
        jobs["A_" + p] = (r, shp[1])
        jobs["B_" + p] = (shp[0], r)
    with ThreadPoolExecutor(max_workers=workers) as ex:
        futs = {n: ex.submit(_normal, g[n], shp, 0.02, dt) for n, shp in jobs.items()}
        out = {n: f.result() for n, f in futs.items()}
        if with_factors:
            k = cfg.est_rank
            ff = {p: ex.submit(svd_factor_pair_subspace, out["W_" + p], k, g["omega_" + p])
                  for p in ("q", "k", "v", "gate", "up")}
            fa = {p: f.result() for p, f in ff.items()}
            out["WA_t_qkv"] = np.ascontiguousarray(np.concatenate([fa[p][0] for p in "qkv"], axis=0))
            out["WA_t_gu"] = np.ascontiguousarray(np.concatenate([fa["gate"][0], fa["up"][0]], axis=0))
            for p in ("q", "k", "v", "gate", "up"):
                out["WB_" + p] = fa[p][1]
    out["roles"], out["scale"] = roles_for(cfg), cfg.lora_scale
    return out
