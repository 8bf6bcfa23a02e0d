"""CPU oracle, fp64 part: the plain definitions of the sparse main branch, the
dense LoRA branch, SwiGLU and the FFN block.

TEST INFRASTRUCTURE ONLY (tests, smoke check, CPU-baseline leg of the benchmark).

Pages followed, all titled "SparseLoRA: Accelerating LLM Fine-Tuning with
Contextual Sparsity":
  * paper-graph summary §3.4, "Preliminary: What channel sparsity means
    structurally": y = x W with W in R^{D_in x D_out}; channel sparsity keeps a
    subset of the D_out output channels and the dropped channels are zero;
  * §3.4 "FFN structure ... cascaded sparsity": h = SiLU(x W_gate) * (x W_up),
    y = h W_down; channel i of h is one column of W_gate and W_up and one row
    of W_down, so the down projection's selection is reused for gate and up;
  * §3.4 "VO projection sparsity": the selection propagates to W_V;
  * §3.4 Algorithm 1 steps 4-6: slice, multiply, add the dense LoRA output BAx;
  * §3.4 "Token Sensitivity", implementation (Figure 8): output tokens take the
    dense path, context tokens the sparse path, results merged at their
    original positions, LoRA added for every position;
  * §3.2 "Information flow during a backward pass": gradients flow only through
    the channels active in the forward pass; LoRA gradients are dense; the
    frozen weights receive no gradient;
  * Paper-Notes page, "整体框架" (same structure) and "Token 敏感性".

Weights are in nn.Linear layout [D_out, D_in] (y = x W_lin^T).  "Output-side"
sparsity (gate, up, q, k, v) selects output features; "input-side" sparsity
(down, o) selects input features.  Everything is computed in float64 from
the given values; the selection (an integer result) comes from ``csa``.
The masked-dense formulation below is the plain definition: it multiplies by
a 0/1 mask instead of gathering, so a reader can check it against the pages.
"""
from fractions import Fraction

import numpy as np

f64 = np.float64


def token_lists(roles):
    """Context rows (role 0) and output rows (role 1), each ascending.
    Pinned: tests/test_oracle_dense.py::test_token_lists (brute force)."""
    r = np.asarray(roles).reshape(-1)
    return (np.nonzero(r == 0)[0].astype(np.int32), np.nonzero(r != 0)[0].astype(np.int32))


def n_keep(C, num, den):
    """Number of kept channels at sparsity num/den: ceil(C * (1 - num/den)),
    formed exactly (paper-graph summary §3.4 Algorithm 1 step 3: the top
    ceil(r * D_out) channels, r = keep ratio).
    Pinned: tests/test_oracle_dense.py::test_n_keep (Fraction + golden table)."""
    C, num, den = int(C), int(num), int(den)
    assert 0 <= num <= den and den > 0
    return (C * (den - num) + den - 1) // den


def expand_gqa(idx_kv, n_rep, head_dim):
    """Key/value-space selection -> query (or o-input) channel selection:
    query channel h*d + j is kept iff key/value channel (h // n_rep)*d + j is.
    Ascending output.  Pinned: tests/test_oracle_dense.py::test_expand_gqa."""
    idx_kv = np.asarray(idx_kv, dtype=np.int64)
    g, j = idx_kv // head_dim, idx_kv % head_dim
    out = [(g * n_rep + r) * head_dim + j for r in range(n_rep)]
    return np.sort(np.concatenate(out)).astype(np.int32) if out else np.zeros(0, np.int32)


def keep_mask(T, C, roles, idx):
    """M[t, c] = 1 if token t is an output token or channel c is selected."""
    sel = np.zeros(C, dtype=bool)
    sel[np.asarray(idx, dtype=np.int64)] = True
    out = (np.asarray(roles).reshape(-1) != 0)
    return (out[:T, None] | sel[None, :]).astype(f64)


def sparse_linear_fwd(side, x, W, roles, idx):
    """Main-branch forward, masked dense.
    side "out": y[t, c] = sum_i x[t, i] W[c, i], set to 0 for context t and
                unselected c.
    side "in" : y[t, o] = sum_{c kept for t} x[t, c] W[o, c], kept = all c for
                output tokens and the selected c for context tokens.
    Pinned: tests/test_oracle_dense.py (sparsity 0 = dense; sliced = masked;
    output rows invariant under the selection; adjoint identity with bwd)."""
    x, W = np.asarray(x, f64), np.asarray(W, f64)
    T = x.shape[0]
    if side == "out":
        return (x @ W.T) * keep_mask(T, W.shape[0], roles, idx)
    if side == "in":
        return (x * keep_mask(T, W.shape[1], roles, idx)) @ W.T
    raise ValueError(side)


def sparse_linear_bwd(side, dy, W, roles, idx):
    """Input gradient of ``sparse_linear_fwd`` with the selection held fixed
    (the adjoint of the same masked linear map); the frozen W gets none.
    side "out": dx = (dy * M) W;  side "in": dx = (dy W) * M.
    Pinned: adjoint identity and torch.autograd in tests/test_oracle_dense.py."""
    dy, W = np.asarray(dy, f64), np.asarray(W, f64)
    T = dy.shape[0]
    if side == "out":
        return (dy * keep_mask(T, W.shape[0], roles, idx)) @ W
    if side == "in":
        return (dy @ W) * keep_mask(T, W.shape[1], roles, idx)
    raise ValueError(side)


def lora_fwd(x, A, B, scale):
    """Dense LoRA branch: xl = x A^T, y_lora = scale * xl B^T (every token and
    every channel).  A: [r, D_in], B: [D_out, r].  Returns (xl, y_lora)."""
    x, A, B = np.asarray(x, f64), np.asarray(A, f64), np.asarray(B, f64)
    xl = x @ A.T
    return xl, scale * (xl @ B.T)


def lora_bwd(x, xl, dy, A, B, scale):
    """Gradients of the LoRA branch: gB = dy B; dA = scale gB^T x;
    dB = scale dy^T xl; dx = scale gB A.  Returns (dx, dA, dB).
    Pinned: finite differences and torch.autograd in tests/test_oracle_dense.py."""
    x, xl, dy = np.asarray(x, f64), np.asarray(xl, f64), np.asarray(dy, f64)
    A, B = np.asarray(A, f64), np.asarray(B, f64)
    gB = dy @ B
    return scale * (gB @ A), scale * (gB.T @ x), scale * (dy.T @ xl)


def silu(z):
    z = np.asarray(z, f64)
    return z / (1.0 + np.exp(-z))


def swiglu_fwd(g, u):
    """h = SiLU(g) * u (paper-graph summary §3.4, FFN structure)."""
    return silu(g) * np.asarray(u, f64)


def swiglu_bwd(dh, g, u):
    """dg = dh * u * SiLU'(g), du = dh * SiLU(g), SiLU'(z) = s (1 + z (1 - s)),
    s = sigmoid(z)."""
    dh, g, u = np.asarray(dh, f64), np.asarray(g, f64), np.asarray(u, f64)
    s = 1.0 / (1.0 + np.exp(-g))
    return dh * u * (s * (1.0 + g * (1.0 - s))), dh * (g * s)


def ffn_block_fwd(inp, idx, g_u=None):
    """Forward of one sparse SwiGLU FFN block with LoRA on gate, up, down.
    idx: selected intermediate channels (shared by gate, up and down).
    ``g_u`` optionally overrides (g, u) with given values (per-op checks)."""
    x, roles, s = inp["x"], inp["roles"], inp["scale"]
    out = {}
    if g_u is None:
        xl_g, lg = lora_fwd(x, inp["A_gate"], inp["B_gate"], s)
        xl_u, lu = lora_fwd(x, inp["A_up"], inp["B_up"], s)
        g = sparse_linear_fwd("out", x, inp["W_gate"], roles, idx) + lg
        u = sparse_linear_fwd("out", x, inp["W_up"], roles, idx) + lu
        out.update(xl_gate=xl_g, xl_up=xl_u)
    else:
        g, u = (np.asarray(a, f64) for a in g_u)
    h = swiglu_fwd(g, u)
    xl_d, ld = lora_fwd(h, inp["A_down"], inp["B_down"], s)
    y = sparse_linear_fwd("in", h, inp["W_down"], roles, idx) + ld
    out.update(g=g, u=u, h=h, xl_down=xl_d, y=y)
    return out


def ffn_block_bwd(inp, fwd, idx, dy=None):
    """Backward of ``ffn_block_fwd`` for upstream gradient dy (default inp["dy"]):
    input gradient dx and the six LoRA gradients; no frozen-weight gradient."""
    x, roles, s = inp["x"], inp["roles"], inp["scale"]
    dy = inp["dy"] if dy is None else dy
    dh_l, dA_d, dB_d = lora_bwd(fwd["h"], fwd["xl_down"], dy, inp["A_down"], inp["B_down"], s)
    dh = sparse_linear_bwd("in", dy, inp["W_down"], roles, idx) + dh_l
    dg, du = swiglu_bwd(dh, fwd["g"], fwd["u"])
    dx_g, dA_g, dB_g = lora_bwd(x, fwd["xl_gate"], dg, inp["A_gate"], inp["B_gate"], s)
    dx_u, dA_u, dB_u = lora_bwd(x, fwd["xl_up"], du, inp["A_up"], inp["B_up"], s)
    dx = (sparse_linear_bwd("out", dg, inp["W_gate"], roles, idx)
          + sparse_linear_bwd("out", du, inp["W_up"], roles, idx) + dx_g + dx_u)
    return dict(dh=dh, dg=dg, du=du, dx=dx, dA_gate=dA_g, dB_gate=dB_g, dA_up=dA_u,
                dB_up=dB_u, dA_down=dA_d, dB_down=dB_d)


def attn_proj_indices(idx_qk, idx_vo, n_rep, head_dim):
    """Per-projection channel selections of the q/k/v/o projections from the two
    key/value-space selections (paper-graph summary §3.4 "QK projection
    sparsity": q and k keep the same channels, here the key channels and their
    query-head expansion under GQA; "VO projection sparsity": v keeps the
    selected value channels and o the same channels on its input side, which
    runs over the query heads).  Returns dict q, k, v (output side) and o
    (input side)."""
    return {"q": expand_gqa(idx_qk, n_rep, head_dim), "k": np.asarray(idx_qk, np.int32),
            "v": np.asarray(idx_vo, np.int32), "o": expand_gqa(idx_vo, n_rep, head_dim)}


def attn_proj_fwd(inp, idx_qk, idx_vo, n_rep, head_dim):
    """Forward of the sparse q, k, v (output side, input x) and o (input side,
    input x_o) projections with dense LoRA on all four (Algorithm 1 steps 4-6,
    "Token Sensitivity": output tokens dense)."""
    x, xo, roles, s = inp["x"], inp["x_o"], inp["roles"], inp["scale"]
    sel = attn_proj_indices(idx_qk, idx_vo, n_rep, head_dim)
    out = {}
    for p in "qkv":
        xl, lp = lora_fwd(x, inp["A_" + p], inp["B_" + p], s)
        out[p] = sparse_linear_fwd("out", x, inp["W_" + p], roles, sel[p]) + lp
        out["xl_" + p] = xl
    xl, lo = lora_fwd(xo, inp["A_o"], inp["B_o"], s)
    out["o"] = sparse_linear_fwd("in", xo, inp["W_o"], roles, sel["o"]) + lo
    out["xl_o"] = xl
    return out


def attn_proj_bwd(inp, fwd, idx_qk, idx_vo, n_rep, head_dim):
    """Backward of ``attn_proj_fwd`` for upstream gradients dy_q, dy_k, dy_v,
    dy_o: dx (sum over q, k, v), dx_o, and the LoRA gradients of all four."""
    x, xo, roles, s = inp["x"], inp["x_o"], inp["roles"], inp["scale"]
    sel = attn_proj_indices(idx_qk, idx_vo, n_rep, head_dim)
    res = {}
    dx = np.zeros(np.shape(x), f64)
    for p in "qkv":
        dy = inp["dy_" + p]
        dxl, dA, dB = lora_bwd(x, fwd["xl_" + p], dy, inp["A_" + p], inp["B_" + p], s)
        dx = dx + sparse_linear_bwd("out", dy, inp["W_" + p], roles, sel[p]) + dxl
        res["dA_" + p], res["dB_" + p] = dA, dB
    dxl, dA, dB = lora_bwd(xo, fwd["xl_o"], inp["dy_o"], inp["A_o"], inp["B_o"], s)
    res["dx_o"] = sparse_linear_bwd("in", inp["dy_o"], inp["W_o"], roles, sel["o"]) + dxl
    res["dA_o"], res["dB_o"], res["dx"] = dA, dB, dx
    return res


def rmsnorm_fwd(x, eps=1e-5):
    """Pre-norm with unit weight: y = x / sqrt(mean_j x_j^2 + eps) per row
    (the pages leave the layer topology around the linears open; the LLaMA
    layers they fine-tune are pre-norm, taken here with unit weight and
    eps = 1e-5).  Returns (y, rstd)."""
    x = np.asarray(x, f64)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=1) + eps)
    return x * r[:, None], r


def rmsnorm_bwd(x, rstd, dy):
    """Gradient of ``rmsnorm_fwd``: dx = r dy - r^3 x (sum_j dy_j x_j) / D."""
    x, dy = np.asarray(x, f64), np.asarray(dy, f64)
    r = np.asarray(rstd, f64)[:, None]
    D = x.shape[1]
    return r * dy - (r ** 3) * x * np.sum(dy * x, axis=1, keepdims=True) / D


def _heads(a, t0, S, H, d):
    return np.asarray(a[t0:t0 + S], f64).reshape(S, H, d).transpose(1, 0, 2)


def attention_fwd(q, k, v, batch, seq, n_heads, n_kv_heads, head_dim):
    """Plain causal softmax attention per sequence and query head: scale
    1/sqrt(d), no position encoding; query head h reads key/value head
    h // (n_heads / n_kv_heads).  q [T, H d], k, v [T, H_kv d], rows are
    sequence-major.  Returns o [T, H d]."""
    n_rep, d = n_heads // n_kv_heads, head_dim
    o = np.zeros((batch * seq, n_heads * d), f64)
    mask = np.tril(np.ones((seq, seq), bool))
    for b in range(batch):
        t0 = b * seq
        Q, K, V = _heads(q, t0, seq, n_heads, d), _heads(k, t0, seq, n_kv_heads, d), _heads(v, t0, seq, n_kv_heads, d)
        for h in range(n_heads):
            s = (Q[h] @ K[h // n_rep].T) / np.sqrt(d)
            s = np.where(mask, s, -np.inf)
            p = np.exp(s - s.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            o[t0:t0 + seq, h * d:(h + 1) * d] = p @ V[h // n_rep]
    return o


def attention_bwd(q, k, v, do, batch, seq, n_heads, n_kv_heads, head_dim):
    """Gradients of ``attention_fwd`` for upstream do: (dq, dk, dv); the
    gradients of a key/value head sum over the query heads that read it."""
    n_rep, d = n_heads // n_kv_heads, head_dim
    T = batch * seq
    dq = np.zeros((T, n_heads * d), f64)
    dk = np.zeros((T, n_kv_heads * d), f64)
    dv = np.zeros((T, n_kv_heads * d), f64)
    mask = np.tril(np.ones((seq, seq), bool))
    for b in range(batch):
        t0 = b * seq
        Q, K, V = _heads(q, t0, seq, n_heads, d), _heads(k, t0, seq, n_kv_heads, d), _heads(v, t0, seq, n_kv_heads, d)
        dO = _heads(do, t0, seq, n_heads, d)
        for h in range(n_heads):
            g = h // n_rep
            s = np.where(mask, (Q[h] @ K[g].T) / np.sqrt(d), -np.inf)
            p = np.exp(s - s.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            dp = dO[h] @ V[g].T
            ds = p * (dp - np.sum(dp * p, axis=1, keepdims=True)) / np.sqrt(d)
            dq[t0:t0 + seq, h * d:(h + 1) * d] = ds @ K[g]
            dk[t0:t0 + seq, g * d:(g + 1) * d] += ds.T @ Q[h]
            dv[t0:t0 + seq, g * d:(g + 1) * d] += p.T @ dO[h]
    return dq, dk, dv


def decoder_layer_fwd(inp, dims, idx_qk, idx_vo, idx_ffn, eps=1e-5):
    """Forward of one decoder layer whose seven linears are sparse (pre-norm
    LLaMA topology, unit-weight RMSNorm, causal softmax attention without
    position encoding; paper-graph summary §3.4: q/k/v/o by the QK and VO
    criteria, gate/up/down by the FFN criterion, output tokens dense, LoRA
    dense everywhere):
        n1 = rmsnorm(x); q, k, v = sparse(n1); a = attention(q, k, v)
        o = sparse_o(a); h1 = x + o; n2 = rmsnorm(h1); y = h1 + ffn(n2)
    dims = (batch, seq, n_heads, n_kv_heads, head_dim).  The selections are
    inputs: the estimator reads n1 (attention group) and n2 (FFN group)."""
    B, S, H, Hkv, d = dims
    n_rep = H // Hkv
    x, roles, s = np.asarray(inp["x"], f64), inp["roles"], inp["scale"]
    sel = attn_proj_indices(idx_qk, idx_vo, n_rep, d)
    f = {}
    f["n1"], f["rstd1"] = rmsnorm_fwd(x, eps)
    for p in "qkv":
        f["xl_" + p], lp = lora_fwd(f["n1"], inp["A_" + p], inp["B_" + p], s)
        f[p] = sparse_linear_fwd("out", f["n1"], inp["W_" + p], roles, sel[p]) + lp
    f["a"] = attention_fwd(f["q"], f["k"], f["v"], B, S, H, Hkv, d)
    f["xl_o"], lo = lora_fwd(f["a"], inp["A_o"], inp["B_o"], s)
    f["o"] = sparse_linear_fwd("in", f["a"], inp["W_o"], roles, sel["o"]) + lo
    f["h1"] = x + f["o"]
    f["n2"], f["rstd2"] = rmsnorm_fwd(f["h1"], eps)
    ffn = ffn_block_fwd(dict(inp, x=f["n2"]), idx_ffn)
    f.update({k + "_ffn" if k in ("y",) else k: v for k, v in ffn.items()})
    f["y"] = f["h1"] + ffn["y"]
    return f


def decoder_layer_bwd(inp, fwd, dims, idx_qk, idx_vo, idx_ffn, dy=None):
    """Backward of ``decoder_layer_fwd`` for upstream dy (default inp["dy"]):
    the gradients of every intermediate, dx, and the LoRA gradients of the
    seven linears (§3.2: dense LoRA gradients, no frozen-weight gradient)."""
    B, S, H, Hkv, d = dims
    n_rep = H // Hkv
    roles, s = inp["roles"], inp["scale"]
    dy = np.asarray(inp["dy"] if dy is None else dy, f64)
    sel = attn_proj_indices(idx_qk, idx_vo, n_rep, d)
    g = {}
    fb = ffn_block_bwd(dict(inp, x=fwd["n2"]), fwd, idx_ffn, dy=dy)
    g.update({k: v for k, v in fb.items() if k != "dx"})
    g["dn2"] = fb["dx"]
    g["dh1"] = rmsnorm_bwd(fwd["h1"], fwd["rstd2"], g["dn2"]) + dy
    dal, g["dA_o"], g["dB_o"] = lora_bwd(fwd["a"], fwd["xl_o"], g["dh1"], inp["A_o"], inp["B_o"], s)
    g["da"] = sparse_linear_bwd("in", g["dh1"], inp["W_o"], roles, sel["o"]) + dal
    g["dq"], g["dk"], g["dv"] = attention_bwd(fwd["q"], fwd["k"], fwd["v"], g["da"], B, S, H, Hkv, d)
    dn1 = np.zeros_like(fwd["n1"])
    for p in "qkv":
        dxl, g["dA_" + p], g["dB_" + p] = lora_bwd(fwd["n1"], fwd["xl_" + p], g["d" + p],
                                                   inp["A_" + p], inp["B_" + p], s)
        dn1 = dn1 + sparse_linear_bwd("out", g["d" + p], inp["W_" + p], roles, sel[p]) + dxl
    g["dn1"] = dn1
    g["dx"] = rmsnorm_bwd(inp["x"], fwd["rstd1"], dn1) + g["dh1"]
    return g


def decoder_stack_fwd(layers, x, roles, scale, dims, sels, eps=1e-5):
    """Forward of a stack of decoder layers: layer l reads the output of layer
    l - 1 (the first reads x); each layer has its own weights and its own
    selections sels[l] = (idx_qk, idx_vo, idx_ffn).  Returns the per-layer
    forward records; the stack output is the last record's "y"."""
    fwds, h = [], np.asarray(x, f64)
    for lw, sel in zip(layers, sels):
        f = decoder_layer_fwd(dict(lw, x=h, roles=roles, scale=scale), dims, *sel, eps=eps)
        fwds.append(f)
        h = f["y"]
    return fwds


def decoder_stack_bwd(layers, x, roles, scale, fwds, dy, dims, sels):
    """Backward of ``decoder_stack_fwd`` for upstream dy at the top: the
    gradient leaving layer l is the upstream gradient of layer l - 1.  Returns
    the per-layer backward records (index = layer); the stack input gradient is
    record 0's "dx"."""
    n = len(layers)
    bwds = [None] * n
    g = np.asarray(dy, f64)
    for l in range(n - 1, -1, -1):
        xin = x if l == 0 else fwds[l - 1]["y"]
        inp = dict(layers[l], x=xin, roles=roles, scale=scale)
        bwds[l] = decoder_layer_bwd(inp, fwds[l], dims, *sels[l], dy=g)
        g = bwds[l]["dx"]
    return bwds


def max_abs_rel(got, ref):
    """max |got - ref| / max(max |ref|, 1e-30), per tensor."""
    got, ref = np.asarray(got, f64), np.asarray(ref, f64)
    return float(np.max(np.abs(got - ref)) / max(float(np.max(np.abs(ref))) if ref.size else 0.0,
                                                  1e-30)) if ref.size else 0.0


def estimator_cost_ratio(k, d_in, d_out):
    """Estimator cost relative to the dense product: k (D_in + D_out) / (D_in D_out)
    (paper-graph summary §3.4, SVD estimator "Cost analysis")."""
    return Fraction(k * (d_in + d_out), d_in * d_out)


def grad_cosine(a, b):
    """cos(a, b) = a.b / (|a| |b|) over all elements, fp64; nan when either
    vector is zero.  Paper-graph summary, "Follow-Up Research This Work
    Enables": the cosine between the dense and the sparse gradient update of
    the LoRA adapters measures gradient fidelity under training sparsity."""
    a, b = np.asarray(a, f64).ravel(), np.asarray(b, f64).ravel()
    na, nb = float(np.sqrt(np.dot(a, a))), float(np.sqrt(np.dot(b, b)))
    return float(np.dot(a, b) / (na * nb)) if na > 0.0 and nb > 0.0 else float("nan")


LORA_GRADS_FFN = ("dA_gate", "dB_gate", "dA_up", "dB_up", "dA_down", "dB_down")


def ffn_grad_fidelity(inp, idx):
    """Per LoRA gradient of the FFN block: the cosine between the gradient with
    the selection idx and the gradient of the dense block (every channel kept)
    on the same inputs."""
    F = np.asarray(inp["W_gate"]).shape[0]
    everything = np.arange(F)
    fs, fd = ffn_block_fwd(inp, idx), ffn_block_fwd(inp, everything)
    bs, bd = ffn_block_bwd(inp, fs, idx), ffn_block_bwd(inp, fd, everything)
    return {k: grad_cosine(bs[k], bd[k]) for k in LORA_GRADS_FFN}


# ---------------------------------------------------------------- training steps
# Paper-graph summary, "Step Sensitivity and Progressive Sparse Fine-Tuning"
# (dense for the first p of the steps, then sparse), "Interaction with the
# learning rate schedule" (cosine with a 4 % warm-up), "Putting It All
# Together" (loss on output positions only, the autoregressive loss; only the
# LoRA parameters are updated).


def round_to(a, dtype):
    """Values rounded to the compute dtype ("f64" keeps them, "f32" to binary32,
    "bf16" to bfloat16 with round-to-nearest-even), returned as float64."""
    a = np.asarray(a, f64)
    if dtype == "f64":
        return a.copy()
    f = a.astype(np.float32)
    if dtype == "f32":
        return f.astype(f64)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16 << 16
    return u.astype(np.uint32).view(np.float32).astype(f64)


def token_ce(logits, labels):
    """Mean softmax cross-entropy of the rows of logits [n, V] against integer
    labels [n], and its gradient with respect to the logits.  A label outside
    [0, V) (an ignore index such as -100) marks a position that is not a
    target: it adds nothing to the loss, has a zero gradient row, and is not
    counted in the mean."""
    z = np.asarray(logits, f64)
    labels = np.asarray(labels).astype(np.int64)
    n, V = z.shape
    keep = (labels >= 0) & (labels < V)
    nv = int(keep.sum())
    if nv == 0:
        return 0.0, np.zeros_like(z)
    zmax = z.max(axis=1, keepdims=True)
    lse = zmax[:, 0] + np.log(np.exp(z - zmax).sum(axis=1))
    rows = np.nonzero(keep)[0]
    loss = float(np.sum(lse[rows] - z[rows, labels[rows]]) / nv)
    p = np.exp(z - lse[:, None])
    p[rows, labels[rows]] -= 1.0
    p[~keep] = 0.0
    return loss, p / nv


def adamw(p, g, m, v, step, lr, b1=0.9, b2=0.999, eps=1e-8, wd=0.0):
    """One AdamW update (decoupled weight decay), textbook form."""
    p = np.asarray(p, f64) * (1.0 - lr * wd)
    m = b1 * m + (1.0 - b1) * g
    v = b2 * v + (1.0 - b2) * g * g
    mh, vh = m / (1.0 - b1 ** step), v / (1.0 - b2 ** step)
    return p - lr * mh / (np.sqrt(vh) + eps), m, v


def lr_schedule(step, total, peak, warmup_ratio=0.04):
    """Rate of 0-based step: linear from 0 over the warm-up steps
    (ceil(warmup_ratio total)), then half a cosine period down to 0 at `total`."""
    w = int(np.ceil(warmup_ratio * total))
    if step < w:
        return peak * step / w
    return peak * 0.5 * (1.0 + np.cos(np.pi * (step - w) / max(1, total - w)))


LORA_FFN = ("A_gate", "B_gate", "A_up", "B_up", "A_down", "B_down")


def ffn_train(inp, W_head, xs, labels, total, n_dense, select, dtype, lr, warmup_ratio=0.04,
              b1=0.9, b2=0.999, eps=1e-8, wd=0.0):
    """len(xs) training steps of the FFN block with a frozen LM head W_head
    [V, D]: step t runs dense (every channel) when t < n_dense, else with the
    selection select(x_t); logits of the output rows, mean cross-entropy
    against their labels, backward, AdamW on the six LoRA tensors (masters in
    float64, the forward and backward use them rounded to `dtype`).  Returns
    the per-step losses and the final masters."""
    F = np.asarray(inp["W_gate"]).shape[0]
    master = {k: np.asarray(inp[k], f64).copy() for k in LORA_FFN}
    mom = {k: np.zeros_like(master[k]) for k in LORA_FFN}
    vel = {k: np.zeros_like(master[k]) for k in LORA_FFN}
    ctx, out = token_lists(inp["roles"])
    Wh = np.asarray(W_head, f64)
    losses = []
    for t, (x, lab) in enumerate(zip(xs, labels)):
        d = dict(inp, x=np.asarray(x, f64), **{k: round_to(master[k], dtype) for k in LORA_FFN})
        idx = np.arange(F) if t < n_dense else select(x)
        fw = ffn_block_fwd(d, idx)
        loss, dlog = token_ce(fw["y"][out] @ Wh.T, np.asarray(lab)[out])
        dy = np.zeros_like(fw["y"])
        dy[out] = dlog @ Wh
        bw = ffn_block_bwd(d, fw, idx, dy)
        rate = lr_schedule(t, total, lr, warmup_ratio)
        for k in LORA_FFN:
            master[k], mom[k], vel[k] = adamw(master[k], bw["d" + k], mom[k], vel[k], t + 1, rate, b1, b2,
                                              eps, wd)
        losses.append(loss)
    return losses, master


def svd_factors(W_lin, k):
    """Rank-k estimator factors of a weight in nn.Linear layout [D_out, D_in]
    (paper-graph summary §3.4 "SVD Sparsity Estimator": with W = W_lin^T =
    U diag(s) V^T, W_A = U_k diag(sqrt(s_k)), W_B = diag(sqrt(s_k)) V_k^T, so
    x W ~ (x W_A) W_B).  Each singular pair is signed so that the
    largest-magnitude entry of its left vector is positive (the first such
    entry on ties).  Returns (W_A^T [k, D_in], W_B [k, D_out]) in float64."""
    W = np.asarray(W_lin, f64).T
    U, s, Vt = np.linalg.svd(W, full_matrices=False)
    U, s, V = U[:, :k], s[:k], Vt[:k].T
    sign = np.sign(U[np.argmax(np.abs(U), axis=0), np.arange(k)])
    sign[sign == 0] = 1.0
    rs = np.sqrt(s)
    return (U * sign * rs).T, (rs[:, None] * (V * sign).T)
