"""Pins of the oracle's fp64 part (main branch, LoRA, SwiGLU, FFN block) and of
the input recipe's estimator factors, against special cases, library
routines, exact identities and calculus."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import reference as ref
from workloads.configs import CONFIGS, scaled
from workloads.gen import make_ffn_inputs, roles_for, svd_factor_pair

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_numbers.json")


# ---------------------------------------------------------------- small helpers

def test_token_lists():
    roles = np.array([0, 1, 1, 0, 0, 1, 0], np.uint8)
    ctx, out = ref.token_lists(roles)
    assert ctx.tolist() == [0, 3, 4, 6] and out.tolist() == [1, 2, 5]
    for cid, cfg in CONFIGS.items():
        ctx, out = ref.token_lists(roles_for(cfg))
        assert len(out) == cfg.batch * cfg.out_per_seq
        assert sorted(np.concatenate([ctx, out]).tolist()) == list(range(cfg.tokens))
        for b in range(cfg.batch):                        # contiguous tail per sequence
            tail = list(range(b * cfg.seq + cfg.seq - cfg.out_per_seq, (b + 1) * cfg.seq))
            assert set(tail) <= set(out.tolist())


def test_n_keep_integer_and_float_trap():
    for C in (1, 7, 688, 1000, 1024, 5120, 13824, 14336):
        for num, den in ((0, 1), (1, 2), (7, 10), (3, 10), (1, 35), (4, 5), (99, 100), (1, 1)):
            exact = Fraction(C) * (1 - Fraction(num, den))
            want = -((-exact.numerator) // exact.denominator)
            assert ref.n_keep(C, num, den) == want
    # the floating-point reading would keep 301 of 1000 at 70% sparsity
    assert int(np.ceil((1 - 0.7) * 1000)) == 301 and ref.n_keep(1000, 7, 10) == 300
    # configuration table
    assert ref.n_keep(688, 1, 2) == 344
    assert ref.n_keep(14336, 7, 10) == 4301
    assert ref.n_keep(13824, 7, 10) == 4148
    cfg5 = CONFIGS[5]
    got = [ref.n_keep(14336, *cfg5.layer_sparsity(l)) for l in (0, 3, 4, 17, 31)]
    assert got == [14336, 14336, 13927, 8602, 2868]
    got = [ref.n_keep(1024, *cfg5.layer_sparsity(l)) for l in (4, 17, 31)]
    assert got == [995, 615, 205]


def test_golden_estimator_cost_ratio():
    with open(GOLDEN) as f:
        g = json.load(f)["estimator_cost_ratio"]
    r = ref.estimator_cost_ratio(g["k"], g["d_in"], g["d_out"])
    assert round(float(r), g["printed_digits"]) == g["printed"]


def test_expand_gqa_enumeration(rng):
    H_kv, n_rep, d = 4, 3, 8
    idx_kv = np.sort(rng.choice(H_kv * d, 11, replace=False)).astype(np.int32)
    q = ref.expand_gqa(idx_kv, n_rep, d)
    kv_set = set(idx_kv.tolist())
    want = [c for c in range(H_kv * n_rep * d) if ((c // d) // n_rep) * d + c % d in kv_set]
    assert q.tolist() == want and len(q) == n_rep * len(idx_kv)
    assert ref.expand_gqa(idx_kv, 1, d).tolist() == idx_kv.tolist()


# ---------------------------------------------------------------- main branch

def _small(rng, T=40, Din=24, Dout=30, r=3):
    roles = (np.arange(T) % 10 >= 7).astype(np.uint8)
    x = rng.standard_normal((T, Din))
    W = rng.standard_normal((Dout, Din))
    A = rng.standard_normal((r, Din))
    B = rng.standard_normal((Dout, r))
    return roles, x, W, A, B


def test_sparsity_zero_is_textbook_dense_lora(rng):
    roles, x, W, A, B = _small(rng)
    s = 2.0
    xt, Wt, At, Bt = (torch.tensor(a, dtype=torch.float64) for a in (x, W, A, B))
    dense = torch.nn.functional.linear(xt, Wt) + s * torch.nn.functional.linear(
        torch.nn.functional.linear(xt, At), Bt)
    all_out = np.arange(W.shape[0])
    y = ref.sparse_linear_fwd("out", x, W, roles, all_out) + ref.lora_fwd(x, A, B, s)[1]
    assert np.allclose(y, dense.numpy(), rtol=1e-13, atol=1e-13)
    all_in = np.arange(W.shape[1])
    y2 = ref.sparse_linear_fwd("in", x, W, roles, all_in) + ref.lora_fwd(x, A, B, s)[1]
    assert np.allclose(y2, dense.numpy(), rtol=1e-13, atol=1e-13)


def test_sliced_equals_masked(rng):
    roles, x, W, A, B = _small(rng)
    ctx, out = ref.token_lists(roles)
    idx = np.sort(rng.choice(W.shape[0], 11, replace=False))
    y = ref.sparse_linear_fwd("out", x, W, roles, idx)
    sliced = np.zeros_like(y)
    sliced[out] = x[out] @ W.T
    sliced[np.ix_(ctx, idx)] = x[ctx] @ W[idx].T
    assert np.allclose(y, sliced, rtol=1e-13, atol=1e-13)
    assert np.all(y[np.ix_(ctx, np.setdiff1d(np.arange(W.shape[0]), idx))] == 0.0)
    idx_in = np.sort(rng.choice(W.shape[1], 9, replace=False))
    y = ref.sparse_linear_fwd("in", x, W, roles, idx_in)
    sliced = np.zeros_like(y)
    sliced[out] = x[out] @ W.T
    sliced[ctx] = x[np.ix_(ctx, idx_in)] @ W[:, idx_in].T
    assert np.allclose(y, sliced, rtol=1e-13, atol=1e-13)


def test_output_rows_untouched_by_selection(rng):
    roles, x, W, A, B = _small(rng)
    _, out = ref.token_lists(roles)
    for side, C in (("out", W.shape[0]), ("in", W.shape[1])):
        a = ref.sparse_linear_fwd(side, x, W, roles, np.arange(0, C, 2))
        b = ref.sparse_linear_fwd(side, x, W, roles, np.arange(3))
        c = ref.sparse_linear_fwd(side, x, W, roles, np.arange(0))
        assert np.array_equal(a[out], b[out]) and np.array_equal(a[out], c[out])
        dy = rng.standard_normal((x.shape[0], W.shape[0]))
        da = ref.sparse_linear_bwd(side, dy, W, roles, np.arange(0, C, 2))
        db = ref.sparse_linear_bwd(side, dy, W, roles, np.arange(0))
        assert np.array_equal(da[out], db[out])


def test_adjoint_identity(rng):
    roles, x, W, A, B = _small(rng)
    for side, C in (("out", W.shape[0]), ("in", W.shape[1])):
        idx = np.sort(rng.choice(C, C // 3, replace=False))
        dy = rng.standard_normal((x.shape[0], W.shape[0]))
        lhs = np.sum(ref.sparse_linear_fwd(side, x, W, roles, idx) * dy)
        rhs = np.sum(x * ref.sparse_linear_bwd(side, dy, W, roles, idx))
        assert abs(lhs - rhs) <= 1e-12 * (abs(lhs) + 1.0)


def _ffn_small(rng):
    cfg = scaled(CONFIGS[1], batch=2, seq=12, out_per_seq=3, hidden=10, inter=14,
                 lora_rank=3, est_rank=2, dtype="f32")
    inp = make_ffn_inputs(cfg, with_factors=False)
    inp = {k: (np.asarray(v, np.float64) if isinstance(v, np.ndarray) and k != "roles" else v)
           for k, v in inp.items()}
    # larger LoRA factors so their gradients are well above rounding noise
    for k in ("A_gate", "B_gate", "A_up", "B_up", "A_down", "B_down"):
        inp[k] = rng.standard_normal(inp[k].shape) * 0.5
    idx = np.sort(rng.choice(cfg.inter, 6, replace=False))
    return cfg, inp, idx


def test_ffn_block_backward_matches_autograd(rng):
    cfg, inp, idx = _ffn_small(rng)
    fwd = ref.ffn_block_fwd(inp, idx)
    bwd = ref.ffn_block_bwd(inp, fwd, idx)
    T = cfg.tokens
    M = torch.tensor(ref.keep_mask(T, cfg.inter, inp["roles"], idx))
    t = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True)
         for k, v in inp.items() if isinstance(v, np.ndarray) and k != "roles"}
    s = inp["scale"]
    lin = torch.nn.functional.linear
    g = lin(t["x"], t["W_gate"]) * M + s * lin(lin(t["x"], t["A_gate"]), t["B_gate"])
    u = lin(t["x"], t["W_up"]) * M + s * lin(lin(t["x"], t["A_up"]), t["B_up"])
    h = torch.nn.functional.silu(g) * u
    y = lin(h * M, t["W_down"]) + s * lin(lin(h, t["A_down"]), t["B_down"])
    assert np.allclose(y.detach().numpy(), fwd["y"], rtol=1e-12, atol=1e-12)
    (y * t["dy"]).sum().backward()
    assert np.allclose(t["x"].grad.numpy(), bwd["dx"], rtol=1e-10, atol=1e-12)
    for p in ("gate", "up", "down"):
        assert np.allclose(t["A_" + p].grad.numpy(), bwd["dA_" + p], rtol=1e-10, atol=1e-12)
        assert np.allclose(t["B_" + p].grad.numpy(), bwd["dB_" + p], rtol=1e-10, atol=1e-12)


def test_lora_grads_finite_differences(rng):
    cfg, inp, idx = _ffn_small(rng)

    def loss(d):
        return float(np.sum(ref.ffn_block_fwd(d, idx)["y"] * inp["dy"]))

    bwd = ref.ffn_block_bwd(inp, ref.ffn_block_fwd(inp, idx), idx)
    eps = 1e-6
    for name in ("A_gate", "B_up", "A_down", "B_down"):
        for _ in range(4):
            pos = tuple(rng.integers(0, s) for s in inp[name].shape)
            d1, d2 = dict(inp), dict(inp)
            d1[name] = inp[name].copy()
            d2[name] = inp[name].copy()
            d1[name][pos] += eps
            d2[name][pos] -= eps
            fd = (loss(d1) - loss(d2)) / (2 * eps)
            assert abs(fd - bwd["d" + name][pos]) <= 1e-6 * (1 + abs(fd))


def test_unselected_context_channels_carry_lora_only(rng):
    cfg, inp, idx = _ffn_small(rng)
    fwd = ref.ffn_block_fwd(inp, idx)
    ctx, _ = ref.token_lists(inp["roles"])
    drop = np.setdiff1d(np.arange(cfg.inter), idx)
    lora_g = ref.lora_fwd(inp["x"], inp["A_gate"], inp["B_gate"], inp["scale"])[1]
    assert np.array_equal(fwd["g"][np.ix_(ctx, drop)], lora_g[np.ix_(ctx, drop)])


# ---------------------------------------------------------------- factors (input recipe)

@pytest.mark.parametrize("shape,k", [((120, 80), 8), ((60, 200), 16), ((2100, 2300), 16)])
def test_factors_eckart_young(rng, shape, k):
    W = (rng.standard_normal(shape) * 0.02).astype(np.float32)   # nn.Linear [D_out, D_in]
    WA_t, WB = svd_factor_pair(W, k)
    Wm = W.T.astype(np.float64)
    s = np.linalg.svd(Wm, compute_uv=False)
    P = WA_t.T.astype(np.float64) @ WB.astype(np.float64)
    R = Wm - P
    assert abs(np.sum(R * R) - np.sum(s[k:] ** 2)) <= 1e-5 * np.sum(Wm * Wm)
    assert abs(np.linalg.norm(R, 2) - s[k]) <= 1e-4 * s[0]
    # W_A^T W_A = diag(s_k) = W_B W_B^T (the sqrt(s) split on both sides)
    GA = WA_t.astype(np.float64) @ WA_t.T.astype(np.float64)
    GB = WB.astype(np.float64) @ WB.T.astype(np.float64)
    assert np.allclose(GA, np.diag(s[:k]), atol=1e-5 * s[0])
    assert np.allclose(GB, np.diag(s[:k]), atol=1e-5 * s[0])


def test_full_rank_factors_reconstruct(rng):
    W = rng.standard_normal((30, 20)).astype(np.float32)
    WA_t, WB = svd_factor_pair(W, 20)
    assert np.allclose(WA_t.T.astype(np.float64) @ WB, W.T, atol=1e-5)


def _attn_small(rng, Hq=4, Hkv=2, d=3, D=10, T=14, r=2):
    roles = np.zeros(T, np.uint8)
    roles[T - 4:] = 1
    Cq, Ckv = Hq * d, Hkv * d
    inp = {"x": rng.standard_normal((T, D)), "x_o": rng.standard_normal((T, Cq)), "roles": roles,
           "scale": 2.0, "W_q": rng.standard_normal((Cq, D)), "W_k": rng.standard_normal((Ckv, D)),
           "W_v": rng.standard_normal((Ckv, D)), "W_o": rng.standard_normal((D, Cq))}
    for p, (cin, cout) in {"q": (D, Cq), "k": (D, Ckv), "v": (D, Ckv), "o": (Cq, D)}.items():
        inp["A_" + p] = rng.standard_normal((r, cin))
        inp["B_" + p] = rng.standard_normal((cout, r))
    for p, c in {"q": Cq, "k": Ckv, "v": Ckv, "o": D}.items():
        inp["dy_" + p] = rng.standard_normal((T, c))
    idx_qk = np.sort(rng.choice(Ckv, 3, replace=False)).astype(np.int32)
    idx_vo = np.sort(rng.choice(Ckv, 4, replace=False)).astype(np.int32)
    return inp, idx_qk, idx_vo, Hq // Hkv, d


def test_attn_projections_match_autograd_with_gqa_masks(rng):
    """q/k/v/o composition against torch autograd on masks built another way:
    the query-head keep mask is the key mask repeated over each group's heads
    (repeat_interleave), not the index arithmetic of expand_gqa."""
    inp, idx_qk, idx_vo, n_rep, d = _attn_small(rng)
    fwd = ref.attn_proj_fwd(inp, idx_qk, idx_vo, n_rep, d)
    bwd = ref.attn_proj_bwd(inp, fwd, idx_qk, idx_vo, n_rep, d)
    t = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True)
         for k, v in inp.items() if isinstance(v, np.ndarray) and k != "roles"}
    lin = torch.nn.functional.linear
    s = inp["scale"]
    ctx = torch.tensor(inp["roles"] == 0)[:, None]
    Ckv = inp["W_k"].shape[0]

    def kv_keep(idx):
        m = torch.zeros(Ckv, dtype=torch.float64)
        m[torch.tensor(idx, dtype=torch.long)] = 1.0
        return m

    def q_keep(idx):
        return kv_keep(idx).view(-1, d).repeat_interleave(n_rep, dim=0).reshape(-1)

    masks = {"q": q_keep(idx_qk), "k": kv_keep(idx_qk), "v": kv_keep(idx_vo)}
    outs = {}
    for p in "qkv":
        y = lin(t["x"], t["W_" + p])
        y = torch.where(ctx, y * masks[p], y) + s * lin(lin(t["x"], t["A_" + p]), t["B_" + p])
        outs[p] = y
        assert np.allclose(y.detach().numpy(), fwd[p], rtol=1e-12, atol=1e-12), p
    mo = q_keep(idx_vo)
    xo = torch.where(ctx, t["x_o"] * mo, t["x_o"])
    o = lin(xo, t["W_o"]) + s * lin(lin(t["x_o"], t["A_o"]), t["B_o"])
    assert np.allclose(o.detach().numpy(), fwd["o"], rtol=1e-12, atol=1e-12)
    loss = sum((outs[p] * t["dy_" + p]).sum() for p in "qkv") + (o * t["dy_o"]).sum()
    loss.backward()
    assert np.allclose(t["x"].grad.numpy(), bwd["dx"], rtol=1e-10, atol=1e-12)
    assert np.allclose(t["x_o"].grad.numpy(), bwd["dx_o"], rtol=1e-10, atol=1e-12)
    for p in "qkvo":
        assert np.allclose(t["A_" + p].grad.numpy(), bwd["dA_" + p], rtol=1e-10, atol=1e-12), p
        assert np.allclose(t["B_" + p].grad.numpy(), bwd["dB_" + p], rtol=1e-10, atol=1e-12), p


def test_attn_projections_all_kept_are_dense(rng):
    inp, _, _, n_rep, d = _attn_small(rng)
    Ckv = inp["W_k"].shape[0]
    allk = np.arange(Ckv, dtype=np.int32)
    fwd = ref.attn_proj_fwd(inp, allk, allk, n_rep, d)
    s = inp["scale"]
    for p in "qkv":
        dense = inp["x"] @ inp["W_" + p].T + s * (inp["x"] @ inp["A_" + p].T) @ inp["B_" + p].T
        assert np.allclose(fwd[p], dense, rtol=1e-12, atol=1e-12)
    dense_o = inp["x_o"] @ inp["W_o"].T + s * (inp["x_o"] @ inp["A_o"].T) @ inp["B_o"].T
    assert np.allclose(fwd["o"], dense_o, rtol=1e-12, atol=1e-12)


def test_rmsnorm_matches_library_and_autograd(rng):
    x = rng.standard_normal((7, 24)) * 3.0
    dy = rng.standard_normal((7, 24))
    y, r = ref.rmsnorm_fwd(x, eps=1e-5)
    xt = torch.tensor(x, requires_grad=True)
    yt = torch.nn.functional.rms_norm(xt, (24,), eps=1e-5)
    assert np.allclose(y, yt.detach().numpy(), rtol=1e-13, atol=1e-13)
    (yt * torch.tensor(dy)).sum().backward()
    assert np.allclose(ref.rmsnorm_bwd(x, r, dy), xt.grad.numpy(), rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (6, 2)])
def test_attention_matches_sdpa_and_autograd(rng, Hq, Hkv):
    """Causal softmax attention against torch's scaled_dot_product_attention in
    fp64 with key/value heads repeated over each group (repeat_interleave)."""
    B, S, d = 2, 9, 5
    T = B * S
    q = rng.standard_normal((T, Hq * d))
    k = rng.standard_normal((T, Hkv * d))
    v = rng.standard_normal((T, Hkv * d))
    do = rng.standard_normal((T, Hq * d))
    o = ref.attention_fwd(q, k, v, B, S, Hq, Hkv, d)
    dq, dk, dv = ref.attention_bwd(q, k, v, do, B, S, Hq, Hkv, d)
    qt, kt, vt = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    sh = lambda a, H: a.view(B, S, H, d).transpose(1, 2)
    kk = sh(kt, Hkv).repeat_interleave(Hq // Hkv, dim=1)
    vv = sh(vt, Hkv).repeat_interleave(Hq // Hkv, dim=1)
    ot = torch.nn.functional.scaled_dot_product_attention(sh(qt, Hq), kk, vv, is_causal=True)
    ot = ot.transpose(1, 2).reshape(T, Hq * d)
    assert np.allclose(o, ot.detach().numpy(), rtol=1e-12, atol=1e-12)
    (ot * torch.tensor(do)).sum().backward()
    assert np.allclose(dq, qt.grad.numpy(), rtol=1e-10, atol=1e-12)
    assert np.allclose(dk, kt.grad.numpy(), rtol=1e-10, atol=1e-12)
    assert np.allclose(dv, vt.grad.numpy(), rtol=1e-10, atol=1e-12)


def _layer_small(rng, B=2, S=7, Hq=4, Hkv=2, d=3, D=10, F=14, r=2):
    T = B * S
    roles = np.zeros(T, np.uint8)
    for b in range(B):
        roles[b * S + S - 2:(b + 1) * S] = 1
    Cq, Ckv = Hq * d, Hkv * d
    shapes = {"q": (Cq, D), "k": (Ckv, D), "v": (Ckv, D), "o": (D, Cq), "gate": (F, D),
              "up": (F, D), "down": (D, F)}
    inp = {"x": rng.standard_normal((T, D)) * 2.0, "dy": rng.standard_normal((T, D)),
           "roles": roles, "scale": 2.0}
    for p, (cout, cin) in shapes.items():
        inp["W_" + p] = rng.standard_normal((cout, cin)) * 0.5
        inp["A_" + p] = rng.standard_normal((r, cin)) * 0.5
        inp["B_" + p] = rng.standard_normal((cout, r)) * 0.5
    idx_qk = np.sort(rng.choice(Ckv, 3, replace=False)).astype(np.int32)
    idx_vo = np.sort(rng.choice(Ckv, 4, replace=False)).astype(np.int32)
    idx_f = np.sort(rng.choice(F, 6, replace=False)).astype(np.int32)
    return inp, (B, S, Hq, Hkv, d), idx_qk, idx_vo, idx_f


def _torch_layer(t, h, dims, roles, sel, s):
    """A torch build of one sparse decoder layer: library RMSNorm, SDPA with
    key/value heads repeated over each group, keep masks formed from the
    selections by scatter and repeat_interleave (t: the layer's weight tensors)."""
    B, S, Hq, Hkv, d = dims
    idx_qk, idx_vo, idx_f = sel
    T, D = h.shape
    lin = torch.nn.functional.linear
    ctx = torch.tensor(roles == 0)[:, None]

    def keep(n, idx):
        m = torch.zeros(n, dtype=torch.float64)
        m[torch.tensor(idx, dtype=torch.long)] = 1.0
        return m

    rep = lambda m: m.view(-1, d).repeat_interleave(Hq // Hkv, dim=0).reshape(-1)
    mk_qk, mk_vo = keep(Hkv * d, idx_qk), keep(Hkv * d, idx_vo)
    lora = lambda z, p: s * lin(lin(z, t["A_" + p]), t["B_" + p])
    out_sparse = lambda z, p, m: torch.where(ctx, lin(z, t["W_" + p]) * m, lin(z, t["W_" + p])) + lora(z, p)
    in_sparse = lambda z, p, m: lin(torch.where(ctx, z * m, z), t["W_" + p]) + lora(z, p)
    n1 = torch.nn.functional.rms_norm(h, (D,), eps=1e-5)
    q, k, v = out_sparse(n1, "q", rep(mk_qk)), out_sparse(n1, "k", mk_qk), out_sparse(n1, "v", mk_vo)
    sh = lambda a, H: a.view(B, S, H, d).transpose(1, 2)
    a = torch.nn.functional.scaled_dot_product_attention(
        sh(q, Hq), sh(k, Hkv).repeat_interleave(Hq // Hkv, dim=1),
        sh(v, Hkv).repeat_interleave(Hq // Hkv, dim=1), is_causal=True).transpose(1, 2).reshape(T, -1)
    h1 = h + in_sparse(a, "o", rep(mk_vo))
    n2 = torch.nn.functional.rms_norm(h1, (D,), eps=1e-5)
    mf = keep(t["W_gate"].shape[0], idx_f)
    hh = torch.nn.functional.silu(out_sparse(n2, "gate", mf)) * out_sparse(n2, "up", mf)
    return {"a": a, "h1": h1, "h": hh, "y": h1 + in_sparse(hh, "down", mf)}


_LIN = ("q", "k", "v", "o", "gate", "up", "down")


def test_decoder_layer_matches_autograd(rng):
    """The layer composition against the torch build of the same layer, with
    autograd for every gradient."""
    inp, dims, idx_qk, idx_vo, idx_f = _layer_small(rng)
    fwd = ref.decoder_layer_fwd(inp, dims, idx_qk, idx_vo, idx_f)
    bwd = ref.decoder_layer_bwd(inp, fwd, dims, idx_qk, idx_vo, idx_f)
    t = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True)
         for k, v in inp.items() if isinstance(v, np.ndarray) and k != "roles"}
    o = _torch_layer(t, t["x"], dims, inp["roles"], (idx_qk, idx_vo, idx_f), inp["scale"])
    for name, val in o.items():
        assert np.allclose(val.detach().numpy(), fwd[name], rtol=1e-11, atol=1e-11), name
    (o["y"] * t["dy"]).sum().backward()
    assert np.allclose(t["x"].grad.numpy(), bwd["dx"], rtol=1e-9, atol=1e-10)
    for p in _LIN:
        assert np.allclose(t["A_" + p].grad.numpy(), bwd["dA_" + p], rtol=1e-9, atol=1e-10), p
        assert np.allclose(t["B_" + p].grad.numpy(), bwd["dB_" + p], rtol=1e-9, atol=1e-10), p


def test_decoder_stack_matches_autograd(rng):
    """Three layers with their own weights and selections: the stack
    composition against the torch build chained by hand, autograd for the
    input gradient and the LoRA gradients of every layer."""
    layers, sels = [], []
    for _ in range(3):
        inp, dims, *sel = _layer_small(rng)
        layers.append({k: v for k, v in inp.items() if k[:2] in ("W_", "A_", "B_")})
        sels.append(tuple(sel))
    x, dy, roles, s = inp["x"], inp["dy"], inp["roles"], inp["scale"]
    fwds = ref.decoder_stack_fwd(layers, x, roles, s, dims, sels)
    bwds = ref.decoder_stack_bwd(layers, x, roles, s, fwds, dy, dims, sels)
    xt = torch.tensor(x, requires_grad=True)
    ts = [{k: torch.tensor(v, requires_grad=True) for k, v in lw.items()} for lw in layers]
    h = xt
    for l in range(3):
        h = _torch_layer(ts[l], h, dims, roles, sels[l], s)["y"]
        assert np.allclose(h.detach().numpy(), fwds[l]["y"], rtol=1e-11, atol=1e-11), l
    (h * torch.tensor(dy)).sum().backward()
    assert np.allclose(xt.grad.numpy(), bwds[0]["dx"], rtol=1e-9, atol=1e-10)
    for l in range(3):
        for p in _LIN:
            assert np.allclose(ts[l]["A_" + p].grad.numpy(), bwds[l]["dA_" + p], rtol=1e-9, atol=1e-10)
            assert np.allclose(ts[l]["B_" + p].grad.numpy(), bwds[l]["dB_" + p], rtol=1e-9, atol=1e-10)


def test_decoder_layer_all_kept_zero_lora_is_plain_layer(rng):
    """Every channel kept and B = 0: the layer reduces to the plain dense
    pre-norm layer (residual + attention + SwiGLU), whatever the roles."""
    inp, dims, *_ = _layer_small(rng)
    B, S, Hq, Hkv, d = dims
    for p in ("q", "k", "v", "o", "gate", "up", "down"):
        inp["B_" + p] = np.zeros_like(inp["B_" + p])
    allkv = np.arange(Hkv * d, dtype=np.int32)
    allf = np.arange(inp["W_gate"].shape[0], dtype=np.int32)
    fwd = ref.decoder_layer_fwd(inp, dims, allkv, allkv, allf)
    x = inp["x"]
    n1 = x / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + 1e-5)
    a = ref.attention_fwd(n1 @ inp["W_q"].T, n1 @ inp["W_k"].T, n1 @ inp["W_v"].T, B, S, Hq, Hkv, d)
    h1 = x + a @ inp["W_o"].T
    n2 = h1 / np.sqrt(np.mean(h1 * h1, axis=1, keepdims=True) + 1e-5)
    g, u = n2 @ inp["W_gate"].T, n2 @ inp["W_up"].T
    y = h1 + (g / (1.0 + np.exp(-g)) * u) @ inp["W_down"].T
    assert np.allclose(fwd["y"], y, rtol=1e-12, atol=1e-12)


def test_subspace_factors_recover_a_planted_spectrum(rng):
    """With a clear gap after the k-th singular value, the randomized subspace
    iteration reaches the exact truncated SVD: same factors as the fp64 SVD."""
    from workloads.gen import svd_factor_pair_subspace
    d_in, d_out, k = 96, 200, 6
    U, _ = np.linalg.qr(rng.standard_normal((d_in, d_in)))
    V, _ = np.linalg.qr(rng.standard_normal((d_out, d_in)))
    s = np.concatenate([np.linspace(5.0, 2.0, k), 0.05 * np.ones(d_in - k)])
    W_lin = ((U * s) @ V.T).T                  # nn.Linear layout [d_out, d_in]
    WA_t, WB = svd_factor_pair(W_lin, k)
    RA_t, RB = svd_factor_pair_subspace(W_lin, k, np.random.default_rng(5))
    assert np.allclose(RA_t, WA_t, atol=2e-4) and np.allclose(RB, WB, atol=2e-4)


def test_subspace_factors_near_optimal_on_gaussian(rng):
    """On an unstructured Gaussian weight the approximate rank-k product's
    Frobenius error stays within 1% of the Eckart-Young optimum, and the
    factor shapes and scaling match the exact recipe's."""
    from workloads.gen import svd_factor_pair_subspace
    W_lin = rng.standard_normal((300, 128)) * 0.02
    k = 8
    WA_t, WB = svd_factor_pair(W_lin, k)
    RA_t, RB = svd_factor_pair_subspace(W_lin, k, np.random.default_rng(6))
    assert RA_t.shape == WA_t.shape and RB.shape == WB.shape
    Wm = W_lin.T
    e_opt = np.linalg.norm(Wm - WA_t.T.astype(np.float64) @ WB)
    e_rnd = np.linalg.norm(Wm - RA_t.T.astype(np.float64) @ RB)
    assert e_opt <= e_rnd <= 1.01 * e_opt
    # W_A and W_B^T share the singular values: column norms of W_A^T rows equal
    assert np.allclose(np.linalg.norm(RA_t, axis=1), np.linalg.norm(RB, axis=1), rtol=1e-5)


def test_grad_cosine_closed_forms(rng):
    """cos of (1, 2, 2) and (2, 1, 2) is 8/9; a vector with a positive multiple
    of itself gives 1, with a negative one -1; orthogonal vectors give 0; a
    zero vector gives nan; shape does not matter (all elements count)."""
    assert ref.grad_cosine([1, 2, 2], [2, 1, 2]) == pytest.approx(8 / 9, abs=1e-15)
    a = rng.standard_normal((7, 5))
    assert ref.grad_cosine(a, 3.0 * a) == pytest.approx(1.0, abs=1e-15)
    assert ref.grad_cosine(a, -0.5 * a) == pytest.approx(-1.0, abs=1e-15)
    b = rng.standard_normal((7, 5))
    b_orth = b - (np.sum(a * b) / np.sum(a * a)) * a
    assert abs(ref.grad_cosine(a, b_orth)) < 1e-14
    assert np.isnan(ref.grad_cosine(np.zeros(3), [1, 2, 3]))
    assert ref.grad_cosine(a, b) == pytest.approx(ref.grad_cosine(a.ravel(), b.T.T.ravel()), abs=0)


def test_ffn_grad_fidelity_matches_autograd_cosines(rng):
    """The per-adapter cosines between the sparse and the dense FFN block's
    LoRA gradients equal torch's cosine_similarity of autograd gradients of the
    masked and the unmasked block; with every channel kept they are 1."""
    cfg, inp, idx = _ffn_small(rng)
    fid = ref.ffn_grad_fidelity(inp, idx)
    T = cfg.tokens
    s = inp["scale"]
    lin = torch.nn.functional.linear

    def grads(mask):
        M = torch.tensor(mask)
        t = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True)
             for k, v in inp.items() if isinstance(v, np.ndarray) and k != "roles"}
        g = lin(t["x"], t["W_gate"]) * M + s * lin(lin(t["x"], t["A_gate"]), t["B_gate"])
        u = lin(t["x"], t["W_up"]) * M + s * lin(lin(t["x"], t["A_up"]), t["B_up"])
        h = torch.nn.functional.silu(g) * u
        y = lin(h * M, t["W_down"]) + s * lin(lin(h, t["A_down"]), t["B_down"])
        (y * t["dy"]).sum().backward()
        return {p: t[p].grad.reshape(-1) for p in ("A_gate", "B_gate", "A_up", "B_up", "A_down", "B_down")}

    gs = grads(ref.keep_mask(T, cfg.inter, inp["roles"], idx))
    gd = grads(np.ones((T, cfg.inter)))
    for p in gs:
        want = float(torch.nn.functional.cosine_similarity(gs[p], gd[p], dim=0))
        assert fid["d" + p] == pytest.approx(want, abs=1e-12), p
    assert min(fid.values()) < 1.0 - 1e-6          # the selection changes some gradient
    full = ref.ffn_grad_fidelity(inp, np.arange(cfg.inter))
    assert all(v == pytest.approx(1.0, abs=1e-14) for v in full.values())
