"""GPU parity of the sparse q/k/v/o projections (QK and VO criteria, GQA
expansion, stacked q|k|v product, input-side o, dense LoRA on all four),
forward and backward, against the CPU oracle.

A scaled bf16 configuration is compared end to end.  The full-size LLaMA3-8B
projections are compared op by op on sampled context and output rows (each
GPU output against the oracle applied to that op's inputs), with the selection
bit-exact and every LoRA gradient in full."""
import functools

import numpy as np
import pytest
import torch

from oracle import csa, reference as ref
from tests.gpu_util import DEV, TOL, host, host_i, mar, need_lib, sample_rows, to_dev
from workloads.configs import CONFIGS, scaled
from workloads.gen import make_attn_inputs

pytestmark = pytest.mark.gpu

SMALL = scaled(CONFIGS[3], batch=2, seq=80, out_per_seq=20, hidden=256, n_q_heads=8, n_kv_heads=2,
               head_dim=32, lora_rank=8, est_rank=8, lora_alpha=16, seed=3003)


@functools.lru_cache(maxsize=2)
def _inputs(key):
    return make_attn_inputs(SMALL if key == "small" else CONFIGS[3])


def _run(key):
    need_lib()
    from contextual_sparsity_lora_amd.attn import SparseAttnProj
    cfg = SMALL if key == "small" else CONFIGS[3]
    inp = _inputs(key)
    dt = cfg.dtype
    d = {k: to_dev(v, dt) for k, v in inp.items()
         if isinstance(v, np.ndarray) and k.startswith(("x", "W_", "A_", "B_", "dy_"))}
    blk = SparseAttnProj(d["W_q"], d["W_k"], d["W_v"], d["W_o"], d["A_q"], d["B_q"], d["A_k"],
                         d["B_k"], d["A_v"], d["B_v"], d["A_o"], d["B_o"],
                         to_dev(np.ascontiguousarray(inp["WA_t_qkv"].T), "f32"),
                         to_dev(inp["WB_q"], "f32"), to_dev(inp["WB_k"], "f32"),
                         to_dev(inp["WB_v"], "f32"), inp["scale"], cfg.n_kv_heads, cfg.head_dim,
                         qk_sparsity=cfg.qk_sparsity, vo_sparsity=cfg.vo_sparsity)
    roles = to_dev(inp["roles"], None)
    blk.forward(d["x"], d["x_o"], roles, cfg.ctx_tokens)
    dqkv = torch.cat([d["dy_q"], d["dy_k"], d["dy_v"]], 1).contiguous()
    blk.backward(dqkv, d["dy_o"])
    torch.cuda.synchronize()
    return cfg, inp, blk


def _selection(cfg, inp):
    ctx, _ = ref.token_lists(inp["roles"])
    k, d = cfg.est_rank, cfg.head_dim
    n_rep = cfg.n_q_heads // cfg.n_kv_heads
    Ckv = cfg.n_kv_heads * d
    xa = csa.stage1(inp["x"], ctx, inp["WA_t_qkv"])
    sq = csa.ssq_l2(xa, inp["WB_q"], off=0)
    sk = csa.ssq_l2(xa, inp["WB_k"], off=k)
    idx_qk = csa.select(csa.qk_combine(sq, sk, cfg.n_kv_heads, n_rep, d), ref.n_keep(Ckv, *cfg.qk_sparsity))
    idx_vo = csa.select(csa.ssq_l2(xa, inp["WB_v"], off=2 * k), ref.n_keep(Ckv, *cfg.vo_sparsity))
    return idx_qk, idx_vo, n_rep, d


def _split_qkv(cfg, a):
    Cq, Ckv = cfg.n_q_heads * cfg.head_dim, cfg.n_kv_heads * cfg.head_dim
    return {"q": a[:, :Cq], "k": a[:, Cq:Cq + Ckv], "v": a[:, Cq + Ckv:]}


def test_attn_projections_small_end_to_end():
    cfg, inp, blk = _run("small")
    print("[attn] scaled GQA projections end to end", flush=True)
    idx_qk, idx_vo, n_rep, d = _selection(cfg, inp)
    assert np.array_equal(host_i(blk.idx_qk), idx_qk)
    assert np.array_equal(host_i(blk.idx_vo), idx_vo)
    f = ref.attn_proj_fwd(inp, idx_qk, idx_vo, n_rep, d)
    b = ref.attn_proj_bwd(inp, f, idx_qk, idx_vo, n_rep, d)
    tol = TOL[cfg.dtype]
    got = _split_qkv(cfg, host(blk.qkv))
    for p in "qkv":
        assert mar(got[p], f[p]) <= tol, p
    assert mar(host(blk.o), f["o"]) <= tol
    assert mar(host(blk.dx), b["dx"]) <= tol
    assert mar(host(blk.dx_o), b["dx_o"]) <= tol
    for p in "qkvo":
        assert mar(host(getattr(blk, "dA_" + p)), b["dA_" + p]) <= 1e-3, p
        assert mar(host(getattr(blk, "dB_" + p)), b["dB_" + p]) <= 1e-3, p


def test_attn_projections_full_size():
    cfg, inp, blk = _run("full")
    print("[attn] config 3 full size", flush=True)
    idx_qk, idx_vo, n_rep, d = _selection(cfg, inp)
    assert np.array_equal(host_i(blk.idx_qk), idx_qk)
    assert np.array_equal(host_i(blk.idx_vo), idx_vo)
    sel = ref.attn_proj_indices(idx_qk, idx_vo, n_rep, d)
    r, s, tol = cfg.lora_rank, inp["scale"], TOL["bf16"]
    ctx, out = ref.token_lists(inp["roles"])
    R = sample_rows(ctx, out, 40)
    rr = inp["roles"][R]
    x, xo = inp["x"], inp["x_o"]
    xl = host(blk.xl_qkv)
    assert mar(xl, x.astype(np.float64) @ np.concatenate([inp["A_" + p] for p in "qkv"]).T) <= 1e-5
    xl_o = host(blk.xl_o)
    assert mar(xl_o, xo.astype(np.float64) @ inp["A_o"].T) <= 1e-5
    got = _split_qkv(cfg, host(blk.qkv))
    for i, p in enumerate("qkv"):
        want = (ref.sparse_linear_fwd("out", x[R], inp["W_" + p], rr, sel[p])
                + s * (xl[R, i * r:(i + 1) * r] @ inp["B_" + p].T))
        assert mar(got[p][R], want) <= tol, p
    o_r = ref.sparse_linear_fwd("in", xo[R], inp["W_o"], rr, sel["o"]) + s * (xl_o[R] @ inp["B_o"].T)
    assert mar(host(blk.o)[R], o_r) <= tol
    dx_r = sum(ref.sparse_linear_bwd("out", inp["dy_" + p][R], inp["W_" + p], rr, sel[p])
               + s * ((inp["dy_" + p][R] @ inp["B_" + p]) @ inp["A_" + p]) for p in "qkv")
    assert mar(host(blk.dx)[R], dx_r) <= tol
    dxo_r = (ref.sparse_linear_bwd("in", inp["dy_o"][R], inp["W_o"], rr, sel["o"])
             + s * ((inp["dy_o"][R] @ inp["B_o"]) @ inp["A_o"]))
    assert mar(host(blk.dx_o)[R], dxo_r) <= tol
    for i, p in enumerate("qkv"):
        _, dA, dB = ref.lora_bwd(x, xl[:, i * r:(i + 1) * r], inp["dy_" + p], inp["A_" + p],
                                 inp["B_" + p], s)
        assert mar(host(getattr(blk, "dA_" + p)), dA) <= 1e-3, p
        assert mar(host(getattr(blk, "dB_" + p)), dB) <= 1e-3, p
    _, dA, dB = ref.lora_bwd(xo, xl_o, inp["dy_o"], inp["A_o"], inp["B_o"], s)
    assert mar(host(blk.dA_o), dA) <= 1e-3 and mar(host(blk.dB_o), dB) <= 1e-3
