"""GPU parity of the criterion ablations (random selection, exact-output
"oracle" criterion, head-level QK selection) against the CPU oracle: the
library's random draws, top-n, exact-output scores and head selection bit for
bit, and the FFN block and attention projections run with each criterion
against the oracle's block with the same selection.

For the exact-output criterion the oracle scores the GPU's own dense outputs
(teacher-forced; they are checked against the fp64 product separately), so the
selection is compared bit for bit."""
import numpy as np
import pytest
import torch

from oracle import csa, reference as ref
from tests.gpu_util import DEV, TOL, bits, empty_pad, host, host_i, mar, need_lib, to_dev
from tests.test_gpu_attn import SMALL, _inputs as _attn_inputs, _split_qkv
from workloads.configs import CONFIGS, scaled
from workloads.gen import make_ffn_inputs, round_dtype

pytestmark = pytest.mark.gpu


def _ops():
    need_lib()
    from contextual_sparsity_lora_amd import ops
    return ops


@pytest.mark.parametrize("seed,C", [(0, 3), (0, 14336), ((1 << 64) - 1, 1000), (12345, 28672)])
def test_random_scores_bits(seed, C):
    ops = _ops()
    s = torch.empty(C, dtype=torch.float32, device=DEV)
    ops.random_scores(seed, s)
    assert np.array_equal(bits(host(s)), bits(csa.random_scores(seed, C)))


@pytest.mark.parametrize("C,n", [(1000, 0), (1000, 1), (1000, 333), (1000, 1000), (14336, 4301), (17, 5),
                                 (32768, 9000), (40000, 12001)])
def test_select_top_bits(C, n, rng):
    ops = _ops()
    s = (rng.integers(0, 50, size=C) / 8.0).astype(np.float32)     # heavy ties
    if C > 100:
        s[rng.choice(C, 3, replace=False)] = [np.inf, np.nan, -np.inf]
    idx = torch.full((max(n, 1),), -1, dtype=torch.int32, device=DEV)
    ops.select_top(to_dev(s, "f32"), n, idx[:n] if n else idx[:0])
    torch.cuda.synchronize()
    assert np.array_equal(host_i(idx[:n]), csa.select(s, n))


@pytest.mark.parametrize("crit,dtype", [("l2", "f32"), ("l2", "bf16"), ("swiglu", "f32"),
                                        ("swiglu", "bf16"), ("qk", "bf16"), ("qk", "f32")])
def test_dense_scores_bits(crit, dtype, rng):
    """Exact-output criteria over a ragged row subset and a ragged channel
    count, inputs as column slices of wider buffers."""
    ops = _ops()
    T, H, n_rep, d = 777, 5, 3, 24
    C = H * d if crit == "qk" else 1003
    W0 = C * n_rep if crit == "qk" else C
    print(f"[dense-scores] {crit} {dtype} C={C}", flush=True)
    buf = round_dtype(rng.standard_normal((T, W0 + C + 16)) * 2.0, dtype)
    rows = np.sort(rng.choice(T, 611, replace=False)).astype(np.int32)
    bd = to_dev(buf, dtype)
    Y0, Y1 = bd[:, :W0], bd[:, W0:W0 + C]
    sc = torch.empty(C, dtype=torch.float32, device=DEV)
    if crit == "l2":
        ops.dense_scores("l2", Y0, None, to_dev(rows, None), sc)
    else:
        ops.dense_scores(crit, Y0, Y1, to_dev(rows, None), sc, C=C, n_rep=n_rep, head_dim=d)
    want = csa.dense_scores(crit, buf[:, :W0], buf[:, W0:W0 + C], rows, H, n_rep, d)
    assert np.array_equal(bits(host(sc)), bits(want))
    # no context rows: zeros
    ops.dense_scores("l2", Y0, None, to_dev(rows[:0], None), sc)
    assert np.all(host(sc) == 0.0)


@pytest.mark.parametrize("H,d,keep", [(8, 128, 4), (32, 16, 1), (40, 128, 20), (8, 128, 8), (8, 128, 0)])
def test_select_heads_bits(H, d, keep, rng):
    ops = _ops()
    s = (rng.integers(0, 5, size=H * d) / 4.0).astype(np.float32)
    idx = torch.full((max(keep * d, 1),), -1, dtype=torch.int32, device=DEV)
    ops.select_heads(to_dev(s, "f32"), H, d, keep, idx)
    torch.cuda.synchronize()
    assert np.array_equal(host_i(idx[:keep * d]), csa.select_heads(s, H, d, keep))


def _ffn_block(cfg, inp, criterion, seed=0):
    from contextual_sparsity_lora_amd.ffn import SparseFFN
    dt = cfg.dtype
    d = {k: to_dev(v, dt) for k, v in inp.items()
         if k in ("x", "W_gate", "W_up", "W_down", "A_gate", "B_gate", "A_up", "B_up", "A_down",
                  "B_down", "dy")}
    blk = SparseFFN(d["W_gate"], d["W_up"], d["W_down"], d["A_gate"], d["B_gate"], d["A_up"],
                    d["B_up"], d["A_down"], d["B_down"], None, None, None, inp["scale"],
                    sparsity=cfg.ffn_sparsity, criterion=criterion, seed=seed)
    roles = to_dev(inp["roles"], None)
    blk.forward(d["x"], roles, cfg.ctx_tokens)
    blk.backward(d["dy"])
    torch.cuda.synchronize()
    return blk, d


@pytest.mark.parametrize("case", ["f32", "bf16"])
@pytest.mark.parametrize("criterion", ["oracle", "random"])
def test_ffn_block_with_criterion(case, criterion):
    ops = _ops()
    if case == "f32":
        cfg = CONFIGS[1]
    else:
        cfg = scaled(CONFIGS[2], batch=2, seq=160, out_per_seq=40, hidden=520, inter=1400)
    inp = make_ffn_inputs(cfg, with_factors=False)
    print(f"[ffn-criterion] {criterion} {case}", flush=True)
    blk, d = _ffn_block(cfg, inp, criterion, seed=77)
    F, tol = cfg.inter, TOL[cfg.dtype]
    n = ref.n_keep(F, *cfg.ffn_sparsity)
    ctx, _ = ref.token_lists(inp["roles"])
    if criterion == "random":
        assert blk.last_seed == 77
        idx = csa.select(csa.random_scores(77, F), n)
    else:
        # the block's exact gate|up outputs, recomputed by the same call
        gu = torch.empty(cfg.tokens, 2 * F, dtype=d["x"].dtype, device=DEV)
        ops.sparse_linear_fwd("out", d["x"], blk.W_gu, None, blk.ctx_rows, blk.out_rows, blk.idx_all, gu)
        torch.cuda.synchronize()
        G, U = host(gu[:, :F]), host(gu[:, F:])
        x64 = inp["x"].astype(np.float64)
        assert mar(G, x64 @ inp["W_gate"].T) <= tol and mar(U, x64 @ inp["W_up"].T) <= tol
        idx = csa.select(csa.dense_scores("swiglu", G, U, ctx), n)
    assert np.array_equal(host_i(blk.idx), idx)
    f = ref.ffn_block_fwd(inp, idx)
    b = ref.ffn_block_bwd(inp, f, idx)
    assert mar(host(blk.y), f["y"]) <= tol
    assert mar(host(blk.dx), b["dx"]) <= tol
    for p in ("gate", "up", "down"):
        assert mar(host(getattr(blk, "dA_" + p)), b["dA_" + p]) <= max(tol, 1e-3), p
        assert mar(host(getattr(blk, "dB_" + p)), b["dB_" + p]) <= max(tol, 1e-3), p


@pytest.mark.parametrize("criterion", ["oracle", "random", "head"])
def test_attn_projections_with_criterion(criterion):
    ops = _ops()
    from contextual_sparsity_lora_amd.attn import SparseAttnProj
    cfg, inp = SMALL, _attn_inputs("small")
    print(f"[attn-criterion] {criterion}", flush=True)
    dt = cfg.dtype
    dd = {k: to_dev(v, dt) for k, v in inp.items()
          if isinstance(v, np.ndarray) and k.startswith(("x", "W_", "A_", "B_", "dy_"))}
    fac = (to_dev(np.ascontiguousarray(inp["WA_t_qkv"].T), "f32"), to_dev(inp["WB_q"], "f32"),
           to_dev(inp["WB_k"], "f32"), to_dev(inp["WB_v"], "f32"))
    blk = SparseAttnProj(dd["W_q"], dd["W_k"], dd["W_v"], dd["W_o"], dd["A_q"], dd["B_q"], dd["A_k"],
                         dd["B_k"], dd["A_v"], dd["B_v"], dd["A_o"], dd["B_o"], *fac, inp["scale"],
                         cfg.n_kv_heads, cfg.head_dim, qk_sparsity=cfg.qk_sparsity,
                         vo_sparsity=cfg.vo_sparsity, criterion=criterion, seed=5)
    roles = to_dev(inp["roles"], None)
    blk.forward(dd["x"], dd["x_o"], roles, cfg.ctx_tokens)
    dqkv = torch.cat([dd["dy_q"], dd["dy_k"], dd["dy_v"]], 1).contiguous()
    blk.backward(dqkv, dd["dy_o"])
    torch.cuda.synchronize()
    H, dh = cfg.n_kv_heads, cfg.head_dim
    n_rep = cfg.n_q_heads // H
    Ckv, Cq = H * dh, cfg.n_q_heads * dh
    ctx, _ = ref.token_lists(inp["roles"])
    n_qk, n_vo = ref.n_keep(Ckv, *cfg.qk_sparsity), ref.n_keep(Ckv, *cfg.vo_sparsity)
    k = cfg.est_rank
    if criterion == "random":
        idx_qk = csa.select(csa.random_scores(5, Ckv), n_qk)
        idx_vo = csa.select(csa.random_scores(5 + (1 << 32), Ckv), n_vo)
    elif criterion == "head":
        xa = csa.stage1(inp["x"], ctx, inp["WA_t_qkv"])
        sq, sk = csa.ssq_l2(xa, inp["WB_q"], off=0), csa.ssq_l2(xa, inp["WB_k"], off=k)
        idx_qk = csa.select_heads(csa.qk_combine(sq, sk, H, n_rep, dh), H, dh, ref.n_keep(H, *cfg.qk_sparsity))
        idx_vo = csa.select(csa.ssq_l2(xa, inp["WB_v"], off=2 * k), n_vo)
    else:
        qkv = torch.empty(cfg.tokens, blk.Cs, dtype=dd["x"].dtype, device=DEV)
        ops.sparse_linear_fwd("out", dd["x"], blk.W_qkv, None, blk.ctx_rows, blk.out_rows, blk.idx_all, qkv)
        torch.cuda.synchronize()
        Y = host(qkv)
        Wqkv = np.concatenate([inp["W_q"], inp["W_k"], inp["W_v"]]).astype(np.float64)
        assert mar(Y, inp["x"].astype(np.float64) @ Wqkv.T) <= TOL[dt]
        idx_qk = csa.select(csa.dense_scores("qk", Y[:, :Cq], Y[:, Cq:Cq + Ckv], ctx, H, n_rep, dh), n_qk)
        idx_vo = csa.select(csa.dense_scores("l2", Y[:, Cq + Ckv:], None, ctx), n_vo)
    assert np.array_equal(host_i(blk.idx_qk), idx_qk)
    assert np.array_equal(host_i(blk.idx_vo), idx_vo)
    f = ref.attn_proj_fwd(inp, idx_qk, idx_vo, n_rep, dh)
    b = ref.attn_proj_bwd(inp, f, idx_qk, idx_vo, n_rep, dh)
    tol = TOL[dt]
    got = _split_qkv(cfg, host(blk.qkv))
    for p in "qkv":
        assert mar(got[p], f[p]) <= tol, p
    assert mar(host(blk.o), f["o"]) <= tol
    assert mar(host(blk.dx), b["dx"]) <= tol
    for p in "qkvo":
        assert mar(host(getattr(blk, "dA_" + p)), b["dA_" + p]) <= 1e-3, p
        assert mar(host(getattr(blk, "dB_" + p)), b["dB_" + p]) <= 1e-3, p
