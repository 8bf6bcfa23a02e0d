"""GPU parity of the selection path (token split, estimator, criteria, top-n,
index propagation): bit-exact against the CPU oracle."""
import numpy as np
import pytest
import torch

from oracle import csa, reference as ref
from tests.gpu_util import DEV, bits, host, host_i, need_lib, to_dev
from workloads.configs import CONFIGS
from workloads.gen import make_attn_inputs, make_ffn_inputs, round_dtype

pytestmark = pytest.mark.gpu


def _ops():
    need_lib()
    from contextual_sparsity_lora_amd import ops
    return ops


def _split(ops, roles):
    ctx, out = ref.token_lists(roles)
    r = to_dev(roles, None)
    c = torch.empty(len(ctx), dtype=torch.int32, device=DEV)
    o = torch.empty(len(out), dtype=torch.int32, device=DEV)
    ops.token_split(r, c, o)
    return ctx, out, c, o


@pytest.mark.parametrize("cid", [1, 2])
def test_ffn_selection_bit_exact(cid):
    ops = _ops()
    cfg = CONFIGS[cid]
    inp = make_ffn_inputs(cfg)
    print(f"[select] config {cid} T={cfg.tokens} F={cfg.inter}", flush=True)
    ctx, out, c_d, o_d = _split(ops, inp["roles"])
    assert np.array_equal(host_i(c_d), ctx) and np.array_equal(host_i(o_d), out)
    x = to_dev(inp["x"], cfg.dtype)
    WA = to_dev(np.ascontiguousarray(inp["WA_t_gu"].T), "f32")
    k = cfg.est_rank
    xa = torch.empty(len(ctx), 2 * k, dtype=torch.float32, device=DEV)
    ops.svd_estimate(x, c_d, WA, xa)
    xa_ref = csa.stage1(inp["x"], ctx, inp["WA_t_gu"])
    assert np.array_equal(bits(host(xa)), bits(xa_ref))
    n = ref.n_keep(cfg.inter, *cfg.ffn_sparsity)
    sc = torch.empty(cfg.inter, dtype=torch.float32, device=DEV)
    idx = torch.empty(n, dtype=torch.int32, device=DEV)
    WBg, WBu = to_dev(inp["WB_gate"], "f32"), to_dev(inp["WB_up"], "f32")
    ops.score_select("swiglu", xa, WBg, WBu, n, idx, scores=sc)
    sc_ref = csa.ssq_swiglu(xa_ref, inp["WB_gate"], inp["WB_up"])
    assert np.array_equal(bits(host(sc)), bits(sc_ref))
    idx_ref = csa.select(sc_ref, n)
    assert np.array_equal(host_i(idx), idx_ref)
    # stacked index for gate|up
    idx2 = torch.empty(2 * n, dtype=torch.int32, device=DEV)
    ops.stack_index(idx, cfg.inter, 2, idx2)
    assert np.array_equal(host_i(idx2), np.concatenate([idx_ref, idx_ref + cfg.inter]))


def test_attention_selection_bit_exact_gqa():
    ops = _ops()
    cfg = CONFIGS[3]
    inp = make_attn_inputs(cfg)
    print("[select] config 3 (QK, VO, GQA 32/8)", flush=True)
    ctx, out, c_d, o_d = _split(ops, inp["roles"])
    k, d = cfg.est_rank, cfg.head_dim
    n_rep = cfg.n_q_heads // cfg.n_kv_heads
    Ckv = cfg.n_kv_heads * d
    x = to_dev(inp["x"], cfg.dtype)
    WA = to_dev(np.ascontiguousarray(inp["WA_t_qkv"].T), "f32")
    xa = torch.empty(len(ctx), 3 * k, dtype=torch.float32, device=DEV)
    ops.svd_estimate(x, c_d, WA, xa)
    xa_ref = csa.stage1(inp["x"], ctx, inp["WA_t_qkv"])
    assert np.array_equal(bits(host(xa)), bits(xa_ref))
    # QK criterion in key/value channel space
    n_qk = ref.n_keep(Ckv, *cfg.qk_sparsity)
    sc = torch.empty(Ckv, dtype=torch.float32, device=DEV)
    idx = torch.empty(n_qk, dtype=torch.int32, device=DEV)
    ops.score_select("qk", xa, to_dev(inp["WB_q"], "f32"), to_dev(inp["WB_k"], "f32"), n_qk, idx,
                     scores=sc, off0=0, off1=k, C=Ckv, n_rep=n_rep, head_dim=d)
    sq = csa.ssq_l2(xa_ref, inp["WB_q"], off=0)
    sk = csa.ssq_l2(xa_ref, inp["WB_k"], off=k)
    sc_ref = csa.qk_combine(sq, sk, cfg.n_kv_heads, n_rep, d)
    assert np.array_equal(bits(host(sc)), bits(sc_ref))
    idx_ref = csa.select(sc_ref, n_qk)
    assert np.array_equal(host_i(idx), idx_ref)
    iq = torch.empty(n_qk * n_rep, dtype=torch.int32, device=DEV)
    ops.expand_gqa(idx, n_rep, d, iq)
    assert np.array_equal(host_i(iq), ref.expand_gqa(idx_ref, n_rep, d))
    # VO criterion: L2 of the estimated values
    n_vo = ref.n_keep(Ckv, *cfg.vo_sparsity)
    idv = torch.empty(n_vo, dtype=torch.int32, device=DEV)
    ops.score_select("l2", xa, to_dev(inp["WB_v"], "f32"), None, n_vo, idv, scores=sc, off0=2 * k)
    sv_ref = csa.ssq_l2(xa_ref, inp["WB_v"], off=2 * k)
    assert np.array_equal(bits(host(sc)), bits(sv_ref))
    assert np.array_equal(host_i(idv), csa.select(sv_ref, n_vo))


def _score_case(ops, xa_np, WB0, WB1, n, crit="swiglu", off1=None):
    xa = to_dev(xa_np, "f32")
    C = WB0.shape[1]
    sc = torch.empty(C, dtype=torch.float32, device=DEV)
    idx = torch.empty(max(n, 1), dtype=torch.int32, device=DEV)
    k = WB0.shape[0]
    ops.score_select(crit, xa, to_dev(WB0, "f32"), None if WB1 is None else to_dev(WB1, "f32"),
                     n, idx[:n] if n else idx[:0], scores=sc, off0=0,
                     off1=(k if off1 is None else off1))
    if crit == "swiglu":
        sref = csa.ssq_swiglu(xa_np, WB0, WB1)
    else:
        sref = csa.ssq_l2(xa_np, WB0)
    assert np.array_equal(csa.keys(host(sc)), csa.keys(sref))   # bit patterns, NaN canonical
    assert np.array_equal(host_i(idx[:n]), csa.select(sref, n))


def test_selection_edge_cases(rng):
    ops = _ops()
    print("[select] edge cases", flush=True)
    # ragged sizes, generic k, n = 0 / 1 / C
    for Tc, k, C in ((130, 5, 100), (1, 16, 64), (64, 8, 65), (200, 3, 1)):
        xa = rng.standard_normal((Tc, 2 * k)).astype(np.float32)
        WBg = rng.standard_normal((k, C)).astype(np.float32)
        WBu = rng.standard_normal((k, C)).astype(np.float32)
        for n in sorted({0, 1, C // 2, C}):
            _score_case(ops, xa, WBg, WBu, n)
            _score_case(ops, xa, WBg, None, n, crit="l2")
    # exact ties: duplicated W_B columns give equal scores -> lower index first
    k, C, Tc = 4, 96, 70
    xa = rng.standard_normal((Tc, 2 * k)).astype(np.float32)
    base = rng.standard_normal((k, 12)).astype(np.float32)
    WB = np.ascontiguousarray(np.tile(base, (1, 8)))
    for n in (5, 12, 13, 50):
        _score_case(ops, xa, WB, WB, n)
    # overflow to +inf scores (ties among infinities)
    WBbig = (rng.standard_normal((k, C)) * 1e18).astype(np.float32)
    _score_case(ops, xa, WBbig, WBbig, 30)
    # no context tokens: all scores +0, the n lowest channel indices win
    xa0 = np.zeros((0, 2 * k), np.float32)
    _score_case(ops, xa0, WB, WB, 7)


def test_token_split_edge_cases(rng):
    ops = _ops()
    for roles in (np.zeros(5, np.uint8), np.ones(7, np.uint8),
                  (rng.random(3001) < 0.3).astype(np.uint8), np.array([0, 2, 0, 255], np.uint8)):
        ctx, out, c, o = _split(ops, roles)
        assert np.array_equal(host_i(c), ctx) and np.array_equal(host_i(o), out)
    ops.sync(0)


def test_estimator_bf16_and_f32_inputs_ragged(rng):
    ops = _ops()
    for dtype in ("bf16", "f32"):
        for T, D, kt in ((70, 200, 7), (130, 4104, 48), (9, 64, 128)):
            x = round_dtype(rng.standard_normal((T, D)), dtype)
            WA_t = rng.standard_normal((kt, D)).astype(np.float32)
            rows = np.sort(rng.choice(T, max(1, T // 2), replace=False)).astype(np.int32)
            xa = torch.empty(len(rows), kt, dtype=torch.float32, device=DEV)
            ops.svd_estimate(to_dev(x, dtype), to_dev(rows, None), to_dev(np.ascontiguousarray(WA_t.T), "f32"), xa)
            assert np.array_equal(bits(host(xa)), bits(csa.stage1(x, rows, WA_t)))


@pytest.mark.parametrize("n_kv,n_rep,d,fq,fv", [(8, 4, 128, 0.5, 0.5), (2, 1, 64, 1.0, 0.25), (4, 2, 32, 0.3, 0.0),
                                                (1, 8, 16, 0.0, 1.0)])
def test_qkv_index(n_kv, n_rep, d, fq, fv, rng):
    """One-call q|k|v index lists: GQA expansions and the stacked list, bit-exact
    against the oracle's expansion and the stacking offsets."""
    need_lib()
    from contextual_sparsity_lora_amd import ops
    Ckv = n_kv * d
    Cq = n_rep * Ckv
    n_qk, n_vo = int(round(fq * Ckv)), int(round(fv * Ckv))
    iqk = np.sort(rng.choice(Ckv, n_qk, replace=False)).astype(np.int32)
    ivo = np.sort(rng.choice(Ckv, n_vo, replace=False)).astype(np.int32)
    dev = lambda a: torch.from_numpy(a).to(DEV)
    iq = torch.full((n_qk * n_rep,), -1, dtype=torch.int32, device=DEV)
    io = torch.full((n_vo * n_rep,), -1, dtype=torch.int32, device=DEV)
    iqkv = torch.full((n_qk * n_rep + n_qk + n_vo,), -1, dtype=torch.int32, device=DEV)
    ops.qkv_index(dev(iqk), dev(ivo), n_kv, n_rep, d, iq, io, iqkv)
    eq, eo = ref.expand_gqa(iqk, n_rep, d), ref.expand_gqa(ivo, n_rep, d)
    assert np.array_equal(host_i(iq), eq)
    assert np.array_equal(host_i(io), eo)
    assert np.array_equal(host_i(iqkv), np.concatenate([eq, iqk + Cq, ivo + Cq + Ckv]))


def test_full_rank_estimator_bit_exact_and_matches_exact_criterion():
    """The estimator at full rank (k = D = 256 at the fp32 FFN shape; W_A has
    2k = 512 columns): the library's stage-1 products, SwiGLU-L2 scores and
    selection equal the oracle's bit for bit, and the scores follow the exact
    (dense-output) criterion within fp32 rounding, so the selection is the
    exact criterion's wherever its n-th and (n+1)-th scores are apart."""
    import dataclasses
    from tests.test_oracle_score import _margin_ok, _top_set
    ops = _ops()
    cfg = dataclasses.replace(CONFIGS[1], est_rank=CONFIGS[1].hidden)
    inp = make_ffn_inputs(cfg)
    k = cfg.est_rank
    print(f"[select] config 1 at full rank k={k}", flush=True)
    ctx, out, c_d, o_d = _split(ops, inp["roles"])
    x = to_dev(inp["x"], cfg.dtype)
    WA = to_dev(np.ascontiguousarray(inp["WA_t_gu"].T), "f32")
    xa = torch.empty(len(ctx), 2 * k, dtype=torch.float32, device=DEV)
    ops.svd_estimate(x, c_d, WA, xa)
    xa_ref = csa.stage1(inp["x"], ctx, inp["WA_t_gu"])
    assert np.array_equal(bits(host(xa)), bits(xa_ref))
    n = ref.n_keep(cfg.inter, *cfg.ffn_sparsity)
    sc = torch.empty(cfg.inter, dtype=torch.float32, device=DEV)
    idx = torch.empty(n, dtype=torch.int32, device=DEV)
    ops.score_select("swiglu", xa, to_dev(inp["WB_gate"], "f32"), to_dev(inp["WB_up"], "f32"), n, idx,
                     scores=sc, off0=0, off1=k)
    sc_ref = csa.ssq_swiglu(xa_ref, inp["WB_gate"], inp["WB_up"])
    got = host(sc)
    assert np.array_equal(bits(got), bits(sc_ref))
    assert np.array_equal(host_i(idx), csa.select(sc_ref, n))
    xc = inp["x"][ctx].astype(np.float64)
    h = ref.silu(xc @ inp["W_gate"].T.astype(np.float64)) * (xc @ inp["W_up"].T.astype(np.float64))
    s64 = np.sum(h * h, axis=0)
    assert np.allclose(got, s64, rtol=1e-3, atol=0)
    if _margin_ok(s64, n, 1e-3):
        assert np.array_equal(host_i(idx), _top_set(s64, n))


def test_r64_rounding_order_golden_on_gpu():
    """The estimator's stage-1 reduction on the hand-derived R64 cases (fp32
    x row = the a terms, W_A column = the b terms): the GPU gives exactly the
    canonical value of each case."""
    import json
    import os
    ops = _ops()
    with open(os.path.join(os.path.dirname(__file__), "golden", "r64_order.json")) as f:
        cases = json.load(f)["cases"]
    print("[select] R64 rounding-order goldens", flush=True)
    for case in cases:
        L = case["L"]
        a = np.zeros((1, L), np.float32)
        b = np.zeros((L, 4), np.float32)      # four identical W_A columns
        for m, av, bv in case["terms"]:
            a[0, m], b[m, :] = av, bv
        x = torch.zeros(1, (L + 3) // 4 * 4, dtype=torch.float32, device=DEV)
        x[:, :L] = torch.from_numpy(a).to(DEV)
        rows = torch.zeros(1, dtype=torch.int32, device=DEV)
        xa = torch.empty(1, 4, dtype=torch.float32, device=DEV)
        ops.svd_estimate(x[:, :L], rows, to_dev(b, "f32"), xa)
        torch.cuda.synchronize()
        got = host(xa)[0]
        want = np.float32(case["r64"])
        assert np.all(got.view(np.uint32) == want.view(np.uint32)), (case["name"], got, want)
