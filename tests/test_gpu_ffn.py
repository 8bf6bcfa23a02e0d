"""GPU parity of the whole sparse SwiGLU FFN block, forward and backward
(selection + gathered GEMMs + dense LoRA + SwiGLU), against the CPU oracle.

The fp32 block is compared end to end.  The full-size bf16 block is compared
op by op (each GPU op against the oracle applied to that op's GPU inputs) on a
sample of context and output rows, plus every LoRA gradient in full, and end
to end on the sampled rows."""
import functools

import numpy as np
import pytest
import torch

from oracle import csa, reference as ref
from tests.gpu_util import DEV, TOL, host, host_i, mar, need_lib, sample_rows, to_dev
from workloads.configs import CONFIGS
from workloads.gen import make_ffn_inputs

pytestmark = pytest.mark.gpu


@functools.lru_cache(maxsize=2)
def _inputs(cid):
    return make_ffn_inputs(CONFIGS[cid])


def _run(cid, keep_h=True, compact_ctx=None):
    need_lib()
    from contextual_sparsity_lora_amd.ffn import SparseFFN
    cfg = CONFIGS[cid]
    inp = _inputs(cid)
    dt = cfg.dtype
    d = {k: to_dev(v, dt) for k, v in inp.items()
         if k in ("x", "W_gate", "W_up", "W_down", "A_gate", "B_gate", "A_up", "B_up", "A_down",
                  "B_down", "dy")}
    blk = SparseFFN(d["W_gate"], d["W_up"], d["W_down"], d["A_gate"], d["B_gate"], d["A_up"],
                    d["B_up"], d["A_down"], d["B_down"],
                    to_dev(np.ascontiguousarray(inp["WA_t_gu"].T), "f32"),
                    to_dev(inp["WB_gate"], "f32"), to_dev(inp["WB_up"], "f32"), inp["scale"],
                    sparsity=cfg.ffn_sparsity)
    blk.keep_h = keep_h      # h of the context rows as well (checked below)
    if compact_ctx is not None:
        blk.compact_ctx = compact_ctx
    roles = to_dev(inp["roles"], None)
    y = blk.forward(d["x"], roles, cfg.ctx_tokens)
    dx = blk.backward(d["dy"])
    torch.cuda.synchronize()
    return cfg, inp, blk, y, dx


def _selection(cfg, inp):
    ctx, _ = ref.token_lists(inp["roles"])
    xa = csa.stage1(inp["x"], ctx, inp["WA_t_gu"])
    sc = csa.ssq_swiglu(xa, inp["WB_gate"], inp["WB_up"])
    return csa.select(sc, ref.n_keep(cfg.inter, *cfg.ffn_sparsity))


def test_ffn_block_f32_end_to_end():
    cfg, inp, blk, y, dx = _run(1)
    print("[ffn] config 1 end to end", flush=True)
    idx = _selection(cfg, inp)
    assert np.array_equal(host_i(blk.idx), idx)
    f = ref.ffn_block_fwd(inp, idx)
    b = ref.ffn_block_bwd(inp, f, idx)
    tol = TOL["f32"]
    F = cfg.inter
    assert mar(host(blk.gu[:, :F]), f["g"]) <= tol
    assert mar(host(blk.gu[:, F:]), f["u"]) <= tol
    assert mar(host(blk.h), f["h"]) <= tol
    assert mar(host(y), f["y"]) <= tol
    assert mar(host(blk.dh), b["dh"]) <= tol
    assert mar(host(blk.dgu[:, :F]), b["dg"]) <= tol
    assert mar(host(blk.dgu[:, F:]), b["du"]) <= tol
    assert mar(host(dx), b["dx"]) <= tol
    for p in ("gate", "up", "down"):
        assert mar(host(getattr(blk, "dA_" + p)), b["dA_" + p]) <= tol, p
        assert mar(host(getattr(blk, "dB_" + p)), b["dB_" + p]) <= tol, p


def test_ffn_block_bf16_full_size():
    _full_size_checks(compact_ctx=False)


def _full_size_checks(compact_ctx):
    cfg, inp, blk, y, dx = _run(2, compact_ctx=compact_ctx)
    print(f"[ffn] config 2 full size (compact context rows: {compact_ctx})", flush=True)
    F, r, s = cfg.inter, cfg.lora_rank, inp["scale"]
    tol = TOL["bf16"]
    idx = _selection(cfg, inp)
    assert np.array_equal(host_i(blk.idx), idx)
    ctx, out = ref.token_lists(inp["roles"])
    # sampled rows plus every row of whole 256-row M-tiles of the products:
    # the first and last tiles of the context-row products (the last ones
    # run as split-tail tiles) and the last tile of the output-row products
    R = np.unique(np.concatenate([sample_rows(ctx, out, 40), ctx[:256], ctx[-256:], out[-256:]]))
    rr = inp["roles"][R]
    x = inp["x"]
    g_d, u_d = host(blk.gu[:, :F]), host(blk.gu[:, F:])
    h_d, dh_d = host(blk.h), host(blk.dh)
    dg_d, du_d = host(blk.dgu[:, :F]), host(blk.dgu[:, F:])
    xl_gu = host(blk.xl_gu)
    xl_dn = host(blk.xl_dn)
    # LoRA down-projections (full)
    assert mar(xl_gu[:, :r], x.astype(np.float64) @ inp["A_gate"].T) <= 1e-5
    assert mar(xl_gu[:, r:], x.astype(np.float64) @ inp["A_up"].T) <= 1e-5
    assert mar(xl_dn, h_d.astype(np.float64) @ inp["A_down"].T) <= 1e-5
    # per-op checks on sampled rows, each against the oracle on the GPU's inputs
    g_r = ref.sparse_linear_fwd("out", x[R], inp["W_gate"], rr, idx) + s * (xl_gu[R, :r] @ inp["B_gate"].T)
    u_r = ref.sparse_linear_fwd("out", x[R], inp["W_up"], rr, idx) + s * (xl_gu[R, r:] @ inp["B_up"].T)
    assert mar(g_d[R], g_r) <= tol and mar(u_d[R], u_r) <= tol
    assert mar(h_d[R], ref.swiglu_fwd(g_d[R], u_d[R])) <= tol
    y_r = ref.sparse_linear_fwd("in", h_d[R], inp["W_down"], rr, idx) + s * (xl_dn[R] @ inp["B_down"].T)
    assert mar(host(y)[R], y_r) <= tol
    dy = inp["dy"]
    dh_r = ref.sparse_linear_bwd("in", dy[R], inp["W_down"], rr, idx) + s * ((dy[R] @ inp["B_down"]) @ inp["A_down"])
    assert mar(dh_d[R], dh_r) <= tol
    dg_r, du_r = ref.swiglu_bwd(dh_d[R], g_d[R], u_d[R])
    assert mar(dg_d[R], dg_r) <= tol and mar(du_d[R], du_r) <= tol
    dx_r = (ref.sparse_linear_bwd("out", dg_d[R], inp["W_gate"], rr, idx)
            + ref.sparse_linear_bwd("out", du_d[R], inp["W_up"], rr, idx)
            + s * ((dg_d[R] @ inp["B_gate"]) @ inp["A_gate"]) + s * ((du_d[R] @ inp["B_up"]) @ inp["A_up"]))
    assert mar(host(dx)[R], dx_r) <= tol
    # LoRA gradients in full, from the GPU's inputs to the backward op
    _, dA, dB = ref.lora_bwd(h_d, xl_dn, dy, inp["A_down"], inp["B_down"], s)
    assert mar(host(blk.dA_down), dA) <= 1e-3 and mar(host(blk.dB_down), dB) <= 1e-3
    _, dA, dB = ref.lora_bwd(x, xl_gu[:, :r], dg_d, inp["A_gate"], inp["B_gate"], s)
    assert mar(host(blk.dA_gate), dA) <= 1e-3 and mar(host(blk.dB_gate), dB) <= 1e-3
    _, dA, dB = ref.lora_bwd(x, xl_gu[:, r:], du_d, inp["A_up"], inp["B_up"], s)
    assert mar(host(blk.dA_up), dA) <= 1e-3 and mar(host(blk.dB_up), dB) <= 1e-3
    # end to end on the sampled rows (oracle intermediates in fp64)
    sub = dict(inp)
    sub["x"], sub["roles"], sub["dy"] = x[R], rr, dy[R]
    f = ref.ffn_block_fwd(sub, idx)
    assert mar(host(y)[R], f["y"]) <= tol
    b = ref.ffn_block_bwd(sub, f, idx)
    assert mar(host(dx)[R], b["dx"]) <= tol


def test_ffn_block_compact_context_rows():
    """The compact context-row path stores h of the context rows only
    compactly (the down product's operand): the same outputs and gradients
    bit for bit as with the whole rows kept, hc equal to those rows' selected
    channels (padding columns zero), and the per-op checks of the full-size
    test hold on it as well."""
    cfg, inp, blk, y, dx = _run(2, keep_h=True, compact_ctx=True)
    print("[ffn] config 2 compact context rows", flush=True)
    if not blk._compact:
        pytest.skip("the block does not take the compact context-row path here")
    ctx, _ = ref.token_lists(inp["roles"])
    n = blk.n
    idx = host_i(blk.idx)
    hc = host(blk.hc)
    h = host(blk.h)
    assert np.array_equal(hc[:, :n], h[ctx][:, idx])
    assert np.all(hc[:, n:] == 0.0)
    ref_out = {k: host(getattr(blk, k)).copy() for k in ("y", "dx", "gu", "dgu", "dA_gate", "dB_gate", "dA_up",
                                                          "dB_up", "dA_down", "dB_down")}
    blk.keep_h = False
    roles = to_dev(inp["roles"], None)
    d = {k: to_dev(inp[k], cfg.dtype) for k in ("x", "dy")}
    blk.forward(d["x"], roles, cfg.ctx_tokens)
    blk.backward(d["dy"])
    torch.cuda.synchronize()
    for k, v in ref_out.items():
        assert np.array_equal(host(getattr(blk, k)), v), k


def test_ffn_block_bf16_full_size_compact_path():
    """The full-size per-op checks on the compact context-row path."""
    _full_size_checks(compact_ctx=True)
