"""HIP graph replay of whole block steps (contextual_sparsity_lora_amd.graph.
StepGraph): a captured forward + backward, replayed several times with eager
steps and synchronisations between the replays, reproduces the eager step bit
for bit every time (every kernel of a step is deterministic), for the sparse
FFN block and the sparse q/k/v/o projections at small bf16 shapes.  The
outputs are cleared before each replay, so a replay that wrote nothing would
fail."""
import numpy as np
import pytest
import torch

from tests.gpu_util import bits, need_lib, to_dev
from workloads.configs import CONFIGS, scaled
from workloads.gen import make_attn_inputs, make_ffn_inputs

pytestmark = pytest.mark.gpu


def _snap(ts):
    return [bits(t.float().cpu().numpy()) if t.is_floating_point() else t.cpu().numpy() for t in ts]


def _check_replays(step, outs, side):
    from contextual_sparsity_lora_amd.graph import StepGraph
    step()
    torch.cuda.synchronize()
    want = _snap(outs)
    g = StepGraph(step, side_streams=side)
    try:
        _replays(g, step, outs, want)
    finally:
        g.close()


def _replays(g, step, outs, want):
    for rep in range(3):
        for t in outs:
            if t.is_floating_point():
                t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _snap(outs)
        for i, (a, b) in enumerate(zip(got, want)):
            assert np.array_equal(a, b), f"replay {rep}: output {i} differs from the eager step"
        step()   # eager work between replays
        torch.cuda.synchronize()
        got = _snap(outs)
        for i, (a, b) in enumerate(zip(got, want)):
            assert np.array_equal(a, b), f"eager step after replay {rep}: output {i} differs"


def test_ffn_step_graph_replays():
    need_lib()
    from contextual_sparsity_lora_amd.ffn import SparseFFN
    print("[graph] ffn block", flush=True)
    cfg = scaled(CONFIGS[2], batch=2, seq=96, out_per_seq=24, hidden=256, inter=640, seed=2002)
    inp = make_ffn_inputs(cfg)
    d = {k: to_dev(v, "bf16") for k, v in inp.items()
         if isinstance(v, np.ndarray) and k.startswith(("x", "W_", "A_", "B_", "dy"))}
    blk = SparseFFN(d["W_gate"], d["W_up"], d["W_down"], d["A_gate"], d["B_gate"], d["A_up"], d["B_up"],
                    d["A_down"], d["B_down"], to_dev(np.ascontiguousarray(inp["WA_t_gu"].T), "f32"),
                    to_dev(inp["WB_gate"], "f32"), to_dev(inp["WB_up"], "f32"), inp["scale"],
                    sparsity=cfg.ffn_sparsity)
    roles = to_dev(inp["roles"], None)
    step = lambda: (blk.forward(d["x"], roles, cfg.ctx_tokens), blk.backward(d["dy"]))
    step()
    torch.cuda.synchronize()
    outs = [blk.y, blk.dx, blk.idx] + [getattr(blk, gname) for _, _, gname in blk.lora_params()]
    _check_replays(step, outs, (blk.side,))


def test_attn_step_graph_replays():
    need_lib()
    from contextual_sparsity_lora_amd.attn import SparseAttnProj
    print("[graph] attention projections", flush=True)
    cfg = scaled(CONFIGS[3], batch=2, seq=80, out_per_seq=20, hidden=256, n_q_heads=8, n_kv_heads=2,
                 head_dim=32, lora_rank=8, est_rank=8, lora_alpha=16, seed=3003)
    inp = make_attn_inputs(cfg)
    d = {k: to_dev(v, "bf16") for k, v in inp.items()
         if isinstance(v, np.ndarray) and k.startswith(("x", "W_", "A_", "B_", "dy_"))}
    blk = SparseAttnProj(d["W_q"], d["W_k"], d["W_v"], d["W_o"], d["A_q"], d["B_q"], d["A_k"], d["B_k"],
                         d["A_v"], d["B_v"], d["A_o"], d["B_o"],
                         to_dev(np.ascontiguousarray(inp["WA_t_qkv"].T), "f32"), to_dev(inp["WB_q"], "f32"),
                         to_dev(inp["WB_k"], "f32"), to_dev(inp["WB_v"], "f32"), inp["scale"], cfg.n_kv_heads,
                         cfg.head_dim, qk_sparsity=cfg.qk_sparsity, vo_sparsity=cfg.vo_sparsity)
    roles = to_dev(inp["roles"], None)
    dqkv = torch.cat([d["dy_q"], d["dy_k"], d["dy_v"]], 1).contiguous()
    step = lambda: (blk.forward(d["x"], d["x_o"], roles, cfg.ctx_tokens), blk.backward(dqkv, d["dy_o"]))
    step()
    torch.cuda.synchronize()
    outs = [blk.qkv, blk.o, blk.dx, blk.dx_o, blk.dA_qkv, blk.dB_q, blk.dB_k, blk.dB_v, blk.dA_o, blk.dB_o]
    _check_replays(step, outs, (blk.side,))
