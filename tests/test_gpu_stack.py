"""GPU parity of a stack of sparse decoder layers (the LLaMA3-8B-shaped
32-layer stack with its per-layer sparsity ramp), one training step forward
and backward, against the CPU oracle.

A scaled 4-layer stack, whose layers carry the sparsities of layers 3, 10, 20
and 31 of the ramp (0 to 80%), is compared end to end against the oracle's
fp64 stack, with every layer's selections bit-exact from the GPU's own
normalised inputs, and layer by layer teacher-forced.  The full 32-layer stack
is compared teacher-forced on sampled layers (the layer's GPU input and
upstream gradient fed to the oracle), on sampled rows, selections bit-exact,
every LoRA gradient of those layers in full."""
import numpy as np
import pytest
import torch

from oracle import reference as ref
from tests.gpu_util import TOL, host, host_i, mar, need_lib, sample_rows, to_dev
from tests.layer_check import check_ops, gpu_record, selections
from workloads.configs import CONFIGS, scaled
from workloads.gen import make_stack_io, make_stack_layer

pytestmark = pytest.mark.gpu

SMALL = scaled(CONFIGS[5], batch=2, seq=96, out_per_seq=24, hidden=256, inter=512, n_q_heads=8,
               n_kv_heads=2, head_dim=32, lora_rank=8, est_rank=8, lora_alpha=16, n_layers=4,
               seed=5005)
SMALL_RAMP = (3, 10, 20, 31)          # ramp positions whose sparsities the 4 layers take


def _dims(cfg):
    return cfg.batch, cfg.seq, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim


def _build_and_run(cfg, ramp, keep_host):
    """Generate, upload and run the stack; returns (io, host layer inputs for
    the layers in keep_host, sparsities, stack)."""
    need_lib()
    from contextual_sparsity_lora_amd.stack import SparseStack
    dt = cfg.dtype
    io = make_stack_io(cfg)
    arrays, sps, kept = [], [], {}
    for l, pos in enumerate(ramp):
        sp = cfg.layer_sparsity(pos)
        lw = make_stack_layer(cfg, l, with_factors=sp[0] != 0)
        d = {k: to_dev(v, dt) for k, v in lw.items() if k[:2] in ("W_", "A_", "B_")}
        f32 = {}
        if sp[0] != 0:
            f32 = {"WA_qkv": to_dev(np.ascontiguousarray(lw["WA_t_qkv"].T), "f32"),
                   "WA_gu": to_dev(np.ascontiguousarray(lw["WA_t_gu"].T), "f32")}
            for p in ("q", "k", "v", "gate", "up"):
                f32["WB_" + p] = to_dev(lw["WB_" + p], "f32")
        arrays.append((d, f32))
        sps.append(sp)
        if l in keep_host:
            kept[l] = lw
        print(f"[stack] layer {l} generated and uploaded (sparsity {sp[0]}/{sp[1]})", flush=True)
    stack = SparseStack.build(cfg, arrays, sps)
    for L in stack.layers:
        L.ffn.keep_h = True  # whole rows of the FFN's h, for the checks
    del arrays
    roles = to_dev(io["roles"], None)
    stack.forward(to_dev(io["x"], dt), roles, cfg.ctx_tokens)
    stack.backward(to_dev(io["dy"], dt))
    torch.cuda.synchronize()
    print("[stack] forward + backward done", flush=True)
    return io, kept, sps, stack


def _layer_case(cfg, io, lw, stack, l, sp):
    """Host record of layer l, its oracle input set (GPU input x and upstream
    gradient dy) and its selections (checked bit-exact when sparse)."""
    L = stack.layers[l]
    g = gpu_record(cfg, L)
    dy = io["dy"] if l == len(stack.layers) - 1 else host(stack.layers[l + 1].dx)
    inp = dict(lw, x=host(L.x), dy=dy, roles=io["roles"], scale=io["scale"])
    sel = selections(cfg, inp, g, sp, sp, sp)
    if sp[0] != 0:
        assert np.array_equal(host_i(L.attn.idx_qk), sel[0]), l
        assert np.array_equal(host_i(L.attn.idx_vo), sel[1]), l
        assert np.array_equal(host_i(L.ffn.idx), sel[2]), l
    return g, inp, sel


def test_stack_small_end_to_end():
    cfg = SMALL
    io, kept, sps, stack = _build_and_run(cfg, SMALL_RAMP, set(range(len(SMALL_RAMP))))
    print("[stack] scaled 4-layer stack", flush=True)
    sels, recs = [], []
    for l in range(len(SMALL_RAMP)):
        g, inp, sel = _layer_case(cfg, io, kept[l], stack, l, sps[l])
        check_ops(cfg, inp, g, sel, np.arange(cfg.tokens),
                  [(b, grp) for b in range(cfg.batch) for grp in range(cfg.n_kv_heads)], tag=f"stack l{l}")
        sels.append(sel)
        recs.append(g)
    layers = [kept[l] for l in range(len(SMALL_RAMP))]
    fwds = ref.decoder_stack_fwd(layers, io["x"], io["roles"], io["scale"], _dims(cfg), sels)
    bwds = ref.decoder_stack_bwd(layers, io["x"], io["roles"], io["scale"], fwds, io["dy"], _dims(cfg),
                                 sels)
    tol = TOL[cfg.dtype]
    assert mar(host(stack.layers[-1].y), fwds[-1]["y"]) <= tol
    assert mar(host(stack.layers[0].dx), bwds[0]["dx"]) <= tol
    for l in range(len(SMALL_RAMP)):
        assert mar(recs[l]["y"], fwds[l]["y"]) <= tol, l
        for p in ("q", "k", "v", "o", "gate", "up", "down"):
            assert mar(recs[l]["dA_" + p], bwds[l]["dA_" + p]) <= tol, (l, p)
            assert mar(recs[l]["dB_" + p], bwds[l]["dB_" + p]) <= tol, (l, p)


@pytest.mark.timeout(900)
def test_stack_full_size_sampled_layers():
    cfg = CONFIGS[5]
    check = (0, 4, 17, 31)
    io, kept, sps, stack = _build_and_run(cfg, list(range(cfg.n_layers)), set(check))
    print("[stack] 32-layer LLaMA3-8B stack", flush=True)
    ctx, out = ref.token_lists(io["roles"])
    R = sample_rows(ctx, out, 16)
    for l in check:
        g, inp, sel = _layer_case(cfg, io, kept[l], stack, l, sps[l])
        pairs = [(l % cfg.batch, l % cfg.n_kv_heads), ((l + 3) % cfg.batch, (l + 5) % cfg.n_kv_heads),
                 ((l + 6) % cfg.batch, (l + 2) % cfg.n_kv_heads)]
        check_ops(cfg, inp, g, sel, R, pairs, tag=f"stack l{l}")
        del g, inp
