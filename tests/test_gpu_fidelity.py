"""GPU gradient-fidelity report: the library's fp64 dot statistics against
numpy, and the per-adapter cosines between the sparse and the dense FFN
block's LoRA gradients against the oracle's (same inputs, same selection)."""
import numpy as np
import pytest
import torch

from oracle import reference as ref
from tests.gpu_util import DEV, need_lib, to_dev
from tests.test_gpu_ffn import _inputs, _selection
from workloads.configs import CONFIGS, scaled
from workloads.gen import make_ffn_inputs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n", [0, 1, 255, 257, 65536 + 13, 3_000_001])
def test_dot_stats_matches_numpy_and_repeats(n, rng):
    need_lib()
    from contextual_sparsity_lora_amd import ops
    print(f"[dot] n={n}", flush=True)
    a = rng.standard_normal(n).astype(np.float32)
    b = (0.3 * a + rng.standard_normal(n)).astype(np.float32)
    ad, bd = to_dev(a, "f32"), to_dev(b, "f32")
    out1 = torch.empty(3, dtype=torch.float64, device=DEV)
    out2 = torch.empty(3, dtype=torch.float64, device=DEV)
    ops.dot_stats(ad, bd, out1)
    ops.dot_stats(ad, bd, out2)
    got = out1.cpu().numpy()
    a64, b64 = a.astype(np.float64), b.astype(np.float64)
    want = np.array([a64 @ b64, a64 @ a64, b64 @ b64])
    assert np.allclose(got, want, rtol=1e-12, atol=0.0)
    assert np.array_equal(got.view(np.uint64), out2.cpu().numpy().view(np.uint64))


def _blocks(cfg, inp):
    from contextual_sparsity_lora_amd.ffn import SparseFFN
    dt = cfg.dtype
    d = {k: to_dev(v, dt) for k, v in inp.items()
         if k in ("x", "W_gate", "W_up", "W_down", "A_gate", "B_gate", "A_up", "B_up", "A_down",
                  "B_down", "dy")}
    roles = to_dev(inp["roles"], None)
    out = []
    for dense in (False, True):
        blk = SparseFFN(d["W_gate"], d["W_up"], d["W_down"], d["A_gate"], d["B_gate"], d["A_up"],
                        d["B_up"], d["A_down"], d["B_down"],
                        to_dev(np.ascontiguousarray(inp["WA_t_gu"].T), "f32"),
                        to_dev(inp["WB_gate"], "f32"), to_dev(inp["WB_up"], "f32"), inp["scale"],
                        sparsity=cfg.ffn_sparsity, dense=dense)
        blk.forward(d["x"], roles, cfg.ctx_tokens)
        blk.backward(d["dy"])
        out.append(blk)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("case", ["f32", "bf16"])
def test_ffn_grad_fidelity_matches_oracle(case):
    """Cosines of the six LoRA gradients (sparse vs dense block): fp32 within
    1e-5, bf16 within 2e-2 of the oracle's fp64 cosines; the selection the
    GPU block made is the oracle's (bit-exact), so both sides compare the
    same sparse and dense computations."""
    need_lib()
    from contextual_sparsity_lora_amd import fidelity
    if case == "f32":
        cfg = CONFIGS[1]
        inp = _inputs(1)
        tol = 1e-5
    else:
        cfg = scaled(CONFIGS[2], batch=2, seq=160, out_per_seq=40, hidden=520, inter=1400)
        inp = make_ffn_inputs(cfg)
        tol = 2e-2
    print(f"[fidelity] {case} T={cfg.tokens} D={cfg.hidden} F={cfg.inter}", flush=True)
    sp, dn = _blocks(cfg, inp)
    idx = _selection(cfg, inp)
    assert np.array_equal(sp.idx.cpu().numpy(), idx)
    got = fidelity.block_fidelity(sp, dn)
    want = ref.ffn_grad_fidelity(inp, idx)
    assert set(got) == set(want)
    for k in want:
        assert abs(got[k] - want[k]) <= tol, (k, got[k], want[k])
