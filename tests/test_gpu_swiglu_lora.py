"""GPU parity of the SwiGLU passes fused with the LoRA reductions that read the
same tensors, against the oracle (SwiGLU, LoRA gradients) and against the
unfused library calls (the elementwise outputs bit for bit)."""
import numpy as np
import pytest
import torch

from oracle import reference as ref
from tests.gpu_util import DEV, TOL, bits, dev_pad, empty_pad, host, mar, need_lib, to_dev
from workloads.gen import round_dtype

pytestmark = pytest.mark.gpu


def _ops():
    need_lib()
    from contextual_sparsity_lora_amd import ops
    return ops


# T ragged against the 4- and 16-row steps; F a multiple of 8 but not of the
# 128-, 512- and 2048-column blocks; r = 24 exercises the second rank chunk
CASES = [(301, 1000, 16, 256), (301, 1000, 24, 8), (37, 2056, 8, 256), (1, 8, 1, 4), (4096, 3072, 32, 256)]


@pytest.mark.parametrize("T,F,r,rows", CASES)
def test_swiglu_lora_fwd_bwd(T, F, r, rows, rng):
    ops = _ops()
    print(f"[swiglu-lora] T={T} F={F} r={r} rows={rows}", flush=True)
    s = 2.0
    g = round_dtype(rng.standard_normal((T, F)) * 2, "bf16")
    u = round_dtype(rng.standard_normal((T, F)), "bf16")
    dh = round_dtype(rng.standard_normal((T, F)), "bf16")
    A = round_dtype(rng.standard_normal((r, F)) * 0.05, "bf16")
    gB = rng.standard_normal((T, r)).astype(np.float32)
    xl_gu = rng.standard_normal((T, 2 * r)).astype(np.float32)
    gd, ud, dhd, Ad = dev_pad(g, "bf16"), dev_pad(u, "bf16"), dev_pad(dh, "bf16"), dev_pad(A, "bf16")
    gBd, xld = to_dev(gB, "f32"), to_dev(xl_gu, "f32")
    # forward: h as the plain pass (bit for bit), xl = h A^T from the stored h
    h1, h2 = empty_pad(T, F, "bf16"), empty_pad(T, F, "bf16")
    xl = torch.full((T, r), 7.0, dtype=torch.float32, device=DEV)
    ops.swiglu_fwd(gd, ud, h1)
    ops.swiglu_fwd_lora(gd, ud, h2, Ad, xl)
    torch.cuda.synchronize()
    hh = host(h2)
    assert np.array_equal(bits(host(h1)), bits(hh))
    assert mar(hh, ref.swiglu_fwd(g, u)) <= TOL["bf16"]
    assert mar(host(xl), hh.astype(np.float64) @ A.T.astype(np.float64)) <= 1e-5
    # backward: dg, du as the plain pass; the three token reductions
    ops.set_option(0, "swiglu_rows", rows)
    try:
        dg1, du1 = empty_pad(T, F, "bf16"), empty_pad(T, F, "bf16")
        dg2, du2 = empty_pad(T, F, "bf16"), empty_pad(T, F, "bf16")
        dA = torch.full((r, F), 7.0, dtype=torch.float32, device=DEV)
        dBg = torch.full((F, r), 7.0, dtype=torch.float32, device=DEV)
        dBu = torch.full((F, r), 7.0, dtype=torch.float32, device=DEV)
        ops.swiglu_bwd(dhd, gd, ud, dg1, du1)
        ops.swiglu_bwd_lora(dhd, gd, ud, dg2, du2, gBd, xld[:, :r], xld[:, r:], s, dA, dBg, dBu)
        torch.cuda.synchronize()
    finally:
        ops.set_option(0, "swiglu_rows", 256)
    dgh, duh = host(dg2), host(du2)
    assert np.array_equal(bits(host(dg1)), bits(dgh))
    assert np.array_equal(bits(host(du1)), bits(duh))
    wdg, wdu = ref.swiglu_bwd(dh, g, u)
    assert mar(dgh, wdg) <= TOL["bf16"] and mar(duh, wdu) <= TOL["bf16"]
    f64 = np.float64
    assert mar(host(dA), s * (gB.astype(f64).T @ hh.astype(f64))) <= 1e-5
    assert mar(host(dBg), s * (dgh.astype(f64).T @ xl_gu[:, :r].astype(f64))) <= 1e-5
    assert mar(host(dBu), s * (duh.astype(f64).T @ xl_gu[:, r:].astype(f64))) <= 1e-5


def test_swiglu_lora_bwd_no_rows():
    """No rows: the three gradients are written as zeros."""
    ops = _ops()
    F, r = 64, 16
    z = empty_pad(0, F, "bf16")
    zf = torch.zeros(0, r, dtype=torch.float32, device=DEV)
    dA = torch.full((r, F), 7.0, dtype=torch.float32, device=DEV)
    dBg = torch.full((F, r), 7.0, dtype=torch.float32, device=DEV)
    dBu = torch.full((F, r), 7.0, dtype=torch.float32, device=DEV)
    ops.swiglu_bwd_lora(z, z, z, z, z, zf, zf, zf, 2.0, dA, dBg, dBu)
    torch.cuda.synchronize()
    assert float(dA.abs().max()) == 0.0 and float(dBg.abs().max()) == 0.0 and float(dBu.abs().max()) == 0.0


def test_swiglu_lora_refuses_f32_and_ragged_width():
    ops = _ops()
    g = torch.zeros(4, 12, dtype=torch.float32, device=DEV)
    with pytest.raises(ops.SLError, match="UNSUPPORTED|bf16"):
        ops.swiglu_fwd_lora(g, g, g, torch.zeros(4, 12, dtype=torch.float32, device=DEV),
                            torch.zeros(4, 4, dtype=torch.float32, device=DEV))
    gb = empty_pad(4, 12, "bf16")
    with pytest.raises(ops.SLError, match="multiple of 8"):
        ops.swiglu_fwd_lora(gb, gb, gb, empty_pad(4, 12, "bf16"), torch.zeros(4, 4, dtype=torch.float32, device=DEV))
