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


@pytest.mark.parametrize("T,T_c,D,F,n", [(300, 230, 136, 1000, 333), (70, 70, 64, 520, 1), (129, 5, 64, 2048, 2048)])
def test_swiglu_fwd_ctx_matches_merge_path(T, T_c, D, F, n, rng):
    """Context rows from the compact gate|up product: the merged gate|up rows
    equal the merge path's bit for bit, h those of the plain SwiGLU pass, hc
    the selected channels of h (padding zero), xl = h A^T within fp32
    rounding, and the down product fed hc equals the one gathering from h."""
    ops = _ops()
    print(f"[swiglu-ctx] T={T} T_c={T_c} F={F} n={n}", flush=True)
    r, s = 16, 2.0
    roles = np.ones(T, np.uint8)
    ctx = np.sort(rng.choice(T, T_c, replace=False)).astype(np.int32)
    roles[ctx] = 0
    out = np.setdiff1d(np.arange(T), ctx).astype(np.int32)
    c_d, o_d = to_dev(ctx, None), to_dev(out, None)
    idx = np.sort(rng.choice(F, n, replace=False)).astype(np.int32)
    idx_d, idx2_d = to_dev(idx, None), to_dev(np.concatenate([idx, idx + F]).astype(np.int32), None)
    x = dev_pad(round_dtype(rng.standard_normal((T, D)), "bf16"), "bf16")
    Wgu = dev_pad(round_dtype(rng.standard_normal((2 * F, D)) * 0.1, "bf16"), "bf16")
    P = to_dev(rng.standard_normal((T, 2 * r)).astype(np.float32), "f32")
    Bbd = np.zeros((2 * F, 2 * r), np.float32)
    Bbd[:F, :r] = round_dtype(rng.standard_normal((F, r)) * 0.3, "bf16")
    Bbd[F:, r:] = round_dtype(rng.standard_normal((F, r)) * 0.3, "bf16")
    Bbd_d = to_dev(Bbd, "bf16")
    A = round_dtype(rng.standard_normal((r, F)) * 0.05, "bf16")
    A_d = dev_pad(A, "bf16")
    lora = (P, Bbd_d, 2 * r, s)
    gu1 = empty_pad(T, 2 * F, "bf16", fill=5.0)
    ops.sparse_linear_fwd("out", x, Wgu, None, c_d, o_d, idx2_d, gu1, lora=lora, flags=ops.ONLY_CTX_ROWS)
    c8 = lambda v: (v + 7) // 8 * 8
    yc = empty_pad(T_c, c8(2 * n), "bf16", fill=9.0)
    ops.sparse_linear_fwd("out", x, Wgu, None, c_d, o_d, idx2_d, yc[:, :2 * n], lora=lora,
                          flags=ops.ONLY_CTX_ROWS | ops.CTX_COMPACT)
    gu2 = empty_pad(T, 2 * F, "bf16", fill=5.0)
    hc = empty_pad(T_c, c8(n), "bf16", fill=3.0)
    hf = empty_pad(T, F, "bf16", fill=4.0)
    xl = torch.full((T, r), 7.0, dtype=torch.float32, device=DEV)
    ops.swiglu_fwd_ctx(yc, c_d, idx_d, lora, gu2, hc, A_d, xl, h_rows=hf)
    hp = empty_pad(T, F, "bf16")
    ops.swiglu_fwd(gu2[:, :F], gu2[:, F:], hp)
    torch.cuda.synchronize()
    g1, g2 = host(gu1), host(gu2)
    assert np.array_equal(bits(g2[ctx]), bits(g1[ctx]))
    assert np.all(g2[out] == 5.0)                                   # other rows untouched
    assert np.array_equal(bits(host(yc)[:, :2 * n]), bits(g1[ctx][:, np.concatenate([idx, idx + F])]))
    hh = host(hf)
    assert np.array_equal(bits(hh[ctx]), bits(host(hp)[ctx]))
    assert np.all(hh[out] == 4.0)
    assert mar(hh[ctx], ref.swiglu_fwd(g2[ctx, :F], g2[ctx, F:])) <= TOL["bf16"]
    hcc = host(hc)
    assert np.array_equal(bits(hcc[:, :n]), bits(hh[ctx][:, idx]))
    assert np.all(hcc[:, n:] == 0.0)
    xlh = host(xl)
    assert mar(xlh[ctx], hh[ctx].astype(np.float64) @ A.T.astype(np.float64)) <= 1e-5
    assert np.all(xlh[out] == 7.0)
    # the down product fed the compact rows equals the one that gathers them
    Wdn = dev_pad(round_dtype(rng.standard_normal((D, F)) * 0.05, "bf16"), "bf16")
    Wdn_t = dev_pad(np.ascontiguousarray(host(Wdn).T), "bf16")
    hfull = dev_pad(np.where(roles[:, None] == 0, hh, round_dtype(rng.standard_normal((T, F)), "bf16")), "bf16")
    y1, y2, y3 = empty_pad(T, D, "bf16"), empty_pad(T, D, "bf16"), empty_pad(T, D, "bf16")
    ws = empty_pad(D, c8(n), "bf16")
    ops.weight_slice(Wdn_t, idx_d, ws)
    ops.sparse_linear_fwd("in", hfull, Wdn, Wdn_t, c_d, o_d, idx_d, y1)
    ops.sparse_linear_fwd("in", hfull, Wdn, Wdn_t, c_d, o_d, idx_d, y2, x_slice=hc)
    ops.sparse_linear_fwd("in", hfull, Wdn, Wdn_t, c_d, o_d, idx_d, y3, x_slice=hc, w_slice=ws)
    torch.cuda.synchronize()
    assert np.array_equal(bits(host(y1)), bits(host(y2)))
    assert np.array_equal(bits(host(y1)), bits(host(y3)))
