"""GPU parity of the sparse main branch (forward and backward, both sides) and
of the dense LoRA branch against the fp64 oracle, within the stated
tolerances (max-abs-relative 1e-4 for fp32, 2e-2 for bf16)."""
import numpy as np
import pytest
import torch

from oracle import reference as ref
from tests.gpu_util import DEV, TOL, bits, dev_pad, empty_pad, host, mar, need_lib, tdt, to_dev
from workloads.gen import round_dtype

pytestmark = pytest.mark.gpu


def _ops():
    need_lib()
    from contextual_sparsity_lora_amd import ops
    return ops


def _roles(B, S, O):
    r = np.zeros((B, S), np.uint8)
    r[:, S - O:] = 1
    return r.reshape(-1)


def _lists(ops, roles):
    ctx, out = ref.token_lists(roles)
    return ctx, out, to_dev(ctx, None), to_dev(out, None)


CASES = [
    # dtype, B, S, O, D_in, D_out, keep
    ("f32", 2, 64, 16, 256, 688, 344),        # the fp32 FFN shape
    ("bf16", 2, 300, 70, 520, 1000, 333),     # several tiles and ragged tails everywhere
    ("bf16", 1, 129, 0, 136, 130, 1),         # no output tokens, one kept channel
    ("bf16", 3, 40, 40, 64, 200, 0),          # no context tokens, nothing kept
]


@pytest.fixture(params=[10, 11, 14, 33], ids=lambda c: f"gemm{c}")
def gemm_cfg(request):
    """Each tile configuration of the bf16 product on every case: 10 the
    default (the eight-wave 256 x 256 kernel), 11 the same kernel named, 14
    the 128 x 128 one, 33 the four-wave LDS-DMA kernel with split tails.  The
    option is put back to 10 afterwards."""
    ops = _ops()
    ops.set_option(0, "gemm_cfg", request.param)
    yield request.param
    ops.set_option(0, "gemm_cfg", 10)


@pytest.mark.parametrize("case", CASES)
def test_sparse_linear_fwd_bwd(case, gemm_cfg, rng):
    ops = _ops()
    dtype, B, S, O, Din, Dout, keep = case
    print(f"[linear] {case} gemm_cfg={gemm_cfg}", flush=True)
    roles = _roles(B, S, O)
    T = B * S
    ctx, out, c_d, o_d = _lists(ops, roles)
    x = round_dtype(rng.standard_normal((T, Din)), dtype)
    W = round_dtype(rng.standard_normal((Dout, Din)) * 0.05, dtype)     # [D_out, D_in]
    dy = round_dtype(rng.standard_normal((T, Dout)), dtype)
    tol = TOL[dtype]
    # output side: channels = output features
    idx = np.sort(rng.choice(Dout, min(keep, Dout), replace=False)).astype(np.int32)
    y = empty_pad(T, Dout, dtype)
    Wd, Wtd = dev_pad(W, dtype), dev_pad(np.ascontiguousarray(W.T), dtype)
    ops.sparse_linear_fwd("out", dev_pad(x, dtype), Wd, None, c_d, o_d, to_dev(idx, None), y)
    yr = ref.sparse_linear_fwd("out", x, W, roles, idx)
    assert mar(host(y), yr) <= tol
    drop = np.setdiff1d(np.arange(Dout), idx)
    assert np.all(host(y)[np.ix_(ctx, drop)] == 0.0)
    dx = empty_pad(T, Din, dtype)
    ops.sparse_linear_bwd("out", dev_pad(dy, dtype), Wd, Wtd, c_d, o_d, to_dev(idx, None), dx)
    assert mar(host(dx), ref.sparse_linear_bwd("out", dy, W, roles, idx)) <= tol
    # input side: W in nn.Linear layout and its transposed copy
    Wi = round_dtype(rng.standard_normal((Din, Dout)) * 0.05, dtype)    # nn.Linear [out=Din, in=Dout]
    Wt = np.ascontiguousarray(Wi.T)
    Wid, Witd = dev_pad(Wi, dtype), dev_pad(Wt, dtype)
    idx_in = np.sort(rng.choice(Dout, min(keep, Dout), replace=False)).astype(np.int32)
    xi = round_dtype(rng.standard_normal((T, Dout)), dtype)
    yi = empty_pad(T, Din, dtype)
    ops.sparse_linear_fwd("in", dev_pad(xi, dtype), Wid, Witd, c_d, o_d, to_dev(idx_in, None), yi)
    assert mar(host(yi), ref.sparse_linear_fwd("in", xi, Wi, roles, idx_in)) <= tol
    dyi = round_dtype(rng.standard_normal((T, Din)), dtype)
    dxi = empty_pad(T, Dout, dtype)
    ops.sparse_linear_bwd("in", dev_pad(dyi, dtype), None, Witd, c_d, o_d, to_dev(idx_in, None), dxi)
    dxr = ref.sparse_linear_bwd("in", dyi, Wi, roles, idx_in)
    assert mar(host(dxi), dxr) <= tol
    assert np.all(host(dxi)[np.ix_(ctx, np.setdiff1d(np.arange(Dout), idx_in))] == 0.0)


def test_output_rows_invariant_and_full_keep_is_dense(rng):
    ops = _ops()
    roles = _roles(2, 256, 64)
    T, Din, Dout = 512, 384, 640
    ctx, out, c_d, o_d = _lists(ops, roles)
    x = to_dev(round_dtype(rng.standard_normal((T, Din)), "bf16"), "bf16")
    Wn = round_dtype(rng.standard_normal((Dout, Din)) * 0.05, "bf16")
    W = to_dev(Wn, "bf16")
    ys = []
    for idx in (np.arange(0, Dout, 3), np.arange(5), np.arange(Dout)):
        y = torch.empty(T, Dout, dtype=torch.bfloat16, device=DEV)
        ops.sparse_linear_fwd("out", x, W, None, c_d, o_d, to_dev(idx.astype(np.int32), None), y)
        ys.append(host(y))
    for y in ys[1:]:
        assert np.array_equal(y[out], ys[0][out])          # bitwise: output rows never see idx
    dense = ref.sparse_linear_fwd("out", host(x), Wn, np.ones(T, np.uint8), np.zeros(0, np.int32))
    assert mar(ys[2], dense) <= TOL["bf16"]                 # keep = C is the dense layer


def test_beta_accumulates(rng):
    ops = _ops()
    roles = _roles(1, 200, 50)
    T, Din, Dout = 200, 128, 256
    ctx, out, c_d, o_d = _lists(ops, roles)
    x = round_dtype(rng.standard_normal((T, Din)), "bf16")
    W = round_dtype(rng.standard_normal((Dout, Din)) * 0.05, "bf16")
    y0 = round_dtype(rng.standard_normal((T, Dout)), "bf16")
    idx = np.sort(rng.choice(Dout, 77, replace=False)).astype(np.int32)
    y = to_dev(y0, "bf16")
    ops.sparse_linear_fwd("out", to_dev(x, "bf16"), to_dev(W, "bf16"), None, c_d, o_d, to_dev(idx, None), y,
                          beta=1)
    assert mar(host(y), y0 + ref.sparse_linear_fwd("out", x, W, roles, idx)) <= TOL["bf16"]


@pytest.mark.parametrize("dtype,T,Din,Dout,r", [("f32", 128, 256, 688, 8), ("bf16", 300, 520, 1000, 16),
                                                ("bf16", 64, 4096, 14336, 16), ("bf16", 33, 200, 72, 32),
                                                ("bf16", 1100, 256, 520, 16), ("bf16", 100, 136, 264, 64)])
def test_lora_fwd_bwd(dtype, T, Din, Dout, r, rng):
    ops = _ops()
    print(f"[lora] {dtype} T={T} D_in={Din} D_out={Dout} r={r}", flush=True)
    s = 2.0
    x = round_dtype(rng.standard_normal((T, Din)), dtype)
    A = round_dtype(rng.standard_normal((r, Din)) * 0.02, dtype)
    Bm = round_dtype(rng.standard_normal((Dout, r)) * 0.02, dtype)
    y0 = round_dtype(rng.standard_normal((T, Dout)), dtype)
    dy = round_dtype(rng.standard_normal((T, Dout)), dtype)
    dx0 = round_dtype(rng.standard_normal((T, Din)), dtype)
    tol = TOL[dtype]
    xl = torch.empty(T, r, dtype=torch.float32, device=DEV)
    y = to_dev(y0, dtype)
    xd, Ad, Bd = to_dev(x, dtype), to_dev(A, dtype), to_dev(Bm, dtype)
    ops.lora_fwd_bwd(ops.LORA_XL | ops.LORA_ADD, xd, Ad, Bd, s, xl, y=y)
    xl_r, yl_r = ref.lora_fwd(x, A, Bm, s)
    assert mar(host(xl), xl_r) <= 1e-5
    assert mar(host(y), y0 + yl_r) <= tol
    y_only = torch.zeros(T, Dout, dtype=tdt(dtype), device=DEV)
    ops.lora_fwd_bwd(ops.LORA_ADD, None, None, Bd, s, xl, y=y_only)
    assert mar(host(y_only), yl_r) <= tol
    dA = torch.empty(r, Din, dtype=torch.float32, device=DEV)
    dB = torch.empty(Dout, r, dtype=torch.float32, device=DEV)
    dx = to_dev(dx0, dtype)
    ops.lora_fwd_bwd(ops.LORA_BWD, xd, Ad, Bd, s, xl, dy=to_dev(dy, dtype), dx=dx, dA=dA, dB=dB)
    dx_r, dA_r, dB_r = ref.lora_bwd(x, host(xl), dy, A, Bm, s)
    assert mar(host(dA), dA_r) <= 1e-4
    assert mar(host(dB), dB_r) <= 1e-4
    assert mar(host(dx), dx0 + dx_r) <= tol


@pytest.mark.parametrize("dtype,T,Din,Dout,r", [("bf16", 700, 520, 1000, 96), ("f32", 90, 136, 200, 128),
                                                ("bf16", 4096, 256, 392, 128)])
def test_lora_high_rank_column_chunks(dtype, T, Din, Dout, r, rng):
    """Ranks above 64 (a stacked q|k|v LoRA of rank 32 per projection has 96):
    xl, gB, dA and dB run as independent column chunks of 64."""
    ops = _ops()
    print(f"[lora] high rank {dtype} T={T} r={r}", flush=True)
    s = 2.0
    x = round_dtype(rng.standard_normal((T, Din)), dtype)
    A = round_dtype(rng.standard_normal((r, Din)) * 0.02, dtype)
    Bm = round_dtype(rng.standard_normal((Dout, r)) * 0.02, dtype)
    dy = round_dtype(rng.standard_normal((T, Dout)), dtype)
    xd, Ad, Bd = to_dev(x, dtype), to_dev(A, dtype), to_dev(Bm, dtype)
    xl = torch.empty(T, r, dtype=torch.float32, device=DEV)
    ops.lora_fwd_bwd(ops.LORA_XL, xd, Ad, None, s, xl)
    assert mar(host(xl), x.astype(np.float64) @ A.T.astype(np.float64)) <= 1e-5
    gB = torch.empty(T, r, dtype=torch.float32, device=DEV)
    dA = torch.empty(r, Din, dtype=torch.float32, device=DEV)
    dB = torch.empty(Dout, r, dtype=torch.float32, device=DEV)
    ops.lora_fwd_bwd(ops.LORA_GB | ops.LORA_DA | ops.LORA_DB, xd, None, Bd, s, xl, dy=to_dev(dy, dtype),
                     dA=dA, dB=dB, gB=gB, D_in=Din)
    _, dA_r, dB_r = ref.lora_bwd(x, host(xl), dy, A, Bm, s)
    assert mar(host(gB), dy.astype(np.float64) @ Bm.astype(np.float64)) <= 1e-5
    assert mar(host(dA), dA_r) <= 1e-4
    assert mar(host(dB), dB_r) <= 1e-4


@pytest.mark.parametrize("dtype,r", [("f32", 8), ("bf16", 16), ("bf16", 32), ("bf16", 96), ("f32", 72)])
def test_fused_lora_term(dtype, r, rng):
    """The LoRA term fused into the main-branch product equals main + s xl B^T,
    and unselected context channels carry the LoRA term alone."""
    ops = _ops()
    roles = _roles(2, 300, 70)
    T, Din, Dout = 600, 520, 1000
    ctx, out, c_d, o_d = _lists(ops, roles)
    tol = TOL[dtype]
    s = 2.0
    x = round_dtype(rng.standard_normal((T, Din)), dtype)
    W = round_dtype(rng.standard_normal((Dout, Din)) * 0.05, dtype)
    P = rng.standard_normal((T, r)).astype(np.float32)
    Bm = round_dtype(rng.standard_normal((Dout, r)) * 0.3, dtype)
    idx = np.sort(rng.choice(Dout, 333, replace=False)).astype(np.int32)
    y = empty_pad(T, Dout, dtype)
    Wd, Wtd = dev_pad(W, dtype), dev_pad(np.ascontiguousarray(W.T), dtype)
    ops.sparse_linear_fwd("out", dev_pad(x, dtype), Wd, None, c_d, o_d, to_dev(idx, None), y,
                          lora=(to_dev(P, "f32"), dev_pad(Bm, dtype), r, s))
    lora = s * (P.astype(np.float64) @ Bm.T.astype(np.float64))
    assert mar(host(y), ref.sparse_linear_fwd("out", x, W, roles, idx) + lora) <= tol
    drop = np.setdiff1d(np.arange(Dout), idx)
    assert mar(host(y)[np.ix_(ctx, drop)], lora[np.ix_(ctx, drop)]) <= tol
    # input side (K-gathered) with the LoRA term, and the backward forms
    Wi = round_dtype(rng.standard_normal((Din, Dout)) * 0.05, dtype)
    xi = round_dtype(rng.standard_normal((T, Dout)), dtype)
    Bi = round_dtype(rng.standard_normal((Din, r)) * 0.3, dtype)
    yi = empty_pad(T, Din, dtype)
    Wid, Witd = dev_pad(Wi, dtype), dev_pad(np.ascontiguousarray(Wi.T), dtype)
    ops.sparse_linear_fwd("in", dev_pad(xi, dtype), Wid, Witd, c_d, o_d,
                          to_dev(idx, None), yi, lora=(to_dev(P, "f32"), dev_pad(Bi, dtype), r, s))
    lora_i = s * (P.astype(np.float64) @ Bi.T.astype(np.float64))
    assert mar(host(yi), ref.sparse_linear_fwd("in", xi, Wi, roles, idx) + lora_i) <= tol
    dy = round_dtype(rng.standard_normal((T, Din)), dtype)
    dx = empty_pad(T, Dout, dtype)
    ops.sparse_linear_bwd("in", dev_pad(dy, dtype), None, Witd, c_d, o_d,
                          to_dev(idx, None), dx, lora=(to_dev(P, "f32"), dev_pad(Bm, dtype), r, s))
    assert mar(host(dx), ref.sparse_linear_bwd("in", dy, Wi, roles, idx) + lora) <= tol
    assert mar(host(dx)[np.ix_(ctx, drop)], lora[np.ix_(ctx, drop)]) <= tol
    dy2 = round_dtype(rng.standard_normal((T, Dout)), dtype)
    dx2 = empty_pad(T, Din, dtype)
    ops.sparse_linear_bwd("out", dev_pad(dy2, dtype), Wd, Wtd, c_d, o_d, to_dev(idx, None), dx2,
                          lora=(to_dev(P, "f32"), dev_pad(Bi, dtype), r, s))
    assert mar(host(dx2), ref.sparse_linear_bwd("out", dy2, W, roles, idx) + lora_i) <= tol


@pytest.mark.parametrize("r,Dout", [(16, 1000), (32, 1003), (64, 136), (96, 520), (128, 264)])
def test_fused_lora_term_accumulates(r, Dout, rng):
    """beta = 1 with the LoRA term: every channel of every row gains exactly one
    copy of the rank-r term (unselected context channels from the rank-r fill,
    the rest from the product's epilogue), on top of what the output held."""
    ops = _ops()
    roles = _roles(3, 130, 30)
    T, Din = 390, 264
    ctx, out, c_d, o_d = _lists(ops, roles)
    s = 0.5
    x = round_dtype(rng.standard_normal((T, Din)), "bf16")
    W = round_dtype(rng.standard_normal((Dout, Din)) * 0.05, "bf16")
    P = rng.standard_normal((T, r)).astype(np.float32)
    Bm = round_dtype(rng.standard_normal((Dout, r)) * 0.3, "bf16")
    y0 = round_dtype(rng.standard_normal((T, Dout)), "bf16")
    idx = np.sort(rng.choice(Dout, Dout // 3, replace=False)).astype(np.int32)
    y = dev_pad(y0, "bf16")
    ops.sparse_linear_fwd("out", dev_pad(x, "bf16"), dev_pad(W, "bf16"), None, c_d, o_d,
                          to_dev(idx, None), y, beta=1,
                          lora=(to_dev(P, "f32"), dev_pad(Bm, "bf16"), r, s))
    lora = s * (P.astype(np.float64) @ Bm.T.astype(np.float64))
    want = y0 + ref.sparse_linear_fwd("out", x, W, roles, idx) + lora
    assert mar(host(y), want) <= TOL["bf16"]
    drop = np.setdiff1d(np.arange(Dout), idx)
    assert mar(host(y)[np.ix_(ctx, drop)], (y0 + lora)[np.ix_(ctx, drop)]) <= TOL["bf16"]


@pytest.mark.parametrize("cfg", [11, 33])
@pytest.mark.parametrize("side", ["out", "in"])
def test_split_tail_chunks(side, cfg, rng):
    """A launch whose tiles do not fill the compute units runs its last partial
    round as K-chunks summed by a second launch (long K, few tiles): the result
    matches the oracle with the LoRA term, rows mapped, and two runs agree bit
    for bit (the chunk sums have a fixed order).  Both 256 x 256 kernels that
    split their tails are run."""
    ops = _ops()
    ops.set_option(0, "gemm_cfg", cfg)
    try:
        _split_tail_case(ops, side, rng)
    finally:
        ops.set_option(0, "gemm_cfg", 10)


def _split_tail_case(ops, side, rng):
    roles = _roles(2, 320, 64)
    T, Din, Dout, r, s = 640, 3072, 1100, 16, 2.0
    ctx, out, c_d, o_d = _lists(ops, roles)
    x = round_dtype(rng.standard_normal((T, Din)), "bf16")
    W = round_dtype(rng.standard_normal((Dout, Din)) * 0.05, "bf16")
    P = rng.standard_normal((T, r)).astype(np.float32)
    print(f"[split-tail] side={side} T={T} K={Din if side == 'out' else Dout}", flush=True)
    if side == "out":
        idx = np.sort(rng.choice(Dout, 700, replace=False)).astype(np.int32)
        Bm = round_dtype(rng.standard_normal((Dout, r)) * 0.3, "bf16")
        runs = []
        for _ in range(2):
            y = empty_pad(T, Dout, "bf16")
            ops.sparse_linear_fwd("out", dev_pad(x, "bf16"), dev_pad(W, "bf16"), None, c_d, o_d,
                                  to_dev(idx, None), y, lora=(to_dev(P, "f32"), dev_pad(Bm, "bf16"), r, s))
            runs.append(host(y))
        want = ref.sparse_linear_fwd("out", x, W, roles, idx) + s * (P.astype(np.float64) @ Bm.T)
    else:
        # input side over a long K: dense output rows and gathered context rows
        Wi = round_dtype(rng.standard_normal((Dout, Din)) * 0.05, "bf16")
        idx = np.sort(rng.choice(Din, 2000, replace=False)).astype(np.int32)
        Bm = round_dtype(rng.standard_normal((Dout, r)) * 0.3, "bf16")
        runs = []
        for _ in range(2):
            y = empty_pad(T, Dout, "bf16")
            ops.sparse_linear_fwd("in", dev_pad(x, "bf16"), dev_pad(Wi, "bf16"),
                                  dev_pad(np.ascontiguousarray(Wi.T), "bf16"), c_d, o_d, to_dev(idx, None), y,
                                  lora=(to_dev(P, "f32"), dev_pad(Bm, "bf16"), r, s))
            runs.append(host(y))
        want = ref.sparse_linear_fwd("in", x, Wi, roles, idx) + s * (P.astype(np.float64) @ Bm.T)
    assert np.array_equal(runs[0], runs[1])
    assert mar(runs[0], want) <= TOL["bf16"]


@pytest.mark.parametrize("dtype,F", [("bf16", 704), ("f32", 700), ("bf16", 701), ("f32", 702)])
def test_swiglu_on_gate_up_slices(dtype, F, rng):
    """SwiGLU forward and backward on the gate and up halves of one stacked
    buffer.  Rows must start on 16-byte boundaries (the kernels move 8
    channels at once): widths that break this are refused before any launch."""
    ops = _ops()
    T = 37
    gu = round_dtype(rng.standard_normal((T, 2 * F)) * 2.0, dtype)
    dh = round_dtype(rng.standard_normal((T, F)), dtype)
    gud = to_dev(gu, dtype)
    h = torch.empty(T, F, dtype=tdt(dtype), device=DEV)
    dgu = torch.empty(T, 2 * F, dtype=tdt(dtype), device=DEV)
    esize = 2 if dtype == "bf16" else 4
    if (F * esize) % 16:
        with pytest.raises(ops.SLError):
            ops.swiglu_fwd(gud[:, :F], gud[:, F:], h)
        with pytest.raises(ops.SLError):
            ops.swiglu_bwd(to_dev(dh, dtype), gud[:, :F], gud[:, F:], dgu[:, :F], dgu[:, F:])
        return
    ops.swiglu_fwd(gud[:, :F], gud[:, F:], h)
    ops.swiglu_bwd(to_dev(dh, dtype), gud[:, :F], gud[:, F:], dgu[:, :F], dgu[:, F:])
    g, u = gu[:, :F], gu[:, F:]
    assert mar(host(h), ref.swiglu_fwd(g, u)) <= TOL[dtype]
    dg_r, du_r = ref.swiglu_bwd(dh, g, u)
    assert mar(host(dgu)[:, :F], dg_r) <= TOL[dtype] and mar(host(dgu)[:, F:], du_r) <= TOL[dtype]


@pytest.mark.parametrize("r", [16, 96])
def test_no_fill_with_concurrent_fill_and_prebuilt_slices(r, rng):
    """The split form of a product equals the one-call form bit for bit: with
    NO_FILL the product leaves the unselected context channels as they were,
    lora_fill_unselected (run on another stream at the same time) writes
    exactly those, and a weight slice built beforehand by weight_slice replaces
    the one the product would gather itself."""
    ops = _ops()
    roles = _roles(2, 300, 70)
    T, Din, Dout, s = 600, 520, 1000, 2.0
    ctx, out, c_d, o_d = _lists(ops, roles)
    print(f"[split-form] r={r}", flush=True)
    x = round_dtype(rng.standard_normal((T, Din)), "bf16")
    W = round_dtype(rng.standard_normal((Dout, Din)) * 0.05, "bf16")
    P = rng.standard_normal((T, r)).astype(np.float32)
    Bo = round_dtype(rng.standard_normal((Dout, r)) * 0.3, "bf16")
    Bi = round_dtype(rng.standard_normal((Din, r)) * 0.3, "bf16")
    idx_o = np.sort(rng.choice(Dout, 333, replace=False)).astype(np.int32)
    idx_i = np.sort(rng.choice(Din, 181, replace=False)).astype(np.int32)
    xd, Wd, Wtd = dev_pad(x, "bf16"), dev_pad(W, "bf16"), dev_pad(np.ascontiguousarray(W.T), "bf16")
    Pd, Bod, Bid = to_dev(P, "f32"), dev_pad(Bo, "bf16"), dev_pad(Bi, "bf16")
    io_d, ii_d = to_dev(idx_o, None), to_dev(idx_i, None)
    dy = round_dtype(rng.standard_normal((T, Dout)), "bf16")
    dyd = dev_pad(dy, "bf16")
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    ev = torch.cuda.Event()
    drop_o = np.setdiff1d(np.arange(Dout), idx_o)
    drop_i = np.setdiff1d(np.arange(Din), idx_i)

    def split_out(fn, y, C, idx_d, lora):
        # product with NO_FILL on the main stream, fill of the rest on the side
        ev.record(main)
        side.wait_event(ev)
        with torch.cuda.stream(side):
            ops.lora_fill_unselected(y, c_d, lora, idx_d)
        fn(y)
        main.wait_stream(side)
        torch.cuda.synchronize()

    # forward, side "out"
    lora_o = (Pd, Bod, r, s)
    y1 = empty_pad(T, Dout, "bf16")
    ops.sparse_linear_fwd("out", xd, Wd, None, c_d, o_d, io_d, y1, lora=lora_o)
    y2 = empty_pad(T, Dout, "bf16", fill=7.0)
    ops.sparse_linear_fwd("out", xd, Wd, None, c_d, o_d, io_d, y2, lora=lora_o, flags=ops.NO_FILL)
    torch.cuda.synchronize()
    assert np.all(host(y2)[np.ix_(ctx, drop_o)] == 7.0)     # left unwritten
    y3 = empty_pad(T, Dout, "bf16", fill=7.0)
    split_out(lambda y: ops.sparse_linear_fwd("out", xd, Wd, None, c_d, o_d, io_d, y, lora=lora_o,
                                              flags=ops.NO_FILL), y3, Dout, io_d, lora_o)
    assert np.array_equal(bits(host(y1)), bits(host(y3)))
    lora = s * (P.astype(np.float64) @ Bo.T.astype(np.float64))
    assert mar(host(y3), ref.sparse_linear_fwd("out", x, W, roles, idx_o) + lora) <= TOL["bf16"]
    # weight_slice: exact copy of the selected rows of the channel-major weight,
    # zero columns up to the next multiple of 8
    ldn = (len(idx_o) + 7) // 8 * 8
    wsl = torch.full((Din, ldn + 8), 5.0, dtype=torch.bfloat16, device=DEV)
    ops.weight_slice(Wd, io_d, wsl)
    torch.cuda.synchronize()
    got = host(wsl)
    assert np.array_equal(got[:, :len(idx_o)], W[idx_o].T.astype(np.float32))
    assert np.all(got[:, len(idx_o):ldn] == 0.0) and np.all(got[:, ldn:] == 5.0)
    # backward, side "out" (contracts over the selected output channels): the
    # slice of W built beforehand
    lora_b = (Pd, Bid, r, s)
    d1 = empty_pad(T, Din, "bf16")
    ops.sparse_linear_bwd("out", dyd, Wd, Wtd, c_d, o_d, io_d, d1, lora=lora_b)
    d2 = empty_pad(T, Din, "bf16")
    ops.sparse_linear_bwd("out", dyd, Wd, Wtd, c_d, o_d, io_d, d2, lora=lora_b, w_slice=wsl[:, :ldn])
    torch.cuda.synchronize()
    assert np.array_equal(bits(host(d1)), bits(host(d2)))
    # forward, side "in" with a slice of Wt (the transposed copy) built beforehand
    xi = round_dtype(rng.standard_normal((T, Din)), "bf16")
    xid = dev_pad(xi, "bf16")
    ldi = (len(idx_i) + 7) // 8 * 8
    wsl_i = torch.empty(Dout, ldi, dtype=torch.bfloat16, device=DEV)
    ops.weight_slice(Wtd, ii_d, wsl_i)
    yi1, yi2 = empty_pad(T, Dout, "bf16"), empty_pad(T, Dout, "bf16")
    ops.sparse_linear_fwd("in", xid, Wd, Wtd, c_d, o_d, ii_d, yi1, lora=lora_o)
    ops.sparse_linear_fwd("in", xid, Wd, Wtd, c_d, o_d, ii_d, yi2, lora=lora_o, w_slice=wsl_i)
    torch.cuda.synchronize()
    assert np.array_equal(bits(host(yi1)), bits(host(yi2)))
    # backward, side "in" (produces the selected input channels): NO_FILL and
    # the fill of the unselected ones on the side stream
    dx1 = empty_pad(T, Din, "bf16")
    ops.sparse_linear_bwd("in", dyd, None, Wtd, c_d, o_d, ii_d, dx1, lora=lora_b)
    dx2 = empty_pad(T, Din, "bf16", fill=7.0)
    split_out(lambda d: ops.sparse_linear_bwd("in", dyd, None, Wtd, c_d, o_d, ii_d, d, lora=lora_b,
                                              flags=ops.NO_FILL), dx2, Din, ii_d, lora_b)
    assert np.array_equal(bits(host(dx1)), bits(host(dx2)))
    lb = s * (P.astype(np.float64) @ Bi.T.astype(np.float64))
    assert mar(host(dx2)[np.ix_(ctx, drop_i)], lb[np.ix_(ctx, drop_i)]) <= TOL["bf16"]
    # refused before any launch: a slice on the side that builds none, bad flags,
    # a slice narrower than ceil8(n), fp32 fills
    with pytest.raises(ops.SLError):
        ops.sparse_linear_fwd("out", xd, Wd, None, c_d, o_d, io_d, y1, w_slice=wsl)
    with pytest.raises(ops.SLError):
        ops.sparse_linear_fwd("out", xd, Wd, None, c_d, o_d, io_d, y1, flags=8)
    with pytest.raises(ops.SLError):
        ops.sparse_linear_fwd("in", xid, Wd, Wtd, c_d, o_d, ii_d, yi1,
                              w_slice=torch.empty(Dout, ldi - 8, dtype=torch.bfloat16, device=DEV))
    with pytest.raises(ops.SLError):
        ops.lora_fill_unselected(empty_pad(T, Dout, "f32"), c_d, lora_o, io_d)


@pytest.mark.parametrize("D_out,r", [(1000, 16), (28672 // 8, 32), (203, 96)])
def test_lora_gb_with_transposed_b(D_out, r, rng):
    """gB = dy B from B^T kept by the caller (LORA_BT, rows padded to a multiple
    of 8) equals the product from B itself bit for bit, and the oracle."""
    ops = _ops()
    T, s = 300, 2.0
    print(f"[lora-bt] D_out={D_out} r={r}", flush=True)
    Bm = round_dtype(rng.standard_normal((D_out, r)) * 0.05, "bf16")
    dy = round_dtype(rng.standard_normal((T, D_out)), "bf16")
    dyd, Bd = dev_pad(dy, "bf16"), to_dev(Bm, "bf16")
    ld = (D_out + 7) // 8 * 8
    Bt = torch.zeros(r, ld, dtype=torch.bfloat16, device=DEV)
    ops.transpose(Bd, Bt[:, :D_out])
    g1 = torch.empty(T, r, dtype=torch.float32, device=DEV)
    g2 = torch.empty(T, r, dtype=torch.float32, device=DEV)
    ops.lora_fwd_bwd(ops.LORA_GB, None, None, Bd, s, None, dy=dyd, gB=g1, D_in=64, r=r)
    ops.lora_fwd_bwd(ops.LORA_GB | ops.LORA_BT, None, None, Bt, s, None, dy=dyd, gB=g2, D_in=64,
                     D_out=D_out, r=r)
    torch.cuda.synchronize()
    assert np.array_equal(bits(host(g1)), bits(host(g2)))
    assert mar(host(g2), dy.astype(np.float64) @ Bm.astype(np.float64)) <= 1e-5
    with pytest.raises(ops.SLError):       # B^T cannot serve the forward add
        ops.lora_fwd_bwd(ops.LORA_ADD | ops.LORA_BT, None, None, Bt, s, g1,
                         y=empty_pad(T, D_out, "bf16"), D_out=D_out, r=r)


@pytest.mark.parametrize("direction", ["fwd", "bwd"])
def test_row_subset_calls(direction, rng):
    """ONLY_OUT_ROWS and ONLY_CTX_ROWS split a side-OUT-shaped product (forward
    side "out", backward side "in") into its two row sets: each call writes its
    rows only, the out-row call does not use the selection (it is given a wrong one), and
    the two together match the oracle.  Row-subset flags on the other shape are
    refused."""
    ops = _ops()
    roles = _roles(2, 300, 70)
    T, Din, Dout, r, s = 600, 520, 1000, 16, 2.0
    ctx, out, c_d, o_d = _lists(ops, roles)
    print(f"[row-subset] {direction}", flush=True)
    x = round_dtype(rng.standard_normal((T, Din)), "bf16")
    W = round_dtype(rng.standard_normal((Dout, Din)) * 0.05, "bf16")
    P = rng.standard_normal((T, r)).astype(np.float32)
    Bm = round_dtype(rng.standard_normal((Dout, r)) * 0.3, "bf16")
    idx = np.sort(rng.choice(Dout, 333, replace=False)).astype(np.int32)
    lora = (to_dev(P, "f32"), dev_pad(Bm, "bf16"), r, s)
    Wd, Wtd = dev_pad(W, "bf16"), dev_pad(np.ascontiguousarray(W.T), "bf16")
    # valid but wrong: the first channels of the complement, ascending and in range
    wrong = np.setdiff1d(np.arange(Dout, dtype=np.int32), idx)[:len(idx)]
    wrong_d = to_dev(wrong, None)
    y = empty_pad(T, Dout, "bf16", fill=7.0)
    lterm = s * (P.astype(np.float64) @ Bm.T.astype(np.float64))
    if direction == "fwd":
        xd = dev_pad(x, "bf16")
        call = lambda ix, f: ops.sparse_linear_fwd("out", xd, Wd, None, c_d, o_d, ix, y, lora=lora, flags=f)
        want = ref.sparse_linear_fwd("out", x, W, roles, idx) + lterm
    else:
        # backward of a side "in" product whose weight is W^T [Din, Dout]: dy has Din columns
        Wi = np.ascontiguousarray(W.T)                       # [D_out', D_in'] = [Din, Dout]
        dyd = dev_pad(x, "bf16")
        call = lambda ix, f: ops.sparse_linear_bwd("in", dyd, None, Wd, c_d, o_d, ix, y, lora=lora, flags=f)
        want = ref.sparse_linear_bwd("in", x, Wi, roles, idx) + lterm
    call(wrong_d, ops.ONLY_OUT_ROWS)
    torch.cuda.synchronize()
    got = host(y)
    assert np.all(got[ctx] == 7.0)                      # context rows untouched
    assert mar(got[out], want[out]) <= TOL["bf16"]
    call(to_dev(idx, None), ops.ONLY_CTX_ROWS)
    torch.cuda.synchronize()
    got2 = host(y)
    assert np.array_equal(got2[out], got[out])          # output rows untouched
    assert mar(got2, want) <= TOL["bf16"]
    with pytest.raises(ops.SLError):
        call(to_dev(idx, None), ops.ONLY_OUT_ROWS | ops.ONLY_CTX_ROWS)
    with pytest.raises(ops.SLError):
        ops.sparse_linear_fwd("in", dev_pad(x[:, :Din], "bf16"), Wd, Wtd, c_d, o_d,
                              to_dev(np.arange(10, dtype=np.int32), None), empty_pad(T, Dout, "bf16"),
                              flags=ops.ONLY_OUT_ROWS)
