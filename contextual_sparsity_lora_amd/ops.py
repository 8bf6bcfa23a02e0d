"""Python binding of the C ABI: torch tensors in, library calls out.

Argument marshalling only: every computation runs in the library's HIP
kernels.  Tensors are device tensors on the handle's device, row-major with
unit column stride; a row stride other than the width is passed as the
leading dimension (so column slices of a wider buffer work).  Calls enqueue
on torch's current stream of that device.
"""
import ctypes

import torch

from . import _lib

SL_F32, SL_BF16 = 0, 1
CRIT = {"l2": 0, "swiglu": 1, "qk": 2}
SIDE = {"out": 0, "in": 1}
LORA_XL, LORA_ADD, LORA_GB, LORA_DA, LORA_DB, LORA_DX, LORA_BT = 1, 2, 4, 8, 16, 32, 64
LORA_BWD = LORA_GB | LORA_DA | LORA_DB | LORA_DX

_handles = {}


class SLError(RuntimeError):
    pass


def _dev(t: torch.Tensor) -> int:
    return t.device.index if t.device.index is not None else torch.cuda.current_device()


def handle(device: int):
    """Library handle for torch's current stream of the device: one handle (and
    one workspace) per (device, stream), so calls enqueued on different streams
    never share scratch memory."""
    L = _lib.load()
    stream = torch.cuda.current_stream(device).cuda_stream
    key = (device, stream)
    h = _handles.get(key)
    if h is None:
        p = ctypes.c_void_p()
        st = L.sl_create(ctypes.byref(p), device)
        if st != 0:
            raise SLError(f"sl_create({device}) failed: {L.sl_status_str(st).decode()}")
        h = _handles[key] = p
        L.sl_set_stream(h, ctypes.c_void_p(stream))
    return h


def _device_handles(device: int):
    handle(device)
    return [h for (d, _), h in _handles.items() if d == device]


def _check(h, st, what):
    if st != 0:
        L = _lib.load()
        raise SLError(f"{what}: {L.sl_status_str(st).decode()}: {L.sl_last_error(h).decode()}")


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SL_BF16
    if t.dtype == torch.float32:
        return SL_F32
    raise SLError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _ld(t: torch.Tensor) -> int:
    if t.dim() == 2 and t.numel() == 0:
        return max(t.shape[1], 1)
    if t.dim() != 2 or t.stride(1) != 1:
        raise SLError("expected a 2-D tensor with unit column stride")
    return t.stride(0)


def _vec(t):
    if t is not None and (t.dim() != 1 or not t.is_contiguous()):
        raise SLError("expected a contiguous 1-D tensor")
    return t


def sync(device: int = 0):
    for h in _device_handles(device):
        _check(h, _lib.load().sl_sync(h), "sl_sync")


def set_option(device: int, name: str, value: int):
    """sl_set_option on every handle of the device (its streams)."""
    for h in _device_handles(device):
        _check(h, _lib.load().sl_set_option(h, name.encode(), int(value)), "sl_set_option")


def fix_workspaces(device: int = 0):
    """After a first step has sized them: the device's handles grow their
    workspaces no more (a call needing more fails instead of allocating)."""
    set_option(device, "workspace_fixed", 1)


def set_stream_option(stream, name: str, value: int):
    """sl_set_option on the one handle of a given stream (created if missing)."""
    with torch.cuda.stream(stream):
        h = handle(stream.device.index if stream.device.index is not None else 0)
    _check(h, _lib.load().sl_set_option(h, name.encode(), int(value)), "sl_set_option")


def workspace_bytes(device: int = 0) -> int:
    tot = 0
    for h in _device_handles(device):
        b = ctypes.c_size_t()
        _check(h, _lib.load().sl_workspace_bytes(h, ctypes.byref(b)), "sl_workspace_bytes")
        tot += b.value
    return tot


def timing_enable(device: int, enable: bool):
    for h in _device_handles(device):
        _check(h, _lib.load().sl_timing_enable(h, int(enable)), "sl_timing_enable")


def timing_only(device: int, kernel_class=None):
    """Record only launches of kernel_class (None: every class)."""
    for h in _device_handles(device):
        _check(h, _lib.load().sl_timing_only(h, (kernel_class or "").encode()), "sl_timing_only")


def timing_reset(device: int):
    for h in _device_handles(device):
        _check(h, _lib.load().sl_timing_reset(h), "sl_timing_reset")


def timing_classes():
    L = _lib.load()
    out, i = [], 0
    while True:
        n = L.sl_timing_class_name(i)
        if n is None:
            return out
        out.append(n.decode())
        i += 1


def timing_query(device: int, kernel_class: str):
    """(launches, total_ms, flops, bytes) recorded for one kernel class, summed
    over the device's handles (streams)."""
    tot = [0, 0.0, 0.0, 0.0]
    for h in _device_handles(device):
        n = ctypes.c_int64()
        ms, fl, by = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
        st = _lib.load().sl_timing_query(h, kernel_class.encode(), ctypes.byref(n), ctypes.byref(ms),
                                         ctypes.byref(fl), ctypes.byref(by))
        _check(h, st, "sl_timing_query")
        tot[0] += n.value
        tot[1] += ms.value
        tot[2] += fl.value
        tot[3] += by.value
    return tuple(tot)


def token_split(roles, ctx_rows, out_rows):
    h = handle(_dev(roles))
    _vec(roles), _vec(ctx_rows), _vec(out_rows)
    st = _lib.load().sl_token_split(h, _ptr(roles), roles.numel(), _ptr(ctx_rows), ctx_rows.numel(),
                                    _ptr(out_rows), out_rows.numel())
    _check(h, st, "sl_token_split")


def svd_estimate(x, ctx_rows, WA, xa):
    """xa [T_c, k_tot] = x[ctx_rows] @ WA (WA: fp32 [D_in, k_tot]) in the library's R64 order."""
    h = handle(_dev(x))
    T_c = ctx_rows.numel()
    D_in, k_tot = WA.shape
    assert WA.is_contiguous() and xa.is_contiguous() and xa.shape == (T_c, k_tot)
    st = _lib.load().sl_svd_estimate(h, _ptr(x), _dt(x), _ld(x), _ptr(ctx_rows), T_c, D_in,
                                     _ptr(WA), k_tot, _ptr(xa))
    _check(h, st, "sl_svd_estimate")


def score_select(crit, xa, WB0, WB1, n_keep, idx, scores=None, off0=0, off1=None, C=None,
                 n_rep=1, head_dim=1):
    h = handle(_dev(xa))
    k = WB0.shape[0]
    if C is None:
        C = WB1.shape[1] if crit == "qk" else WB0.shape[1]
    if off1 is None:
        off1 = off0 + k
    T_c = xa.shape[0]
    st = _lib.load().sl_score_select(h, CRIT[crit], _ptr(xa), _ld(xa), T_c, off0, _ptr(WB0), off1,
                                     _ptr(WB1), k, C, n_rep, head_dim, n_keep, _ptr(scores),
                                     _ptr(idx))
    _check(h, st, "sl_score_select")


def select_top(scores, n_keep, idx):
    """idx = the n_keep channels with the largest scores (ties: lower index), ascending."""
    h = handle(_dev(scores))
    st = _lib.load().sl_select_top(h, _ptr(scores), scores.numel(), int(n_keep), _ptr(idx))
    _check(h, st, "sl_select_top")


def random_scores(seed, scores):
    """scores (fp32 [C]) = the library's counter-based uniform draws for seed."""
    h = handle(_dev(scores))
    st = _lib.load().sl_random_scores(h, ctypes.c_uint64(int(seed) & ((1 << 64) - 1)), scores.numel(),
                                      _ptr(scores))
    _check(h, st, "sl_random_scores")


def dense_scores(crit, Y0, Y1, rows, scores, C=None, n_rep=1, head_dim=1):
    """Criterion on exact outputs: Y0 (and Y1) are [T, *] views of the dense
    main-branch outputs; rows the context rows; scores fp32 [C] out."""
    h = handle(_dev(Y0))
    if C is None:
        C = Y1.shape[1] if crit in ("qk", "swiglu") else Y0.shape[1]
    st = _lib.load().sl_dense_scores(h, CRIT[crit], _dt(Y0), _ptr(Y0), _ld(Y0), _ptr(Y1),
                                     _ld(Y1) if Y1 is not None else 0, _ptr(rows), rows.numel(), C,
                                     n_rep, head_dim, _ptr(scores))
    _check(h, st, "sl_dense_scores")


def select_heads(scores, n_heads, head_dim, heads_keep, idx):
    """Keep the heads_keep heads with the largest summed channel score; idx
    [heads_keep * head_dim] lists their channels ascending."""
    h = handle(_dev(scores))
    st = _lib.load().sl_select_heads(h, _ptr(scores), n_heads, head_dim, int(heads_keep), _ptr(idx))
    _check(h, st, "sl_select_heads")


def expand_gqa(idx_kv, n_rep, head_dim, idx_q):
    h = handle(_dev(idx_kv))
    st = _lib.load().sl_expand_gqa(h, _ptr(idx_kv), idx_kv.numel(), n_rep, head_dim, _ptr(idx_q))
    _check(h, st, "sl_expand_gqa")


def stack_index(idx, C, copies, idx_out):
    h = handle(_dev(idx))
    st = _lib.load().sl_stack_index(h, _ptr(idx), idx.numel(), C, copies, _ptr(idx_out))
    _check(h, st, "sl_stack_index")


def offset_index(idx, offset, C_max, idx_out):
    """idx_out[q] = idx[q] + offset (idx_out may be a slice of a larger list)."""
    h = handle(_dev(idx))
    st = _lib.load().sl_offset_index(h, _ptr(idx), idx.numel(), int(offset), int(C_max), _ptr(idx_out))
    _check(h, st, "sl_offset_index")


def qkv_index(idx_qk, idx_vo, n_kv_heads, n_rep, head_dim, idx_q, idx_o, idx_qkv):
    """idx_q, idx_o: GQA expansions of idx_qk, idx_vo; idx_qkv: the stacked
    q|k|v channel list [idx_q | idx_qk + Cq | idx_vo + Cq + Ckv]."""
    h = handle(_dev(idx_qkv))
    st = _lib.load().sl_qkv_index(h, _ptr(idx_qk), idx_qk.numel(), _ptr(idx_vo), idx_vo.numel(), n_kv_heads,
                                  n_rep, head_dim, _ptr(idx_q), _ptr(idx_o), _ptr(idx_qkv))
    _check(h, st, "sl_qkv_index")


def _lora_args(lora):
    """lora = (P fp32 [T, >= r], Bm [C, >= r], r, scale) or None."""
    if lora is None:
        return (None, 0, None, 0, 0, 0.0)
    P, Bm, r, scale = lora
    return (_ptr(P), _ld(P), _ptr(Bm), _ld(Bm), int(r), float(scale))


NO_FILL = 1
ONLY_OUT_ROWS = 2
ONLY_CTX_ROWS = 4
CTX_COMPACT = 8


def sparse_linear_fwd(side, x, W, Wt, ctx_rows, out_rows, idx, y, beta=0, lora=None,
                      w_slice=None, flags=0, x_slice=None):
    """W: frozen weight [D_out, D_in] (nn.Linear layout); Wt: its transposed
    copy [D_in, D_out] (read for side "in" only; may be None for side "out").
    lora = (xl, B, r, scale) fuses y += scale * xl B^T into the same pass.
    w_slice: weight_slice(Wt, idx) built beforehand (side "in"); x_slice: the
    context rows' selected columns of x, compact and zero-padded (side "in");
    flags: NO_FILL leaves the unselected context channels (side "out")
    unwritten; CTX_COMPACT | ONLY_CTX_ROWS writes the context rows' product
    compactly to y [T_c, n]."""
    h = handle(_dev(x))
    T, D_in = x.shape
    D_out = W.shape[0]
    n = idx.numel() if idx is not None else 0
    st = _lib.load().sl_sparse_linear_fwd(h, SIDE[side], _dt(x), _ptr(x), _ld(x), T, D_in,
                                          _ptr(W), _ld(W), _ptr(Wt), _ld(Wt) if Wt is not None else 0,
                                          D_out, _ptr(ctx_rows), ctx_rows.numel(), _ptr(out_rows),
                                          out_rows.numel(), _ptr(idx), n, _ptr(y), _ld(y), int(beta),
                                          *_lora_args(lora), _ptr(w_slice),
                                          _ld(w_slice) if w_slice is not None else 0, _ptr(x_slice),
                                          _ld(x_slice) if x_slice is not None else 0, int(flags))
    _check(h, st, "sl_sparse_linear_fwd")


def sparse_linear_bwd(side, dy, W, Wt, ctx_rows, out_rows, idx, dx, beta=0, lora=None,
                      w_slice=None, flags=0, x_slice=None):
    """Input gradient of sparse_linear_fwd.  Wt [D_in, D_out] is read by every
    product; W [D_out, D_in] only for side "out" (may be None for side "in").
    lora = (gB, A^T, r, scale) fuses dx += scale * gB A into the same pass.
    w_slice: weight_slice(W, idx) built beforehand (side "out"); flags as for
    the forward (NO_FILL applies to side "in")."""
    h = handle(_dev(dy))
    T, D_out = dy.shape
    D_in = Wt.shape[0]
    n = idx.numel() if idx is not None else 0
    st = _lib.load().sl_sparse_linear_bwd(h, SIDE[side], _dt(dy), _ptr(dy), _ld(dy), T, D_out,
                                          _ptr(W), _ld(W) if W is not None else 0, _ptr(Wt), _ld(Wt),
                                          D_in, _ptr(ctx_rows), ctx_rows.numel(), _ptr(out_rows),
                                          out_rows.numel(), _ptr(idx), n, _ptr(dx), _ld(dx),
                                          int(beta), *_lora_args(lora), _ptr(w_slice),
                                          _ld(w_slice) if w_slice is not None else 0, _ptr(x_slice),
                                          _ld(x_slice) if x_slice is not None else 0, int(flags))
    _check(h, st, "sl_sparse_linear_bwd")


def weight_slice(Wc, idx, out):
    """out[o, j] = Wc[idx[j], o] (zero columns up to ceil8(n)); Wc bf16 [C, Nout],
    out bf16 [Nout, >= ceil8(n)]."""
    h = handle(_dev(Wc))
    C, Nout = Wc.shape
    st = _lib.load().sl_weight_slice(h, _dt(Wc), _ptr(Wc), _ld(Wc), C, _ptr(idx), idx.numel(), Nout,
                                     _ptr(out), _ld(out))
    _check(h, st, "sl_weight_slice")


def lora_fill_unselected(y, ctx_rows, lora, idx):
    """Write the dense LoRA term alone into the unselected channels of context
    rows of y (bf16 [T, C]); lora = (P, B, r, scale) as for sparse_linear_fwd."""
    h = handle(_dev(y))
    C = y.shape[1]
    st = _lib.load().sl_lora_fill_unselected(h, _dt(y), _ptr(y), _ld(y), _ptr(ctx_rows), ctx_rows.numel(),
                                             C, *_lora_args(lora), _ptr(idx), idx.numel())
    _check(h, st, "sl_lora_fill_unselected")


def lora_fwd_bwd(mode, x, A, B, scale, xl, y=None, dy=None, dx=None, dA=None, dB=None,
                 D_out=None, gB=None, r=None, D_in=None):
    """A: [r, D_in]; B: [D_out, r]; xl, gB: fp32 [T, >= r].  Sizes are taken from
    whichever arguments are present unless given."""
    t = next(v for v in (x, xl, dy, gB) if v is not None)
    h = handle(_dev(t))
    if r is None:
        r = next(v for v in (A.shape[0] if A is not None else None,
                             B.shape[1] if B is not None else None,
                             dA.shape[0] if dA is not None else None,
                             dB.shape[1] if dB is not None else None) if v is not None)
    T = next(v.shape[0] for v in (x, xl, dy, gB, y, dx) if v is not None)
    if D_in is None:
        D_in = next((v for v in (A.shape[1] if A is not None else None,
                                 x.shape[1] if x is not None else None,
                                 dA.shape[1] if dA is not None else None,
                                 dx.shape[1] if dx is not None else None) if v is not None), 1)
    if D_out is None:
        D_out = next((v for v in (B.shape[0] if B is not None else None,
                                  dy.shape[1] if dy is not None else None,
                                  y.shape[1] if y is not None else None,
                                  dB.shape[0] if dB is not None else None) if v is not None), 1)
    dt = _dt(next(v for v in (x, y, dy, dx, A, B) if v is not None))
    ld = lambda v: _ld(v) if v is not None else 0
    st = _lib.load().sl_lora_fwd_bwd(
        h, mode, dt, _ptr(x), ld(x), T, D_in, D_out, _ptr(A), _ptr(B), r, float(scale), _ptr(xl),
        ld(xl), _ptr(y), ld(y), _ptr(dy), ld(dy), _ptr(dx), ld(dx), _ptr(dA), _ptr(dB), _ptr(gB),
        ld(gB))
    _check(h, st, "sl_lora_fwd_bwd")


def swiglu_fwd(g, u, hout):
    h = handle(_dev(g))
    T, F = g.shape
    st = _lib.load().sl_swiglu_fwd(h, _dt(g), _ptr(g), _ld(g), _ptr(u), _ld(u), T, F, _ptr(hout),
                                   _ld(hout))
    _check(h, st, "sl_swiglu_fwd")


def swiglu_bwd(dh, g, u, dg, du):
    h = handle(_dev(g))
    T, F = g.shape
    st = _lib.load().sl_swiglu_bwd(h, _dt(g), _ptr(dh), _ld(dh), _ptr(g), _ld(g), _ptr(u), _ld(u),
                                   T, F, _ptr(dg), _ld(dg), _ptr(du), _ld(du))
    _check(h, st, "sl_swiglu_bwd")


def swiglu_fwd_lora(g, u, hout, A, xl, rows=None):
    """hout = silu(g) u and xl = hout A^T (fp32 [T, r]) in one pass over g, u
    (bf16; A [r, F]); rows: only those rows (int32 device list)."""
    h = handle(_dev(g))
    T, F = g.shape
    st = _lib.load().sl_swiglu_fwd_lora(h, _dt(g), _ptr(g), _ld(g), _ptr(u), _ld(u), T, F, _ptr(rows),
                                        rows.numel() if rows is not None else 0, _ptr(hout), _ld(hout),
                                        _ptr(A), _ld(A), A.shape[0], _ptr(xl), _ld(xl))
    _check(h, st, "sl_swiglu_fwd_lora")


def swiglu_fwd_ctx(Yc, ctx_rows, idx, lora, gu, hc, A, xl, h_rows=None):
    """Context rows of a sparse SwiGLU FFN from the compact gate|up product Yc
    [T_c, >= 2n]: merged gate|up rows into gu [T, 2F], compact h into hc
    [T_c, >= ceil8(n)], and xl = h A^T rows (fp32); h_rows [T, F] optionally
    receives the whole h rows.  lora = (xl_gu, B_bd, 2r, scale) as for the
    gate|up product."""
    h = handle(_dev(gu))
    T, F2 = gu.shape
    P, B, r2, s = lora
    n = idx.numel()
    st = _lib.load().sl_swiglu_fwd_ctx(h, _dt(gu), _ptr(Yc), _ld(Yc), _ptr(ctx_rows), ctx_rows.numel(), T,
                                       F2 // 2, _ptr(idx), n, _ptr(P), _ld(P), _ptr(B), _ld(B), int(r2), float(s),
                                       _ptr(gu), _ld(gu), _ptr(hc), _ld(hc), _ptr(A), _ld(A), A.shape[0],
                                       _ptr(xl), _ld(xl), _ptr(h_rows), _ld(h_rows) if h_rows is not None else 0)
    _check(h, st, "sl_swiglu_fwd_ctx")


def swiglu_bwd_lora(dh, g, u, dg, du, gB, xl_g, xl_u, scale, dA, dB_g, dB_u):
    """dg, du as swiglu_bwd, with dA = scale gB^T h ([r, F]), dB_g = scale
    dg^T xl_g and dB_u = scale du^T xl_u ([F, r]) from the same pass (bf16)."""
    h = handle(_dev(g))
    T, F = g.shape
    r = gB.shape[1]
    st = _lib.load().sl_swiglu_bwd_lora(h, _dt(g), _ptr(dh), _ld(dh), _ptr(g), _ld(g), _ptr(u), _ld(u), T, F,
                                        _ptr(dg), _ld(dg), _ptr(du), _ld(du), _ptr(gB), _ld(gB), _ptr(xl_g),
                                        _ld(xl_g), _ptr(xl_u), _ld(xl_u), r, float(scale), _ptr(dA), _ptr(dB_g),
                                        _ptr(dB_u))
    _check(h, st, "sl_swiglu_bwd_lora")


def svd_factors(W, Wt, k, WA_t, WB, oversample=16, iters=3, seed=0):
    """Rank-k estimator factors of W [D_out, D_in] (with its transposed copy Wt)
    into WA_t fp32 [k, D_in] and WB fp32 [k, D_out]."""
    h = handle(_dev(W))
    D_out, D_in = W.shape
    st = _lib.load().sl_svd_factors(h, _dt(W), _ptr(W), _ld(W), _ptr(Wt), _ld(Wt), D_out, D_in, int(k),
                                    int(oversample), int(iters), ctypes.c_uint64(int(seed) & ((1 << 64) - 1)),
                                    _ptr(WA_t), _ptr(WB))
    _check(h, st, "sl_svd_factors")


def token_ce(logits, rows, labels, dlogits, loss, scale=None):
    """Softmax cross-entropy of logits [T, V] on the listed rows against
    labels[row]; dlogits = scale (softmax - onehot) on those rows; loss (fp64
    [1] on the device) = scale * sum of row losses (scale default 1/len(rows)).
    A row whose label is outside [0, V) is ignored (zero loss, zero gradient);
    pass scale = 1 / (rows with a label in range) for the mean over the rest."""
    h = handle(_dev(logits))
    n = rows.numel()
    if scale is None:
        scale = 1.0 / max(n, 1)
    st = _lib.load().sl_token_ce(h, _dt(logits), _ptr(logits), _ld(logits), _ptr(rows), n, _ptr(labels),
                                 logits.shape[1], float(scale), _ptr(dlogits), _ld(dlogits), _ptr(loss))
    _check(h, st, "sl_token_ce")


class AdamwTensor(ctypes.Structure):
    _fields_ = [("param", ctypes.c_void_p), ("grad", ctypes.c_void_p), ("m", ctypes.c_void_p),
                ("v", ctypes.c_void_p), ("out", ctypes.c_void_p), ("ld_out", ctypes.c_int64),
                ("rows", ctypes.c_int64), ("cols", ctypes.c_int64), ("out_dtype", ctypes.c_int)]


def adamw_step(groups, lr, step, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0):
    """groups: list of (param fp32, grad fp32, m, v, out view (bf16 or fp32) or
    None), param/grad/m/v contiguous of one shape [rows, cols] (or 1-d)."""
    if not groups:
        return
    h = handle(_dev(groups[0][0]))
    arr = (AdamwTensor * len(groups))()
    for i, (p, g, m, v, out) in enumerate(groups):
        assert all(t.is_contiguous() and t.dtype == torch.float32 and t.shape == p.shape for t in (p, g, m, v))
        rows, cols = (p.shape[0], p.shape[1]) if p.dim() == 2 else (1, p.numel())
        if out is not None:
            assert tuple(out.shape) == (rows, cols) and (out.stride(1) == 1 or cols == 1)
        arr[i] = AdamwTensor(p.data_ptr(), g.data_ptr(), m.data_ptr(), v.data_ptr(),
                             out.data_ptr() if out is not None else None,
                             out.stride(0) if out is not None else 0, rows, cols,
                             _dt(out) if out is not None else 0)
    st = _lib.load().sl_adamw_step(h, arr, len(groups), float(lr), float(beta1), float(beta2), float(eps),
                                   float(weight_decay), int(step))
    _check(h, st, "sl_adamw_step")


def dot_stats(a, b, out):
    """out (fp64 [3] on the device) = (a.b, a.a, b.b) over the fp32 elements of
    two contiguous tensors of the same size."""
    assert a.is_contiguous() and b.is_contiguous() and a.numel() == b.numel()
    assert a.dtype == torch.float32 and b.dtype == torch.float32 and out.dtype == torch.float64
    h = handle(_dev(a))
    st = _lib.load().sl_dot_stats(h, _ptr(a), _ptr(b), a.numel(), _ptr(out))
    _check(h, st, "sl_dot_stats")


def transpose(inp, out):
    h = handle(_dev(inp))
    rows, cols = inp.shape
    st = _lib.load().sl_transpose(h, _dt(inp), _ptr(inp), _ld(inp), rows, cols, _ptr(out), _ld(out))
    _check(h, st, "sl_transpose")


def rmsnorm_fwd(x, y, rstd, res=None, hsum=None, eps=1e-5):
    """y = hsum / sqrt(mean(hsum^2) + eps) with hsum = x (+ res; stored to hsum)."""
    h = handle(_dev(x))
    T, D = x.shape
    ld = lambda v: _ld(v) if v is not None else 0
    st = _lib.load().sl_rmsnorm_fwd(h, _dt(x), _ptr(x), _ld(x), _ptr(res), ld(res), T, D, float(eps),
                                    _ptr(hsum), ld(hsum), _ptr(y), _ld(y), _ptr(rstd))
    _check(h, st, "sl_rmsnorm_fwd")


def rmsnorm_bwd(x, rstd, dy, dx, dres=None):
    h = handle(_dev(x))
    T, D = x.shape
    st = _lib.load().sl_rmsnorm_bwd(h, _dt(x), _ptr(x), _ld(x), _ptr(rstd), _ptr(dy), _ld(dy),
                                    _ptr(dres), _ld(dres) if dres is not None else 0, T, D, _ptr(dx),
                                    _ld(dx))
    _check(h, st, "sl_rmsnorm_bwd")


def add(a, b, out):
    h = handle(_dev(a))
    T, D = a.shape
    st = _lib.load().sl_add(h, _dt(a), _ptr(a), _ld(a), _ptr(b), _ld(b), T, D, _ptr(out), _ld(out))
    _check(h, st, "sl_add")


def attention_fwd(q, k, v, batch, seq, n_heads, n_kv_heads, head_dim, o, lse):
    h = handle(_dev(q))
    st = _lib.load().sl_attention_fwd(h, _dt(q), _ptr(q), _ld(q), _ptr(k), _ld(k), _ptr(v), _ld(v),
                                      batch, seq, n_heads, n_kv_heads, head_dim, _ptr(o), _ld(o),
                                      _ptr(lse))
    _check(h, st, "sl_attention_fwd")


def attention_bwd(q, k, v, o, dout, lse, batch, seq, n_heads, n_kv_heads, head_dim, dq, dk, dv):
    h = handle(_dev(q))
    st = _lib.load().sl_attention_bwd(h, _dt(q), _ptr(q), _ld(q), _ptr(k), _ld(k), _ptr(v), _ld(v),
                                      _ptr(o), _ld(o), _ptr(dout), _ld(dout), _ptr(lse), batch, seq,
                                      n_heads, n_kv_heads, head_dim, _ptr(dq), _ld(dq), _ptr(dk),
                                      _ld(dk), _ptr(dv), _ld(dv))
    _check(h, st, "sl_attention_bwd")
