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
LORA_XL, LORA_ADD, LORA_BWD = 1, 2, 4

_handles = {}


class SLError(RuntimeError):
    pass


def _dev(t: torch.Tensor) -> int:
    return t.device.index if t.device.index is not None else torch.cuda.current_device()


def handle(device: int):
    """Per-device library handle, bound to torch's current stream at each call."""
    L = _lib.load()
    h = _handles.get(device)
    if h is None:
        p = ctypes.c_void_p()
        st = L.sl_create(ctypes.byref(p), device)
        if st != 0:
            raise SLError(f"sl_create({device}) failed: {L.sl_status_str(st).decode()}")
        h = _handles[device] = p
    L.sl_set_stream(h, ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream))
    return h


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
    h = handle(device)
    _check(h, _lib.load().sl_sync(h), "sl_sync")


def timing_enable(device: int, enable: bool):
    h = handle(device)
    _check(h, _lib.load().sl_timing_enable(h, int(enable)), "sl_timing_enable")


def timing_reset(device: int):
    h = handle(device)
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
    """(launches, total_ms, flops, bytes) recorded for one kernel class."""
    h = handle(device)
    n = ctypes.c_int64()
    ms, fl, by = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
    st = _lib.load().sl_timing_query(h, kernel_class.encode(), ctypes.byref(n), ctypes.byref(ms),
                                     ctypes.byref(fl), ctypes.byref(by))
    _check(h, st, "sl_timing_query")
    return n.value, ms.value, fl.value, by.value


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


def expand_gqa(idx_kv, n_rep, head_dim, idx_q):
    h = handle(_dev(idx_kv))
    st = _lib.load().sl_expand_gqa(h, _ptr(idx_kv), idx_kv.numel(), n_rep, head_dim, _ptr(idx_q))
    _check(h, st, "sl_expand_gqa")


def stack_index(idx, C, copies, idx_out):
    h = handle(_dev(idx))
    st = _lib.load().sl_stack_index(h, _ptr(idx), idx.numel(), C, copies, _ptr(idx_out))
    _check(h, st, "sl_stack_index")


def sparse_linear_fwd(side, x, W, ctx_rows, out_rows, idx, y, beta=0):
    """side "out": W [D_out, D_in]; side "in": W is the transposed copy [D_in, D_out]."""
    h = handle(_dev(x))
    T, D_in = x.shape
    D_out = W.shape[0] if side == "out" else W.shape[1]
    n = idx.numel() if idx is not None else 0
    st = _lib.load().sl_sparse_linear_fwd(h, SIDE[side], _dt(x), _ptr(x), _ld(x), T, D_in,
                                          _ptr(W), _ld(W), D_out, _ptr(ctx_rows), ctx_rows.numel(),
                                          _ptr(out_rows), out_rows.numel(), _ptr(idx), n, _ptr(y),
                                          _ld(y), int(beta))
    _check(h, st, "sl_sparse_linear_fwd")


def sparse_linear_bwd(side, dy, W, ctx_rows, out_rows, idx, dx, beta=0):
    h = handle(_dev(dy))
    T, D_out = dy.shape
    D_in = W.shape[1] if side == "out" else W.shape[0]
    n = idx.numel() if idx is not None else 0
    st = _lib.load().sl_sparse_linear_bwd(h, SIDE[side], _dt(dy), _ptr(dy), _ld(dy), T, D_out,
                                          _ptr(W), _ld(W), D_in, _ptr(ctx_rows), ctx_rows.numel(),
                                          _ptr(out_rows), out_rows.numel(), _ptr(idx), n, _ptr(dx),
                                          _ld(dx), int(beta))
    _check(h, st, "sl_sparse_linear_bwd")


def lora_fwd_bwd(mode, x, A, B, scale, xl, y=None, dy=None, dx=None, dA=None, dB=None,
                 D_out=None):
    """A: [r, D_in]; B: [D_out, r]; xl: fp32 [T, >= r]."""
    t = x if x is not None else xl
    h = handle(_dev(t))
    r = A.shape[0] if A is not None else B.shape[1]
    T = xl.shape[0]
    D_in = A.shape[1] if A is not None else (x.shape[1] if x is not None else 1)
    if D_out is None:
        D_out = B.shape[0] if B is not None else 1
    dt = _dt(x if x is not None else (y if y is not None else dy))
    st = _lib.load().sl_lora_fwd_bwd(
        h, mode, dt, _ptr(x), _ld(x) if x is not None else 0, T, D_in, D_out, _ptr(A), _ptr(B), r,
        float(scale), _ptr(xl), _ld(xl), _ptr(y), _ld(y) if y is not None else 0, _ptr(dy),
        _ld(dy) if dy is not None else 0, _ptr(dx), _ld(dx) if dx is not None else 0, _ptr(dA),
        _ptr(dB))
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


def transpose(inp, out):
    h = handle(_dev(inp))
    rows, cols = inp.shape
    st = _lib.load().sl_transpose(h, _dt(inp), _ptr(inp), _ld(inp), rows, cols, _ptr(out), _ld(out))
    _check(h, st, "sl_transpose")
