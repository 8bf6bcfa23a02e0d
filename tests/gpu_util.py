"""Helpers shared by the GPU parity tests (host-side conversions only)."""
import numpy as np
import pytest
import torch

DEV = "cuda:0"


def need_lib():
    from contextual_sparsity_lora_amd import _lib
    try:
        _lib.load()
    except RuntimeError as e:  # a GPU run without the built library must fail, not skip
        pytest.fail(str(e))


def to_dev(a, dtype):
    """numpy values (already representable in dtype) -> device tensor."""
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype == "bf16":
        return t.to(torch.bfloat16).to(DEV)
    if dtype == "f32":
        return t.to(torch.float32).to(DEV)
    return t.to(DEV)


def tdt(dtype):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def host(t):
    return t.detach().float().cpu().numpy()


def host_i(t):
    return t.detach().cpu().numpy()


def bits(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


TOL = {"f32": 1e-4, "bf16": 2e-2}


def mar(got, ref):
    """max |got - ref| / max(max |ref|, 1e-30)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    return float(np.max(np.abs(got - ref)) / max(float(np.max(np.abs(ref))), 1e-30))


def sample_rows(ctx, out, n_each, seed=0):
    rng = np.random.default_rng(seed)
    a = rng.choice(ctx, min(n_each, len(ctx)), replace=False) if len(ctx) else np.zeros(0, int)
    b = rng.choice(out, min(n_each, len(out)), replace=False) if len(out) else np.zeros(0, int)
    # always include the first/last rows of each role (tile edges)
    extra = [x for x in (ctx[:1], ctx[-1:], out[:1], out[-1:]) if len(x)]
    return np.unique(np.concatenate([a, b] + extra)).astype(np.int64)


def _padded_cols(cols, dtype):
    q = 8 if dtype == "bf16" else 4
    return max(q, (cols + q - 1) // q * q)


def empty_pad(rows, cols, dtype, fill=None):
    """Device matrix [rows, cols] whose rows are padded to 16 bytes (a view)."""
    buf = torch.empty(rows, _padded_cols(cols, dtype), dtype=tdt(dtype), device=DEV)
    if fill is not None:
        buf.fill_(fill)
    return buf[:, :cols]


def dev_pad(a, dtype):
    a = np.asarray(a)
    v = empty_pad(a.shape[0], a.shape[1], dtype)
    v.copy_(torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(tdt(dtype)).to(DEV))
    return v
