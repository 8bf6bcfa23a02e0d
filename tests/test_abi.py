"""The C-ABI library loads without a GPU and exports every entry point that
include/sparselora.h declares; the binding's signature table matches them."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparselora.h")


def declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(sl_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_method_calls():
    names = declared()
    for n in ("sl_svd_estimate", "sl_score_select", "sl_sparse_linear_fwd",
              "sl_sparse_linear_bwd", "sl_lora_fwd_bwd", "sl_token_split"):
        assert n in names


def test_library_exports_every_declared_symbol():
    from contextual_sparsity_lora_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from contextual_sparsity_lora_amd import build
        build.build()
    L = ctypes.CDLL(_lib.LIB_PATH)
    missing = [n for n in declared() if not hasattr(L, n)]
    assert not missing, missing
    assert set(_lib.SIGNATURES) == set(declared())
    _lib.load()
    assert L.sl_version  # loads and resolves without a GPU


def test_calls_without_device_fail_cleanly():
    from contextual_sparsity_lora_amd import _lib
    L = _lib.load()
    p = ctypes.c_void_p()
    st = L.sl_create(ctypes.byref(p), 0)
    try:
        import torch
        has_gpu = torch.cuda.is_available()
    except Exception:
        has_gpu = False
    if not has_gpu:
        assert st != 0 and not p.value          # no device: clean error, no handle
    assert L.sl_status_str(-1) == b"SL_ERR_INVALID"
    # NULL handle is rejected everywhere
    assert L.sl_sync(None) == -1
    assert L.sl_set_stream(None, None) == -1
