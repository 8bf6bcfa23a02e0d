"""The allocation-free score selection (sl_score_select_noalloc) against the
allocating entry point: same scores and the same selected channels, bit for
bit, on two calls in a row (the second smaller), for the QK criterion (which
uses the library scratch for its ssq vectors and chain partials) and the
L2 / SwiGLU criteria with the scores kept in the scratch.  Calls go through
the C ABI with ctypes."""
import ctypes

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

CRIT = {"l2": 0, "swiglu": 1, "qk": 2}


def _handle(torch, L):
    h = ctypes.c_void_p()
    assert L.sl_create(ctypes.byref(h), 0) == 0
    L.sl_set_stream(h, ctypes.c_void_p(torch.cuda.current_stream(0).cuda_stream))
    return h


def _run(torch, L, h, fn, crit, xa, WB0, WB1, k, C, n_rep, d, n_keep, off1, with_scores):
    dev = xa.device
    idx = torch.full((max(n_keep, 1),), -1, dtype=torch.int32, device=dev)
    sc = torch.full((C,), -1.0, dtype=torch.float32, device=dev) if with_scores else None
    p = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None
    st = fn(h, CRIT[crit], p(xa), xa.shape[1], xa.shape[0], 0, p(WB0), off1, p(WB1), k, C, n_rep, d,
            n_keep, p(sc), p(idx))
    assert st == 0, L.sl_last_error(h).decode()
    torch.cuda.synchronize()
    return (sc.cpu().numpy().view(np.uint32) if sc is not None else None), idx[:n_keep].cpu().numpy()


CASES = [
    # crit, T_c, k, C (selection space), n_rep, head_dim, n_keep, scores given
    [("qk", 3072, 16, 1024, 4, 128, 512, True), ("qk", 700, 16, 256, 2, 64, 100, True)],
    [("l2", 3072, 16, 4096, 1, 1, 2049, False), ("l2", 513, 8, 1000, 1, 1, 7, False)],
    [("swiglu", 3072, 16, 14336, 1, 1, 4301, False), ("swiglu", 96, 8, 688, 1, 1, 344, False)],
]


@pytest.mark.parametrize("pair", CASES, ids=["qk", "l2", "swiglu"])
def test_noalloc_matches_score_select(pair):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from contextual_sparsity_lora_amd import _lib
    L = _lib.load()
    h = _handle(torch, L)
    try:
        g = torch.Generator(device="cuda:0")
        g.manual_seed(77)
        for crit, T_c, k, C, n_rep, d, n_keep, given in pair:
            ktot = 2 * k
            xa = torch.randn(T_c, ktot, generator=g, device="cuda:0")
            WB0 = torch.randn(k, C * n_rep, generator=g, device="cuda:0")
            WB1 = torch.randn(k, C, generator=g, device="cuda:0") if crit != "l2" else None
            args = (crit, xa, WB0, WB1, k, C, n_rep, d, n_keep, k, given)
            ref_sc, ref_idx = _run(torch, L, h, L.sl_score_select, *args)
            got_sc, got_idx = _run(torch, L, h, L.sl_score_select_noalloc, *args)
            assert np.array_equal(got_idx, ref_idx), (crit, T_c, C)
            assert np.all(np.diff(got_idx) > 0) and got_idx.min() >= 0 and got_idx.max() < C
            if given:
                assert np.array_equal(got_sc, ref_sc), (crit, T_c, C)
    finally:
        L.sl_destroy(h)


def test_noalloc_rejects_oversized_scratch():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from contextual_sparsity_lora_amd import _lib
    L = _lib.load()
    h = _handle(torch, L)
    try:
        xa = torch.zeros(4, 32, device="cuda:0")
        WB = torch.zeros(16, 8, device="cuda:0")
        idx = torch.zeros(1, dtype=torch.int32, device="cuda:0")
        p = lambda t: ctypes.c_void_p(t.data_ptr())
        # QK over 16384 key/value channels with 128 query heads per group:
        # 8 MiB of ssq scratch, above the fixed 4 MiB (rejected before any launch)
        st = L.sl_score_select_noalloc(h, 2, p(xa), 32, 4, 0, p(WB), 16, p(WB), 16, 16384, 128, 128, 1,
                                       None, p(idx))
        assert st == -4 and b"scratch" in L.sl_last_error(h)
    finally:
        L.sl_destroy(h)
