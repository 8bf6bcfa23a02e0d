"""Handle options on the GPU: debug mode's host check of index lists, and a
fixed workspace that refuses to grow."""
import numpy as np
import pytest
import torch

from oracle import reference as ref
from tests.gpu_util import TOL, bits, dev_pad, empty_pad, host, mar, need_lib, to_dev
from workloads.gen import round_dtype

pytestmark = pytest.mark.gpu


def _ops():
    need_lib()
    from contextual_sparsity_lora_amd import ops
    return ops


def _problem(rng, T, T_c, Din, Dout, n):
    roles = np.zeros(T, dtype=np.uint8)
    roles[T_c:] = 1
    ctx, out = ref.token_lists(roles)
    x = round_dtype(rng.standard_normal((T, Din)), "bf16")
    W = round_dtype(rng.standard_normal((Dout, Din)) * 0.05, "bf16")
    idx = np.sort(rng.choice(Dout, n, replace=False)).astype(np.int32)
    return roles, to_dev(ctx, None), to_dev(out, None), x, W, idx


def test_debug_rejects_bad_lists_before_launch(rng):
    """With "debug" on, an index list out of range or not strictly ascending
    is refused on the host before anything is launched; a valid one runs."""
    ops = _ops()
    roles, c, o, x, W, idx = _problem(rng, 300, 200, 256, 512, 100)
    print("[options] debug lists", flush=True)
    xd, Wd = dev_pad(x, "bf16"), dev_pad(W, "bf16")
    y = empty_pad(x.shape[0], W.shape[0], "bf16", fill=3.0)
    oob, neg = idx.copy(), idx.copy()
    oob[-1] = W.shape[0]
    neg[0] = -1
    bad = [oob, neg, idx[::-1].copy(), np.concatenate([idx[:50], idx[49:99]])]
    ops.set_option(0, "debug", 1)
    try:
        for b in bad:
            with pytest.raises(ops.SLError, match="idx"):
                ops.sparse_linear_fwd("out", xd, Wd, None, c, o, to_dev(b.astype(np.int32), None), y)
        torch.cuda.synchronize()
        assert np.all(host(y) == 3.0)   # nothing was launched
        ops.sparse_linear_fwd("out", xd, Wd, None, c, o, to_dev(idx, None), y)
        torch.cuda.synchronize()
        assert mar(host(y), ref.sparse_linear_fwd("out", x, W, roles, idx)) <= TOL["bf16"]
    finally:
        ops.set_option(0, "debug", 0)


def test_fixed_workspace_refuses_growth(rng):
    """On a handle of its own (a new stream): a first call sizes the
    workspace; with "workspace_fixed" on the same call runs and a call needing
    more is refused without allocating; with it off again that call runs."""
    ops = _ops()
    print("[options] fixed workspace", flush=True)
    small = _problem(rng, 300, 200, 256, 512, 100)
    large = _problem(rng, 1200, 1000, 256, 2048, 1500)
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        dev = [(r, c, o, x, W, i, dev_pad(x, "bf16"), dev_pad(W, "bf16"),
                empty_pad(x.shape[0], W.shape[0], "bf16")) for r, c, o, x, W, i in (small, large)]

        def call(k):
            r, c, o, x, W, i, xd, Wd, y = dev[k]
            ops.sparse_linear_fwd("out", xd, Wd, None, c, o, to_dev(i, None), y)

        call(0)
        st.synchronize()
        held = ops.workspace_bytes(0)
        ops.set_option(0, "workspace_fixed", 1)
        try:
            call(0)
            with pytest.raises(ops.SLError, match="workspace"):
                call(1)
            st.synchronize()
            assert ops.workspace_bytes(0) == held
        finally:
            ops.set_option(0, "workspace_fixed", 0)
        call(1)
        st.synchronize()
        assert ops.workspace_bytes(0) > held
        for k in (0, 1):
            r, c, o, x, W, i, xd, Wd, y = dev[k]
            assert mar(host(y), ref.sparse_linear_fwd("out", x, W, r, i)) <= TOL["bf16"]


def test_tuning_options_refuse_bad_values():
    """The launch-tuning options validate their values; a refused value leaves
    the handle's setting as it was."""
    ops = _ops()
    print("[options] tuning refusals", flush=True)
    for name, bad in (("merge_rows", 48), ("merge_rows", 0), ("splitk_min", 1), ("splitk_min", 17),
                      ("splitk_max", 0), ("swiglu_rows", 3)):
        with pytest.raises(ops.SLError):
            ops.set_option(0, name, bad)
    with pytest.raises(ops.SLError):
        ops.set_option(0, "no_such_option", 1)


@pytest.mark.parametrize("rows", [16, 32, 64])
def test_merge_rows_per_wave(rows, rng):
    """Every rows-per-wave form of the compact-product merge (the context rows
    of an output-side bf16 product with its rank-r term) matches the oracle,
    over a ragged row count and channel blocks with and without selected
    channels, and the three forms agree bit for bit."""
    ops = _ops()
    print(f"[options] merge_rows={rows}", flush=True)
    T, T_c, Din, Dout, n, r, s = 301, 250, 136, 1000, 300, 16, 2.0
    roles, c, o, x, W, idx = _problem(rng, T, T_c, Din, Dout, n)
    idx = idx[idx < 600]                                  # the last channel blocks select nothing
    P = rng.standard_normal((T, r)).astype(np.float32)
    Bm = round_dtype(rng.standard_normal((Dout, r)) * 0.3, "bf16")
    ys = []
    for v in (rows, 64):
        y = empty_pad(T, Dout, "bf16", fill=3.0)
        ops.set_option(0, "merge_rows", v)
        try:
            ops.sparse_linear_fwd("out", dev_pad(x, "bf16"), dev_pad(W, "bf16"), None, c, o, to_dev(idx, None), y,
                                  lora=(to_dev(P, "f32"), dev_pad(Bm, "bf16"), r, s))
            torch.cuda.synchronize()
        finally:
            ops.set_option(0, "merge_rows", 64)
        ys.append(host(y))
    want = ref.sparse_linear_fwd("out", x, W, roles, idx) + s * (P.astype(np.float64) @ Bm.T)
    assert mar(ys[0], want) <= TOL["bf16"]
    assert np.array_equal(bits(ys[0]), bits(ys[1]))


def test_splitk_sum_in_tail_launch(rng):
    """An input-side bf16 product whose output rows are split along K (C about
    3n) and whose last partial round is split into K-chunks: the output rows'
    ordered partial sum runs in the tail-sum launch.  With the split tail off
    ("gemm_split" 0) the same sum runs as its own launch after whole tiles:
    the output rows agree bit for bit (same partials, same order), and both
    results match the oracle.  Sizes: 48 output-row partial tiles + 224
    context tiles = 272 tiles, so the 16-tile tail lies in the context rows."""
    ops = _ops()
    print("[options] split-K sum in the tail launch", flush=True)
    T_o, T_c, C, Dout, n = 256, 3584, 1600, 4096, 520
    T = T_o + T_c
    roles, c, o, x, W, _ = _problem(rng, T, T_c, C, Dout, n)
    # an input-side product selects among its C input channels
    idx = np.sort(rng.choice(C, n, replace=False)).astype(np.int32)
    assert idx[0] >= 0 and idx[-1] < C and np.all(np.diff(idx) > 0)
    xd, Wd = dev_pad(x, "bf16"), dev_pad(W, "bf16")
    Wtd = dev_pad(np.ascontiguousarray(W.T), "bf16")
    ys = []
    for split in (1, 0):
        y = empty_pad(T, Dout, "bf16", fill=3.0)
        ops.set_option(0, "gemm_split", split)
        ops.set_option(0, "debug", 1)      # index lists checked on the host before any launch
        try:
            ops.sparse_linear_fwd("in", xd, Wd, Wtd, c, o, to_dev(idx, None), y)
            torch.cuda.synchronize()
        finally:
            ops.set_option(0, "gemm_split", 1)
            ops.set_option(0, "debug", 0)
        ys.append(host(y))
    out = np.arange(T_c, T)
    assert np.array_equal(bits(ys[0][out]), bits(ys[1][out]))
    want = ref.sparse_linear_fwd("in", x, W, roles, idx)
    for yv in ys:
        assert mar(yv, want) <= TOL["bf16"]
