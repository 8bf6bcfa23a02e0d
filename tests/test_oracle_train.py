"""Pins of the oracle's training-step functions (CPU): the token loss against
torch's cross_entropy and autograd, AdamW against torch.optim.AdamW, the
learning-rate schedule's closed forms, bf16 rounding against torch's
conversion, and one whole step against a torch build of the same step."""
import math

import numpy as np
import pytest
import torch

from oracle import reference as ref
from workloads.configs import CONFIGS, scaled
from workloads.gen import make_ffn_inputs


def test_token_ce_matches_torch(rng):
    z = rng.standard_normal((9, 31)) * 3
    y = rng.integers(0, 31, size=9)
    loss, dz = ref.token_ce(z, y)
    zt = torch.tensor(z, requires_grad=True)
    lt = torch.nn.functional.cross_entropy(zt, torch.tensor(y))
    lt.backward()
    assert loss == pytest.approx(float(lt.detach()), abs=1e-13)
    assert np.allclose(dz, zt.grad.numpy(), atol=1e-15, rtol=1e-12)
    assert ref.token_ce(np.zeros((0, 5)), np.zeros(0, int))[0] == 0.0


def test_token_ce_ignored_labels_match_torch(rng):
    """Positions whose label is the ignore index -100 drop out of the loss, its
    mean and its gradient, as torch's cross_entropy(ignore_index=-100) does."""
    z = rng.standard_normal((12, 23)) * 3
    y = rng.integers(0, 23, size=12)
    y[[0, 5, 6, 11]] = -100
    loss, dz = ref.token_ce(z, y)
    zt = torch.tensor(z, requires_grad=True)
    lt = torch.nn.functional.cross_entropy(zt, torch.tensor(y), ignore_index=-100)
    lt.backward()
    assert loss == pytest.approx(float(lt.detach()), abs=1e-13)
    assert np.allclose(dz, zt.grad.numpy(), atol=1e-15, rtol=1e-12)
    assert np.all(dz[[0, 5, 6, 11]] == 0.0)
    # every label ignored: zero loss, zero gradient
    l0, d0 = ref.token_ce(z[:3], np.array([-100, 23, 99]))
    assert l0 == 0.0 and np.all(d0 == 0.0)


def test_adamw_matches_torch(rng):
    p0 = rng.standard_normal((4, 6))
    pt = torch.tensor(p0, requires_grad=True)
    opt = torch.optim.AdamW([pt], lr=0.01, betas=(0.8, 0.95), eps=1e-6, weight_decay=0.1)
    p, m, v = p0.copy(), np.zeros_like(p0), np.zeros_like(p0)
    for step in range(1, 6):
        g = rng.standard_normal(p0.shape)
        lr = 0.01 * step / 5
        for grp in opt.param_groups:
            grp["lr"] = lr
        pt.grad = torch.tensor(g)
        opt.step()
        p, m, v = ref.adamw(p, g, m, v, step, lr, 0.8, 0.95, 1e-6, 0.1)
        assert np.allclose(p, pt.detach().numpy(), atol=1e-14, rtol=1e-12)


def test_lr_schedule_closed_forms():
    N, peak = 200, 2.0
    w = math.ceil(0.04 * N)     # 8
    assert ref.lr_schedule(0, N, peak) == 0.0
    assert ref.lr_schedule(w // 2, N, peak) == pytest.approx(peak / 2)
    assert ref.lr_schedule(w, N, peak) == pytest.approx(peak)
    assert ref.lr_schedule(w + (N - w) // 2, N, peak) == pytest.approx(peak / 2)
    assert ref.lr_schedule(N, N, peak) == pytest.approx(0.0, abs=1e-15)
    vals = [ref.lr_schedule(s, N, peak) for s in range(w, N)]
    assert all(a >= b for a, b in zip(vals, vals[1:]))


def test_bf16_rounding_matches_torch(rng):
    a = np.concatenate([rng.standard_normal(5000) * 10.0 ** rng.integers(-30, 30, 5000),
                        [0.0, -0.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 65504.0]])
    want = torch.tensor(a.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(ref.round_to(a, "bf16"), want)


def test_one_training_step_matches_torch(rng):
    """A dense step and a sparse step of ffn_train against autograd through the
    masked block, the head and cross_entropy, with torch's AdamW."""
    cfg = scaled(CONFIGS[1], batch=2, seq=12, out_per_seq=3, hidden=10, inter=14, lora_rank=3, est_rank=2)
    inp = make_ffn_inputs(cfg, with_factors=False)
    inp = {k: (np.asarray(v, np.float64) if isinstance(v, np.ndarray) and k != "roles" else v)
           for k, v in inp.items()}
    for k in ref.LORA_FFN:
        inp[k] = rng.standard_normal(inp[k].shape) * 0.5
    V = 7
    W_head = rng.standard_normal((V, cfg.hidden))
    xs = [rng.standard_normal((cfg.tokens, cfg.hidden)) for _ in range(2)]
    labels = [rng.integers(0, V, size=cfg.tokens) for _ in range(2)]
    idx = np.sort(rng.choice(cfg.inter, 6, replace=False))
    losses, master = ref.ffn_train(inp, W_head, xs, labels, total=2, n_dense=1, select=lambda x: idx,
                                   dtype="f64", lr=0.05, warmup_ratio=0.0, wd=0.01)
    # torch
    T, F, s = cfg.tokens, cfg.inter, inp["scale"]
    ctx, out = ref.token_lists(inp["roles"])
    params = {k: torch.tensor(inp[k], requires_grad=True) for k in ref.LORA_FFN}
    opt = torch.optim.AdamW(list(params.values()), lr=0.05, weight_decay=0.01)
    lin = torch.nn.functional.linear
    W = {k: torch.tensor(inp[k]) for k in ("W_gate", "W_up", "W_down")}
    for t in range(2):
        M = torch.ones(T, F, dtype=torch.float64) if t == 0 else torch.tensor(ref.keep_mask(T, F, inp["roles"], idx))
        x = torch.tensor(xs[t])
        g = lin(x, W["W_gate"]) * M + s * lin(lin(x, params["A_gate"]), params["B_gate"])
        u = lin(x, W["W_up"]) * M + s * lin(lin(x, params["A_up"]), params["B_up"])
        h = torch.nn.functional.silu(g) * u
        y = lin(h * M, W["W_down"]) + s * lin(lin(h, params["A_down"]), params["B_down"])
        logits = lin(y[torch.tensor(out)], torch.tensor(W_head))
        loss = torch.nn.functional.cross_entropy(logits, torch.tensor(labels[t][out]))
        assert losses[t] == pytest.approx(float(loss), rel=1e-11)
        opt.zero_grad()
        loss.backward()
        for grp in opt.param_groups:
            grp["lr"] = ref.lr_schedule(t, 2, 0.05, 0.0)
        opt.step()
    for k in ref.LORA_FFN:
        assert np.allclose(master[k], params[k].detach().numpy(), atol=1e-12, rtol=1e-10), k
