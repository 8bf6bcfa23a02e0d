"""GPU parity of the causal attention core (forward with its log-sum-exp, and
backward) against the fp64 oracle: bf16 on the matrix-core kernels (head
dimensions 32, 64, 128; GQA; ragged sequence lengths; q, k, v as column
slices of one stacked buffer) and fp32 on the plain kernels."""
import numpy as np
import pytest
import torch

from oracle import reference as ref
from tests.gpu_util import DEV, TOL, host, mar, need_lib
from workloads.gen import round_dtype

pytestmark = pytest.mark.gpu

CASES = [
    # dtype, B, S, H, Hkv, d
    ("bf16", 2, 150, 4, 2, 32),
    ("bf16", 1, 97, 2, 2, 64),
    ("bf16", 2, 200, 8, 2, 128),
    ("bf16", 1, 64, 2, 1, 128),
    ("bf16", 1, 1, 2, 2, 64),
    ("f32", 2, 70, 4, 2, 32),
]


def _lse(q, k, B, S, H, Hkv, d):
    n_rep = H // Hkv
    out = np.zeros((B, H, S))
    mask = np.tril(np.ones((S, S), bool))
    for b in range(B):
        Q = q[b * S:(b + 1) * S].reshape(S, H, d).transpose(1, 0, 2).astype(np.float64)
        K = k[b * S:(b + 1) * S].reshape(S, Hkv, d).transpose(1, 0, 2).astype(np.float64)
        for h in range(H):
            s = np.where(mask, Q[h] @ K[h // n_rep].T / np.sqrt(d), -np.inf)
            mx = s.max(axis=1)
            out[b, h] = mx + np.log(np.exp(s - mx[:, None]).sum(axis=1))
    return out.reshape(-1)


@pytest.mark.parametrize("case", CASES)
def test_attention_core(case, rng):
    need_lib()
    from contextual_sparsity_lora_amd import ops
    dt, B, S, H, Hkv, d = case
    print(f"[attn-core] {case}", flush=True)
    T, Cq, Ckv = B * S, H * d, Hkv * d
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    qkv = round_dtype(rng.standard_normal((T, Cq + 2 * Ckv)) * 1.5, dt)
    q, k, v = qkv[:, :Cq], qkv[:, Cq:Cq + Ckv], qkv[:, Cq + Ckv:]
    buf = torch.from_numpy(qkv.astype(np.float32)).to(tdt).to(DEV)
    qd, kd, vd = buf[:, :Cq], buf[:, Cq:Cq + Ckv], buf[:, Cq + Ckv:]
    o = torch.empty(T, Cq, dtype=tdt, device=DEV)
    lse = torch.empty(B * H * S, dtype=torch.float32, device=DEV)
    ops.attention_fwd(qd, kd, vd, B, S, H, Hkv, d, o, lse)
    torch.cuda.synchronize()
    tol = TOL[dt]
    assert mar(host(o), ref.attention_fwd(q, k, v, B, S, H, Hkv, d)) <= tol
    assert np.max(np.abs(host(lse) - _lse(q, k, B, S, H, Hkv, d))) <= (5e-3 if dt == "bf16" else 1e-4)
    # backward, with the GPU's own o and lse
    do = round_dtype(rng.standard_normal((T, Cq)), dt)
    dq = torch.empty(T, Cq, dtype=tdt, device=DEV)
    dk = torch.empty(T, Ckv, dtype=tdt, device=DEV)
    dv = torch.empty(T, Ckv, dtype=tdt, device=DEV)
    ops.attention_bwd(qd, kd, vd, o, torch.from_numpy(do.astype(np.float32)).to(tdt).to(DEV), lse, B, S, H, Hkv,
                      d, dq, dk, dv)
    torch.cuda.synchronize()
    dq_r, dk_r, dv_r = ref.attention_bwd(q, k, v, do, B, S, H, Hkv, d)
    if S == 1:
        # one visible key: softmax is 1, dS = P (dP - delta) = 0, so dQ and dK
        # are exactly zero and only rounding of dP against delta remains
        assert np.max(np.abs(host(dq))) <= 1e-3 and np.max(np.abs(host(dk))) <= 1e-3
        assert np.all(dq_r == 0) and np.all(dk_r == 0)
    else:
        assert mar(host(dq), dq_r) <= tol
        assert mar(host(dk), dk_r) <= tol
    assert mar(host(dv), dv_r) <= tol


def test_attention_rejects_unaligned_rows():
    """Rows that are not 16-byte aligned (q, k, v one column into a stacked
    buffer) are refused with an error before any launch."""
    need_lib()
    from contextual_sparsity_lora_amd import ops
    B, S, H, Hkv, d = 1, 16, 2, 2, 32
    T, Cq, Ckv = B * S, H * d, Hkv * d
    buf = torch.zeros(T, 1 + Cq + 2 * Ckv, dtype=torch.bfloat16, device=DEV)
    qd, kd, vd = buf[:, 1:1 + Cq], buf[:, 1 + Cq:1 + Cq + Ckv], buf[:, 1 + Cq + Ckv:]
    o = torch.empty(T, Cq, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(B * H * S, dtype=torch.float32, device=DEV)
    with pytest.raises(ops.SLError):
        ops.attention_fwd(qd, kd, vd, B, S, H, Hkv, d, o, lse)
