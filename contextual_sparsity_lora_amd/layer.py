"""One decoder layer whose seven linears are contextually sparse with dense
LoRA: pre-norm attention (q/k/v/o sparse by the QK and VO criteria, plain
causal softmax core) and a pre-norm SwiGLU FFN (gate/up/down sparse by the FFN
criterion), residual adds, forward and backward.

Pages ("SparseLoRA: Accelerating LLM Fine-Tuning with Contextual Sparsity"):
the method applies to every linear of LLaMA decoder layers (paper-graph summary
§3.4, one selection per layer group per batch, estimated from that group's
input); the layer topology around the linears is pre-RMSNorm with unit weight,
residual adds, causal softmax attention with scale 1/sqrt(d) and no position
encoding.  Everything below is marshalling: each step is one C-ABI call.

    n1 = rmsnorm(x);  qkv = sparse q|k|v(n1);  a = attention(q, k, v)
    o = sparse o(a);  h1 = x + o;  n2 = rmsnorm(h1);  y = h1 + ffn(n2)
"""
import torch

from . import ops
from .attn import SparseAttnProj
from .ffn import SparseFFN


class SparseDecoderLayer:
    def __init__(self, attn: SparseAttnProj, ffn: SparseFFN, batch, seq, n_heads, n_kv_heads,
                 head_dim, eps=1e-5):
        self.attn, self.ffn = attn, ffn
        self.B, self.S, self.H, self.Hkv, self.hd = batch, seq, n_heads, n_kv_heads, head_dim
        self.eps = eps
        self._T = None

    @classmethod
    def from_arrays(cls, d, f32, cfg, qk_sparsity, vo_sparsity, ffn_sparsity, dense=False):
        """Build from device tensors d[...] (dtype of the layer) and fp32 factor
        tensors f32[...]: WA_qkv [D, 3k], WA_gu [D, 2k] (estimator W_A factors
        side by side) and WB_q, WB_k, WB_v, WB_gate, WB_up (may be absent when
        dense)."""
        f32 = dict(f32)
        attn = SparseAttnProj(d["W_q"], d["W_k"], d["W_v"], d["W_o"], d["A_q"], d["B_q"], d["A_k"],
                              d["B_k"], d["A_v"], d["B_v"], d["A_o"], d["B_o"], f32.get("WA_qkv"),
                              f32.get("WB_q"), f32.get("WB_k"), f32.get("WB_v"), cfg.lora_scale, cfg.n_kv_heads,
                              cfg.head_dim, qk_sparsity=qk_sparsity, vo_sparsity=vo_sparsity,
                              dense=dense)
        ffn = SparseFFN(d["W_gate"], d["W_up"], d["W_down"], d["A_gate"], d["B_gate"], d["A_up"],
                        d["B_up"], d["A_down"], d["B_down"], f32.get("WA_gu"), f32.get("WB_gate"),
                        f32.get("WB_up"), cfg.lora_scale, sparsity=ffn_sparsity, dense=dense)
        return cls(attn, ffn, cfg.batch, cfg.seq, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim)

    def _alloc(self, T, D, dev, dt):
        if self._T == T:
            return
        e = lambda *s, **kw: torch.empty(*s, device=dev, **kw)
        Cq = self.H * self.hd
        self.n1, self.h1, self.n2, self.y = (e(T, D, dtype=dt) for _ in range(4))
        self.rstd1, self.rstd2 = e(T, dtype=torch.float32), e(T, dtype=torch.float32)
        self.a = e(T, Cq, dtype=dt)
        self.lse = e(self.B * self.H * self.S, dtype=torch.float32)
        self.dh1, self.dx = e(T, D, dtype=dt), e(T, D, dtype=dt)
        self.dqkv = e(T, self.attn.Cs, dtype=dt)
        self._T = T

    def forward(self, x, roles, T_c):
        T, D = x.shape
        assert T == self.B * self.S
        self._alloc(T, D, x.device, x.dtype)
        self.x = x
        Cq, Ckv = self.attn.Cq, self.attn.Ckv
        ops.rmsnorm_fwd(x, self.n1, self.rstd1, eps=self.eps)
        qkv = self.attn.forward_qkv(self.n1, roles, T_c)
        self.q, self.k, self.v = qkv[:, :Cq], qkv[:, Cq:Cq + Ckv], qkv[:, Cq + Ckv:]
        ops.attention_fwd(self.q, self.k, self.v, self.B, self.S, self.H, self.Hkv, self.hd, self.a,
                          self.lse)
        o = self.attn.forward_o(self.a)
        ops.rmsnorm_fwd(o, self.n2, self.rstd2, res=x, hsum=self.h1, eps=self.eps)
        f = self.ffn.forward(self.n2, roles, T_c)
        ops.add(self.h1, f, self.y)
        return self.y

    def backward(self, dy):
        Cq, Ckv = self.attn.Cq, self.attn.Ckv
        dn2 = self.ffn.backward(dy)
        ops.rmsnorm_bwd(self.h1, self.rstd2, dn2, self.dh1, dres=dy)
        da = self.attn.backward_o(self.dh1)
        ops.attention_bwd(self.q, self.k, self.v, self.a, da, self.lse, self.B, self.S, self.H,
                          self.Hkv, self.hd, self.dqkv[:, :Cq], self.dqkv[:, Cq:Cq + Ckv],
                          self.dqkv[:, Cq + Ckv:])
        dn1 = self.attn.backward_qkv(self.dqkv)
        ops.rmsnorm_bwd(self.x, self.rstd1, dn1, self.dx, dres=self.dh1)
        return self.dx
