"""Whole LoRA fine-tuning steps around a sparse block, with the progressive
schedule: the first ceil(p N) of N steps run dense (every channel, no
estimator), the rest sparse.

Pages ("SparseLoRA: Accelerating LLM Fine-Tuning with Contextual Sparsity"),
paper-graph summary: "Step Sensitivity and Progressive Sparse Fine-Tuning"
(dense for the first p <= 10 % of steps; the overall speedup is bounded by
1 / (p + (1 - p) / s)); "Interaction with the learning rate schedule" (cosine
schedule with a 4 % warm-up); "Putting It All Together" (next-token
cross-entropy taken over the output-token positions alone; the adapters' A
and B are the only trained tensors, the base weights stay frozen).

One step: block forward -> logits of the output rows through a frozen LM head
W_head [V, D] -> softmax cross-entropy against the labels of those rows (mean
over output tokens) -> its gradient back through the head -> block backward
-> AdamW on the LoRA tensors (fp32 masters, the bf16 copies the products
read are rewritten by the same kernel).  Every step is a library call.
"""
import math

import torch

from . import ops


def lr_at(step, total, peak, warmup_ratio=0.04):
    """Learning rate of 0-based step: linear warm-up over ceil(warmup_ratio
    total) steps from 0, then cosine decay to 0 at step `total`."""
    w = math.ceil(warmup_ratio * total)
    if step < w:
        return peak * step / w
    prog = (step - w) / max(1, total - w)
    return peak * 0.5 * (1.0 + math.cos(math.pi * prog))


class LoRATrainer:
    def __init__(self, block, W_head, total_steps, dense_frac=0.1, lr=3e-4, warmup_ratio=0.04,
                 betas=(0.9, 0.999), eps=1e-8, weight_decay=0.0):
        self.block = block
        dev = W_head.device
        self.W_head = W_head.contiguous()                       # [V, D], frozen
        self.V, self.D = self.W_head.shape
        # rows of V elements are padded to 16 bytes (the products' row alignment)
        q = 8 if W_head.dtype == torch.bfloat16 else 4
        self.Vp = (self.V + q - 1) // q * q
        self.W_headT = torch.empty(self.D, self.Vp, dtype=W_head.dtype, device=dev)[:, :self.V]
        ops.transpose(self.W_head, self.W_headT)
        self.total = int(total_steps)
        self.n_dense = math.ceil(dense_frac * self.total)
        self.lr, self.warmup_ratio, self.betas, self.eps, self.wd = lr, warmup_ratio, betas, eps, weight_decay
        self.params = []
        for name, view, gname in block.lora_params():
            p = view.float().contiguous().clone()
            self.params.append((name, p, torch.zeros_like(p), torch.zeros_like(p), view, gname))
        self.idx_V = torch.arange(self.V, dtype=torch.int32, device=dev)
        self.idx_D = torch.arange(self.D, dtype=torch.int32, device=dev)
        self.loss = torch.zeros(1, dtype=torch.float64, device=dev)
        self.t = 0
        self._T = None

    def _alloc(self, T, dt, dev):
        if self._T == T:
            return
        self.logits = torch.empty(T, self.Vp, dtype=dt, device=dev)[:, :self.V]
        self.dlogits = torch.empty(T, self.Vp, dtype=dt, device=dev)[:, :self.V]
        self.dy = torch.zeros(T, self.D, dtype=dt, device=dev)   # context rows stay 0
        self._T = T

    def step(self, x, labels, roles, T_c):
        """One training step on batch x [T, D] with labels [T] (read on output
        rows); returns the device fp64 mean loss of this step (before the update)."""
        blk = self.block
        self._alloc(x.shape[0], x.dtype, x.device)
        blk.set_dense(self.t < self.n_dense)
        y = blk.forward(x, roles, T_c)
        ctx, out = blk.ctx_rows, blk.out_rows
        ops.sparse_linear_fwd("out", y, self.W_head, None, ctx, out, self.idx_V, self.logits,
                              flags=ops.ONLY_OUT_ROWS)
        ops.token_ce(self.logits, out, labels, self.dlogits, self.loss)
        # dy = dlogits W_head on the output rows: the NT product over W_head^T
        ops.sparse_linear_fwd("out", self.dlogits, self.W_headT, None, ctx, out, self.idx_D, self.dy,
                              flags=ops.ONLY_OUT_ROWS)
        blk.backward(self.dy)
        lr = lr_at(self.t, self.total, self.lr, self.warmup_ratio)
        groups = [(p, getattr(blk, gname), m, v, view) for _, p, m, v, view, gname in self.params]
        ops.adamw_step(groups, lr, self.t + 1, self.betas[0], self.betas[1], self.eps, self.wd)
        self.t += 1
        return self.loss

    def masters(self):
        return {name: p for name, p, _, _, _, _ in self.params}
