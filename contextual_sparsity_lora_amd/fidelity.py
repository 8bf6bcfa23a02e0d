"""Gradient fidelity of training sparsity: the cosine between the LoRA
gradients a sparse block computes and those the dense block computes on the
same inputs, per adapter tensor.

Pages ("SparseLoRA: Accelerating LLM Fine-Tuning with Contextual Sparsity"),
paper-graph summary, "Follow-Up Research This Work Enables": gradient cosine
similarity between the dense and the sparse update of the LoRA adapters, per
sparsity configuration, as a measure of how much the sparsity changes
training.  The dot products run in the library (fp64, fixed order); only the
final cos = a.b / sqrt(a.a b.b) of three numbers is formed here.
"""
import math
import re

import torch

from . import ops

_GRAD = re.compile(r"d[AB]_(gate|up|down|q|k|v|o)")


def grad_cosine(a: torch.Tensor, b: torch.Tensor) -> float:
    """cos(a, b) of two fp32 device tensors of one shape (nan if either is 0)."""
    out = torch.empty(3, dtype=torch.float64, device=a.device)
    ops.dot_stats(a.contiguous().view(-1), b.contiguous().view(-1), out)
    ab, aa, bb = out.tolist()
    return ab / math.sqrt(aa * bb) if aa > 0.0 and bb > 0.0 else float("nan")


def lora_grads(block) -> dict:
    """The per-projection LoRA gradient tensors of a block (SparseFFN or
    SparseAttnProj) after its backward: name -> fp32 device tensor."""
    return {k: v for k, v in vars(block).items() if _GRAD.fullmatch(k) and torch.is_tensor(v)}


def block_fidelity(sparse, dense) -> dict:
    """name -> cosine between the sparse and the dense block's LoRA gradient."""
    gs, gd = lora_grads(sparse), lora_grads(dense)
    return {k: grad_cosine(gs[k], gd[k]) for k in sorted(gs) if k in gd}


def layer_fidelity(sparse_layer, dense_layer) -> dict:
    """Per decoder layer: "attn.dA_q", ..., "ffn.dB_down" -> cosine."""
    out = {}
    for part in ("attn", "ffn"):
        for k, c in block_fidelity(getattr(sparse_layer, part), getattr(dense_layer, part)).items():
            out[f"{part}.{k}"] = c
    return out


def stack_fidelity(sparse_stack, dense_stack) -> list:
    """One layer_fidelity dict per layer of two stacks run on the same inputs."""
    return [layer_fidelity(s, d) for s, d in zip(sparse_stack.layers, dense_stack.layers)]
