"""Seeded synthetic workloads for the contextually-sparse LoRA linear path.

This package holds the five workload configurations (sizes, dtypes, sparsity
ratios as exact rationals) and the seeded generators of every input tensor.
It is shared by the tests, the benchmark and the CPU oracle's callers, and it
contains none of the method's per-batch arithmetic: no estimator, no scoring,
no selection, no masked or sliced matmul, no LoRA.  The estimator factors are
generated here as an input (the pages' method computes them offline from the
frozen weight and loads them with the weights), see ``gen.svd_factor_pair``.
"""
from .configs import CONFIGS, Config, get_config  # noqa: F401
from .gen import (  # noqa: F401
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    make_ffn_inputs,
    make_attn_inputs,
    roles_for,
    svd_factor_pair,
)
