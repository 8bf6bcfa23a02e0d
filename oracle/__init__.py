"""CPU oracle of the contextually-sparse LoRA linear path.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by the smoke check and by the
benchmark's CPU-baseline leg, never by the library or its binding.  It shares
no code with the GPU path.

Two parts:
  * ``csa`` -- the fp32 canonical score arithmetic (C, ``csa.c``): estimator
    stage 1, estimator stage 2 fused with the FFN / VO / QK criteria, keys and
    the top-n selection by its definition.  The selection is an integer result
    decided by floating point, so it is computed in binary32 with a stated
    operation order that the GPU reproduces.
  * ``reference`` -- everything else in fp64 (numpy): token-role lists, the
    kept-channel count, masked-dense main-branch forward and backward, the
    dense LoRA branch and its gradients, SwiGLU and the FFN block.

Pins against what the pages and mathematics fix live in ``tests/test_oracle_*``.
Parity status per function is listed in each function's docstring.
"""
from . import csa, reference  # noqa: F401
