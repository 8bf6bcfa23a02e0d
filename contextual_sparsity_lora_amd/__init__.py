"""MI355X (gfx950) implementation of SparseLoRA's contextually-sparse frozen
main-branch linear layer (forward and backward), with a C ABI
(include/sparselora.h, libsparselora.so) and this thin Python binding.

Modules:
  build   -- hipcc build of libsparselora.so (in-tree)
  _lib    -- ctypes loader; raises if the library is not built
  ops     -- one Python function per C-ABI entry point (marshalling only)
  ffn     -- the sparse SwiGLU FFN block (fwd + bwd) as a sequence of calls
"""
__all__ = ["ops", "ffn", "build"]
