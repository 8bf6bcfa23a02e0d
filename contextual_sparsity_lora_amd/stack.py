"""A stack of sparse decoder layers (every linear of every layer contextually
sparse, dense LoRA), one training step's forward and backward.

Pages ("SparseLoRA: Accelerating LLM Fine-Tuning with Contextual Sparsity"),
paper-graph summary §3.4 "Layer Sensitivity": deeper layers tolerate more
sparsity, so the sparsity is set per layer (the first layers stay dense);
each layer makes its own selection from its own input.  A layer whose
sparsity is 0 keeps every channel and runs the library's dense path (no
estimator: its selection would be every channel).
"""
from .layer import SparseDecoderLayer


class SparseStack:
    def __init__(self, layers):
        self.layers = list(layers)

    @classmethod
    def build(cls, cfg, layer_arrays, sparsities):
        """layer_arrays: per layer (d, f32) as taken by SparseDecoderLayer.from_arrays;
        sparsities: per layer (num, den), applied to the FFN, QK and VO groups."""
        layers = []
        for (d, f32), sp in zip(layer_arrays, sparsities):
            layers.append(SparseDecoderLayer.from_arrays(d, f32, cfg, sp, sp, sp, dense=(sp[0] == 0)))
        return cls(layers)

    def forward(self, x, roles, T_c):
        h = x
        for L in self.layers:
            h = L.forward(h, roles, T_c)
        return h

    def backward(self, dy):
        g = dy
        for L in reversed(self.layers):
            g = L.backward(g)
        return g
