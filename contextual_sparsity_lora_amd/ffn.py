"""One contextually-sparse SwiGLU FFN block (gate, up, down) with dense LoRA on
all three projections: the forward and backward of the frozen main branch as a
sequence of library calls.

Pages ("SparseLoRA: Accelerating LLM Fine-Tuning with Contextual Sparsity"),
paper-graph summary: §3.4 Algorithm 1 (estimate, score, keep the top
ceil(r D_out), sliced matmul, add dense LoRA); §3.4 "FFN structure": the
selection over the intermediate channels is shared by gate, up and down; §3.4
"Token Sensitivity": output tokens dense, context tokens sparse; §3.2
backward: gradients only through active channels, LoRA gradients dense.

Layout in device memory (allocated once, reused every step):
  W_gu  [2F, D]   gate rows then up rows (nn.Linear layout)
  W_guT [D, 2F]   its transposed copy (backward products)
  W_dn  [D, F]    down weight (nn.Linear layout, forward products)
  Wt_dn [F, D]    its transposed copy: one intermediate channel per row
  A_gu  [2r, D]   LoRA A of gate then up
  B_bd  [2F, 2r]  LoRA B of gate and up, block diagonal (gate in [:F, :r], up in
                  [F:, r:], zeros elsewhere), so one rank-2r term serves the
                  stacked gate|up product
  WA    [D, 2k]   estimator W_A of gate then up (fp32); WB_* [k, F] (fp32)
  gu    [T, 2F]   gate pre-activation | up pre-activation (main + LoRA)
  dgu   [T, 2F]   their gradients
The LoRA terms of the outputs (y += s xl B^T) and of the input gradients
(dx += s gB A) are fused into the main-branch GEMMs; LoRA gradients dA, dB are
separate reductions over tokens.  Everything below is marshalling: each step
is one C-ABI call.
"""
import torch

from . import ops


def keep_count(C: int, num: int, den: int) -> int:
    """Kept channels at sparsity num/den: ceil(C (den - num) / den), in integers."""
    return (C * (den - num) + den - 1) // den


class SparseFFN:
    CRITERIA = ("svd", "oracle", "random")

    def __init__(self, W_gate, W_up, W_down, A_gate, B_gate, A_up, B_up, A_down, B_down,
                 WA_gu, WB_gate, WB_up, scale, sparsity=(7, 10), dense=False, criterion="svd",
                 seed=0, single_stream=False):
        dev = W_gate.device
        self.dtype = W_gate.dtype
        self.F, self.D = W_gate.shape
        self.r = A_gate.shape[0]
        self.k = WB_gate.shape[0] if WB_gate is not None else 0   # factors: None when dense
        self.scale = float(scale)
        # dense=True: the library's dense path at the same shape (every channel
        # kept, no estimator, same LoRA) -- the baseline the sparse block is
        # compared with.
        self.dense = dense
        # criterion ablations (paper-graph summary, Table 7 and Table 10):
        # "svd" the rank-k estimate (the method), "oracle" the same SwiGLU-L2
        # criterion on the exact gate/up outputs of the frozen weights, "random"
        # a uniformly random channel set (library draws, seed + call number)
        assert criterion in self.CRITERIA, criterion
        self.criterion = criterion
        self.seed, self.calls, self.last_seed = int(seed), 0, None
        self.n_sparse = keep_count(self.F, *sparsity)
        self.n = self.F if dense else self.n_sparse
        self.W_gu = torch.cat([W_gate, W_up], 0).contiguous()
        self.W_guT = torch.empty(self.D, 2 * self.F, dtype=self.dtype, device=dev)
        ops.transpose(self.W_gu, self.W_guT)
        self.W_dn = W_down.contiguous()
        self.Wt_dn = torch.empty(self.F, self.D, dtype=self.dtype, device=dev)
        ops.transpose(self.W_dn, self.Wt_dn)
        self.A_gu = torch.cat([A_gate, A_up], 0).contiguous()
        r = self.r
        self.B_bd = torch.zeros(2 * self.F, 2 * r, dtype=self.dtype, device=dev)
        self.B_bd[:self.F, :r] = B_gate
        self.B_bd[self.F:, r:] = B_up
        self.A_down, self.B_down = A_down.contiguous(), B_down.contiguous()
        self.A_guT = torch.empty(self.D, 2 * r, dtype=self.dtype, device=dev)
        self.A_dT = torch.empty(self.F, r, dtype=self.dtype, device=dev)
        # transposed B copies for the backward's gB step (rows padded to a
        # multiple of 8), refreshed with the A transposes in every forward
        c8 = lambda n: (n + 7) // 8 * 8
        self.B_dnT = torch.empty(r, c8(self.D), dtype=self.dtype, device=dev)
        self.B_bdT = torch.empty(2 * r, c8(2 * self.F), dtype=self.dtype, device=dev)
        cont = lambda w: w.contiguous() if w is not None else None
        self.WA = cont(WA_gu)                        # [D, 2k] fp32
        self.WB_gate, self.WB_up = cont(WB_gate), cont(WB_up)
        # a second stream (default priority) for the LoRA reductions that nothing
        # later in the block reads, so they overlap the main-branch products;
        # single_stream=True issues everything on the caller's stream in the
        # same order (each kernel then runs alone: clean per-kernel times)
        self.side = torch.cuda.current_stream(dev) if single_stream else torch.cuda.Stream(device=dev)
        self._ev = [torch.cuda.Event() for _ in range(5)]
        assert dense or criterion != "svd" or self.k > 0, "the estimator factors are required"
        # stream plan: the gate|up product of the output rows on the second
        # stream during the selection, and the LoRA gradient reductions on the
        # second stream next to the backward products
        self.overlap_out_rows = True
        self.side_lora_grads = True
        # bf16 blocks run the SwiGLU passes fused with the LoRA reductions that
        # read the same tensors (h A_down^T forward; dA_down, dB_gate, dB_up
        # backward), so h, dh, g, u, dg and du are each read once
        self.fused_swiglu_lora = (self.dtype == torch.bfloat16 and self.r <= 32 and self.F % 8 == 0)
        # compact_ctx (sparse bf16 forward): the context rows' gate|up product
        # stays compact and one pass forms their merged gate|up rows (kept for
        # the backward), the compact h the down product reads, and their
        # h A_down^T; h itself is then written for the output rows only
        # (keep_h: for the context rows too, as a check of that pass).  Off by
        # default: measured slower than merge + fused SwiGLU + gather so far.
        self.compact_ctx = False
        self.keep_h = False
        self._T = None

    def set_dense(self, dense: bool):
        """Switch between the dense path (every channel kept, no selection) and
        the sparse path at the block's sparsity -- the two phases of a
        progressive schedule (paper-graph summary, "Step Sensitivity and
        Progressive Sparse Fine-Tuning").  Takes effect at the next forward."""
        dense = bool(dense)
        if dense == self.dense:
            return
        assert dense or self.criterion != "svd" or self.k > 0, "the estimator factors are required"
        self.dense = dense
        self.n = self.F if dense else self.n_sparse
        self._T = None

    def lora_params(self):
        """(name, bf16 view the products read, name of the fp32 gradient) per
        LoRA tensor; the views point into the stacked copies."""
        r, F = self.r, self.F
        return [("A_gate", self.A_gu[:r], "dA_gate"), ("A_up", self.A_gu[r:], "dA_up"),
                ("B_gate", self.B_bd[:F, :r], "dB_gate"), ("B_up", self.B_bd[F:, r:], "dB_up"),
                ("A_down", self.A_down, "dA_down"), ("B_down", self.B_down, "dB_down")]

    def _alloc(self, T, T_c, T_o, dev):
        if self._T == (T, T_c, T_o):
            return
        F, D, r, k, dt = self.F, self.D, self.r, self.k, self.dtype
        e = lambda *s, **kw: torch.empty(*s, device=dev, **kw)
        self.ctx_rows = e(T_c, dtype=torch.int32)
        self.out_rows = e(T_o, dtype=torch.int32)
        self.xa = e(T_c, 2 * k, dtype=torch.float32)
        self.scores = e(F, dtype=torch.float32)
        self.idx = e(self.n, dtype=torch.int32)
        self.idx2 = e(2 * self.n, dtype=torch.int32)
        if self.dense:
            torch.arange(self.F, out=self.idx)
            torch.arange(2 * self.F, out=self.idx2)
        self.idx_all = torch.arange(2 * F, dtype=torch.int32, device=dev) if self.criterion == "oracle" else None
        self.gu = e(T, 2 * F, dtype=dt)
        self.h = e(T, F, dtype=dt)
        self.y = e(T, D, dtype=dt)
        self.xl_gu = e(T, 2 * r, dtype=torch.float32)
        self.xl_dn = e(T, r, dtype=torch.float32)
        self.dh = e(T, F, dtype=dt)
        self.dgu = e(T, 2 * F, dtype=dt)
        self.dx = e(T, D, dtype=dt)
        f32 = torch.float32
        self.dA_gu = e(2 * r, D, dtype=f32)
        self.dA_gate, self.dA_up = self.dA_gu[:r], self.dA_gu[r:]
        self.dB_gate, self.dB_up = e(F, r, dtype=f32), e(F, r, dtype=f32)
        self.dA_down, self.dB_down = e(r, F, dtype=f32), e(D, r, dtype=f32)
        self.gB_gu = e(T, 2 * r, dtype=f32)
        self.gB_dn = e(T, r, dtype=f32)
        # K-gathered weight slices of the selection (bf16 only): down's input
        # channels for the forward, gate|up's rows for the backward
        c8 = lambda n: (n + 7) // 8 * 8
        self.ws_dn = e(D, c8(self.n), dtype=dt) if dt == torch.bfloat16 else None
        self.ws_gu = e(D, c8(2 * self.n), dtype=dt) if dt == torch.bfloat16 else None
        # compact context-row operands: gate|up product [T_c, 2n], h [T_c, n]
        self.yc_gu = e(T_c, c8(2 * self.n), dtype=dt) if dt == torch.bfloat16 else None
        self.hc = e(T_c, c8(self.n), dtype=dt) if dt == torch.bfloat16 else None
        self._T = (T, T_c, T_o)

    def forward(self, x, roles, T_c):
        T = x.shape[0]
        F, r = self.F, self.r
        self._alloc(T, T_c, T - T_c, x.device)
        self.x = x
        main = torch.cuda.current_stream(x.device)
        ops.token_split(roles, self.ctx_rows, self.out_rows)
        # side stream: the LoRA down-projection of the block input, then (with
        # the estimator) the gate|up product of the output rows (dense over
        # every channel, so it does not wait for the selection) -- both overlap
        # the estimator, scoring and selection on the main stream, whose small
        # launches leave most compute units idle
        overlap = (self.overlap_out_rows and not self.dense
                   and self.criterion != "oracle")   # "oracle" scores in gu first
        self._ev[0].record(main)
        if not self.dense and self.criterion == "svd":
            # the estimator's first product goes out first, so the main stream
            # has work while the host issues the side stream's calls
            ops.svd_estimate(x, self.ctx_rows, self.WA, self.xa)
        self.side.wait_event(self._ev[0])
        lora = (self.xl_gu, self.B_bd, 2 * r, self.scale)
        with torch.cuda.stream(self.side):
            ops.lora_fwd_bwd(ops.LORA_XL, x, self.A_gu, None, self.scale, self.xl_gu)
            self._ev[1].record(self.side)
            if overlap:
                ops.sparse_linear_fwd("out", x, self.W_gu, None, self.ctx_rows, self.out_rows, self.idx2,
                                      self.gu, lora=lora, flags=ops.ONLY_OUT_ROWS)
            # the backward's transposed LoRA factors (after the product, which
            # they would otherwise delay)
            ops.transpose(self.A_down, self.A_dT)
            ops.transpose(self.A_gu, self.A_guT)
            ops.transpose(self.B_down, self.B_dnT[:, :self.D])
            ops.transpose(self.B_bd, self.B_bdT[:, :2 * F])
        if not self.dense:
            self._select(x, estimated=self.criterion == "svd")
        # the weight slices need only the selection: built on the second stream
        # while the main stream runs the context rows' gate|up product
        self._slices = overlap and self.ws_dn is not None
        if self._slices:
            self._ev[4].record(main)
            self.side.wait_event(self._ev[4])
        with torch.cuda.stream(self.side):
            if self._slices:
                ops.weight_slice(self.Wt_dn, self.idx, self.ws_dn)
                ops.weight_slice(self.W_gu, self.idx2, self.ws_gu)
            self._ev[3].record(self.side)
        main.wait_event(self._ev[1])
        g, u = self.gu[:, :F], self.gu[:, F:]
        self._compact = compact = overlap and self.compact_ctx and self._slices
        if compact:
            # the context rows' gate|up product over the selected channels,
            # stored compactly (LoRA term of those channels fused)
            ops.sparse_linear_fwd("out", x, self.W_gu, None, self.ctx_rows, self.out_rows, self.idx2,
                                  self.yc_gu[:, :2 * self.n], lora=lora,
                                  flags=ops.ONLY_CTX_ROWS | ops.CTX_COMPACT)
            ops.swiglu_fwd_ctx(self.yc_gu, self.ctx_rows, self.idx, lora, self.gu, self.hc, self.A_down,
                               self.xl_dn, h_rows=self.h if self.keep_h else None)
            main.wait_event(self._ev[3])
            ops.swiglu_fwd_lora(g, u, self.h, self.A_down, self.xl_dn, rows=self.out_rows)
        else:
            # the gate|up main branch of the context rows (gathered channels;
            # every row when dense or not overlapped) with the LoRA term fused
            # into the same accumulators
            ops.sparse_linear_fwd("out", x, self.W_gu, None, self.ctx_rows, self.out_rows, self.idx2, self.gu,
                                  lora=lora, flags=ops.ONLY_CTX_ROWS if overlap else 0)
            main.wait_event(self._ev[3])
            if self.fused_swiglu_lora:
                ops.swiglu_fwd_lora(g, u, self.h, self.A_down, self.xl_dn)
            else:
                ops.swiglu_fwd(g, u, self.h)
                ops.lora_fwd_bwd(ops.LORA_XL, self.h, self.A_down, None, self.scale, self.xl_dn)
        # down main branch: input channels = the same selection; LoRA fused
        ops.sparse_linear_fwd("in", self.h, self.W_dn, self.Wt_dn, self.ctx_rows, self.out_rows,
                              self.idx, self.y, lora=(self.xl_dn, self.B_down, r, self.scale),
                              w_slice=self.ws_dn if self._slices else None,
                              x_slice=self.hc if compact else None)
        return self.y

    def _select(self, x, estimated=False):
        """The shared gate/up/down selection idx (and its stacked form idx2);
        estimated: the estimator's product xa is already computed."""
        F = self.F
        if self.criterion == "svd":
            # estimator on context tokens, SwiGLU-L2 criterion, top-n
            if not estimated:
                ops.svd_estimate(x, self.ctx_rows, self.WA, self.xa)
            ops.score_select("swiglu", self.xa, self.WB_gate, self.WB_up, self.n, self.idx,
                             scores=self.scores, off0=0, off1=self.k)
        elif self.criterion == "oracle":
            # exact gate|up outputs of the frozen weights (no LoRA) in gu, which
            # the product below then overwrites
            ops.sparse_linear_fwd("out", x, self.W_gu, None, self.ctx_rows, self.out_rows, self.idx_all,
                                  self.gu)
            ops.dense_scores("swiglu", self.gu[:, :F], self.gu[:, F:], self.ctx_rows, self.scores)
            ops.select_top(self.scores, self.n, self.idx)
        else:
            self.last_seed = self.seed + self.calls
            ops.random_scores(self.last_seed, self.scores)
            ops.select_top(self.scores, self.n, self.idx)
        self.calls += 1
        ops.stack_index(self.idx, F, 2, self.idx2)

    def backward(self, dy):
        F, D, r, s = self.F, self.D, self.r, self.scale
        main = torch.cuda.current_stream(dy.device)
        # down: LoRA gB (main stream: the dh product reads it); dA and dB on the
        # side stream, overlapping the dh product
        ops.lora_fwd_bwd(ops.LORA_GB | ops.LORA_BT, None, None, self.B_dnT, s, None, dy=dy, gB=self.gB_dn,
                         D_in=F, D_out=D, r=r)
        self._ev[0].record(main)
        ops.sparse_linear_bwd("in", dy, None, self.Wt_dn, self.ctx_rows, self.out_rows, self.idx,
                              self.dh, lora=(self.gB_dn, self.A_dT, r, s))
        # (issued after the main-stream product: the host's time on these calls
        # overlaps that product)
        self.side.wait_event(self._ev[0])
        fused = self.fused_swiglu_lora
        with torch.cuda.stream(self.side if self.side_lora_grads else main):
            if fused:   # dA_down comes with the SwiGLU backward below
                ops.lora_fwd_bwd(ops.LORA_DB, None, None, None, s, self.xl_dn, dy=dy, dB=self.dB_down,
                                 D_in=F, r=r)
            else:
                ops.lora_fwd_bwd(ops.LORA_DA | ops.LORA_DB, self.h, None, None, s, self.xl_dn, dy=dy,
                                 dA=self.dA_down, dB=self.dB_down, gB=self.gB_dn, D_in=F, r=r)
        g, u = self.gu[:, :F], self.gu[:, F:]
        dg, du = self.dgu[:, :F], self.dgu[:, F:]
        if fused:
            ops.swiglu_bwd_lora(self.dh, g, u, dg, du, self.gB_dn, self.xl_gu[:, :r], self.xl_gu[:, r:], s,
                                self.dA_down, self.dB_gate, self.dB_up)
        else:
            ops.swiglu_bwd(self.dh, g, u, dg, du)
        # gate|up: gB for both through the block-diagonal B (main stream); dA
        # and the per-projection dB on the side stream, overlapping the dx product
        ops.lora_fwd_bwd(ops.LORA_GB | ops.LORA_BT, None, None, self.B_bdT, s, None, dy=self.dgu,
                         gB=self.gB_gu, D_in=D, D_out=2 * F, r=2 * r)
        self._ev[1].record(main)
        ops.sparse_linear_bwd("out", self.dgu, self.W_gu, self.W_guT, self.ctx_rows, self.out_rows,
                              self.idx2, self.dx, lora=(self.gB_gu, self.A_guT, 2 * r, s),
                              w_slice=self.ws_gu if self._slices else None)
        self.side.wait_event(self._ev[1])
        with torch.cuda.stream(self.side if self.side_lora_grads else main):
            ops.lora_fwd_bwd(ops.LORA_DA, self.x, None, None, s, None, dy=self.dgu, dA=self.dA_gu,
                             gB=self.gB_gu, D_in=D, r=2 * r)
            if not fused:
                ops.lora_fwd_bwd(ops.LORA_DB, None, None, None, s, self.xl_gu[:, :r], dy=dg,
                                 dB=self.dB_gate, r=r, D_in=D)
                ops.lora_fwd_bwd(ops.LORA_DB, None, None, None, s, self.xl_gu[:, r:], dy=du,
                                 dB=self.dB_up, r=r, D_in=D)
            self._ev[2].record(self.side)
        # the block's gradients are complete when both streams are
        main.wait_event(self._ev[2])
        return self.dx
