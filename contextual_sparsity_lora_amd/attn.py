"""The contextually-sparse q/k/v/o projections of one attention layer (GQA
allowed) with dense LoRA on all four: forward and backward of the frozen main
branch as a sequence of library calls.

Pages ("SparseLoRA: Accelerating LLM Fine-Tuning with Contextual Sparsity"),
paper-graph summary: §3.4 "QK projection sparsity" (channels scored by the
product of the query and key norms over context tokens; q and k keep the same
channels), "VO projection sparsity" (channels scored by the norm of the
values; v keeps them as outputs and o as inputs), Algorithm 1 (estimate,
score, keep the top ceil(r C), sliced products, dense LoRA), "Token
Sensitivity" (output tokens dense).  Under grouped-query attention the
selection is made in key/value channel space and each kept channel carries its
group's query heads (the query-norm term sums the group's heads).

Layout in device memory (allocated once, reused every step):
  W_qkv  [Cq + 2 Ckv, D]  q rows, then k rows, then v rows (nn.Linear layout)
  W_qkvT [D, Cq + 2 Ckv]  its transposed copy (backward products)
  W_o    [D, Cq], Wt_o [Cq, D]
  A_qkv  [3r, D]; B_bd [Cq + 2 Ckv, 3r] block diagonal (q, k, v blocks), so one
         rank-3r term serves the stacked product
  WA     [D, 3k] estimator W_A of q, k, v side by side (fp32); WB_* [k, C*]
  qkv    [T, Cq + 2 Ckv]  q | k | v (main + LoRA); o [T, D]
Everything below is marshalling: each step is one C-ABI call.
"""
import torch

from . import ops
from .ffn import keep_count


class SparseAttnProj:
    def __init__(self, W_q, W_k, W_v, W_o, A_q, B_q, A_k, B_k, A_v, B_v, A_o, B_o, WA_qkv,
                 WB_q, WB_k, WB_v, scale, n_kv_heads, head_dim, qk_sparsity=(1, 2),
                 vo_sparsity=(1, 2), dense=False, criterion="svd", seed=0):
        dev = W_q.device
        self.dtype = W_q.dtype
        self.Cq, self.D = W_q.shape
        self.Ckv = W_k.shape[0]
        self.d = head_dim
        self.n_rep = self.Cq // self.Ckv
        assert self.Cq == self.n_rep * self.Ckv and self.Ckv == n_kv_heads * head_dim
        self.r = A_q.shape[0]
        self.k = WB_q.shape[0] if WB_q is not None else 0   # estimator factors: None when dense
        self.scale = float(scale)
        self.dense = dense
        # criterion ablations (paper-graph summary, Tables 7 and 10): "svd" the
        # rank-k estimate (the method); "oracle" the QK and VO criteria on the
        # exact q, k, v outputs of the frozen weights; "random" uniformly random
        # channel sets (library draws, seed + call number); "head" the QK
        # selection made per key/value head (the estimate's channel scores
        # summed per head, whole heads kept; VO stays per channel)
        assert criterion in ("svd", "oracle", "random", "head"), criterion
        self.criterion = criterion
        self.seed, self.calls, self.last_seed = int(seed), 0, None
        self.n_kv_heads = n_kv_heads
        self.n_qk = self.Ckv if dense else keep_count(self.Ckv, *qk_sparsity)
        if criterion == "head" and not dense:
            self.heads_keep = keep_count(n_kv_heads, *qk_sparsity)
            self.n_qk = self.heads_keep * head_dim
        self.n_vo = self.Ckv if dense else keep_count(self.Ckv, *vo_sparsity)
        Cq, Ckv, r = self.Cq, self.Ckv, self.r
        self.Cs = Cq + 2 * Ckv
        self.W_qkv = torch.cat([W_q, W_k, W_v], 0).contiguous()
        self.W_qkvT = torch.empty(self.D, self.Cs, dtype=self.dtype, device=dev)
        ops.transpose(self.W_qkv, self.W_qkvT)
        self.W_o = W_o.contiguous()
        self.Wt_o = torch.empty(Cq, self.D, dtype=self.dtype, device=dev)
        ops.transpose(self.W_o, self.Wt_o)
        self.A_qkv = torch.cat([A_q, A_k, A_v], 0).contiguous()
        self.B_bd = torch.zeros(self.Cs, 3 * r, dtype=self.dtype, device=dev)
        self.B_bd[:Cq, :r] = B_q
        self.B_bd[Cq:Cq + Ckv, r:2 * r] = B_k
        self.B_bd[Cq + Ckv:, 2 * r:] = B_v
        self.A_o, self.B_o = A_o.contiguous(), B_o.contiguous()
        self.A_qkvT = torch.empty(self.D, 3 * r, dtype=self.dtype, device=dev)
        self.A_oT = torch.empty(Cq, r, dtype=self.dtype, device=dev)
        # transposed B copies for the backward's gB steps (rows padded to a
        # multiple of 8), refreshed with the A transposes in every forward
        c8 = lambda n: (n + 7) // 8 * 8
        self.B_bdT = torch.empty(3 * r, c8(self.Cs), dtype=self.dtype, device=dev)
        self.B_oT = torch.empty(r, c8(self.D), dtype=self.dtype, device=dev)
        cont = lambda w: w.contiguous() if w is not None else None
        self.WA = cont(WA_qkv)                         # [D, 3k] fp32
        self.WB_q, self.WB_k, self.WB_v = (cont(w) for w in (WB_q, WB_k, WB_v))
        assert dense or criterion in ("oracle", "random") or self.k > 0, "the estimator factors are required"
        # a second stream (default priority): the q|k|v product of the output
        # rows and the LoRA down-projection overlap the selection; the LoRA
        # reductions nothing later reads overlap the backward products
        self.side = torch.cuda.Stream(device=dev)
        self._ev = [torch.cuda.Event() for _ in range(7)]
        self._T = None

    def _alloc(self, T, T_c, T_o, dev):
        if self._T == (T, T_c, T_o):
            return
        Cq, Ckv, r, k, dt, D = self.Cq, self.Ckv, self.r, self.k, self.dtype, self.D
        e = lambda *s, **kw: torch.empty(*s, device=dev, **kw)
        i32, f32 = torch.int32, torch.float32
        self.ctx_rows, self.out_rows = e(T_c, dtype=i32), e(T_o, dtype=i32)
        self.xa = e(T_c, 3 * k, dtype=f32)
        self.scores = e(Ckv, dtype=f32)
        self.scores_vo = e(Ckv, dtype=f32)
        self.idx_all = torch.arange(self.Cs, dtype=i32, device=dev) if self.criterion == "oracle" else None
        self.idx_qk, self.idx_vo = e(self.n_qk, dtype=i32), e(self.n_vo, dtype=i32)
        self.idx_q = e(self.n_qk * self.n_rep, dtype=i32)
        self.idx_o = e(self.n_vo * self.n_rep, dtype=i32)
        self.idx_qkv = e(self.n_qk * self.n_rep + self.n_qk + self.n_vo, dtype=i32)
        if self.dense:
            torch.arange(self.Cs, out=self.idx_qkv)
            torch.arange(Cq, out=self.idx_o)
        self.qkv = e(T, self.Cs, dtype=dt)
        self.o = e(T, D, dtype=dt)
        self.xl_qkv = e(T, 3 * r, dtype=f32)
        self.xl_o = e(T, r, dtype=f32)
        self.dx = e(T, D, dtype=dt)
        self.dx_o = e(T, Cq, dtype=dt)
        self.dA_qkv = e(3 * r, D, dtype=f32)
        self.dA_q, self.dA_k, self.dA_v = self.dA_qkv[:r], self.dA_qkv[r:2 * r], self.dA_qkv[2 * r:]
        self.dB_q, self.dB_k, self.dB_v = e(Cq, r, dtype=f32), e(Ckv, r, dtype=f32), e(Ckv, r, dtype=f32)
        self.dA_o, self.dB_o = e(r, Cq, dtype=f32), e(D, r, dtype=f32)
        self.gB_qkv, self.gB_o = e(T, 3 * r, dtype=f32), e(T, r, dtype=f32)
        # K-gathered weight slices of the selection (bf16 only): o's input
        # channels for the forward, q|k|v's rows for the backward's dx product
        c8 = lambda n: (n + 7) // 8 * 8
        bf = dt == torch.bfloat16
        self.ws_o = e(D, c8(self.n_vo * self.n_rep), dtype=dt) if bf else None
        self.ws_qkv = e(D, c8(self.idx_qkv.numel()), dtype=dt) if bf else None
        self._slices = False
        self._T = (T, T_c, T_o)

    def select(self, estimated=False):
        """QK and VO selections from the estimator on the context tokens, their
        GQA expansions and the stacked q|k|v channel list (estimated: xa is
        already computed)."""
        k, Ckv, Cq = self.k, self.Ckv, self.Cq
        crit = self.criterion
        if crit in ("svd", "head"):
            if not estimated:
                ops.svd_estimate(self.x, self.ctx_rows, self.WA, self.xa)
            ops.score_select("qk", self.xa, self.WB_q, self.WB_k, 0 if crit == "head" else self.n_qk,
                             self.idx_qk, scores=self.scores, off0=0, off1=k, C=Ckv, n_rep=self.n_rep,
                             head_dim=self.d)
            if crit == "head":
                ops.select_heads(self.scores, self.n_kv_heads, self.d, self.heads_keep, self.idx_qk)
            ops.score_select("l2", self.xa, self.WB_v, None, self.n_vo, self.idx_vo,
                             scores=self.scores_vo, off0=2 * k)
        elif crit == "oracle":
            # exact q|k|v outputs of the frozen weights (no LoRA) in qkv, which
            # the product then overwrites
            ops.sparse_linear_fwd("out", self.x, self.W_qkv, None, self.ctx_rows, self.out_rows,
                                  self.idx_all, self.qkv)
            q, kk, v = self.qkv[:, :Cq], self.qkv[:, Cq:Cq + Ckv], self.qkv[:, Cq + Ckv:]
            ops.dense_scores("qk", q, kk, self.ctx_rows, self.scores, C=Ckv, n_rep=self.n_rep,
                             head_dim=self.d)
            ops.select_top(self.scores, self.n_qk, self.idx_qk)
            ops.dense_scores("l2", v, None, self.ctx_rows, self.scores_vo)
            ops.select_top(self.scores_vo, self.n_vo, self.idx_vo)
        else:
            # two independent draws: QK from seed', VO from seed' + 2^32
            self.last_seed = self.seed + self.calls
            ops.random_scores(self.last_seed, self.scores)
            ops.select_top(self.scores, self.n_qk, self.idx_qk)
            ops.random_scores(self.last_seed + (1 << 32), self.scores_vo)
            ops.select_top(self.scores_vo, self.n_vo, self.idx_vo)
        self.calls += 1
        ops.qkv_index(self.idx_qk, self.idx_vo, self.n_kv_heads, self.n_rep, self.d, self.idx_q, self.idx_o,
                      self.idx_qkv)

    def forward_qkv(self, x, roles, T_c):
        """Token split, selection and the stacked q|k|v product (main + LoRA)."""
        T = x.shape[0]
        r = self.r
        self._alloc(T, T_c, T - T_c, x.device)
        self.x = x
        main, ev = torch.cuda.current_stream(x.device), self._ev
        ops.token_split(roles, self.ctx_rows, self.out_rows)
        # side stream: x A^T, then (unless the selection itself writes qkv) the
        # q|k|v product of the output rows, which does not read the selection
        overlap = not self.dense and self.criterion != "oracle"
        lora = (self.xl_qkv, self.B_bd, 3 * r, self.scale)
        ev[0].record(main)
        if not self.dense and self.criterion in ("svd", "head"):
            # the estimator's first product goes first, so the GPU has work
            # while the host issues the side-stream calls
            ops.svd_estimate(self.x, self.ctx_rows, self.WA, self.xa)
        self.side.wait_event(ev[0])
        with torch.cuda.stream(self.side):
            ops.lora_fwd_bwd(ops.LORA_XL, x, self.A_qkv, None, self.scale, self.xl_qkv)
            ev[1].record(self.side)
            if overlap:
                ops.sparse_linear_fwd("out", x, self.W_qkv, None, self.ctx_rows, self.out_rows, self.idx_qkv,
                                      self.qkv, lora=lora, flags=ops.ONLY_OUT_ROWS)
            # the backward's transposed LoRA factors (after the product, which
            # they would otherwise delay)
            ops.transpose(self.A_qkv, self.A_qkvT)
            ops.transpose(self.A_o, self.A_oT)
            ops.transpose(self.B_bd, self.B_bdT[:, :self.Cs])
            ops.transpose(self.B_o, self.B_oT[:, :self.D])
        if not self.dense:
            self.select(estimated=True)
        # the weight slices need only the selection: built on the second stream
        # while the main stream runs the context rows' q|k|v product
        self._slices = overlap and self.ws_o is not None
        if self._slices:
            ev[6].record(main)
            self.side.wait_event(ev[6])
        with torch.cuda.stream(self.side):
            if self._slices:
                ops.weight_slice(self.Wt_o, self.idx_o, self.ws_o)
                ops.weight_slice(self.W_qkv, self.idx_qkv, self.ws_qkv)
            ev[2].record(self.side)
        main.wait_event(ev[1])
        ops.sparse_linear_fwd("out", x, self.W_qkv, None, self.ctx_rows, self.out_rows, self.idx_qkv,
                              self.qkv, lora=lora, flags=ops.ONLY_CTX_ROWS if overlap else 0)
        main.wait_event(ev[2])
        return self.qkv

    def forward_o(self, x_o):
        """The o projection (input side: kept channels only on context rows)."""
        r = self.r
        self.x_o = x_o
        ops.lora_fwd_bwd(ops.LORA_XL, x_o, self.A_o, None, self.scale, self.xl_o)
        ops.sparse_linear_fwd("in", x_o, self.W_o, self.Wt_o, self.ctx_rows, self.out_rows, self.idx_o,
                              self.o, lora=(self.xl_o, self.B_o, r, self.scale),
                              w_slice=self.ws_o if self._slices else None)
        return self.o

    def forward(self, x, x_o, roles, T_c):
        self.forward_qkv(x, roles, T_c)
        self.forward_o(x_o)
        return self.qkv, self.o

    def backward_o(self, dy_o):
        """o: LoRA gB, dA, dB; then dx_o (input side: kept channels only) with
        the LoRA term fused."""
        r, s = self.r, self.scale
        main, ev = torch.cuda.current_stream(dy_o.device), self._ev
        # gB on the main stream (the dx_o product reads it); dA, dB on the side stream
        ops.lora_fwd_bwd(ops.LORA_GB | ops.LORA_BT, None, None, self.B_oT, s, None, dy=dy_o, gB=self.gB_o,
                         D_in=self.Cq, D_out=self.D, r=r)
        ev[3].record(main)
        ops.sparse_linear_bwd("in", dy_o, None, self.Wt_o, self.ctx_rows, self.out_rows, self.idx_o,
                              self.dx_o, lora=(self.gB_o, self.A_oT, r, s))
        # (issued after the main-stream product, so the host's time on these
        # calls overlaps that product instead of delaying it)
        self.side.wait_event(ev[3])
        with torch.cuda.stream(self.side):
            ops.lora_fwd_bwd(ops.LORA_DA | ops.LORA_DB, self.x_o, None, None, s, self.xl_o, dy=dy_o,
                             dA=self.dA_o, dB=self.dB_o, gB=self.gB_o, D_in=self.Cq, r=r)
        return self.dx_o

    def backward_qkv(self, dqkv):
        """dqkv [T, Cq + 2 Ckv]: gradients of q | k | v.  gB and dA through the
        block-diagonal B, dB per projection, then dx with the LoRA term fused."""
        Cq, Ckv, r, s = self.Cq, self.Ckv, self.r, self.scale
        main, ev = torch.cuda.current_stream(dqkv.device), self._ev
        # gB through the block-diagonal B on the main stream; dA and the
        # per-projection dB on the side stream, next to the dx product
        ops.lora_fwd_bwd(ops.LORA_GB | ops.LORA_BT, None, None, self.B_bdT, s, None, dy=dqkv, gB=self.gB_qkv,
                         D_in=self.D, D_out=self.Cs, r=3 * r)
        ev[4].record(main)
        ops.sparse_linear_bwd("out", dqkv, self.W_qkv, self.W_qkvT, self.ctx_rows, self.out_rows,
                              self.idx_qkv, self.dx, lora=(self.gB_qkv, self.A_qkvT, 3 * r, s),
                              w_slice=self.ws_qkv if self._slices else None)
        self.side.wait_event(ev[4])
        with torch.cuda.stream(self.side):
            ops.lora_fwd_bwd(ops.LORA_DA, self.x, None, None, s, None, dy=dqkv, dA=self.dA_qkv,
                             gB=self.gB_qkv, D_in=self.D, r=3 * r)
            parts = ((self.dB_q, 0, Cq), (self.dB_k, Cq, Cq + Ckv), (self.dB_v, Cq + Ckv, self.Cs))
            for i, (dB, c0, c1) in enumerate(parts):
                ops.lora_fwd_bwd(ops.LORA_DB, None, None, None, s, self.xl_qkv[:, i * r:(i + 1) * r],
                                 dy=dqkv[:, c0:c1], dB=dB, r=r, D_in=self.D)
            ev[5].record(self.side)
        # the projections' gradients are complete when both streams are
        main.wait_event(ev[5])
        return self.dx

    def backward(self, dqkv, dy_o):
        self.backward_o(dy_o)
        self.backward_qkv(dqkv)
        return self.dx, self.dx_o
