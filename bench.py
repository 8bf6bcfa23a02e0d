#!/usr/bin/env python3
"""Benchmark of the contextually-sparse LoRA FFN block (forward + backward) on
one MI355X at the LLaMA3-8B FFN shape: hidden 4096, intermediate 14336,
batch 8 x seq 512 (last 128 tokens of each sequence are output tokens),
bf16, LoRA rank 16 on gate/up/down, estimator rank 16, 70% channel sparsity.

One step = token split, estimator, SwiGLU-L2 scoring, top-n selection,
gathered/dense main-branch GEMMs, dense LoRA, SwiGLU, and the whole backward
(input gradient and the six LoRA gradients), on synthetic inputs already in
HBM.  Prints one JSON line (rank 0, N = 1).
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
# fp32 vector arithmetic without packed (two-wide) fp32 instructions, which
# this library does not use: 256 CUs x 4 SIMDs x 16 lanes x 2 flops (FMA) x
# 2.4 GHz
PEAK_F32_VALU_TFLOPS = 78.6


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-ablations", action="store_true",
                    help="skip the step times with the random and the exact-output criteria")
    ap.add_argument("--no-schedule", action="store_true",
                    help="skip the whole-training-step run with the dense-then-sparse schedule")
    ap.add_argument("--schedule-steps", type=int, default=20)
    ap.add_argument("--no-factors", action="store_true",
                    help="skip timing the on-GPU estimator factor preparation")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the sparse/dense step times of the other workloads (projections, "
                         "layer, 32-layer stack, fp32 block)")
    ap.add_argument("--single-stream", action="store_true",
                    help="issue every launch of the block on one stream (clean per-kernel times "
                         "for profiles; the default overlaps LoRA reductions and the output-row "
                         "product on a second stream)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="end with one plain 256 MiB device copy (reference for HBM byte counters)")
    return ap.parse_args()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_nt_ffn_llama3_8b_hbm_traffic.md")
KERNEL_SOURCES = [os.path.join(ROOT, "contextual_sparsity_lora_amd", "csrc", f)
                  for f in ("k_gemm.hip", "sl_internal.h")]


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch of the dominant GEMM kernel from the committed
    rocprofv3 counter summary, or None when that summary is missing or was
    taken on a different version of the kernel sources."""
    try:
        with open(TRAFFIC_FILE) as fh:
            text = fh.read()
    except OSError:
        return None
    vals = {}
    for line in text.splitlines():
        if line.startswith("traffic:"):
            for kv in line[len("traffic:"):].split():
                k, _, v = kv.partition("=")
                vals[k] = v
    if vals.get("kernel_source_sha256") != kernel_source_hash():
        return None
    try:
        return float(vals["bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def build_block(inp, cfg, dense, criterion="svd", single_stream=False):
    import numpy as np
    import torch
    from contextual_sparsity_lora_amd.ffn import SparseFFN
    dev = "cuda:0"
    t = {k: torch.from_numpy(v).to(torch.bfloat16).to(dev) for k, v in inp.items()
         if isinstance(v, np.ndarray) and k.startswith(("x", "W_", "A_", "B_", "dy"))}
    blk = SparseFFN(t["W_gate"], t["W_up"], t["W_down"], t["A_gate"], t["B_gate"], t["A_up"],
                    t["B_up"], t["A_down"], t["B_down"],
                    torch.from_numpy(np.ascontiguousarray(inp["WA_t_gu"].T)).to(dev),
                    torch.from_numpy(inp["WB_gate"]).to(dev), torch.from_numpy(inp["WB_up"]).to(dev),
                    inp["scale"], sparsity=cfg.ffn_sparsity, dense=dense, criterion=criterion,
                    single_stream=single_stream)
    roles = torch.from_numpy(inp["roles"]).to(dev)
    return blk, t["x"], roles, t["dy"]


def time_steps(blk, x, roles, dy, T_c, steps, warmup, ops, record=False, only=None):
    """Mean ms per step over `steps` steps after `warmup` untimed ones.  With
    record, the library brackets its launches (of class `only`, else of every
    class) with HIP events on their own streams."""
    import torch
    for _ in range(warmup):
        blk.forward(x, roles, T_c)
        blk.backward(dy)
    torch.cuda.synchronize()
    # the warm-up sized every workspace: the timed steps allocate nothing
    ops.set_option(0, "workspace_fixed", 1)
    if record:
        ops.timing_reset(0)
        ops.timing_only(0, only)
        ops.timing_enable(0, True)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(steps):
        blk.forward(x, roles, T_c)
        blk.backward(dy)
    stop.record()
    torch.cuda.synchronize()
    ops.set_option(0, "workspace_fixed", 0)
    if record:
        ops.timing_enable(0, False)
        ops.timing_only(0, None)
    return start.elapsed_time(stop) / steps


def step_distribution(blk, x, roles, dy, T_c, steps, ops):
    """Per-step times (ms) of `steps` further steps, each bracketed by its own
    events on the caller's stream (the block joins its second stream before
    returning, so the end event follows all of the step's work)."""
    import torch
    ops.set_option(0, "workspace_fixed", 1)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    for a, b in ev:
        a.record()
        blk.forward(x, roles, T_c)
        blk.backward(dy)
        b.record()
    torch.cuda.synchronize()
    ops.set_option(0, "workspace_fixed", 0)
    return [a.elapsed_time(b) for a, b in ev]


def graph_step_ms(step, side, steps):
    """Mean ms per step with the whole step (forward + backward, both streams)
    replayed from a HIP graph (StepGraph: captured after eager warm-up steps
    on its own stream); the host issues one replay per step.  None (with the
    reason on stderr) when the capture fails: these are side figures, and the
    bench line must not depend on them."""
    try:
        return _graph_step_ms(step, side, steps)
    except Exception as e:   # noqa: BLE001 - reported, the rest of the bench goes on
        print(f"[bench] HIP graph timing skipped: {type(e).__name__}: {e}", file=sys.stderr, flush=True)
        return None


def _graph_step_ms(step, side, steps):
    import torch
    from contextual_sparsity_lora_amd.graph import StepGraph
    g = StepGraph(step, side_streams=(side,))
    try:
        for _ in range(2):
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps
    finally:
        g.close()


def percentiles(v):
    import numpy as np
    return [round(float(q), 4) for q in np.percentile(np.asarray(v), [10, 50, 90])]


def training_schedule(inp, cfg, ops, steps, dense_frac=0.1, vocab=32000):
    """Whole training steps (block forward, LM-head logits of the output rows,
    cross-entropy, backward, AdamW on LoRA) over `steps` steps: once with the
    first ceil(dense_frac steps) dense and the rest sparse, once all dense.
    Returns the timings, the sparse-phase speedup s and the bound
    1 / (p + (1 - p) / s) on the overall speedup."""
    import math
    import numpy as np
    import torch
    from contextual_sparsity_lora_amd.train import LoRATrainer
    dev = "cuda:0"
    rng = np.random.default_rng(cfg.seed + 77)
    bf = torch.bfloat16
    W_head = (torch.from_numpy(rng.standard_normal((vocab, cfg.hidden)).astype(np.float32)) * 0.02).to(bf).to(dev)
    # a synthetic stream of two batches (hidden states and next-token labels)
    xs = [torch.from_numpy(inp["x"]).to(bf).to(dev),
          torch.from_numpy(rng.standard_normal((cfg.tokens, cfg.hidden)).astype(np.float32)).to(bf).to(dev)]
    labels = [torch.from_numpy(rng.integers(0, vocab, size=cfg.tokens).astype(np.int32)).to(dev) for _ in xs]
    roles = torch.from_numpy(inp["roles"]).to(dev)

    def run(frac, n, record=None):
        blk, _, _, _ = build_block(inp, cfg, dense=False)
        # one untimed step in the mode of the first timed step (buffers of the
        # block and the head made once, outside the timed steps)
        LoRATrainer(blk, W_head, total_steps=1, dense_frac=1.0 if frac > 0 else 0.0).step(
            xs[0], labels[0], roles, cfg.ctx_tokens)
        tr = LoRATrainer(blk, W_head, total_steps=n, dense_frac=frac)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
        torch.cuda.synchronize()
        ev[0].record()
        for t in range(n):
            tr.step(xs[t % 2], labels[t % 2], roles, cfg.ctx_tokens)
            ev[t + 1].record()
        torch.cuda.synchronize()
        ms = [ev[t].elapsed_time(ev[t + 1]) for t in range(n)]
        del tr, blk
        torch.cuda.empty_cache()
        return ms

    run(0.5, 4)                                   # warm-up: every kernel of both phases
    sched = run(dense_frac, steps)
    dense = run(1.0, steps)
    nd = math.ceil(dense_frac * steps)
    d_step = float(np.median(dense))
    s_step = float(np.median(sched[nd:]))
    s = d_step / s_step
    return {"steps": steps, "dense_frac": dense_frac, "dense_steps": nd, "vocab": vocab,
            "note": "totals include the switch from the dense to the sparse phase; per-phase step "
                    "times are medians",
            "lr_schedule": "cosine, 4% warm-up", "optimizer": "AdamW on LoRA (fp32 masters)",
            "dense_step_ms": round(d_step, 4), "sparse_step_ms": round(s_step, 4),
            "scheduled_total_ms": round(sum(sched), 3), "dense_total_ms": round(sum(dense), 3),
            "sparse_phase_speedup": round(s, 4), "overall_speedup": round(sum(dense) / sum(sched), 4),
            "bound": round(1.0 / (dense_frac + (1.0 - dense_frac) / s), 4)}


def _rand_layer_arrays(cfg, gen, dev):
    """Device weights of one decoder layer, N(0, 0.02^2) in bf16, and fp32
    estimator factors N(0, 1/rows), drawn from a seeded torch generator (step
    times do not depend on the values; parity tests use the oracle's inputs)."""
    import torch
    D, F, r, k = cfg.hidden, cfg.inter, cfg.lora_rank, cfg.est_rank
    Cq, Ckv = cfg.n_q_heads * cfg.head_dim, cfg.n_kv_heads * cfg.head_dim
    w = lambda *sh: (torch.randn(*sh, generator=gen, device=dev) * 0.02).to(torch.bfloat16)
    f = lambda *sh: torch.randn(*sh, generator=gen, device=dev) / sh[0] ** 0.5
    d = {"W_q": w(Cq, D), "W_k": w(Ckv, D), "W_v": w(Ckv, D), "W_o": w(D, Cq)}
    for p, co, ci in (("q", Cq, D), ("k", Ckv, D), ("v", Ckv, D), ("o", D, Cq)):
        d["A_" + p], d["B_" + p] = w(r, ci), w(co, r)
    if F:
        d.update({"W_gate": w(F, D), "W_up": w(F, D), "W_down": w(D, F)})
        for p, co, ci in (("gate", F, D), ("up", F, D), ("down", D, F)):
            d["A_" + p], d["B_" + p] = w(r, ci), w(co, r)
    f32 = {"WA_qkv": f(D, 3 * k), "WB_q": f(k, Cq), "WB_k": f(k, Ckv), "WB_v": f(k, Ckv)}
    if F:
        f32.update({"WA_gu": f(D, 2 * k), "WB_gate": f(k, F), "WB_up": f(k, F)})
    return d, f32


def other_configs(steps=3):
    """fwd+bwd step times, sparse and dense (every channel kept, same LoRA), of
    the other workloads: the fp32 FFN block (config 1), the LLaMA3-8B q/k/v/o
    projections (config 3), one LLaMA2-13B decoder layer (config 4) and the
    32-layer LLaMA3-8B stack with its per-layer sparsity ramp (config 5)."""
    import torch
    from contextual_sparsity_lora_amd.attn import SparseAttnProj
    from contextual_sparsity_lora_amd.layer import SparseDecoderLayer
    from contextual_sparsity_lora_amd.stack import SparseStack
    from workloads.configs import CONFIGS
    from workloads.gen import make_ffn_inputs, roles_for
    dev = "cuda:0"

    def timed(step, n, warm=3):
        for _ in range(warm):
            step()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            step()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    out = {}
    # config 1: the fp32 FFN block
    cfg = CONFIGS[1]
    inp = make_ffn_inputs(cfg)
    ms, gms = {}, {}
    for dense in (False, True):
        import numpy as np
        from contextual_sparsity_lora_amd.ffn import SparseFFN
        t = {k: torch.from_numpy(v).to(dev) for k, v in inp.items() if isinstance(v, np.ndarray)
             and k.startswith(("x", "W_", "A_", "B_", "dy"))}
        blk = SparseFFN(t["W_gate"], t["W_up"], t["W_down"], t["A_gate"], t["B_gate"], t["A_up"], t["B_up"],
                        t["A_down"], t["B_down"], torch.from_numpy(np.ascontiguousarray(inp["WA_t_gu"].T)).to(dev),
                        t["WB_gate"] if "WB_gate" in t else torch.from_numpy(inp["WB_gate"]).to(dev),
                        torch.from_numpy(inp["WB_up"]).to(dev), inp["scale"], sparsity=cfg.ffn_sparsity, dense=dense)
        roles = torch.from_numpy(inp["roles"]).to(dev)
        step1 = lambda: (blk.forward(t["x"], roles, cfg.ctx_tokens), blk.backward(t["dy"]))
        ms[dense] = timed(step1, 20)
        gms[dense] = graph_step_ms(step1, blk.side, 20)
    out["1"] = {"workload": cfg.name, "tokens": cfg.tokens, "sparse_ms": round(ms[False], 4),
                "dense_ms": round(ms[True], 4), "speedup": round(ms[True] / ms[False], 3)}
    if gms.get(False) is not None and gms.get(True) is not None:
        out["1"].update({"graph_sparse_ms": round(gms[False], 4), "graph_dense_ms": round(gms[True], 4),
                         "graph_speedup": round(gms[True] / gms[False], 3)})
    gen = torch.Generator(device=dev)
    for cid in (3, 4, 5):
        cfg = CONFIGS[cid]
        roles = torch.from_numpy(roles_for(cfg)).to(dev)
        T, D = cfg.tokens, cfg.hidden
        ms, gms = {}, {}
        for dense in (False, True):
            gen.manual_seed(cfg.seed)
            x = (torch.randn(T, D, generator=gen, device=dev)).to(torch.bfloat16)
            dy = torch.randn(T, D, generator=gen, device=dev).to(torch.bfloat16)
            if cid == 3:
                d, f32 = _rand_layer_arrays(cfg, gen, dev)
                blk = SparseAttnProj(d["W_q"], d["W_k"], d["W_v"], d["W_o"], d["A_q"], d["B_q"], d["A_k"], d["B_k"],
                                     d["A_v"], d["B_v"], d["A_o"], d["B_o"], f32["WA_qkv"], f32["WB_q"], f32["WB_k"],
                                     f32["WB_v"], cfg.lora_scale, cfg.n_kv_heads, cfg.head_dim,
                                     qk_sparsity=cfg.qk_sparsity, vo_sparsity=cfg.vo_sparsity, dense=dense)
                Cs = blk.Cs
                xo = torch.randn(T, blk.Cq, generator=gen, device=dev).to(torch.bfloat16)
                dqkv = torch.randn(T, Cs, generator=gen, device=dev).to(torch.bfloat16)
                step = lambda: (blk.forward(x, xo, roles, cfg.ctx_tokens), blk.backward(dqkv, dy[:, :D]))
            elif cid == 4:
                d, f32 = _rand_layer_arrays(cfg, gen, dev)
                blk = SparseDecoderLayer.from_arrays(d, f32, cfg, cfg.qk_sparsity, cfg.vo_sparsity,
                                                     cfg.ffn_sparsity, dense=dense)
                step = lambda: (blk.forward(x, roles, cfg.ctx_tokens), blk.backward(dy))
            else:
                arrays, sps = [], []
                for layer in range(cfg.n_layers):
                    arrays.append(_rand_layer_arrays(cfg, gen, dev))
                    sps.append((0, 1) if dense else cfg.layer_sparsity(layer))
                blk = SparseStack.build(cfg, arrays, sps)
                del arrays
                step = lambda: (blk.forward(x, roles, cfg.ctx_tokens), blk.backward(dy))
            # (the one-layer workloads take about a millisecond a step: 20 timed
            # steps keep launch jitter out; the 32-layer stack takes the given count)
            ms[dense] = timed(step, steps if cid == 5 else max(steps, 20), warm=1 if cid == 5 else 3)
            if cid == 3:   # one block with one second stream: also replayed from a HIP graph
                gms[dense] = graph_step_ms(step, blk.side, 20)
            del blk, step
            torch.cuda.empty_cache()
        out[str(cid)] = {"workload": cfg.name, "tokens": T, "sparse_ms": round(ms[False], 3),
                         "dense_ms": round(ms[True], 3), "speedup": round(ms[True] / ms[False], 3),
                         "sparse_tokens_per_s": round(T / (ms[False] * 1e-3), 1)}
        if gms.get(False) is not None and gms.get(True) is not None:
            out[str(cid)].update({"graph_sparse_ms": round(gms[False], 3), "graph_dense_ms": round(gms[True], 3),
                                  "graph_speedup": round(gms[True] / gms[False], 3)})
        print(f"[bench] config {cid} ({cfg.name}): sparse {ms[False]:.3f} ms, dense {ms[True]:.3f} ms",
              file=sys.stderr, flush=True)
    return out


def cpu_baseline(inp, cfg, min_s=10.0, threads=None):
    """The CPU oracle on whole sequences of the workload (512 tokens each: 384
    context, 128 output), one after another until at least `min_s` seconds have
    passed or the batch is done: per sequence, selection over its context
    tokens (fp32 C) + masked-dense fp64 forward and backward.  threads: cap on
    the BLAS threads (None: as configured)."""
    if threads is not None:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=threads):
            return cpu_baseline(inp, cfg, min_s, None)
    from oracle import csa, reference as ref
    try:
        from threadpoolctl import threadpool_info
        cores = max([d.get("num_threads", 1) for d in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count() or 1
    S = cfg.seq
    done, t0 = 0, time.perf_counter()
    for b in range(cfg.batch):
        sub = dict(inp)
        for k in ("x", "dy"):
            sub[k] = inp[k][b * S:(b + 1) * S]
        sub["roles"] = inp["roles"][b * S:(b + 1) * S]
        ctx, _ = ref.token_lists(sub["roles"])
        sc = csa.ssq_swiglu(csa.stage1(sub["x"], ctx, inp["WA_t_gu"]), inp["WB_gate"], inp["WB_up"])
        idx = csa.select(sc, ref.n_keep(cfg.inter, *cfg.ffn_sparsity))
        f = ref.ffn_block_fwd(sub, idx)
        ref.ffn_block_bwd(sub, f, idx)
        done += 1
        if time.perf_counter() - t0 >= min_s:
            break
    dt = time.perf_counter() - t0
    return {"value": done * S / dt, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{done} of the workload's {cfg.batch} sequences, each {S} tokens "
                      f"({S - cfg.out_per_seq} context, {cfg.out_per_seq} output) with its own selection: "
                      f"fp32 selection + fp64 masked-dense fwd+bwd, {dt:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)
    import torch
    from contextual_sparsity_lora_amd import ops
    from workloads.configs import CONFIGS
    from workloads.gen import make_ffn_inputs

    cfg = CONFIGS[2]
    t0 = time.perf_counter()
    inp = make_ffn_inputs(cfg)
    print(f"[bench] inputs ready in {time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)
    blk, x, roles, dy = build_block(inp, cfg, dense=False, single_stream=args.single_stream)
    T = cfg.tokens
    # per-class breakdown from a short instrumented pass of its own: events
    # around every launch add time between launches, so the timed pass below
    # brackets only the dominant kernel class
    psteps = max(1, min(args.steps, 5))
    pms = time_steps(blk, x, roles, dy, cfg.ctx_tokens, psteps, args.warmup, ops, record=True)
    per_class = {}
    for c in ops.timing_classes():
        n, tms, fl, by = ops.timing_query(0, c)
        if n:
            per_class[c] = {"launches_per_step": n / psteps, "ms_per_step": tms / psteps,
                            "gflop_per_step": fl / psteps / 1e9,
                            "gbyte_per_step": by / psteps / 1e9}
    print(f"[bench] instrumented step {pms:.3f} ms (events around every launch)", file=sys.stderr,
          flush=True)
    for c, v in sorted(per_class.items(), key=lambda kv: -kv[1]["ms_per_step"]):
        print(f"[bench]   {c:13s} {v['ms_per_step']:8.3f} ms  {v['gflop_per_step']:9.2f} GF  "
              f"{v['gbyte_per_step']:7.3f} GB  x{v['launches_per_step']:.0f}", file=sys.stderr)
    # dominant kernel: the class with the most time per step
    dom = max(per_class, key=lambda c: per_class[c]["ms_per_step"])
    ms = time_steps(blk, x, roles, dy, cfg.ctx_tokens, args.steps, 1, ops, record=True, only=dom)
    # the spread of single steps (each between its own events), beside the
    # bracketed mean that `value` is computed from
    step_pct = percentiles(step_distribution(blk, x, roles, dy, cfg.ctx_tokens, args.steps, ops))
    print(f"[bench] sparse step {ms:.3f} ms (events around {dom} only)", file=sys.stderr, flush=True)
    dn, dms, dfl, dby = ops.timing_query(0, dom)
    if dom.startswith("gemm"):
        achieved = dfl / (dms * 1e-3) / 1e12
        tr = measured_traffic()
        roof = {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": round(tr) if tr is not None else None,
                "algorithmic_bytes_per_launch": round(dby / dn),
                "launches": dn, "avg_launch_ms": round(dms / dn, 4)}
    else:
        achieved = dby / (dms * 1e-3) / 1e9
        roof = {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 2),
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                "traffic": None, "launches": dn, "avg_launch_ms": round(dms / dn, 4)}
    # the same per-class pass with every launch on one stream (each kernel
    # alone on the GPU: clean per-kernel times), and the selection chain's
    # kernels against their bounds
    side = blk.side
    blk.side = torch.cuda.current_stream()
    sms = time_steps(blk, x, roles, dy, cfg.ctx_tokens, psteps, 1, ops, record=True)
    blk.side = side
    per_class_1s = {}
    for c in ops.timing_classes():
        n, tms, fl, by = ops.timing_query(0, c)
        if n:
            sec = tms * 1e-3
            per_class_1s[c] = {"launches_per_step": n / psteps, "ms_per_step": round(tms / psteps, 4),
                               "gbs": round(by / sec / 1e9, 1), "hbm_frac": round(by / sec / 1e9 / PEAK_HBM_GBS, 4),
                               "tflops": round(fl / sec / 1e12, 2)}
    ops.timing_reset(0)
    selection = {}
    for c in ("estimate", "score", "topk"):
        if c in per_class_1s:
            v = dict(per_class_1s[c])
            v["valu_frac"] = round(v["tflops"] / PEAK_F32_VALU_TFLOPS, 4)
            selection[c] = v
    print(f"[bench] single-stream instrumented step {sms:.3f} ms; selection: {selection}", file=sys.stderr,
          flush=True)
    gemm_fl = sum(v["gflop_per_step"] for c, v in per_class.items() if c.startswith("gemm"))
    gemm_ms = sum(v["ms_per_step"] for c, v in per_class.items() if c.startswith("gemm"))
    step_gf = sum(v["gflop_per_step"] for v in per_class.values())
    ops.timing_reset(0)
    extra = {"gemm_tflops": round(gemm_fl / gemm_ms, 2) if gemm_ms else None,
             "mfma_util_gemm": round(gemm_fl / gemm_ms / PEAK_BF16_TFLOPS, 4) if gemm_ms else None,
             "step_tflops": round(step_gf / ms, 2), "per_class": per_class,
             "per_class_note": f"separate instrumented pass of {psteps} steps "
                               f"({pms:.3f} ms/step with events around every launch)",
             "per_class_single_stream": per_class_1s,
             "per_class_single_stream_note": f"{psteps} steps with every launch on one stream "
                                             f"({sms:.3f} ms/step with events around every launch)",
             "selection_chain": selection,
             "selection_chain_note": "single-stream pass; gbs/hbm_frac against 8 TB/s, tflops/valu_frac "
                                     "against the 78.6 TF/s fp32 vector peak without packed fp32"}
    graph = {}
    if not args.single_stream:
        g_ms = graph_step_ms(lambda: (blk.forward(x, roles, cfg.ctx_tokens), blk.backward(dy)), blk.side,
                             args.steps)
        if g_ms is not None:
            graph["sparse_ms"] = round(g_ms, 4)
            print(f"[bench] sparse step replayed from a HIP graph {graph['sparse_ms']:.3f} ms", file=sys.stderr,
                  flush=True)
    if not args.no_dense:
        import types
        from contextual_sparsity_lora_amd import fidelity
        # the sparse block's LoRA gradients of its last step (same inputs every step)
        sparse_grads = types.SimpleNamespace(**{k: v.clone() for k, v in fidelity.lora_grads(blk).items()})
        del blk
        torch.cuda.empty_cache()
        dblk, x, roles, dy = build_block(inp, cfg, dense=True, single_stream=args.single_stream)
        dms_step = time_steps(dblk, x, roles, dy, cfg.ctx_tokens, args.steps, args.warmup, ops)
        extra["dense_ms_per_step"] = round(dms_step, 4)
        extra["dense_step_ms_p10_p50_p90"] = percentiles(
            step_distribution(dblk, x, roles, dy, cfg.ctx_tokens, args.steps, ops))
        extra["speedup_vs_dense"] = round(dms_step / ms, 3)
        print(f"[bench] dense step {dms_step:.3f} ms", file=sys.stderr, flush=True)
        if graph:
            g_ms = graph_step_ms(lambda: (dblk.forward(x, roles, cfg.ctx_tokens), dblk.backward(dy)), dblk.side,
                                 args.steps)
            if g_ms is not None:
                graph["dense_ms"] = round(g_ms, 4)
                graph["speedup"] = round(graph["dense_ms"] / graph["sparse_ms"], 3)
                print(f"[bench] dense step replayed from a HIP graph {graph['dense_ms']:.3f} ms", file=sys.stderr,
                      flush=True)
        # gradient fidelity: cosine between the sparse and the dense block's
        # LoRA gradients on the same synthetic inputs (random weights: a
        # measurement of the tool, not a result about the method)
        extra["grad_fidelity"] = {k: round(v, 6) for k, v in
                                  fidelity.block_fidelity(sparse_grads, dblk).items()}
        print(f"[bench] LoRA gradient cosines sparse vs dense: {extra['grad_fidelity']}",
              file=sys.stderr, flush=True)
        del dblk
    if graph:
        extra["graph_replay"] = graph
    out = {
        "metric": "sparse-LoRA linear fwd+bwd tokens/s and MFMA util at LLaMA3-8B FFN shape, 1 GPU",
        "value": round(T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "step_ms_p10_p50_p90": step_pct,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "llama3-8b-ffn-block-fwd-bwd", "hidden": cfg.hidden,
                   "intermediate": cfg.inter, "batch": cfg.batch, "seq": cfg.seq,
                   "output_tokens_per_seq": cfg.out_per_seq, "lora_rank": cfg.lora_rank,
                   "estimator_rank": cfg.est_rank, "ffn_sparsity": "7/10",
                   "kept_channels": blk_n(cfg), "global_batch": cfg.batch, "seq_len": cfg.seq,
                   "parallelism": "single-gpu", "streams": 1 if args.single_stream else 2},
        "roofline": roof,
        "cpu_baseline": None,
    }
    if not args.no_factors:
        # the offline step: rank-16 factors of gate and up (randomized subspace
        # iteration, 3 power steps, 16 extra columns) from the bf16 weights
        import numpy as np
        F, D, k = cfg.inter, cfg.hidden, cfg.est_rank
        W = torch.from_numpy(np.concatenate([inp["W_gate"], inp["W_up"]])).to(torch.bfloat16).to("cuda:0")
        Wt = torch.empty(D, 2 * F, dtype=torch.bfloat16, device="cuda:0")
        ops.transpose(W, Wt)
        WA_t = torch.empty(k, D, dtype=torch.float32, device="cuda:0")
        WB = torch.empty(k, F, dtype=torch.float32, device="cuda:0")
        ops.svd_factors(W[:F], Wt[:, :F], k, WA_t, WB)          # warm-up
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for half in range(2):
            ops.svd_factors(W[half * F:(half + 1) * F], Wt[:, half * F:(half + 1) * F], k, WA_t, WB, seed=half)
        e1.record()
        torch.cuda.synchronize()
        extra["factor_prep_ms_per_matrix"] = round(e0.elapsed_time(e1) / 2, 3)
        print(f"[bench] factor preparation {extra['factor_prep_ms_per_matrix']} ms per {F}x{D} matrix",
              file=sys.stderr, flush=True)
        del W, Wt
    if not args.no_configs:
        extra["other_configs"] = other_configs()
    if not args.no_schedule:
        extra["training_schedule"] = training_schedule(inp, cfg, ops, args.schedule_steps)
        print(f"[bench] training schedule: {extra['training_schedule']}", file=sys.stderr, flush=True)
    if not args.no_ablations:
        # the same step with the selection made at random (no estimator: the
        # difference is the estimator's cost) and by the exact-output criterion
        # (dense gate|up outputs first: what the estimator avoids)
        # (all three timed alike, without events)
        crit_ms = {}
        for crit in ("svd", "random", "oracle"):
            ablk, x, roles, dy = build_block(inp, cfg, dense=False, criterion=crit)
            crit_ms[crit] = round(time_steps(ablk, x, roles, dy, cfg.ctx_tokens, args.steps,
                                             args.warmup, ops), 4)
            del ablk
            torch.cuda.empty_cache()
        extra["criterion_ms_per_step"] = crit_ms
        extra["estimator_overhead_vs_random"] = round(crit_ms["svd"] / crit_ms["random"] - 1.0, 4)
        print(f"[bench] step ms by criterion: {crit_ms}", file=sys.stderr, flush=True)
    if args.calibrate_copy:
        src = torch.empty(128 * 1024 * 1024, dtype=torch.bfloat16, device="cuda:0")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    out.update(extra)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, cfg)
        out["cpu_baseline"]["affinity_cpus"] = len(os.sched_getaffinity(0))
        # one core: one sequence (its oracle work alone takes tens of seconds)
        one = cpu_baseline(inp, cfg, min_s=1.0, threads=1)
        out["cpu_baseline"]["single_core"] = {k: one[k] for k in ("value", "unit", "cores", "sample")}
        print(f"[bench] cpu baseline {out['cpu_baseline']['value']:.1f} tokens/s "
              f"({out['cpu_baseline']['cores']} threads), {one['value']:.1f} tokens/s on one core",
              file=sys.stderr, flush=True)
    print(json.dumps(out), flush=True)


def blk_n(cfg):
    from contextual_sparsity_lora_amd.ffn import keep_count
    return keep_count(cfg.inter, *cfg.ffn_sparsity)


if __name__ == "__main__":
    main()
