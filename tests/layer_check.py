"""Teacher-forced checks of one GPU decoder layer against the CPU oracle
(host-side helpers shared by the layer and stack parity tests): every op's
GPU output is compared with the oracle applied to that op's GPU inputs."""
import numpy as np

from oracle import csa, reference as ref
from tests.gpu_util import TOL, host, mar


def gpu_record(cfg, L):
    """Host copies of every intermediate of the GPU layer."""
    Cq, Ckv, F, r = cfg.n_q_heads * cfg.head_dim, cfg.n_kv_heads * cfg.head_dim, cfg.inter, cfg.lora_rank
    g = {k: host(getattr(L, k)) for k in ("n1", "rstd1", "a", "h1", "n2", "rstd2", "y", "dh1", "dx")}
    qkv, dqkv = host(L.attn.qkv), host(L.dqkv)
    xl = host(L.attn.xl_qkv)
    for i, (p, c0, c1) in enumerate((("q", 0, Cq), ("k", Cq, Cq + Ckv), ("v", Cq + Ckv, Cq + 2 * Ckv))):
        g[p], g["d" + p], g["xl_" + p] = qkv[:, c0:c1], dqkv[:, c0:c1], xl[:, i * r:(i + 1) * r]
    g["o"], g["xl_o"], g["da"], g["dn1"] = host(L.attn.o), host(L.attn.xl_o), host(L.attn.dx_o), host(L.attn.dx)
    gu, dgu, xl_gu = host(L.ffn.gu), host(L.ffn.dgu), host(L.ffn.xl_gu)
    g["g"], g["u"], g["dg"], g["du"] = gu[:, :F], gu[:, F:], dgu[:, :F], dgu[:, F:]
    g["xl_gate"], g["xl_up"] = xl_gu[:, :r], xl_gu[:, r:]
    g["h"], g["xl_down"], g["f"], g["dh"], g["dn2"] = (host(L.ffn.h), host(L.ffn.xl_dn), host(L.ffn.y),
                                                       host(L.ffn.dh), host(L.ffn.dx))
    for p in "qkvo":
        g["dA_" + p], g["dB_" + p] = host(getattr(L.attn, "dA_" + p)), host(getattr(L.attn, "dB_" + p))
    for p in ("gate", "up", "down"):
        g["dA_" + p], g["dB_" + p] = host(getattr(L.ffn, "dA_" + p)), host(getattr(L.ffn, "dB_" + p))
    return g


def selections(cfg, inp, g, qk=None, vo=None, ffn=None):
    """Selections from the GPU's normalised group inputs, canonical arithmetic
    (sparsities default to the configuration's; 0 keeps every channel)."""
    qk, vo, ffn = qk or cfg.qk_sparsity, vo or cfg.vo_sparsity, ffn or cfg.ffn_sparsity
    ctx, _ = ref.token_lists(inp["roles"])
    n_rep, Ckv = cfg.n_q_heads // cfg.n_kv_heads, cfg.n_kv_heads * cfg.head_dim
    if qk[0] == 0 and vo[0] == 0 and ffn[0] == 0:
        allkv = np.arange(Ckv, dtype=np.int32)
        return allkv, allkv, np.arange(cfg.inter, dtype=np.int32)
    idx_qk, idx_vo = csa.select_attn(g["n1"], ctx, inp["WA_t_qkv"], inp["WB_q"], inp["WB_k"],
                                     inp["WB_v"], cfg.n_kv_heads, n_rep, cfg.head_dim,
                                     ref.n_keep(Ckv, *qk), ref.n_keep(Ckv, *vo))
    idx_f = csa.select_ffn(g["n2"], ctx, inp["WA_t_gu"], inp["WB_gate"], inp["WB_up"],
                           ref.n_keep(cfg.inter, *ffn))
    return idx_qk, idx_vo, idx_f


def attn_slices(cfg, g, b, grp):
    """q (the group's query heads), k, v, o, da, dq, dk, dv of sequence b and
    key/value head grp, as a 1-sequence, 1-group problem."""
    S, d = cfg.seq, cfg.head_dim
    n_rep = cfg.n_q_heads // cfg.n_kv_heads
    t = slice(b * S, (b + 1) * S)
    cq = slice(grp * n_rep * d, (grp + 1) * n_rep * d)
    ck = slice(grp * d, (grp + 1) * d)
    return {"q": g["q"][t, cq], "k": g["k"][t, ck], "v": g["v"][t, ck], "a": g["a"][t, cq],
            "da": g["da"][t, cq], "dq": g["dq"][t, cq], "dk": g["dk"][t, ck], "dv": g["dv"][t, ck],
            "n_rep": n_rep}


def check_ops(cfg, inp, g, sel, R, attn_parts, tag="layer"):
    """Teacher-forced per-op checks of one decoder layer on rows R (inp: the
    layer's weights with its input x and upstream gradient dy); attention on
    (sequence, group) pairs attn_parts."""
    tol, s, roles = TOL[cfg.dtype], inp["scale"], inp["roles"]
    rr = roles[R]
    idx_qk, idx_vo, idx_f = sel
    ps = ref.attn_proj_indices(idx_qk, idx_vo, cfg.n_q_heads // cfg.n_kv_heads, cfg.head_dim)
    x, dy = inp["x"], inp["dy"]
    chk = lambda name, got, want, t=tol: (name, mar(got, want), t)
    res = []
    n1, r1 = ref.rmsnorm_fwd(x[R])
    res += [chk("n1", g["n1"][R], n1), chk("rstd1", g["rstd1"][R], r1, 1e-5)]
    for p in "qkv":
        res.append(chk("xl_" + p, g["xl_" + p], g["n1"].astype(np.float64) @ inp["A_" + p].T, 1e-5))
        want = ref.sparse_linear_fwd("out", g["n1"][R], inp["W_" + p], rr, ps[p]) \
            + s * (g["xl_" + p][R] @ inp["B_" + p].T)
        res.append(chk(p, g[p][R], want))
    for b, grp in attn_parts:
        a = attn_slices(cfg, g, b, grp)
        o = ref.attention_fwd(a["q"], a["k"], a["v"], 1, cfg.seq, a["n_rep"], 1, cfg.head_dim)
        res.append(chk(f"attn[{b},{grp}]", a["a"], o))
        dq, dk, dv = ref.attention_bwd(a["q"], a["k"], a["v"], a["da"], 1, cfg.seq, a["n_rep"], 1,
                                       cfg.head_dim)
        res += [chk(f"dq[{b},{grp}]", a["dq"], dq), chk(f"dk[{b},{grp}]", a["dk"], dk),
                chk(f"dv[{b},{grp}]", a["dv"], dv)]
    res.append(chk("xl_o", g["xl_o"], g["a"].astype(np.float64) @ inp["A_o"].T, 1e-5))
    o = ref.sparse_linear_fwd("in", g["a"][R], inp["W_o"], rr, ps["o"]) + s * (g["xl_o"][R] @ inp["B_o"].T)
    res.append(chk("o", g["o"][R], o))
    res.append(chk("h1", g["h1"][R], x[R].astype(np.float64) + g["o"][R]))
    n2, r2 = ref.rmsnorm_fwd(g["h1"][R])
    res += [chk("n2", g["n2"][R], n2), chk("rstd2", g["rstd2"][R], r2, 1e-5)]
    for p in ("gate", "up"):
        gp = g["g" if p == "gate" else "u"]
        res.append(chk("xl_" + p, g["xl_" + p], g["n2"].astype(np.float64) @ inp["A_" + p].T, 1e-5))
        want = ref.sparse_linear_fwd("out", g["n2"][R], inp["W_" + p], rr, idx_f) \
            + s * (g["xl_" + p][R] @ inp["B_" + p].T)
        res.append(chk(p, gp[R], want))
    res.append(chk("h", g["h"][R], ref.swiglu_fwd(g["g"][R], g["u"][R])))
    res.append(chk("xl_down", g["xl_down"], g["h"].astype(np.float64) @ inp["A_down"].T, 1e-5))
    f = ref.sparse_linear_fwd("in", g["h"][R], inp["W_down"], rr, idx_f) \
        + s * (g["xl_down"][R] @ inp["B_down"].T)
    res.append(chk("ffn", g["f"][R], f))
    res.append(chk("y", g["y"][R], g["h1"][R].astype(np.float64) + g["f"][R]))
    # backward
    dh = ref.sparse_linear_bwd("in", dy[R], inp["W_down"], rr, idx_f) \
        + s * ((dy[R] @ inp["B_down"]) @ inp["A_down"])
    res.append(chk("dh", g["dh"][R], dh))
    dg, du = ref.swiglu_bwd(g["dh"][R], g["g"][R], g["u"][R])
    res += [chk("dg", g["dg"][R], dg), chk("du", g["du"][R], du)]
    dn2 = sum(ref.sparse_linear_bwd("out", g[gp][R], inp["W_" + p], rr, idx_f)
              + s * ((g[gp][R] @ inp["B_" + p]) @ inp["A_" + p]) for p, gp in (("gate", "dg"), ("up", "du")))
    res.append(chk("dn2", g["dn2"][R], dn2))
    res.append(chk("dh1", g["dh1"][R], ref.rmsnorm_bwd(g["h1"][R], g["rstd2"][R], g["dn2"][R]) + dy[R]))
    da = ref.sparse_linear_bwd("in", g["dh1"][R], inp["W_o"], rr, ps["o"]) \
        + s * ((g["dh1"][R] @ inp["B_o"]) @ inp["A_o"])
    res.append(chk("da", g["da"][R], da))
    dn1 = sum(ref.sparse_linear_bwd("out", g["d" + p][R], inp["W_" + p], rr, ps[p])
              + s * ((g["d" + p][R] @ inp["B_" + p]) @ inp["A_" + p]) for p in "qkv")
    res.append(chk("dn1", g["dn1"][R], dn1))
    res.append(chk("dx", g["dx"][R], ref.rmsnorm_bwd(x[R], g["rstd1"][R], g["dn1"][R]) + g["dh1"][R]))
    # LoRA gradients in full, from the GPU's own inputs of each linear
    lg = [("q", "n1", "xl_q", "dq"), ("k", "n1", "xl_k", "dk"), ("v", "n1", "xl_v", "dv"),
          ("o", "a", "xl_o", "dh1"), ("gate", "n2", "xl_gate", "dg"), ("up", "n2", "xl_up", "du")]
    for p, xi, xl, dyo in lg:
        _, dA, dB = ref.lora_bwd(g[xi], g[xl], g[dyo], inp["A_" + p], inp["B_" + p], s)
        res += [chk("dA_" + p, g["dA_" + p], dA, 1e-3), chk("dB_" + p, g["dB_" + p], dB, 1e-3)]
    _, dA, dB = ref.lora_bwd(g["h"], g["xl_down"], dy, inp["A_down"], inp["B_down"], s)
    res += [chk("dA_down", g["dA_down"], dA, 1e-3), chk("dB_down", g["dB_down"], dB, 1e-3)]
    bad = [(n, e, t) for n, e, t in res if not e <= t]
    worst = max(res, key=lambda z: z[1] / z[2])
    print(f"[{tag}] {len(res)} op checks, worst {worst[0]} {worst[1]:.2e} (tol {worst[2]:.0e})", flush=True)
    assert not bad, bad
