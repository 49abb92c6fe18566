"""A second, loop-only implementation of the three drafters for micro shapes (test infrastructure only).

Plain Python floats and explicit loops, no NumPy arithmetic: every sum, norm, rotation and softmax is spelled out
element by element, in a different structure from the vectorised oracle, so that a transposed operand, a wrong
index or a dropped term in either one shows up as a disagreement.  Only for shapes of a few dozen features.

Weights come in already decoded to float64 (the vectorised oracle's decoding is pinned separately).
"""
from __future__ import annotations

import math


def _mat(W):
    return [[float(v) for v in row] for row in W]


def _vec(v):
    return [float(x) for x in v]


def lin(x, W, b=None):
    """x: list of rows; W: [out][in]."""
    out = []
    for row in x:
        y = []
        for m in range(len(W)):
            acc = 0.0
            for k in range(len(row)):
                acc += row[k] * W[m][k]
            if b is not None:
                acc += b[m]
            y.append(acc)
        out.append(y)
    return out


def rms(row, w, eps):
    ss = 0.0
    for v in row:
        ss += v * v
    r = 1.0 / math.sqrt(ss / len(row) + eps)
    return [row[i] * r * w[i] for i in range(len(row))]


def lnm(row, scale, shift, eps):
    n = len(row)
    mu = sum(row) / n
    var = 0.0
    for v in row:
        var += (v - mu) * (v - mu)
    var /= n
    r = 1.0 / math.sqrt(var + eps)
    return [(row[i] - mu) * r * (1.0 + scale[i]) + shift[i] for i in range(n)]


def head_rms(row, heads, w, eps):
    hd = len(row) // heads
    out = []
    for h in range(heads):
        out += rms(row[h * hd:(h + 1) * hd], w, eps)
    return out


def rope_pairs(row, heads, p, theta):
    """Interleaved pairs (2i, 2i+1) of each head rotated by p * theta^(-2i/hd)."""
    hd = len(row) // heads
    out = list(row)
    for h in range(heads):
        for i in range(hd // 2):
            a = p / (theta ** (2.0 * i / hd))
            c, s = math.cos(a), math.sin(a)
            x0, x1 = row[h * hd + 2 * i], row[h * hd + 2 * i + 1]
            out[h * hd + 2 * i] = x0 * c - x1 * s
            out[h * hd + 2 * i + 1] = x1 * c + x0 * s
    return out


def rope_halves(row, heads, p, rot, theta):
    """NEOX pairs (i, i + rot/2), i < rot/2, of each head; dims >= rot untouched."""
    hd = len(row) // heads
    out = list(row)
    for h in range(heads):
        for i in range(rot // 2):
            a = p * theta ** (-2.0 * i / rot)
            c, s = math.cos(a), math.sin(a)
            x0, x1 = row[h * hd + i], row[h * hd + i + rot // 2]
            out[h * hd + i] = x0 * c - x1 * s
            out[h * hd + i + rot // 2] = x1 * c + x0 * s
    return out


def attend(qs, ks, vs, heads, scale, kv_heads=None, allowed=None):
    """Per query row and head: softmax over allowed keys of q.k * scale, then the weighted sum of values."""
    kv_heads = kv_heads or heads
    hd = len(qs[0]) // heads
    group = heads // kv_heads
    out = []
    for t, q in enumerate(qs):
        row = [0.0] * (heads * hd)
        for h in range(heads):
            kh = h // group
            keys = [j for j in range(len(ks)) if allowed is None or allowed(t, j)]
            sc = []
            for j in keys:
                d = 0.0
                for e in range(hd):
                    d += q[h * hd + e] * ks[j][kh * hd + e]
                sc.append(d * scale)
            mx = max(sc)
            ex = [math.exp(s - mx) for s in sc]
            z = sum(ex)
            for e in range(hd):
                acc = 0.0
                for jj, j in enumerate(keys):
                    acc += ex[jj] / z * vs[j][kh * hd + e]
                row[h * hd + e] = acc
        out.append(row)
    return out


def gelu(v):
    return 0.5 * v * (1.0 + math.erf(v / math.sqrt(2.0)))


def gelu_t(v):
    return 0.5 * v * (1.0 + math.tanh(math.sqrt(2.0 / math.pi) * (v + 0.044715 * v * v * v)))


def sig(v):
    return 1.0 / (1.0 + math.exp(-v))


# ── flow-map ────────────────────────────────────────────────────────────────────────────────────


def flowmap_forward(cfg, W, ctx_taps, anchor, pos):
    """Append ctx_taps at positions 0..n-1, then draft at pos (<= n).  W: name -> float64 array.
    Returns (out rows [T][Ht], logits [T][V])."""
    D, H, hd, L, T = cfg["dim"], cfg["heads"], cfg["head_dim"], cfg["layers"], cfg["block"]
    th, re, qe, le = cfg["rope_theta"], cfg["rms_eps"], cfg["qk_eps"], cfg["ln_eps"]
    g = {k: (_mat(v) if getattr(v, "ndim", 1) == 2 else _vec(v)) for k, v in W.items()}
    Kc = [dict() for _ in range(L)]
    Vc = [dict() for _ in range(L)]

    def put(c_rows, p0):
        for l in range(L):
            ks = lin(c_rows, g[f"layers.{l}.cross_attn.k_proj.weight"])
            vs = lin(c_rows, g[f"layers.{l}.cross_attn.v_proj.weight"])
            for t in range(len(c_rows)):
                k = head_rms(ks[t], H, g[f"layers.{l}.cross_attn.k_norm.weight"], qe)
                Kc[l][p0 + t] = rope_pairs(k, H, p0 + t, th)
                Vc[l][p0 + t] = vs[t]

    c = [rms(r, g["hidden_norm.weight"], re) for r in lin([_vec(r) for r in ctx_taps], g["fc.weight"])]
    put(c, 0)
    E = g["lm_head.weight"]
    a = lin([E[anchor]], g["anchor_proj.weight"], g["anchor_proj.bias"])
    put([rms(a[0], g["anchor_norm.weight"], re)], pos)

    V = len(E)
    mean = [sum(E[v][i] for v in range(V)) / V for i in range(len(E[0]))]
    h0 = lin([rms(mean, g["state_norm.weight"], re)], g["x_embed.weight"], g["x_embed.bias"])[0]
    x = [list(h0) for _ in range(T)]
    md = g["mod"]

    def mod(n):
        return md[n * 3 * D:n * 3 * D + D], md[n * 3 * D + D:n * 3 * D + 2 * D], md[n * 3 * D + 2 * D:(n + 1) * 3 * D]

    def add_gated(x, gate, y):
        return [[x[t][i] + gate[i] * y[t][i] for i in range(D)] for t in range(T)]

    sc = 1.0 / math.sqrt(hd)
    for l in range(L):
        pfx = f"layers.{l}."
        s, b, gt = mod(3 * l)
        h = [lnm(r, s, b, le) for r in x]
        q = [rope_pairs(head_rms(r, H, g[pfx + "self_attn.q_norm.weight"], qe), H, pos + 1 + t, th)
             for t, r in enumerate(lin(h, g[pfx + "self_attn.q_proj.weight"]))]
        k = [rope_pairs(head_rms(r, H, g[pfx + "self_attn.k_norm.weight"], qe), H, pos + 1 + t, th)
             for t, r in enumerate(lin(h, g[pfx + "self_attn.k_proj.weight"]))]
        v = lin(h, g[pfx + "self_attn.v_proj.weight"])
        x = add_gated(x, gt, lin(attend(q, k, v, H, sc), g[pfx + "self_attn.o_proj.weight"]))
        s, b, gt = mod(3 * l + 1)
        h = [lnm(r, s, b, le) for r in x]
        q = [rope_pairs(head_rms(r, H, g[pfx + "cross_attn.q_norm.weight"], qe), H, pos + 1 + t, th)
             for t, r in enumerate(lin(h, g[pfx + "cross_attn.q_proj.weight"]))]
        keys = [Kc[l][j] for j in range(pos + 1)]
        vals = [Vc[l][j] for j in range(pos + 1)]
        x = add_gated(x, gt, lin(attend(q, keys, vals, H, sc), g[pfx + "cross_attn.o_proj.weight"]))
        s, b, gt = mod(3 * l + 2)
        h = [lnm(r, s, b, le) for r in x]
        u = [[gelu(vv) for vv in r] for r in lin(h, g[pfx + "mlp.fc1.weight"], g[pfx + "mlp.fc1.bias"])]
        x = add_gated(x, gt, lin(u, g[pfx + "mlp.fc2.weight"], g[pfx + "mlp.fc2.bias"]))
    s, b, _ = mod(3 * L)
    out = lin([lnm(r, s, b, le) for r in x], g["head.weight"], g["head.bias"])
    return out, lin(out, E)


# ── KV-injection ────────────────────────────────────────────────────────────────────────────────


def kvinject_forward(cfg, W, ctx_taps, anchor):
    d, H, L = cfg["dim"], cfg["heads"], cfg["layers"]
    hd = d // H
    eps = cfg["rms_eps"]
    g = {k: (_mat(v) if getattr(v, "ndim", 1) == 2 else _vec(v)) for k, v in W.items()}
    hc = [rms(r, g["ctx_norm"], eps) for r in lin([_vec(r) for r in ctx_taps], g["W_c"])]
    E = g["lm_head.weight"]
    bp = g["block_pos"]
    first = lin([E[anchor]], g["tok_proj"])[0]
    x = [[first[i] + bp[0][i] for i in range(d)]]
    for k in range(1, cfg["block"]):
        x.append([g["mask_emb"][k - 1][i] + bp[k][i] for i in range(d)])
    for i in range(L):
        p = f"bb.{i}."
        nd = [rms(r, g[p + "attn_norm"], eps) for r in x]
        nc = [rms(r, g[p + "attn_norm"], eps) for r in hc]
        q = lin(nd, g[p + "q"])
        keys = lin(nc, g[p + "k"]) + lin(nd, g[p + "k"])
        vals = lin(nc, g[p + "v"]) + lin(nd, g[p + "v"])
        o = lin(attend(q, keys, vals, H, hd ** -0.5), g[p + "o"])
        x = [[x[t][j] + o[t][j] for j in range(d)] for t in range(len(x))]
        n2 = [rms(r, g[p + "ff_norm"], eps) for r in x]
        ga = lin(n2, g[p + "gate"])
        up = lin(n2, g[p + "up"])
        m = lin([[gelu_t(ga[t][j]) * up[t][j] for j in range(len(ga[t]))] for t in range(len(x))], g[p + "down"])
        x = [[x[t][j] + m[t][j] for j in range(d)] for t in range(len(x))]
    out = lin([rms(r, g["out_norm"], eps) for r in x], g["out_proj"])
    return out, lin(out, E)


# ── MTP ─────────────────────────────────────────────────────────────────────────────────────────


def mtp_forward(cfg, W, e_rows, h_rows, kcache, vcache, pos0, kv_lo):
    """kcache / vcache: rows for positions [0, pos0).  Returns (out rows, logits)."""
    NH, NKV, HD, ROT, th = cfg["heads"], cfg["kv_heads"], cfg["head_dim"], cfg["rope_dims"], cfg["rope_theta"]
    eps = cfg["rms_eps"]
    g = {k: (_mat(v) if getattr(v, "ndim", 1) == 2 else _vec(v)) for k, v in W.items()}
    M = len(e_rows)
    xc = [rms(_vec(e_rows[m]), g["enorm"], eps) + rms(_vec(h_rows[m]), g["hnorm"], eps) for m in range(M)]
    x = lin(xc, g["eh_proj"])
    a = [rms(r, g["attn_norm"], eps) for r in x]
    qf = lin(a, g["attn_q"])
    kt = lin(a, g["attn_k"])
    vt = lin(a, g["attn_v"])
    Ks = [_vec(r) for r in kcache] + [None] * M
    Vs = [_vec(r) for r in vcache] + [None] * M
    qs, gates = [], []
    for m in range(M):
        qrow, grow = [], []
        for h in range(NH):
            qrow += qf[m][h * 2 * HD:h * 2 * HD + HD]
            grow += qf[m][h * 2 * HD + HD:(h + 1) * 2 * HD]
        qs.append(rope_halves(head_rms(qrow, NH, g["attn_q_norm"], eps), NH, pos0 + m, ROT, th))
        gates.append(grow)
        Ks[pos0 + m] = rope_halves(head_rms(kt[m], NKV, g["attn_k_norm"], eps), NKV, pos0 + m, ROT, th)
        Vs[pos0 + m] = vt[m]
    keys = Ks[kv_lo:pos0 + M]
    vals = Vs[kv_lo:pos0 + M]
    o = attend(qs, keys, vals, NH, HD ** -0.5, kv_heads=NKV, allowed=lambda t, j: kv_lo + j <= pos0 + t)
    o = [[o[m][i] * sig(gates[m][i]) for i in range(len(o[m]))] for m in range(M)]
    y = lin(o, g["attn_output"])
    x = [[x[m][i] + y[m][i] for i in range(len(x[m]))] for m in range(M)]
    n = [rms(r, g["post_attention_norm"], eps) for r in x]
    gg = lin(n, g["ffn_gate"])
    uu = lin(n, g["ffn_up"])
    f = lin([[gg[m][i] * sig(gg[m][i]) * uu[m][i] for i in range(len(gg[m]))] for m in range(M)], g["ffn_down"])
    x = [[x[m][i] + f[m][i] for i in range(len(x[m]))] for m in range(M)]
    out = [rms(r, g["shared_head_norm"], eps) for r in x]
    return out, lin(out, g["lm_head"])
