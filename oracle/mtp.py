"""One-layer MTP draft head over Q8_0 weights, float64 oracle (test infrastructure only).

Follows page "diskformer 0.5.3 -> 0.6.4", engines/ternary_bonsai_2_mtp.js: the file header (the head's graph),
MTPHead.forward and the WGSL kernels it dispatches (WG_NORM, WG_Q8, WG_QKPREP, WG_ATTN, WG_SILU_MUL):

  x   = eh_proj([enorm(e); hnorm(h)])
  x  += attn_output(attention(attn_norm(x)) * sigmoid(gate))   q/k RMSNorm, NEOX RoPE on the first 64 dims,
                                                               grouped-query (24 q heads over 4 kv heads), causal
  x  += ffn_down(silu(ffn_gate(n)) * ffn_up(n)),  n = post_attention_norm(x)
  out = shared_head_norm(x);  token = argmax(out · lm_headᵀ)

Each q head's projection is 512 wide: [query 256 | gate 256].  Row m sits at position pos0 + m, its K/V are
written to the cache there, and it attends to keys kv_lo .. pos0 + m.  The attention scale is 1/sqrt(256).

Chained depth (the file header: "Depth N chains the head"; MTPRunner's draft loop): every further single-row pass
takes the embedding row of the previous draft token and the previous pass's output h' = shared_head_norm(x), one
position later.  The embedding row of a token is the dequantised row of the Q8_0 lm_head table (the pages use the
target's tied token table; the build's reading).
"""
from __future__ import annotations

import numpy as np

from . import prims as P


class MTPOracle:
    def __init__(self, cfg: dict, weights: dict):
        self.cfg = cfg
        self.raw = weights
        self._w: dict[str, np.ndarray] = {}
        w = cfg["kv_heads"] * cfg["head_dim"]
        self.Kc = np.zeros((cfg["max_ctx"], w))
        self.Vc = np.zeros((cfg["max_ctx"], w))

    def w(self, name: str) -> np.ndarray:
        if name not in self._w:
            self._w[name] = P.weight_f64(self.raw[name])
        return self._w[name]

    def set_cache_rows(self, k: np.ndarray, v: np.ndarray, start: int = 0):
        self.Kc[start:start + k.shape[0]] = k
        self.Vc[start:start + v.shape[0]] = v

    def forward(self, e: np.ndarray, h: np.ndarray, pos0: int, kv_lo: int = 0):
        cfg = self.cfg
        M = e.shape[0]
        if M < 1 or M > cfg["block"]:
            raise ValueError("rows out of range")
        if pos0 < 0 or pos0 + M > cfg["max_ctx"] or kv_lo < 0 or kv_lo > pos0:
            raise ValueError("positions beyond the KV cache")
        eps = cfg["rms_eps"]
        NH, NKV, HD, ROT = cfg["heads"], cfg["kv_heads"], cfg["head_dim"], cfg["rope_dims"]
        xc = np.concatenate([P.rmsnorm(e, self.w("enorm"), eps), P.rmsnorm(h, self.w("hnorm"), eps)], axis=1)
        x = P.linear(xc, self.w("eh_proj"))
        a = P.rmsnorm(x, self.w("attn_norm"), eps)
        qf = P.linear(a, self.w("attn_q")).reshape(M, NH, 2 * HD)
        q, gate = qf[:, :, :HD].reshape(M, NH * HD), qf[:, :, HD:].reshape(M, NH * HD)
        k = P.linear(a, self.w("attn_k"))
        v = P.linear(a, self.w("attn_v"))
        pos = np.arange(pos0, pos0 + M)
        q = P.rope_neox_partial(P.head_rmsnorm(q, NH, self.w("attn_q_norm"), eps), pos, NH, ROT, cfg["rope_theta"])
        k = P.rope_neox_partial(P.head_rmsnorm(k, NKV, self.w("attn_k_norm"), eps), pos, NKV, ROT, cfg["rope_theta"])
        self.Kc[pos0:pos0 + M] = k
        self.Vc[pos0:pos0 + M] = v
        keys = self.Kc[kv_lo:pos0 + M]
        vals = self.Vc[kv_lo:pos0 + M]
        kp = np.arange(kv_lo, pos0 + M)
        mask = np.where(kp[None, :] <= pos[:, None], 0.0, -np.inf)
        o = P.attention(q, keys, vals, NH, HD ** -0.5, mask=mask, kv_heads=NKV) * P.sigmoid(gate)
        x = x + P.linear(o, self.w("attn_output"))
        n = P.rmsnorm(x, self.w("post_attention_norm"), eps)
        x = x + P.linear(P.silu(P.linear(n, self.w("ffn_gate"))) * P.linear(n, self.w("ffn_up")), self.w("ffn_down"))
        return P.rmsnorm(x, self.w("shared_head_norm"), eps)

    def lm_argmax(self, hidden: np.ndarray):
        z = P.linear(hidden, self.w("lm_head"))
        return P.argmax_rows(z), z

    def embed_row(self, tok: int) -> np.ndarray:
        """The embedding row of a token: row tok of the dequantised Q8_0 lm_head table (d * q per element)."""
        return self.w("lm_head")[int(tok)]

    def chain(self, tok0: int, h: np.ndarray, steps: int, pos: int, kv_lo: int = 0, follow=None):
        """steps chained single-row passes from draft token tok0 and hidden row h (MTPRunner: drafts[d] comes from a
        pass over [drafts[d - 1]] with the previous pass's output as h, at the next position).  Pass i runs at
        position pos + i.  follow (optional): tokens to chain instead of this oracle's own argmax (a device run that
        took the other side of a near-tie).  Returns (tokens [steps], hidden rows [steps][H], logits [steps][V])."""
        toks, hs, zs = [], [], []
        t, hp = int(tok0), np.asarray(h, np.float64)
        for i in range(steps):
            out = self.forward(self.embed_row(t)[None, :], hp[None, :], pos + i, kv_lo)
            nt, z = self.lm_argmax(out)
            t = int(nt[0]) if follow is None else int(follow[i])
            toks.append(int(nt[0]))
            hs.append(out[0])
            zs.append(z[0])
            hp = out[0]
        return np.array(toks), np.stack(hs), np.stack(zs)
