"""KV-injection (DFlash / DSpark) block drafter, float64 oracle (test infrastructure only).

Follows page "mlx-bun 0.4.0 -> 1.0.0", src/spec/dspark/module-dflash.ts: the file header (DSpark Eq 2 and Eq 3),
#buildContext, #buildBlock, #layer, #backbone, projectContextRows and #baseLogits.

  Eq 2   H_ctx = RMSNorm(W_c [H^l1; ...; H^lm])
  Eq 3   K_i = [W_i^K n(H_ctx); W_i^K n(H_d)], V_i likewise, Q_i = W_i^Q n(H_d), n = the layer's attn_norm applied to
         context and block alike; the block attends bidirectionally over [context ++ block].

Readings: no RoPE, no q/k norm, no mask (batch of one); the head output is not cast before the lm_head; the lm_head
table E is also the embedding table. The activation the page calls geluApprox is read as the tanh form (parity
unpinned beyond that reading; the formula is pinned against PyTorch's tanh-approximate GELU).

Markov decode (forwardRows' greedy loop with the Markov head, #markov, #confidence): with block = RMSNorm(H_d;
out_norm) and base logits z = (block out_proj) E^T, step k takes e1 = w1[prev] (prev = the anchor, then the
previous step's token), scores_k = z_k + e1 w2, token_k = argmax scores_k and conf_k = sigmoid([block_k; e1] conf.w
+ conf.b). draft_block/lm_argmax alone are the page's parallel route (w2 = 0, its initialisation). Confidence pruning
(forwardRows' thresholds / minConf): a step k >= 1 whose confidence is below its threshold drops position k and ends
the block.
"""
from __future__ import annotations

import numpy as np

from . import prims as P
from .flowmap import ContextFull


class KVInjectOracle:
    def __init__(self, cfg: dict, weights: dict):
        self.cfg = cfg
        self.raw = weights
        self._w: dict[str, np.ndarray] = {}
        d, L = cfg["dim"], cfg["layers"]
        self.K = [np.zeros((cfg["max_ctx"], d)) for _ in range(L)]
        self.V = [np.zeros((cfg["max_ctx"], d)) for _ in range(L)]
        self.length = 0

    def w(self, name: str) -> np.ndarray:
        if name not in self._w:
            self._w[name] = P.weight_f64(self.raw[name])
        return self._w[name]

    def build_context(self, taps: np.ndarray) -> np.ndarray:
        """Eq 2: H_ctx = RMSNorm(W_c taps; ctx_norm)."""
        return P.rmsnorm(P.linear(taps, self.w("W_c")), self.w("ctx_norm"), self.cfg["rms_eps"])

    def context_append(self, taps: np.ndarray, start: int):
        """Retained context projection (projectContextRows): per layer K = W_k RMSNorm(H_ctx; attn_norm), V likewise,
        written at rows start .. start + n - 1."""
        cfg = self.cfg
        n = taps.shape[0]
        if start < 0 or start > self.length:
            raise ValueError("start beyond the current context length")
        # capacity: the flow-map page's extendContext rule (room for a block and one more row), taken for every
        # variant; the KV-injection page grows its arrays and states no limit
        if start + n + cfg["block"] + 1 > cfg["max_ctx"]:
            raise ContextFull("context full")
        hc = self.build_context(taps)
        for i in range(cfg["layers"]):
            nc = P.rmsnorm(hc, self.w(f"bb.{i}.attn_norm"), cfg["rms_eps"])
            self.K[i][start:start + n] = P.linear(nc, self.w(f"bb.{i}.k"))
            self.V[i][start:start + n] = P.linear(nc, self.w(f"bb.{i}.v"))
        self.length = start + n
        return hc

    def build_block(self, anchor: int) -> np.ndarray:
        """H_d[0] = tok_proj(E[anchor]) + block_pos[0]; H_d[k] = mask_emb[k-1] + block_pos[k]."""
        e = self.w("lm_head.weight")[anchor][None, :]
        bp = self.w("block_pos")
        first = P.linear(e, self.w("tok_proj")) + bp[0]
        return np.concatenate([first, self.w("mask_emb") + bp[1:]], axis=0)

    def _layer(self, i: int, hd_x: np.ndarray, kc: np.ndarray, vc: np.ndarray) -> np.ndarray:
        cfg = self.cfg
        H, hdim = cfg["heads"], cfg["head_dim"]
        n = P.rmsnorm(hd_x, self.w(f"bb.{i}.attn_norm"), cfg["rms_eps"])
        q = P.linear(n, self.w(f"bb.{i}.q"))
        keys = np.concatenate([kc, P.linear(n, self.w(f"bb.{i}.k"))], axis=0)
        vals = np.concatenate([vc, P.linear(n, self.w(f"bb.{i}.v"))], axis=0)
        a = P.attention(q, keys, vals, H, hdim ** -0.5)
        x = hd_x + P.linear(a, self.w(f"bb.{i}.o"))
        n2 = P.rmsnorm(x, self.w(f"bb.{i}.ff_norm"), cfg["rms_eps"])
        m = P.gelu_tanh(P.linear(n2, self.w(f"bb.{i}.gate"))) * P.linear(n2, self.w(f"bb.{i}.up"))
        return x + P.linear(m, self.w(f"bb.{i}.down"))

    def draft_block(self, anchor: int):
        """Block output out_proj(RMSNorm(H_d; out_norm)) [gamma, Ht] over the retained context rows [0, length)."""
        cfg = self.cfg
        x = self.build_block(anchor)
        xs = []
        for i in range(cfg["layers"]):
            x = self._layer(i, x, self.K[i][:self.length], self.V[i][:self.length])
            xs.append(x.copy())
        self.block_n = P.rmsnorm(x, self.w("out_norm"), cfg["rms_eps"])
        out = P.linear(self.block_n, self.w("out_proj"))
        return out, xs

    def draft_block_reproject(self, taps_all: np.ndarray, anchor: int) -> np.ndarray:
        """The same block with the context re-projected inside every layer from all tap rows (the page's route
        without a retained context); equal to draft_block when the cache holds exactly those rows."""
        cfg = self.cfg
        hc = self.build_context(taps_all)
        x = self.build_block(anchor)
        for i in range(cfg["layers"]):
            nc = P.rmsnorm(hc, self.w(f"bb.{i}.attn_norm"), cfg["rms_eps"])
            x = self._layer(i, x, P.linear(nc, self.w(f"bb.{i}.k")), P.linear(nc, self.w(f"bb.{i}.v")))
        return P.linear(P.rmsnorm(x, self.w("out_norm"), cfg["rms_eps"]), self.w("out_proj"))

    def lm_argmax(self, hidden: np.ndarray):
        z = P.linear(hidden, self.w("lm_head.weight"))
        return P.argmax_rows(z), z

    def markov_decode(self, block_n: np.ndarray, hidden: np.ndarray, anchor: int, follow=None, thresholds=None):
        """Greedy decode with the Markov correction and the confidence head over the rows of one block: block_n the
        normed backbone rows [gamma][dDraft], hidden = out_proj(block_n) [gamma][Ht]. follow (optional): tokens to
        condition the next step on instead of this oracle's own argmax (a device run that took the other side of a
        near-tie). thresholds (optional, gamma values): confidence pruning as DF forwardRows does it with
        thresholds / minConf -- after step k >= 1 has its token and confidence, a confidence below thresholds[k]
        drops position k and ends the block (position 0 is always kept). Returns (tokens, scores, conf) over the
        positions kept."""
        z = P.linear(hidden, self.w("lm_head.weight"))
        w1, w2 = self.w("markov.w1"), self.w("markov.w2")
        cw, cb = self.w("conf.w")[:, 0], self.w("conf.b")[0]
        prev = int(anchor)
        toks, scores, conf = [], [], []
        for k in range(z.shape[0]):
            e1 = w1[prev]
            s = z[k] + e1 @ w2
            t = int(P.argmax_rows(s[None, :])[0])
            toks.append(t)
            scores.append(s)
            conf.append(P.sigmoid(np.concatenate([block_n[k], e1]) @ cw + cb))
            if thresholds is not None and k > 0 and conf[k] < thresholds[k]:
                return np.array(toks[:k]), np.stack(scores[:k]), np.array(conf[:k])
            prev = t if follow is None else int(follow[k])
        return np.array(toks), np.stack(scores), np.array(conf)
