"""Flow-map (FlashMap) block drafter, float64 oracle (test infrastructure only).

Follows page "diskformer 0.5.4 -> 0.6.6", engines/flashmap_drafter.js: the file header (the method in prose),
FlashMapDrafter.extendContext (context append), FlashMapDrafter.draft (anchor slot, the 16-slot jump, head,
lm_head + argmax) and the WGSL kernels those call (rmsRows, lnMod, headNormRope, attn, gelu, gateAdd, broadcast,
colMeanQ8).

Readings taken where the page leaves a step open:
  * biases exist on anchor_proj, x_embed, fc1, fc2 and head only (the page passes bias=false for q/k/v/o and fc);
  * the token table E (anchor embedding, mean row) is the bf16 lm_head table itself (tied);
  * cross-attention keys are cache rows [0, pos], the anchor slot at pos included (L = pos + 1);
  * self-attention is unmasked over the T slots; slot s sits at position pos + 1 + s;
  * RoPE angles are exact (float64), caches are float64.

Time conditioning (timeConditioning, the page's FlashMapDraftModel.time_conditioning): the modulation table of a
jump s -> t from the time MLPs. A time is embedded sinusoidally (frequencies and angles rounded to f32 as the page
does, cos and sin of those angles), passed through linear_1, SiLU, linear_2 of time_embed (for s) or jump_embed
(for t); cond = SiLU(sum of the two); each norm's [scale | shift | gate] is its adaLN linear of cond.
"""
from __future__ import annotations

import numpy as np

from . import prims as P


class ContextFull(Exception):
    pass


class FlowMapOracle:
    def __init__(self, cfg: dict, weights: dict):
        self.cfg = cfg
        self.raw = weights
        self._w: dict[str, np.ndarray] = {}
        D, L = cfg["dim"], cfg["layers"]
        self.K = [np.zeros((cfg["max_ctx"], D)) for _ in range(L)]
        self.V = [np.zeros((cfg["max_ctx"], D)) for _ in range(L)]
        self.length = 0
        self._h0 = None

    # decoded (float64) weights, cached on first use
    def w(self, name: str) -> np.ndarray:
        if name not in self._w:
            self._w[name] = P.weight_f64(self.raw[name])
        return self._w[name]

    def lw(self, l: int, name: str) -> np.ndarray:
        return self.w(f"layers.{l}.{name}")

    def time_conditioning(self, s: float, t: float) -> np.ndarray:
        """The [(3 layers + 1) * 3 D] modulation table of the jump s -> t (norm order per layer: self, cross, mlp;
        then the final norm), float64 arithmetic after the page's f32 angles."""
        cfg = self.cfg
        half = cfg["time_dim"] // 2

        def embed(prefix, time):
            i = np.arange(half, dtype=np.float64)
            f = np.exp(-np.log(10000.0) * i / half).astype(np.float32)
            a = (np.float32(np.float32(time) * np.float32(cfg["time_scale"])) * f).astype(np.float64)
            e = np.concatenate([np.cos(a), np.sin(a)])
            h = P.silu(P.linear(e[None, :], self.w(f"{prefix}.linear_1.weight"), self.w(f"{prefix}.linear_1.bias")))
            return P.linear(h, self.w(f"{prefix}.linear_2.weight"), self.w(f"{prefix}.linear_2.bias"))[0]

        cond = P.silu(embed("time_embed", s) + embed("jump_embed", t))
        rows = [f"layers.{l}.{n}_adaln.linear" for l in range(cfg["layers"]) for n in ("self_attn", "cross_attn", "mlp")]
        rows.append("final_adaln.linear")
        return np.concatenate([P.linear(cond[None, :], self.w(f"{r}.weight"), self.w(f"{r}.bias"))[0] for r in rows])

    def use_table(self, table: np.ndarray):
        """Draft with this modulation table instead of the stored one."""
        self._w["mod"] = np.asarray(table, np.float64)

    def mod(self, n: int):
        """Row n of the modulation table: (scale, shift, gate), each [D] (norm order per layer: self, cross, mlp;
        then the final norm)."""
        D = self.cfg["dim"]
        m = self.w("mod")[n * 3 * D:(n + 1) * 3 * D]
        return m[:D], m[D:2 * D], m[2 * D:3 * D]

    # ── context ────────────────────────────────────────────────────────────────────────────────
    def _cache_rows(self, c: np.ndarray, start: int):
        """K/V of normalised context rows c written at positions start .. start + n - 1 of every layer:
        K = RoPE(headRMSNorm(c W_kᵀ)), V = c W_vᵀ."""
        cfg = self.cfg
        n = c.shape[0]
        pos = np.arange(start, start + n)
        for l in range(cfg["layers"]):
            k = P.linear(c, self.lw(l, "cross_attn.k_proj.weight"))
            k = P.head_rmsnorm(k, cfg["heads"], self.lw(l, "cross_attn.k_norm.weight"), cfg["qk_eps"])
            k = P.rope_interleaved(k, pos, cfg["heads"], cfg["rope_theta"])
            self.K[l][start:start + n] = k
            self.V[l][start:start + n] = P.linear(c, self.lw(l, "cross_attn.v_proj.weight"))

    def context_append(self, taps: np.ndarray, start: int):
        """Append n tapped feature rows as positions start .. start+n-1: c = RMSNorm(fc(taps)), then every layer's
        cross-attention K/V.  Any start <= length may be rewritten; length becomes start + n."""
        cfg = self.cfg
        n = taps.shape[0]
        if start < 0 or start > self.length:
            raise ValueError("start beyond the current context length")
        if start + n + cfg["block"] + 1 > cfg["max_ctx"]:
            raise ContextFull("context full")
        c = P.rmsnorm(P.linear(taps, self.w("fc.weight")), self.w("hidden_norm.weight"), cfg["rms_eps"])
        self._cache_rows(c, start)
        self.length = start + n
        return c

    # ── the zero-noise slot input ──────────────────────────────────────────────────────────────
    def h0(self) -> np.ndarray:
        """x_embed(state_norm(uniform_embeds)) + b, uniform_embeds = the mean row of E (computed once)."""
        if self._h0 is None:
            cfg = self.cfg
            E = self.w("lm_head.weight")
            u = E.mean(axis=0)
            s = P.rmsnorm(u[None, :], self.w("state_norm.weight"), cfg["rms_eps"])
            self._h0 = P.linear(s, self.w("x_embed.weight"), self.w("x_embed.bias"))[0]
        return self._h0

    # ── the draft ──────────────────────────────────────────────────────────────────────────────
    def anchor_slot(self, anchor: int, pos: int) -> np.ndarray:
        """The anchor's context slot: anchor_norm(anchor_proj(E[anchor])) through every layer's k/v path at pos."""
        cfg = self.cfg
        e = self.w("lm_head.weight")[anchor][None, :]
        c = P.rmsnorm(P.linear(e, self.w("anchor_proj.weight"), self.w("anchor_proj.bias")),
                      self.w("anchor_norm.weight"), cfg["rms_eps"])
        self._cache_rows(c, pos)
        return c

    def draft_block(self, anchor: int, pos: int, rope: bool = True, slot_pos: np.ndarray | None = None):
        """The T draft slots after `anchor`, which sits at context position pos.  Returns (out [T, Ht], xs) where xs
        holds the residual stream after each layer.  `rope=False` and `slot_pos` exist for the invariance tests."""
        cfg = self.cfg
        T, D, H, hd = cfg["block"], cfg["dim"], cfg["heads"], cfg["head_dim"]
        if pos < 0 or pos > self.length:
            raise ValueError("pos beyond the current context length")
        if pos + T + 1 > cfg["max_ctx"]:
            raise ContextFull("context full")
        self.anchor_slot(anchor, pos)
        x = np.tile(self.h0()[None, :], (T, 1))
        sp = np.arange(pos + 1, pos + 1 + T) if slot_pos is None else np.asarray(slot_pos)
        th = cfg["rope_theta"]
        rot = (lambda a, p: P.rope_interleaved(a, p, H, th)) if rope else (lambda a, p: a)
        scale = 1.0 / np.sqrt(hd)
        xs = []
        for l in range(cfg["layers"]):
            # self-attention over the T slots, no mask
            sc, sh, g = self.mod(3 * l)
            h = P.ln_mod(x, sc, sh, cfg["ln_eps"])
            q = rot(P.head_rmsnorm(P.linear(h, self.lw(l, "self_attn.q_proj.weight")), H,
                                   self.lw(l, "self_attn.q_norm.weight"), cfg["qk_eps"]), sp)
            k = rot(P.head_rmsnorm(P.linear(h, self.lw(l, "self_attn.k_proj.weight")), H,
                                   self.lw(l, "self_attn.k_norm.weight"), cfg["qk_eps"]), sp)
            v = P.linear(h, self.lw(l, "self_attn.v_proj.weight"))
            o = P.attention(q, k, v, H, scale)
            x = x + g * P.linear(o, self.lw(l, "self_attn.o_proj.weight"))
            # cross-attention over the cached context rows [0, pos]
            sc, sh, g = self.mod(3 * l + 1)
            h = P.ln_mod(x, sc, sh, cfg["ln_eps"])
            q = rot(P.head_rmsnorm(P.linear(h, self.lw(l, "cross_attn.q_proj.weight")), H,
                                   self.lw(l, "cross_attn.q_norm.weight"), cfg["qk_eps"]), sp)
            o = P.attention(q, self.K[l][:pos + 1], self.V[l][:pos + 1], H, scale)
            x = x + g * P.linear(o, self.lw(l, "cross_attn.o_proj.weight"))
            # MLP: fc1, exact GELU, fc2
            sc, sh, g = self.mod(3 * l + 2)
            h = P.ln_mod(x, sc, sh, cfg["ln_eps"])
            u = P.gelu_erf(P.linear(h, self.lw(l, "mlp.fc1.weight"), self.lw(l, "mlp.fc1.bias")))
            x = x + g * P.linear(u, self.lw(l, "mlp.fc2.weight"), self.lw(l, "mlp.fc2.bias"))
            xs.append(x.copy())
        sc, sh, _ = self.mod(3 * cfg["layers"])
        out = P.linear(P.ln_mod(x, sc, sh, cfg["ln_eps"]), self.w("head.weight"), self.w("head.bias"))
        return out, xs

    def lm_argmax(self, hidden: np.ndarray):
        """Logits z = hidden Eᵀ over the bf16 lm_head table, and the per-row argmax (lowest index on ties)."""
        z = P.linear(hidden, self.w("lm_head.weight"))
        return P.argmax_rows(z), z
