"""Seeded synthetic inputs for every drafter shape: weights, tables, taps, anchors, schedules.

This module holds no arithmetic of the drafter itself.  It only draws random
numbers and stores them in the formats the weights travel in:

* bf16 (round to nearest even from f32), weights ~ N(0, 0.02), norm weights 1 + N(0, 0.01);
* f32 for activations (taps, hidden rows) and for the flow-map modulation table;
* Q8_0: per 32-element block an f16 scale d = f16(max|w| / 127) and int8 codes
  q = rint(w / d), the GGML block layout (page "diskformer 0.5.3 -> 0.6.4",
  MTPHead.loadWeights) split into a code array [rows][K] and a scale array [rows][K/32].

Every tensor has its own stream: numpy's PCG64 seeded with SeedSequence(seed, spawn_key=(crc32(name),)),
drawn in fixed chunks of 2**22 values, so a tensor's values do not depend on which other tensors are drawn
or in which order.  Both the oracle and the GPU binding read these arrays; neither generates its own.
"""
from __future__ import annotations

import zlib

import numpy as np

CHUNK = 1 << 22


def _rng(seed: int, name: str) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(entropy=seed, spawn_key=(zlib.crc32(name.encode()),)))


def normal_f32(seed: int, name: str, n: int, std: float = 1.0, mean: float = 0.0) -> np.ndarray:
    """n values of N(mean, std^2) as float32, from the tensor's own stream."""
    g = _rng(seed, name)
    out = np.empty(n, dtype=np.float32)
    for i in range(0, n, CHUNK):
        m = min(CHUNK, n - i)
        out[i:i + m] = g.standard_normal(m, dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    if mean != 0.0:
        out += np.float32(mean)
    return out


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns the 16-bit patterns as uint16."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u >> 16) & 1
    return ((u + np.uint32(0x7FFF) + r) >> 16).astype(np.uint16)


def bf16_weight(seed: int, name: str, shape, std: float = 0.02, mean: float = 0.0) -> np.ndarray:
    n = int(np.prod(shape))
    return f32_to_bf16_bits(normal_f32(seed, name, n, std, mean)).reshape(shape)


def q8_0_weight(seed: int, name: str, rows: int, cols: int, std: float = 0.02):
    """Q8_0 codes (int8 [rows, cols]) and scales (f16 bits as uint16 [rows, cols/32]) of N(0, std) weights."""
    assert cols % 32 == 0
    q = np.empty((rows, cols), dtype=np.int8)
    d = np.empty((rows, cols // 32), dtype=np.uint16)
    g = _rng(seed, name)
    step = max(1, CHUNK // cols)
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        w = g.standard_normal((r1 - r0) * cols, dtype=np.float32).reshape(r1 - r0, cols // 32, 32)
        w *= np.float32(std)
        amax = np.abs(w).max(axis=2)
        dh = (amax / np.float32(127.0)).astype(np.float16)
        df = dh.astype(np.float32)
        inv = np.where(df > 0, 1.0 / np.where(df > 0, df, 1), 0).astype(np.float32)
        qq = np.clip(np.rint(w * inv[:, :, None]), -127, 127).astype(np.int8)
        q[r0:r1] = qq.reshape(r1 - r0, cols)
        d[r0:r1] = dh.view(np.uint16)
    return q, d


# ── weight lists per variant ────────────────────────────────────────────────────────────────────

def flowmap_weight_specs(cfg: dict):
    """(name, shape, kind) for the flow-map drafter; kinds: w (bf16 N(0,.02)), b (bf16 bias N(0,.02)),
    n (bf16 norm weight 1+N(0,.01)), mod (f32 modulation table). Weights are [out][in]."""
    D, Ht, F, hd, L = cfg["dim"], cfg["target_dim"], cfg["ffn"], cfg["head_dim"], cfg["layers"]
    s = [("fc.weight", (D, cfg["n_taps"] * Ht), "w"), ("hidden_norm.weight", (D,), "n"),
         ("anchor_proj.weight", (D, Ht), "w"), ("anchor_proj.bias", (D,), "b"), ("anchor_norm.weight", (D,), "n"),
         ("state_norm.weight", (Ht,), "n"), ("x_embed.weight", (D, Ht), "w"), ("x_embed.bias", (D,), "b")]
    for l in range(L):
        for br in ("self_attn", "cross_attn"):
            for p in ("q", "k", "v", "o"):
                s.append((f"layers.{l}.{br}.{p}_proj.weight", (D, D), "w"))
            s.append((f"layers.{l}.{br}.q_norm.weight", (hd,), "n"))
            s.append((f"layers.{l}.{br}.k_norm.weight", (hd,), "n"))
        s += [(f"layers.{l}.mlp.fc1.weight", (F, D), "w"), (f"layers.{l}.mlp.fc1.bias", (F,), "b"),
              (f"layers.{l}.mlp.fc2.weight", (D, F), "w"), (f"layers.{l}.mlp.fc2.bias", (D,), "b")]
    s += [("head.weight", (Ht, D), "w"), ("head.bias", (Ht,), "b"),
          ("lm_head.weight", (cfg["vocab"], Ht), "w"), ("mod", ((3 * L + 1) * 3 * D,), "mod")]
    td, cd = cfg.get("time_dim", 0), cfg.get("cond_dim", 0)
    if td:
        # time conditioning (the page's timeConditioning): two time MLPs [cond x time_dim], [cond x cond] and one
        # adaLN linear [3 D x cond] per norm, all with biases
        for pre in ("time_embed", "jump_embed"):
            s += [(f"{pre}.linear_1.weight", (cd, td), "w"), (f"{pre}.linear_1.bias", (cd,), "b"),
                  (f"{pre}.linear_2.weight", (cd, cd), "w"), (f"{pre}.linear_2.bias", (cd,), "b")]
        for l in range(L):
            for n in ("self_attn", "cross_attn", "mlp"):
                s += [(f"layers.{l}.{n}_adaln.linear.weight", (3 * D, cd), "w"),
                      (f"layers.{l}.{n}_adaln.linear.bias", (3 * D,), "b")]
        s += [("final_adaln.linear.weight", (3 * D, cd), "w"), ("final_adaln.linear.bias", (3 * D,), "b")]
    return s


def kvinject_weight_specs(cfg: dict):
    """Parameter list of the KV-injection drafter (module-dflash.ts buildNames, minus the Markov / confidence /
    RNN heads), stored [out][in]."""
    d, Ht, F, L, g = cfg["dim"], cfg["target_dim"], cfg["ffn"], cfg["layers"], cfg["block"]
    s = []
    for i in range(L):
        s.append((f"bb.{i}.attn_norm", (d,), "n"))
        for p in ("q", "k", "v", "o"):
            s.append((f"bb.{i}.{p}", (d, d), "w"))
        s += [(f"bb.{i}.ff_norm", (d,), "n"), (f"bb.{i}.gate", (F, d), "w"), (f"bb.{i}.up", (F, d), "w"),
              (f"bb.{i}.down", (d, F), "w")]
    s += [("W_c", (d, cfg["n_taps"] * Ht), "w"), ("ctx_norm", (d,), "n"), ("tok_proj", (d, Ht), "w"),
          ("mask_emb", (g - 1, d), "w"), ("block_pos", (g, d), "w"), ("out_norm", (d,), "n"),
          ("out_proj", (Ht, d), "w"), ("lm_head.weight", (cfg["vocab"], Ht), "w")]
    r = cfg.get("markov_rank", 0)
    if r:
        # DSpark Markov head and confidence head in the page's own layouts: w1 [V][r] (rows gathered by token),
        # w2 [r][V] (bias = e1 w2), conf.w [(dDraft + r)][1], conf.b [1]. The page zero-initialises w2 and conf.w
        # (a pure parallel drafter at init); the synthetic set draws them N(0, .02) so that both heads act.
        s += [("markov.w1", (cfg["vocab"], r), "w"), ("markov.w2", (r, cfg["vocab"]), "w"),
              ("conf.w", (d + r, 1), "w"), ("conf.b", (1,), "b")]
    return s


def mtp_weight_specs(cfg: dict):
    """The MTP head's tensors (ternary_bonsai_2_mtp.js MTP_HEAD) with their [N][K] shapes; kinds q8 (Q8_0
    matrix) and nf (f32 norm weight 1+N(0,.01)). lm_head is the Q8_0 [vocab][H] table."""
    H, I, NH, NKV, HD = cfg["dim"], cfg["ffn"], cfg["heads"], cfg["kv_heads"], cfg["head_dim"]
    return [("eh_proj", (H, 2 * H), "q8"), ("attn_norm", (H,), "nf"), ("attn_q", (NH * 2 * HD, H), "q8"),
            ("attn_k", (NKV * HD, H), "q8"), ("attn_v", (NKV * HD, H), "q8"), ("attn_q_norm", (HD,), "nf"),
            ("attn_k_norm", (HD,), "nf"), ("attn_output", (H, NH * HD), "q8"), ("post_attention_norm", (H,), "nf"),
            ("ffn_gate", (I, H), "q8"), ("ffn_up", (I, H), "q8"), ("ffn_down", (H, I), "q8"),
            ("shared_head_norm", (H,), "nf"), ("enorm", (H,), "nf"), ("hnorm", (H,), "nf"),
            ("lm_head", (cfg["vocab"], H), "q8")]


def weight_specs(cfg: dict):
    return {"flowmap": flowmap_weight_specs, "kvinject": kvinject_weight_specs,
            "mtp": mtp_weight_specs}[cfg["variant"]](cfg)


def make_tensor(cfg: dict, name: str, shape, kind: str, seed: int = 0):
    """One tensor of a drafter, in its storage format:
    bf16 bits (uint16), f32, or a (codes int8, scales f16-bits) pair for Q8_0."""
    if kind == "w" or kind == "b":
        return bf16_weight(seed, name, shape, 0.02)
    if kind == "n":
        return bf16_weight(seed, name, shape, 0.01, 1.0)
    if kind == "nf":
        return normal_f32(seed, name, int(np.prod(shape)), 0.01, 1.0).reshape(shape)
    if kind == "mod":
        # Per norm [scale D | shift D | gate D]: scale, shift ~ N(0, .02); gate ~ 1 + N(0, .01).
        D = cfg["dim"]
        n_norm = shape[0] // (3 * D)
        t = normal_f32(seed, name, shape[0], 0.02).reshape(n_norm, 3, D)
        t[:, 2, :] = normal_f32(seed, name + ".gate", n_norm * D, 0.01, 1.0).reshape(n_norm, D)
        return t.reshape(shape)
    if kind == "q8":
        return q8_0_weight(seed, name, shape[0], shape[1])
    raise ValueError(kind)


def make_weights(cfg: dict, seed: int = 0, skip=()) -> dict:
    """Every tensor of the drafter `cfg` (name -> array, or (codes, scales) for Q8_0)."""
    return {name: make_tensor(cfg, name, shape, kind, seed)
            for name, shape, kind in weight_specs(cfg) if name not in skip}


# ── activations and schedules ───────────────────────────────────────────────────────────────────

def taps(cfg: dict, key: str, n: int, seed: int = 0) -> np.ndarray:
    """n context rows of tapped target features [n, n_taps * target_dim], f32 N(0, 1)."""
    w = cfg["n_taps"] * cfg["target_dim"]
    return normal_f32(seed, f"taps/{key}", n * w).reshape(n, w)


def anchors(cfg: dict, key: str, n: int, seed: int = 0) -> np.ndarray:
    """n anchor token ids, uniform over the vocabulary."""
    g = _rng(seed, f"anchors/{key}")
    return g.integers(0, cfg["vocab"], size=n, dtype=np.int64).astype(np.int32)


def longctx_schedule(cfg: dict, seed: int = 0):
    """Draft / append schedule of the long-context workload: after the prefill of ctx_rows rows, step s drafts at
    pos_s with anchor a_s, then appends n_s ~ U{1..16} rows at start pos_s; pos_{s+1} = pos_s + n_s."""
    steps = cfg.get("draft_steps", 64)
    g = _rng(seed, "longctx/schedule")
    ns = g.integers(1, 17, size=steps)
    an = g.integers(0, cfg["vocab"], size=steps)
    pos = cfg["ctx_rows"]
    out = []
    for s in range(steps):
        out.append((int(an[s]), int(pos), int(ns[s])))
        pos += int(ns[s])
    return out


def mtp_inputs(cfg: dict, M: int, key: str = "mtp", seed: int = 0):
    """Inputs of one MTP pass over M rows: embedding rows e [M, H] (f32 N(0, .02), the scale of a token table) and
    normed trunk rows h [M, H] (f32 N(0, 1))."""
    H = cfg["dim"]
    e = normal_f32(seed, f"{key}/e{M}", M * H, 0.02).reshape(M, H)
    h = normal_f32(seed, f"{key}/h{M}", M * H).reshape(M, H)
    return e, h


def mtp_cache_rows(cfg: dict, rows: int, seed: int = 0):
    """Synthetic K and V cache contents for positions [0, rows): f32 N(0, 1), [rows, kv_heads * head_dim]."""
    w = cfg["kv_heads"] * cfg["head_dim"]
    return (normal_f32(seed, "mtp/kcache", rows * w).reshape(rows, w),
            normal_f32(seed, "mtp/vcache", rows * w).reshape(rows, w))
