"""Primitive operations of the drafter, float64 (oracle; test infrastructure only).

Citations name the page and the unit on it:
  [FM]  "diskformer 0.5.4 -> 0.6.6", engines/flashmap_drafter.js
  [MTP] "diskformer 0.5.3 -> 0.6.4", engines/ternary_bonsai_2_mtp.js
  [DF]  "mlx-bun 0.4.0 -> 1.0.0", src/spec/dspark/module-dflash.ts
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import erf as _erf

# ── storage formats ─────────────────────────────────────────────────────────────────────────────


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 is the upper half of an f32 ([FM] the BF helper: the 16 bits shifted into the high half)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f16_to_f64(bits: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def q8_0_to_f64(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Q8_0: weight = d * q with one f16 scale d per 32 consecutive codes of a row ([MTP] WG_Q8: acc += s * dot)."""
    rows, K = codes.shape
    d = f16_to_f64(scales).reshape(rows, K // 32, 1)
    return (codes.astype(np.float64).reshape(rows, K // 32, 32) * d).reshape(rows, K)


def weight_f64(w) -> np.ndarray:
    """Decode any stored weight: bf16 bits, f32, or a Q8_0 (codes, scales) pair."""
    if isinstance(w, tuple):
        return q8_0_to_f64(*w)
    if w.dtype == np.uint16:
        return bf16_to_f64(w)
    return np.asarray(w, dtype=np.float64)


# ── linear algebra and norms ────────────────────────────────────────────────────────────────────


def linear(x: np.ndarray, W: np.ndarray, b: np.ndarray | None = None) -> np.ndarray:
    """y[t, m] = sum_k x[t, k] W[m, k] (+ b[m]); W stored [out][in] ([FM] gemmBf16 and gemvT: y = x Wᵀ + b)."""
    y = np.asarray(x, np.float64) @ np.asarray(W, np.float64).T
    if b is not None:
        y = y + b
    return y


def rmsnorm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """x * w / sqrt(mean(x^2) + eps) over the last axis ([FM] rmsRows; [MTP] WG_NORM)."""
    x = np.asarray(x, np.float64)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return x * r * w


def layernorm(x: np.ndarray, eps: float) -> np.ndarray:
    """(x - mean) / sqrt(var + eps), biased variance, no affine ([FM] lnMod, its two reductions)."""
    x = np.asarray(x, np.float64)
    mu = np.mean(x, axis=-1, keepdims=True)
    d = x - mu
    var = np.mean(d * d, axis=-1, keepdims=True)
    return d / np.sqrt(var + eps)


def ln_mod(x: np.ndarray, scale: np.ndarray, shift: np.ndarray, eps: float) -> np.ndarray:
    """adaLN modulation LN(x) (1 + scale) + shift ([FM] lnMod; the file header's DiT layer)."""
    return layernorm(x, eps) * (1.0 + scale) + shift


def head_rmsnorm(x: np.ndarray, heads: int, w: np.ndarray, eps: float) -> np.ndarray:
    """Per-head RMSNorm over the head dimension of rows [..., heads * hd] ([FM] headNormRope, first half)."""
    s = x.shape
    xh = np.asarray(x, np.float64).reshape(s[:-1] + (heads, s[-1] // heads))
    return rmsnorm(xh, w, eps).reshape(s)


# ── rotary position embedding ───────────────────────────────────────────────────────────────────


def rope_interleaved(x: np.ndarray, pos: np.ndarray, heads: int, theta: float) -> np.ndarray:
    """Rotate channel pairs (2i, 2i+1) of every head by angle pos * theta^(-2i/hd):
    x'_2i = x_2i cos a - x_2i+1 sin a;  x'_2i+1 = x_2i+1 cos a + x_2i sin a  ([FM] headNormRope and ropeRows).
    Angles are exact in float64.  x: [rows, heads * hd]; pos: [rows]."""
    rows, width = x.shape
    hd = width // heads
    xh = np.asarray(x, np.float64).reshape(rows, heads, hd // 2, 2)
    i = np.arange(hd // 2, dtype=np.float64)
    inv = theta ** (-2.0 * i / hd)
    a = np.asarray(pos, np.float64)[:, None] * inv[None, :]          # [rows, hd/2]
    c = np.cos(a)[:, None, :]
    s = np.sin(a)[:, None, :]
    x0, x1 = xh[..., 0], xh[..., 1]
    out = np.empty_like(xh)
    out[..., 0] = x0 * c - x1 * s
    out[..., 1] = x1 * c + x0 * s
    return out.reshape(rows, width)


def rope_neox_partial(x: np.ndarray, pos: np.ndarray, heads: int, rot: int, theta: float) -> np.ndarray:
    """NEOX RoPE on the first `rot` dims of every head: pairs (i, i + rot/2) for i < rot/2, angle
    pos * theta^(-2i/rot); dims >= rot pass through ([MTP] WG_QKPREP).  x: [rows, heads * hd]; pos: [rows]."""
    rows, width = x.shape
    hd = width // heads
    half = rot // 2
    xh = np.asarray(x, np.float64).reshape(rows, heads, hd).copy()
    i = np.arange(half, dtype=np.float64)
    a = np.asarray(pos, np.float64)[:, None] * theta ** (-2.0 * i / rot)[None, :]
    c = np.cos(a)[:, None, :]
    s = np.sin(a)[:, None, :]
    lo = xh[:, :, :half].copy()
    hi = xh[:, :, half:rot].copy()
    xh[:, :, :half] = lo * c - hi * s
    xh[:, :, half:rot] = hi * c + lo * s
    return xh.reshape(rows, width)


# ── attention ───────────────────────────────────────────────────────────────────────────────────


def softmax(s: np.ndarray, axis: int = -1) -> np.ndarray:
    m = np.max(s, axis=axis, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=axis, keepdims=True)


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, heads: int, scale: float,
              mask: np.ndarray | None = None, kv_heads: int | None = None) -> np.ndarray:
    """softmax(q kᵀ scale [+ mask]) v per head, with max subtraction ([FM] attn; [MTP] WG_ATTN; [DF] sdpa).
    q: [Tq, heads*hd]; k, v: [L, kv_heads*hd]; query head h reads kv head h // (heads // kv_heads) (grouped-query,
    [MTP] WG_ATTN kvh = h / 6).  mask: additive [Tq, L] (use -inf for excluded keys)."""
    kv_heads = kv_heads or heads
    Tq = q.shape[0]
    L = k.shape[0]
    hd = q.shape[1] // heads
    qh = np.asarray(q, np.float64).reshape(Tq, heads, hd).transpose(1, 0, 2)
    kh = np.asarray(k, np.float64).reshape(L, kv_heads, hd).transpose(1, 0, 2)
    vh = np.asarray(v, np.float64).reshape(L, kv_heads, hd).transpose(1, 0, 2)
    g = heads // kv_heads
    kh = np.repeat(kh, g, axis=0)
    vh = np.repeat(vh, g, axis=0)
    s = np.einsum("htd,hld->htl", qh, kh) * scale
    if mask is not None:
        s = s + mask[None]
    p = softmax(s, axis=-1)
    o = np.einsum("htl,hld->htd", p, vh)
    return o.transpose(1, 0, 2).reshape(Tq, heads * hd)


# ── activations ─────────────────────────────────────────────────────────────────────────────────


def gelu_erf(x: np.ndarray) -> np.ndarray:
    """Exact GELU x * Phi(x) = x/2 (1 + erf(x / sqrt 2)) ([FM] gelu, which approximates erf)."""
    x = np.asarray(x, np.float64)
    return 0.5 * x * (1.0 + _erf(x / math.sqrt(2.0)))


def gelu_tanh(x: np.ndarray) -> np.ndarray:
    """tanh-approximate GELU x/2 (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))) (Hendrycks & Gimpel 2016), the reading of
    the activation [DF] calls geluApprox."""
    x = np.asarray(x, np.float64)
    return 0.5 * x * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (x + 0.044715 * x ** 3)))


def sigmoid(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, np.float64)
    return 1.0 / (1.0 + np.exp(-x))


def silu(x: np.ndarray) -> np.ndarray:
    """x * sigmoid(x) ([MTP] WG_SILU_MUL)."""
    return np.asarray(x, np.float64) * sigmoid(x)


def argmax_rows(z: np.ndarray) -> np.ndarray:
    """Per-row argmax, lowest index among equal maxima (numpy's argmax returns the first)."""
    return np.argmax(np.asarray(z), axis=-1).astype(np.int64)


def top2_gap(z: np.ndarray) -> np.ndarray:
    """Per row: largest minus second-largest value."""
    part = np.partition(np.asarray(z, np.float64), -2, axis=-1)
    return part[..., -1] - part[..., -2]
