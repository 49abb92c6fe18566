"""Pins of the oracle's primitive operations against closed forms, textbook identities and the pages' bounds.

Each test states what fixes the expected value (never the oracle itself).
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import prims as P
from oracle import loops
from inputs import gen

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")))
rng = np.random.default_rng(1234)


# ── storage formats ─────────────────────────────────────────────────────────────────────────────

def test_bf16_decode_known_patterns():
    # IEEE bit patterns: bf16 0x3F80 is 1.0, 0xC000 is -2.0, 0x0001 is the smallest subnormal 2^-133.
    v = P.bf16_to_f64(np.array([0x3F80, 0xC000, 0x0001, 0x4049], dtype=np.uint16))
    assert v[0] == 1.0 and v[1] == -2.0 and v[2] == 2.0 ** -133
    assert v[3] == 3.140625  # 0x4049 = 1.5703125 * 2


def test_bf16_encode_rounds_to_nearest_even():
    # 1 + 2^-8 lies halfway between bf16 neighbours 1 and 1 + 2^-7: ties go to the even one (1.0).
    x = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -9], dtype=np.float32)
    back = P.bf16_to_f64(gen.f32_to_bf16_bits(x))
    assert back[0] == 1.0 and back[1] == 1 + 2 ** -6 and back[2] == 1.0


def test_f16_decode_known_patterns():
    v = P.f16_to_f64(np.array([0x3C00, 0x0001, 0xC400], dtype=np.uint16))
    assert v[0] == 1.0 and v[1] == 2.0 ** -24 and v[2] == -4.0


def test_q8_0_decode_blockwise_loop_and_roundtrip():
    q, d = gen.q8_0_weight(0, "pin/q8", 3, 96)
    w = P.q8_0_to_f64(q, d)
    # element by element: w[r, k] = d[r, k // 32] * q[r, k]
    for r in range(3):
        for k in range(0, 96, 7):
            dd = float(np.frombuffer(np.uint16(d[r, k // 32]).tobytes(), np.float16)[0])
            assert w[r, k] == dd * float(q[r, k])
    # encoding error of the generator's recipe: |w_true - d q| <= d / 2 (plus the f16 rounding of d)
    g = np.random.default_rng(np.random.SeedSequence(entropy=0, spawn_key=(__import__("zlib").crc32(b"pin/q8"),)))
    wt = g.standard_normal(3 * 96, dtype=np.float32).reshape(3, 3, 32) * np.float32(0.02)
    dd = P.f16_to_f64(d).reshape(3, 3, 1)
    err = np.abs(wt.astype(np.float64) - w.reshape(3, 3, 32))
    assert np.all(err <= dd / 2 * (1 + 2 ** -10) + 1e-12)


# ── linear ──────────────────────────────────────────────────────────────────────────────────────

def test_linear_matches_triple_loop_and_orientation():
    x = rng.standard_normal((3, 5))
    W = rng.standard_normal((7, 5))
    b = rng.standard_normal(7)
    y = P.linear(x, W, b)
    ref = loops.lin(x.tolist(), W.tolist(), b.tolist())
    assert np.allclose(y, ref, rtol=1e-13, atol=1e-13)
    # identity weight copies the input; W stored [out][in]
    assert np.array_equal(P.linear(x, np.eye(5)), x)
    e = np.zeros((1, 5)); e[0, 2] = 1.0
    assert np.array_equal(P.linear(e, W)[0], W[:, 2])


# ── norms ───────────────────────────────────────────────────────────────────────────────────────

def test_rmsnorm_closed_form():
    x = rng.standard_normal((4, 64)) * 3.0
    y = P.rmsnorm(x, np.ones(64), 0.0)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=1)), 1.0, atol=1e-14)
    assert np.allclose(P.rmsnorm(5.0 * x, np.ones(64), 0.0), y, atol=1e-13)        # scale invariance
    w = rng.standard_normal(64)
    assert np.allclose(P.rmsnorm(x, w, 0.0), y * w, atol=1e-13)                    # weight multiplies after
    # with eps: rms of the output is sqrt(ms / (ms + eps))
    ms = np.mean(x * x, axis=1)
    y2 = P.rmsnorm(x, np.ones(64), 0.5)
    assert np.allclose(np.mean(y2 * y2, axis=1), ms / (ms + 0.5), atol=1e-13)


def test_layernorm_closed_form():
    x = rng.standard_normal((5, 48)) * 2.0 + 3.0
    eps = 0.25
    y = P.layernorm(x, eps)
    var = x.var(axis=1)
    assert np.allclose(y.mean(axis=1), 0.0, atol=1e-14)
    assert np.allclose(y.var(axis=1), var / (var + eps), atol=1e-13)
    assert np.allclose(P.layernorm(x + 7.0, eps), y, atol=1e-12)                     # shift invariance
    s, b = rng.standard_normal(48), rng.standard_normal(48)
    assert np.allclose(P.ln_mod(x, s, b, eps), y * (1 + s) + b, atol=1e-13)
    assert np.allclose(P.ln_mod(x, np.zeros(48), np.zeros(48), eps), y)


def test_head_rmsnorm_is_per_head():
    x = rng.standard_normal((2, 24))
    w = rng.standard_normal(8)
    y = P.head_rmsnorm(x, 3, w, 1e-5)
    for h in range(3):
        assert np.allclose(y[:, 8 * h:8 * h + 8], P.rmsnorm(x[:, 8 * h:8 * h + 8], w, 1e-5))


# ── RoPE ────────────────────────────────────────────────────────────────────────────────────────

def test_rope_interleaved_equals_complex_rotation():
    # A pair (x_2i, x_2i+1) read as the complex number x_2i + i x_2i+1 is multiplied by e^{i p w_i},
    # w_i = theta^(-2i/hd): the textbook form of a counter-clockwise plane rotation.
    heads, hd, theta = 2, 8, 10000.0
    x = rng.standard_normal((3, heads * hd))
    pos = np.array([0, 5, 1234])
    y = P.rope_interleaved(x, pos, heads, theta)
    z = x.reshape(3, heads, hd // 2, 2)
    zc = z[..., 0] + 1j * z[..., 1]
    w = theta ** (-np.arange(hd // 2) * 2.0 / hd)
    zc = zc * np.exp(1j * pos[:, None, None] * w[None, None, :])
    ref = np.stack([zc.real, zc.imag], axis=-1).reshape(3, heads * hd)
    assert np.allclose(y, ref, atol=1e-13)
    assert np.array_equal(y[0], x[0])                                                # p = 0 is the identity


def test_rope_norm_and_relative_offset():
    heads, hd = 4, 16
    q = rng.standard_normal((1, heads * hd))
    k = rng.standard_normal((1, heads * hd))
    for p in (0, 3, 4097, 9216):
        y = P.rope_interleaved(q, np.array([p]), heads, 1e4)
        for h in range(heads):
            assert math.isclose(np.linalg.norm(y[0, h * hd:(h + 1) * hd]), np.linalg.norm(q[0, h * hd:(h + 1) * hd]),
                                rel_tol=1e-13)
    # <RoPE_p q, RoPE_r k> per head depends only on p - r
    def dots(p, r):
        a = P.rope_interleaved(q, np.array([p]), heads, 1e4).reshape(heads, hd)
        b = P.rope_interleaved(k, np.array([r]), heads, 1e4).reshape(heads, hd)
        return np.sum(a * b, axis=1)
    assert np.allclose(dots(10, 3), dots(1010, 1003), atol=1e-11)
    assert np.allclose(dots(8200, 8192), dots(8, 0), atol=1e-10)


def test_rope_neox_partial_equals_complex_rotation_and_passes_tail():
    heads, hd, rot, theta = 3, 16, 8, 1e7
    x = rng.standard_normal((2, heads * hd))
    pos = np.array([7, 4095])
    y = P.rope_neox_partial(x, pos, heads, rot, theta)
    xh = x.reshape(2, heads, hd)
    yh = y.reshape(2, heads, hd)
    assert np.array_equal(yh[:, :, rot:], xh[:, :, rot:])                           # dims >= rot untouched
    zc = xh[:, :, :rot // 2] + 1j * xh[:, :, rot // 2:rot]
    w = theta ** (-np.arange(rot // 2) * 2.0 / rot)
    zc = zc * np.exp(1j * pos[:, None, None] * w[None, None, :])
    assert np.allclose(yh[:, :, :rot // 2], zc.real, atol=1e-12)
    assert np.allclose(yh[:, :, rot // 2:rot], zc.imag, atol=1e-12)


def test_rope_loops_agree():
    x = rng.standard_normal((1, 16))
    assert np.allclose(P.rope_interleaved(x, np.array([9]), 2, 1e4)[0], loops.rope_pairs(x[0].tolist(), 2, 9, 1e4))
    assert np.allclose(P.rope_neox_partial(x, np.array([9]), 2, 4, 1e7)[0],
                       loops.rope_halves(x[0].tolist(), 2, 9, 4, 1e7))


# ── attention ───────────────────────────────────────────────────────────────────────────────────

def test_attention_closed_forms():
    heads, hd = 2, 4
    q = rng.standard_normal((3, heads * hd))
    v = rng.standard_normal((6, heads * hd))
    kk = np.tile(rng.standard_normal((1, heads * hd)), (6, 1))                      # identical keys
    o = P.attention(q, kk, v, heads, 0.5)
    assert np.allclose(o, np.tile(v.mean(axis=0), (3, 1)), atol=1e-14)             # -> the mean of V
    o1 = P.attention(q, kk[:1], v[:1], heads, 0.5)
    assert np.allclose(o1, np.tile(v[0], (3, 1)), atol=1e-15)                       # one key -> V
    k = rng.standard_normal((6, heads * hd))
    perm = rng.permutation(6)
    assert np.allclose(P.attention(q, k[perm], v[perm], heads, 0.5), P.attention(q, k, v, heads, 0.5), atol=1e-14)
    # a key aligned with the query under a huge scale takes all the weight
    k2 = k.copy(); k2[4] = q[0] * 10
    o2 = P.attention(q[:1], k2, v, heads, 1e3)
    assert np.allclose(o2[0], v[4], atol=1e-9)


def test_attention_softmax_rows_sum_to_one():
    s = rng.standard_normal((5, 9)) * 30
    p = P.softmax(s)
    assert np.allclose(p.sum(axis=1), 1.0, atol=1e-15) and np.all(p >= 0)


def test_attention_matches_loops_with_gqa_and_mask():
    heads, kvh, hd = 4, 2, 3
    q = rng.standard_normal((3, heads * hd))
    k = rng.standard_normal((5, kvh * hd))
    v = rng.standard_normal((5, kvh * hd))
    mask = np.where(np.arange(5)[None, :] <= np.arange(2, 5)[:, None], 0.0, -np.inf)
    o = P.attention(q, k, v, heads, 0.7, mask=mask, kv_heads=kvh)
    ref = loops.attend(q.tolist(), k.tolist(), v.tolist(), heads, 0.7, kv_heads=kvh, allowed=lambda t, j: j <= t + 2)
    assert np.allclose(o, ref, atol=1e-13)


# ── activations ─────────────────────────────────────────────────────────────────────────────────

def test_gelu_erf_within_the_pages_erf_bound():
    # The page's kernel evaluates erf by Abramowitz & Stegun 7.1.26 and states |error| <= 1.5e-7; the exact GELU
    # must sit within x/2 * 1.5e-7 of the kernel's formula everywhere.
    bound = GOLD["erf_approx"]["bound"]
    x = np.linspace(-8, 8, 4001)
    z = np.abs(x) / math.sqrt(2)
    t = 1.0 / (1.0 + 0.3275911 * z)
    poly = t * (0.254829592 + t * (-0.284496736 + t * (1.421413741 + t * (-1.453152027 + t * 1.061405429))))
    erf_as = np.sign(x) * (1.0 - poly * np.exp(-z * z))
    gelu_as = 0.5 * x * (1.0 + erf_as)
    assert np.all(np.abs(P.gelu_erf(x) - gelu_as) <= 0.5 * np.abs(x) * bound + 1e-15)


def test_gelu_textbook_values():
    # Phi(1) = 0.8413447460685429, Phi(-1) = 0.15865525393145707 (standard normal CDF tables)
    assert math.isclose(P.gelu_erf(np.array([1.0]))[0], 0.8413447460685429, rel_tol=1e-14)
    assert math.isclose(P.gelu_erf(np.array([-1.0]))[0], -0.15865525393145707, rel_tol=1e-13)
    assert P.gelu_erf(np.array([0.0]))[0] == 0.0


def test_gelu_tanh_is_close_to_exact_gelu():
    # Property of the tanh form (not a pin of its exact values): it tracks exact GELU to about 1e-3.
    x = np.linspace(-6, 6, 2001)
    assert np.max(np.abs(P.gelu_tanh(x) - P.gelu_erf(x))) < 1e-3
    assert P.gelu_tanh(np.array([0.0]))[0] == 0.0


def test_gelu_tanh_matches_an_independent_implementation():
    # The tanh form (Hendrycks & Gimpel) as PyTorch implements it, in float64 on the CPU: a second, independent
    # implementation of the published formula; plus its odd-part identity gelu(x) - gelu(-x) = x.
    torch = pytest.importorskip("torch")
    x = np.concatenate([np.linspace(-12, 12, 4801), [1e-8, -3e-5, 0.5, 1.0, 2.0, 40.0, -40.0]])
    ref = torch.nn.functional.gelu(torch.from_numpy(x), approximate="tanh").numpy()
    # relative 1e-13 where the value is not tiny; on the far negative side 1 + tanh cancels, so absolute there
    assert np.all(np.abs(P.gelu_tanh(x) - ref) <= 1e-13 * np.abs(ref) + 1e-15)
    assert np.max(np.abs(P.gelu_tanh(x) - P.gelu_tanh(-x) - x)) < 1e-13 * 40


def test_silu_sigmoid_values():
    assert P.sigmoid(np.array([0.0]))[0] == 0.5
    assert math.isclose(P.silu(np.array([2.0]))[0], 2.0 / (1.0 + math.exp(-2.0)), rel_tol=1e-15)
    assert np.allclose(P.sigmoid(np.array([-3.0, 3.0])).sum(), 1.0)


def test_argmax_lowest_index_and_gap():
    z = np.array([[1.0, 3.0, 3.0, 2.0], [5.0, 5.0, 5.0, 5.0]])
    assert list(P.argmax_rows(z)) == [1, 0]
    assert list(P.top2_gap(z)) == [0.0, 0.0]
    assert P.top2_gap(np.array([[1.0, 4.0, 2.5]]))[0] == 1.5
