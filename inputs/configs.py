"""The five drafter shapes the hot path is built and measured on.

Only sizes and constants live here (no arithmetic of the method), so both the
CPU oracle and the GPU binding read the same description of a workload.

Variants
  flowmap  : flow-map DiT drafter (page "diskformer 0.5.4 -> 0.6.6",
             engines/flashmap_drafter.js: the file header and the CFG constant)
  kvinject : DFlash / DSpark KV-injection drafter (page "mlx-bun 0.4.0 -> 1.0.0",
             src/spec/dspark/module-dflash.ts: the DflashConfig defaults and #layer)
  mtp      : one-layer MTP head over Q8_0 weights (page "diskformer 0.5.3 -> 0.6.4",
             engines/ternary_bonsai_2_mtp.js: the MCFG constant and MTPHead.forward)
"""
from __future__ import annotations

import copy

# Flow-map constants shared by every flow-map shape (flashmap_drafter.js, CFG):
# theta 1e4, LN eps 1e-6, RMSNorm eps 1e-6, q/k-norm eps 1e-5.
_FLOWMAP_CONSTS = dict(rope="interleaved", rope_theta=1e4, ln_eps=1e-6, rms_eps=1e-6, qk_eps=1e-5,
                       mlp="gelu_erf", kv_dtype="f16", wtype="bf16")

CONFIGS: dict[str, dict] = {
    # Tiny flow-map drafter: small enough that the oracle runs in well under a second.
    "tiny": dict(
        variant="flowmap", dim=256, heads=4, head_dim=64, kv_heads=4, layers=2, ffn=1024, block=16,
        target_dim=512, n_taps=3, vocab=4096, max_ctx=128, rope_dims=64,
        ctx_rows=64, **_FLOWMAP_CONSTS),
    # FlashMap-Qwen3-4B-shaped drafter (CFG of flashmap_drafter.js; Qwen3-4B vocab 151936, width 2560).
    "flashmap": dict(
        variant="flowmap", dim=2048, heads=16, head_dim=128, kv_heads=16, layers=6, ffn=8192, block=16,
        target_dim=2560, n_taps=5, vocab=151936, max_ctx=1024, rope_dims=128,
        ctx_rows=512, **_FLOWMAP_CONSTS),
    # The same drafter at long context: one 8192-row prefill, then 64 draft + append steps.
    "longctx": dict(
        variant="flowmap", dim=2048, heads=16, head_dim=128, kv_heads=16, layers=6, ffn=8192, block=16,
        target_dim=2560, n_taps=5, vocab=151936, max_ctx=8192 + 64 * 16 + 32, rope_dims=128,
        ctx_rows=8192, draft_steps=64, **_FLOWMAP_CONSTS),
    # DFlash-style KV-injection drafter (DEFAULT_DFLASH_CONFIG: gamma 5, dDraft 1024, 5 layers, 8 heads,
    # ffMult 2, 4 taps) over a 2560-wide target with a 262144-token vocabulary.
    "kvinject": dict(
        variant="kvinject", dim=1024, heads=8, head_dim=128, kv_heads=8, layers=5, ffn=2048, block=5,
        target_dim=2560, n_taps=4, vocab=262144, max_ctx=2048 + 64, rope="none", rope_dims=0,
        rope_theta=0.0, ln_eps=1e-6, rms_eps=1e-6, qk_eps=1e-6, mlp="geglu_tanh", kv_dtype="f32",
        wtype="bf16", ctx_rows=2048, markov_rank=256),
    # MTP head (MCFG: H 5120, I 17408, 24 q heads, 4 kv heads, head dim 256, 64 rotated dims, theta 1e7,
    # eps 1e-6, vocab 248320, at most 8 rows); Q8_0 weights, 4096-position KV cache.
    "mtp": dict(
        variant="mtp", dim=5120, heads=24, head_dim=256, kv_heads=4, layers=1, ffn=17408, block=8,
        target_dim=5120, n_taps=2, vocab=248320, max_ctx=4096, rope="neox", rope_dims=64,
        rope_theta=1e7, ln_eps=1e-6, rms_eps=1e-6, qk_eps=1e-6, mlp="swiglu", kv_dtype="f32",
        wtype="q8_0", ctx_rows=4096),
}

# Short aliases in the order the shapes are usually listed.
ORDER = ["tiny", "flashmap", "longctx", "kvinject", "mtp"]


def get(name: str, **overrides) -> dict:
    """A copy of a named shape, with optional field overrides (for reduced-size test shapes)."""
    cfg = copy.deepcopy(CONFIGS[name])
    cfg.update(overrides)
    cfg["name"] = name
    return cfg


def scaled(name: str, **overrides) -> dict:
    """Alias of :func:`get` used where a test shrinks a shape but keeps its structure."""
    return get(name, **overrides)
