"""CPU oracle of the block drafter forward: plain, slow, obviously correct NumPy in float64.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links this package; only the tests,
the smoke check and the benchmark's CPU-baseline leg use it.  It shares no code with the HIP path: it reads the
same seeded inputs (package `inputs`) and nothing else.

Every bf16 / f16 / Q8_0 value is decoded exactly and every sum accumulates in float64.  K/V caches are kept in
float64 (the f16 / f32 rounding of the GPU caches is not modelled).

Modules
  prims     decoding of the storage formats and the primitive operations (linear, norms, RoPE, attention,
            activations, argmax)
  flowmap   the flow-map DiT drafter (context append, anchor slot, 16-slot jump, head, lm_head + argmax)
  kvinject  the KV-injection (DFlash) drafter
  mtp       the one-layer MTP head over Q8_0 weights
  loops     a pure-Python-loop second implementation of the flow-map forward for tiny shapes

Parity pins: every function is checked in tests/test_oracle_*.py against closed forms, invariants, hand-worked
values from the pages' formulas or brute-force loops.  One reading is not pinned by any of these: that the
gated-GELU activation of the KV-injection drafter (the page only names it) is the tanh form -- parity unpinned
beyond that reading; the tanh formula itself is pinned against PyTorch's tanh-approximate GELU.
"""
from . import prims, flowmap, kvinject, mtp, loops  # noqa: F401
