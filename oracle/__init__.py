"""CPU oracle for one MoE layer forward — TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously-correct numpy (float64) definitions of every step of
the layer: weight-format decode, router top-k with renormalised weights,
token->expert permutation, per-expert SwiGLU FFN, weighted combine (plus an
optional always-on shared expert), and the deterministic LRU slot policy of
the expert cache.

Only the test-suite, the smoke entry point and the CPU-baseline leg of the
benchmark may import this package.  The GPU library never calls it and shares
no code with it; the only thing both sides see is the input bytes made by the
seeded generator in `synth`.

Sources.  The FreeToken pages describe an MoE serving engine whose layers
route each token to a few experts (supported-models guide, section "MoE
strategies"), store experts as MXFP4 / NVFP4 / FP8 / BF16 weights (README
feature list; guide, "how quantizations land" and "CPU layer split"), and keep
them in a global LRU slot cache keyed by (layer, expert) with the most recent
active step as recency (guide, "expert bank & LRU slot cache").  The pages give
no formula for routing, activation or combine; each reading taken here is the
plainest one and is stated in the module that takes it.

Parity status per function is stated in each module's header.
"""
from . import formats, route, permute, ffn, combine, lru, layer  # noqa: F401
