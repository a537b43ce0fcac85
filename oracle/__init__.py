"""Oracle for the layer-streamed training step — TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct NumPy implementation of one training step
of the Llama-style decoder (forward, next-token cross-entropy, analytic
backward, Adam).  Only the tests, the smoke entry and the benchmark's CPU
baseline may import it; the product path never does.  It shares no code with
the HIP library: its only common dependency is the seeded input generator in
``datagen``.

What it computes follows the MegaTrain pages (arXiv 2026; radar.chestersoft.de
"Methodik" and the chatpaper.ai abstract): streaming weights per layer and
checkpoint-recompute change where and when work runs, not the result, so the
oracle is the plain definition of one training step; "streamed" mode
(per-layer checkpoints, recompute in backward) must equal "resident" mode
bit for bit.

Pins (tests marked "not gpu"): finite differences in float64 on the tiny
shape, Adam's closed form at t = 1, streamed == resident, brute-force loops
for attention and cross-entropy on tiny inputs, single rows and key tails
of attention against the full matrices, closed forms for RoPE,
RMSNorm, SiLU and the uniform-logit loss, and causality of the forward.
Parity unpinned: the architectural readings (untied head, gains = 1, eps,
RoPE base and half-split pairing) are not fixed by the pages; they are
checked for internal consistency only.
"""
from .model import (  # noqa: F401
    Oracle, adam_update, attention_bwd, attention_fwd, attention_key_tail, attention_rows,
    cross_entropy,
    rmsnorm_bwd, rmsnorm_fwd, rope_apply, rope_tables, silu, silu_grad,
)
