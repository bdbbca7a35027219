"""CPU oracle for mixed-precision tiled attention prefill.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously correct
numpy (fp64) statement of what the GPU library computes.  Only the test suite,
the smoke check and the CPU-baseline leg of the benchmark may import it; the
product path (the HIP library and its Python binding) never does, and this
package imports nothing from the product.

Sources (pages, by title and section):

* "TileMix: Mixed-Precision Attention for Faster LLM Prefill" (explainer page),
  section 2 "How It Works": score tiles ("The Tile Architecture"), the packed
  per-query-row bitmask with one bit per group of key tiles ("Packed
  Bitmasks"), and the dual-path engine with per-block scale factors feeding one
  shared online-softmax state ("The Dual-Path Engine").
* "LampAttention: Look-Ahead Mixed-Precision FlashAttention for Dedicated
  Accelerators", Abstract: 8-bit key-query products and 8-bit exponentials,
  adaptive detection of sensitive sub-blocks, 16-bit recompute.

Modules:
    e4m3      OCP E4M3FN encode/decode (round-to-nearest-even, saturating)
    quant     per-block absmax quantisation to int8 / e4m3
    mask      SplitMix64 counter hash and the random packed mask template
    attention logits per path, TileMix direct softmax, Lamp online emulation,
              route counts and the fragility analysis for 8-bit rounding

Parity status: every function here is pinned by tests under ``tests/`` against
closed forms, library routines on special cases, brute force on tiny inputs or
published known-answer values, except where a module header says
"parity unpinned".  The pages print no worked numerical example, so no pin
comes from them directly.
"""
