"""CPU oracle for the KV-cached decoder step -- TEST INFRASTRUCTURE ONLY.

A plain, slow, float64 numpy implementation of what the decoder step computes,
written from the source pages' definitions.  It exists to check the HIP path:
only the test suite, the smoke check in ``__graft_entry__`` and the benchmark's
CPU-baseline leg may import it.  The product path (the HIP library and its
Python binding) never imports, calls or links anything here, and this package
imports nothing from the product path.

Modules:
  numerics  rounding to f16/bf16, LayerNorm, RMSNorm, erf-GELU, SiLU, softmax,
            NeoX RoPE
  whisper   Whisper-style decoder: cross K/V, cached step, beam reorder, and the
            full-prefix recompute that pins the cached step
  qwen3     Qwen3-ASR-style causal LM: cached step, prefill with audio splice,
            full-prefix recompute
  beams     the beam-selection rule used to drive the beam reorder

Parity status: every function is pinned by a ``-m "not gpu"`` test against a
closed form, a library routine, an invariant or a brute-force recompute.  The
end-to-end decoder values themselves are pinned only through the composition of
those checks (no page prints numbers for random weights).
"""
