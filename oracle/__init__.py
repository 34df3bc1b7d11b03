"""CPU oracle for block-scaled mixed-precision attention (test infrastructure).

This package is the slow, plain reference that the HIP library is checked
against.  It is NOT part of the product path: only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may import
it.  It shares no code with ``bit_mixed_precision_mxq_amd`` and imports nothing
from it.

What it follows (the pages and the readings of them):

* ThriftAttention: Selective Mixed Precision for Long-Context FP4 Attention
  (abstract): a heuristic first picks a few important query-key block pairs
  for FP16, then the picked blocks run in FP16 and the rest in FP4, and both
  are merged through one online softmax.
* HyQuant: Hybrid-Precision Quantization for LLM Attention (summary and
  abstract): vertical-line tokens (single key positions: the attention sink or
  CLS token and the keys a head's probe query scores highest) and a local
  window stay in high precision; in decode the KV cache is compressed and
  dequantisation is fused into attention.
* The "Attention Quantization" topic page (overview): block-scaled FP8/FP4
  formats; softmax amplifies small quantisation errors, so softmax runs in
  full precision.
* "Diagonal-Tiled Mixed-Precision Attention for Efficient Low-Bit MXFP
  Inference" (a title listed on that topic page): the diagonal tiles are the
  local window.

Element formats follow the public OCP Microscaling (MX) v1.0 rules (E2M1 and
E4M3 elements with an E8M0 shared exponent per 32 elements), which is what
"MX-style" means.  Every point the pages leave open is settled by a numbered
reading (R1-R34); the functions below state the reading they implement.

Parity status: every function here is pinned by tests in
``tests/test_oracle_*.py`` against closed forms, brute force, exhaustive
enumeration or special cases.  The heuristic's *quality* claims (the share of
the FP4-to-FP16 gap it recovers) cannot be pinned without the models and
benchmarks the pages used: that is "parity unpinned" and is not computed here.
"""

from .formats import (  # noqa: F401
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    E2M1_VALUES,
    e2m1_round_code,
    e2m1_value,
    e4m3_round_code,
    e4m3_value,
    quantize_mxfp4,
    hadamard_rotate,
    dequantize_mxfp4,
    pack_nibbles,
    unpack_nibbles,
    quantize_mxfp8_keys,
    dequantize_mxfp8_keys,
    quantize_int4_g32,
    dequantize_int4_g32,
    round_f16,
    fma_f32,
    P_GRID_MAGIC,
    p_exponent_grid,
    p_e4m3_code,
)
from .select import (  # noqa: F401
    tile_sets, pooled_means, tile_scores, select_blocks, select_lines, used_lines,
)
from .attention import (  # noqa: F401
    attn_mixed_ref,
    attn_exact_ref,
    softmax_scale_log2,
)
from .decode import build_kv_cache_ref, attn_decode_ref, append_kv_ref, used_decode_lines  # noqa: F401
