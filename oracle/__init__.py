"""CPU oracle for the DeepSeek-V4.1 Engram forward -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct implementation of what the Engram forward
computes, written from three public pages about the method:

* [spark] "Module engram_v41" (spark_model layers API docs),
* [NeMo]  "nemo_automodel.components.models.deepseek_v41.engram",
* [vLLM]  "vllm.models.deepseek_v41.common.engram".

Only the test suite, the smoke check and the CPU-baseline leg of the
benchmark may import this package.  The HIP library never calls it, links it
or reads anything it wrote; the two implementations share no code.  Floating
point is float64 (rounded to the storage precision -- bf16 or fp32 -- only
where the method stores a value); integers are exact Python integers.

Every function is pinned by tests against hand-worked values, library
decoders, closed forms or invariants.  The pins cover the oracle's readings
of the pages and stop there.  Two things stay "parity unpinned" because
neither the released model nor its files are available:
* whether DeepSeek's own hash combines the n-gram terms by XOR (reading A1);
* whether real GGUF Q2_K files use the quant interleave of reading A10.
The multiplier draw is pinned by literal values computed from the vLLM
page's rule and by a second, from-scratch implementation of the generator
that rule names (tests/test_oracle_multipliers.py).
"""

from .layout import is_prime, next_unused_prime, engram_layout, hash_multipliers
from .numerics import (bf16_round, bf16_bits, bf16_value, fp16_value,
                       e4m3fn_value, e8m0_scale)
from .engram import (hash_ids, history_update, rows_q2k, rows_fp8, project, gate, forward,
                     Q2K_ROW_BYTES, FP8_ROW_BYTES, HEAD_DIM)
from .mx import (e8m0_mx_scale, quantize_mxfp8, mx_values, rows_fp8_mx, project_mxfp8,
                 MX_BLOCK)

__all__ = [
    "is_prime", "next_unused_prime", "engram_layout", "hash_multipliers",
    "bf16_round", "bf16_bits", "bf16_value", "fp16_value", "e4m3fn_value",
    "e8m0_scale", "hash_ids", "history_update", "rows_q2k", "rows_fp8", "project", "gate",
    "forward", "Q2K_ROW_BYTES", "FP8_ROW_BYTES", "HEAD_DIM", "e8m0_mx_scale",
    "quantize_mxfp8", "mx_values", "rows_fp8_mx", "project_mxfp8", "MX_BLOCK",
]
