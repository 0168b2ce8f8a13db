"""DeepSeek-V4.1 Engram forward on one AMD Instinct MI355X (gfx950).

The package is a thin ctypes binding over libengram.so: a C-ABI library of
hand-written HIP kernels (hash, row gather + dequant, bf16 MFMA projection,
the projection fused with the Q2_K row dequant, the MXFP8 projection of raw
FP8 rows, and the gate) plus their composition.  Build the library with
`python gram_hash_memory_amd/build.py`.  Importing the package without it,
or with a library built from other sources than those beside it, raises
ImportError; there is no CPU fallback.
"""

from ._binding import (  # noqa: F401
    ENGRAM_OK, ENGRAM_ERR_ARG, ENGRAM_ERR_UNSUPPORTED, ENGRAM_ERR_HIP,
    ENGRAM_ROWS_Q2K, ENGRAM_ROWS_FP8_E4M3_E8M0, HEAD_DIM, Q2K_ROW_BYTES, FP8_ROW_BYTES,
    FP8_SCALE_BYTES, EXPORTS, LIB_PATH, EngramError, HashParams, Tokens, Layer,
    engram_hash, engram_history_update, engram_rows, engram_project, engram_project_q2k,
    engram_project_fp8, engram_quantize_mxfp8,
    engram_project_mxfp8, engram_stage_mxfp8, engram_project_mxfp8_staged, engram_gate,
    engram_gate_layers, engram_workspace_bytes, engram_forward, engram_last_error,
    engram_build_id, BUILD_ID, engram_forward_noalloc, FORWARD_NOALLOC_MAX_BYTES,
)
