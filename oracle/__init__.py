"""CPU oracle for the GPTQ weight-only GEMM -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct numpy implementation (fp64 arithmetic) of what
the GPU path computes.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import it; the library under ``weight_only_bit_gptq_amd``
never does, and shares no code with it.

Every function is pinned by the CPU tests (``tests/test_oracle_*.py``) against
closed forms, invariants, hand-derived golden words and brute-force
re-implementations.  One part is "parity unpinned": that the bit order inside a
packed word (LSB-first bitstream) matches real GPTQ checkpoints; no checkpoint
or format document is available to pin it.
"""
from .gptq_ref import (  # noqa: F401
    fp16_rne,
    bf16_rne,
    bf16_bits,
    bf16_from_bits,
    max_q,
    num_groups,
    group_of_rows,
    quantize_minmax,
    store_zeros,
    convert_zeros_v1_to_v2,
    convert_zeros_v2_to_v1,
    convert_zeros_packed,
    repack_tiled,
    unrepack_tiled,
    TILE_COLS,
    pack_fields,
    unpack_fields,
    pack_along_k,
    pack_along_n,
    unpack_along_k,
    unpack_along_n,
    dequant_ref,
    gemm_ref,
    gptq_gemm_ref,
    moe_gemm_ref,
    sort_act_order,
    quantize_layer,
    QuantizedLayer,
)
