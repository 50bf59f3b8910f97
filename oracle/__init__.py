"""CPU oracle for the multi-destination all-gather, the all-to-all and the fused GEMM + all-gather.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke entry point and the
benchmark's CPU-baseline leg may import this package.  The product path (the
HIP library and its Python binding) never imports, calls or falls back to it,
and this package imports nothing from the product path.
"""

from .ag_oracle import (  # noqa: F401
    F16,
    BF16,
    F32,
    ELEM_BYTES,
    all_gather_oracle,
    store_to_members,
    all_gather_expected_block,
    group_members,
    all_to_all_oracle,
    all_to_all_expected_block,
    round_f64_to_f16_bits,
    round_f64_to_bf16_bits,
    f16_bits_to_f64,
    bf16_bits_to_f64,
    decode_bits,
    gemm_exact,
    gemm_exact_entries,
    gemm_oracle,
    gemm_oracle_entries,
    gemm_all_gather_oracle,
)
