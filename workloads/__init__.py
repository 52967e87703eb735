"""Seeded synthetic inputs for the CSA/HCA hot path.

This package only draws random numbers and stores them in the formats the
layer keeps (float32, bfloat16 bit patterns, OCP e4m3fn codes with per-row
float32 scales).  It holds none of the method's arithmetic, and it is the only
code that both the oracle side and the HIP side use.
"""

from .gen import (  # noqa: F401
    tiny_case,
    flash_csa_decode,
    flash_hca_decode,
    pro_csa_decode,
    flash_prefill,
    with_norm_rope,
    with_fp8bf16_cache,
    with_pages,
    block_table,
    CONFIG_NAMES,
)
