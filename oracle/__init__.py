"""CPU oracle for the block-quantized weight x bf16 activation product.

TEST INFRASTRUCTURE ONLY: imported by tests/, by ``__graft_entry__.smoke()`` and
by ``bench.py``'s cpu_baseline leg.  The GPU library never imports it.
"""
from .oracle import (  # noqa: F401
    Q8_0, Q4_K, Q6_K, NVFP4, Q5_K, FP8, FORMATS,
    build, load, block_values, block_bytes, packed_bytes,
    dequant_rows, gemm, max_threads, round_bf16, moe_block,
)
