"""Seeded synthetic inputs for the block-quantized GEMV workloads.

This module is shared by the tests, the benchmark and the oracle harness.  It
only *draws* inputs and encodes them in the canonical block byte layout; it
holds none of the method's arithmetic (no decoding, no dot products), so the
oracle and the HIP path cannot agree with each other through it.
"""
from .gen import (  # noqa: F401
    FMT_Q8_0, FMT_Q4_0, FMT_MXFP4, FMT_NVFP4, FMT_Q4_K, FMT_Q6_K, FMT_NAMES, BLOCK_BYTES, BLOCK_LEN, QK,
    canon_bytes, bytes_per_weight,
    rng_for, q8_0_blocks, q4_0_blocks, q4_0_zero_heavy_blocks, mxfp4_blocks, nvfp4_tensor, q4_k_blocks, q6_k_blocks,
    blocks_for,
    x_f32, x_bf16_bits, x_mixed_f32, f32_to_bf16_bits_rne, router_topk, norm_weight_f32,
    encode_q8_0, encode_q4_0, encode_mxfp4,
)
from .configs import CONFIGS, c2_sweep_shapes  # noqa: F401
