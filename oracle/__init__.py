"""CPU oracle for the blockwise NF4 quantize / dequantize / dequant-matmul path.

TEST INFRASTRUCTURE ONLY.  This package is the slow, plain, obviously-correct
reference the HIP library is checked against.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it; the product path (``dequant_gemm_nf4_amd``) never does, and the
two share no code, tables or constant generators.

Every function follows the passage of the pages it cites; where the pages are
silent the reading taken is stated at the function.  Parity status:

* codebook            -- pinned (invariants, mpmath / scipy recomputation,
                         CDF round trip)
* thresholds / encode -- pinned (brute-force nearest level in fp64, ties)
* pack                -- pinned (hand-built bytes)
* double quant        -- pinned (exact rational mean, bounds, saturation,
                         constructed half-way ties)
* dynamic 8-bit map   -- pinned (the bit layout decoded independently, the
                         decade structure, brute-force nearest value)
* dequant             -- pinned (absmax 1 block, bounds)
* matmul              -- pinned (unit vector, brute-force loops; the dX
                         product by its transpose identity with the forward)
* memory arithmetic   -- pinned against the figures the pages print
* FP4 levels          -- pinned (the E2M1 value table, brute-force nearest
                         level over the 15 distinct values, error bound)
* FP16 rounding       -- pinned (hand-worked ties, subnormals, overflow;
                         torch's own float -> half conversion)
"""

from .nf4 import (  # noqa: F401
    BLOCKSIZE,
    DQ_GROUP,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    f16_bits_to_f32,
    f32_to_f16_bits,
    bits_to_f32,
    f32_to_bits,
    QUANT_TYPES,
    DTYPES,
    fp4_codebook,
    levels_by_code,
    sorted_codes,
    normal_quantile,
    codebook,
    thresholds,
    block_absmax,
    encode,
    pack_nibbles,
    unpack_nibbles,
    double_quant,
    DQ_MAPS,
    dynamic_map,
    double_quant_dynamic,
    block_scales,
    quantize,
    dequantize,
    matmul_ref,
    dequant_matmul_ref,
    dequant_matmul_dx_ref,
    lora_matmul_ref,
    lora_down_ref,
    rel_frobenius,
    storage_bytes,
)
