"""CPU oracle for the trellis / MXFP4 routed-expert contraction.

TEST INFRASTRUCTURE ONLY. This package is a plain, slow, obviously-correct CPU
reference written from the pages and from FORMAT.md. Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may import
it. The product path (``trellis_quantized_moe_amd``) never imports, calls or links
anything here, and nothing here imports the product path. The two share no code;
only the seeded input generators in ``workloads/`` (which hold none of the method's
arithmetic) feed both.

Floating point is FP64 unless a step's rounding is itself part of the definition
(the fp32 Hadamard stage order and the bf16 rounding of its output, FORMAT F8).

Pins: every function here is checked in ``tests/test_oracle_*.py`` against facts the
pages or mathematics fix (closed forms, exhaustive enumerations, library routines,
exact-rational brute force). Parity with real T16 / TrellisMX / exlr8 files is
unpinned: the pages print no worked example and no such file is available.
"""

from .t16 import (T16_MULT, t16_value, t16_value_array, tile_bits_scalar,
                  tile_states_scalar, decode_tile_scalar, decode_unit_scalar,
                  decode_unit, unit_bytes, decode_units128)
from .mxfp4 import (E2M1_VALUES, e2m1_value, e8m0_value, decode_mxfp4_unit,
                    mxfp4_unit_bytes, mxfp4_to_nvfp4, decode_nvfp4,
                    e4m3_value, nvfp4_unit_bytes)
from .fpbits import (bf16_bits_to_f64, f16_bits_to_f64, f64_to_bf16_bits_exact,
                     f32_to_bf16_bits_rne)
from .hadamard import (sylvester_hadamard, hadamard128_f64, hadamard128_fp32_order,
                       rotate128_values, output_rotation128)
from .routing import route_bucket
from .gemm import expert_gemm, expert_gemm_values, expert_gemm_exact, combine_slots
from .ffn import silu, silu_scalar, expert_ffn
from .fp8b32 import fp8b32_unit_bytes, decode_fp8b32_unit, decode_fp8b32_weight_scalar
from .codebooks import (MUL1_MULT, PMCGX_MULTS, mul1_value, mul1_value_array, decode_unit_mul1,
                        decode_unit_mul1_scalar, pmcgx_half_sum, pmcgx_pair_codes,
                        decode_unit_pmcgx, decode_unit_pmcgx_scalar, pmcgx_values, mul1_e4m3)
from .mx import (E4M3_MAX, e4m3_all_values, e4m3_round, mx_block_scale, quantize_mxfp8_rows,
                 dequantize_mxfp8_rows, t16_e4m3, t16_e4m3_codes, mxfp8_values)

__all__ = [name for name in dir() if not name.startswith("_")]
