"""CPU oracle for the BitLinear forward -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  It shares no code with the HIP path.
"""
from .bitlinear_oracle import *  # noqa: F401,F403
from .bitlinear_oracle import (EPS32, absmax_quantize, absmean_gamma, absmean_gamma_fsum,
                               abs_sum_f64, bitlinear_forward, dequant, exact_abs_sum_units,
                               forward_from_codes, pack_codes, padded_k, quantize_weights,
                               sampled_forward, ternary_codes, unpack_codes, zero_gemm,
                               zero_gemm_dot, zero_gemm_naive)
from .bitlinear_oracle import deinterleave_units, interleave_units
from .bitlinear_oracle import dequant_f32, ffn_forward, ffn_from_codes, relu2
from .bitlinear_oracle import dequant_activations_bf16, pack_mask_bits, ste_backward, ste_weight_mask, unpack_mask_bits
from .bitlinear_oracle import (R3_UNIT, pack_codes_r3, r3_byte, r3_packed_bytes, r3_padded_k,
                               r3_value, r3_value_of_byte, unpack_codes_r3)
from .bitlinear_oracle import (LUT_ENTRIES, LUT_GROUP, lut_digits, lut_forward, lut_gemv, lut_index,
                               lut_table)
