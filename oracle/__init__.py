"""CPU oracle of the W4A8 MoE routed-expert layer (test infrastructure only).

Imported by the tests, the smoke check and the benchmark's CPU-baseline leg;
never by the product path.
"""
from .w4a8_oracle import *  # noqa: F401,F403
from .w4a8_oracle import (E4M3_VALUES, FP8_MAX, GROUP, SHRINK_RATIOS,  # noqa: F401
                          bf16_bits_to_f32, dequant_weights, e4m3_decode, e4m3_encode,
                          f32_to_bf16_bits, fp8_block_quant_dequant, grouped_gemm,
                          grouped_gemm_exact_groups, int4_pack, int4_unpack, moe_layer,
                          permute, quant_act, quant_rows, quantize_int4_g128, relative_l2,
                          route, swiglu, swiglu_f32, unpermute)
from .channel_int8_oracle import (code_row_sums, grouped_gemm_i8, moe_layer_i8,  # noqa: F401
                                  quant_act_i8, quant_rows_i8, quantize_int4_channel, swiglu_i8)
from .mxfp4_oracle import (dequant_mxfp4, e2m1_decode, e2m1_encode, fp4_pack, fp4_unpack,  # noqa: F401
                           grouped_gemm_mxfp4, moe_layer_mxfp4, quantize_mxfp4)
