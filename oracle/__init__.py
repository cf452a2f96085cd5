"""CPU oracle (test infrastructure only; never on the product path)."""
from .qoq_oracle import *  # noqa: F401,F403
from .qoq_oracle import (PROTECT, ACT_MAX, Q4_MAX, rne_div, ceil_div,  # noqa: F401
                         level1_per_channel, level2_per_group, dequantize_level2,
                         quantize_weights, quantize_act, int_gemm, int_gemm_fp64,
                         epilogue, w4a8_linear)
from .variants import (W8_MAX, INT4_MAX, w8a8_quantize_weights, w8a8_linear,  # noqa: F401
                       w4a4_quantize_weights, w4a4_quantize_act, w4a4_partial_sums,
                       w4a4_linear, w4a16_quantize_weights, w4a16_dequantize,
                       w4a16_linear)
from .kv4 import (smooth_factors, kv4_quantize, kv4_dequantize,  # noqa: F401
                  kv4_encode, smooth_query, attention_core, kv4_decode_attention,
                  fp16_decode_attention)
