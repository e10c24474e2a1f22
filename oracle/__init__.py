"""CPU oracle for the BinaryAttention forward (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The HIP library never does, and this package imports
nothing from it.
"""

from .dense_fp64 import (  # noqa: F401
    binarize_backward,
    binary_attention,
    binary_attention_backward,
    binary_attention_dense_bias_rows,
    binary_attention_int8_pv_rows,
    binary_attention_rows,
    binary_scores,
    pack_sign_bits,
    pack_words,
    quantize_probs_u8,
    quantize_values_int8,
    rel_pos_bias,
    sign_dots,
    sign_dots_from_bits,
    sign_pm1,
    softmax_rows,
    token_scale,
    unpack_sign_bits,
)
