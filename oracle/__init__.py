"""CPU oracle (f64) for the weight-dequantizing linear layer.

TEST INFRASTRUCTURE: only ``tests/``, ``__graft_entry__.smoke()`` and the
bench's CPU-baseline leg may import this package. The HIP library never calls
it and shares no code with it.

The linear layer is in ``reference``; the rest of the encoder block around it
(LayerNorm, q/k norm with the rotary embedding, masked attention, the block and
the forward) is in ``encoder``.

Pins (what checks the oracle against something other than itself) live in
``tests/test_oracle_*.py``. Every function here is pinned; none is "parity
unpinned".
"""
from .reference import (  # noqa: F401
    FLAG_BIAS, FLAG_GELU, FLAG_RELU, FLAG_RESIDUAL, FLAG_SILU, FLAG_TANH, QBLOCK, QBYTES, W_BF16,
    W_F16, W_F32, W_Q4_0, W_Q4_K, W_Q8_0, Q4K_BYTES, QK_K, bf16_bits_to_f64, f32_bits_to_f64, decode, decode_q4_0,
    decode_q4_k, decode_q4_k_parts, decode_q8_0, encode_q8_0, q4_k_part_scale, q4_k_scale_min,
    epilogue, f16_bits_to_f64, gelu_erf, linear, linear_dual, moe, pad_weight, padded_k, relu, silu, tanh, weight_nbytes,
)
from . import encoder  # noqa: F401,E402
