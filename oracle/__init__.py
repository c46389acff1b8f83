"""Plain, slow CPU oracle for the block-scaled FP8 linear layer.

THIS PACKAGE IS TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it. The GPU library never
calls it, and it shares no code with the HIP path: it has its own E4M3 table,
its own bf16 rounding, its own dequant, quantizer and matmul, all written from
the definitions on the pages.

Sources (page titles and sections, not line numbers):

* FastVideo PR #1829, "[feat] MiniMax H3: block-FP8 text encoder on Hopper, its
  converter, and a 4xH100 FastH3 profile":
    - "Purpose": the Hopper route converts each layer's block-scaled weight
      to BF16 just ahead of an ordinary matmul.
    - "Changes", converter bullet: E4M3 weight plus a [N/128, K/128]
      ``weight_scale_inv`` grid.
    - "Changes", tests bullet: the dequantizer must equal, bit for bit, a
      decode multiplied by the scale grid expanded over its blocks, and
      quantizing then dequantizing must lose no more than E4M3 resolution.
* LightX2V PR #1657, "Walkthrough": FP8 GEMM with FP32 accumulation.
* FastVideo PR #1829, "Changes", first bullet: the Blackwell route also
  needs a Triton quantizer beside the FlashInfer groupwise GEMM; read here as
  per-token 1x128 activation quantization for a W8A8 product.
* FastVideo ``fasth3_omniref_b200`` README, "What --lossless-accel turns on":
  bf16 rounding happens at the same points as the eager ops.

Every function is pinned by a ``-m "not gpu"`` test against something other
than itself (closed forms, exact rational arithmetic, exhaustive enumeration,
library routines on the host); see ``tests/test_oracle.py``. The only result
left without such a pin is end-to-end model quality, which no page measures.
"""

from .fp8_block_ref import (  # noqa: F401
    BLOCK,
    E4M3_MAX,
    BF16_CANONICAL_NAN,
    e4m3_value,
    e4m3_table,
    bf16_bits_to_f32,
    bf16_rne_bits,
    bf16_rne_bits_nearest,
    scale_grid_shape,
    dequant,
    dequant_rows,
    e4m3_encode_nearest,
    e4m3_encode_bits,
    quantize,
    quantize_bf16,
    linear_exact,
    linear_value,
    linear_sampled,
    gemm_bound_ratio,
    linear_bf16,
    swiglu_bf16,
    SILU_SLOPE_MAX,
    silu_exact,
    swiglu_bound_ratio,
    act_quantize,
    act_dequant_f64,
    weight_dequant_f64,
    linear_w8a8_exact,
    linear_w8a8_sampled,
)
