"""CPU oracle for exact attention forward and its FP8 variant (test infrastructure).

Plain, slow fp64 (numpy) implementations of what the HIP library computes, used
only by ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py``.  The product path never imports this package, and this package
shares no code with the HIP library.

Sources (page titles as published):
  [FA3-report]  "深度解读报告：FlashAttention-3（2024）", zako-mio LLM papers knowledge base
  [FA3-blog]    0539edu.com blog on the FlashAttention V3 technical report
  [FA-explain]  "Efficient Attention & FlashAttention", talentme science-depth M4-054

Modules:
  attention  -- naive exact softmax attention (the definition, with the GQA/MQA
                K/V head mapping) and the tiled online-softmax recurrence,
                both in fp64.
  backward   -- the gradients dQ, dK, dV of exact attention (the definition).
  rope       -- rotary position embedding (fp64 definition, fp32 emulation),
                applied before the FP8 pre-pass in the fused form.
  fp8        -- OCP e4m3 encode/decode, fast Walsh-Hadamard transform, the
                block-quantise + incoherent-processing pre-pass, and the FP8
                attention emulation.
"""
from .attention import kv_head, naive_attention, naive_attention_rows, tiled_attention  # noqa: F401
from .backward import attention_backward, attention_backward_heads  # noqa: F401
from .rope import rope_fp32, rope_fp64  # noqa: F401
from .fp8 import (  # noqa: F401
    E4M3_MAX, e4m3_decode_table, e4m3_encode, e4m3_decode, fwht, sylvester_hadamard,
    rotate_fp64, blockquant_hadamard, dequantize, fp8_attention_emulation,
)
