"""CPU fp64 oracle for packed varlen vision attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product package
(``vision_encoder_varlen_amd``) imports this package, and the product path never
calls it.  Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may import it.  It shares no code with the HIP path: no
kernels, headers, helpers or tables.  It takes the seeded inputs as plain NumPy
arrays and computes everything in float64.

What it computes, and what the pages say about it:

* ``prepass`` -- Q/K RMSNorm (fp32-reduce RMSNorm of the vLLM page
  ``vllm.models.dots3_note.nvidia.vision_attention``, class ``_RMSNorm``)
  followed by 2D rotary embedding (``VisionRotaryEmbedding`` on the same page,
  applied rotate-half with the cosine widened by concatenation as in the native
  rotary branch of ``MultimodalEncoderAttention.forward`` on the tokenspeed page
  ``mm_encoder_attention.py``), in the order ``_qkv_with_rope`` applies them.
* ``attention`` -- per-segment ``softmax(Q K^T * scale) V``, the formulation of
  ``VisionAttentionV2.forward`` on the vLLM page.
* ``worklist`` -- the longest-first (segment, q-tile) list the attention
  kernel is scheduled by.  The pages have no scheduler; this rule is the
  library's own and is stated in ``worklist.py``.
* ``rounding`` -- storage rounding of fp64 results to bf16 / fp32.
* ``segment_lse`` / ``varlen_lse`` -- the log-sum-exp of each row's scores
  (natural log), the optional second result of the attention.
* variants on the pages: the ``causal`` flag of the attention functions
  (``is_causal`` of the vLLM page), ``uniform_cu_seqlens`` /
  ``dense_batch_attention`` (the ``cu_seqlens = None`` batch of
  ``_varlen_metadata`` on the tokenspeed page) and ``apply_rope_2d_complex``
  (``position_embedding_mode = "complex_rope"`` on the tokenspeed page).

Pins: every function here (the storage roundings included) is checked by
``tests/test_oracle_*.py`` against
something other than itself (an independent formulation from the pages, a
library routine, a closed form, brute force on tiny inputs, or an invariant).
No function is "parity unpinned".
"""
from .attention import (dense_batch_attention, segment_attention, segment_lse,
                        uniform_cu_seqlens, varlen_attention, varlen_attention_rows, varlen_lse)
from .prepass import (ROPE_MODES, apply_rope_2d, apply_rope_2d_complex, qk_norm_rope, rms_norm,
                      rope_angles, rope_inv_freq)
from .rounding import round_to_bf16, round_to_f32, round_to_dtype
from .worklist import worklist

__all__ = [
    "segment_attention", "segment_lse", "varlen_attention", "varlen_attention_rows", "varlen_lse",
    "uniform_cu_seqlens", "dense_batch_attention",
    "ROPE_MODES", "apply_rope_2d", "apply_rope_2d_complex", "qk_norm_rope", "rms_norm", "rope_angles", "rope_inv_freq",
    "round_to_bf16", "round_to_f32", "round_to_dtype", "worklist",
]
