"""Storage rounding of fp64 results (oracle; test infrastructure only).

``_RMSNorm.forward`` on the vLLM page ``vllm.models.dots3_note.nvidia.vision_attention``
casts its fp32 result back to the input dtype (``type_as``); the library's
pre-pass writes q and k back in place in their own dtype.  The oracle models
that as one round-to-nearest-even of the exact (fp64) value.
"""
from __future__ import annotations

import numpy as np


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp64 values to the nearest bfloat16 value (ties to even), returned as fp64.

    bfloat16 keeps 8 significant bits.  With ``x = m * 2**e`` and
    ``0.5 <= |m| < 1`` (``frexp``), the result is ``rint(m * 2**8) * 2**(e - 8)``;
    ``rint`` rounds half to even.  Exact in fp64 for normal bf16 values (the
    inputs here never reach the bf16 subnormal range).
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)


def round_to_f32(x: np.ndarray) -> np.ndarray:
    """Round fp64 values to the nearest float32 (ties to even), returned as fp64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return round_to_bf16(x)
    if dtype == "f32":
        return round_to_f32(x)
    raise ValueError(f"unknown dtype {dtype!r}")
