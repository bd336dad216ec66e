"""fp64 Q/K RMSNorm and 2D rotary embedding (oracle; test infrastructure only).

Readings of the pages taken here (the pages leave these open):

* The vLLM page ``vllm.models.dots3_note.nvidia.vision_attention`` builds a
  1-D frequency table in ``VisionRotaryEmbedding``:
  ``inv_freq[j] = 1 / theta**(2j/dim)`` for ``j < dim/2``, and the table row for
  position ``p`` is ``p * inv_freq``.  The body of ``apply_rotary_pos_emb_vision``
  is not on the page.  We read the 2D table as the row index and the column index
  each looking up the 1-D table, concatenated (row half first), with
  ``dim = D/2``; so there are ``D/4`` frequencies per axis and the angle vector
  has width ``D/2``.
* The width-``D/2`` angle vector is widened to ``D`` by concatenating it with
  itself and applied rotate-half (NeoX pairing ``(m, m + D/2)``), as the native
  rotary branch of ``MultimodalEncoderAttention.forward`` on the tokenspeed page
  ``mm_encoder_attention.py`` does when ``cos`` has half the head size.
* ``_RMSNorm`` on the vLLM page reduces in fp32 and casts back before the weight
  multiply.  The oracle keeps everything in fp64 and rounds once at storage
  (``rounding.py``); the difference is below one output ulp.
* ``_qkv_with_rope`` on the vLLM page applies the norm first, then the rotary.
* ``complex_rope``: ``MultimodalEncoderAttention`` on the tokenspeed page
  accepts ``position_embedding_mode = "complex_rope"`` and then calls
  ``packed_qkv_complex_rotary``, whose body is not on the page.  Reading: the
  complex form of the same rotation -- consecutive elements ``(x[2j], x[2j+1])``
  are one complex number ``x[2j] + i x[2j+1]``, multiplied by ``e^{i a_j}``
  with the same ``D/2`` angles ``a_j`` (row table for ``j < D/4``, column
  table after).  It differs from the rotate-half form only in which elements
  form a pair: ``(2j, 2j+1)`` instead of ``(j, j + D/2)``.
"""
from __future__ import annotations

from typing import Optional

import numpy as np


def rope_inv_freq(D: int, theta: float = 10000.0) -> np.ndarray:
    """fp64 ``[D/4]`` inverse frequencies of the 1-D table for ``dim = D/2``.

    ``VisionRotaryEmbedding.__init__``: ``1 / theta**(arange(0, dim, 2) / dim)``.
    """
    if D % 4 != 0:
        raise ValueError("head dim must be a multiple of 4 for 2D rotary")
    dim = D // 2
    exponents = np.arange(0, dim, 2, dtype=np.float64) / dim
    return 1.0 / (float(theta) ** exponents)


def rope_angles(pos: np.ndarray, D: int, theta: float = 10000.0) -> np.ndarray:
    """fp64 ``[T, D/2]`` angles: row-index table entries, then column-index entries.

    ``VisionRotaryEmbedding._compute_freqs`` gives ``outer(positions, inv_freq)``;
    each token looks up its row and its column and the two lookups are
    concatenated.
    """
    pos = np.asarray(pos, dtype=np.float64)
    inv = rope_inv_freq(D, theta)
    row_part = np.outer(pos[:, 0], inv)
    col_part = np.outer(pos[:, 1], inv)
    return np.concatenate([row_part, col_part], axis=1)


def _rotate_half(x: np.ndarray) -> np.ndarray:
    half = x.shape[-1] // 2
    return np.concatenate([-x[..., half:], x[..., :half]], axis=-1)


def apply_rope_2d(x: np.ndarray, pos: np.ndarray, theta: float = 10000.0) -> np.ndarray:
    """Rotate-half RoPE of ``x`` ``[T, H, D]`` with per-token 2D angles (fp64).

    ``y = x * cos + rotate_half(x) * sin`` with ``cos = [cos(a), cos(a)]`` and
    ``sin = [sin(a), sin(a)]`` broadcast over heads.
    """
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    ang = rope_angles(pos, D, theta)               # [T, D/2]
    cos = np.concatenate([np.cos(ang), np.cos(ang)], axis=1)[:, None, :]
    sin = np.concatenate([np.sin(ang), np.sin(ang)], axis=1)[:, None, :]
    return x * cos + _rotate_half(x) * sin


def apply_rope_2d_complex(x: np.ndarray, pos: np.ndarray, theta: float = 10000.0) -> np.ndarray:
    """Complex-form RoPE of ``x`` ``[T, H, D]`` (fp64): pair ``j`` is the complex
    number ``x[..., 2j] + i x[..., 2j+1]``, multiplied by ``exp(i a_j)``."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    ang = rope_angles(pos, D, theta)[:, None, :]     # [T, 1, D/2]
    z = (x[..., 0::2] + 1j * x[..., 1::2]) * np.exp(1j * ang)
    y = np.empty_like(x)
    y[..., 0::2] = z.real
    y[..., 1::2] = z.imag
    return y


ROPE_MODES = ("neox", "complex")


def rms_norm(x: np.ndarray, weight: np.ndarray, eps: float) -> np.ndarray:
    """``_RMSNorm``: ``x * rsqrt(mean(x**2, -1) + eps) * weight`` (fp64)."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(weight, dtype=np.float64)


def qk_norm_rope(q: np.ndarray, k: np.ndarray, pos: Optional[np.ndarray],
                 theta: float = 10000.0, wq: Optional[np.ndarray] = None,
                 wk: Optional[np.ndarray] = None, eps: float = 1e-6, rope_mode: str = "neox"):
    """The pre-pass on q and k, ``[T, H, D]`` each, in fp64.

    Norm (when weights are given) then rotary (when positions are given), the
    order of ``_qkv_with_rope``.  ``rope_mode`` is ``"neox"`` (rotate-half) or
    ``"complex"``.  Returns unrounded fp64 arrays.
    """
    if rope_mode not in ROPE_MODES:
        raise ValueError(f"unknown rope mode {rope_mode!r}")
    rope = apply_rope_2d if rope_mode == "neox" else apply_rope_2d_complex
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    if (wq is None) != (wk is None):
        raise ValueError("give both norm weights or neither")
    if wq is not None:
        q = rms_norm(q, wq, eps)
        k = rms_norm(k, wk, eps)
    if pos is not None:
        q = rope(q, pos, theta)
        k = rope(k, pos, theta)
    return q, k
