"""fp64 per-segment non-causal attention (oracle; test infrastructure only).

Follows ``VisionAttentionV2.forward`` on the vLLM page
``vllm.models.dots3_note.nvidia.vision_attention``: the packed ``[T, H, D]``
tensors are split at the ``cu_seqlens`` boundaries and every segment computes
``softmax(q_i k_i^T * scale) v_i`` on its own, per head.  The block-diagonal
mask of ``VisionAttention.forward`` on the same page computes the same result
(masked entries get weight exactly zero).

Variants on the pages, also here:

* ``causal``: ``_VisionAttentionBase`` on the vLLM page carries an
  ``is_causal`` parameter (the encoder path passes ``False``).  Reading: query
  ``a`` of a segment sees keys ``0..a`` of the same segment (equal query and
  key lengths, so the diagonal starts at the segment's first token); masked
  scores get weight exactly zero.
* ``uniform_cu_seqlens``: ``_varlen_metadata`` on the tokenspeed page fills in
  ``arange(0, (bsz + 1) * seq_len, step=seq_len)`` when ``cu_seqlens`` is None,
  a batch of ``bsz`` segments of ``seq_len`` tokens each.

Readings: the page's eager forms divide by ``sqrt(head_dim)``; the tokenspeed
page ``mm_encoder_attention.py`` (``vision_attn_flashinfer_cudnn``) defaults
the scale to ``head_size**-0.5``.  Here the scale is an explicit argument.  The
eager forms cast the fp32 softmax to the input dtype before the PV product;
the oracle keeps the weights in fp64 (the exact value).
"""
from __future__ import annotations

import numpy as np

_ROW_BLOCK = 1024


def _softmax_rows(s: np.ndarray) -> np.ndarray:
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def _causal_mask(scores: np.ndarray, r0: int, causal: bool) -> np.ndarray:
    """Scores of query rows ``r0..`` with keys after the query set to -inf."""
    if not causal:
        return scores
    rows = np.arange(r0, r0 + scores.shape[0])[:, None]
    cols = np.arange(scores.shape[1])[None, :]
    return np.where(cols <= rows, scores, -np.inf)


def segment_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                      causal: bool = False) -> np.ndarray:
    """One segment: q, k, v ``[s, H, D]`` -> ``[s, H, D]`` (fp64).

    Query rows are taken in blocks of at most 1024 so a 16384-token segment never
    holds its full score matrix; each row's softmax still sees every key (with
    ``causal``, every key up to its own position).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    s, H, D = q.shape
    out = np.empty((s, H, v.shape[-1]), dtype=np.float64)
    for h in range(H):
        kh = k[:, h, :]
        vh = v[:, h, :]
        for r0 in range(0, s, _ROW_BLOCK):
            qh = q[r0:r0 + _ROW_BLOCK, h, :]
            scores = _causal_mask((qh @ kh.T) * scale, r0, causal)
            out[r0:r0 + _ROW_BLOCK, h, :] = _softmax_rows(scores) @ vh
    return out


def segment_lse(q: np.ndarray, k: np.ndarray, scale: float, causal: bool = False) -> np.ndarray:
    """Log-sum-exp of one segment's scores: ``[s, H]`` (fp64, natural log).

    ``lse[a, h] = log sum_b exp(scale * <q[a,h], k[b,h]>)`` over the segment's
    keys -- the second result the tokenspeed page's FA4 varlen call can return
    next to the output (``vision_attn_fa4``), and what ``return_lse`` asks the
    cuDNN prefill call for (``vision_attn_flashinfer_cudnn``).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    s, H, _ = q.shape
    out = np.empty((s, H), dtype=np.float64)
    for h in range(H):
        kh = k[:, h, :]
        for r0 in range(0, s, _ROW_BLOCK):
            scores = _causal_mask((q[r0:r0 + _ROW_BLOCK, h, :] @ kh.T) * scale, r0, causal)
            m = np.max(scores, axis=-1)
            out[r0:r0 + _ROW_BLOCK, h] = m + np.log(np.sum(np.exp(scores - m[:, None]), axis=-1))
    return out


def varlen_lse(q: np.ndarray, k: np.ndarray, cu_seqlens: np.ndarray, scale: float,
               causal: bool = False) -> np.ndarray:
    """Log-sum-exp ``[T, H]`` of every segment's scores; rows outside ``[0, cu[N])`` are NaN."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    q = np.asarray(q, dtype=np.float64)
    out = np.full(q.shape[:2], np.nan, dtype=np.float64)
    for i in range(len(cu) - 1):
        a, b = int(cu[i]), int(cu[i + 1])
        if b > a:
            out[a:b] = segment_lse(q[a:b], k[a:b], scale, causal)
    return out


def varlen_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                     cu_seqlens: np.ndarray, scale: float, causal: bool = False) -> np.ndarray:
    """All segments of a packed batch; rows outside ``[0, cu[N])`` are NaN."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    q = np.asarray(q, dtype=np.float64)
    out = np.full(q.shape[:2] + (np.asarray(v).shape[-1],), np.nan, dtype=np.float64)
    for i in range(len(cu) - 1):
        a, b = int(cu[i]), int(cu[i + 1])
        if b > a:
            out[a:b] = segment_attention(q[a:b], k[a:b], v[a:b], scale, causal)
    return out


def uniform_cu_seqlens(bsz: int, seq_len: int) -> np.ndarray:
    """``cu_seqlens`` of a uniform batch: ``[0, s, 2s, ..., bsz*s]`` (int32 ``[bsz + 1]``).

    ``_varlen_metadata`` (tokenspeed page) when ``cu_seqlens`` is None.
    """
    if bsz < 0 or seq_len < 0:
        raise ValueError("bsz and seq_len must be >= 0")
    return (np.arange(bsz + 1, dtype=np.int64) * seq_len).astype(np.int32)


def dense_batch_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, bsz: int, seq_len: int,
                          scale: float, causal: bool = False) -> np.ndarray:
    """Attention of a uniform batch, ``[bsz * seq_len, H, D]`` packed (fp64)."""
    return varlen_attention(q, k, v, uniform_cu_seqlens(bsz, seq_len), scale, causal)


def varlen_attention_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                          cu_seqlens: np.ndarray, scale: float,
                          tokens: np.ndarray, heads: np.ndarray,
                          causal: bool = False) -> np.ndarray:
    """Selected output rows ``(tokens[j], heads[j])`` -> ``[n, D]`` (fp64).

    Each row is computed on its own from its segment's keys and values (with
    ``causal``, the keys up to the row's own token), which is how full-size
    workloads are checked one sampled row at a time.
    """
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    tokens = np.asarray(tokens, dtype=np.int64)
    heads = np.asarray(heads, dtype=np.int64)
    seg = np.searchsorted(cu, tokens, side="right") - 1
    out = np.empty((tokens.shape[0], np.asarray(v).shape[-1]), dtype=np.float64)
    for j in range(tokens.shape[0]):
        a, b = int(cu[seg[j]]), int(cu[seg[j] + 1])
        if causal:
            b = int(tokens[j]) + 1
        h = int(heads[j])
        qrow = np.asarray(q[tokens[j], h, :], dtype=np.float64)
        kh = np.asarray(k[a:b, h, :], dtype=np.float64)
        vh = np.asarray(v[a:b, h, :], dtype=np.float64)
        w = _softmax_rows((kh @ qrow)[None, :] * scale)[0]
        out[j] = w @ vh
    return out
