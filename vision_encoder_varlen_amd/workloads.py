"""Seeded synthetic inputs for packed varlen vision attention.

This module only draws random numbers and lays them out; it computes nothing
that the attention path computes.  Both the HIP path (through the tests and the
benchmark) and the CPU oracle consume what it produces, so it must stay free of
any normalisation, rotary or softmax arithmetic.

Layout (the packed varlen convention of the tokenspeed page
``mm_encoder_attention.py``, ``_varlen_metadata`` and the backend calls):

* ``q``, ``k``, ``v``: ``[T, H, D]`` contiguous, element ``(t, h, d)`` at
  ``(t*H + h)*D + d``.
* ``cu_seqlens``: int32 ``[N+1]``, ``cu_seqlens[0] = 0``, segment ``i`` owns
  tokens ``[cu_seqlens[i], cu_seqlens[i+1])``.
* ``pos``: int32 ``[T, 2]``, the (row, col) of each token inside its image's
  patch grid, tokens laid out row-major inside a segment.

Random draws (``numpy.random.default_rng(seed)``), in this order: image grids
(ragged workload only), then ``q``, ``k``, ``v`` as ``standard_normal((T,H,D),
float32)``, then the two RMSNorm weight vectors as ``1 + 0.1*standard_normal(D)``
in float32.  bf16 workloads round each fp32 draw to the nearest bf16 value (ties
to even) and keep the exact values.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Tuple

import numpy as np

F32 = "f32"
BF16 = "bf16"


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the raw bits as uint16."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    bias = np.uint64(0x7FFF) + ((bits >> np.uint64(16)) & np.uint64(1))
    out = ((bits + bias) >> np.uint64(16)).astype(np.uint16)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen raw bfloat16 bits (uint16) to float32 exactly."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Workload:
    """One synthetic packed batch of images (segments)."""

    name: str
    dtype: str                      # "f32" or "bf16"
    grids: List[Tuple[int, int]]    # (rows, cols) of each image's patch grid
    H: int
    D: int
    seed: int
    theta: float = 10000.0
    use_norm: bool = False
    eps: float = 1e-6
    scale: Optional[float] = None   # None -> 1/sqrt(D)
    ragged_images: int = 0          # >0: the grids were drawn from this workload's own RNG first
    seqlens_override: Optional[List[int]] = field(default=None, repr=False)

    @property
    def seqlens(self) -> np.ndarray:
        if self.seqlens_override is not None:
            return np.asarray(self.seqlens_override, dtype=np.int64)
        return np.asarray([h * w for h, w in self.grids], dtype=np.int64)

    @property
    def num_seqs(self) -> int:
        return int(self.seqlens.shape[0])

    @property
    def total_tokens(self) -> int:
        return int(self.seqlens.sum())

    @property
    def max_seqlen(self) -> int:
        s = self.seqlens
        return int(s.max()) if s.size else 0

    @property
    def softmax_scale(self) -> float:
        return float(self.scale) if self.scale is not None else float(1.0 / np.sqrt(self.D))

    @property
    def cu_seqlens(self) -> np.ndarray:
        cu = np.zeros(self.num_seqs + 1, dtype=np.int64)
        np.cumsum(self.seqlens, out=cu[1:])
        return cu.astype(np.int32)

    @property
    def sum_sq(self) -> int:
        s = self.seqlens.astype(np.int64)
        return int((s * s).sum())

    @property
    def attn_flops(self) -> float:
        """Algorithmic attention FLOPs, 4*H*D*sum(s_i^2): QK^T and PV, two FLOPs per MAC."""
        return 4.0 * self.H * self.D * self.sum_sq

    def positions(self) -> np.ndarray:
        """int32 [T, 2] (row, col) of each token, row-major inside each image grid."""
        parts = []
        if self.seqlens_override is not None:
            # Explicit lengths without a grid: treat each segment as a 1-row strip.
            for n in self.seqlens_override:
                ell = np.arange(n, dtype=np.int64)
                parts.append(np.stack([np.zeros_like(ell), ell], axis=1))
        else:
            for h, w in self.grids:
                ell = np.arange(h * w, dtype=np.int64)
                parts.append(np.stack([ell // w, ell % w], axis=1))
        if not parts:
            return np.zeros((0, 2), dtype=np.int32)
        return np.concatenate(parts, axis=0).astype(np.int32)


@dataclass
class Inputs:
    """Generated tensors.  Float tensors hold exactly the values the device sees."""

    q: np.ndarray          # float32 [T,H,D] (bf16-representable for bf16 workloads)
    k: np.ndarray
    v: np.ndarray
    wq: np.ndarray         # float32 [D]
    wk: np.ndarray
    pos: np.ndarray        # int32 [T,2]
    cu_seqlens: np.ndarray  # int32 [N+1]


def generate(wl: Workload) -> Inputs:
    rng = np.random.default_rng(wl.seed)
    if wl.ragged_images:
        # Grid draws come first for the ragged workload; consume them so the
        # tensor draws that follow match the recipe.
        _ragged_grid_draw(rng, wl.ragged_images)
    T, H, D = wl.total_tokens, wl.H, wl.D
    tensors = []
    for _ in range(3):
        x = rng.standard_normal((T, H, D), dtype=np.float32)
        if wl.dtype == BF16:
            x = bf16_bits_to_f32(f32_to_bf16_bits(x)).reshape(T, H, D)
        tensors.append(np.ascontiguousarray(x))
    wq = (1.0 + 0.1 * rng.standard_normal(D, dtype=np.float32)).astype(np.float32)
    wk = (1.0 + 0.1 * rng.standard_normal(D, dtype=np.float32)).astype(np.float32)
    return Inputs(q=tensors[0], k=tensors[1], v=tensors[2], wq=wq, wk=wk,
                  pos=wl.positions(), cu_seqlens=wl.cu_seqlens)


def _ragged_grid_draw(rng: np.random.Generator, n_images: int = 24,
                      cap: int = 65536) -> List[Tuple[int, int]]:
    hw = rng.integers(4, 33, size=(n_images, 2)) * 2  # even sides in [8, 64]
    grids = [(int(h), int(w)) for h, w in hw]
    kept, total = [], 0
    for h, w in grids:
        if total + h * w > cap:
            break
        kept.append((h, w))
        total += h * w
    return kept


def config(n: int) -> Workload:
    """The five seeded workloads (1-based), each named by its shape."""
    if n == 1:
        return Workload("fp32_3seg", F32, [(4, 4), (6, 8), (1, 1)], H=2, D=32, seed=1)
    if n == 2:
        return Workload("bf16_4x1024", BF16, [(32, 32)] * 4, H=16, D=80, seed=2)
    if n == 3:
        grids = _ragged_grid_draw(np.random.default_rng(3))
        return Workload("ragged24", BF16, grids, H=16, D=128, seed=3, use_norm=True,
                        ragged_images=24)
    if n == 4:
        return Workload("bf16_1x16384", BF16, [(128, 128)], H=12, D=128, seed=4, use_norm=True)
    if n == 5:
        return Workload("bf16_2048x64", BF16, [(8, 8)] * 2048, H=16, D=64, seed=5, use_norm=True)
    raise ValueError(f"no workload {n}; expected 1..5")


def custom(grids: Sequence[Tuple[int, int]], H: int, D: int, dtype: str = BF16,
           seed: int = 0, use_norm: bool = False, scale: Optional[float] = None,
           name: str = "custom") -> Workload:
    return Workload(name, dtype, list(grids), H=H, D=D, seed=seed, use_norm=use_norm, scale=scale)


def from_seqlens(seqlens: Sequence[int], H: int, D: int, dtype: str = BF16, seed: int = 0,
                 use_norm: bool = False, scale: Optional[float] = None,
                 name: str = "seqlens") -> Workload:
    """Segments given by length only (zero-length allowed); positions are (0, l)."""
    return Workload(name, dtype, [], H=H, D=D, seed=seed, use_norm=use_norm, scale=scale,
                    seqlens_override=[int(s) for s in seqlens])
