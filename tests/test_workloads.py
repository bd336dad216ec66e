"""The seeded generator reproduces the stated workload shapes."""
import numpy as np

from vision_encoder_varlen_amd import workloads as W


def test_ragged_workload_totals():
    wl = W.config(3)
    assert wl.num_seqs == 24
    assert wl.total_tokens == 28740
    assert wl.sum_sq == 48_806_608
    assert wl.max_seqlen == 3100
    assert all(h % 2 == 0 and w % 2 == 0 and 8 <= h <= 64 and 8 <= w <= 64 for h, w in wl.grids)


def test_fixed_workload_shapes():
    shapes = {1: (65, 2, 32, 3), 2: (4096, 16, 80, 4), 4: (16384, 12, 128, 1), 5: (131072, 16, 64, 2048)}
    for n, (T, H, D, N) in shapes.items():
        wl = W.config(n)
        assert (wl.total_tokens, wl.H, wl.D, wl.num_seqs) == (T, H, D, N)
    assert W.config(1).seqlens.tolist() == [16, 48, 1]
    assert W.config(1).dtype == "f32" and W.config(2).dtype == "bf16"
    assert not W.config(1).use_norm and not W.config(2).use_norm
    assert W.config(3).use_norm and W.config(4).use_norm and W.config(5).use_norm


def test_positions_are_row_major_grid_coordinates():
    wl = W.custom([(2, 3), (1, 1)], H=1, D=32)
    assert wl.positions().tolist() == [[0, 0], [0, 1], [0, 2], [1, 0], [1, 1], [1, 2], [0, 0]]
    assert wl.cu_seqlens.tolist() == [0, 6, 7]


def test_generation_is_seeded_and_bf16_exact():
    wl = W.custom([(4, 4), (2, 8)], H=2, D=64, seed=5)
    a, b = W.generate(wl), W.generate(wl)
    assert np.array_equal(a.q, b.q) and np.array_equal(a.v, b.v)
    bits = W.f32_to_bf16_bits(a.q)
    assert np.array_equal(W.bf16_bits_to_f32(bits).reshape(a.q.shape), a.q)
    assert a.q.shape == (32, 2, 64) and a.wq.shape == (64,)


def test_bf16_rounding_ties_to_even():
    x = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -2.5], dtype=np.float32)
    got = W.bf16_bits_to_f32(W.f32_to_bf16_bits(x))
    assert got.tolist() == [1.0, 1.0 + 2.0 ** -6, -2.5]
