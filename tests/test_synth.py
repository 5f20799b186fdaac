"""The seeded workload generators: determinism, bf16 rounding and mask statistics."""
import numpy as np

import synth
from synth import Shape


def test_bf16_rounding_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -9, -2.5, 3.0e-3, 0.0], dtype=np.float32)
    b = synth.bf16_bits_from_f32(x)
    back = synth.f32_from_bf16_bits(b)
    assert back[0] == 1.0
    assert back[1] == 1.0                          # exact tie rounds to even (1.0)
    assert back[2] == np.float32(1.0 + 2 ** -7)    # above half-way rounds up
    assert back[3] == -2.5 and back[5] == 0.0
    assert abs(back[4] - 3.0e-3) <= 3.0e-3 * 2 ** -8


def test_generators_deterministic():
    s = Shape(1, 2, 1, 200, 16)
    a = synth.gen_qkv(s, 5)
    b = synth.gen_qkv(s, 5)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    m1 = synth.gen_block_mask(Shape(1, 4, 1, 64 * 40, 16), 3, 0.7).mask
    m2 = synth.gen_block_mask(Shape(1, 4, 1, 64 * 40, 16), 3, 0.7).mask
    assert np.array_equal(m1, m2)


def test_block_mask_structure_and_density():
    shape = Shape(1, 8, 2, 64 * 256, 16)
    info = synth.gen_block_mask(shape, 7, 0.9)
    m = info.mask.astype(bool)
    nb = 256
    assert np.all(m[..., np.arange(nb), np.arange(nb)])     # diagonal
    assert np.all(m[..., :, 0])                             # sink
    assert not np.any(np.triu(np.ones((nb, nb), dtype=bool), 1) & m[0, 0])
    for h, cols in enumerate(info.stripes):
        assert len(cols) == 4
        for c in cols:
            assert np.all(m[0, h, c:, c])
    assert abs(info.mean_sparsity - 0.9) < 0.01


def test_per_head_sparsity_mean():
    rng = np.random.Generator(np.random.PCG64(0))
    s = synth.per_head_sparsity(32, 0.8, 0.97, 0.9, rng)
    assert abs(s.mean() - 0.9) < 1e-4
    assert s.min() >= 0.8 and s.max() <= 0.97


def test_tiny_mask():
    info = synth.workload_mask("tiny_s512")
    m = info.mask
    assert m.shape == (1, 2, 8, 8)
    assert np.all(m[..., np.arange(8), np.arange(8)] == 1) and np.all(m[..., :, 0] == 1)
    assert not np.any(np.triu(m[0, 0], 1))


def test_planted_structure():
    shape = Shape(1, 4, 2, 64 * 16, 32)
    q, k, v, info = synth.gen_planted_qk(shape, 9)
    kf = synth.f32_from_bf16_bits(k).astype(np.float64)
    for g in range(2):
        u = info.directions[0, g]
        proj = kf[0, g] @ u
        per_block = proj.reshape(16, 64).mean(axis=1)
        hot = set(info.hot_blocks[0, g].tolist())
        cold = [per_block[j] for j in range(16) if j not in hot]
        for j in hot:
            assert per_block[j] > max(cold)
