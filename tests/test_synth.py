"""The seeded input generator (CPU only)."""
import numpy as np

from synth import rng, configs


def test_splitmix64_matches_sequential_definition():
    # the vectorised stream equals the generator stepped one output at a time
    M = (1 << 64) - 1
    state = 0 ^ 3
    seq = []
    for _ in range(6):
        state = (state + 0x9E3779B97F4A7C15) & M
        z = state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M
        seq.append(z ^ (z >> 31))
    assert [int(x) for x in rng.splitmix64(0, 3, 6)] == seq
    assert [int(x) for x in rng.splitmix64(0, 3, 3, offset=3)] == seq[3:]


def test_normals_moments_and_determinism():
    x = rng.normal(0, 1, 200001)
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1) < 0.01
    assert np.array_equal(x, rng.normal(0, 1, 200001))
    assert not np.array_equal(x[:100], rng.normal(0, 2, 100))


def test_bf16_rounding_is_rne():
    f = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1.0 + 2 ** -8 + 2 ** -20, 0.0], dtype=np.float32)
    b = rng.bf16_bits_to_f32(rng.f32_to_bf16_bits(f))
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: rounds to even (1); 1 + 3*2^-8 rounds to 1 + 2^-6
    assert b.tolist() == [1.0, 1.0, 1.0 + 2 ** -6, -2.5, 1.0 + 2 ** -7, 0.0]


def test_workload_shapes():
    w = configs.H3_S20423
    assert w.tokens == 20423 and len(w.segments) == 8
    assert configs.H3_S25103.tokens == 25103
    assert configs.TINY_F32.tokens == 128 and configs.TWO_SEG.tokens == 5120
    assert abs(w.attention_flops() - 3.256e12) / 3.256e12 < 1e-3
    r = configs.RAGGED64
    assert len(r.segments) == 64
    for (T, H, W, L) in r.segments:
        assert 128 <= L <= 2048 and T == 1 and H == 16 and W == -(-L // 16) and L <= T * H * W


def test_make_tensors_small():
    t = configs.make_tensors(configs.TINY_F32)
    assert t.q.dtype == np.float32 and t.q.shape == (128, 2, 64)
    assert t.gamma_q.shape == (64,) and abs(t.gamma_q.mean() - 1) < 0.1
