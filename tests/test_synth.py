"""The seeded input generator: determinism, shapes and distributions (CPU)."""
import numpy as np

from bit_quantized_matmul_affine_amd import synth


def test_same_seed_same_inputs():
    a = synth.small(3, bits=3, K=256, N=32, M=4)
    b = synth.small(3, bits=3, K=256, N=32, M=4)
    for f in ("w", "scales", "biases", "x"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
    c = synth.small(4, bits=3, K=256, N=32, M=4)
    assert not np.array_equal(a.w, c.w)


def test_small_workload_shapes_and_ranges():
    (p,) = synth.workload(0)
    assert (p.bits, p.K, p.N, p.M) == (4, 512, 512, 1)
    assert p.w.shape == (512, 64) and p.w.dtype == np.uint32
    assert p.x.dtype == np.float32 and p.scales.dtype == np.float32
    assert np.all((p.scales >= 0.005) & (p.scales < 0.02))
    # bias = -8*scale + N(0, 1e-3): the noise is small next to 8*scale
    assert np.max(np.abs(p.biases + 8 * p.scales)) < 0.006


def test_bf16_rounding_is_nearest_even():
    v = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, -2.5, 1e-30], dtype=np.float32)
    bits = synth.f32_to_bf16_bits(v)
    back = synth.bf16_bits_to_f32(bits)
    assert back[0] == 1.0
    assert back[1] == 1.0                       # tie -> even
    assert back[2] == np.float32(1.0 + 4 * 2**-8)  # tie -> even (up)
    assert back[3] == -2.5


def test_prefix_rows_share_weights():
    a = synth.Problem("t", 3, 128, 16, 8, "bf16", "bf16",
                      np.zeros((16, 12), np.uint32), np.zeros((16, 2), np.uint16),
                      np.zeros((16, 2), np.uint16), np.arange(8 * 128, dtype=np.uint16).reshape(8, 128))
    b = a.rows(3)
    assert b.M == 3 and np.array_equal(b.x, a.x[:3]) and b.w is a.w


def test_words_use_all_bits():
    p = synth.small(9, bits=4, K=1024, N=64, M=1)
    ones = np.unpackbits(p.w.view(np.uint8)).mean()
    assert 0.48 < ones < 0.52
