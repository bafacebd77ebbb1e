"""Pins for the oracle on the other MLX affine formats (bits 2, 3, 4, 8 with
groups of 32, 64 or 128; "@mlx-bun/inference 0.0.0-stage -> 1.0.0" page,
affine-split-mma.ts: w = s*q + b per group, codes packed least significant
bits first): codes packed here by an independent bit-stream packer, an
activation that selects one group, and the closed form of all-maximum codes."""
import numpy as np
import pytest

import oracle


def _pack_stream(codes, bits):
    """uint32 words of each row's LSB-first bit stream (any width)."""
    N, K = codes.shape
    words = np.zeros((N, K * bits // 32), dtype=np.uint32)
    for n in range(N):
        acc = 0
        for k in range(K - 1, -1, -1):
            acc = (acc << bits) | int(codes[n, k])
        for i in range(words.shape[1]):
            words[n, i] = (acc >> (32 * i)) & 0xFFFFFFFF
    return words


FORMATS = [(2, 32), (2, 128), (3, 32), (3, 128), (4, 32), (4, 128), (8, 32), (8, 64), (8, 128)]


@pytest.mark.parametrize("bits,gs", FORMATS)
def test_one_group_selected_by_the_activation(bits, gs):
    rng = np.random.default_rng(bits * 1000 + gs)
    K, N = 256, 5
    q = rng.integers(0, 2 ** bits, (N, K))
    w = _pack_stream(q, bits)
    assert np.array_equal(oracle.unpack(bits, K, N, w), q)
    G = K // gs
    s = rng.uniform(0.01, 0.05, (N, G))
    b = rng.uniform(-1, 1, (N, G))
    for g in range(G):
        x = np.zeros((1, K))
        x[0, g * gs:(g + 1) * gs] = 1.0
        y = oracle.matmul(bits, K, x, w, s, b, group_size=gs)
        expect = s[:, g] * q[:, g * gs:(g + 1) * gs].sum(axis=1) + gs * b[:, g]
        assert np.allclose(y[0], expect, rtol=0, atol=1e-12)


@pytest.mark.parametrize("bits,gs", FORMATS)
def test_all_maximum_codes(bits, gs):
    # every code 2^bits - 1 (every word all ones): y = sum_g gs ((2^b - 1) s_g + b_g)
    K, N = 384, 3
    w = np.full((N, K * bits // 32), 0xFFFFFFFF, dtype=np.uint32)
    G = K // gs
    s = np.linspace(0.01, 0.03, N * G).reshape(N, G)
    b = np.linspace(-0.5, 0.5, N * G).reshape(N, G)
    y = oracle.matmul(bits, K, np.ones((1, K)), w, s, b, group_size=gs)
    expect = (gs * ((2 ** bits - 1) * s + b)).sum(axis=1)
    assert np.allclose(y[0], expect, rtol=1e-12, atol=0)


def test_group_size_changes_which_scale_applies():
    # the same codes and per-column scales read with groups of 32 and 128
    # differ unless the scales repeat
    rng = np.random.default_rng(5)
    K, N = 256, 2
    q = rng.integers(0, 4, (N, K))
    w = _pack_stream(q, 2)
    x = rng.standard_normal((1, K))
    s32 = rng.uniform(0.01, 0.05, (N, K // 32))
    b32 = np.zeros((N, K // 32))
    s128 = s32[:, ::4].copy()
    y32 = oracle.matmul(2, K, x, w, s32, b32, group_size=32)
    y128 = oracle.matmul(2, K, x, w, s128, b32[:, ::4], group_size=128)
    assert not np.allclose(y32, y128)
    y32r = oracle.matmul(2, K, x, w, np.repeat(s128, 4, axis=1), b32, group_size=32)
    assert np.allclose(y32r, y128, rtol=1e-13, atol=1e-13)
