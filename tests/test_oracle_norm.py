"""Pins for the oracle's residual add + RMS normalization
("@mlx-bun/inference 0.0.0-stage -> 1.0.0" page, residual-rms-norm.ts):
closed forms (constant rows, power-of-two scaling), and an independent
computation in the page's own precision (float32 arithmetic, integer bf16
rounding, sequential sum of squares)."""
import numpy as np
import pytest

import oracle


def _bf16_bits_round(f32):
    u = np.asarray(f32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return (r.astype(np.uint32) << 16).view(np.float32)


def _page_precision(x, u, w, eps, dtype):
    """The page's algorithm in float32 arithmetic, one row at a time."""
    R = _bf16_bits_round if dtype == "bf16" else (lambda v: np.asarray(v, dtype=np.float32))
    x = x.astype(np.float32)
    u = u.astype(np.float32)
    w = w.astype(np.float32)
    res = R(x + u)
    out = np.empty_like(res)
    for i in range(res.shape[0]):
        acc = np.float32(0)
        for v in res[i]:
            acc = np.float32(acc + np.float32(v * v))
        inv = np.float32(1) / np.sqrt(np.float32(acc / np.float32(res.shape[1]) + np.float32(eps)))
        out[i] = R(w * R(res[i] * inv))
    return res.astype(np.float64), out.astype(np.float64)


def _inputs(rng, rows, D, dtype):
    R = oracle.round_bf16 if dtype == "bf16" else oracle.round_f32
    x = R(rng.standard_normal((rows, D)))
    u = R(rng.standard_normal((rows, D)) * 0.5)
    w = R(1.0 + 0.1 * rng.standard_normal(D))
    return x, u, w


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("D", [8, 64, 1000])
def test_agrees_with_page_precision(dtype, D):
    rng = np.random.default_rng(D)
    x, u, w = _inputs(rng, 5, D, dtype)
    res, norm = oracle.residual_rms_norm(x, u, w, 1e-5, dtype)
    pres, pnorm = _page_precision(x, u, w, 1e-5, dtype)
    assert np.array_equal(res, pres)  # the rounded sum is the same decision on both sides
    tol = oracle.residual_rms_norm_tolerance(norm, D, dtype)
    assert np.all(np.abs(norm - pnorm) <= tol)
    if dtype == "bf16":
        # the f32 error rarely reaches a bf16 rounding decision
        assert np.mean(norm == pnorm) > 0.95


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_constant_rows_normalize_to_the_weight(dtype):
    # with eps = 0 a row of equal values c has mean c^2: every value becomes
    # R(w * R(sign c)) = sign(c) * w exactly
    D = 64
    rng = np.random.default_rng(1)
    w = oracle.round_bf16(1.0 + 0.1 * rng.standard_normal(D))
    x = np.full((3, D), 0.75)
    u = np.array([[0.5], [-2.0], [1.5]]) * np.ones((3, D))
    res, norm = oracle.residual_rms_norm(x, u, w, 0.0, dtype)
    assert np.array_equal(res, x + u)
    assert np.array_equal(norm, np.sign(x + u) * w)


def test_power_of_two_scaling_leaves_the_normalization():
    rng = np.random.default_rng(2)
    x, u, w = _inputs(rng, 4, 256, "bf16")
    _, a = oracle.residual_rms_norm(x, u, w, 0.0, "bf16")
    _, b = oracle.residual_rms_norm(x * 8.0, u * 8.0, w, 0.0, "bf16")
    assert np.array_equal(a, b)


def test_rounding_points():
    # residual: 1 + 2^-9 is a bf16 tie that rounds to 1.0 before squaring
    x = np.array([[1.0, 3.0]])
    u = np.array([[2.0 ** -9, 0.0]])
    res, norm = oracle.residual_rms_norm(x, u, np.ones(2), 0.0, "bf16")
    assert res.tolist() == [[1.0, 3.0]]
    # mean square (1 + 9) / 2 = 5; 1/sqrt(5) = 0.44721... = 228.97 steps of 2^-9
    # -> 229/512; 3/sqrt(5) = 1.34164 = 171.73 steps of 2^-7 -> 172/128
    assert norm.tolist() == [[229 / 512, 172 / 128]]
    # the weight multiplies the ROUNDED normalized value: with w = 1.5,
    # 1.5 * 0.447265625 = 0.6708984375 = 171.75 steps of 2^-8 -> 172/256; from the
    # unrounded 0.4472136 it would be 0.6708204 = 171.73 steps -> also 172/256,
    # so check a case where it matters: w = 1.0078125 (1 + 2^-7)
    res, norm = oracle.residual_rms_norm(x, u, np.array([1.0078125, 1.0078125]), 0.0, "bf16")
    # 1.0078125 * 229/512 = 0.450759 = 230.79 steps of 2^-9 -> 231/512
    assert norm[0, 0] == 231 / 512


def test_group_sums_hand_worked():
    """Group-major sums of hand-worked rows (groups of 4): row 0 is 1..8, row
    1 mixes signs; out[g, m] is group g of row m."""
    v = np.array([[1, 2, 3, 4, 5, 6, 7, 8], [-1, 0, 1, 0, 2, 2, 2, 2]], dtype=np.float64)
    got = oracle.group_sums(v, 4)
    assert got.shape == (2, 2)
    assert got.tolist() == [[10.0, 0.0], [26.0, 8.0]]
    assert oracle.group_sums(np.ones((3, 128)), 64).tolist() == [[64.0] * 3, [64.0] * 3]
    with pytest.raises(ValueError):
        oracle.group_sums(v, 3)


def test_group_sum_tolerance_covers_f32_orders():
    """The bound holds for the sequential f32 sum and a pairwise f32 sum of
    bf16 values, and is zero-width where the terms are exact in f32 (small
    integers)."""
    rng = np.random.default_rng(5)
    v = oracle.round_bf16(rng.standard_normal((4, 256)) * 3.0)
    exact = oracle.group_sums(v, 64)
    tol = oracle.group_sum_tolerance(v, 64)
    f = v.astype(np.float32).reshape(4, 4, 64)
    seq = np.zeros((4, 4), dtype=np.float32)
    for i in range(64):
        seq = np.float32(seq + f[:, :, i])
    pair = f
    while pair.shape[-1] > 1:
        pair = (pair[..., 0::2] + pair[..., 1::2]).astype(np.float32)
    for got in (seq.T, pair[..., 0].T):
        assert np.all(np.abs(got.astype(np.float64) - exact) <= tol)
    ints = np.arange(128, dtype=np.float64).reshape(1, 128)
    assert oracle.group_sums(ints, 64).tolist() == [[2016.0], [6112.0]]
