"""Pins for the oracle's fused gate/up epilogue (bf16 rounding, sigmoid, SiLU
and the product chain of the shared-M gate/up kernel in trellis-shared-m.ts on
the "mlx-bun 0.4.0 -> 1.0.0" page),
checked against facts other than the oracle's own formulas: an integer
round-to-nearest-even on float32 bit patterns, hand-worked bf16 values,
the tanh form of the sigmoid, and the SiLU identity silu(z) - silu(-z) = z."""
import math

import numpy as np
import pytest

import oracle


def _rne_bf16_bits(f32: np.ndarray) -> np.ndarray:
    """bf16 rounding of float32 values by integer arithmetic on their bits."""
    u = f32.astype(np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return (rounded.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_round_bf16_matches_integer_rounding_on_float32_values():
    rng = np.random.default_rng(7)
    v = (rng.standard_normal(200000) * np.exp(rng.uniform(-30, 30, 200000))).astype(np.float32)
    v = np.concatenate([v, np.float32([0.0, -0.0, 1.0, -1.0, 3.0e38, 1.2e-38, 6.0e-39])])
    got = oracle.round_bf16(v.astype(np.float64))
    want = _rne_bf16_bits(v)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("v,want", [
    (1.0 + 2.0 ** -8, 1.0),                      # halfway, 1.0 is even
    (1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -6),      # halfway, 1 + 2^-6 is even
    (1.0 + 2.0 ** -8 + 2.0 ** -30, 1.0 + 2.0 ** -7),
    (-255.5, -256.0),                            # 255.5 needs 9 bits; tie goes to 256
    (0.1, 0.10009765625),                        # 0x3DCD
    (1e39, math.inf),
])
def test_round_bf16_hand_values(v, want):
    assert oracle.round_bf16(np.float64(v)) == want


def test_sigmoid_agrees_with_tanh_form():
    # with the gate already a bf16 value and up = 1, silu_mul_bf16 is
    # R(g * R(sigmoid(g))); compare the sigmoid inside it with (1 + tanh(g/2)) / 2
    g = oracle.round_bf16(np.linspace(-20, 20, 4001))
    got = oracle.silu_mul_bf16(g, np.ones_like(g))
    sig_tanh = oracle.round_bf16((1.0 + np.tanh(g / 2.0)) / 2.0)
    want = oracle.round_bf16(oracle.round_bf16(g * sig_tanh) * 1.0)
    # the two sigmoid forms agree to far below half a bf16 step except at
    # exact rounding ties, where one bf16 step may separate them
    step = np.abs(want) * 2.0 ** -7 + 1e-40
    assert np.all(np.abs(got - want) <= step)
    assert np.mean(got == want) > 0.999


def test_hand_worked_chain_values():
    # sigmoid(1) = 0.73105857... -> bf16 0.73046875 (187/256); silu = 0.73046875;
    # times up = 2 -> 1.4609375 exactly
    assert oracle.silu_mul_bf16(np.float64(1.0), np.float64(2.0)) == 1.4609375
    # sigmoid(-1) = 0.26894142... -> bf16 0.26953125 (138/512); silu = -0.26953125
    assert oracle.silu_mul_bf16(np.float64(-1.0), np.float64(1.0)) == -0.26953125
    # zero gate gives zero; a large gate passes through (sigmoid rounds to 1)
    assert oracle.silu_mul_bf16(np.float64(0.0), np.float64(5.0)) == 0.0
    assert oracle.silu_mul_bf16(np.float64(40.0), np.float64(0.5)) == 20.0
    # a very negative gate gives -0 (sigmoid underflows to 0)
    assert oracle.silu_mul_bf16(np.float64(-800.0), np.float64(1.0)) == 0.0


def test_every_rounding_of_the_chain_matters():
    # sigmoid(3.125) = 0.957912... -> bf16 245/256 = 0.95703125; 3.125 times that
    # is 2.99072265625 = 191.41 steps of 2^-6 -> 2.984375.  Without the
    # sigmoid rounding: 3.125 * 0.957912 = 2.993476 = 191.58 steps -> 3.0.
    assert oracle.silu_mul_bf16(np.float64(3.125), np.float64(1.0)) == 2.984375
    # gate 3.13 rounds to 3.125 first (200.32 steps of 2^-6); unrounded it
    # would give 3.13 * 0.95703125 = 2.99551 = 191.71 steps -> 3.0
    assert oracle.silu_mul_bf16(np.float64(3.13), np.float64(1.0)) == 2.984375
    # up = 1 + 2^-8 is a tie that rounds to 1.0; unrounded the product would
    # be 2.984375 * 1.00390625 = 2.99603 = 191.75 steps -> 3.0
    assert oracle.silu_mul_bf16(np.float64(3.125), np.float64(1.00390625)) == 2.984375
    # the SiLU product itself is rounded: 2.984375 * (1 + 2^-7) = 3.00769 = 192.49
    # steps -> 3.0; from the unrounded 2.99072 it would be 3.01408 = 192.9 -> 3.015625
    assert oracle.silu_mul_bf16(np.float64(3.125), np.float64(1.0078125)) == 3.0


def test_silu_identity_without_rounding_noise():
    # silu(z) - silu(-z) = z: with up = 1 the chain gives R(R(z s(z))) and
    # R(-z s(-z)); their difference stays within two bf16 steps of z
    z = oracle.round_bf16(np.linspace(-8, 8, 1601))
    a = oracle.silu_mul_bf16(z, np.ones_like(z))
    b = oracle.silu_mul_bf16(-z, np.ones_like(z))
    assert np.all(np.abs((a - b) - z) <= 2 * 2.0 ** -7 * np.maximum(np.abs(z), 1e-30) + 1e-30)


def test_gate_up_composes_the_two_projections():
    from bit_quantized_matmul_affine_amd import synth
    p = synth.small(3, bits=4, K=256, N=32, M=3)
    q = synth.small(4, bits=4, K=256, N=32, M=3)
    h = oracle.gate_up(4, 256, p.x, p.w, p.scales, p.biases, q.w, q.scales, q.biases)
    g = oracle.matmul(4, 256, p.x, p.w, p.scales, p.biases)
    u = oracle.matmul(4, 256, p.x, q.w, q.scales, q.biases)
    assert np.array_equal(h, oracle.silu_mul_bf16(g, u))
    # swapping the projections changes the result (gate and up are not symmetric)
    h2 = oracle.gate_up(4, 256, p.x, q.w, q.scales, q.biases, p.w, p.scales, p.biases)
    assert not np.array_equal(h, h2)


def test_gate_up_tolerance_covers_an_ulp_of_gate():
    # moving the gate by its matmul bound moves the chain by less than the bound
    rng = np.random.default_rng(11)
    g = rng.standard_normal(5000) * 4
    u = rng.standard_normal(5000) * 4
    tg = np.abs(g) * 1e-3 + 1e-3
    tu = np.abs(u) * 1e-3 + 1e-3
    tol = oracle.gate_up_tolerance(g, u, tg, tu)
    for sg in (-1, 1):
        for su in (-1, 1):
            moved = oracle.silu_mul_bf16(g + sg * tg, u + su * tu)
            assert np.all(np.abs(moved - oracle.silu_mul_bf16(g, u)) <= tol)
