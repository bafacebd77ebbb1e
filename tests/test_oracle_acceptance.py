"""Pins for the acceptance checks of the matmul parity tests (CPU only).

The two factors of the acceptance bound (sum_k |x| per activation row, max_k
|W| per weight row) and the term magnitudes of the factored form are pinned
to hand-worked values; the strict bound is shown to hold for f32 evaluations
of the factored form in several orders, and to reject outputs with
kernel-sized mistakes that the acceptance bound alone lets through at the
3-bit 5120 -> 10240 shape.
"""
import numpy as np
import pytest

import oracle
from bit_quantized_matmul_affine_amd import synth


def _hand_problem():
    """4-bit, K = 128 (two groups of 64), two weight rows, two activation rows.
    Row 0: scales (0.5, 0.25), biases (-4, 1); code 15 at k = 3 and k = 70,
    every other code 0.  Row 1: scales (0.125, 0.5), biases (-3, -2); code 15
    at k = 10, code 8 at k = 100.  x row 0: 1, -2 at k = 0, 1; 0.25 at k = 64;
    -3 at k = 127; zeros elsewhere.  x row 1: -0.5 everywhere."""
    K = 128
    codes = np.zeros((2, K), dtype=np.uint64)
    codes[0, 3] = 15
    codes[0, 70] = 15
    codes[1, 10] = 15
    codes[1, 100] = 8
    w = np.zeros((2, K // 8), dtype=np.uint64)
    for n in range(2):
        for k in range(K):
            w[n, k // 8] |= codes[n, k] << np.uint64(4 * (k % 8))
    w = w.astype(np.uint32)
    scales = np.array([[0.5, 0.25], [0.125, 0.5]], dtype=np.float32)
    biases = np.array([[-4.0, 1.0], [-3.0, -2.0]], dtype=np.float32)
    x = np.zeros((2, K), dtype=np.float32)
    x[0, 0], x[0, 1], x[0, 64], x[0, 127] = 1.0, -2.0, 0.25, -3.0
    x[1, :] = -0.5
    return K, x, w, scales, biases


def test_bound_terms_hand_worked():
    K, x, w, s, b = _hand_problem()
    sx, mw = oracle.bound_terms(4, K, x, w, s, b)
    # sum |x|: 1 + 2 + 0.25 + 3 and 128 * 0.5
    assert np.array_equal(sx, [6.25, 64.0])
    # row 0: weights -4 (code 0, group 0), 3.5 (code 15), 1 (group 1),
    # 0.25 * 15 + 1 = 4.75; row 1: -3 (group 0), 0.125 * 15 - 3 = -1.125,
    # -2 (group 1), 0.5 * 8 - 2 = 2: the largest magnitude is a negative
    # weight, and each row has its own maximum (a global 4.75 fails row 1)
    assert np.array_equal(mw, [4.75, 3.0])


def test_accumulation_terms_hand_worked():
    K, x, w, s, b = _hand_problem()
    A = oracle.accumulation_terms(4, K, x, w, s, b)
    # A(0,0): (0 + 4)*1 + (0 + 4)*2 + (0 + 1)*0.25 + (0 + 1)*3
    # A(0,1): (0 + 3)*1 + (0 + 3)*2 + (0 + 2)*0.25 + (0 + 2)*3
    # A(1,0): 0.5 * (0.5*15 + 64*4 + 0.25*15 + 64*1)
    # A(1,1): 0.5 * (0.125*15 + 64*3 + 0.5*8 + 64*2)
    assert np.array_equal(A, [[15.25, 15.5], [165.625, 162.9375]])
    y = oracle.matmul(4, K, x, w, s, b)
    # y(0,0) = -4 + 8 + 0.25 - 3; y(1,0) = -0.5 * (63*(-4) + 3.5 + 63*1 + 4.75)
    assert y[0, 0] == 1.25 and y[1, 0] == 90.375
    sampled = oracle.accumulation_terms_at(4, K, x, w, s, b, [0, 1, 1], [1, 0, 1])
    assert np.array_equal(sampled, [15.5, 165.625, 162.9375])


def test_accumulation_terms_invariants():
    p = synth.small(5, bits=3, K=640, N=48, M=3, x_dtype="f32", sb_dtype="f32")
    y = oracle.matmul(3, p.K, p.x, p.w, p.scales, p.biases)
    A = oracle.accumulation_terms(3, p.K, p.x, p.w, p.scales, p.biases)
    assert np.all(A >= np.abs(y))            # triangle inequality
    # non-negative activations, scales and biases: nothing cancels, A = y
    xp, sp, bp = np.abs(p.x), np.abs(p.scales), np.abs(p.biases)
    assert np.allclose(oracle.accumulation_terms(3, p.K, xp, p.w, sp, bp),
                       oracle.matmul(3, p.K, xp, p.w, sp, bp), rtol=1e-13)
    # A grows with |bias| and with each code's |scale| term
    A2 = oracle.accumulation_terms(3, p.K, p.x, p.w, p.scales, 2 * p.biases)
    assert np.all(A2 >= A)


def test_rounding_step_values():
    st = oracle.rounding_step([1.0, 1.5, 3.0, -6.0, 0.0, 2.0 ** -130], "bf16")
    assert np.array_equal(st, [2.0 ** -7, 2.0 ** -7, 2.0 ** -6, 2.0 ** -5, 2.0 ** -133,
                               2.0 ** -133])
    assert np.array_equal(oracle.rounding_step([1.0, 0.75], "f32"), [2.0 ** -23, 2.0 ** -24])


def _f32_factored(codes, s, b, x, order_rng=None, gs=64):
    """y = sum_g s_g sum_k q x + b_g sum_k x evaluated entirely in float32,
    the sums in a shuffled order when order_rng is given."""
    M, K = x.shape
    N = codes.shape[0]
    G = K // gs
    y = np.zeros((M, N), dtype=np.float32)
    xs = x.astype(np.float32)
    for n in range(N):
        for m in range(M):
            terms = []
            for g in range(G):
                ks = np.arange(g * gs, (g + 1) * gs)
                if order_rng is not None:
                    ks = order_rng.permutation(ks)
                qx = np.float32(0)
                sx = np.float32(0)
                for k in ks:
                    qx = np.float32(qx + np.float32(codes[n, k]) * xs[m, k])
                    sx = np.float32(sx + xs[m, k])
                terms += [np.float32(np.float32(s[n, g]) * qx), np.float32(np.float32(b[n, g]) * sx)]
            if order_rng is not None:
                terms = [terms[i] for i in order_rng.permutation(len(terms))]
            acc = np.float32(0)
            for t in terms:
                acc = np.float32(acc + t)
            y[m, n] = acc
    return y.astype(np.float64)


@pytest.mark.parametrize("bits", [3, 4])
def test_strict_bound_holds_for_f32_evaluations(bits):
    p = synth.small(40 + bits, bits=bits, K=1024, N=6, M=3)
    x = oracle.decode_bf16(p.x)
    s, b = oracle.decode_bf16(p.scales), oracle.decode_bf16(p.biases)
    codes = oracle.unpack(bits, p.K, p.N, p.w)
    ref = oracle.matmul(bits, p.K, p.x, p.w, p.scales, p.biases)
    A = oracle.accumulation_terms(bits, p.K, p.x, p.w, p.scales, p.biases)
    sx, mw = oracle.bound_terms(bits, p.K, p.x, p.w, p.scales, p.biases)
    tol = 8e-3 * np.outer(sx, mw) + 1e-6
    for seed in (None, 1, 2):
        y32 = _f32_factored(codes, s, b, x, None if seed is None else np.random.default_rng(seed))
        assert np.any(y32 != ref)                       # f32 rounding is visible
        r = oracle.check_outputs(y32, ref, A, tol, p.K, "f32")
        assert r["ok"], r
        r16 = oracle.check_outputs(oracle.round_bf16(y32), ref, A, tol, p.K, "bf16")
        assert r16["ok"], r16


@pytest.fixture(scope="module")
def workload2_sample():
    """3-bit 5120 -> 10240 (the workload-2 weights and first 16 activation
    rows), 3000 sampled outputs."""
    (p,) = synth.workload(2, M=16)
    rng = np.random.default_rng(123)
    ms = rng.integers(0, p.M, 3000)
    ns = rng.integers(0, p.N, 3000)
    ref = oracle.matmul_at(3, p.K, p.x, p.w, p.scales, p.biases, ms, ns)
    A = oracle.accumulation_terms_at(3, p.K, p.x, p.w, p.scales, p.biases, ms, ns)
    sx, mw = oracle.bound_terms(3, p.K, p.x, p.w, p.scales, p.biases)
    tol = 8e-3 * sx[ms] * mw[ns] + 1e-6
    return p, ms, ns, ref, A, tol


def test_correct_outputs_pass_at_workload2_shape(workload2_sample):
    p, ms, ns, ref, A, tol = workload2_sample
    r = oracle.check_outputs(oracle.round_bf16(ref), ref, A, tol, p.K, "bf16")
    assert r["ok"], r
    r = oracle.check_outputs(oracle.round_f32(ref), ref, A, tol, p.K, "f32")
    assert r["ok"], r


def _perturbed(p, ms, ns, scales, biases):
    return oracle.matmul_at(3, p.K, p.x, p.w, scales, biases, ms, ns)


def test_kernel_sized_mistakes_fail_at_workload2_shape(workload2_sample):
    """Outputs computed by the oracle from perturbed inputs, as a kernel with
    that mistake would produce them: one group dropped (its scale and bias
    zeroed), every code read as q + 1 (the bias raised by one scale), zeros,
    and a 1/64 relative error.  The acceptance bound alone passes the first
    two and the last; the strict and median checks reject all of them, as
    bf16 and as f32 outputs."""
    p, ms, ns, ref, A, tol = workload2_sample
    s = oracle.decode_bf16(p.scales)
    b = oracle.decode_bf16(p.biases)
    s_drop, b_drop = s.copy(), b.copy()
    s_drop[:, 17] = 0.0
    b_drop[:, 17] = 0.0
    cases = {
        "one group dropped": _perturbed(p, ms, ns, s_drop, b_drop),
        "codes read as q+1": _perturbed(p, ms, ns, s, b + s),
        "zeros": np.zeros_like(ref),
        "relative error 1/64": ref * (1 + 2.0 ** -6),
    }
    for name, y in cases.items():
        for out in ("bf16", "f32"):
            yo = oracle.round_bf16(y) if out == "bf16" else oracle.round_f32(y)
            r = oracle.check_outputs(yo, ref, A, tol, p.K, out)
            assert not r["ok"], (name, out, r)
            assert r["strict"] > 1.0 or r["median"] > r["median_cap"], (name, out, r)
        if name != "zeros":
            # the acceptance bound by itself cannot see it
            r = oracle.check_outputs(oracle.round_bf16(y), ref, A, tol, p.K, "bf16")
            assert r["bound"] <= 1.0, (name, r)


def test_bf16_weight_operands_need_the_weight_rounding_term():
    """The exact result of products with every weight rounded to bf16 (the
    operand type of a bf16 matrix-core product) stays within the bound with
    the weight-rounding term, 2^-9 of the terms, and leaves the bound of f32
    sums over exact weights on some outputs: kernels that round weights to
    bf16 are judged with the wider bound, all others with the narrower one."""
    p = synth.small(77, bits=4, K=256, N=256, M=8)
    codes = oracle.unpack(4, p.K, p.N, p.w).astype(np.float64)
    s = np.repeat(oracle.decode_bf16(p.scales), 64, axis=1)
    b = np.repeat(oracle.decode_bf16(p.biases), 64, axis=1)
    w16 = oracle.round_bf16(s * codes + b)                    # [N, K]
    y16 = oracle.decode_bf16(p.x) @ w16.T                     # exact up to f64 rounding
    ref = oracle.matmul(4, p.K, p.x, p.w, p.scales, p.biases)
    A = oracle.accumulation_terms(4, p.K, p.x, p.w, p.scales, p.biases)
    err = np.abs(y16 - ref)
    assert np.all(err <= oracle.f32_sum_bound(p.K, A, oracle.BF16_WEIGHT_ROUNDING))
    assert np.any(err > oracle.f32_sum_bound(p.K, A))
