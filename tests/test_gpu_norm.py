"""GPU parity of the residual add + RMS normalization kernel
(qmm_residual_rms_norm) against the float64 oracle's residual_rms_norm()
("@mlx-bun/inference 0.0.0-stage -> 1.0.0" page, residual-rms-norm.ts): the
rounded residual is the same decision on both sides and must match bit for
bit; the normalized output is within the oracle's bound for an f32 sum of
squares, and nearly all of it agrees exactly."""
import numpy as np
import pytest

import oracle
from bit_quantized_matmul_affine_amd import binding as b, synth
from tests.gpu_util import say

pytestmark = pytest.mark.gpu


def _decode(raw, dtype):
    return oracle.decode_bf16(raw) if dtype == "bf16" else oracle.decode_f32(raw)


def _run(rows, D, dtype, seed, eps=1e-5):
    import torch
    say("norm", dtype, "rows", rows, "D", D, "seed", seed)
    xr, ur, wr = synth.norm_inputs(seed, rows, D, dtype)
    x, u, w = b.to_device(xr), b.to_device(ur), b.to_device(wr)
    res, norm = b.residual_rms_norm(x, u, w, eps)
    torch.cuda.synchronize()
    ref_res, ref_norm = oracle.residual_rms_norm(_decode(xr, dtype), _decode(ur, dtype),
                                                 _decode(wr, dtype), eps, dtype)
    got_res = _decode(b.to_numpy_bits(res), dtype)
    got_norm = _decode(b.to_numpy_bits(norm), dtype)
    return got_res, got_norm, ref_res, ref_norm


def _check(rows, D, dtype, seed, eps=1e-5):
    got_res, got_norm, ref_res, ref_norm = _run(rows, D, dtype, seed, eps)
    label = "%s rows=%d D=%d" % (dtype, rows, D)
    assert np.array_equal(got_res, ref_res), label + ": residual differs"
    tol = oracle.residual_rms_norm_tolerance(ref_norm, D, dtype)
    err = np.abs(got_norm - ref_norm)
    worst = np.unravel_index(np.argmax(err / tol), err.shape)
    assert err[worst] <= tol[worst], "%s: normalized err %.3g > tol %.3g at %s" % (
        label, err[worst], tol[worst], worst)
    if dtype == "bf16":
        assert np.mean(got_norm == ref_norm) > 0.97, label + ": too few exact matches"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rows,D", [(1, 8), (3, 200), (4, 3840), (16, 5120), (2, 2056),
                                    (5, 16384), (1, 16376), (64, 2048)])
def test_matches_oracle(dtype, rows, D):
    _check(rows, D, dtype, seed=rows * 7 + D)


def test_full_size_rows():
    # the hidden size of the 3-bit 3840-wide model's layers, at a decode batch
    _check(64, 3840, "bf16", seed=11)


def test_eps_zero_and_large():
    _check(4, 1024, "bf16", seed=3, eps=0.0)
    _check(4, 1024, "bf16", seed=4, eps=10.0)


def test_rejects_unsupported():
    import torch
    x = torch.zeros(2, 12, dtype=torch.bfloat16, device="cuda")
    w = torch.ones(12, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(b.QmmError, match="multiple of 8"):
        b.residual_rms_norm(x, x, w, 1e-5)
    x = torch.zeros(2, 16392, dtype=torch.bfloat16, device="cuda")
    w = torch.ones(16392, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(b.QmmError, match="multiple of 8"):
        b.residual_rms_norm(x, x, w, 1e-5)
    x = torch.zeros(2, 16, dtype=torch.bfloat16, device="cuda")
    w = torch.ones(16, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(b.QmmError, match="eps"):
        b.residual_rms_norm(x, x, w, -1.0)
