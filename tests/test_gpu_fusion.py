"""GPU checks of the norm -> projection hand-off of the group sums of x:
qmm_residual_rms_norm_ex writes, with the normalized activations, the sum of
every quantization group of them, and qmm_run_sums lets the streaming and
resident kernels take those sums for the bias term of the factored form
("@mlx-bun/inference 0.0.0-stage -> 1.0.0" page, affine3-rows.ts header:
s * sum(q x) + b * sum(x); residual-rms-norm.ts for the norm).

The norm's outputs must not change (bit for bit) when it also writes sums;
the sums must be within the f32 bound of the exact sums of the stored
values; the projection with given sums must meet the same oracle acceptance
as qmm_run; and the sums must really be used (zero sums change the result).
"""
import numpy as np
import pytest

import oracle
from bit_quantized_matmul_affine_amd import binding as b, synth
from tests.gpu_util import Runner, check_against_oracle, say

pytestmark = pytest.mark.gpu


def _decode(raw, dtype):
    return oracle.decode_bf16(raw) if dtype == "bf16" else oracle.decode_f32(raw)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rows,D,gs", [(1, 5120, 64), (5, 3840, 32), (16, 5120, 128),
                                       (3, 16384, 64), (64, 2048, 64)])
def test_norm_group_sums(dtype, rows, D, gs):
    import torch
    say("norm sums", dtype, rows, D, gs)
    xr, ur, wr = synth.norm_inputs(rows * 13 + D + gs, rows, D, dtype)
    x, u, w = b.to_device(xr), b.to_device(ur), b.to_device(wr)
    res0, norm0 = b.residual_rms_norm(x, u, w, 1e-5)
    ld = rows + 3
    sums = torch.full((D // gs, ld), 7.0, dtype=torch.float32, device="cuda")
    res1, norm1 = b.residual_rms_norm(x, u, w, 1e-5, group_sums=sums, group_size=gs)
    torch.cuda.synchronize()
    assert np.array_equal(b.to_numpy_bits(res0), b.to_numpy_bits(res1))
    assert np.array_equal(b.to_numpy_bits(norm0), b.to_numpy_bits(norm1))
    got = sums.cpu().numpy().astype(np.float64)
    assert np.all(got[:, rows:] == 7.0), "columns past the rows were written"
    v = _decode(b.to_numpy_bits(norm1), dtype)
    ref = oracle.group_sums(v, gs)
    tol = oracle.group_sum_tolerance(v, gs)
    assert np.all(np.abs(got[:, :rows] - ref) <= tol)


# (bits, group size, K, N, rows): the native layout on the streaming (1, 2
# rows) and resident (9, 16 rows) kernels; step-layout formats on both, one
# in two resident blocks (20 rows: 16 + 4, the second reading its sums from
# column 16), and one whose resident shape forms its own sums (8-bit, groups
# of 32: no registers for given ones)
CHAIN = [(3, 64, 5120, 1024, 1), (3, 64, 5120, 1024, 2), (3, 64, 5120, 1024, 9),
         (4, 64, 5120, 1024, 16), (4, 128, 3840, 512, 9), (2, 64, 1024, 512, 20),
         (2, 32, 2048, 512, 1), (8, 32, 5120, 512, 12), (8, 128, 2048, 512, 2),
         # 12 rows per resident launch at K = 6656: the second block (row 12)
         # forms its own sums (the given ones are read 16 rows at a time from
         # a block start that is a multiple of 16)
         (2, 128, 6656, 512, 13)]


@pytest.mark.parametrize("case", CHAIN, ids=lambda c: "b%d_g%d_K%d_N%d_M%d" % c)
def test_norm_then_projection_with_sums(case):
    import torch
    bits, gs, K, N, M = case
    say("chain", case)
    xr, ur, wr = synth.norm_inputs(900 + M + bits, M, K, "bf16")
    x, u, w = b.to_device(xr), b.to_device(ur), b.to_device(wr)
    p = synth.small(910 + M + bits, bits=bits, K=K, N=N, M=M, group_size=gs)
    plan = b.Plan(bits, K, N, M, "bf16", group_size=gs)
    sg = plan.sum_group()
    ld = (M + 15) // 16 * 16
    sums = torch.zeros((K // sg, ld), dtype=torch.float32, device="cuda")
    _, xn = b.residual_rms_norm(x, u, w, 1e-5, group_sums=sums, group_size=sg)
    torch.cuda.synchronize()
    p.x = b.to_numpy_bits(xn)
    r = Runner(p)
    y_sums = b.to_numpy_bits(r.lin.plan.run_sums(r.x, sums, r.lin.codes, r.lin.sb))
    torch.cuda.synchronize()
    check_against_oracle(p, y_sums, label="%s with sums" % (case,))
    y_plain = r.run()
    a, c = oracle.decode_bf16(y_sums), oracle.decode_bf16(y_plain)
    assert np.max(np.abs(a - c)) <= 4 * 2.0 ** -8 * np.max(np.abs(c)) + 1e-6
    zero = torch.zeros_like(sums)
    y_zero = oracle.decode_bf16(b.to_numpy_bits(
        r.lin.plan.run_sums(r.x, zero, r.lin.codes, r.lin.sb)))
    torch.cuda.synchronize()
    if not (bits == 8 and gs == 32 and M > 2):  # that shape forms its own sums
        assert np.max(np.abs(y_zero - c)) > 0.05 * np.max(np.abs(c)), "the sums were not used"
