"""GPU parity of the fused gate/up kernel (qmm_run_gate_up) against the
float64 oracle's gate_up(): both projections, then the SiLU-times-up chain
with bf16 roundings ("mlx-bun 0.4.0 -> 1.0.0" page, trellis-shared-m.ts,
its shared-M gate/up kernel)."""
import numpy as np
import pytest

import oracle
from bit_quantized_matmul_affine_amd import binding as b, synth
from tests.gpu_util import say

pytestmark = pytest.mark.gpu


def _pair(bits, K, N, M, seed):
    g = synth.small(seed, bits=bits, K=K, N=N, M=M)
    u = synth.small(seed + 1000, bits=bits, K=K, N=N, M=M)
    return g, u


def _check(x, g, u, h_bits, label, ms=None, ns=None):
    bits, K = g.bits, g.K
    if ms is None:
        gate = oracle.matmul(bits, K, x, g.w, g.scales, g.biases, threads=8)
        up = oracle.matmul(bits, K, x, u.w, u.scales, u.biases, threads=8)
        h = oracle.decode_bf16(h_bits)
    else:
        gate = oracle.matmul_at(bits, K, x, g.w, g.scales, g.biases, ms, ns)
        up = oracle.matmul_at(bits, K, x, u.w, u.scales, u.biases, ms, ns)
        h = oracle.decode_bf16(h_bits)[ms, ns]
    sx, mwg = oracle.bound_terms(bits, K, x, g.w, g.scales, g.biases)
    _, mwu = oracle.bound_terms(bits, K, x, u.w, u.scales, u.biases)
    c = oracle.tolerance_coefficient("bf16")
    if ms is None:
        tg, tu = c * np.outer(sx, mwg) + 1e-6, c * np.outer(sx, mwu) + 1e-6
    else:
        tg, tu = c * sx[ms] * mwg[ns] + 1e-6, c * sx[ms] * mwu[ns] + 1e-6
    ref = oracle.silu_mul_bf16(gate, up)
    tol = oracle.gate_up_tolerance(gate, up, tg, tu)
    assert np.all(np.isfinite(h)), label + ": non-finite output"
    ratio = np.abs(h - ref) / tol
    worst = np.unravel_index(np.argmax(ratio), ratio.shape)
    assert ratio[worst] <= 1.0, "%s: err %.3g > tol %.3g at %s" % (
        label, abs(h - ref)[worst], tol[worst], worst)
    # the bound is a worst case (it grows with sum |x|); a wrong kernel can hide
    # under it for large K, so the typical error must also be far below it
    assert np.median(ratio) < 0.05, "%s: median err/tol %.3f" % (label, np.median(ratio))


@pytest.mark.parametrize("case", [(3, 640, 208, 3), (4, 1024, 400, 1), (4, 640, 208, 16),
                                  (3, 2048, 48, 17), (4, 256, 16, 5), (3, 5120, 32, 9)],
                         ids=lambda c: "b%d_K%d_N%d_M%d" % c)
def test_gate_up_small(case):
    bits, K, N, M = case
    g, u = _pair(bits, K, N, M, 500 + M)
    lg = b.QuantizedLinear(g, max_rows=M)
    lu = b.QuantizedLinear(u, max_rows=M)
    x = b.to_device(g.x)
    import torch
    for pairs in (0, 1, 2):
        say(case, "tile_pairs", pairs)
        h = lg.plan.run_gate_up(x, lg.codes, lg.sb, lu.codes, lu.sb, tile_pairs=pairs)
        torch.cuda.synchronize()
        _check(g.x, g, u, b.to_numpy_bits(h), "%s pairs=%d" % (case, pairs))


def test_gate_up_mlp_shapes_sampled():
    """The MLP trio's gate and up projections (4-bit, 3840 -> 15360, 4 rows
    with outlier channels), checked at sampled outputs."""
    import torch
    gate, up, _ = synth.workload(3)
    lg = b.QuantizedLinear(gate)
    lu = b.QuantizedLinear(up)
    x = b.to_device(gate.x)
    h = lg.plan.run_gate_up(x, lg.codes, lg.sb, lu.codes, lu.sb)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    ms = rng.integers(0, gate.M, 4000)
    ns = rng.integers(0, gate.N, 4000)
    _check(gate.x, gate, up, b.to_numpy_bits(h), "mlp gate/up", ms, ns)


def test_gate_up_rejects_what_it_does_not_cover():
    p = synth.small(9, bits=4, K=256, N=32, M=2, x_dtype="f32")
    lg = b.QuantizedLinear(p)
    x = b.to_device(p.x)
    with pytest.raises(b.QmmError) as ei:
        lg.plan.run_gate_up(x, lg.codes, lg.sb, lg.codes, lg.sb)
    assert ei.value.status == b.QMM_ERR_UNSUPPORTED
    q = synth.small(9, bits=4, K=16384, N=32, M=2)
    lq = b.QuantizedLinear(q)
    with pytest.raises(b.QmmError) as ei:
        lq.plan.run_gate_up(b.to_device(q.x), lq.codes, lq.sb, lq.codes, lq.sb)
    assert ei.value.status == b.QMM_ERR_UNSUPPORTED
