"""GPU parity of the affine format variants (bits 2, 3, 4, 8 with groups of
32, 64, 128 other than 3/4-bit group 64) on the generic kernel against the
float64 oracle, element by element at small sizes and on sampled outputs at
the 5120 -> 10240 shape."""
import numpy as np
import pytest

from bit_quantized_matmul_affine_amd import binding as b, synth
from tests.gpu_util import Runner, check_against_oracle, say

pytestmark = pytest.mark.gpu

FORMATS = [(2, 32), (2, 64), (2, 128), (3, 32), (3, 128), (4, 32), (4, 128), (8, 32), (8, 64),
           (8, 128)]


@pytest.mark.parametrize("bits,gs", FORMATS, ids=lambda v: str(v))
def test_small_every_format(bits, gs):
    # K = 640 leaves lanes idle in the second slice pass; 3 rows take two launches
    for x_dtype, sb_dtype, M in (("bf16", "bf16", 3), ("f32", "f32", 1), ("bf16", "f32", 2)):
        p = synth.small(40 + bits * 7 + gs, bits=bits, K=640, N=48, M=M, x_dtype=x_dtype,
                        sb_dtype=sb_dtype, group_size=gs)
        say("format", bits, gs, x_dtype, sb_dtype, M)
        r = Runner(p)
        y = r.run()
        assert r.lin.plan.stats()["last_variant"] == "generic"
        check_against_oracle(p, y, label="b%d g%d %s/%s M=%d" % (bits, gs, x_dtype, sb_dtype, M))


@pytest.mark.parametrize("bits,gs", [(2, 64), (8, 64), (4, 128), (3, 32)], ids=lambda v: str(v))
def test_full_shape_sampled(bits, gs):
    p = synth.small(77 + bits, bits=bits, K=5120, N=10240, M=2, group_size=gs)
    say("format full shape", bits, gs)
    r = Runner(p)
    check_against_oracle(p, r.run(), sample=(3000, bits), label="b%d g%d full" % (bits, gs))


@pytest.mark.parametrize("K", [2048, 4096, 6144, 8192, 8320])
def test_slice_passes(K):
    """One to five slice passes per lane (2048 values per pass of a wave),
    with a ragged last pass at 6144 and 8320."""
    for bits, gs, x_dtype, sb_dtype, M in ((2, 32, "bf16", "bf16", 2), (8, 128, "f32", "bf16", 1),
                                          (3, 128, "bf16", "f32", 1)):
        p = synth.small(500 + K // 128 + bits, bits=bits, K=K, N=32, M=M, x_dtype=x_dtype,
                        sb_dtype=sb_dtype, group_size=gs)
        say("format K", K, bits, gs, x_dtype, sb_dtype, M)
        r = Runner(p)
        check_against_oracle(p, r.run(), label="K=%d b%d g%d %s/%s M=%d" % (K, bits, gs, x_dtype,
                                                                         sb_dtype, M))


def test_variant_rules():
    p = synth.small(3, bits=2, K=256, N=16, M=1, group_size=64)
    r = Runner(p)
    for v in ("mfma", "gemv", "stream", "resident", "slab"):
        with pytest.raises(b.QmmError) as ei:
            r.run(variant=v)
        assert ei.value.status == b.QMM_ERR_UNSUPPORTED
    check_against_oracle(p, r.run(variant="generic"), label="forced generic")
    q = synth.small(4, bits=4, K=256, N=16, M=1)
    rq = Runner(q)
    with pytest.raises(b.QmmError) as ei:
        rq.run(variant="generic")
    assert ei.value.status == b.QMM_ERR_UNSUPPORTED
    import torch
    x = b.to_device(p.x)
    with pytest.raises(b.QmmError) as ei:
        r.lin.plan.run_gate_up(x, r.lin.codes, r.lin.sb, r.lin.codes, r.lin.sb)
    assert ei.value.status == b.QMM_ERR_UNSUPPORTED
    torch.cuda.synchronize()
