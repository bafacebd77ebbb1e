"""GPU parity of the affine format variants (bits 2, 3, 4, 8 with groups of
32, 64, 128 other than 3/4-bit group 64) against the float64 oracle, element
by element at small sizes and on sampled outputs at the 5120 -> 10240 shape.

Three paths: 3- and 4-bit weights with groups of 128 run on the native
layout (each group's scale and bias serving both 64-value halves of a chunk)
and every native kernel family; the other formats with bf16 activations and
bf16 scales run on the step layout through the streaming kernel (1 or 2
rows) and the resident kernel (up to 16 rows per launch); f32 activations or
f32 scales keep MLX's layout on the vector-ALU kernel (variant "generic")."""
import numpy as np
import pytest

import oracle
from bit_quantized_matmul_affine_amd import binding as b, synth
from tests.gpu_util import Runner, check_against_oracle, say

pytestmark = pytest.mark.gpu

FORMATS = [(2, 32), (2, 64), (2, 128), (3, 32), (3, 128), (4, 32), (4, 128), (8, 32), (8, 64),
           (8, 128)]
STEP_FORMATS = [(2, 32), (2, 64), (2, 128), (3, 32), (4, 32), (8, 32), (8, 64), (8, 128)]


def _native(bits, gs):
    return bits in (3, 4) and gs in (64, 128)


def _launches(r):
    """Launches of the kernels a step-layout or MLX-layout plan runs on."""
    n = r.lin.plan.stats()["launches"]
    return n["stream"] + n["resident"] + n["generic"]


@pytest.mark.parametrize("bits,gs", STEP_FORMATS, ids=lambda v: str(v))
def test_debug_unpack_step_layout(bits, gs):
    """The step layout's decode (the B operands the kernel forms) gives back
    every code: seeded codes over several tiles and chunks, then all-ones and
    single-bit MLX words (every code at its maximum, each field boundary)."""
    K, N = 640, 48
    p = synth.small(60 + bits + gs, bits=bits, K=K, N=N, M=1, group_size=gs)
    say("step debug_unpack", bits, gs)
    r = Runner(p)
    got = r.lin.plan.debug_unpack(r.lin.codes).cpu().numpy()
    assert np.array_equal(got, oracle.unpack(bits, K, N, p.w))
    w = np.zeros_like(p.w)
    w[0:16] = 0xFFFFFFFF
    for n in range(16, N):
        w[n, :] = np.uint32(1) << np.uint32(n % 32)
    p.w = w
    r = Runner(p)
    got = r.lin.plan.debug_unpack(r.lin.codes).cpu().numpy()
    assert np.array_equal(got, oracle.unpack(bits, K, N, w))


@pytest.mark.parametrize("bits,gs", FORMATS, ids=lambda v: str(v))
def test_small_every_format(bits, gs):
    # K = 640 leaves waves without a chunk on the four-wave shapes and lanes
    # idle in the vector-ALU kernel's second slice pass; 3 rows take two
    # launches of the vector-ALU kernel, one of the step-layout kernel
    for x_dtype, sb_dtype, M in (("bf16", "bf16", 3), ("f32", "f32", 1), ("bf16", "f32", 2)):
        p = synth.small(40 + bits * 7 + gs, bits=bits, K=640, N=48, M=M, x_dtype=x_dtype,
                        sb_dtype=sb_dtype, group_size=gs)
        say("format", bits, gs, x_dtype, sb_dtype, M)
        r = Runner(p)
        y = r.run()
        last = r.lin.plan.stats()["last_variant"]
        if _native(bits, gs):
            assert last != "generic"
        elif x_dtype == "f32" or sb_dtype == "f32":
            assert last == "generic"
        else:
            assert last == "resident"
        check_against_oracle(p, y, label="b%d g%d %s/%s M=%d" % (bits, gs, x_dtype, sb_dtype, M))


@pytest.mark.parametrize("bits,gs", STEP_FORMATS, ids=lambda v: str(v))
def test_step_layout_rows(bits, gs):
    """1 and 2 rows on the streaming kernel, 3..16 in one launch of the
    resident kernel (rows past the last one never stored), 17 rows in two;
    both kernels forced at 4 rows; f32 outputs as well."""
    p = synth.small(90 + bits + gs, bits=bits, K=1024, N=208, M=17, group_size=gs)
    r = Runner(p)
    for rows in (1, 2, 3, 5, 13, 16, 17):
        say("step rows", bits, gs, rows)
        before = _launches(r)
        y = r.run(rows=rows)
        assert _launches(r) - before == (1 if rows <= 16 else 2)
        assert r.lin.plan.stats()["last_variant"] == ("stream" if rows <= 2 else "resident")
        check_against_oracle(p, y, rows=rows, label="b%d g%d rows=%d" % (bits, gs, rows))
    for variant in ("stream", "resident"):
        y = r.run(rows=4, variant=variant)
        assert r.lin.plan.stats()["last_variant"] == variant
        check_against_oracle(p, y, rows=4, label="b%d g%d rows=4 %s" % (bits, gs, variant))
    rf = Runner(p, f32_out=True)
    check_against_oracle(p, rf.run(rows=9), rows=9, out_dtype="f32",
                         label="b%d g%d rows=9 f32 out" % (bits, gs))


@pytest.mark.parametrize("bits,gs", [(2, 64), (8, 64), (2, 128), (3, 32), (4, 32), (8, 32)],
                         ids=lambda v: str(v))
def test_full_shape_sampled(bits, gs):
    """The 5120 -> 10240 projection (640 tiles) at 1 row (streaming kernel),
    9 and 16 rows (resident kernel, two or three tile slots per workgroup),
    and at 2 rows with f32 scales (vector-ALU kernel)."""
    p = synth.small(77 + bits, bits=bits, K=5120, N=10240, M=16, group_size=gs)
    r = Runner(p)
    for rows in (1, 9, 16):
        say("format full shape", bits, gs, rows)
        before = _launches(r)
        y = r.run(rows=rows)
        assert _launches(r) - before == 1
        check_against_oracle(p, y, rows=rows, sample=(3000, bits + rows),
                             label="b%d g%d full rows=%d" % (bits, gs, rows))
    q = synth.small(78 + bits, bits=bits, K=5120, N=10240, M=2, group_size=gs, sb_dtype="f32")
    say("format full shape, f32 scales", bits, gs)
    check_against_oracle(q, Runner(q).run(), sample=(2000, bits),
                         label="b%d g%d full f32 scales" % (bits, gs))


@pytest.mark.parametrize("K", [2048, 4096, 6144, 8192, 8320, 16384])
def test_k_range(K):
    """Every wave shape of the resident kernel on the step layout (eight waves
    of 4, 5, 8 chunks, sixteen waves of 8; 8320 leaves waves a chunk short)
    and, at K = 16384, five rows per launch (the LDS holds 5 x 32 KB of
    activations); one row on the streaming kernel where its registers fit;
    f32 scales on the vector-ALU kernel with one to eight slice passes."""
    cases = [(2, 32, "bf16", "bf16", 7), (8, 128, "bf16", "bf16", 6), (4, 32, "bf16", "bf16", 3),
             (2, 128, "bf16", "bf16", 1), (8, 64, "bf16", "bf16", 1), (8, 128, "f32", "bf16", 1),
             (2, 64, "bf16", "f32", 1)]
    for bits, gs, x_dtype, sb_dtype, M in cases:
        p = synth.small(500 + K // 128 + bits, bits=bits, K=K, N=32, M=M, x_dtype=x_dtype,
                        sb_dtype=sb_dtype, group_size=gs)
        say("format K", K, bits, gs, x_dtype, sb_dtype, M)
        r = Runner(p)
        before = _launches(r)
        y = r.run()
        if x_dtype == "bf16" and sb_dtype == "bf16":
            per = min(16, 160 * 1024 // (2 * K))
            assert _launches(r) - before == -(-M // per)
        check_against_oracle(p, y, label="K=%d b%d g%d %s/%s M=%d" % (K, bits, gs, x_dtype,
                                                                    sb_dtype, M))


@pytest.mark.parametrize("bits", [3, 4])
def test_group128_on_every_native_family(bits):
    """Groups of 128 on the native layout: the streaming, resident, slab,
    MFMA, vector-ALU and wide kernels and the fused gate/up pair all give the
    oracle's result (each 64-value half of a group takes the group's scale
    and bias)."""
    p = synth.small(120 + bits, bits=bits, K=5120, N=208, M=100, group_size=128)
    r = Runner(p)
    for variant, rows in (("stream", 1), ("resident", 9), ("slab", 40), ("mfma", 20),
                          ("gemv", 3), ("wide", 100), ("auto", 64)):
        say("group 128 native", bits, variant, rows)
        y = r.run(rows=rows, variant=variant)
        check_against_oracle(p, y, rows=rows, bf16_weights=variant == "wide",
                             label="b%d g128 %s rows=%d" % (bits, variant, rows))
    import torch
    K, N, M = 1024, 64, 4
    g = synth.small(130 + bits, bits=bits, K=K, N=N, M=M, group_size=128)
    u = synth.small(140 + bits, bits=bits, K=K, N=N, M=M, group_size=128)
    lg, lu = b.QuantizedLinear(g, max_rows=M), b.QuantizedLinear(u, max_rows=M)
    x = b.to_device(g.x)
    h = oracle.decode_bf16(b.to_numpy_bits(lg.plan.run_gate_up(x, lg.codes, lg.sb, lu.codes,
                                                                 lu.sb)))
    torch.cuda.synchronize()
    gate = oracle.matmul(bits, K, g.x, g.w, g.scales, g.biases, group_size=128)
    up = oracle.matmul(bits, K, g.x, u.w, u.scales, u.biases, group_size=128)
    sx, mwg = oracle.bound_terms(bits, K, g.x, g.w, g.scales, g.biases, group_size=128)
    _, mwu = oracle.bound_terms(bits, K, g.x, u.w, u.scales, u.biases, group_size=128)
    c = oracle.tolerance_coefficient("bf16")
    tol = oracle.gate_up_tolerance(gate, up, c * np.outer(sx, mwg) + 1e-6,
                                   c * np.outer(sx, mwu) + 1e-6)
    ratio = np.abs(h - oracle.silu_mul_bf16(gate, up)) / tol
    assert np.all(np.isfinite(h)) and ratio.max() <= 1.0 and np.median(ratio) < 0.05


def test_variant_rules():
    """Step-layout plans run on the streaming and resident kernels only;
    MLX-layout plans (f32 scales here) on the vector-ALU kernel only; the
    native plans never on the vector-ALU kernel of MLX's layout; the fused
    gate/up pair takes native plans only."""
    p = synth.small(3, bits=2, K=256, N=16, M=1, group_size=64)
    r = Runner(p)
    for v in ("mfma", "gemv", "slab", "wide", "generic"):
        with pytest.raises(b.QmmError) as ei:
            r.run(variant=v)
        assert ei.value.status == b.QMM_ERR_UNSUPPORTED
    for v in ("stream", "resident"):
        check_against_oracle(p, r.run(variant=v), label="forced " + v)
    pf = synth.small(5, bits=2, K=256, N=16, M=1, group_size=64, sb_dtype="f32")
    rf = Runner(pf)
    for v in ("mfma", "gemv", "stream", "resident", "slab"):
        with pytest.raises(b.QmmError) as ei:
            rf.run(variant=v)
        assert ei.value.status == b.QMM_ERR_UNSUPPORTED
    check_against_oracle(pf, rf.run(variant="generic"), label="forced generic")
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


def _random_step_cases(seed, n):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        bits, gs = STEP_FORMATS[int(rng.integers(0, len(STEP_FORMATS)))]
        out.append((bits, gs, 128 * int(rng.integers(1, 41)), 16 * int(rng.integers(1, 31)),
                    int(rng.integers(1, 21))))
    return out


@pytest.mark.parametrize("case", _random_step_cases(20261204, 16),
                         ids=lambda c: "b%d_g%d_K%d_N%d_M%d" % c)
def test_random_step_layout_shapes(case):
    """Seeded random shapes of the step-layout formats (K a multiple of 128 up
    to 5120, N a multiple of 16 up to 480, 1..20 rows): the library's choice,
    and the streaming and resident kernels forced where they take the shape."""
    bits, gs, K, N, M = case
    p = synth.small(7000 + K + N + M + bits, bits=bits, K=K, N=N, M=M, group_size=gs)
    r = Runner(p)
    say("random step shape", case)
    check_against_oracle(p, r.run(), label="random %s auto" % (case,))
    for v in ("stream", "resident"):
        try:
            y = r.run(rows=min(M, 4), variant=v)
        except b.QmmError as e:
            assert e.status == b.QMM_ERR_UNSUPPORTED, (case, v, e.status)
            continue
        check_against_oracle(p, y, rows=min(M, 4), label="random %s %s" % (case, v))

