"""GPU parity: the HIP path through the C ABI against the float64 oracle.

Bar: unpacked codes bit-exact; outputs within
    |y - y_ref| <= c * sum_k|x(m,k)| * max_k|W(n,k)| + 1e-6,
c = 1e-3 for f32 activations and 8e-3 for bf16 activations, element by element.
"""
import numpy as np
import pytest

import oracle
from bit_quantized_matmul_affine_amd import binding as b
from bit_quantized_matmul_affine_amd import synth
from tests.gpu_util import Runner, check_against_oracle, resident_ok, say, stream_ok, y_to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    b.lib()


# ------------------------------------------------------------------ unpack

@pytest.mark.parametrize("bits,K,N", [(3, 128, 16), (4, 128, 16), (3, 640, 48), (4, 384, 80)])
def test_debug_unpack_small(bits, K, N):
    say("debug_unpack", bits, K, N)
    p = synth.small(21, bits=bits, K=K, N=N, M=1)
    r = Runner(p)
    got = r.lin.plan.debug_unpack(r.lin.codes).cpu().numpy()
    assert np.array_equal(got, oracle.unpack(bits, K, N, p.w))


@pytest.mark.parametrize("idx", [0, 1, 2, 3, 4])
def test_debug_unpack_workloads(idx):
    for p in synth.workload(idx, M=1) if idx == 2 else synth.workload(idx):
        say("debug_unpack workload", idx, p.name)
        r = Runner(p)
        got = r.lin.plan.debug_unpack(r.lin.codes).cpu().numpy()
        assert np.array_equal(got, oracle.unpack(p.bits, p.K, p.N, p.w)), p.name
        del r


def test_debug_unpack_extreme_words():
    """All-ones and single-bit words: every code at its maximum, and each code
    boundary, through the device unpack."""
    for bits in (3, 4):
        K, N = 256, 32
        p = synth.small(1, bits=bits, K=K, N=N, M=1)
        w = np.zeros_like(p.w)
        w[0:16] = 0xFFFFFFFF
        for n in range(16, 32):
            w[n, :] = np.uint32(1) << np.uint32(n % 32)
        p.w = w
        r = Runner(p)
        got = r.lin.plan.debug_unpack(r.lin.codes).cpu().numpy()
        assert np.array_equal(got, oracle.unpack(bits, K, N, w))


# ------------------------------------------------------------------ small parity

SMALL = [
    # bits, K, N, M, x_dtype, sb_dtype
    (4, 128, 16, 1, "bf16", "bf16"),
    (3, 128, 16, 1, "bf16", "bf16"),
    (4, 640, 208, 3, "bf16", "bf16"),     # ragged tile blocks
    (3, 640, 208, 5, "bf16", "bf16"),
    (3, 1280, 96, 9, "bf16", "bf16"),
    (4, 1280, 96, 16, "bf16", "bf16"),
    (3, 512, 144, 17, "bf16", "bf16"),
    (4, 384, 64, 33, "bf16", "bf16"),
    (3, 768, 48, 64, "bf16", "bf16"),
    (4, 256, 32, 100, "bf16", "bf16"),
    (3, 256, 32, 130, "bf16", "bf16"),    # two MFMA row blocks
    (4, 512, 64, 1, "f32", "f32"),
    (3, 512, 64, 7, "f32", "f32"),
    (4, 512, 64, 11, "f32", "f32"),       # two GEMV row blocks
    (4, 512, 64, 2, "bf16", "f32"),
    (3, 512, 64, 2, "f32", "bf16"),
]


def _variants(x_dtype, M, K, N):
    out = ["gemv"]
    if x_dtype == "bf16":
        out += ["mfma"] + (["stream"] if stream_ok(K, M, N) else []) + (
            ["resident"] if resident_ok(K, M) else [])
    return out


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "b%d_K%d_N%d_M%d_%s_%s" % c)
def test_small_parity(case):
    bits, K, N, M, xd, sd = case
    p = synth.small(100 + M, bits=bits, K=K, N=N, M=M, x_dtype=xd, sb_dtype=sd)
    r = Runner(p)
    for v in _variants(xd, M, K, N):
        shapes = {"stream": [(0, 0, 0)],
                  "resident": [(0, 0, 0), (1, 0, 0), (2, 0, 0), (3, 0, 0), (4, 0, 0)]}.get(
            v, [(0, 0, 0), (1, 1, 1), (2, 2, 2), (1, 4, 3), (2, 4, 1), (4, 1, 2)])
        for ntw, kw, s in shapes:
            if s > K // 128:
                continue
            label = "%s %s ntw=%d kwaves=%d S=%d" % (case, v, ntw, kw, s)
            say(label)
            y = r.run(variant=v, ntw=ntw, kwaves=kw, splitk=s)
            check_against_oracle(p, y, label=label)


def _random_cases(seed, n):
    rng = np.random.default_rng(seed)
    return [(int(rng.choice([3, 4])), 128 * int(rng.integers(1, 49)), 16 * int(rng.integers(1, 41)),
             int(rng.integers(1, 21))) for _ in range(n)]


RANDOM = _random_cases(20261203, 24)


@pytest.mark.parametrize("case", RANDOM, ids=lambda c: "b%d_K%d_N%d_M%d" % c)
def test_random_shapes_every_family(case):
    """Seeded random shapes (K a multiple of 128 up to 6144, N a multiple of
    16 up to 640, 1..20 rows) on every family that takes them, default
    launch shapes: indexing that depends on the shape (chunks per wave, tile
    slots, ragged waves and tile groups) is checked away from the fixed
    cases."""
    bits, K, N, M = case
    p = synth.small(5000 + K + N + M, bits=bits, K=K, N=N, M=M)
    r = Runner(p)
    fams = ["auto", "mfma", "gemv"] + (["stream"] if stream_ok(K, M, N) else []) + (
        ["resident"] if resident_ok(K, M) else [])
    for v in fams:
        say("random shape", case, v)
        check_against_oracle(p, r.run(variant=v), label="random %s %s" % (case, v))


# ------------------------------------------------------------------ properties

def test_determinism_and_row_independence():
    p = synth.small(7, bits=3, K=1024, N=320, M=16)
    r = Runner(p)
    for v, ntw, kw, s in (("mfma", 1, 2, 4), ("mfma", 2, 4, 1), ("gemv", 1, 0, 4), ("stream", 0, 0, 0),
                          ("resident", 0, 0, 0)):
        say("determinism", v)
        a = r.run(variant=v, ntw=ntw, kwaves=kw, splitk=s)
        b2 = r.run(variant=v, ntw=ntw, kwaves=kw, splitk=s)
        assert np.array_equal(a, b2)
        if v in ("mfma", "stream", "resident"):
            a9 = r.run(rows=9, variant=v, ntw=ntw, kwaves=kw, splitk=s)
            assert np.array_equal(a9[:9], a[:9])


def test_rows_past_m_and_past_end_untouched():
    import torch
    p = synth.small(8, bits=4, K=512, N=64, M=5)
    r = Runner(p, max_rows=8)
    for v in ("mfma", "gemv", "stream", "resident"):
        say("canary", v)
        out = torch.full((9, 64), 7.0, dtype=torch.bfloat16, device="cuda")
        r.lin.plan.run(r.x[:5], r.lin.codes, r.lin.sb, out=out[:5], variant=v, splitk=2)
        torch.cuda.synchronize()
        o = out.float().cpu().numpy()
        assert np.all(o[5:] == 7.0)
        check_against_oracle(p, b.to_numpy_bits(out[:5]), label="canary " + v)


def test_non_default_stream_and_workspace_reuse():
    import torch
    p = synth.small(9, bits=3, K=1024, N=128, M=16)
    r = Runner(p, max_rows=16)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        for rows in (16, 3, 9, 1, 16):   # tickets must be re-armed between calls
            say("stream/workspace rows", rows)
            y = r.lin.plan.run(r.x[:rows], r.lin.codes, r.lin.sb, variant="mfma", splitk=4,
                               stream=s)
            s.synchronize()
            check_against_oracle(p.rows(rows), b.to_numpy_bits(y), label="rows %d" % rows)


def test_concurrent_streams_with_their_own_workspaces():
    """Two streams run the split-K 64-row kernel on different inputs at the
    same time, each with its own workspace (the ticket words live in the
    workspace, nothing in the library is shared between calls); each result
    must equal the same call run alone, bit for bit, over several rounds."""
    import torch
    probs = [synth.small(31 + i, bits=3, K=5120, N=416, M=64) for i in range(2)]
    lins = [b.QuantizedLinear(p, max_rows=64) for p in probs]
    xs = [b.to_device(p.x) for p in probs]
    need = lins[0].plan.workspace_bytes(64)
    assert need > 0
    wss = [torch.zeros(need, dtype=torch.uint8, device="cuda") for _ in range(2)]
    alone = []
    for lin, x, ws in zip(lins, xs, wss):
        alone.append(lin(x, workspace=ws))
        torch.cuda.synchronize()
        assert lin.plan.stats()["last_splitk"] == 2
    for p, y in zip(probs, alone):
        check_against_oracle(p, b.to_numpy_bits(y), label="alone")
    streams = [torch.cuda.Stream() for _ in range(2)]
    outs = [torch.empty_like(y) for y in alone]
    for rnd in range(4):
        say("concurrent round", rnd)
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        for lin, x, ws, s, o in zip(lins, xs, wss, streams, outs):
            with torch.cuda.stream(s):
                for _ in range(3):  # several launches in flight on each stream
                    lin(x, out=o, workspace=ws, stream=s)
        torch.cuda.synchronize()
        for i, (o, y) in enumerate(zip(outs, alone)):
            assert torch.equal(o.view(torch.int16), y.view(torch.int16)), \
                "stream %d, round %d differs from the call run alone" % (i, rnd)


def test_resident_rejects_blocks_too_long_for_lds():
    p = synth.small(13, bits=4, K=6144, N=32, M=16)   # 16*6144*2 bytes > 160 KB
    r = Runner(p)
    with pytest.raises(b.QmmError) as ei:
        r.run(variant="resident")
    assert ei.value.status == b.QMM_ERR_UNSUPPORTED
    check_against_oracle(p, r.run(rows=13, variant="resident"), rows=13, label="13 rows fit")


@pytest.mark.parametrize("case", [(3, 640, 208, 3), (4, 1024, 400, 1), (4, 640, 208, 16),
                                  (4, 15360, 48, 4), (3, 10240, 80, 7)],
                         ids=lambda c: "b%d_K%d_N%d_M%d" % c)
def test_resident_every_slot_count(case):
    """Four-wave workgroups (one wave per SIMD) issue the unpack and the MFMAs
    that read its results back to back; every slot count must match the oracle.
    The long-K cases run the sixteen-wave shapes (up to 128 chunks, some
    waves with fewer chunks than others)."""
    bits, K, N, M = case
    p = synth.small(100 + M, bits=bits, K=K, N=N, M=M)
    r = Runner(p)
    for tm in (1, 2, 3, 4):
        say(case, "resident tm", tm)
        check_against_oracle(p, r.run(variant="resident", ntw=tm), label="%s tm=%d" % (case, tm))


def test_stream_rejects_shapes_it_does_not_cover():
    # K past 128 chunks of 128: no wave shape of the streaming kernel covers it
    p = synth.small(11, bits=3, K=16512, N=32, M=1)
    r = Runner(p)
    with pytest.raises(b.QmmError) as ei:
        r.run(variant="stream")
    assert ei.value.status == b.QMM_ERR_UNSUPPORTED
    check_against_oracle(p, r.run(), label="auto falls back")   # auto picks another family
    # 260 tiles (more than one pass over the compute units) leave 64 KB of LDS
    # per workgroup: one row of K=16384 fits the 16 waves' slices, two do not
    p = synth.small(12, bits=4, K=16384, N=4160, M=2)
    r = Runner(p)
    with pytest.raises(b.QmmError) as ei:
        r.run(variant="stream")
    assert ei.value.status == b.QMM_ERR_UNSUPPORTED
    check_against_oracle(p, r.run(rows=1, variant="stream"), rows=1, label="one row fits")


def test_large_n_every_default_family():
    """131072 outputs (8192 W tiles, grids far beyond one pass over the
    compute units): the default family at 1, 9, 40 and 100 rows (streaming,
    resident, MFMA, wide), checked on sampled outputs."""
    p = synth.small(14, bits=4, K=256, N=131072, M=100)
    r = Runner(p)
    for rows, fam in ((1, "stream"), (9, "resident"), (40, "mfma"), (100, "wide")):
        say("large N rows", rows)
        y = r.run(rows=rows)
        assert r.lin.plan.stats()["last_variant"] == fam, (rows, r.lin.plan.stats())
        check_against_oracle(p, y, rows=rows, sample=(2000, rows), label="large N rows %d" % rows,
                             bf16_weights=fam == "wide")


def test_stats_report_the_family_that_ran():
    p = synth.small(10, bits=4, K=512, N=64, M=4)
    r = Runner(p)
    r.run(variant="gemv")
    st = r.lin.plan.stats()
    assert st["last_variant"] == "gemv" and st["launches"]["gemv"] >= 1
    r.run(variant="mfma")
    st = r.lin.plan.stats()
    assert st["last_variant"] == "mfma" and st["launches"]["mfma"] >= 1
    r.run(rows=2)  # one or two rows: the streaming kernel by default
    st = r.lin.plan.stats()
    assert st["last_variant"] == "stream" and st["launches"]["stream"] >= 1
    r.run()  # 4 rows whose activations fit one compute unit's LDS: resident
    st = r.lin.plan.stats()
    assert st["last_variant"] == "resident" and st["launches"]["resident"] >= 1


# ------------------------------------------------------------------ workloads

@pytest.mark.parametrize("variant", ["auto", "gemv"])
def test_workload0_full(variant):
    (p,) = synth.workload(0)
    say("workload 0", variant)
    r = Runner(p)
    check_against_oracle(p, r.run(variant=variant), label="w0 " + variant)


@pytest.mark.parametrize("variant", ["auto", "gemv", "mfma", "stream", "resident"])
def test_workload1_full(variant):
    (p,) = synth.workload(1)
    say("workload 1", variant)
    r = Runner(p)
    check_against_oracle(p, r.run(variant=variant), label="w1 " + variant)


@pytest.mark.parametrize("rows", synth.C2_ROWS)
def test_workload2_full(rows):
    (p,) = synth.workload(2)
    r = Runner(p, max_rows=64)
    variants = ["auto", "mfma", "resident", "slab"] + (["gemv"] if rows <= 9 else []) + (
        ["stream"] if stream_ok(p.K, rows, p.N) else [])
    for v in variants:
        say("workload 2 rows", rows, v)
        check_against_oracle(p.rows(rows), r.run(rows=rows, variant=v), rows=rows,
                             label="w2 M=%d %s" % (rows, v))


def test_workload3_full():
    for p in synth.workload(3):
        r = Runner(p)
        for v in ("auto", "gemv", "mfma") + (("stream",) if stream_ok(p.K, p.M, p.N) else ()) + (
                ("resident",) if resident_ok(p.K, p.M) else ()):
            say("workload 3", p.name, v)
            check_against_oracle(p, r.run(variant=v), label="w3 %s %s" % (p.name, v))
        del r


SLAB = [
    # bits, K, N, M, sb_dtype: ragged tile slots (N/16 not a multiple of 3), both row-tile
    # widths, two row blocks, f32 scales
    (3, 5120, 208, 17, "bf16"),
    (4, 5120, 208, 32, "bf16"),
    (3, 5120, 176, 33, "bf16"),
    (4, 5120, 48, 64, "f32"),
    (3, 5120, 80, 100, "bf16"),
    (4, 8192, 112, 40, "bf16"),
    (3, 8192, 64, 9, "f32"),
]


@pytest.mark.parametrize("case", SLAB, ids=lambda c: "b%d_K%d_N%d_M%d_%s" % c)
def test_slab_parity(case):
    bits, K, N, M, sd = case
    p = synth.small(300 + M, bits=bits, K=K, N=N, M=M, sb_dtype=sd)
    r = Runner(p)
    say("slab", case)
    check_against_oracle(p, r.run(variant="slab"), label="slab %s" % (case,))


@pytest.mark.parametrize("case", [(3, 5120, 208, 17, "bf16"), (4, 5120, 176, 32, "f32"),
                                  (3, 5120, 96, 64, "bf16"), (4, 8192, 112, 40, "bf16"),
                                  (3, 8192, 64, 29, "bf16"), (3, 5120, 208, 33, "bf16"),
                                  (4, 5120, 96, 48, "f32"), (3, 8192, 160, 49, "bf16")],
                         ids=lambda c: "b%d_K%d_N%d_M%d_%s" % c)
def test_slab_split_and_unsplit_forms(case):
    """Both slab forms on one problem: the split form (six W tiles per
    workgroup, K in two parts added through the workspace; ragged tile groups
    where N/16 is not a multiple of 6; three row tiles at 33..48 rows, four
    above) and the unsplit form, twice in a row so the workspace's tickets
    are reused."""
    bits, K, N, M, sd = case
    p = synth.small(700 + M, bits=bits, K=K, N=N, M=M, sb_dtype=sd)
    r = Runner(p)
    for ntw, sk in ((2, 2), (1, 0), (2, 2)):
        say("slab form ntw", ntw, "splitk", sk, case)
        y = r.run(variant="slab", ntw=ntw, splitk=sk)
        st = r.lin.plan.stats()
        assert st["last_splitk"] == (2 if ntw == 2 else 1)
        check_against_oracle(p, y, label="slab ntw=%d %s" % (ntw, case))


def test_slab_rejects_unbuilt_k():
    p = synth.small(14, bits=4, K=1024, N=32, M=20)
    r = Runner(p)
    with pytest.raises(b.QmmError) as ei:
        r.run(variant="slab")
    assert ei.value.status == b.QMM_ERR_UNSUPPORTED


def test_resident_and_slab_more_tiles_than_workgroups():
    """More tiles than one pass of resident workgroups holds (N/16 > 4 x compute
    units forces the resident kernel's fallback slot count) and ragged slab
    tile slots at K=8192."""
    p = synth.small(12, bits=3, K=640, N=16400, M=5)
    r = Runner(p)
    for tm in (1, 4):
        say("resident tm", tm)
        check_against_oracle(p, r.run(variant="resident", ntw=tm), label="resident tm=%d" % tm)
    q = synth.small(15, bits=4, K=8192, N=16 * 260, M=20)
    rq = Runner(q)
    say("slab ragged K=8192")
    check_against_oracle(q, rq.run(variant="slab"), label="slab ragged")


@pytest.mark.parametrize("variant", ["auto", "wide", "slab", "mfma"])
def test_workload4_sampled(variant):
    (p,) = synth.workload(4)
    say("workload 4", variant)
    r = Runner(p)
    y = r.run(variant=variant)
    check_against_oracle(p, y, sample=(3000, 4), label="w4 sampled " + variant,
                         bf16_weights=variant in ("auto", "wide"))
    # every output row and column is finite and rows are distinct results
    yf = oracle.decode_bf16(y)
    assert np.all(np.isfinite(yf))


def test_workload4_families_agree_everywhere():
    """All 128 x 28672 outputs of the 4-bit 8192 -> 28672 block, from three
    kernel families: the wide kernel (bf16-rounded weights, no per-group
    epilogue) and the split slab and MFMA kernels (the factored form).  Each
    is within the acceptance bound of the exact result where the oracle
    samples it, so at every output any two must agree within twice that
    bound; a missing, stale or misplaced tile in one of them shows as a gap
    of the outputs' own size.  Most outputs agree to a small fraction of it."""
    (p,) = synth.workload(4)
    say("workload 4, every output, three families")
    r = Runner(p)
    ys = {v: y_to_f64(r.run(variant=v), p.x_dtype) for v in ("wide", "slab", "mfma")}
    sx, mw = oracle.bound_terms(p.bits, p.K, p.x, p.w, p.scales, p.biases)
    tol = oracle.tolerance_coefficient(p.x_dtype) * np.outer(sx, mw) + 1e-6
    for v, y in ys.items():
        assert y.shape == (p.M, p.N) and np.all(np.isfinite(y)), v
    for a, c in (("wide", "mfma"), ("slab", "mfma")):
        ratio = np.abs(ys[a] - ys[c]) / tol
        worst = np.unravel_index(np.argmax(ratio), ratio.shape)
        assert ratio.max() <= 2.0, "%s vs %s: ratio %.3f at %s" % (a, c, ratio.max(), worst)
        assert np.median(ratio) < 0.01, "%s vs %s: median ratio %.4f" % (a, c, np.median(ratio))


@pytest.mark.parametrize("bits", [3, 4])
def test_degenerate_weights_every_family(bits):
    """Zero scales and biases give exact zeros; a zero activation block gives
    exact zeros; all-maximum codes (every word all ones) match the oracle; in
    every kernel family that takes the shape."""
    import dataclasses
    base = synth.small(60 + bits, bits=bits, K=5120, N=48, M=3)
    zero_sb = dataclasses.replace(base, scales=np.zeros_like(base.scales),
                                  biases=np.zeros_like(base.biases))
    zero_x = dataclasses.replace(base, x=np.zeros_like(base.x))
    max_codes = dataclasses.replace(base, w=np.full_like(base.w, 0xFFFFFFFF))
    variants = ["auto", "gemv", "mfma", "stream", "resident", "slab"]
    for label, p in (("zero scales and biases", zero_sb), ("zero activations", zero_x)):
        r = Runner(p)
        for v in variants:
            say("degenerate", bits, label, v)
            y = y_to_f64(r.run(variant=v), p.x_dtype)
            assert np.all(y == 0.0), "%s %s: %s" % (label, v, y[y != 0][:4])
    r = Runner(max_codes)
    for v in variants:
        say("degenerate", bits, "all-maximum codes", v)
        check_against_oracle(max_codes, r.run(variant=v), label="max codes %s" % v)


def test_degenerate_weights_generic_formats():
    import dataclasses
    for bits, gs in ((2, 32), (8, 128)):
        base = synth.small(70 + bits, bits=bits, K=1024, N=32, M=2, group_size=gs)
        zero_sb = dataclasses.replace(base, scales=np.zeros_like(base.scales),
                                      biases=np.zeros_like(base.biases))
        y = y_to_f64(Runner(zero_sb).run(), base.x_dtype)
        assert np.all(y == 0.0)
        max_codes = dataclasses.replace(base, w=np.full_like(base.w, 0xFFFFFFFF))
        check_against_oracle(max_codes, Runner(max_codes).run(), label="max codes b%d" % bits)


WIDE = [
    # bits, K, N, M, sb_dtype: one and many slices, ragged tile groups (N/16 not a
    # multiple of 8), a second row block, f32 scales
    (3, 5120, 208, 65, "bf16"),
    (4, 8192, 112, 128, "bf16"),
    (4, 5120, 48, 100, "f32"),
    (3, 256, 16, 130, "bf16"),
    (4, 2048, 400, 97, "bf16"),
    (3, 5120, 208, 96, "bf16"),
    (4, 1024, 144, 80, "f32"),
]


@pytest.mark.parametrize("case", WIDE, ids=lambda c: "b%d_K%d_N%d_M%d_%s" % c)
def test_wide_parity(case):
    """The wide kernel (65..128 rows per launch, weights dequantized to bf16;
    six row tiles up to 96 rows (65, 80, 96 and the 2-row tail of 130), eight
    above), forced: these N are too small for it to be the default."""
    bits, K, N, M, sd = case
    p = synth.small(800 + M, bits=bits, K=K, N=N, M=M, sb_dtype=sd)
    r = Runner(p)
    say("wide", case)
    y = r.run(variant="wide")
    assert r.lin.plan.stats()["last_variant"] == "wide"
    check_against_oracle(p, y, label="wide %s" % (case,), bf16_weights=True)
    # the same rows through the slab or MFMA families agree within the bound too
    check_against_oracle(p, r.run(variant="mfma"), label="mfma %s" % (case,))


def test_rows_above_64_dispatch():
    """Above 64 rows the wide kernel is the default only where its grid (eight
    W tiles per workgroup) fills at least half the compute units; else the
    rows run in 64-row blocks on another family."""
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    big_n = 16 * 8 * ((cus + 1) // 2)           # exactly half the units
    for N, want_wide in ((big_n, True), (big_n // 2, False)):
        p = synth.small(900 + N % 97, bits=4, K=256, N=N, M=100)
        r = Runner(p)
        say("rows above 64, N", N)
        y = r.run()
        fam = r.lin.plan.stats()["last_variant"]
        assert (fam == "wide") == want_wide, (N, fam)
        check_against_oracle(p, y, label="dispatch N=%d (%s)" % (N, fam),
                             bf16_weights=fam == "wide")


def test_blocks_of_a_long_call_pick_their_own_family():
    """A 65- and an 80-row call where the wide kernel is not the default run
    a 64-row block on the slab family, then the last block on the family of
    its own row count (one row: streaming; 16 rows: resident)."""
    for M, last in ((65, "stream"), (80, "resident")):
        p = synth.small(950 + M, bits=3, K=5120, N=208, M=M)
        r = Runner(p)
        say("long call", M)
        before = dict(r.lin.plan.stats()["launches"])
        y = r.run()
        st = r.lin.plan.stats()
        assert st["last_variant"] == last, (M, st)
        assert st["launches"]["slab"] == before["slab"] + 1, (M, st)
        check_against_oracle(p, y, label="long call M=%d" % M)


def test_wide_rejects_k_not_multiple_of_256():
    p = synth.small(16, bits=4, K=640, N=32, M=70)
    r = Runner(p)
    with pytest.raises(b.QmmError) as ei:
        r.run(variant="wide")
    assert ei.value.status == b.QMM_ERR_UNSUPPORTED
    check_against_oracle(p, r.run(), label="K=640 above 64 rows")


# ------------------------------------------------------------------ f32 outputs

def _families(p, rows):
    """Every family that takes `rows` rows of problem p (bf16 activations)."""
    out = ["auto", "mfma"]
    if rows <= 8:
        out.append("gemv")
    if stream_ok(p.K, rows, p.N):
        out.append("stream")
    if resident_ok(p.K, rows):
        out.append("resident")
    if p.K in (5120, 8192) and rows >= 9:
        out.append("slab")
    return out


@pytest.mark.parametrize("widx,rows", [(1, 1), (2, 1), (2, 9), (2, 16), (2, 32), (2, 48),
                                       (2, 64)])
def test_f32_outputs_full_workloads(widx, rows):
    """QMM_FLAG_F32_OUT: the f32 sums themselves at the full 5120 -> 10240
    shapes, every family that takes the row count, against the strict bound
    of an f32 evaluation of the factored form (no bf16 rounding to hide
    behind) and the median check at the rounding level."""
    (p,) = synth.workload(widx, M=64) if widx == 2 else synth.workload(widx)
    r = Runner(p, max_rows=max(rows, p.M), f32_out=True)
    q = p.rows(rows)
    for v in _families(q, rows):
        say("f32 out workload", widx, "rows", rows, v)
        y = r.run(rows=rows, variant=v)
        assert y.dtype == np.float32
        check_against_oracle(q, y, rows=rows, label="f32 out w%d M=%d %s" % (widx, rows, v),
                             out_dtype="f32")


def test_f32_outputs_mlp_trio():
    for p in synth.workload(3):
        r = Runner(p, f32_out=True)
        for v in _families(p, p.M):
            say("f32 out workload 3", p.name, v)
            check_against_oracle(p, r.run(variant=v), label="f32 out w3 %s %s" % (p.name, v),
                                 out_dtype="f32")
        del r


@pytest.mark.parametrize("variant", ["auto", "wide", "slab", "mfma"])
def test_f32_outputs_workload4_sampled(variant):
    (p,) = synth.workload(4)
    say("f32 out workload 4", variant)
    r = Runner(p, f32_out=True)
    check_against_oracle(p, r.run(variant=variant), sample=(3000, 5),
                         label="f32 out w4 " + variant, out_dtype="f32",
                         bf16_weights=variant in ("auto", "wide"))


@pytest.mark.parametrize("case", [(4, 512, 64, 1, "f32", "f32"), (3, 640, 208, 5, "bf16", "bf16"),
                                  (4, 1280, 96, 16, "bf16", "f32"), (3, 768, 48, 64, "bf16", "bf16"),
                                  (4, 256, 32, 100, "bf16", "bf16")],
                         ids=lambda c: "b%d_K%d_N%d_M%d_%s_%s" % c)
def test_f32_outputs_small(case):
    """f32 outputs on ragged small shapes, every family and K split."""
    bits, K, N, M, xd, sd = case
    p = synth.small(400 + M, bits=bits, K=K, N=N, M=M, x_dtype=xd, sb_dtype=sd)
    r = Runner(p, f32_out=True)
    fams = ["gemv"] if xd == "f32" else _families(p, M) + (["wide"] if M > 64 else [])
    for v in fams:
        for s in (0, 2):
            if v not in ("gemv", "mfma") and s:
                continue
            label = "f32 out %s %s S=%d" % (case, v, s)
            say(label)
            check_against_oracle(p, r.run(variant=v, splitk=s), label=label, out_dtype="f32",
                                 bf16_weights=v == "wide")


def test_f32_output_rows_past_m_untouched():
    import torch
    p = synth.small(18, bits=3, K=5120, N=96, M=40)
    r = Runner(p, max_rows=48, f32_out=True)
    for v in ("auto", "slab", "mfma", "resident"):
        rows = 16 if v == "resident" else 40
        say("f32 out canary", v)
        out = torch.full((rows + 3, 96), 7.0, dtype=torch.float32, device="cuda")
        r.lin.plan.run(r.x[:rows], r.lin.codes, r.lin.sb, out=out[:rows], variant=v)
        torch.cuda.synchronize()
        o = out.cpu().numpy()
        assert np.all(o[rows:] == 7.0)
        check_against_oracle(p.rows(rows), o[:rows], label="f32 canary " + v, out_dtype="f32")


def test_wide_call_tail_picks_its_own_family():
    """A 129-row call on a shape where the wide kernel is the default: one
    128-row block on the wide kernel, then the one-row tail on the streaming
    kernel (not a second wide launch padded to 96 rows)."""
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    N = 16 * 8 * cus
    p = synth.small(129, bits=4, K=256, N=N, M=129)
    r = Runner(p)
    before = dict(r.lin.plan.stats()["launches"])
    y = r.run()
    st = r.lin.plan.stats()
    assert st["launches"]["wide"] == before["wide"] + 1, st
    assert st["last_variant"] == "stream", st
    check_against_oracle(p, y, sample=(3000, 129), label="129 rows", bf16_weights=True)
