"""GPU parity of decode attention over an affine-quantized KV cache
(qmm_decode_attention) against the float64 oracle's decode_attention()
("mlx-bun 0.0.4" page, fused-decode-kernel.ts): every output within the
derived bound, at least 95 % of them within one bf16 step of the oracle
(a score's rounding rarely flips), bitwise-repeatable runs, and exact
agreement up to one bf16 step where the scores are exact by construction."""
import numpy as np
import pytest

import oracle
from bit_quantized_matmul_affine_amd import binding as b, synth
from tests.gpu_util import say

pytestmark = pytest.mark.gpu


def _dev(cache):
    return tuple(b.to_device(x) for x in cache)


def _ref(q, k, v, bits, gs):
    d = oracle.decode_bf16
    args = (d(q), k[0], d(k[1]), d(k[2]), v[0], d(v[1]), d(v[2]), bits, gs)
    out = oracle.decode_attention(*args)
    return out, oracle.decode_attention_tolerance(out, *args)


def _run(q, k, v, bits, gs):
    import torch
    out = b.decode_attention(b.to_device(q), _dev(k), _dev(v), bits, gs)
    torch.cuda.synchronize()
    return oracle.decode_bf16(b.to_numpy_bits(out))


def _check(got, ref, tol, label, within_step=0.95):
    assert np.all(np.isfinite(got)), label + ": non-finite output"
    err = np.abs(got - ref)
    worst = np.unravel_index(np.argmax(err / tol), err.shape)
    assert err[worst] <= tol[worst], "%s: err %.3g > tol %.3g at %s" % (
        label, err[worst], tol[worst], worst)
    step = 2.0 ** -7 * np.abs(ref) + 1e-6
    frac = float(np.mean(err <= step))
    assert frac >= within_step, "%s: only %.3f of outputs within one bf16 step" % (label, frac)
    return frac


CASES = [
    # H, KV, N, D, bits, group size: one row, one partial block, ragged blocks,
    # every head-group width, both code widths, every group size
    (4, 4, 1, 128, 4, 64),
    (2, 1, 127, 256, 8, 32),
    (8, 2, 257, 128, 4, 128),
    (2, 2, 300, 512, 8, 128),
    (8, 1, 1000, 128, 8, 32),
    (4, 2, 2048, 512, 4, 32),
    (16, 4, 513, 256, 4, 64),
    (16, 8, 4099, 256, 8, 64),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "H%d_KV%d_N%d_D%d_b%d_g%d" % c)
def test_matches_oracle(case):
    H, KV, N, D, bits, gs = case
    say("attention", case)
    q, k, v = synth.attention_inputs(900 + N, H=H, KV=KV, N=N, D=D, bits=bits, group_size=gs)
    ref, tol = _ref(q, k, v, bits, gs)
    got = _run(q, k, v, bits, gs)
    _check(got, ref, tol, "attention %s" % (case,))


def _random_attention_cases(seed, n):
    # supported shapes only: D in {128, 256, 512}, H/KV in {1, 2, 4, 8} with
    # D * H/KV <= 1024; N from one row to a dozen blocks (ragged last block)
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        D = int(rng.choice([128, 256, 512]))
        rep = int(rng.choice([1, 2, 4, 8]))
        if D * rep > 1024:
            continue
        KV = int(rng.integers(1, 5))
        out.append((KV * rep, KV, int(rng.integers(1, 3073)), D, int(rng.choice([4, 8])),
                    int(rng.choice([32, 64, 128]))))
    return out


@pytest.mark.parametrize("case", _random_attention_cases(20261205, 12),
                         ids=lambda c: "H%d_KV%d_N%d_D%d_b%d_g%d" % c)
def test_random_shapes(case):
    # seeded random shapes: block counts, ragged last blocks, head groups and
    # code widths away from the fixed cases
    H, KV, N, D, bits, gs = case
    say("random attention", case)
    q, k, v = synth.attention_inputs(3000 + N + D, H=H, KV=KV, N=N, D=D, bits=bits, group_size=gs)
    ref, tol = _ref(q, k, v, bits, gs)
    got = _run(q, k, v, bits, gs)
    _check(got, ref, tol, "random attention %s" % (case,))


def test_full_size_and_repeatable():
    # 16 query heads over 8 KV heads of 256 values, 8192 cached rows, 4-bit
    # group-64 keys and values
    say("attention 16x8 heads, D=256, N=8192")
    q, k, v = synth.attention_inputs(11, H=16, KV=8, N=8192, D=256, bits=4, group_size=64)
    ref, tol = _ref(q, k, v, 4, 64)
    got = _run(q, k, v, 4, 64)
    frac = _check(got, ref, tol, "attention full size")
    say("within one bf16 step:", frac)
    again = _run(q, k, v, 4, 64)
    assert np.array_equal(again, got)


def test_reused_workspace():
    # one workspace serves call after call (the partial outputs and block
    # statistics are rewritten by each call before the merge reads them)
    import torch
    H, KV, N, D = 16, 8, 4099, 256
    q, k, v = synth.attention_inputs(21, H=H, KV=KV, N=N, D=D, bits=4, group_size=64)
    qd, kd, vd = b.to_device(q), _dev(k), _dev(v)
    need = b.lib().qmm_attention_workspace_bytes(H, N, D)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")  # no zero-fill needed
    outs = []
    for _ in range(3):
        outs.append(b.to_numpy_bits(b.decode_attention(qd, kd, vd, 4, 64, workspace=ws)))
        torch.cuda.synchronize()
    assert all(np.array_equal(o, outs[0]) for o in outs)
    ref, tol = _ref(q, k, v, 4, 64)
    _check(oracle.decode_bf16(outs[0]), ref, tol, "attention, reused workspace")


def test_exact_scores_agree_within_one_step():
    # integer queries, small codes, key scale 1/8: every score's f32 sum is
    # exact, so both sides round the same value and only the f32 sums of the
    # weights and values differ from the oracle
    rng = np.random.default_rng(3)
    H, KV, N, D = 4, 2, 700, 128
    q = synth.f32_to_bf16_bits(rng.integers(-2, 3, (H, D)).astype(np.float32))
    codes = rng.integers(0, 4, (KV, N, D))
    one = synth.f32_to_bf16_bits(np.float32(0.125))
    ks = np.full((KV, N, D // 64), one, dtype=np.uint16)
    kb = np.full((KV, N, D // 64), synth.f32_to_bf16_bits(np.float32(-0.25)), dtype=np.uint16)
    k = (synth.pack_lsb(codes, 4), ks, kb)
    _, _, v = synth.attention_inputs(4, H=H, KV=KV, N=N, D=D, bits=4, group_size=64)
    ref, scores = oracle.decode_attention(
        oracle.decode_bf16(q), k[0], oracle.decode_bf16(ks), oracle.decode_bf16(kb), v[0],
        oracle.decode_bf16(v[1]), oracle.decode_bf16(v[2]), 4, 64, return_scores=True)
    assert np.array_equal(scores, np.round(scores * 8) / 8)  # exact multiples of 1/8
    got = _run(q, k, v, 4, 64)
    err = np.abs(got - ref)
    assert np.all(err <= 2.0 ** -7 * np.abs(ref) + 1e-6), float(np.max(err))


def test_rejects_unsupported_and_bad_arguments():
    import torch
    q, k, v = synth.attention_inputs(5, H=4, KV=2, N=300, D=128, bits=4, group_size=64)
    qd, kd, vd = b.to_device(q), _dev(k), _dev(v)
    for bits, gs, match in ((3, 64, "bits"), (4, 16, "group_size")):
        with pytest.raises(b.QmmError, match=match):
            b.decode_attention(qd, kd, vd, bits, gs)
    with pytest.raises(b.QmmError, match="workspace"):
        b.decode_attention(qd, kd, vd, 4, 64, workspace=torch.empty(16, dtype=torch.uint8,
                                                                        device="cuda"))
    q3 = b.to_device(synth.attention_inputs(6, H=3, KV=2, N=4, D=128, bits=4, group_size=64)[0])
    with pytest.raises(b.QmmError, match="multiple of KV"):
        b.decode_attention(q3, kd, vd, 4, 64)
