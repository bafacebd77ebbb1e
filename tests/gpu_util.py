"""Helpers for the GPU parity tests: run a problem through the C ABI and
compare with the float64 oracle element by element."""
import sys

import numpy as np

import oracle
from bit_quantized_matmul_affine_amd import binding as b


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def stream_shape(K: int):
    """(waves, chunks per wave) of the streaming kernel for this K, or None."""
    nC = K // 128
    for nw, cpw in ((4, 2), (4, 4), (8, 4), (8, 5), (8, 8), (16, 8)):
        if (nC < 16) != (nw == 4):
            continue
        if nC <= nw * cpw:
            return nw, cpw
    return None


def stream_ok(K: int, rows: int, N: int = 1 << 30) -> bool:
    """Whether the streaming kernel takes blocks of `rows` rows at this K (it
    runs at most 4 rows per launch; each wave stages its chunks' activation
    slices and their group sums in LDS: 64 KB per workgroup, or all 160 KB
    when the N/16 tiles fit in one pass over the 256 compute units)."""
    shape = stream_shape(K)
    if shape is None:
        return False
    nw, cpw = shape
    rows = min(rows, 4)
    lds_cap = 160 * 1024 if N // 16 <= 256 else 65536
    return nw * rows * (cpw * 256 + 16 + cpw * 8) + (nw - 1) * 1024 <= lds_cap


def resident_ok(K: int, rows: int) -> bool:
    """Whether the resident kernel takes a block of `rows` rows at this K
    (the whole activation block of up to 16 rows in one compute unit's LDS,
    K covered by at most 64 chunks of 128)."""
    return min(rows, 16) * K * 2 <= 160 * 1024 and K // 128 <= 64


def y_to_f64(y_bits: np.ndarray, x_dtype: str) -> np.ndarray:
    if x_dtype == "bf16":
        return oracle.decode_bf16(y_bits)
    return y_bits.astype(np.float64)


class Runner:
    """A problem on the device: plan, native weights, activations."""

    def __init__(self, p, max_rows=None, device="cuda", f32_out=False):
        import torch
        self.p = p
        self.lin = b.QuantizedLinear(p, max_rows=max_rows or p.M, device=device, f32_out=f32_out)
        self.x = b.to_device(p.x, device)
        torch.cuda.synchronize()

    def run(self, rows=None, **kw):
        import torch
        rows = rows or self.p.M
        y = self.lin(self.x[:rows], **kw)
        torch.cuda.synchronize()
        return b.to_numpy_bits(y)


# oracle results of the last few full checks (the same problem is checked
# once per kernel family); keyed by the input arrays, verified on every hit
_ORACLE_CACHE = {}


def check_against_oracle(p, y_bits, rows=None, sample=None, threads=8, label="",
                         out_dtype=None, bf16_weights=False):
    """The output block against the float64 oracle (oracle.check_outputs):
    every element within the acceptance bound c*sum|x|*max|W| + 1e-6, every
    element within the strict bound of an f32 evaluation of the factored form
    (plus half a bf16 step for bf16 outputs), and the median error at the
    rounding level.  sample=(count, seed) checks a random subset computed one
    by one by the oracle.  out_dtype: the dtype y was written in (x's dtype
    unless the plan asked for f32 outputs).  bf16_weights: the output came
    from the wide kernel, whose matrix-core products take bf16-rounded
    weights (the strict bound then adds their rounding, 2^-9 of the terms).
    Returns the worst ratio to the acceptance bound."""
    wr = oracle.BF16_WEIGHT_ROUNDING if bf16_weights else 0.0
    rows = rows or p.M
    out_dtype = out_dtype or p.x_dtype
    y = y_to_f64(y_bits, out_dtype)[:rows]
    x = p.x[:rows]
    gs = getattr(p, "group_size", 64)
    sx, mw = oracle.bound_terms(p.bits, p.K, x, p.w, p.scales, p.biases, group_size=gs)
    c = oracle.tolerance_coefficient(p.x_dtype)
    assert np.all(np.isfinite(y)), label + ": non-finite output"
    if sample is None:
        key = (p.bits, p.K, p.N, rows, gs, p.w.ctypes.data, x.ctypes.data, p.scales.ctypes.data,
               p.biases.ctypes.data, p.x_dtype, p.sb_dtype)
        hit = _ORACLE_CACHE.get(key)
        if hit is None or not all(np.array_equal(u, v) for u, v in zip(hit[0], (p.w, x, p.scales,
                                                                               p.biases))):
            ref = oracle.matmul(p.bits, p.K, x, p.w, p.scales, p.biases, group_size=gs,
                                threads=threads)
            acc = oracle.accumulation_terms(p.bits, p.K, x, p.w, p.scales, p.biases,
                                            group_size=gs, threads=threads)
            if len(_ORACLE_CACHE) >= 4:
                _ORACLE_CACHE.pop(next(iter(_ORACLE_CACHE)))
            _ORACLE_CACHE[key] = ((p.w.copy(), x.copy(), p.scales.copy(), p.biases.copy()),
                                  ref, acc)
        else:
            ref, acc = hit[1], hit[2]
        tol = c * np.outer(sx, mw) + 1e-6
        got = y
    else:
        count, seed = sample
        rng = np.random.default_rng(seed)
        ms = rng.integers(0, rows, count)
        ns = rng.integers(0, p.N, count)
        ref = oracle.matmul_at(p.bits, p.K, x, p.w, p.scales, p.biases, ms, ns, group_size=gs)
        acc = oracle.accumulation_terms_at(p.bits, p.K, x, p.w, p.scales, p.biases, ms, ns,
                                           group_size=gs)
        tol = c * sx[ms] * mw[ns] + 1e-6
        got = y[ms, ns]
    r = oracle.check_outputs(got, ref, acc, tol, p.K, out_dtype, wr)
    err = np.abs(got - ref)
    worst = np.unravel_index(np.argmax(err / tol), err.shape)
    assert r["bound"] <= 1.0, "%s: err %.3g > tol %.3g at %s (ratio %.3f)" % (
        label, err[worst], tol[worst], worst, r["bound"])
    st = oracle.strict_tolerance(ref, acc, p.K, out_dtype, wr)
    ws = np.unravel_index(np.argmax(err / st), err.shape)
    assert r["strict"] <= 1.0, "%s: err %.3g > strict %.3g at %s (ratio %.3f)" % (
        label, err[ws], st[ws], ws, r["strict"])
    assert r["median"] <= r["median_cap"], "%s: median error ratio %.3g > %.3g" % (
        label, r["median"], r["median_cap"])
    return r["bound"]
