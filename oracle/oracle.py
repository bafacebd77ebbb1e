"""ctypes front end of the float64 CPU oracle (``qmm_oracle.c``).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

Decoding of the stored input dtypes to float64 lives here:
  * f32 values widen exactly;
  * a bf16 value is the upper half of an f32, so its bits shifted left by 16
    and read as f32 give the exact value.
Everything else (unpack, dequantize, dot product) is in the C file, which
follows the plain definition from the pages one step at a time.

Acceptance bound used by the parity tests (an element-wise bound, checked per
output element):
    |y(m,n) - y_ref(m,n)| <= c * sum_k |x(m,k)| * max_k |W(n,k)| + 1e-6
with c = 1e-3 for f32 activations and c = 8e-3 for bf16 activations.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qmm_oracle.c")
_LIB = os.path.join(_HERE, "libqmm_oracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (-O2, no fast-math, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(
            ["gcc", "-O2", "-fno-fast-math", "-fopenmp", "-shared", "-fPIC",
             "-std=c11", "-Wall", "-o", tmp, _SRC, "-lm"],
            check=True,
        )
        os.replace(tmp, _LIB)
    return _LIB


def load_library(path: str):
    """Open an oracle shared object and declare its entry points."""
    lib = ctypes.CDLL(path)
    i64, i32 = ctypes.c_int64, ctypes.c_int
    p = ctypes.c_void_p
    lib.qmm_oracle_unpack.argtypes = [i32, i64, i64, p, p]
    lib.qmm_oracle_matmul.argtypes = [i32, i64, i64, i64, i64, p, p, p, p, p, i32]
    lib.qmm_oracle_matmul_at.argtypes = [i32, i64, i64, i64, i64, p, p, p, p, i64, p, p, p]
    lib.qmm_oracle_bound_terms.argtypes = [i32, i64, i64, i64, i64, p, p, p, p, p, p]
    for f in (lib.qmm_oracle_unpack, lib.qmm_oracle_matmul,
              lib.qmm_oracle_matmul_at, lib.qmm_oracle_bound_terms):
        f.restype = ctypes.c_int
    return lib


def _load(lib=None):
    global _lib
    if lib is not None:
        return lib
    with _lock:
        if _lib is None:
            _lib = load_library(build())
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def decode_bf16(raw: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact float64 values."""
    raw = np.ascontiguousarray(raw, dtype=np.uint16)
    return (raw.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def decode_f32(raw: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(raw, dtype=np.float32).astype(np.float64)


def _as_f64(a: np.ndarray) -> np.ndarray:
    """Accepts float64 values, f32 values, or bf16 bit patterns (uint16)."""
    if a.dtype == np.uint16:
        return decode_bf16(a)
    if a.dtype == np.float32:
        return decode_f32(a)
    return np.ascontiguousarray(a, dtype=np.float64)


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise ValueError("oracle %s rejected its arguments" % what)


def unpack(bits: int, K: int, N: int, w: np.ndarray, lib=None) -> np.ndarray:
    """Codes q(n,k) as uint8 [N, K] from MLX-layout words [N, K*bits/32]."""
    w = np.ascontiguousarray(w, dtype=np.uint32)
    if (K * bits) % 32 != 0 or w.size != N * K * bits // 32:
        raise ValueError("packed words do not match K=%d, N=%d, bits=%d" % (K, N, bits))
    codes = np.empty((N, K), dtype=np.uint8)
    _check(_load(lib).qmm_oracle_unpack(bits, K, N, _ptr(w), _ptr(codes)), "unpack")
    return codes


def _prep(bits, K, x, w, scales, biases, group_size):
    x = _as_f64(x)
    M = x.size // K
    x = x.reshape(M, K)
    w = np.ascontiguousarray(w, dtype=np.uint32)
    N = w.size * 32 // (K * bits)
    s = _as_f64(scales).reshape(N, K // group_size)
    b = _as_f64(biases).reshape(N, K // group_size)
    return x, w, s, b, M, N


def matmul(bits: int, K: int, x, w, scales, biases, group_size: int = 64,
           threads: int = 1, lib=None) -> np.ndarray:
    """y = x . W^T in float64 for all rows; returns [M, N]."""
    x, w, s, b, M, N = _prep(bits, K, x, w, scales, biases, group_size)
    y = np.empty((M, N), dtype=np.float64)
    _check(_load(lib).qmm_oracle_matmul(bits, group_size, K, N, M, _ptr(x), _ptr(w),
                                     _ptr(s), _ptr(b), _ptr(y), threads), "matmul")
    return y


def matmul_at(bits: int, K: int, x, w, scales, biases, ms, ns,
              group_size: int = 64) -> np.ndarray:
    """y(ms[i], ns[i]) for sampled output coordinates."""
    x, w, s, b, M, N = _prep(bits, K, x, w, scales, biases, group_size)
    ms = np.ascontiguousarray(ms, dtype=np.int64)
    ns = np.ascontiguousarray(ns, dtype=np.int64)
    out = np.empty(ms.size, dtype=np.float64)
    _check(_load().qmm_oracle_matmul_at(bits, group_size, K, N, M, _ptr(x), _ptr(w),
                                        _ptr(s), _ptr(b), ms.size, _ptr(ms), _ptr(ns),
                                        _ptr(out)), "matmul_at")
    return out


def bound_terms(bits: int, K: int, x, w, scales, biases, group_size: int = 64):
    """(sum_k |x(m,k)| [M], max_k |W(n,k)| [N])."""
    x, w, s, b, M, N = _prep(bits, K, x, w, scales, biases, group_size)
    sx = np.empty(M, dtype=np.float64)
    mw = np.empty(N, dtype=np.float64)
    _check(_load().qmm_oracle_bound_terms(bits, group_size, K, N, M, _ptr(x), _ptr(w),
                                          _ptr(s), _ptr(b), _ptr(sx), _ptr(mw)),
           "bound_terms")
    return sx, mw


def _abs_inputs(bits, K, x, w, scales, biases, group_size):
    x, w, s, b, M, N = _prep(bits, K, x, w, scales, biases, group_size)
    return np.abs(x), w, np.abs(s), np.abs(b)


def accumulation_terms(bits: int, K: int, x, w, scales, biases, group_size: int = 64,
                       threads: int = 1) -> np.ndarray:
    """A(m,n) = sum_k (|s(n,g)| q(n,k) + |b(n,g)|) |x(m,k)|, g = k // group_size,
    for every row and column ([M, N]).

    A is the sum of the magnitudes of the terms that the pages' factored form
    adds up, y = sum_g s_g (sum_k q_k x_k) + b_g (sum_k x_k) ("@mlx-bun/inference
    0.0.0-stage -> 1.0.0" page, affine3-rows.ts header comment: the algebra of
    MLX's kernels, scale times the sum of q x plus bias times the sum of x), so
    the rounding error of any f32 evaluation of that form is bounded by a
    multiple of A (f32_sum_bound).  Every term is non-negative, so A is the
    oracle's own matmul over |x|, |s| and |b| (codes are non-negative)."""
    xa, w, sa, ba = _abs_inputs(bits, K, x, w, scales, biases, group_size)
    return matmul(bits, K, xa, w, sa, ba, group_size, threads)


def accumulation_terms_at(bits: int, K: int, x, w, scales, biases, ms, ns,
                          group_size: int = 64) -> np.ndarray:
    """A(ms[i], ns[i]) of accumulation_terms for sampled output coordinates."""
    xa, w, sa, ba = _abs_inputs(bits, K, x, w, scales, biases, group_size)
    return matmul_at(bits, K, xa, w, sa, ba, ms, ns, group_size)


F32_UNIT = 2.0 ** -24   # unit roundoff of f32 (round to nearest)


BF16_WEIGHT_ROUNDING = 2.0 ** -9   # relative rounding of a weight stored as bf16


def f32_sum_bound(K: int, acc_terms, weight_rounding: float = 0.0) -> np.ndarray:
    """Bound on |fl(y) - y| for an f32 evaluation, in any order, of the
    factored form over exact bf16/f32 inputs.  Along the path from any term to
    the result there are at most K + 3 roundings: the product q*x, at most
    group_size - 1 additions inside its group, the product with the scale or
    bias, and at most 2*K/group_size - 1 additions of the group terms (fewer
    than K + 3 for every group size and K >= group_size).  The standard bound
    for such a computation (a sum whose every term passes through at most p
    roundings of relative size u: |error| <= p u / (1 - p u) times the sum of
    the terms' magnitudes) with p = K + 3 gives gamma * A.

    weight_rounding = r: every weight is first rounded to a type of relative
    precision r (bf16 weight operands of a matrix-core product: r = 2^-9),
    which moves the exact sum by at most r * sum_k |x_k w_k| <= r * A (|w| <=
    |s| q + |b|), and the f32 sums then run over terms up to (1 + r) times
    larger: (r + gamma (1 + r)) * A."""
    p = K + 3
    gamma = p * F32_UNIT / (1.0 - p * F32_UNIT)
    r = float(weight_rounding)
    return (r + gamma * (1.0 + r)) * np.asarray(acc_terms, dtype=np.float64)


def rounding_step(v, out_dtype: str) -> np.ndarray:
    """The spacing of the output type's values at magnitude |v| (one unit in
    the last place): bf16 keeps 8 significant bits, f32 24; below the
    smallest normal the subnormal spacing (2^-133 for bf16, 2^-149 for f32)."""
    v = np.abs(np.asarray(v, dtype=np.float64))
    sig = {"bf16": 8, "f32": 24}[out_dtype]
    tiny = {"bf16": 2.0 ** -133, "f32": 2.0 ** -149}[out_dtype]
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(v > 0, v, 1.0)))
    step = np.ldexp(1.0, (e - (sig - 1)).astype(np.int64))
    return np.where((v > 0) & (step > tiny), step, tiny)


def strict_tolerance(y_ref, acc_terms, K: int, out_dtype: str,
                     weight_rounding: float = 0.0) -> np.ndarray:
    """Element-wise bound a correct kernel meets whatever its summation order:
    its f32 result differs from y_ref by at most E = f32_sum_bound(K, A); an
    f32 output is that result itself (bound E), a bf16 output rounds it to
    nearest, moving it by at most half a bf16 step at |y_ref| + E
    (bound E + step/2).  weight_rounding: see f32_sum_bound."""
    E = f32_sum_bound(K, acc_terms, weight_rounding)
    if out_dtype == "f32":
        return E
    return E + 0.5 * rounding_step(np.abs(y_ref) + E, out_dtype)


def check_outputs(y, y_ref, acc_terms, ns_tol, K: int, out_dtype: str,
                  weight_rounding: float = 0.0):
    """The acceptance of an output block against the oracle; returns a dict
    with the three figures and whether each passes:
      * bound:  max |y - y_ref| / ns_tol <= 1 (the acceptance bound above,
        ns_tol = tolerance(...));
      * strict: max |y - y_ref| / strict_tolerance <= 1 (a correct f32
        evaluation of the factored form meets it in any summation order);
      * median: the median of |y - y_ref| / ns_tol (bf16 outputs) or of
        |y - y_ref| / E (f32 outputs) at most 0.01 or 0.05: the bulk of the
        outputs must sit at the rounding level, not merely under the bound,
        so a kernel-sized mistake cannot hide under a bound that grows with
        K.
    weight_rounding: 0 for kernels whose products use the exact weights (or
    codes), BF16_WEIGHT_ROUNDING for a kernel that multiplies bf16-rounded
    weights (see f32_sum_bound)."""
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    err = np.abs(y - y_ref)
    st = strict_tolerance(y_ref, acc_terms, K, out_dtype, weight_rounding)
    r_bound = err / ns_tol
    with np.errstate(divide="ignore", invalid="ignore"):
        r_strict = np.where(err == 0, 0.0, err / st)
    if out_dtype == "f32":
        E = f32_sum_bound(K, acc_terms, weight_rounding)
        with np.errstate(divide="ignore", invalid="ignore"):
            r_med = np.where(err == 0, 0.0, err / E)
        med_cap = 0.05
    else:
        r_med = r_bound
        med_cap = 0.01
    out = {"finite": bool(np.all(np.isfinite(y))),
           "bound": float(np.max(r_bound)) if err.size else 0.0,
           "strict": float(np.max(r_strict)) if err.size else 0.0,
           "median": float(np.median(r_med)) if err.size else 0.0,
           "median_cap": med_cap}
    out["ok"] = (out["finite"] and out["bound"] <= 1.0 and out["strict"] <= 1.0
                 and out["median"] <= med_cap)
    return out


def tolerance_coefficient(x_dtype: str) -> float:
    """c of the acceptance bound: 1e-3 for f32 activations, 8e-3 for bf16."""
    return {"f32": 1e-3, "bf16": 8e-3}[x_dtype]


def tolerance(bits: int, K: int, x, w, scales, biases, x_dtype: str,
              group_size: int = 64) -> np.ndarray:
    """Element-wise acceptance bound [M, N]."""
    sx, mw = bound_terms(bits, K, x, w, scales, biases, group_size)
    return tolerance_coefficient(x_dtype) * np.outer(sx, mw) + 1e-6


# ---------------------------------------------------------------------------
# Fused gate/up epilogue ("mlx-bun 0.4.0 -> 1.0.0" page, trellis-shared-m.ts,
# its shared-M gate/up kernel of the trellis path: gate and up are rounded to
# the activation type, then the sigmoid of the rounded gate, the SiLU product
# and the final product are each rounded to that type).  Applied here to the
# affine projections.

def round_bf16(v) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value (8 significant bits,
    ties to even), returned as float64.  Values below 2^-126 use the subnormal
    spacing 2^-133; magnitudes from (2 - 2^-8) * 2^127 up overflow to inf."""
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)  # v = m * 2^e, 0.5 <= |m| < 1
    r = np.ldexp(np.round(m * 256.0), e - 8)  # numpy rounds halves to even
    small = np.abs(v) < 2.0 ** -126
    r = np.where(small, np.round(v * 2.0 ** 133) * 2.0 ** -133, r)
    big = np.abs(v) >= (2.0 - 2.0 ** -8) * 2.0 ** 127
    return np.where(big, np.copysign(np.inf, v), r)


def silu_mul_bf16(gate, up) -> np.ndarray:
    """h = R(R(R(g) * R(sigmoid(R(g)))) * R(u)) with R = round_bf16 and
    sigmoid(z) = 1 / (1 + e^-z), on float64 gate and up values."""
    g = round_bf16(gate)
    u = round_bf16(up)
    with np.errstate(over="ignore"):
        sig = round_bf16(1.0 / (1.0 + np.exp(-g)))
    silu = round_bf16(g * sig)
    return round_bf16(silu * u)


def gate_up(bits: int, K: int, x, wg, sg, bg, wu, su, bu, group_size: int = 64,
            threads: int = 1, lib=None) -> np.ndarray:
    """The fused gate/up output for every row and column: both projections by
    matmul(), then silu_mul_bf16()."""
    g = matmul(bits, K, x, wg, sg, bg, group_size, threads, lib)
    u = matmul(bits, K, x, wu, su, bu, group_size, threads, lib)
    return silu_mul_bf16(g, u)


def gate_up_tolerance(gate, up, tol_gate, tol_up) -> np.ndarray:
    """Element-wise acceptance bound for the fused gate/up output, from the
    exact gate/up values and the matmul bounds of the two projections: the
    gate error (the matmul bound plus one bf16 step where the two sides round
    it differently) times the largest slope of SiLU (1.1) times |up|, the up
    error likewise times |silu(gate)|, and four bf16 steps of the result for
    the chain's roundings."""
    gate = np.asarray(gate, dtype=np.float64)
    up = np.asarray(up, dtype=np.float64)
    with np.errstate(over="ignore"):
        silu = gate / (1.0 + np.exp(-gate))
    return (1.1 * np.abs(up) * (tol_gate + 2.0 ** -8 * np.abs(gate))
            + np.abs(silu) * (tol_up + 2.0 ** -8 * np.abs(up))
            + 2.0 ** -6 * np.abs(silu * up) + 1e-6)


# ---------------------------------------------------------------------------
# Residual add + RMS normalization ("@mlx-bun/inference 0.0.0-stage ->
# 1.0.0" page, residual-rms-norm.ts): the residual sum is rounded to the
# storage type before it is squared, the normalized value is rounded before
# the weight multiplies it, and the product is stored in that type.

def round_f32(v) -> np.ndarray:
    """Round float64 values to the nearest float32 (ties to even), as float64."""
    return np.asarray(v, dtype=np.float64).astype(np.float32).astype(np.float64)


def residual_rms_norm(x, update, weight, eps: float, dtype: str):
    """(residual, normalized) in float64 for decoded inputs x, update [rows, D]
    and weight [D]; dtype 'bf16' or 'f32' names the storage type T:
        residual   = R(x + update)
        normalized = R(weight * R(residual / sqrt(mean(residual^2) + eps)))
    with R the rounding to T and everything else exact (float64)."""
    R = round_bf16 if dtype == "bf16" else round_f32
    x = np.asarray(x, dtype=np.float64)
    update = np.asarray(update, dtype=np.float64)
    weight = np.asarray(weight, dtype=np.float64)
    res = R(x + update)
    ms = np.mean(res * res, axis=-1, keepdims=True)
    inv = 1.0 / np.sqrt(ms + float(np.float32(eps)))
    return res, R(weight * R(res * inv))


def residual_rms_norm_tolerance(normalized_ref, D: int, dtype: str) -> np.ndarray:
    """Bound on |normalized - reference| for an implementation that sums the
    squares in f32 in any order: that sum and the f32 square root are off by
    at most about (D + 2) * 2^-24 relative, which can move R(residual * inv)
    across one rounding step of T and the weighted product across another:
    two steps of T (2^-7 relative for bf16) plus the f32 error itself."""
    ulp = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -23
    return np.abs(normalized_ref) * (2 * ulp + (D + 2) * 2.0 ** -24) + 1e-30


def group_sums(values, group_size: int) -> np.ndarray:
    """Sum of every group of group_size consecutive values of each row, in
    float64, group-major: out[g, m] = sum of values[m, g*G .. (g+1)*G) for
    G = group_size.  The sum of x per quantization group is what the bias
    term of the factored form takes ("@mlx-bun/inference 0.0.0-stage ->
    1.0.0" page, affine3-rows.ts header: s * sum(q x) + b * sum(x)); the
    residual add + RMS norm can hand it to the projection it feeds."""
    v = np.asarray(values, dtype=np.float64)
    rows, D = v.shape
    if D % group_size != 0:
        raise ValueError("D=%d is not a multiple of group_size=%d" % (D, group_size))
    out = np.zeros((D // group_size, rows), dtype=np.float64)
    for g in range(D // group_size):
        for i in range(g * group_size, (g + 1) * group_size):
            out[g] += v[:, i]
    return out


def group_sum_tolerance(values, group_size: int) -> np.ndarray:
    """Bound on |f32 sum - exact sum| of each group (group-major like
    group_sums) for an f32 evaluation in any order of group_size exact
    terms: at most group_size - 1 roundings of relative size u = 2^-24 on any
    term's path, so (G-1) u / (1 - (G-1) u) times the sum of the magnitudes."""
    p = (group_size - 1) * F32_UNIT
    return p / (1.0 - p) * group_sums(np.abs(np.asarray(values, dtype=np.float64)), group_size)


# ---------------------------------------------------------------------------
# Decode attention over an affine-quantized KV cache ("mlx-bun 0.0.4" page,
# fused-decode-kernel.ts): one query row per head attends to all N cached
# rows of its KV head (head h reads KV head h // (H / KV)); keys and values
# are stored like the weights (codes packed along D, least significant bits
# first, one scale and bias per group of `group_size` values of a row).
#   score[h, n] = R(sum_d q[h, d] * k[kv, n, d])      (rounded to bf16)
#   out[h, :]   = R(sum_n e^score[h, n] * v[kv, n, :] / sum_n e^score[h, n])
# with k = s*code + b and v likewise, R the rounding to bf16 and everything
# else exact in float64.  No extra score scale: the query arrives scaled.

def unpack_lsb(words, bits: int, D: int) -> np.ndarray:
    """Codes [..., D] from uint32 words [..., D*bits/32], each word holding
    32/bits codes with the first in its least significant bits."""
    w = np.asarray(words, dtype=np.uint64)
    per = 32 // bits
    shifts = (np.arange(per, dtype=np.uint64) * np.uint64(bits))
    codes = (w[..., :, None] >> shifts) & np.uint64((1 << bits) - 1)
    return codes.reshape(w.shape[:-1] + (w.shape[-1] * per,))[..., :D].astype(np.int64)


def dequant_rows(words, scales, biases, bits: int, D: int, group_size: int) -> np.ndarray:
    """float64 values s*code + b of rows stored as words [..., D*bits/32] with
    scales/biases [..., D/group_size] (decoded float64)."""
    codes = unpack_lsb(words, bits, D).astype(np.float64)
    s = np.repeat(np.asarray(scales, dtype=np.float64), group_size, axis=-1)
    b = np.repeat(np.asarray(biases, dtype=np.float64), group_size, axis=-1)
    return s * codes + b


def decode_attention(q, k_words, k_scales, k_biases, v_words, v_scales, v_biases,
                     bits: int, group_size: int, return_scores: bool = False):
    """out [H, D] (float64 values of bf16 results) for decoded q [H, D] and a
    cache of KV heads: words [KV, N, D*bits/32], scales/biases [KV, N, D/gs]."""
    q = np.asarray(q, dtype=np.float64)
    H, D = q.shape
    KV = k_words.shape[0]
    rep = H // KV
    k = dequant_rows(k_words, k_scales, k_biases, bits, D, group_size)  # [KV, N, D]
    v = dequant_rows(v_words, v_scales, v_biases, bits, D, group_size)
    out = np.empty((H, D))
    scores = np.empty((H, k.shape[1]))
    for h in range(H):
        kv = h // rep
        s = round_bf16(k[kv] @ q[h])
        e = np.exp(s - s.max())
        out[h] = round_bf16((e @ v[kv]) / e.sum())
        scores[h] = s
    return (out, scores) if return_scores else out


def score_terms(q, k_words, k_scales, k_biases, bits: int, group_size: int) -> np.ndarray:
    """T[h, n] = sum_d (|s_nd| c_nd + |b_nd|) |q_hd| over the KV head of head
    h: the sum of the magnitudes of the terms of the page's factored score,
    s * sum_d c_d q_d + b * sum_d q_d ("mlx-bun 0.0.4" page,
    fused-decode-kernel.ts, SCORE_PREAMBLE comment: the dequant is factored
    out of the inner loop).  Any f32 evaluation of that form is within
    f32_sum_bound(D, T) of the exact score."""
    q = np.asarray(q, dtype=np.float64)
    H, D = q.shape
    KV = k_words.shape[0]
    rep = H // KV
    codes = unpack_lsb(k_words, bits, D).astype(np.float64)          # [KV, N, D]
    s = np.repeat(np.abs(np.asarray(k_scales, dtype=np.float64)), group_size, axis=-1)
    b = np.repeat(np.abs(np.asarray(k_biases, dtype=np.float64)), group_size, axis=-1)
    mag = s * codes + b                                                # [KV, N, D]
    return np.stack([mag[h // rep] @ np.abs(q[h]) for h in range(H)])


def decode_attention_tolerance(out_ref, q, k_words, k_scales, k_biases, v_words, v_scales,
                               v_biases, bits: int, group_size: int) -> np.ndarray:
    """Bound on |out - out_ref| for an implementation that evaluates each
    score in f32 in the page's factored form (any order) and the softmax sums
    in f32.  The score's f32 sum is off by at most
    eps_n = f32_sum_bound(D, T_n) (T = score_terms, the magnitudes of the
    factored form's terms), so its bf16 rounding moves by at most
    delta_n = eps_n + 2^-7 (|score_n| + eps_n) (one bf16 step where the two
    sides round differently).  With softmax weights w_n, shifting score n by
    at most delta_n scales w_n by at most e^(delta_n + delta_w),
    delta_w = log sum_m w_m e^(delta_m) (the change of the normaliser), so
    the unrounded output moves by at most sum_n w_n (e^(delta_n + delta_w) - 1)
    |v_n - out|; the f32 sums of the weights and weighted values add
    (N + 8) 2^-24 max|v|; the final bf16 rounding of either side adds one bf16
    step, 2^-7 |out|.  Nothing here depends on how a kernel orders or splits
    its sums."""
    q = np.asarray(q, dtype=np.float64)
    H, D = q.shape
    KV = k_words.shape[0]
    rep = H // KV
    k = dequant_rows(k_words, k_scales, k_biases, bits, D, group_size)
    v = dequant_rows(v_words, v_scales, v_biases, bits, D, group_size)
    N = k.shape[1]
    T = score_terms(q, k_words, k_scales, k_biases, bits, group_size)
    tol = np.empty((H, D))
    for h in range(H):
        kv = h // rep
        sig = k[kv] @ q[h]
        eps = f32_sum_bound(D, T[h])
        delta = eps + 2.0 ** -7 * (np.abs(sig) + eps)
        s = round_bf16(sig)
        w = np.exp(s - s.max())
        w /= w.sum()
        dw = np.log(np.sum(w * np.exp(delta)))
        growth = w * np.expm1(delta + dw)                       # [N]
        unrounded = (w @ v[kv])
        move = growth @ np.abs(v[kv] - unrounded[None, :])      # [D]
        vmax = np.max(np.abs(v[kv]), axis=0)
        tol[h] = (2.0 ** -7 * np.abs(out_ref[h]) + move + (N + 8) * 2.0 ** -24 * vmax + 1e-6)
    return tol
