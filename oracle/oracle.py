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


def decode_attention_tolerance(out_ref, q, k_words, k_scales, k_biases, v_words, v_scales,
                               v_biases, bits: int, group_size: int) -> np.ndarray:
    """Bound on |out - out_ref| for an implementation whose score sums chain at
    most D/16 + 8 f32 roundings per term (sums over slices of D/16 values,
    then a tree over the slices and the affine step), in the factored form
    that offsets each code by up to 2176 (an 8-bit code as two nibbles
    offset by 128, the high one against 16 q, before the slice's offset is
    removed with its sum of q): terms are at most |q_d| (|k_nd| + 2560
    |scale_nd|), so score n's sum is off by at most
    eps_n = (D/16 + 8) 2^-24 sum_d |q_d| (|k_nd| + 2560 |scale_nd|), which
    moves its bf16 rounding by at most delta_n = eps_n + 2^-7 (|score_n| + eps_n).  With softmax
    weights w_n, shifting score n by at most delta_n scales w_n by at most
    e^(delta_n + delta_w), delta_w = log sum_m w_m e^(delta_m) (the change of
    the normaliser), so the unrounded output moves by at most
    sum_n w_n (e^(delta_n + delta_w) - 1) |v_n - out|; the f32 sums of the
    weights and weighted values add (N + 8) 2^-24 max|v|; the final bf16
    rounding of either side adds one bf16 step, 2^-7 |out|."""
    q = np.asarray(q, dtype=np.float64)
    H, D = q.shape
    KV = k_words.shape[0]
    rep = H // KV
    k = dequant_rows(k_words, k_scales, k_biases, bits, D, group_size)
    v = dequant_rows(v_words, v_scales, v_biases, bits, D, group_size)
    N = k.shape[1]
    tol = np.empty((H, D))
    for h in range(H):
        kv = h // rep
        sig = k[kv] @ q[h]
        ksc = np.repeat(np.abs(np.asarray(k_scales, dtype=np.float64)[kv]), group_size, axis=-1)
        eps = (D / 16 + 8) * 2.0 ** -24 * ((np.abs(k[kv]) + 2560.0 * ksc) @ np.abs(q[h]))
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
