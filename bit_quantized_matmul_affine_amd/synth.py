"""Seeded synthetic inputs for the affine group-quantized matmul.

This module only draws random numbers and stores them in the input dtypes; it
holds none of the operation's arithmetic (no unpacking, no dequantization, no
dot products). Both the GPU tests and the oracle tests take their inputs from
here.

Recipe (one numpy PCG64 generator per workload, seeded with the workload index):
  1. packed weight words, uint32 [N, K*bits/32], every word uniform on
     [0, 2^32).  Each code is `bits` consecutive bits of the LSB-first stream,
     so uniform words are exactly "codes uniform on [0, 2^bits), packed
     LSB-first" (the bits of uniform codes are independent fair coins);
  2. scales [N, K/64] uniform on [lo, hi);
  3. bias noise [N, K/64] normal(0, sigma) (skipped when sigma == 0);
     bias = -c * scale + noise, formed in float64 from the unrounded scale;
  4. activations x [M, K] standard normal;
  5. outlier channels (when asked): ceil(frac*K) column indices drawn without
     replacement; those columns of x are multiplied by the factor.
Values stored as bf16 are rounded from float64 through float32 with
round-to-nearest-even; f32 values are rounded from float64 once.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

GROUP = 64


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 values -> bf16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _store(values_f64: np.ndarray, dtype: str) -> np.ndarray:
    f32 = values_f64.astype(np.float32)
    if dtype == "f32":
        return f32
    if dtype == "bf16":
        return f32_to_bf16_bits(f32)
    raise ValueError(dtype)


@dataclass
class Problem:
    """One projection: raw stored arrays plus their description."""
    name: str
    bits: int
    K: int
    N: int
    M: int
    x_dtype: str          # "f32" or "bf16" (y has the same dtype)
    sb_dtype: str         # dtype of scales and biases
    w: np.ndarray         # uint32 [N, K*bits/32], MLX layout
    scales: np.ndarray    # f32 values or bf16 bits, [N, K/64]
    biases: np.ndarray    # same dtype as scales
    x: np.ndarray         # f32 values or bf16 bits, [M, K]
    meta: dict = field(default_factory=dict)
    group_size: int = GROUP

    def rows(self, m: int) -> "Problem":
        """The same weights with the first m activation rows."""
        return Problem(self.name, self.bits, self.K, self.N, m, self.x_dtype,
                       self.sb_dtype, self.w, self.scales, self.biases,
                       self.x[:m], dict(self.meta), self.group_size)

    @property
    def weight_bytes(self) -> int:
        sb = 2 if self.sb_dtype == "bf16" else 4
        return self.N * self.K * self.bits // 8 + 2 * self.N * (self.K // self.group_size) * sb


def draw(rng: np.random.Generator, *, name: str, bits: int, K: int, N: int, M: int,
         x_dtype: str, sb_dtype: str, scale_lo: float, scale_hi: float,
         bias_c: float, bias_sigma: float, outlier_frac: float = 0.0,
         outlier_factor: float = 1.0, x_override: np.ndarray | None = None,
         group_size: int = GROUP) -> Problem:
    """Draw one projection in the recipe's order."""
    assert K % group_size == 0 and (K * bits) % 32 == 0
    G = K // group_size
    w = rng.integers(0, 2**32, size=(N, K * bits // 32), dtype=np.uint64).astype(np.uint32)
    scale = rng.uniform(scale_lo, scale_hi, size=(N, G))
    bias = -bias_c * scale
    if bias_sigma > 0:
        bias = bias + rng.normal(0.0, bias_sigma, size=(N, G))
    if x_override is None:
        x = rng.standard_normal(size=(M, K))
        if outlier_frac > 0:
            cols = rng.choice(K, size=int(math.ceil(outlier_frac * K)), replace=False)
            x[:, cols] *= outlier_factor
        xs = _store(x, x_dtype)
    else:
        xs = x_override
    return Problem(name, bits, K, N, M, x_dtype, sb_dtype, w, _store(scale, sb_dtype),
                   _store(bias, sb_dtype), xs, {}, group_size)


# The five workloads.  Index = seed.
WORKLOADS = {
    0: "4-bit group-64 qmm, M=1, K=512, N=512, f32 activations and scales",
    1: "4-bit group-64 GEMV, M=1, K=5120, N=10240, bf16",
    2: "3-bit group-64 qmm, K=5120, N=10240, M in {1,9,16,32,64}, bf16",
    3: "4-bit group-64 MLP trio at M=4: gate/up 3840->15360, down 15360->3840, bf16, outlier channels",
    4: "4-bit group-64 qmm, M=128, K=8192, N=28672, bf16",
}
C2_ROWS = (1, 9, 16, 32, 64)


def workload(idx: int, M: int | None = None) -> list[Problem]:
    """Problems of workload `idx` (a list: three projections for the MLP trio)."""
    rng = np.random.default_rng(idx)
    if idx == 0:
        return [draw(rng, name="c0", bits=4, K=512, N=512, M=1, x_dtype="f32",
                     sb_dtype="f32", scale_lo=0.005, scale_hi=0.02, bias_c=8.0,
                     bias_sigma=0.001)]
    if idx == 1:
        return [draw(rng, name="c1", bits=4, K=5120, N=10240, M=1, x_dtype="bf16",
                     sb_dtype="bf16", scale_lo=0.005, scale_hi=0.02, bias_c=8.0,
                     bias_sigma=0.001)]
    if idx == 2:
        # One 64-row activation draw; smaller row counts use its first rows.
        p = draw(rng, name="c2", bits=3, K=5120, N=10240, M=64, x_dtype="bf16",
                 sb_dtype="bf16", scale_lo=0.01, scale_hi=0.04, bias_c=4.0,
                 bias_sigma=0.002)
        return [p.rows(M if M is not None else 64)]
    if idx == 3:
        common = dict(bits=4, M=4, x_dtype="bf16", sb_dtype="bf16", scale_lo=0.005,
                      scale_hi=0.02, bias_c=8.0, bias_sigma=0.001, outlier_frac=0.01,
                      outlier_factor=20.0)
        gate = draw(rng, name="c3_gate", K=3840, N=15360, **common)
        # gate and up consume the same activations (the MLP input).
        up = draw(rng, name="c3_up", K=3840, N=15360, x_override=gate.x, **common)
        down = draw(rng, name="c3_down", K=15360, N=3840, **common)
        return [gate, up, down]
    if idx == 4:
        return [draw(rng, name="c4", bits=4, K=8192, N=28672, M=128, x_dtype="bf16",
                     sb_dtype="bf16", scale_lo=0.005, scale_hi=0.02, bias_c=8.0,
                     bias_sigma=0.0)]
    raise KeyError(idx)


def small(seed: int, *, bits: int, K: int, N: int, M: int, x_dtype: str = "bf16",
          sb_dtype: str | None = None, group_size: int = GROUP) -> Problem:
    """A small seeded problem with the distributions of the matching workload
    (3-bit: scale U[0.01,0.04], bias -4s+N(0,.002); 4-bit: U[0.005,0.02],
    -8s+N(0,.001)); other widths: a weight range of about 0.16 split into
    2^bits steps, bias -2^(bits-1) s + N(0, .001)."""
    rng = np.random.default_rng(seed)
    if bits == 3:
        lo, hi, c, sig = 0.01, 0.04, 4.0, 0.002
    elif bits == 4:
        lo, hi, c, sig = 0.005, 0.02, 8.0, 0.001
    else:
        step = 0.16 / 2 ** bits
        lo, hi, c, sig = 0.5 * step, 2.0 * step, float(2 ** (bits - 1)), 0.001
    return draw(rng, name="small", bits=bits, K=K, N=N, M=M, x_dtype=x_dtype,
                sb_dtype=sb_dtype or x_dtype, scale_lo=lo, scale_hi=hi, bias_c=c,
                bias_sigma=sig, group_size=group_size)


def norm_inputs(seed: int, rows: int, D: int, dtype: str = "bf16"):
    """Seeded inputs of a residual add + RMS normalization, as stored arrays
    (uint16 bf16 patterns or float32): hidden state x ~ N(0, 1) [rows, D],
    block output update ~ N(0, 0.5^2) [rows, D], weight ~ 1 + N(0, 0.1^2) [D]."""
    rng = np.random.default_rng(seed)
    x = _store(rng.standard_normal((rows, D)), dtype)
    update = _store(0.5 * rng.standard_normal((rows, D)), dtype)
    weight = _store(1.0 + 0.1 * rng.standard_normal(D), dtype)
    return x, update, weight


def pack_lsb(codes: np.ndarray, bits: int) -> np.ndarray:
    """uint32 words [..., D*bits/32] holding codes [..., D] (values < 2^bits),
    32/bits per word, the first in the least significant bits."""
    per = 32 // bits
    c = codes.astype(np.uint64).reshape(codes.shape[:-1] + (codes.shape[-1] // per, per))
    shifts = np.arange(per, dtype=np.uint64) * np.uint64(bits)
    return np.bitwise_or.reduce(c << shifts, axis=-1).astype(np.uint32)


def attention_inputs(seed: int, *, H: int, KV: int, N: int, D: int, bits: int,
                     group_size: int):
    """Seeded decode-attention inputs as stored arrays (bf16 as uint16):
    q [H, D] ~ N(0, 1.4^2 / D) (scores of a few units); for keys and values,
    per group of a row a range [lo, hi] with -lo, hi ~ 2 + 0.5|N(0, 1)|,
    scale = (hi - lo) / (2^bits - 1), bias = lo (both bf16), codes uniform.
    Returns q, (k_words, k_scales, k_biases), (v_words, v_scales, v_biases)."""
    rng = np.random.default_rng(seed)
    q = _store(rng.standard_normal((H, D)) * 1.4 / np.sqrt(D), "bf16")

    def cache():
        G = D // group_size
        lo = -(2.0 + 0.5 * np.abs(rng.standard_normal((KV, N, G))))
        hi = 2.0 + 0.5 * np.abs(rng.standard_normal((KV, N, G)))
        scales = _store((hi - lo) / (2 ** bits - 1), "bf16")
        biases = _store(lo, "bf16")
        codes = rng.integers(0, 2 ** bits, size=(KV, N, D), dtype=np.int64)
        return pack_lsb(codes, bits), scales, biases

    return q, cache(), cache()
