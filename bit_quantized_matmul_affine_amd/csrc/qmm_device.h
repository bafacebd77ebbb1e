// qmm_device.h -- device-side helpers shared by the gfx950 kernels of libqmm
// (y = x . W^T over affine 3/4-bit, group-64 quantized weights): the
// native layout, the unpack to bf16 pairs, the factored group affine, the
// scale/bias loads, the output store, the split-K fold and the wait helpers.
// Not installed.
//
// Sources.  [P1] = page "@mlx-bun/inference 0.0.0-stage -> 1.0.0" (diffend npm
// page 53).  [P3] = page "mlx-bun 0.0.4" (diffend npm page 56).
//   * The operation and the MLX packing: [P1] affine-split-mma.ts header
//     comment and helper affine_unit; affine3-mma.ts helper affine_q3;
//     affine4-mma.ts helper affine_q4; weight = scale*q + bias per group of 64.
//   * Decode each weight once and reuse it for every activation row:
//     [P1] affine3-rows.ts / affine4-rows.ts header comments.
//   * Factored per-group algebra sum_g scale*sum(q*x) + bias*sum(x):
//     [P1] affine3-rows.ts header comment; [P3] fused-decode-kernel.ts
//     SCORE_PREAMBLE comment (dequant factored out of the inner loop).
//   * K split across workers, partials added in a fixed order with no
//     atomics on the data: [P1] affine-split-mma.ts (threadgroup fold over
//     SPLITS, summed in split order); [P3] fused-decode-kernel.ts header
//     (deterministic merge, no atomic adds).
//   * Rows past the last activation row are never written: [P1]
//     affine-split-mma.ts fold ("columns below M only").
//
// What is ours (gfx950, not the pages' Metal design):
//   * Codes become bf16 values 128+q (or 128+8q) with one and-or per PAIR of
//     codes: (w >> shift) & mask | 0x43004300 (bf16 0x4300 is 128.0 and the
//     code fits the 7 mantissa bits exactly).  The offset is removed per group
//     through the factored form: for one group with values v_k = 128 + f q_k,
//         sum_k (s*q_k + b) x_k = (s/f) sum_k v_k x_k + (b - (128/f) s) sum_k x_k.
//   * A one-time repack ("native layout") makes every wavefront load 768 or
//     1024 contiguous bytes per instruction and hands each lane exactly the
//     codes its MFMA operand needs.  Byte count is unchanged.
//   * MFMA path: v_mfma_f32_16x16x32_bf16 with A = 16 activation rows and
//     B = 16 weight rows; per group the B operand is the 128+q pairs, a second
//     product against all-ones gives sum_k x_k, and the accumulator is scaled
//     in f32 before the next group.
//   * Vector-ALU path: v_dot2_f32_bf16 on (128+q) pairs against activation
//     pairs staged in LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "qmm_internal.h"

namespace qmm {

typedef __bf16 bf16x8 __attribute__((__vector_size__(16)));
typedef __bf16 bf16x2 __attribute__((__vector_size__(4)));
typedef float f32x4 __attribute__((__vector_size__(16)));
typedef uint32_t u32x4 __attribute__((__vector_size__(16)));

// ---------------------------------------------------------------------------
// Native layout.
//
// Tiles of 16 rows of W (nT = N/16) by chunks of 128 columns (nC = K/128, two
// quantization groups).  Block (tile t, chunk c) has index t*nC + c.
// Codes: block b occupies words [b*64*BITS, (b+1)*64*BITS); lane l of the
// block owns words [l*BITS, (l+1)*BITS).  Lane l serves row r = l & 15 of the
// tile and quarter kg = l >> 4 of each group: its 32 codes are
//     (g', i) for g' in {0,1}, i in [0,16):  k = 128c + 64g' + 16kg + i.
// The codes are grouped in 16 pairs p = 8g' + u holding (g', 2u) in the low
// and (g', 2u+1) in the high 16 bits after the unpack:
//   4-bit: pair p = 4j + t sits in word j, low code at bits [4t, 4t+4),
//          high code at bits [16+4t, 16+4t+4).
//   3-bit: each word holds five fields f = 0..4 (low code at bits
//          [3f, 3f+3), high code at [16+3f, 16+3f+3)) and one bit at 15 / 31.
//          Pairs 0..7 (group 0) are f0, f2, f4 of word 0, f0, f2, f4 of
//          word 1, f0, f2 of word 2; pairs 8..14 (group 1) are f1, f3 of
//          words 0, 1, 2 and f4 of word 2; pair 15 keeps bit b of its low
//          code in bit 15 of word b and bit b of its high code in bit 31.
// Scales/biases: block b holds 16 rows x {s_g0, s_g1, b_g0, b_g1}.
// ---------------------------------------------------------------------------

// (x & mask) | or_v as one v_and_or_b32: the masks sit in SGPRs and the
// or-value 0x43004300 in a VGPR, each produced once by an opaque move (gfx9
// VOP3 instructions take no literal and read at most one scalar, so with two
// visible constants the compiler would split the expression in two).  The
// and-or itself stays ordinary code: its results feed MFMA operands, and the
// compiler inserts the wait states between a vector write and an MFMA read
// only for instructions it can see (not for inline assembly).
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t mask_s, uint32_t or_v) {
  return (x & mask_s) | or_v;
}
__device__ __forceinline__ uint32_t opaque_sgpr(uint32_t v) {
  uint32_t r;
  asm volatile("s_mov_b32 %0, %1" : "=s"(r) : "i"(v));
  return r;
}

// The or-value of unpack_pairs in a VGPR and the field masks in SGPRs.
struct PairMasks {
  uint32_t orv;
  uint32_t m4, m0, m3, m5;  // 0x000F000F, 0x00070007, 0x00380038, 0x00200020
};
template <int BITS>
__device__ __forceinline__ PairMasks pair_mask_vgpr() {
  PairMasks k;
  asm volatile("v_mov_b32 %0, %1" : "=v"(k.orv) : "s"(0x43004300u));
  if constexpr (BITS == 4) {
    k.m4 = opaque_sgpr(0x000F000Fu);
  } else {
    k.m0 = opaque_sgpr(0x00070007u);
    k.m3 = opaque_sgpr(0x00380038u);
    k.m5 = opaque_sgpr(0x00200020u);
  }
  return k;
}

// 16 pairs of bf16 values from one lane's BITS words; pair p = 8g' + u holds
// codes (g', 2u) in its low half and (g', 2u+1) in its high half.
//   4-bit: pair p = 4j + t is field t (bits 4t / 16+4t) of word j; value 128+q.
//   3-bit: a word holds five fields f = 0..4 at bits 3f / 16+3f, plus bit 15 /
//   bit 31.  Group 0 (pairs 0..7) uses fields placed at mantissa bits 0..2
//   (value 128+q): f0 and f2 of every word and f4 of words 0 and 1.  Group 1
//   (pairs 8..15) uses fields placed at mantissa bits 3..5 (value 128+8q):
//   f1 and f3 of every word, f4 of word 2, and the pair whose code bit b sits
//   in bit 15 / bit 31 of word b.  Fields f0/f1 need no shift and f2/f3 share
//   one, so 32 codes cost 6 shifts, 15 and-ors and 7 instructions for the
//   split pair.  group_affine() folds the factor 8 into the group's scale.
template <int BITS>
__device__ __forceinline__ void unpack_pairs(const uint32_t* w, uint32_t* P, const PairMasks& k) {
  if constexpr (BITS == 4) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int t = 0; t < 4; ++t) P[4 * j + t] = and_or(w[j] >> (4 * t), k.m4, k.orv);
  } else {
    const uint32_t m0 = k.m0, m3 = k.m3;
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const uint32_t w6 = w[j] >> 6;
      P[j < 2 ? 3 * j : 6] = and_or(w[j], m0, k.orv);      // f0 -> group 0
      P[j < 2 ? 3 * j + 1 : 7] = and_or(w6, m0, k.orv);    // f2 -> group 0
      P[8 + 2 * j] = and_or(w[j], m3, k.orv);              // f1 -> group 1
      P[9 + 2 * j] = and_or(w6, m3, k.orv);                // f3 -> group 1
      if (j < 2)
        P[3 * j + 2] = and_or(w[j] >> 12, m0, k.orv);      // f4 -> group 0
      else
        P[14] = and_or(w[j] >> 9, m3, k.orv);              // f4 -> group 1
    }
    // pair 15 (group 1): bit b of each code sits in bit 15 / bit 31 of word b
    const uint32_t b0 = (w[0] >> 12) & 0x00080008u;
    const uint32_t b1 = (w[1] >> 11) & 0x00100010u;
    const uint32_t b2 = and_or(w[2] >> 10, k.m5, k.orv);
    P[15] = b0 | b1 | b2;
  }
}

// Per-group factors for the values unpack_pairs produces: with v = 128 + f*q
// (f = 1, or 8 for group 1 of the 3-bit layout),
//   sum_k (s*q_k + b) x_k = (s/f) * sum_k v_k x_k + (b - (128/f) s) * sum_k x_k.
struct Affine {
  float sc, bp;
};
template <int BITS>
__device__ __forceinline__ Affine group_affine(int gp, float s, float b) {
  const bool c3 = BITS == 3 && gp == 1;
  return Affine{c3 ? s * 0.125f : s, b - (c3 ? 16.f : 128.f) * s};
}

// Inverse of unpack_pairs for one code: OR code q of (g', i) into w.
template <int BITS>
__device__ __forceinline__ void place_code(uint32_t* w, int gp, int i, uint32_t q) {
  const int p = 8 * gp + (i >> 1), half = 16 * (i & 1);
  if constexpr (BITS == 4) {
    w[p >> 2] |= q << (half + 4 * (p & 3));
  } else {
    // (word, field) of pair p, see unpack_pairs
    static constexpr int8_t kWord[15] = {0, 0, 0, 1, 1, 1, 2, 2, 0, 0, 1, 1, 2, 2, 2};
    static constexpr int8_t kField[15] = {0, 2, 4, 0, 2, 4, 0, 2, 1, 3, 1, 3, 1, 3, 4};
    if (p < 15) {
      w[kWord[p]] |= q << (half + 3 * kField[p]);
    } else {
#pragma unroll
      for (int b = 0; b < 3; ++b) w[b] |= ((q >> b) & 1u) << (half + 15);
    }
  }
}

// Code k of an MLX row: bits [k*BITS, (k+1)*BITS) of the row's LSB-first
// stream; a field crossing a word boundary takes its high bits from the next
// word ([P1] affine3-mma.ts, affine_q3).
template <int BITS>
__device__ __forceinline__ uint32_t mlx_code(const uint32_t* row, int k) {
  const int p = k * BITS, wi = p >> 5, off = p & 31;
  uint32_t v = row[wi] >> off;
  if (off + BITS > 32) v |= row[wi + 1] << (32 - off);
  return v & ((1u << BITS) - 1u);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
  u += 0x7FFFu + ((u >> 16) & 1u);                                            // nearest even
  return (uint16_t)(u >> 16);
}

// Workgroups go to the eight XCDs round-robin by id.  Renumber them so that
// each XCD gets a contiguous range of work items: the K splits of one tile
// block then share an L2.
__device__ __forceinline__ int xcd_item(int bid, int total) {
  const int xcd = bid & 7, j = bid >> 3, q = total >> 3, rem = total & 7;
  return xcd * q + (xcd < rem ? xcd : rem) + j;
}

// ---------------------------------------------------------------------------
// Scales and biases of one (tile row, chunk): s_g0, s_g1, b_g0, b_g1.
// ---------------------------------------------------------------------------
template <typename ST> struct SBPair;
template <> struct SBPair<uint16_t> {
  uint32_t s2, b2;
  __device__ __forceinline__ void load(const uint16_t* p) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    s2 = v.x;
    b2 = v.y;
  }
  __device__ __forceinline__ float s(int g) const {
    return __uint_as_float(g ? (s2 & 0xFFFF0000u) : (s2 << 16));
  }
  __device__ __forceinline__ float b(int g) const {
    return __uint_as_float(g ? (b2 & 0xFFFF0000u) : (b2 << 16));
  }
};
template <> struct SBPair<float> {
  float4 v;
  __device__ __forceinline__ void load(const float* p) { v = *reinterpret_cast<const float4*>(p); }
  __device__ __forceinline__ float s(int g) const { return g ? v.y : v.x; }
  __device__ __forceinline__ float b(int g) const { return g ? v.w : v.z; }
};

// ---------------------------------------------------------------------------
// Split-K epilogue.  S > 1: every workgroup stores its partial tile to
// part[s][m][n]; the last workgroup of a tile block to take a ticket adds the
// S partials in split order 0..S-1 and writes y, then re-arms the ticket.
// The sum order never depends on arrival order, so results are bitwise
// reproducible.
// ---------------------------------------------------------------------------
// Output element idx of y: f32 for f32 activations or when the plan asks for
// f32 outputs (a.y_f32), else bf16 rounded to nearest even.
template <bool Y_F32>
__device__ __forceinline__ void store_y(const LaunchArgs& a, long idx, float v) {
  if (Y_F32 || a.y_f32)
    reinterpret_cast<float*>(a.y)[idx] = v;
  else
    reinterpret_cast<uint16_t*>(a.y)[idx] = f32_to_bf16(v);
}

template <bool Y_F32>
__device__ void fold_partials(const LaunchArgs& a, int tb, int n0, int n1) {
  __shared__ int s_last;
  __syncthreads();  // this workgroup's partial stores are complete
  if (threadIdx.x == 0) {
    __threadfence();  // publish them device-wide: one release per workgroup
    s_last = atomicAdd(&a.tickets[tb], 1u) == (uint32_t)(a.S - 1);
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();  // acquire the other workgroups' partials
  const int width = n1 - n0;
  const long plane = (long)a.M * a.N;
  for (int idx = threadIdx.x; idx < a.M * width; idx += blockDim.x) {
    const int m = idx / width, n = n0 + idx % width;
    const float* p = a.part + (long)m * a.N + n;
    float sum = 0.f;
    for (int s = 0; s < a.S; ++s) sum += __builtin_nontemporal_load(p + s * plane);
    store_y<Y_F32>(a, (long)m * a.ldy + n, sum);
  }
  if (threadIdx.x == 0) atomicExch(&a.tickets[tb], 0u);
}

// Chunks of one workgroup's K split handed to wave wk of WK: c0+wk, c0+wk+WK, ...
struct ChunkRange {
  int c0, step, count;
  __device__ __forceinline__ int at(int j) const { return c0 + j * step; }
};

__device__ __forceinline__ ChunkRange wave_chunks(int c0, int c1, int wk, int WK) {
  ChunkRange cr;
  cr.c0 = c0 + wk;
  cr.step = WK;
  cr.count = c1 - c0 > wk ? (c1 - c0 - wk + WK - 1) / WK : 0;
  return cr;
}

// Per-wave timestamps of the timing build (compiled with QMM_WAVE_STAMPS; in
// ordinary builds every call below is empty).  mark(k) reads s_memrealtime,
// a 100 MHz counter common to the whole device, into a register; flush()
// writes the 16 stamps of the wave once, at its end, from lane 0 to
// 64-bit word skip + 16 * wave_index of a.part (skip: the words a kernel keeps
// for its own use there; the caller passes a workspace large enough; no store
// happens while the kernel runs, so the stamps do not delay it).
struct WaveStamps {
#ifdef QMM_WAVE_STAMPS
  uint64_t t[16];
  uint64_t* dst;
  __device__ __forceinline__ WaveStamps(const LaunchArgs& a, long wave_index, long skip = 0) {
    dst = a.part ? reinterpret_cast<uint64_t*>(a.part) + skip + wave_index * 16 : nullptr;
#pragma unroll
    for (int k = 0; k < 16; ++k) t[k] = 0;
  }
  __device__ __forceinline__ void mark(int k) {
    __builtin_amdgcn_sched_barrier(0);
    t[k] = __builtin_amdgcn_s_memrealtime();
    __builtin_amdgcn_sched_barrier(0);
  }
  __device__ __forceinline__ void flush(int lane) {
    if (dst && lane == 0) {
#pragma unroll
      for (int k = 0; k < 16; ++k) dst[k] = t[k];
    }
  }
#else
  __device__ __forceinline__ WaveStamps(const LaunchArgs&, long, long = 0) {}
  __device__ __forceinline__ void mark(int) {}
  __device__ __forceinline__ void flush(int) {}
#endif
};

// Wait and barrier helpers of the resident and slab kernels.
__device__ __forceinline__ void wg_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// s_waitcnt with only the vector-memory counter limited to N (N <= 63).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt out of range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// wait_vm<N>() that also waits for every outstanding LDS access.
template <int N>
__device__ __forceinline__ void wait_vm_lds() {
  static_assert(N >= 0 && N < 64, "vmcnt out of range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4));
}

// wait_vm<n * RPL>() for a count n in 0..C known once the caller is unrolled.
template <int RPL, int C>
__device__ __forceinline__ void wait_slices(int n) {
  if constexpr (C <= 0) {
    wait_vm<0>();
  } else {
    if (n >= C)
      wait_vm<C * RPL>();
    else
      wait_slices<RPL, C - 1>(n);
  }
}

// Timing build only: wait until at most n vector-memory loads of the wave are
// outstanding (n = the loads issued after the ones whose arrival is stamped).
template <int N>
__device__ __forceinline__ void stamp_wait() {
#ifdef QMM_WAVE_STAMPS
  wait_vm<(N < 63 ? N : 63)>();
#endif
}

// s_waitcnt for every outstanding LDS access (vector-memory counter untouched).
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }

}  // namespace qmm
