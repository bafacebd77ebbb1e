// qmm_kernels.hip -- gfx950 kernels for y = x . W^T over affine 3/4-bit,
// group-64 quantized weights.
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
// One-time loader and the test decoder.
// ---------------------------------------------------------------------------

template <int BITS, typename ST>
__global__ void __launch_bounds__(256) repack_kernel(const uint32_t* __restrict__ w,
                                                     const ST* __restrict__ scales,
                                                     const ST* __restrict__ biases,
                                                     uint32_t* __restrict__ codes,
                                                     ST* __restrict__ sb, int N, int K) {
  const long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const int nC = K / kChunkK, nT = N / kTileN;
  if (gid >= (long)nT * nC * 64) return;
  const int lane = (int)(gid & 63);
  const long blk = gid >> 6;
  const int c = (int)(blk % nC), tile = (int)(blk / nC);
  const int r = lane & 15, kg = lane >> 4, n = tile * kTileN + r;
  const uint32_t* row = w + (long)n * (K * BITS / 32);
  uint32_t out[BITS];
#pragma unroll
  for (int j = 0; j < BITS; ++j) out[j] = 0u;
  for (int gp = 0; gp < 2; ++gp)
    for (int i = 0; i < 16; ++i)
      place_code<BITS>(out, gp, i, mlx_code<BITS>(row, kChunkK * c + 64 * gp + 16 * kg + i));
#pragma unroll
  for (int j = 0; j < BITS; ++j) codes[blk * 64 * BITS + lane * BITS + j] = out[j];
  if (kg == 0) {
    const int G = K / 64;
    ST* e = sb + (blk * kTileN + r) * 4;
    e[0] = scales[(long)n * G + 2 * c];
    e[1] = scales[(long)n * G + 2 * c + 1];
    e[2] = biases[(long)n * G + 2 * c];
    e[3] = biases[(long)n * G + 2 * c + 1];
  }
}

template <int BITS>
__global__ void __launch_bounds__(256) debug_unpack_kernel(const uint32_t* __restrict__ codes,
                                                           uint8_t* __restrict__ out, int N,
                                                           int K) {
  const long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const int nC = K / kChunkK, nT = N / kTileN;
  if (gid >= (long)nT * nC * 64) return;
  const int lane = (int)(gid & 63);
  const long blk = gid >> 6;
  const int c = (int)(blk % nC), tile = (int)(blk / nC);
  const int r = lane & 15, kg = lane >> 4, n = tile * kTileN + r;
  uint32_t w[BITS], P[16];
#pragma unroll
  for (int j = 0; j < BITS; ++j) w[j] = codes[blk * 64 * BITS + lane * BITS + j];
  unpack_pairs<BITS>(w, P, pair_mask_vgpr<BITS>());
#pragma unroll
  for (int p = 0; p < 16; ++p) {
    const int gp = p >> 3, u = p & 7;
    const long k = (long)kChunkK * c + 64 * gp + 16 * kg + 2 * u;
    const int sh = (BITS == 3 && gp == 1) ? 3 : 0;  // group 1 of the 3-bit layout holds 8q
    out[(long)n * K + k] = (uint8_t)(((P[p] & 0xFFFFu) - 0x4300u) >> sh);
    out[(long)n * K + k + 1] = (uint8_t)(((P[p] >> 16) - 0x4300u) >> sh);
  }
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
template <bool Y_F32>
__device__ __forceinline__ void store_y(void* y, long idx, float v) {
  if constexpr (Y_F32)
    reinterpret_cast<float*>(y)[idx] = v;
  else
    reinterpret_cast<uint16_t*>(y)[idx] = f32_to_bf16(v);
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
    store_y<Y_F32>(a.y, (long)m * a.ldy + n, sum);
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

// ---------------------------------------------------------------------------
// MFMA kernel (bf16 activations).  Workgroup = 4 wavefronts arranged as
// WT = 4/WK tile groups x WK K-groups.  Wave (wt, wk) multiplies NTW tiles of
// W (16 rows each) by MT tiles of 16 activation rows over every WK-th chunk
// of the workgroup's K split; the WK partial tiles are added through LDS in
// order wk = 0, 1, ...  Loads run D chunks ahead in a statically indexed
// ring, so several chunks of weights are in flight per wave.
// ---------------------------------------------------------------------------
template <int BITS, int MT, int NTW, int WK, int D, typename ST>
__global__ void __launch_bounds__(kBlockThreads) mfma_kernel(LaunchArgs a) {
  constexpr int WT = kWaves / WK;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wt = wave / WK, wk = wave - wt * WK;
  const int r = lane & 15, kg = lane >> 4;
  const int item = xcd_item(blockIdx.x, a.nTB * a.S);
  const int tb = item / a.S, s = item - tb * a.S;
  const int nT = a.N / kTileN, nC = a.K / kChunkK;
  const int c0 = (int)((long)s * nC / a.S), c1 = (int)((long)(s + 1) * nC / a.S);
  const int tile0 = (tb * WT + wt) * NTW;
  const ChunkRange cr = wave_chunks(c0, c1, wk, WK);
  const uint16_t* __restrict__ x = reinterpret_cast<const uint16_t*>(a.x);
  const ST* __restrict__ sbp = reinterpret_cast<const ST*>(a.sb);

  f32x4 acc[NTW][MT];
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[nt][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (tile0 < nT && cr.count > 0) {
    bool tvalid[NTW];
    const uint32_t* cptr[NTW];
    const ST* sptr[NTW];
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
      const int t = tile0 + nt < nT ? tile0 + nt : nT - 1;
      tvalid[nt] = tile0 + nt < nT;
      cptr[nt] = a.codes + ((long)t * nC) * 64 * BITS + lane * BITS;
      sptr[nt] = sbp + ((long)t * nC * kTileN + r) * 4;
    }
    // Rows past the last activation row read the last row; their outputs are
    // never stored.
    const uint16_t* xrow[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = min(16 * mt + r, a.M - 1);
      xrow[mt] = x + (long)m * a.ldx + 16 * kg;
    }
    const PairMasks mask_v = pair_mask_vgpr<BITS>();
    const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};  // bf16 1.0 pairs
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};

    uint32_t W[D][NTW][BITS];
    SBPair<ST> SBv[D][NTW];
    u32x4 A[D][MT][4];
    auto load = [&](int j, int d) {
      const int c = cr.at(j);
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) {
        const uint32_t* p = cptr[nt] + (long)c * 64 * BITS;
#pragma unroll
        for (int q = 0; q < BITS; ++q) W[d][nt][q] = __builtin_nontemporal_load(p + q);
        SBv[d][nt].load(sptr[nt] + (long)c * kTileN * 4);
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int t = 0; t < 4; ++t)  // step t: group g' = t>>1, half h = t&1
          A[d][mt][t] = *reinterpret_cast<const u32x4*>(xrow[mt] + (long)kChunkK * c +
                                                        64 * (t >> 1) + 8 * (t & 1));
    };
    auto compute = [&](int d) {
      // sum_k x_k of each group, replicated in every column
      f32x4 EX[MT][2];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int gp = 0; gp < 2; ++gp) {
          const f32x4 e = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, A[d][mt][2 * gp]), __builtin_bit_cast(bf16x8, ones), zero,
              0, 0, 0);
          EX[mt][gp] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, A[d][mt][2 * gp + 1]), __builtin_bit_cast(bf16x8, ones),
              e, 0, 0, 0);
        }
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) {
        if (!tvalid[nt]) continue;
        uint32_t P[16];
        unpack_pairs<BITS>(W[d][nt], P, mask_v);
#pragma unroll
        for (int gp = 0; gp < 2; ++gp) {
          const Affine af = group_affine<BITS>(gp, SBv[d][nt].s(gp), SBv[d][nt].b(gp));
          const float sc = af.sc, bp = af.bp;
          const u32x4 B0 = {P[8 * gp + 0], P[8 * gp + 1], P[8 * gp + 2], P[8 * gp + 3]};
          const u32x4 B1 = {P[8 * gp + 4], P[8 * gp + 5], P[8 * gp + 6], P[8 * gp + 7]};
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            f32x4 dd = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, A[d][mt][2 * gp]), __builtin_bit_cast(bf16x8, B0), zero,
                0, 0, 0);
            dd = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, A[d][mt][2 * gp + 1]), __builtin_bit_cast(bf16x8, B1), dd,
                0, 0, 0);
#pragma unroll
            for (int q = 0; q < 4; ++q)
              if (16 * mt + q < a.M)
                acc[nt][mt][q] = fmaf(sc, dd[q], fmaf(bp, EX[mt][gp][q], acc[nt][mt][q]));
          }
        }
      }
    };
#pragma unroll
    for (int d = 0; d < D; ++d)
      if (d < cr.count) load(d, d);
    for (int j0 = 0; j0 < cr.count; j0 += D) {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        if (j0 + d < cr.count) {
          compute(d);
          if (j0 + d + D < cr.count) load(j0 + d + D, d);
        }
      }
    }
  }

  if constexpr (WK > 1) {
    __shared__ f32x4 red[WK - 1][WT][NTW * MT][64];
    if (wk > 0) {
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) red[wk - 1][wt][nt * MT + mt][lane] = acc[nt][mt];
    }
    __syncthreads();
    if (wk == 0) {
#pragma unroll
      for (int w = 1; w < WK; ++w)
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) acc[nt][mt] += red[w - 1][wt][nt * MT + mt][lane];
    }
  }

  // Output: lane holds column n = 16*tile + r, rows m = 16*mt + 4*kg + q.
  const bool writer = wk == 0 && tile0 < nT;
  if (a.S == 1) {
    if (!writer) return;
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
      if (tile0 + nt >= nT) continue;
      const int n = (tile0 + nt) * kTileN + r;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int m = 16 * mt + 4 * kg + q;
          if (m < a.M) store_y<false>(a.y, (long)m * a.ldy + n, acc[nt][mt][q]);
        }
    }
    return;
  }
  if (writer) {
    float* part = a.part + (long)s * a.M * a.N;
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
      if (tile0 + nt >= nT) continue;
      const int n = (tile0 + nt) * kTileN + r;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int m = 16 * mt + 4 * kg + q;
          if (m < a.M) __builtin_nontemporal_store(acc[nt][mt][q], part + (long)m * a.N + n);
        }
    }
  }
  const int n0 = tb * WT * NTW * kTileN;
  const int n1 = min(a.N, n0 + WT * NTW * kTileN);
  fold_partials<false>(a, tb, n0, n1);
}

// ---------------------------------------------------------------------------
// Streaming MFMA kernel for short activation blocks (at most 4 rows).  One
// workgroup owns one tile of W (16 rows) and all of K; its NW wavefronts take
// every NW-th chunk, at most CPW each.  Every wave works on its own data only
// until the final sum:
//   1. it loads the activation slices of its chunks (rows x 128 values each,
//      XL vectors of 16 bytes per lane), then issues the loads of ALL its
//      weight chunks, so a compute unit's whole share of W is in flight;
//   2. once the slices arrive (loads retire in issue order, so the weights
//      stay in flight) it stores them in its own LDS area, together with the
//      sum of every (row, group) slice (needed for the bias and the offset of
//      the unpacked codes);
//   3. per chunk, in arrival order: unpack, MFMA, per-group scale;
//   4. the NW partial tiles are added through LDS in wave order.
// No barrier precedes step 3: a wave's compute starts as soon as its own
// slices arrive, not when the slowest wave of the workgroup has its.
// LDS per wave: rows x (CPW*256 + 16) bytes of slices (the 16-byte pad puts
// consecutive rows on different banks) and rows x CPW x 2 group sums.
// ---------------------------------------------------------------------------
constexpr int kStreamRowPad = 16;
__device__ __forceinline__ float dpp_sum8(float s) {
  // sum over each aligned group of 8 lanes: swap neighbours, pairs, halves
  s += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, s), 0xB1, 0xF, 0xF, true));
  s += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, s), 0x4E, 0xF, 0xF, true));
  s += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, s), 0x141, 0xF, 0xF, true));
  return s;
}

// Vectors of 16 bytes per lane for rows (<= MQ) x CPW slices of 128 values.
template <int MQ, int CPW>
struct StreamXL { static constexpr int value = (MQ * CPW * 16 + 63) / 64; };

template <int BITS, int NW, int CPW, int MQ, typename ST>
__global__ void __launch_bounds__(NW * 64) stream_kernel(LaunchArgs a) {
  constexpr int XL = StreamXL<MQ, CPW>::value;
  constexpr int ROWB = CPW * 256 + kStreamRowPad;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, kg = lane >> 4;
  const int tile = blockIdx.x;
  const int nC = a.K / kChunkK;
  const int count = nC > w ? (nC - w + NW - 1) / NW : 0;  // chunks w, w+NW, ...
  const int clast = count > 0 ? w + (count - 1) * NW : 0;  // waves without chunks re-read chunk 0
  const ST* __restrict__ sbp = reinterpret_cast<const ST*>(a.sb);
  const uint16_t* __restrict__ xg = reinterpret_cast<const uint16_t*>(a.x);
  unsigned char* xw = lds + (size_t)w * a.M * ROWB;                           // [M][ROWB]
  float* xsum = reinterpret_cast<float*>(lds + (size_t)NW * a.M * ROWB) +
                (size_t)w * a.M * CPW * 2;                                     // [M][CPW][2]

  // 1. activation slices: vector v = (row m, slot j, part e); slots past
  //    `count` hold the last chunk's slice again (its results are dropped)
  const int nv = a.M * CPW * 16;
  u32x4 xv[XL];
  int xo[XL];
#pragma unroll
  for (int i = 0; i < XL; ++i) {
    const int v = min(lane + 64 * i, nv - 1);
    const int m = v / (CPW * 16), rem = v - m * (CPW * 16);
    const int j = rem >> 4, e = rem & 15;
    const int c = min(w + j * NW, clast);
    xv[i] = *reinterpret_cast<const u32x4*>(xg + (long)m * a.ldx + kChunkK * c + 8 * e);
    xo[i] = m * ROWB + j * 256 + 16 * e;
  }
  __builtin_amdgcn_sched_barrier(0);

  // weight loads of every slot; slots past `count` re-read the last chunk
  const uint32_t* cbase = a.codes + ((long)tile * nC) * 64 * BITS + lane * BITS;
  const ST* sbase = sbp + ((long)tile * nC * kTileN + r) * 4;
  uint32_t W[CPW][BITS];
  SBPair<ST> SBv[CPW];
#pragma unroll
  for (int j = 0; j < CPW; ++j) {
    const int c = min(w + j * NW, clast);
    const uint32_t* p = cbase + (long)c * 64 * BITS;
#pragma unroll
    for (int q = 0; q < BITS; ++q) W[j][q] = __builtin_nontemporal_load(p + q);
    SBv[j].load(sbase + (long)c * kTileN * 4);
  }
  __builtin_amdgcn_sched_barrier(0);

  // 2. slices and their group sums to this wave's LDS area.  The 8 lanes
  //    holding one (row, slot, group) are an aligned group of 8; lanes whose
  //    vector index is past the end hold a repeated vector and write no sum.
  const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
#pragma unroll
  for (int i = 0; i < XL; ++i) {
    *reinterpret_cast<u32x4*>(xw + xo[i]) = xv[i];
    // (each element is copied out first: a bit cast of a vector subscript
    // compiles to element 0 here)
    float s = 0.f;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t xd = xv[i][d], od = ones[d];
      s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, xd),
                                          __builtin_bit_cast(bf16x2, od), s, false);
    }
    s = dpp_sum8(s);
    const int v = lane + 64 * i;
    if (v < nv && (lane & 7) == 0) {
      const int m = v / (CPW * 16), rem = v - m * (CPW * 16);
      xsum[(m * CPW + (rem >> 4)) * 2 + ((rem >> 3) & 1)] = s;
    }
  }
  // other lanes of this wave read what these lanes wrote: keep the compiler
  // from moving the reads above the writes (LDS runs a wave's accesses in order)
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // 3. compute in load order; rows past the last one read the last row
  //    (never stored)
  const unsigned char* xrow = xw + min(r, a.M - 1) * ROWB + 32 * kg;
  const float* srow[MQ];
#pragma unroll
  for (int q = 0; q < MQ; ++q) srow[q] = xsum + min(4 * kg + q, a.M - 1) * CPW * 2;
  const PairMasks mask_v = pair_mask_vgpr<BITS>();
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  f32x4 acc = zero;
#pragma unroll
  for (int j = 0; j < CPW; ++j) {
    const bool live = j < count;
    u32x4 A[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
      A[t] = *reinterpret_cast<const u32x4*>(xrow + 256 * j + 128 * (t >> 1) + 16 * (t & 1));
    float2 ex[MQ];
#pragma unroll
    for (int q = 0; q < MQ; ++q) ex[q] = *reinterpret_cast<const float2*>(srow[q] + 2 * j);
    uint32_t P[16];
    unpack_pairs<BITS>(W[j], P, mask_v);
#pragma unroll
    for (int gp = 0; gp < 2; ++gp) {
      const u32x4 B0 = {P[8 * gp + 0], P[8 * gp + 1], P[8 * gp + 2], P[8 * gp + 3]};
      const u32x4 B1 = {P[8 * gp + 4], P[8 * gp + 5], P[8 * gp + 6], P[8 * gp + 7]};
      f32x4 dd = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          __builtin_bit_cast(bf16x8, A[2 * gp]), __builtin_bit_cast(bf16x8, B0), zero, 0, 0, 0);
      dd = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, A[2 * gp + 1]),
                                                   __builtin_bit_cast(bf16x8, B1), dd, 0, 0, 0);
      const Affine af = group_affine<BITS>(gp, SBv[j].s(gp), SBv[j].b(gp));
      const float sc = af.sc, bp = af.bp;
#pragma unroll
      for (int q = 0; q < MQ; ++q) {
        const float v = fmaf(sc, dd[q], fmaf(bp, gp ? ex[q].y : ex[q].x, acc[q]));
        acc[q] = live ? v : acc[q];
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  // 4. add the NW partial tiles in wave order and store rows < M
  f32x4* red = reinterpret_cast<f32x4*>(lds + (size_t)NW * a.M * (ROWB + CPW * 8));  // [NW-1][64]
  if (w > 0) red[(w - 1) * 64 + lane] = acc;
  __syncthreads();
  if (w != 0) return;
#pragma unroll
  for (int i = 1; i < NW; ++i) acc += red[(i - 1) * 64 + lane];
  const int n = tile * kTileN + r;
#pragma unroll
  for (int q = 0; q < MQ; ++q) {
    const int m = 4 * kg + q;
    if (m < a.M) store_y<false>(a.y, (long)m * a.ldy + n, acc[q]);
  }
}

size_t stream_lds_bytes(int nw, int cpw, int M) {
  return (size_t)nw * M * (cpw * 256 + kStreamRowPad + cpw * 8) + (size_t)(nw - 1) * 64 * 16;
}
bool stream_fits(int nw, int cpw, int M, size_t max_lds) {
  return M >= 1 && M <= kStreamMaxRows && stream_lds_bytes(nw, cpw, M) <= max_lds;
}


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

// s_waitcnt for every outstanding LDS access (vector-memory counter untouched).
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// ---------------------------------------------------------------------------
// Resident MFMA kernel for blocks of up to 16 activation rows whose whole
// activation block fits in LDS (rows*K*2 <= 160 KB).  Workgroup g owns the
// TM tiles g, g+G, g+2G, ... (G = grid size); its NW wavefronts split K:
// wave w takes chunks w, w+NW, ... (at most CPW) of every one of those tiles,
// so each activation fragment it reads, and each group sum it forms, serves
// TM tiles.  Order of work in a wave:
//   1. LDS-direct loads (no registers) of the activation slices of its
//      chunks, then the loads of ALL its weights (CPW chunks x TM tiles), so
//      a compute unit's whole share of W is in flight at once;
//   2. a wait for its own activation slices only (loads retire in issue
//      order, so the weights stay in flight); no barrier;
//   3. per chunk, in arrival order: the A fragments and the group sums
//      (all-ones MFMA), then per tile: unpack, MFMA, per-group scale;
//   4. the NW partial tiles of each tile are added through LDS (reusing the
//      activation space) in wave order.
// LDS holds chunk c's slice at c*M*256 bytes, row m's 16-byte vector e at
// position e ^ (m & 15) of its row, so the 16 rows an A-fragment read
// touches fall on distinct banks.  Tile slots past the last tile re-read the
// workgroup's first tile (cache hits; never stored).
// GU (fused gate/up): slots 0..TM/2-1 are gate tiles and slots TM/2..TM-1 the
// up tiles of the same columns (codes2/sb2); the store applies silu_mul().
// ---------------------------------------------------------------------------
// The fused gate/up epilogue ("mlx-bun 0.4.0 -> 1.0.0" page, the shared-M
// gate/up kernel of trellis-shared-m.ts): gate and up rounded to bf16 first,
// then the sigmoid of the rounded gate, the SiLU product and the final
// product, each rounded to bf16 (the unfused chain's roundings).
__device__ __forceinline__ float bf16_round(float v) { return bf16_to_f32(f32_to_bf16(v)); }
__device__ __forceinline__ float silu_mul(float gate, float up) {
  const float g = bf16_round(gate), u = bf16_round(up);
  const float sg = bf16_round(1.f / (1.f + expf(-g)));
  const float silu = bf16_round(g * sg);
  return silu * u;  // rounded to bf16 by the store
}

template <int BITS, int NW, int CPW, int TM, typename ST, bool GU = false>
__global__ void __launch_bounds__(NW * 64) resident_kernel(LaunchArgs a) {
  constexpr int TMH = GU ? TM / 2 : TM;  // distinct tiles per workgroup
  static_assert(!GU || TM % 2 == 0, "gate/up slots come in pairs");
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, kg = lane >> 4;
  const int G = gridDim.x, g = blockIdx.x;
  const int nT = a.N / kTileN, nC = a.K / kChunkK;
  const int M = a.M;
  const int count = nC > w ? (nC - w + NW - 1) / NW : 0;  // chunks w, w+NW, ...
  const int clast = count > 0 ? w + (count - 1) * NW : 0;  // waves without chunks re-read chunk 0
  const uint16_t* __restrict__ xg = reinterpret_cast<const uint16_t*>(a.x);
  const ST* __restrict__ sbp = reinterpret_cast<const ST*>(a.sb);

  // 1a. activation slices: 4 rows x 16 vectors per instruction, lanes of
  //     rows >= M masked off
#pragma unroll
  for (int j = 0; j < CPW; ++j) {
    const int c = min(w + j * NW, clast);
    unsigned char* region = lds + (size_t)c * M * 256;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (4 * i < M) {  // wave-uniform
        const int m = 4 * i + (lane >> 4);
        const int e = (lane & 15) ^ (m & 15);
        const uint16_t* src = xg + (long)min(m, M - 1) * a.ldx + kChunkK * c + 8 * e;
        if (m < M)
          __builtin_amdgcn_global_load_lds(
              (const __attribute__((address_space(1))) void*)src,
              (__attribute__((address_space(3))) void*)(region + i * 1024), 16, 0, 0);
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  // 1b. every weight load, chunk-major
  int tl[TM];
#pragma unroll
  for (int t = 0; t < TM; ++t) {
    const int tile = g + (t % TMH) * G;
    tl[t] = tile < nT ? tile : g;
  }
  const ST* __restrict__ sbp2 = reinterpret_cast<const ST*>(a.sb2);
  uint32_t W[CPW][TM][BITS];
  SBPair<ST> SBv[CPW][TM];
#pragma unroll
  for (int j = 0; j < CPW; ++j) {
    const int c = min(w + j * NW, clast);
#pragma unroll
    for (int t = 0; t < TM; ++t) {
      const bool second = GU && t >= TMH;  // compile-time once unrolled
      const uint32_t* p = (second ? a.codes2 : a.codes) + ((long)tl[t] * nC + c) * 64 * BITS +
                          lane * BITS;
#pragma unroll
      for (int q = 0; q < BITS; ++q) W[j][t][q] = __builtin_nontemporal_load(p + q);
      SBv[j][t].load((second ? sbp2 : sbp) + (((long)tl[t] * nC + c) * kTileN + r) * 4);
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  // 2. this wave's activation slices have landed once at most its weight
  //    loads (two per chunk and tile) are outstanding
  wait_vm<CPW * TM * 2>();

  // 3. compute in load order; rows past the last one read the last row
  //    (never stored)
  const int xm = min(r, M - 1);
  const int sw = xm & 15;
  const PairMasks mask_v = pair_mask_vgpr<BITS>();
  const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  f32x4 acc[TM];
#pragma unroll
  for (int t = 0; t < TM; ++t) acc[t] = zero;
#pragma unroll
  for (int j = 0; j < CPW; ++j) {
    const bool live = j < count;
    const int c = min(w + j * NW, clast);
    const u32x4* xrow = reinterpret_cast<const u32x4*>(lds + (size_t)c * M * 256) + xm * 16;
    u32x4 A[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)  // vector of (group q>>1, quarter kg, half q&1)
      A[q] = xrow[(8 * (q >> 1) + 2 * kg + (q & 1)) ^ sw];
    __builtin_amdgcn_sched_barrier(0);
    f32x4 ex[2];
#pragma unroll
    for (int gp = 0; gp < 2; ++gp) {
      const f32x4 e = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          __builtin_bit_cast(bf16x8, A[2 * gp]), __builtin_bit_cast(bf16x8, ones), zero, 0, 0, 0);
      ex[gp] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          __builtin_bit_cast(bf16x8, A[2 * gp + 1]), __builtin_bit_cast(bf16x8, ones), e, 0, 0, 0);
    }
#pragma unroll
    for (int t = 0; t < TM; ++t) {
      uint32_t P[16];
      unpack_pairs<BITS>(W[j][t], P, mask_v);
#pragma unroll
      for (int gp = 0; gp < 2; ++gp) {
        const u32x4 B0 = {P[8 * gp + 0], P[8 * gp + 1], P[8 * gp + 2], P[8 * gp + 3]};
        const u32x4 B1 = {P[8 * gp + 4], P[8 * gp + 5], P[8 * gp + 6], P[8 * gp + 7]};
        f32x4 dd = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, A[2 * gp]), __builtin_bit_cast(bf16x8, B0), zero, 0, 0, 0);
        dd = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, A[2 * gp + 1]),
                                                     __builtin_bit_cast(bf16x8, B1), dd, 0, 0, 0);
        const Affine af = group_affine<BITS>(gp, SBv[j][t].s(gp), SBv[j][t].b(gp));
        const float sc = live ? af.sc : 0.f, bp = live ? af.bp : 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[t][q] = fmaf(sc, dd[q], fmaf(bp, ex[gp][q], acc[t][q]));
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  // 4. add the NW partial tiles of each tile in wave order (slices are dead)
  __syncthreads();
  f32x4* red = reinterpret_cast<f32x4*>(lds);  // [TM][NW][64]
#pragma unroll
  for (int t = 0; t < TM; ++t) red[(t * NW + w) * 64 + lane] = acc[t];
  __syncthreads();
  if (w >= TMH) return;
  const int tile = g + w * G;
  if (tile >= nT) return;
  f32x4 v = red[(w * NW) * 64 + lane];
  for (int i = 1; i < NW; ++i) v += red[(w * NW + i) * 64 + lane];
  const int n = tile * kTileN + r;
  if constexpr (GU) {
    f32x4 u = red[((w + TMH) * NW) * 64 + lane];
    for (int i = 1; i < NW; ++i) u += red[((w + TMH) * NW + i) * 64 + lane];
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = silu_mul(v[q], u[q]);
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int m = 4 * kg + q;
    if (m < M) store_y<false>(a.y, (long)m * a.ldy + n, v[q]);
  }
}

// ---------------------------------------------------------------------------
// Slab kernel for 17..64 activation rows.  One workgroup per compute unit
// owning TM tiles of W; K is walked in NS slices of four chunks (512 k).
//   * four loader waves copy activation slices straight from global memory
//     into a ring of RB LDS slots (LDS-direct loads: no registers), running
//     up to RB-1 slices ahead; they wait only on their own loads;
//   * 4*TM compute waves: wave (i, kp) owns tile slot i and chunk kp of every
//     slice, keeps its weight loads DR slices ahead in a register ring, and
//     forms the per-group activation sums with an all-ones MFMA;
//   * one barrier per slice; the slice loop is unrolled, so every wait on
//     memory is an exact count and no wave waits on another's loads.
// An LDS slot holds [16*MT rows][64 vectors of 16 bytes]; row m keeps its
// vector v at v ^ (m & 15) (16 rows reading one column hit distinct banks).
// Rows >= M repeat row M-1 (their outputs are never stored).  The four
// partial tiles of each tile are added through LDS in K order at the end.
// ---------------------------------------------------------------------------
template <int BITS, int MT, int TM, int NS, int RB, int DR, typename ST>
__global__ void __launch_bounds__((TM * 4 + 4) * 64) slab_kernel(LaunchArgs a) {
  constexpr int KP = 4, NWC = TM * KP, NWL = 4;
  constexpr int ROWS = 16 * MT;
  constexpr int SK = KP * kChunkK;  // k per slice
  constexpr int SLOT = ROWS * 64;   // vectors per slot
  constexpr int RPL = ROWS / NWL;   // rows per loader wave per slice
  constexpr int NB = RB < NS ? RB : NS;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  u32x4* xs = reinterpret_cast<u32x4*>(lds);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nT = a.N / kTileN, nC = a.K / kChunkK;
  const int M = a.M;
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};

  if (wave >= NWC) {
    // ---- loader waves
    const int lw = __builtin_amdgcn_readfirstlane(wave - NWC);  // wave-uniform
    const uint16_t* __restrict__ xg = reinterpret_cast<const uint16_t*>(a.x);
    auto issue = [&](int s) {
      u32x4* slot = xs + (s % RB) * SLOT;
#pragma unroll
      for (int i = 0; i < RPL; ++i) {
        const int m = lw + i * NWL;
        const int v = lane ^ (m & 15);
        const int col = min(s * SK + 8 * v, a.K - 8);
        const uint16_t* src = xg + (long)min(m, M - 1) * a.ldx + col;
        __builtin_amdgcn_global_load_lds(
            (const __attribute__((address_space(1))) void*)src,
            (__attribute__((address_space(3))) void*)(slot + m * 64), 16, 0, 0);
      }
    };
#pragma unroll
    for (int s = 0; s < NB; ++s) issue(s);
    wait_vm<(NB - 1) * RPL>();
    wg_barrier();
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      // after barrier j every compute wave is done with slice j-1
      if (j >= 1 && j - 1 + RB < NS) issue(j - 1 + RB);
      if (j + 1 < NS) {
        // slices issued after slice j+1 may stay in flight
        const int last = min(j >= 1 ? j - 1 + RB : RB - 1, NS - 1);
        wait_slices<RPL, RB - 2>(last - (j + 1));
      }
      wg_barrier();
    }
  } else {
    // ---- compute waves
    const int slot_i = __builtin_amdgcn_readfirstlane(wave / KP);  // wave-uniform
    const int kp = __builtin_amdgcn_readfirstlane(wave - slot_i * KP);
    const int r = lane & 15, kg = lane >> 4;
    const int tile = blockIdx.x + slot_i * gridDim.x;
    const bool active = tile < nT;
    const int t = active ? tile : nT - 1;
    const ST* __restrict__ sbp = reinterpret_cast<const ST*>(a.sb);
    const uint32_t* cbase = a.codes + ((long)t * nC) * 64 * BITS + lane * BITS;
    const ST* sbase = sbp + ((long)t * nC * kTileN + r) * 4;
    uint32_t W[DR][BITS];
    SBPair<ST> SBv[DR];
    auto load = [&](int s, int d) {
      const int c = min(s * KP + kp, nC - 1);
      const uint32_t* p = cbase + (long)c * 64 * BITS;
#pragma unroll
      for (int q = 0; q < BITS; ++q) W[d][q] = __builtin_nontemporal_load(p + q);
      SBv[d].load(sbase + (long)c * kTileN * 4);
    };
#pragma unroll
    for (int d = 0; d < DR; ++d)
      if (d < NS) load(d, d);
    const PairMasks mask_v = pair_mask_vgpr<BITS>();
    const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
    f32x4 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = zero;
    wg_barrier();
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const int d = j % DR;
      const bool live = j * KP + kp < nC;
      const u32x4* slot = xs + (j % RB) * SLOT;
      uint32_t P[16];
      unpack_pairs<BITS>(W[d], P, mask_v);
      float sc[2], bp[2];
#pragma unroll
      for (int gp = 0; gp < 2; ++gp) {
        // group_affine() spelled out: this form keeps the kernel within 128 VGPRs
        const float s0 = SBv[d].s(gp);
        constexpr bool c3 = BITS == 3;
        sc[gp] = live ? (c3 && gp == 1 ? s0 * 0.125f : s0) : 0.f;
        bp[gp] = live ? SBv[d].b(gp) - (c3 && gp == 1 ? 16.f : 128.f) * s0 : 0.f;
      }
      // every activation read of the slice is issued before its first MFMA
      constexpr int MA = MT <= 2 ? MT : 2;  // m-tiles whose fragments are read together
#pragma unroll
      for (int m0 = 0; m0 < MT; m0 += MA) {
        u32x4 A[MA][4];
#pragma unroll
        for (int mi = 0; mi < MA; ++mi) {
          const u32x4* xrow = slot + (16 * (m0 + mi) + r) * 64;
#pragma unroll
          for (int q = 0; q < 4; ++q)  // vector of (chunk kp, group q>>1, quarter kg, half q&1)
            A[mi][q] = xrow[(16 * kp + 8 * (q >> 1) + 2 * kg + (q & 1)) ^ r];
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int mi = 0; mi < MA; ++mi) {
          const int mt = m0 + mi;
#pragma unroll
          for (int gp = 0; gp < 2; ++gp) {
            const f32x4 e = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, A[mi][2 * gp]), __builtin_bit_cast(bf16x8, ones), zero, 0,
                0, 0);
            const f32x4 ex = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, A[mi][2 * gp + 1]), __builtin_bit_cast(bf16x8, ones), e, 0,
                0, 0);
            const u32x4 B0 = {P[8 * gp + 0], P[8 * gp + 1], P[8 * gp + 2], P[8 * gp + 3]};
            const u32x4 B1 = {P[8 * gp + 4], P[8 * gp + 5], P[8 * gp + 6], P[8 * gp + 7]};
            f32x4 dd = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, A[mi][2 * gp]), __builtin_bit_cast(bf16x8, B0), zero, 0, 0,
                0);
            dd = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, A[mi][2 * gp + 1]),
                                                         __builtin_bit_cast(bf16x8, B1), dd, 0, 0, 0);
#pragma unroll
            for (int q = 0; q < 4; ++q)
              acc[mt][q] = fmaf(sc[gp], dd[q], fmaf(bp[gp], ex[q], acc[mt][q]));
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (j + DR < NS) load(j + DR, d);
      wait_lds();
      wg_barrier();
    }
    // fold the KP partial tiles of this tile slot in K order (slots are dead)
    f32x4* red = reinterpret_cast<f32x4*>(lds);  // [TM][MT][KP][64]
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) red[((slot_i * MT + mt) * KP + kp) * 64 + lane] = acc[mt];
    __syncthreads();
    if (kp != 0 || !active) return;
    const int n = tile * kTileN + r;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      f32x4 v = acc[mt];
#pragma unroll
      for (int i = 1; i < KP; ++i) v += red[((slot_i * MT + mt) * KP + i) * 64 + lane];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m = 16 * mt + 4 * kg + q;
        if (m < M) store_y<false>(a.y, (long)m * a.ldy + n, v[q]);
      }
    }
    return;
  }
  __syncthreads();  // loader waves: partner of the compute waves' fold barrier
}

// ---------------------------------------------------------------------------
// Split slab kernel for 17..64 activation rows.  The slab kernel's loader /
// compute structure, changed where a 64-row block spends its time: every
// compute unit of the slab kernel takes in the whole activation block
// (655 KB at K = 5120) and reads each fragment from LDS once per W tile.
//   * K is cut into S parts (S = 1 or 2): workgroup (g, s) covers the
//     TG = NSLOT*TW W tiles of tile group g over the NS slices of part s, so
//     a compute unit takes in only its part of the activations;
//   * compute wave (slot, kp) serves TW tiles (chunk kp of every slice):
//     each A fragment it reads and each group sum (all-ones MFMA) it forms
//     serves TW tiles; a tile's packed weights are unpacked once per slice,
//     DR slices of weight loads are kept in flight in a register ring.
// The KP = 4 partial tiles of a tile are added through LDS in K order.  With
// S = 2 each workgroup then stores its partial tiles with device-coherent
// stores (written through to the point of coherence for the whole device,
// so no L2 write-back is needed), waits for them, and takes a ticket; the
// workgroup that arrives second adds the two partials (a + b is the same in
// either order) and writes y, then re-arms the ticket.  Workgroups are
// numbered g*S + s and dealt to the XCDs round-robin, so with S = 2 each
// XCD's L2 holds one part of the activation block.
// ---------------------------------------------------------------------------
template <int BITS, int MT, int TW, int NSLOT, int NS, int RB, int DR, typename ST>
__global__ void __launch_bounds__((NSLOT * 4 + 4) * 64) split_slab_kernel(LaunchArgs a) {
  constexpr int KP = 4, NWC = NSLOT * KP, NWL = 4;
  constexpr int ROWS = 16 * MT;
  constexpr int SK = KP * kChunkK;  // k per slice
  constexpr int SLOT = ROWS * 64;   // vectors per slot
  constexpr int RPL = ROWS / NWL;   // rows per loader wave per slice
  constexpr int NB = RB < NS ? RB : NS;
  constexpr int TG = NSLOT * TW;    // W tiles per workgroup
  static_assert(MT >= 2 && MT <= KP, "one folded row tile per compute wave");
  static_assert(TG * MT * KP * 1024 <= RB * SLOT * 16, "fold area exceeds the ring");
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  __shared__ int s_last;
  u32x4* xs = reinterpret_cast<u32x4*>(lds);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nT = a.N / kTileN, nC = a.K / kChunkK;
  const int M = a.M, S = a.S;
  const int grp = blockIdx.x / S, kpart = blockIdx.x - grp * S;
  const int sl0 = kpart * NS;  // first slice of this workgroup's part of K
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  const int slot_i = __builtin_amdgcn_readfirstlane(wave / KP);  // wave-uniform
  const int kp = __builtin_amdgcn_readfirstlane(wave - slot_i * KP);
  const int r = lane & 15, kg = lane >> 4;
  f32x4* red = reinterpret_cast<f32x4*>(lds);  // fold area [TG][MT][KP][64], after the loop

  if (wave >= NWC) {
    // ---- loader waves
    const int lw = __builtin_amdgcn_readfirstlane(wave - NWC);  // wave-uniform
    const uint16_t* __restrict__ xg = reinterpret_cast<const uint16_t*>(a.x);
    auto issue = [&](int s) {
      u32x4* slot = xs + (s % RB) * SLOT;
#pragma unroll
      for (int i = 0; i < RPL; ++i) {
        const int m = lw + i * NWL;
        const int v = lane ^ (m & 15);
        const int col = min((sl0 + s) * SK + 8 * v, a.K - 8);
        const uint16_t* src = xg + (long)min(m, M - 1) * a.ldx + col;
        __builtin_amdgcn_global_load_lds(
            (const __attribute__((address_space(1))) void*)src,
            (__attribute__((address_space(3))) void*)(slot + m * 64), 16, 0, 0);
      }
    };
#pragma unroll
    for (int s = 0; s < NB; ++s) issue(s);
    wait_vm<(NB - 1) * RPL>();
    wg_barrier();
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      // after barrier j every compute wave is done with slice j-1
      if (j >= 1 && j - 1 + RB < NS) issue(j - 1 + RB);
      if (j + 1 < NS) {
        const int last = min(j >= 1 ? j - 1 + RB : RB - 1, NS - 1);
        wait_slices<RPL, RB - 2>(last - (j + 1));
      }
      wg_barrier();
    }
  } else {
    // ---- compute waves
    const ST* __restrict__ sbp = reinterpret_cast<const ST*>(a.sb);
    int tl[TW];
#pragma unroll
    for (int i = 0; i < TW; ++i) tl[i] = min(grp * TG + slot_i * TW + i, nT - 1);
    // weight ring: slice j's codes and scales/biases in slot j % DR
    uint32_t W[DR][TW][BITS];
    SBPair<ST> SBv[DR][TW];
    auto load = [&](int j) {
      const int c = min((sl0 + j) * KP + kp, nC - 1);
      const int d = j % DR;
#pragma unroll
      for (int i = 0; i < TW; ++i) {
        const uint32_t* p = a.codes + ((long)tl[i] * nC + c) * 64 * BITS + lane * BITS;
#pragma unroll
        for (int q = 0; q < BITS; ++q) W[d][i][q] = __builtin_nontemporal_load(p + q);
        SBv[d][i].load(sbp + ((long)tl[i] * nC * kTileN + r) * 4 + (long)c * kTileN * 4);
      }
    };
#pragma unroll
    for (int j = 0; j < DR; ++j)
      if (j < NS) load(j);
    const PairMasks mask_v = pair_mask_vgpr<BITS>();
    const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
    f32x4 acc[TW][MT];
#pragma unroll
    for (int i = 0; i < TW; ++i)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[i][mt] = zero;
    wg_barrier();
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const bool live = (sl0 + j) * KP + kp < nC;
      const u32x4* slot = xs + (j % RB) * SLOT;
      // group by group: only one group's unpacked pairs are live at a time
      // (the other half of each unpack is dead code); slice j + DR's weight
      // loads go out once the second group is unpacked
#pragma unroll
      for (int gp = 0; gp < 2; ++gp) {
        uint32_t P[TW][16];
        float sc[TW], bp[TW];
#pragma unroll
        for (int i = 0; i < TW; ++i) {
          unpack_pairs<BITS>(W[j % DR][i], P[i], mask_v);
          const float s0 = SBv[j % DR][i].s(gp);
          constexpr bool c3 = BITS == 3;
          sc[i] = live ? (c3 && gp == 1 ? s0 * 0.125f : s0) : 0.f;
          bp[i] = live ? SBv[j % DR][i].b(gp) - (c3 && gp == 1 ? 16.f : 128.f) * s0 : 0.f;
        }
        if (gp == 1 && j + DR < NS) load(j + DR);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const u32x4* xrow = slot + (16 * mt + r) * 64;
          u32x4 A[2];
#pragma unroll
          for (int h = 0; h < 2; ++h)  // vector of (chunk kp, group gp, quarter kg, half h)
            A[h] = xrow[(16 * kp + 8 * gp + 2 * kg + h) ^ r];
          __builtin_amdgcn_sched_barrier(0);
          const f32x4 e = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, A[0]), __builtin_bit_cast(bf16x8, ones), zero, 0, 0, 0);
          const f32x4 ex = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, A[1]), __builtin_bit_cast(bf16x8, ones), e, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < TW; ++i) {
            const u32x4 B0 = {P[i][8 * gp + 0], P[i][8 * gp + 1], P[i][8 * gp + 2], P[i][8 * gp + 3]};
            const u32x4 B1 = {P[i][8 * gp + 4], P[i][8 * gp + 5], P[i][8 * gp + 6], P[i][8 * gp + 7]};
            f32x4 dd = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, A[0]), __builtin_bit_cast(bf16x8, B0), zero, 0, 0, 0);
            dd = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, A[1]),
                                                         __builtin_bit_cast(bf16x8, B1), dd, 0, 0, 0);
#pragma unroll
            for (int q = 0; q < 4; ++q)
              acc[i][mt][q] = fmaf(sc[i], dd[q], fmaf(bp[i], ex[q], acc[i][mt][q]));
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      wait_lds();
      wg_barrier();
    }
    // the slots are dead: park the partial tiles for the fold
#pragma unroll
    for (int i = 0; i < TW; ++i)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        red[(((slot_i * TW + i) * MT + mt) * KP + kp) * 64 + lane] = acc[i][mt];
  }
  __syncthreads();
  // wave (slot, kp) folds row tile mt = kp of its TW tiles in K order
  const bool folds = wave < NWC && kp < MT;
  const int mt = kp;
  f32x4 v[TW];
  if (folds) {
#pragma unroll
    for (int i = 0; i < TW; ++i) {
      const int base = ((slot_i * TW + i) * MT + mt) * KP;
      v[i] = red[base * 64 + lane];
#pragma unroll
      for (int k = 1; k < KP; ++k) v[i] += red[(base + k) * 64 + lane];
    }
  }
  auto store_tiles = [&]() {
#pragma unroll
    for (int i = 0; i < TW; ++i) {
      const int tile = grp * TG + slot_i * TW + i;
      if (tile >= nT) continue;
      const int n = tile * kTileN + r;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m = 16 * mt + 4 * kg + q;
        if (m < M) store_y<false>(a.y, (long)m * a.ldy + n, v[i][q]);
      }
    }
  };
  if (S == 1) {
    if (folds) store_tiles();
    return;
  }
  // S == 2: partial tile (grp, kpart, slot, i, mt) at part[(((grp*S + kpart)*TG + slot*TW + i)*MT
  // + mt)*256 + q*64 + lane]
  auto part_at = [&](int kq, int i, int q) {
    return a.part + ((((long)(grp * S + kq) * TG + slot_i * TW + i) * MT + mt) * 4 + q) * 64 + lane;
  };
  if (folds) {
#pragma unroll
    for (int i = 0; i < TW; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        __hip_atomic_store(part_at(kpart, i, q), v[i][q], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    wait_vm<0>();  // the partials have reached the point of coherence
  }
  __syncthreads();
  if (threadIdx.x == 0)
    s_last = __hip_atomic_fetch_add(&a.tickets[grp], 1u, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)(S - 1);
  __syncthreads();
  if (!s_last) return;
  if (folds) {
#pragma unroll
    for (int i = 0; i < TW; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        v[i][q] += __hip_atomic_load(part_at(1 - kpart, i, q), __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
    store_tiles();
  }
  if (threadIdx.x == 0)
    __hip_atomic_store(&a.tickets[grp], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// Wide kernel for 65..128 activation rows (the compute/bandwidth crossover).
// At 128 rows the per-group epilogue of the factored dequant (two FMAs per
// output and group) would cost more vector instructions than the weights
// themselves, so here every weight is dequantized once, in registers, to
// bf16 (w = s*q + b from the same unpacked pairs and group factors, rounded
// to nearest even) and the MFMAs accumulate y directly over all of K: no
// all-ones MFMA, no epilogue.  The rounding of w to bf16 (relative 2^-9) is
// inside the accuracy bound of bf16 activations.
//   * one workgroup owns TG = 8 W tiles (4 slots of 2) over all of K and all
//     16*MT rows (MT = 6 up to 96 rows, else 8); 8 compute waves = 4
//     tile-pair slots x 2 chunk positions, 4 loader waves;
//   * activation slices of 256 columns x 16*MT rows (48 or 64 KB) through a
//     2-slot LDS ring by LDS-direct loads; each A fragment read from LDS serves the
//     wave's 2 tiles; one barrier per slice; the slice loop is a run-time
//     loop (with a 2-slot ring every wait is the same count);
//   * within a slice the work goes k-step by k-step (32 k): dequantize the
//     step's B fragments of both tiles, then its 16 MFMAs (8 row tiles x 2
//     tiles), with no scheduling barriers, so the next step's dequant and
//     fragment reads overlap the MFMAs;
//   * the next slice's weight words are loaded as soon as the current ones
//     are unpacked; the 2 chunk positions' partial tiles are added through
//     LDS in K order at the end.
// ---------------------------------------------------------------------------
template <int BITS, int MT, typename ST>
__global__ void __launch_bounds__(12 * 64) wide_kernel(LaunchArgs a) {
  constexpr int TW = 2, NSLOT = 4, KP = 2, NWC = NSLOT * KP, NWL = 4;
  static_assert(MT % KP == 0 && MT <= kWideRowTiles, "whole row tiles per chunk position");
  constexpr int ROWS = 16 * MT;
  constexpr int SK = KP * kChunkK;  // k per slice (256)
  constexpr int VPR = SK / 8;       // 16-byte vectors per row per slice (32)
  constexpr int SLOT = ROWS * VPR;  // vectors per slot
  constexpr int RB = 2;
  constexpr int TG = NSLOT * TW;
  constexpr int PAIRS = ROWS / 2 / NWL;  // row pairs per loader wave per slice (16)
  static_assert(TG * MT * KP * 1024 <= RB * SLOT * 16, "fold area exceeds the ring");
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  u32x4* xs = reinterpret_cast<u32x4*>(lds);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nT = a.N / kTileN, nC = a.K / kChunkK;
  const int NS = nC / KP;
  const int M = a.M;
  const int r = lane & 15, kg = lane >> 4;
  const int slot_i = __builtin_amdgcn_readfirstlane(wave / KP);
  const int kp = __builtin_amdgcn_readfirstlane(wave - slot_i * KP);
  f32x4* red = reinterpret_cast<f32x4*>(lds);  // [TG][MT][KP][64] after the loop

  if (wave >= NWC) {
    // ---- loader waves: row pair p of this wave covers rows 2p', 2p'+1 with
    // p' = lw + p * NWL; lanes 0..31 the first row, 32..63 the second
    const int lw = __builtin_amdgcn_readfirstlane(wave - NWC);
    const uint16_t* __restrict__ xg = reinterpret_cast<const uint16_t*>(a.x);
    auto issue = [&](int s) {
      u32x4* slot = xs + (s & 1) * SLOT;
#pragma unroll
      for (int i = 0; i < PAIRS; ++i) {
        const int m0 = 2 * (lw + i * NWL);
        const int m = m0 + (lane >> 5);
        const int v = (lane & 31) ^ (m & 15);
        const uint16_t* src = xg + (long)min(m, M - 1) * a.ldx + s * SK + 8 * v;
        __builtin_amdgcn_global_load_lds(
            (const __attribute__((address_space(1))) void*)src,
            (__attribute__((address_space(3))) void*)(slot + m0 * VPR), 16, 0, 0);
      }
    };
    issue(0);
    if (NS > 1) {
      issue(1);
      wait_vm<PAIRS>();
    } else {
      wait_vm<0>();
    }
    wg_barrier();
    for (int j = 0; j < NS; ++j) {
      if (j + 1 < NS) wait_vm<0>();  // slice j+1 has landed
      wg_barrier();                  // and every compute wave is done with slice j
      if (j + 2 < NS) issue(j + 2);  // into slice j's slot
    }
  } else {
    // ---- compute waves: slot slot_i (tiles g*TG + 2 slot_i + {0,1}), chunk kp
    const ST* __restrict__ sbp = reinterpret_cast<const ST*>(a.sb);
    int tl[TW];
#pragma unroll
    for (int i = 0; i < TW; ++i) tl[i] = min(blockIdx.x * TG + slot_i * TW + i, nT - 1);
    uint32_t W[TW][BITS];
    SBPair<ST> SBv[TW];
    auto load = [&](int j) {
      const int c = j * KP + kp;
#pragma unroll
      for (int i = 0; i < TW; ++i) {
        const uint32_t* p = a.codes + ((long)tl[i] * nC + c) * 64 * BITS + lane * BITS;
#pragma unroll
        for (int q = 0; q < BITS; ++q) W[i][q] = __builtin_nontemporal_load(p + q);
        SBv[i].load(sbp + ((long)tl[i] * nC * kTileN + r) * 4 + (long)c * kTileN * 4);
      }
    };
    load(0);
    const PairMasks mask_v = pair_mask_vgpr<BITS>();
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    f32x4 acc[TW][MT];
#pragma unroll
    for (int i = 0; i < TW; ++i)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[i][mt] = zero;
    wg_barrier();
    for (int j = 0; j < NS; ++j) {
      const u32x4* slot = xs + (j & 1) * SLOT;
      // k-step by k-step (32 k): step q's B fragments of both tiles are
      // dequantized, then its MFMAs run for every row tile.  No scheduling
      // barriers here: the compiler overlaps the next step's dequant and
      // A-fragment reads with this step's MFMAs (16 independent accumulators)
#pragma unroll
      for (int gp = 0; gp < 2; ++gp) {
        uint32_t P[TW][16];
        Affine f[TW];
#pragma unroll
        for (int i = 0; i < TW; ++i) {
          unpack_pairs<BITS>(W[i], P[i], mask_v);
          f[i] = group_affine<BITS>(gp, SBv[i].s(gp), SBv[i].b(gp));
        }
        if (gp == 1 && j + 1 < NS) load(j + 1);  // the raw words are unpacked
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int q = 2 * gp + h;
          u32x4 B[TW];
#pragma unroll
          for (int i = 0; i < TW; ++i) {
            uint32_t bd[4];
#pragma unroll
            for (int pp = 0; pp < 4; ++pp) {
              const uint32_t v = P[i][8 * gp + 4 * h + pp];
              const float lo = fmaf(f[i].sc, __uint_as_float(v << 16), f[i].bp);
              const float hi = fmaf(f[i].sc, __uint_as_float(v & 0xFFFF0000u), f[i].bp);
              typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
              const bf16x2_t pk = {(__bf16)lo, (__bf16)hi};
              bd[pp] = __builtin_bit_cast(uint32_t, pk);
            }
            B[i] = u32x4{bd[0], bd[1], bd[2], bd[3]};
          }
          u32x4 A[MT];  // vector (chunk kp, group gp, quarter kg, half h) of each row tile
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            A[mt] = slot[(16 * mt + r) * VPR + ((16 * kp + 8 * gp + 2 * kg + h) ^ r)];
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < TW; ++i)
              acc[i][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  __builtin_bit_cast(bf16x8, A[mt]), __builtin_bit_cast(bf16x8, B[i]), acc[i][mt], 0, 0, 0);
        }
      }
      wait_lds();
      wg_barrier();
    }
    // park the partial tiles (the slots are dead)
#pragma unroll
    for (int i = 0; i < TW; ++i)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        red[(((slot_i * TW + i) * MT + mt) * KP + kp) * 64 + lane] = acc[i][mt];
  }
  __syncthreads();
  if (wave >= NWC) return;
  // wave (slot, kp) adds the two chunk positions of row tiles kp*MT/2 .. and stores y
#pragma unroll
  for (int i = 0; i < TW; ++i) {
    const int tile = blockIdx.x * TG + slot_i * TW + i;
    if (tile >= nT) continue;
    const int n = tile * kTileN + r;
#pragma unroll
    for (int h = 0; h < MT / KP; ++h) {
      const int mt = kp * (MT / KP) + h;
      const int base = ((slot_i * TW + i) * MT + mt) * KP;
      f32x4 v = red[base * 64 + lane];
#pragma unroll
      for (int k = 1; k < KP; ++k) v += red[(base + k) * 64 + lane];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m = 16 * mt + 4 * kg + q;
        if (m < M) store_y<false>(a.y, (long)m * a.ldy + n, v[q]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Vector-ALU kernel: up to MR activation rows per pass, activations of the
// workgroup's K split staged in LDS together with per-(row, group, quarter)
// sums.  Each of the 4 wavefronts owns NTW tiles; lane (r, kg) accumulates
// its quarter of each group with v_dot2_f32_bf16 on (128+q, x) pairs, and the
// four quarters are added with cross-lane shuffles at the end.  Weight loads
// run D chunks ahead in a statically indexed ring.
// ---------------------------------------------------------------------------
template <bool X_F32>
using XStore = typename std::conditional<X_F32, float, uint16_t>::type;

size_t gemv_lds_bytes(bool x_f32, int mr, int kslice) {
  return (size_t)mr * kslice * (x_f32 ? 4 : 2) + (size_t)mr * (kslice / 64) * 4 * sizeof(float);
}

template <int BITS, int MR, int NTW, bool X_F32, typename ST>
__global__ void __launch_bounds__(kBlockThreads) gemv_kernel(LaunchArgs a) {
  constexpr int D = 4;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  using XT = XStore<X_F32>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, kg = lane >> 4;
  const int item = xcd_item(blockIdx.x, a.nTB * a.S);
  const int tb = item / a.S, s = item - tb * a.S;
  const int nT = a.N / kTileN, nC = a.K / kChunkK;
  const int c0 = (int)((long)s * nC / a.S), c1 = (int)((long)(s + 1) * nC / a.S);
  const int ks = (c1 - c0) * kChunkK, gs = ks / 64;
  const int tile0 = (tb * kWaves + wave) * NTW;
  const int nchunks = c1 - c0;
  const ST* __restrict__ sbp = reinterpret_cast<const ST*>(a.sb);
  XT* xs = reinterpret_cast<XT*>(lds);                                       // [MR][ks]
  float* xq = reinterpret_cast<float*>(lds + (size_t)MR * ks * sizeof(XT));  // [MR][gs][4]

  bool tvalid[NTW];
  const uint32_t* cptr[NTW];
  const ST* sptr[NTW];
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
    const int t = tile0 + nt < nT ? tile0 + nt : nT - 1;
    tvalid[nt] = tile0 + nt < nT;
    cptr[nt] = a.codes + ((long)t * nC) * 64 * BITS + lane * BITS;
    sptr[nt] = sbp + ((long)t * nC * kTileN + r) * 4;
  }
  uint32_t W[D][NTW][BITS];
  SBPair<ST> SBv[D][NTW];
  auto load = [&](int j, int d) {
    const int c = c0 + j;
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
      const uint32_t* p = cptr[nt] + (long)c * 64 * BITS;
#pragma unroll
      for (int q = 0; q < BITS; ++q) W[d][nt][q] = __builtin_nontemporal_load(p + q);
      SBv[d][nt].load(sptr[nt] + (long)c * kTileN * 4);
    }
  };
  const bool active = tile0 < nT && nchunks > 0;
  // First weight loads go out before the activation staging.
  if (active) {
#pragma unroll
    for (int d = 0; d < D; ++d)
      if (d < nchunks) load(d, d);
  }

  // Stage the activation slice, 16 bytes per thread per step.
  {
    constexpr int per16 = 16 / sizeof(XT);
    const int vecs_per_row = ks / per16;
    const XT* xg = reinterpret_cast<const XT*>(a.x);
    for (int idx = threadIdx.x; idx < a.M * vecs_per_row; idx += kBlockThreads) {
      const int m = idx / vecs_per_row, v = idx - m * vecs_per_row;
      const uint4 val = *reinterpret_cast<const uint4*>(xg + (long)m * a.ldx +
                                                        (long)kChunkK * c0 + v * per16);
      *reinterpret_cast<uint4*>(xs + (long)m * ks + v * per16) = val;
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < a.M * gs * 4; idx += kBlockThreads) {
    const int m = idx / (gs * 4), rem = idx - m * gs * 4;
    const XT* p = xs + (long)m * ks + 16 * rem;  // rem = g*4 + quarter
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if constexpr (X_F32)
        sum += p[i];
      else
        sum += bf16_to_f32(p[i]);
    }
    xq[idx] = sum;
  }
  __syncthreads();

  float acc[NTW][MR];
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
    for (int m = 0; m < MR; ++m) acc[nt][m] = 0.f;

  if (active) {
    const PairMasks mask_v = pair_mask_vgpr<BITS>();
    auto compute = [&](int j, int d) {
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) {
        if (!tvalid[nt]) continue;
        uint32_t P[16];
        unpack_pairs<BITS>(W[d][nt], P, mask_v);
#pragma unroll
        for (int gp = 0; gp < 2; ++gp) {
          const Affine af = group_affine<BITS>(gp, SBv[d][nt].s(gp), SBv[d][nt].b(gp));
          const float sc = af.sc, bp = af.bp;
          const int kl = kChunkK * j + 64 * gp + 16 * kg;  // lane's 16 columns
#pragma unroll
          for (int m = 0; m < MR; ++m) {
            if (m >= a.M) break;
            float dot = 0.f;
            if constexpr (X_F32) {
              const float4* xp = reinterpret_cast<const float4*>(xs + (long)m * ks + kl);
#pragma unroll
              for (int v = 0; v < 4; ++v) {
                const float4 xv = xp[v];
                const uint32_t p0 = P[8 * gp + 2 * v], p1 = P[8 * gp + 2 * v + 1];
                dot = fmaf(__uint_as_float(p0 << 16), xv.x, dot);
                dot = fmaf(__uint_as_float(p0 & 0xFFFF0000u), xv.y, dot);
                dot = fmaf(__uint_as_float(p1 << 16), xv.z, dot);
                dot = fmaf(__uint_as_float(p1 & 0xFFFF0000u), xv.w, dot);
              }
            } else {
              const uint4* xp = reinterpret_cast<const uint4*>(xs + (long)m * ks + kl);
#pragma unroll
              for (int v = 0; v < 2; ++v) {
                const uint4 xv = xp[v];
                const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
                for (int e = 0; e < 4; ++e)
                  dot = __builtin_amdgcn_fdot2_f32_bf16(
                      __builtin_bit_cast(bf16x2, P[8 * gp + 4 * v + e]),
                      __builtin_bit_cast(bf16x2, xw[e]), dot, false);
              }
            }
            const float xsum = xq[((long)m * gs + 2 * j + gp) * 4 + kg];
            acc[nt][m] = fmaf(sc, dot, fmaf(bp, xsum, acc[nt][m]));
          }
        }
      }
    };
    for (int j0 = 0; j0 < nchunks; j0 += D) {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        if (j0 + d < nchunks) {
          compute(j0 + d, d);
          if (j0 + d + D < nchunks) load(j0 + d + D, d);
        }
      }
    }
  }
  // Add the four quarters: (q0+q1) + (q2+q3) on every lane.
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      acc[nt][m] += __shfl_xor(acc[nt][m], 16);
      acc[nt][m] += __shfl_xor(acc[nt][m], 32);
    }

  if (a.S == 1) {
    if (tile0 >= nT || kg != 0) return;
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
      if (tile0 + nt >= nT) continue;
      const int n = (tile0 + nt) * kTileN + r;
#pragma unroll
      for (int m = 0; m < MR; ++m)
        if (m < a.M) store_y<X_F32>(a.y, (long)m * a.ldy + n, acc[nt][m]);
    }
    return;
  }
  if (tile0 < nT && kg == 0) {
    float* part = a.part + (long)s * a.M * a.N;
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
      if (tile0 + nt >= nT) continue;
      const int n = (tile0 + nt) * kTileN + r;
#pragma unroll
      for (int m = 0; m < MR; ++m)
        if (m < a.M) __builtin_nontemporal_store(acc[nt][m], part + (long)m * a.N + n);
    }
  }
  const int n0 = tb * kWaves * NTW * kTileN;
  const int n1 = min(a.N, n0 + kWaves * NTW * kTileN);
  fold_partials<X_F32>(a, tb, n0, n1);
}

// ---------------------------------------------------------------------------
// HBM read probe: every thread streams 16-byte words with a grid stride.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) probe_kernel(const u32x4* __restrict__ buf, long n16,
                                                    uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  const long stride = (long)gridDim.x * blockDim.x;
  long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 v0 = __builtin_nontemporal_load(buf + i);
    const u32x4 v1 = __builtin_nontemporal_load(buf + i + stride);
    const u32x4 v2 = __builtin_nontemporal_load(buf + i + 2 * stride);
    const u32x4 v3 = __builtin_nontemporal_load(buf + i + 3 * stride);
    acc ^= v0[0] ^ v1[1] ^ v2[2] ^ v3[3] ^ v0[3] ^ v1[0] ^ v2[1] ^ v3[2];
  }
  for (; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(buf + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  acc ^= __shfl_xor(acc, 1);
  if (threadIdx.x == 0) sink[blockIdx.x] = acc;
}

// ---------------------------------------------------------------------------
// Launchers.
// ---------------------------------------------------------------------------
static inline unsigned blocks_for(long threads, int per) { return (unsigned)((threads + per - 1) / per); }

hipError_t launch_repack(int bits, bool sb_f32, const uint32_t* w, const void* scales,
                         const void* biases, uint32_t* codes, void* sb, int N, int K,
                         hipStream_t st) {
  const long threads = (long)(N / kTileN) * (K / kChunkK) * 64;
  const unsigned grid = blocks_for(threads, 256);
  if (bits == 3 && !sb_f32)
    repack_kernel<3, uint16_t><<<grid, 256, 0, st>>>(w, (const uint16_t*)scales, (const uint16_t*)biases, codes, (uint16_t*)sb, N, K);
  else if (bits == 3)
    repack_kernel<3, float><<<grid, 256, 0, st>>>(w, (const float*)scales, (const float*)biases, codes, (float*)sb, N, K);
  else if (!sb_f32)
    repack_kernel<4, uint16_t><<<grid, 256, 0, st>>>(w, (const uint16_t*)scales, (const uint16_t*)biases, codes, (uint16_t*)sb, N, K);
  else
    repack_kernel<4, float><<<grid, 256, 0, st>>>(w, (const float*)scales, (const float*)biases, codes, (float*)sb, N, K);
  return hipGetLastError();
}

hipError_t launch_debug_unpack(int bits, const uint32_t* codes, uint8_t* out, int N, int K,
                               hipStream_t st) {
  const long threads = (long)(N / kTileN) * (K / kChunkK) * 64;
  const unsigned grid = blocks_for(threads, 256);
  if (bits == 3)
    debug_unpack_kernel<3><<<grid, 256, 0, st>>>(codes, out, N, K);
  else
    debug_unpack_kernel<4><<<grid, 256, 0, st>>>(codes, out, N, K);
  return hipGetLastError();
}

template <int BITS, typename ST>
static hipError_t mfma_dispatch(int mt, int ntw, int wk, const LaunchArgs& a, hipStream_t st) {
  const unsigned grid = (unsigned)(a.nTB * a.S);
#define QMM_MFMA(MTV, NTV, WKV, DV)                                                  \
  if (mt == MTV && ntw == NTV && wk == WKV) {                                        \
    mfma_kernel<BITS, MTV, NTV, WKV, DV, ST><<<grid, kBlockThreads, 0, st>>>(a);     \
    return hipGetLastError();                                                        \
  }
  QMM_MFMA(1, 1, 1, 4) QMM_MFMA(1, 1, 2, 4) QMM_MFMA(1, 1, 4, 4)
  QMM_MFMA(1, 2, 1, 4) QMM_MFMA(1, 2, 2, 4) QMM_MFMA(1, 2, 4, 4)
  QMM_MFMA(1, 4, 1, 3) QMM_MFMA(1, 4, 2, 3) QMM_MFMA(1, 4, 4, 3)
  QMM_MFMA(2, 1, 1, 3) QMM_MFMA(2, 1, 2, 3) QMM_MFMA(2, 1, 4, 3)
  QMM_MFMA(2, 2, 1, 3) QMM_MFMA(2, 2, 2, 3) QMM_MFMA(2, 2, 4, 3)
  QMM_MFMA(4, 1, 1, 2) QMM_MFMA(4, 1, 2, 2) QMM_MFMA(4, 1, 4, 2)
  QMM_MFMA(4, 2, 1, 2) QMM_MFMA(4, 2, 2, 2) QMM_MFMA(4, 2, 4, 2)
#undef QMM_MFMA
  return hipErrorInvalidValue;
}

hipError_t launch_mfma(int bits, bool sb_f32, int mt, int ntw, int wk, const LaunchArgs& a,
                       hipStream_t st) {
  if (bits == 3) return sb_f32 ? mfma_dispatch<3, float>(mt, ntw, wk, a, st) : mfma_dispatch<3, uint16_t>(mt, ntw, wk, a, st);
  return sb_f32 ? mfma_dispatch<4, float>(mt, ntw, wk, a, st) : mfma_dispatch<4, uint16_t>(mt, ntw, wk, a, st);
}

template <int BITS, bool XF, typename ST>
static hipError_t gemv_dispatch(int mr, int ntw, const LaunchArgs& a, size_t lds,
                                hipStream_t st) {
  const unsigned grid = (unsigned)(a.nTB * a.S);
#define QMM_GEMV(MRV, NTV)                                                          \
  if (mr == MRV && ntw == NTV) {                                                    \
    gemv_kernel<BITS, MRV, NTV, XF, ST><<<grid, kBlockThreads, lds, st>>>(a);      \
    return hipGetLastError();                                                       \
  }
  QMM_GEMV(1, 1) QMM_GEMV(1, 2) QMM_GEMV(1, 4)
  QMM_GEMV(2, 1) QMM_GEMV(2, 2)
  QMM_GEMV(4, 1) QMM_GEMV(4, 2)
  QMM_GEMV(8, 1)
#undef QMM_GEMV
  return hipErrorInvalidValue;
}

hipError_t launch_gemv(int bits, bool x_f32, bool sb_f32, int mr, int ntw, const LaunchArgs& a,
                       size_t lds_bytes, hipStream_t st) {
  if (bits == 3) {
    if (x_f32) return sb_f32 ? gemv_dispatch<3, true, float>(mr, ntw, a, lds_bytes, st) : gemv_dispatch<3, true, uint16_t>(mr, ntw, a, lds_bytes, st);
    return sb_f32 ? gemv_dispatch<3, false, float>(mr, ntw, a, lds_bytes, st) : gemv_dispatch<3, false, uint16_t>(mr, ntw, a, lds_bytes, st);
  }
  if (x_f32) return sb_f32 ? gemv_dispatch<4, true, float>(mr, ntw, a, lds_bytes, st) : gemv_dispatch<4, true, uint16_t>(mr, ntw, a, lds_bytes, st);
  return sb_f32 ? gemv_dispatch<4, false, float>(mr, ntw, a, lds_bytes, st) : gemv_dispatch<4, false, uint16_t>(mr, ntw, a, lds_bytes, st);
}

template <int BITS, typename ST, int MQ>
static hipError_t stream_dispatch_mq(int nw, int cpw, const LaunchArgs& a, size_t lds,
                                     hipStream_t st) {
  const unsigned grid = (unsigned)(a.N / kTileN);
#define QMM_STREAM(NWV, CPWV)                                                                \
  if (nw == NWV && cpw == CPWV) {                                                            \
    auto* kfn = &stream_kernel<BITS, NWV, CPWV, MQ, ST>;                                     \
    if (lds > 64 * 1024) {                                                                   \
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kfn),                 \
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds); \
      if (e != hipSuccess) return e;                                                         \
    }                                                                                        \
    kfn<<<grid, NWV * 64, lds, st>>>(a);                                                     \
    return hipGetLastError();                                                                \
  }
  QMM_STREAM(4, 2) QMM_STREAM(4, 4) QMM_STREAM(8, 4) QMM_STREAM(8, 5) QMM_STREAM(8, 8)
  QMM_STREAM(16, 8)
#undef QMM_STREAM
  return hipErrorInvalidValue;
}

template <int BITS, typename ST>
static hipError_t stream_dispatch(int nw, int cpw, const LaunchArgs& a, size_t lds,
                                  hipStream_t st) {
  if (a.M == 1) return stream_dispatch_mq<BITS, ST, 1>(nw, cpw, a, lds, st);
  if (a.M == 2) return stream_dispatch_mq<BITS, ST, 2>(nw, cpw, a, lds, st);
  return stream_dispatch_mq<BITS, ST, 4>(nw, cpw, a, lds, st);
}

hipError_t launch_stream(int bits, bool sb_f32, int nw, int cpw, const LaunchArgs& a,
                         size_t lds_bytes, hipStream_t st) {
  if (bits == 3) return sb_f32 ? stream_dispatch<3, float>(nw, cpw, a, lds_bytes, st) : stream_dispatch<3, uint16_t>(nw, cpw, a, lds_bytes, st);
  return sb_f32 ? stream_dispatch<4, float>(nw, cpw, a, lds_bytes, st) : stream_dispatch<4, uint16_t>(nw, cpw, a, lds_bytes, st);
}

// (waves, chunks per wave, tile slots) shapes of the resident kernel.  The
// 16-wave shapes cover 65..128 chunks (K up to 16384, a few rows): 10.3 us
// against 10.7 us for the streaming kernel on the 4-bit 15360 -> 3840
// projection at 4 rows (eight waves of 15 chunks: 11.6 us).
#define QMM_RESIDENT_SHAPES(X)                                                               \
  X(4, 2, 1) X(4, 2, 2) X(4, 2, 3) X(4, 2, 4) X(4, 4, 1) X(4, 4, 2) X(4, 4, 3) X(4, 4, 4)     \
  X(8, 4, 1) X(8, 4, 2) X(8, 4, 3) X(8, 4, 4) X(8, 5, 1) X(8, 5, 2) X(8, 5, 3) X(8, 5, 4)     \
  X(8, 8, 1) X(8, 8, 2) X(16, 8, 1) X(16, 8, 2)

bool resident_shape(int nC, int tm, int* nw, int* cpw) {
  // the fewest chunks per wave that cover K: four waves below 16 chunks
  int best_w = 0, best_c = 0;
#define QMM_PICK(W, C, T)                                                                  \
  if (T == tm && (nC < 16) == (W == 4) && W * C >= nC && (best_c == 0 || C < best_c)) { \
    best_w = W;                                                                           \
    best_c = C;                                                                           \
  }
  QMM_RESIDENT_SHAPES(QMM_PICK)
#undef QMM_PICK
  *nw = best_w;
  *cpw = best_c;
  return best_c > 0;
}

size_t resident_lds_bytes(int nw, int tm, int M, int K) {
  return std::max((size_t)M * K * 2, (size_t)tm * nw * 64 * 16);
}

template <int BITS, typename ST>
static hipError_t resident_dispatch(int nw, int cpw, int tm, const LaunchArgs& a, int grid,
                                    size_t lds, hipStream_t st) {
#define QMM_GO(W, C, T)                                                                     \
  if (nw == W && cpw == C && tm == T) {                                                     \
    auto* kfn = &resident_kernel<BITS, W, C, T, ST>;                                        \
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kfn),                  \
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds); \
    if (e != hipSuccess) return e;                                                          \
    kfn<<<grid, W * 64, lds, st>>>(a);                                                      \
    return hipGetLastError();                                                               \
  }
  QMM_RESIDENT_SHAPES(QMM_GO)
#undef QMM_GO
  return hipErrorInvalidValue;
}

hipError_t launch_resident(int bits, bool sb_f32, int nw, int cpw, int tm, const LaunchArgs& a,
                           int grid, size_t lds_bytes, hipStream_t st) {
  if (bits == 3)
    return sb_f32 ? resident_dispatch<3, float>(nw, cpw, tm, a, grid, lds_bytes, st)
                  : resident_dispatch<3, uint16_t>(nw, cpw, tm, a, grid, lds_bytes, st);
  return sb_f32 ? resident_dispatch<4, float>(nw, cpw, tm, a, grid, lds_bytes, st)
                : resident_dispatch<4, uint16_t>(nw, cpw, tm, a, grid, lds_bytes, st);
}

// (waves, chunks per wave, tile pairs) shapes of the fused gate/up kernel.
#define QMM_GATE_UP_SHAPES(X) X(4, 2, 1) X(4, 2, 2) X(4, 4, 1) X(4, 4, 2) X(8, 4, 1) X(8, 4, 2) \
  X(8, 5, 1) X(8, 5, 2) X(8, 8, 1)

bool gate_up_shape(int nC, int pairs, int* nw, int* cpw) {
  int best_w = 0, best_c = 0;
#define QMM_PICK(W, C, P)                                                                  \
  if (P == pairs && (nC < 16) == (W == 4) && W * C >= nC && (best_c == 0 || C < best_c)) { \
    best_w = W;                                                                           \
    best_c = C;                                                                           \
  }
  QMM_GATE_UP_SHAPES(QMM_PICK)
#undef QMM_PICK
  *nw = best_w;
  *cpw = best_c;
  return best_c > 0;
}

template <int BITS, typename ST>
static hipError_t gate_up_dispatch(int nw, int cpw, int pairs, const LaunchArgs& a, int grid,
                                   size_t lds, hipStream_t st) {
#define QMM_GO(W, C, P)                                                                     \
  if (nw == W && cpw == C && pairs == P) {                                                  \
    auto* kfn = &resident_kernel<BITS, W, C, 2 * P, ST, true>;                              \
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kfn),                  \
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds); \
    if (e != hipSuccess) return e;                                                          \
    kfn<<<grid, W * 64, lds, st>>>(a);                                                      \
    return hipGetLastError();                                                               \
  }
  QMM_GATE_UP_SHAPES(QMM_GO)
#undef QMM_GO
  return hipErrorInvalidValue;
}

hipError_t launch_gate_up(int bits, bool sb_f32, int nw, int cpw, int pairs, const LaunchArgs& a,
                          int grid, size_t lds_bytes, hipStream_t st) {
  if (bits == 3)
    return sb_f32 ? gate_up_dispatch<3, float>(nw, cpw, pairs, a, grid, lds_bytes, st)
                  : gate_up_dispatch<3, uint16_t>(nw, cpw, pairs, a, grid, lds_bytes, st);
  return sb_f32 ? gate_up_dispatch<4, float>(nw, cpw, pairs, a, grid, lds_bytes, st)
                : gate_up_dispatch<4, uint16_t>(nw, cpw, pairs, a, grid, lds_bytes, st);
}

// (row tiles, slices of 512 k) shapes of the slab kernel; three tile slots.
#define QMM_SLAB_SHAPES(X) X(1, 10) X(1, 16) X(2, 10) X(2, 16) X(4, 10) X(4, 16)

int slab_slices(int mt, int nC) {
  const int ns = (nC + 3) / 4;
#define QMM_HAS(MTV, NSV) if (mt == MTV && ns == NSV) return ns;
  QMM_SLAB_SHAPES(QMM_HAS)
#undef QMM_HAS
  return 0;
}

// LDS ring slots and weight ring depth (slices of loads in flight per
// compute wave), measured on the 3-bit 5120x10240 workload: deeper weight
// rings queue the activation slices behind weight loads and run slower.
// LDS ring slots per row-tile count (128 KB at one, two and four row tiles,
// 144 KB at three; three row tiles run in the split form only)
static constexpr int slab_ring(int mt) { return mt == 4 ? 2 : (mt == 3 ? 3 : 4); }
static constexpr int slab_depth(int mt) { return mt == 2 ? 2 : 3; }
size_t slab_lds_bytes(int mt) { return (size_t)slab_ring(mt) * 16 * mt * 1024; }

template <int BITS, typename ST>
static hipError_t slab_dispatch(int mt, int ns, const LaunchArgs& a, int grid, size_t lds,
                                hipStream_t st) {
#define QMM_SLAB(MTV, NSV)                                                                    \
  if (mt == MTV && ns == NSV) {                                                               \
    auto* kfn = &slab_kernel<BITS, MTV, kSlabTiles, NSV, slab_ring(MTV), slab_depth(MTV), ST>; \
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kfn),                    \
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds); \
    if (e != hipSuccess) return e;                                                            \
    kfn<<<grid, (kSlabTiles * 4 + 4) * 64, lds, st>>>(a);                                     \
    return hipGetLastError();                                                                 \
  }
  QMM_SLAB_SHAPES(QMM_SLAB)
#undef QMM_SLAB
  return hipErrorInvalidValue;
}

hipError_t launch_slab(int bits, bool sb_f32, int mt, int ns, const LaunchArgs& a, int grid,
                       size_t lds_bytes, hipStream_t st) {
  if (bits == 3)
    return sb_f32 ? slab_dispatch<3, float>(mt, ns, a, grid, lds_bytes, st)
                  : slab_dispatch<3, uint16_t>(mt, ns, a, grid, lds_bytes, st);
  return sb_f32 ? slab_dispatch<4, float>(mt, ns, a, grid, lds_bytes, st)
                : slab_dispatch<4, uint16_t>(mt, ns, a, grid, lds_bytes, st);
}

// (row tiles, slices per workgroup) and (tiles per wave, tile slots) shapes
// of the split slab kernel that are built: two K parts of K = 5120 or 8192
// (5 or 8 slices each), two W tiles per wave in three slots (three tiles per
// wave in two slots spills registers at four row tiles and measured no
// faster; one K part leaves half the compute units idle).
#define QMM_SPLIT_SLAB_SHAPES(X) X(2, 5) X(3, 5) X(4, 5) X(2, 8) X(3, 8) X(4, 8)
#define QMM_SPLIT_SLAB_WAVES(X) X(2, 3)

bool split_slab_shape(int mt, int tw, int nC, int S, int* ns, int* nslot) {
  if (S != 2 || nC % (4 * S) != 0) return false;
  const int want = nC / (4 * S);
  bool shape = false, waves = false;
#define QMM_HAS(MTV, NSV) if (mt == MTV && want == NSV) shape = true;
  QMM_SPLIT_SLAB_SHAPES(QMM_HAS)
#undef QMM_HAS
#define QMM_HASW(TWV, NSL) if (tw == TWV) { waves = true; *nslot = NSL; }
  QMM_SPLIT_SLAB_WAVES(QMM_HASW)
#undef QMM_HASW
  *ns = want;
  return shape && waves;
}

// weight ring depth: two slices ahead where the registers allow it
static constexpr int split_slab_depth(int mt) { return mt == 2 ? 2 : 1; }
size_t split_slab_lds_bytes(int mt) { return (size_t)slab_ring(mt) * 16 * mt * 1024; }

size_t split_slab_part_bytes(int mt, int tw, int nslot, int groups, int S) {
  return S > 1 ? (size_t)groups * S * tw * nslot * mt * 1024 : 0;
}

template <int BITS, typename ST>
static hipError_t split_slab_dispatch(int mt, int ns, int tw, const LaunchArgs& a, int grid,
                                      size_t lds, hipStream_t st) {
#define QMM_SSLAB_W(MTV, NSV, TWV, NSL)                                                      \
  if (mt == MTV && ns == NSV && tw == TWV) {                                                \
    auto* kfn = &split_slab_kernel<BITS, MTV, TWV, NSL, NSV, slab_ring(MTV),               \
                                   split_slab_depth(MTV), ST>;                             \
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kfn),                  \
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds); \
    if (e != hipSuccess) return e;                                                          \
    kfn<<<grid, (NSL * 4 + 4) * 64, lds, st>>>(a);                                          \
    return hipGetLastError();                                                               \
  }
#define QMM_SSLAB(MTV, NSV) QMM_SSLAB_W(MTV, NSV, 2, 3)
  QMM_SPLIT_SLAB_SHAPES(QMM_SSLAB)
#undef QMM_SSLAB
#undef QMM_SSLAB_W
  return hipErrorInvalidValue;
}

hipError_t launch_split_slab(int bits, bool sb_f32, int mt, int ns, int tw, const LaunchArgs& a,
                             int grid, size_t lds_bytes, hipStream_t st) {
  if (bits == 3)
    return sb_f32 ? split_slab_dispatch<3, float>(mt, ns, tw, a, grid, lds_bytes, st)
                  : split_slab_dispatch<3, uint16_t>(mt, ns, tw, a, grid, lds_bytes, st);
  return sb_f32 ? split_slab_dispatch<4, float>(mt, ns, tw, a, grid, lds_bytes, st)
                : split_slab_dispatch<4, uint16_t>(mt, ns, tw, a, grid, lds_bytes, st);
}

size_t wide_lds_bytes(int mt) { return (size_t)2 * 16 * mt * 32 * 16; }

bool wide_fits(int nC) { return nC >= 2 && nC % 2 == 0; }

template <int BITS, int MT, typename ST>
static hipError_t wide_launch(const LaunchArgs& a, int grid, size_t lds, hipStream_t st) {
  auto* kfn = &wide_kernel<BITS, MT, ST>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kfn),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  kfn<<<grid, 12 * 64, lds, st>>>(a);
  return hipGetLastError();
}

// row tiles per launch: 6 (up to 96 rows) or 8
template <int BITS, typename ST>
static hipError_t wide_dispatch(int mt, const LaunchArgs& a, int grid, size_t lds,
                                hipStream_t st) {
  if (mt == 6) return wide_launch<BITS, 6, ST>(a, grid, lds, st);
  if (mt == 8) return wide_launch<BITS, 8, ST>(a, grid, lds, st);
  return hipErrorInvalidValue;
}

hipError_t launch_wide(int bits, bool sb_f32, int mt, const LaunchArgs& a, int grid,
                       size_t lds_bytes, hipStream_t st) {
  if (bits == 3)
    return sb_f32 ? wide_dispatch<3, float>(mt, a, grid, lds_bytes, st)
                  : wide_dispatch<3, uint16_t>(mt, a, grid, lds_bytes, st);
  return sb_f32 ? wide_dispatch<4, float>(mt, a, grid, lds_bytes, st)
                : wide_dispatch<4, uint16_t>(mt, a, grid, lds_bytes, st);
}

hipError_t launch_probe(const void* buf, size_t bytes, uint32_t* sink, int grid, hipStream_t st) {
  probe_kernel<<<grid, 256, 0, st>>>(reinterpret_cast<const u32x4*>(buf), (long)(bytes / 16), sink);
  return hipGetLastError();
}

}  // namespace qmm
