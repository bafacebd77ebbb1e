// qmm_attention.hip -- decode attention over an affine-quantized KV cache
// ("mlx-bun 0.0.4" page, fused-decode-kernel.ts: flash-decoding split over
// the cached rows, the dequant factored out of the dot products, and a
// deterministic merge of the per-block partials).
//
// One query row per head; head h reads KV head h / REP (REP = H / KV).  Keys
// and values are stored like the projection weights: codes packed along D
// into uint32 words (least significant bits first), one bf16 scale and bias
// per group of GS values of a row.  For every head:
//   score[n] = bf16(sum_d q[d] * (s_k * code_k[n, d] + b_k))
//   out      = bf16(sum_n e^(score[n] - M) v[n] / sum_n e^(score[n] - M))
// with M the largest score, v = s_v * code_v + b_v, all sums in f32.
//
// gfx950 design:
//   * kernel 1, one 512-thread workgroup per (block of 256 cached rows, KV
//     head) serving all REP query heads of that KV head, so every key and
//     value byte is read once per head group; 256 workgroups at 8 KV heads
//     and 8192 rows (measured against 256 threads and 128 rows: 11.8 against
//     12.0 us for the block kernel, and half as many blocks to merge);
//   * 16 lanes per cached row (a wave covers 4 rows at once, the 16 lanes
//     reading one row's words as one contiguous run); lane j owns values
//     j*D/16 .. (j+1)*D/16 - 1 of a row for the score and of the output;
//   * scores in the page's factored form s * sum_d c_d q_d + b * sum_d q_d
//     with exact products: each code becomes its exact bf16 value (4-bit:
//     the word's two nibble planes read as e4m3 bytes and converted two at a
//     time with a scale of 2^9; 8-bit: one v_cvt_f32_ubyteN per byte, then
//     two codes per v_cvt_pk_bf16_f32; every code below 256 is exact in
//     bf16), pairs of codes meet the matching pairs of query values in
//     v_dot2_f32_bf16 (8-bit by 8-bit significands: exact products), each
//     lane applies its group's scale and
//     bias, the 16 lanes add their parts with DPP row operations, and the
//     score is rounded to bf16;
//   * two passes over the wave's rows held in registers: the scores first
//     (the wave's maximum M_w by cross-lane swaps, no barrier, so a wave
//     whose rows have landed goes on at once), then the weights e^(s - M_w)
//     and the values, accumulated per lane as sum p s_v c (one FMA per
//     value) plus one sum p b_v per row slice -- no rescaling of running
//     sums;
//   * the 16 lane groups' partial outputs are added through LDS in a fixed
//     order, each scaled by its wave's e^(M_w - M) (M the block maximum);
//     the block writes its unnormalized output and (M, sum e^(s - M)) to the
//     workspace, or, when one block covers the cache, the result;
//   * kernel 2 merges the blocks of each head (64 values per workgroup) in a
//     fixed order (deterministic).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qmm_internal.h"

namespace qmm {

namespace {

constexpr int kAttnThreads = 512;
constexpr int kAttnLanesPerRow = 16;
constexpr int kAttnGroups = kAttnThreads / kAttnLanesPerRow;  // lane groups per workgroup
constexpr int kAttnRowsPerGroup = kAttnBlock / kAttnGroups;    // rows per lane group

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u) return (u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;  // round to nearest, ties to even
}
// Round to bf16 (nearest, ties to even) and back, for finite values and
// infinities (a score is never NaN for finite inputs).
__device__ __forceinline__ float round_bf16(float v) {
  const uint32_t u = __float_as_uint(v);
  return __uint_as_float((u + 0x7FFFu + ((u >> 16) & 1u)) & 0xFFFF0000u);
}

typedef short bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Sum over the 16 lanes of a DPP row (every lane receives the sum).
__device__ __forceinline__ float row_sum16(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x141, 0xF, 0xF, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x140, 0xF, 0xF, true));
  return v;
}

// `WPL` consecutive words of a lane, as 4-, 8- or 16-byte loads.
template <int WPL>
__device__ __forceinline__ void load_words(const uint32_t* __restrict__ p, uint32_t* w) {
  if constexpr (WPL == 1) {
    w[0] = p[0];
  } else if constexpr (WPL == 2) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    w[0] = v.x;
    w[1] = v.y;
  } else {
#pragma unroll
    for (int i = 0; i < WPL / 4; ++i) {
      const uint4 v = reinterpret_cast<const uint4*>(p)[i];
      w[4 * i] = v.x;
      w[4 * i + 1] = v.y;
      w[4 * i + 2] = v.z;
      w[4 * i + 3] = v.w;
    }
  }
}

// The nibble mask moved into an SGPR by an instruction the compiler cannot
// see through, so that it is materialized once rather than as a literal in
// every and.
__device__ __forceinline__ uint32_t sgpr_const(uint32_t v) {
  uint32_t r;
  asm volatile("s_mov_b32 %0, %1" : "=s"(r) : "i"(v));
  return r;
}

// The lane's 8-bit codes as floats, in value order: one v_cvt_f32_ubyteN
// per byte of a word.
template <int WPL>
__device__ __forceinline__ void code_floats8(const uint32_t* w, float* c) {
#pragma unroll
  for (int j = 0; j < WPL; ++j)
#pragma unroll
    for (int t = 0; t < 4; ++t) c[4 * j + t] = (float)((w[j] >> (8 * t)) & 0xFFu);
}

// 4-bit codes: each nibble plane of a word (w & 0x0F0F0F0F, (w >> 4) &
// 0x0F0F0F0F) holds one code per byte, and a byte c below 16 read as an OCP
// e4m3 value is exactly c * 2^-9 (a subnormal below 8, exponent field 1
// from 8), so one scaled conversion by 2^9 turns two of them into two exact
// bf16 or f32 values.  Plane byte t of word j is value 8j + 2t (low plane)
// or 8j + 2t + 1 (high plane); half h of a plane holds bytes 2h and 2h+1.
//   pair 4j + 2*plane + h = values (8j + 4h + plane, 8j + 4h + plane + 2)
template <int WPL>
__device__ __forceinline__ void code_pairs4(const uint32_t* w, uint32_t* P, uint32_t nib) {
#pragma unroll
  for (int j = 0; j < WPL; ++j) {
    const uint32_t pl[2] = {w[j] & nib, (w[j] >> 4) & nib};
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      P[4 * j + 2 * k] = __builtin_bit_cast(
          uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(pl[k], 512.0f, false));
      P[4 * j + 2 * k + 1] = __builtin_bit_cast(
          uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(pl[k], 512.0f, true));
    }
  }
}
template <int WPL>
__device__ __forceinline__ void code_floats4(const uint32_t* w, float* c, uint32_t nib) {
#pragma unroll
  for (int j = 0; j < WPL; ++j) {
    const uint32_t pl[2] = {w[j] & nib, (w[j] >> 4) & nib};
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const f32x2_t v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(pl[k], 512.0f, false);
      const f32x2_t v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(pl[k], 512.0f, true);
      c[8 * j + k] = v0[0];
      c[8 * j + k + 2] = v0[1];
      c[8 * j + k + 4] = v1[0];
      c[8 * j + k + 6] = v1[1];
    }
  }
}
// The value index of the first member of bf16 pair p (the second is 1 or 2
// later): 4-bit pairs follow code_pairs4, 8-bit pairs are consecutive.
template <int BITS>
__device__ __forceinline__ constexpr int pair_first(int p) {
  return BITS == 4 ? 8 * (p / 4) + 4 * (p % 2) + (p / 2) % 2 : 2 * p;
}
template <int BITS>
__device__ __forceinline__ constexpr int pair_step() {
  return BITS == 4 ? 2 : 1;
}

// Two exact bf16 values in one word (low half first): integers below 256
// convert exactly.
typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const bf16x2_v v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

template <int BITS, int D, int REP>
__global__ void __launch_bounds__(kAttnThreads) attn_block_kernel(AttnArgs a) {
  constexpr int EPL = D / kAttnLanesPerRow;  // values per lane
  constexpr int WPL = EPL * BITS / 32;       // words per lane
  constexpr int NP = EPL / 2;                // bf16 pairs per lane
  constexpr int R = kAttnRowsPerGroup;
  extern __shared__ float lds[];             // [kAttnGroups][REP][D] partial outputs
  __shared__ float red_max[kAttnThreads / 64][REP];
  const int blk = blockIdx.x, kv = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane & 15;
  const int lg = wave * 4 + (lane >> 4);
  const int N = a.N;
  const int n0 = blk * kAttnBlock;
  const int d0 = sub * EPL;
  const int gpr = D / a.GS;  // groups per row
  const int grp = d0 / a.GS;
  const uint16_t* __restrict__ qg = reinterpret_cast<const uint16_t*>(a.q);
  const uint16_t* __restrict__ ksg = reinterpret_cast<const uint16_t*>(a.ks);
  const uint16_t* __restrict__ kbg = reinterpret_cast<const uint16_t*>(a.kb);
  const uint16_t* __restrict__ vsg = reinterpret_cast<const uint16_t*>(a.vs);
  const uint16_t* __restrict__ vbg = reinterpret_cast<const uint16_t*>(a.vb);

  // query slices of the REP heads: value-order bf16 pairs for the scores,
  // and their sums (the bias term)
  uint32_t Q[REP][NP];
  float qsum[REP];
#pragma unroll
  for (int r = 0; r < REP; ++r) {
    const int h = kv * REP + r;
    uint32_t qb[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) qb[e] = qg[(long)h * D + d0 + e];
#pragma unroll
    for (int p = 0; p < NP; ++p)
      Q[r][p] = qb[pair_first<BITS>(p)] | (qb[pair_first<BITS>(p) + pair_step<BITS>()] << 16);
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) s += bf16_bits_to_f32(qb[e]);
    qsum[r] = s;
  }

  // this lane group's rows: n0 + lg + 16 i (32-bit offsets from the KV
  // head's uniform base; rows past the cache re-read the last row)
  constexpr int RW = D * BITS / 32;  // words per cached row
  const long head = (long)kv * N;
  const uint32_t* __restrict__ kwh = a.kw + head * RW;
  const uint32_t* __restrict__ vwh = a.vw + head * RW;
  const uint16_t* __restrict__ ksh = ksg + head * gpr;
  const uint16_t* __restrict__ kbh = kbg + head * gpr;
  const uint16_t* __restrict__ vsh = vsg + head * gpr;
  const uint16_t* __restrict__ vbh = vbg + head * gpr;
  uint32_t KW[R][WPL], VW[R][WPL];
  float ks[R], kb[R], vs[R], vb[R];
  bool valid[R];
  uint32_t wofs[R], sofs[R];  // unsigned: SGPR base + 32-bit VGPR offset addressing
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int n = n0 + lg + kAttnGroups * i;
    valid[i] = n < N;
    const uint32_t row = (uint32_t)min(n, N - 1);
    wofs[i] = row * RW + (uint32_t)(sub * WPL);
    sofs[i] = row * (uint32_t)gpr + (uint32_t)grp;
    load_words<WPL>(kwh + wofs[i], KW[i]);
    ks[i] = bf16_bits_to_f32(ksh[sofs[i]]);
    kb[i] = bf16_bits_to_f32(kbh[sofs[i]]);
  }
#pragma unroll
  for (int i = 0; i < R; ++i) {
    load_words<WPL>(vwh + wofs[i], VW[i]);
    vs[i] = bf16_bits_to_f32(vsh[sofs[i]]);
    vb[i] = bf16_bits_to_f32(vbh[sofs[i]]);
  }

  const uint32_t nib_mask = sgpr_const(0x0F0F0F0Fu);

  // pass 1: scores (bf16-rounded) and the wave's maximum
  float sc[REP][R];
  float mx[REP];
#pragma unroll
  for (int r = 0; r < REP; ++r) mx[r] = -INFINITY;
#pragma unroll
  for (int i = 0; i < R; ++i) {
    uint32_t P[NP];
    if constexpr (BITS == 4) {
      code_pairs4<WPL>(KW[i], P, nib_mask);
    } else {
      float c[EPL];
      code_floats8<WPL>(KW[i], c);
#pragma unroll
      for (int p = 0; p < NP; ++p) P[p] = pack_bf16(c[2 * p], c[2 * p + 1]);
    }
#pragma unroll
    for (int r = 0; r < REP; ++r) {
      float dsum = 0.f;
#pragma unroll
      for (int p = 0; p < NP; ++p) dsum = dot2(P[p], Q[r][p], dsum);
      const float part = fmaf(ks[i], dsum, kb[i] * qsum[r]);
      const float s = round_bf16(row_sum16(part));
      sc[r][i] = valid[i] ? s : -INFINITY;
      mx[r] = fmaxf(mx[r], sc[r][i]);
    }
  }
  // over the 4 lane groups of the wave: each wave goes on to its values
  // without waiting for the others (their partials are rescaled to the
  // block maximum when they are added); a wave whose rows all lie past the
  // cache has weight 0 everywhere
  float Mw[REP];
#pragma unroll
  for (int r = 0; r < REP; ++r) {
    float m = mx[r];
    m = fmaxf(m, __shfl_xor(m, 16));
    m = fmaxf(m, __shfl_xor(m, 32));
    if (lane == 0) red_max[wave][r] = m;
    Mw[r] = m == -INFINITY ? 0.f : m;
  }

  // pass 2: weights and values
  float o[REP][EPL], lsum[REP], pb[REP];
#pragma unroll
  for (int r = 0; r < REP; ++r) {
    lsum[r] = 0.f;
    pb[r] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[r][e] = 0.f;
  }
#pragma unroll
  for (int i = 0; i < R; ++i) {
    float c[EPL];
    if constexpr (BITS == 4)
      code_floats4<WPL>(VW[i], c, nib_mask);
    else
      code_floats8<WPL>(VW[i], c);
#pragma unroll
    for (int r = 0; r < REP; ++r) {
      const float p = __expf(sc[r][i] - Mw[r]);  // 0 for rows past the cache
      lsum[r] += p;
      pb[r] = fmaf(p, vb[i], pb[r]);
      const float ps = p * vs[i];
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[r][e] = fmaf(ps, c[e], o[r][e]);
    }
  }

  // add the lane groups' partials in lane-group order
#pragma unroll
  for (int r = 0; r < REP; ++r)
#pragma unroll
    for (int e = 0; e < EPL; ++e) lds[(lg * REP + r) * D + d0 + e] = o[r][e] + pb[r];
  __shared__ float red_sum[kAttnGroups][REP];
  if (sub == 0)
#pragma unroll
    for (int r = 0; r < REP; ++r) red_sum[lg][r] = lsum[r];
  // the block maximum, and each wave's factor e^(M_w - M) (0 for a wave
  // without rows in the cache)
  __shared__ float cw[REP][kAttnThreads / 64];
  __syncthreads();
  float M[REP];
#pragma unroll
  for (int r = 0; r < REP; ++r) {
    M[r] = red_max[0][r];
#pragma unroll
    for (int w = 1; w < kAttnThreads / 64; ++w) M[r] = fmaxf(M[r], red_max[w][r]);
  }
  if (threadIdx.x < REP * (kAttnThreads / 64)) {
    const int r = threadIdx.x / (kAttnThreads / 64), w = threadIdx.x % (kAttnThreads / 64);
    const float m = red_max[w][r];
    float mb = red_max[0][r];
    for (int u = 1; u < kAttnThreads / 64; ++u) mb = fmaxf(mb, red_max[u][r]);
    cw[r][w] = m == -INFINITY ? 0.f : __expf(m - mb);
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < REP * D; idx += kAttnThreads) {
    const int r = idx / D, d = idx - r * D;
    float v = 0.f, l = 0.f;
#pragma unroll
    for (int j = 0; j < kAttnGroups; ++j) {
      const float c = cw[r][j / 4];  // lane group j belongs to wave j / 4
      v = fmaf(lds[(j * REP + r) * D + d], c, v);
      l = fmaf(red_sum[j][r], c, l);
    }
    const int h = kv * REP + r;
    if (a.G == 1) {
      reinterpret_cast<uint16_t*>(a.out)[(long)h * D + d] = (uint16_t)f32_to_bf16_bits(v / l);
    } else {
      a.opart[((long)h * a.G + blk) * D + d] = v;
      if (d == 0) {
        a.stats[((long)h * a.G + blk) * 2] = M[r];
        a.stats[((long)h * a.G + blk) * 2 + 1] = l;
      }
    }
  }
}

// Merge of the blocks of one head: workgroup (h, y) of 256 threads takes the
// 64 values y*64 .. y*64 + 63 of head h; thread (c, j) adds the partials of
// value j over the c-th of 4 contiguous runs of blocks, issuing its first 16
// loads before anything else so that they overlap the weights' computation.
// M = max_g M_g; block weights w_g = e^(M_g - M) into LDS; the normaliser
// sum_g l_g w_g by a fixed-shape reduction; the 4 run sums are added in run
// order.  Every order is fixed by G alone: bitwise reproducible.
constexpr int kMergeThreads = 256, kMergeValues = 64, kMergeRuns = kMergeThreads / kMergeValues;
__global__ void __launch_bounds__(kMergeThreads) attn_merge_kernel(AttnArgs a, int D) {
  extern __shared__ float wts[];  // [G]
  __shared__ float red[kMergeThreads / 64];
  __shared__ float runs[kMergeRuns][kMergeValues];
  const int h = blockIdx.x, t = threadIdx.x;
  const int G = a.G;
  const int j = t & (kMergeValues - 1), c = t / kMergeValues;
  const int d = blockIdx.y * kMergeValues + j;
  const int per = (G + kMergeRuns - 1) / kMergeRuns;
  const int g0 = min(G, c * per), g1 = min(G, g0 + per);
  const float* op = a.opart + (long)h * G * D + d;
  // 0. the first 16 partials of this thread's run (clamped, never stored past)
  float v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = op[(long)min(g0 + i, G - 1) * D];
  // 1. the largest block maximum
  const float* st = a.stats + (long)h * G * 2;
  float m = -INFINITY;
  for (int g = t; g < G; g += kMergeThreads) m = fmaxf(m, st[2 * g]);
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if ((t & 63) == 0) red[t >> 6] = m;
  __syncthreads();
  float M = red[0];
  for (int w = 1; w < kMergeThreads / 64; ++w) M = fmaxf(M, red[w]);
  __syncthreads();
  // 2. block weights, and this thread's share of the normaliser (blocks
  //    t, t + 256, ... in order); shares added by a fixed tree per wave,
  //    then the waves in order
  float den = 0.f;
  for (int g = t; g < G; g += kMergeThreads) {
    const float w = __expf(st[2 * g] - M);
    wts[g] = w;
    den = fmaf(st[2 * g + 1], w, den);
  }
  for (int off = 1; off < 64; off <<= 1) {
    const float o = __shfl_down(den, off);
    if ((t & (2 * off - 1)) == 0) den += o;
  }
  __syncthreads();  // the weights are in LDS, red is free
  if ((t & 63) == 0) red[t >> 6] = den;
  __syncthreads();
  float denom = red[0];
  for (int w = 1; w < kMergeThreads / 64; ++w) denom += red[w];
  // 3. this thread's run, in block order
  float o = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) o = fmaf(g0 + i < g1 ? v[i] : 0.f, wts[min(g0 + i, G - 1)], o);
  for (int g = g0 + 16; g < g1; g += 16) {
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = op[(long)min(g + i, G - 1) * D];
#pragma unroll
    for (int i = 0; i < 16; ++i) o = fmaf(g + i < g1 ? v[i] : 0.f, wts[min(g + i, G - 1)], o);
  }
  runs[c][j] = o;
  __syncthreads();
  if (c == 0) {
    float tot = runs[0][j];
    for (int k = 1; k < kMergeRuns; ++k) tot += runs[k][j];
    reinterpret_cast<uint16_t*>(a.out)[(long)h * D + d] = (uint16_t)f32_to_bf16_bits(tot / denom);
  }
}

template <int BITS, int D, int REP>
hipError_t attn_launch(const AttnArgs& a, hipStream_t st) {
  const size_t lds = (size_t)kAttnGroups * REP * D * sizeof(float);
  auto* kfn = &attn_block_kernel<BITS, D, REP>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kfn),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  kfn<<<dim3(a.G, a.KV), kAttnThreads, lds, st>>>(a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (a.G > 1) {
    attn_merge_kernel<<<dim3(a.H, D / kMergeValues), kMergeThreads, (size_t)a.G * sizeof(float),
                        st>>>(a, D);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace

// (D, REP) pairs that are built: REP * D <= 1024 keeps a lane's query pairs
// and partial outputs within its registers.
#define QMM_ATTN_SHAPES(X) \
  X(128, 1) X(256, 1) X(512, 1) X(128, 2) X(256, 2) X(512, 2) X(128, 4) X(256, 4) X(128, 8)

bool attention_supported(int D, int rep) {
#define QMM_HAS(DV, RV) if (D == DV && rep == RV) return true;
  QMM_ATTN_SHAPES(QMM_HAS)
#undef QMM_HAS
  return false;
}

hipError_t launch_attention(int bits, int D, int rep, const AttnArgs& a, hipStream_t st) {
#define QMM_ATTN(DV, RV)                                                        \
  if (D == DV && rep == RV)                                                     \
    return bits == 4 ? attn_launch<4, DV, RV>(a, st) : attn_launch<8, DV, RV>(a, st);
  QMM_ATTN_SHAPES(QMM_ATTN)
#undef QMM_ATTN
  return hipErrorInvalidValue;
}

}  // namespace qmm
