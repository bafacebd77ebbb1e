// qmm_fmt.hip -- the other MLX affine formats on the matrix cores: 2- and
// 8-bit weights with groups of 32, 64 or 128 values, and 3- and 4-bit weights
// with groups of 32.  (3- and 4-bit weights with groups of 64 or 128 use the
// native layout of qmm_layout.hip.)
//
// [P1] = page "@mlx-bun/inference 0.0.0-stage -> 1.0.0": affine-split-mma.ts
// (MLX affine weights, w = s * q + b per group); affine3-rows.ts header (the
// factored sum_g s * sum(q x) + b * sum(x), each weight decoded once for
// every activation row).  [P3] = page "mlx-bun 0.0.4", fused-decode-kernel.ts:
// widths 4 and 8 and group sizes 32, 64 and 128 of affine-quantized tensors.
//
// Step layout (written once by repack_fmt_kernel; byte count unchanged).
// Tiles of 16 rows of W and chunks of 128 columns as in the native layout;
// block (tile t, chunk c) has index t*nC + c and holds 64 lanes x BITS words.
// Lane l = (r = l & 15, kb = l >> 4) holds the 32 codes e = 8s + i of row
// 16t + r at columns
//     k = 128c + 32s + 8kb + i,   s = 0..3 (step), i = 0..7,
// which is exactly the lane's B operand of the 16x16x32 product of step s.
// A group of 32, 64 or 128 columns is 1, 2 or 4 whole steps, so every
// product covers one group only.  Code e is half h = e & 1 of pair p = e >> 1:
//   4-bit: pair p in word p >> 2, field u = p & 3: bits 4u (h = 0), 16+4u;
//   2-bit: pair p in word p >> 3, field u = p & 7: bits 2u (h = 0), 16+2u;
//   3-bit: the two low bits of the codes as the 2-bit layout in words 0 and
//          1, bit 2 of pair p's codes in word 2 at bits p (h = 0) and 16+p;
//   8-bit: code e in byte e & 3 of word e >> 2; the lane's words 0..3 and
//          4..7 are two 16-byte vectors, each contiguous over the 64 lanes.
// The lane's words are contiguous (8-bit: per vector), so a wave reads 512,
// 768, 1024 or 2 x 1024 contiguous bytes per block.
// B operands.  For 2, 3 and 4 bits one and-or per pair makes bf16 values
// 128 + q (0x4300 | q: 128 + q is exact in bf16's 7 mantissa bits) and the
// offset is removed with the group's sum of x:
//     sum_k (s q_k + b) x_k = s * sum_k (128 + q_k) x_k + (b - 128 s) * sum_k x_k.
// 8-bit codes go through byte-to-float conversions and a packed bf16
// conversion (exact: integers up to 256 are bf16 values), offset 0.
// Scales and biases (bf16): block b holds 16 rows x (Gc scales, then Gc
// biases), Gc = 128 / group_size.
//
// The kernel (fmt_kernel) has the resident kernel's shape: up to 16
// activation rows staged in LDS by LDS-direct loads, TM tiles per workgroup
// shared by its NW waves, wave w taking chunks w, w + NW, ... of all TM tiles
// with every weight load issued up front, and the waves' partial tiles added
// through LDS in wave order (bitwise reproducible).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "qmm_device.h"

namespace qmm {

namespace {

typedef uint32_t u32x2 __attribute__((__vector_size__(8)));

// Mask constants of the pair extraction: the or-value 0x43004300 in a VGPR,
// the field masks in SGPRs (an and-or takes no literal on this chip).
struct FmtMasks {
  uint32_t orv, m2, m4, b2;  // 0x43004300, 0x00030003, 0x000F000F, 0x00040004
};
template <int BITS>
__device__ __forceinline__ FmtMasks fmt_masks() {
  FmtMasks k{};
  asm volatile("v_mov_b32 %0, %1" : "=v"(k.orv) : "s"(0x43004300u));
  if constexpr (BITS == 4) k.m4 = opaque_sgpr(0x000F000Fu);
  if constexpr (BITS == 2 || BITS == 3) k.m2 = opaque_sgpr(0x00030003u);
  if constexpr (BITS == 3) k.b2 = opaque_sgpr(0x00040004u);
  return k;
}

typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const bf16x2_v v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Value offset of the B operands: 128 for the and-or forms, 0 for 8 bits.
template <int BITS>
constexpr float kFmtOffset = BITS == 8 ? 0.f : 128.f;

// Pair p of a lane's codes (codes 2p, 2p+1) as two bf16 values.
template <int BITS>
__device__ __forceinline__ uint32_t fmt_pair(const uint32_t* w, int p, const FmtMasks& k) {
  if constexpr (BITS == 4) {
    return and_or(w[p >> 2] >> (4 * (p & 3)), k.m4, k.orv);
  } else if constexpr (BITS == 2) {
    return and_or(w[p >> 3] >> (2 * (p & 7)), k.m2, k.orv);
  } else if constexpr (BITS == 3) {
    const uint32_t lo = and_or(w[p >> 3] >> (2 * (p & 7)), k.m2, k.orv);
    const uint32_t hi = p >= 2 ? w[2] >> (p - 2) : w[2] << (2 - p);
    return (hi & k.b2) | lo;
  } else {
    // byte-to-float conversions (v_cvt_f32_ubyteN), then one packed bf16 conversion
    const uint32_t v = w[p >> 1] >> (16 * (p & 1));
    return pack_bf16((float)(v & 0xFFu), (float)((v >> 8) & 0xFFu));
  }
}

// Inverse of fmt_pair for one code: OR code q of lane code e into w.
template <int BITS>
__device__ __forceinline__ void fmt_place(uint32_t* w, int e, uint32_t q) {
  const int p = e >> 1, h = 16 * (e & 1);
  if constexpr (BITS == 4) {
    w[p >> 2] |= q << (h + 4 * (p & 3));
  } else if constexpr (BITS == 2) {
    w[p >> 3] |= q << (h + 2 * (p & 7));
  } else if constexpr (BITS == 3) {
    w[p >> 3] |= (q & 3u) << (h + 2 * (p & 7));
    w[2] |= ((q >> 2) & 1u) << (h + p);
  } else {
    w[e >> 2] |= q << (8 * (e & 3));
  }
}

// Word j of a lane in its block (8-bit: two vectors, each lane-contiguous).
template <int BITS>
__device__ __forceinline__ long fmt_word(long blk, int lane, int j) {
  if constexpr (BITS == 8)
    return blk * 64 * 8 + (j >> 2) * 256 + lane * 4 + (j & 3);
  else
    return blk * 64 * BITS + lane * BITS + j;
}

// Code k of an MLX row of any width: bits [k*BITS, (k+1)*BITS) of the row's
// LSB-first stream, the high bits from the next word where a field crosses a
// word boundary.
template <int BITS>
__device__ __forceinline__ uint32_t mlx_code_any(const uint32_t* row, long k) {
  const long pos = k * BITS;
  const long wi = pos >> 5;
  const int off = (int)(pos & 31);
  uint32_t v = row[wi] >> off;
  if (off + BITS > 32) v |= row[wi + 1] << (32 - off);
  return v & ((1u << BITS) - 1u);
}

template <int BITS>
__global__ void __launch_bounds__(256) repack_fmt_kernel(const uint32_t* __restrict__ w,
                                                         const uint16_t* __restrict__ scales,
                                                         const uint16_t* __restrict__ biases,
                                                         uint32_t* __restrict__ codes,
                                                         uint16_t* __restrict__ sb, int N, int K,
                                                         int gs) {
  const long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const int nC = K / kChunkK, nT = N / kTileN;
  if (gid >= (long)nT * nC * 64) return;
  const int lane = (int)(gid & 63);
  const long blk = gid >> 6;
  const int c = (int)(blk % nC), tile = (int)(blk / nC);
  const int r = lane & 15, kb = lane >> 4, n = tile * kTileN + r;
  const uint32_t* row = w + (long)n * (K / 32 * BITS);
  uint32_t out[BITS];
#pragma unroll
  for (int j = 0; j < BITS; ++j) out[j] = 0u;
  for (int e = 0; e < 32; ++e)
    fmt_place<BITS>(out, e,
                    mlx_code_any<BITS>(row, (long)kChunkK * c + 32 * (e >> 3) + 8 * kb + (e & 7)));
#pragma unroll
  for (int j = 0; j < BITS; ++j) codes[fmt_word<BITS>(blk, lane, j)] = out[j];
  if (kb == 0) {
    const int Gc = kChunkK / gs, G = K / gs;
    uint16_t* d = sb + (blk * kTileN + r) * 2 * Gc;
    for (int q = 0; q < Gc; ++q) {
      d[q] = scales[(long)n * G + (long)Gc * c + q];
      d[Gc + q] = biases[(long)n * G + (long)Gc * c + q];
    }
  }
}

// Test decoder: the codes as fmt_pair sees them, written to out[n*K + k].
template <int BITS>
__global__ void __launch_bounds__(256) debug_unpack_fmt_kernel(const uint32_t* __restrict__ codes,
                                                               uint8_t* __restrict__ out, int N,
                                                               int K) {
  const long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const int nC = K / kChunkK, nT = N / kTileN;
  if (gid >= (long)nT * nC * 64) return;
  const int lane = (int)(gid & 63);
  const long blk = gid >> 6;
  const int c = (int)(blk % nC), tile = (int)(blk / nC);
  const int r = lane & 15, kb = lane >> 4, n = tile * kTileN + r;
  uint32_t w[BITS];
#pragma unroll
  for (int j = 0; j < BITS; ++j) w[j] = codes[fmt_word<BITS>(blk, lane, j)];
  const FmtMasks mk = fmt_masks<BITS>();
#pragma unroll
  for (int p = 0; p < 16; ++p) {
    const uint32_t v = fmt_pair<BITS>(w, p, mk);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int e = 2 * p + h;
      const float val = bf16_to_f32(h ? v >> 16 : v & 0xFFFFu) - kFmtOffset<BITS>;
      out[(long)n * K + (long)kChunkK * c + 32 * (e >> 3) + 8 * kb + (e & 7)] = (uint8_t)val;
    }
  }
}

// One lane's words of a block: one vector load (3-bit: three words, 8-bit:
// two vectors).  The loads are counted by fmt_code_loads.
template <int BITS>
__device__ __forceinline__ void fmt_load_codes(const uint32_t* __restrict__ codes, long blk,
                                               int lane, uint32_t* w) {
  if constexpr (BITS == 2) {
    const u32x2 v = __builtin_nontemporal_load(
        reinterpret_cast<const u32x2*>(codes + fmt_word<2>(blk, lane, 0)));
    w[0] = v[0];
    w[1] = v[1];
  } else if constexpr (BITS == 3) {
    const uint32_t* p = codes + fmt_word<3>(blk, lane, 0);
#pragma unroll
    for (int q = 0; q < 3; ++q) w[q] = __builtin_nontemporal_load(p + q);
  } else {
#pragma unroll
    for (int i = 0; i < BITS / 4; ++i) {
      const u32x4 v = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(codes + fmt_word<BITS>(blk, lane, 4 * i)));
      w[4 * i] = v[0];
      w[4 * i + 1] = v[1];
      w[4 * i + 2] = v[2];
      w[4 * i + 3] = v[3];
    }
  }
}

// Vector-memory instructions of fmt_load_codes, counted low (the three
// 3-bit words may become one instruction): a wait computed from it never
// ends too early.
template <int BITS>
constexpr int fmt_code_loads() {
  return BITS == 8 ? 2 : 1;
}

// The GC scales and GC biases of one (row, chunk), raw bf16 words.
template <int GC>
struct FmtSB {
  uint32_t raw[GC];  // bf16 values 0..GC-1 scales, GC..2GC-1 biases
  __device__ __forceinline__ void load(const uint16_t* p) {
    if constexpr (GC == 4) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(p);
      raw[0] = v[0];
      raw[1] = v[1];
      raw[2] = v[2];
      raw[3] = v[3];
    } else if constexpr (GC == 2) {
      const uint2 v = *reinterpret_cast<const uint2*>(p);
      raw[0] = v.x;
      raw[1] = v.y;
    } else {
      raw[0] = *reinterpret_cast<const uint32_t*>(p);
    }
  }
  __device__ __forceinline__ float value(int i) const {
    const uint32_t v = raw[i >> 1];
    return __uint_as_float((i & 1) ? (v & 0xFFFF0000u) : (v << 16));
  }
  __device__ __forceinline__ float s(int q) const { return value(q); }
  __device__ __forceinline__ float b(int q) const { return value(GC + q); }
};

template <int BITS, int GS, int NW, int CPW, int TM>
__global__ void __launch_bounds__(NW * 64) fmt_kernel(LaunchArgs a) {
  constexpr int GC = kChunkK / GS;  // groups per chunk
  constexpr int SPG = GS / 32;      // steps per group
  constexpr int LPT = fmt_code_loads<BITS>() + 1;  // loads per (chunk, tile)
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, kb = lane >> 4;
  const int G = gridDim.x, g = blockIdx.x;
  const int nT = a.N / kTileN, nC = a.K / kChunkK;
  const int M = a.M;
  const int count = nC > w ? (nC - w + NW - 1) / NW : 0;  // chunks w, w+NW, ...
  const int clast = count > 0 ? w + (count - 1) * NW : 0;  // waves without chunks re-read chunk 0
  const uint16_t* __restrict__ xg = reinterpret_cast<const uint16_t*>(a.x);
  const uint16_t* __restrict__ sbp = reinterpret_cast<const uint16_t*>(a.sb);

  // 1a. activation slices straight to LDS: 4 rows x 16 vectors per
  //     instruction, lanes of rows >= M masked off
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

  // 1b. every weight load, chunk-major; tile slots past the last tile re-read
  //     the workgroup's first tile (never stored)
  int tl[TM];
#pragma unroll
  for (int t = 0; t < TM; ++t) {
    const int tile = g + t * G;
    tl[t] = tile < nT ? tile : g;
  }
  uint32_t W[CPW][TM][BITS];
  FmtSB<GC> SBv[CPW][TM];
#pragma unroll
  for (int j = 0; j < CPW; ++j) {
    const int c = min(w + j * NW, clast);
#pragma unroll
    for (int t = 0; t < TM; ++t) {
      const long blk = (long)tl[t] * nC + c;
      fmt_load_codes<BITS>(a.codes, blk, lane, W[j][t]);
      SBv[j][t].load(sbp + (blk * kTileN + r) * 2 * GC);
    }
    __builtin_amdgcn_sched_barrier(0);  // chunk j's loads issue before chunk j+1's
  }
  __builtin_amdgcn_sched_barrier(0);

  // 2. the activation slices have landed once at most the weight loads are
  //    outstanding (loads retire in issue order).  The wait also drains the
  //    LDS counter: until it does, the compiler counts the LDS-direct loads
  //    as pending on both counters and makes every later weight wait a full
  //    one (vmcnt(0)) instead of one per chunk.
  wait_vm_lds<(CPW * TM * LPT < 63 ? CPW * TM * LPT : 63)>();

  // 3. per chunk in load order: the A fragments of the four steps, each
  //    group's sum of x (all-ones product), then per tile and group the
  //    products of its steps and s * sum(v x) + (b - offset s) * sum(x);
  //    rows past the last one read the last row (never stored)
  const int xm = min(r, M - 1);
  const int sw = xm & 15;
  const FmtMasks mk = fmt_masks<BITS>();
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
    for (int s = 0; s < 4; ++s) A[s] = xrow[(4 * s + kb) ^ sw];  // columns 32s + 8kb + 0..7
    __builtin_amdgcn_sched_barrier(0);
    f32x4 ex[GC];
#pragma unroll
    for (int q = 0; q < GC; ++q) {
      f32x4 e = zero;
#pragma unroll
      for (int u = 0; u < SPG; ++u)
        e = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, A[q * SPG + u]),
                                                    __builtin_bit_cast(bf16x8, ones), e, 0, 0, 0);
      ex[q] = e;
    }
#pragma unroll
    for (int t = 0; t < TM; ++t) {
#pragma unroll
      for (int q = 0; q < GC; ++q) {
        f32x4 dd = zero;
#pragma unroll
        for (int u = 0; u < SPG; ++u) {
          const int s = q * SPG + u;
          const u32x4 B = {fmt_pair<BITS>(W[j][t], 4 * s, mk),
                           fmt_pair<BITS>(W[j][t], 4 * s + 1, mk),
                           fmt_pair<BITS>(W[j][t], 4 * s + 2, mk),
                           fmt_pair<BITS>(W[j][t], 4 * s + 3, mk)};
          dd = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, A[s]),
                                                       __builtin_bit_cast(bf16x8, B), dd, 0, 0, 0);
        }
        const float s = SBv[j][t].s(q), b = SBv[j][t].b(q);
        const float sc = live ? s : 0.f, bp = live ? b - kFmtOffset<BITS> * s : 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[t][i] = fmaf(sc, dd[i], fmaf(bp, ex[q][i], acc[t][i]));
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
  if (w >= TM) return;
  const int tile = g + w * G;
  if (tile >= nT) return;
  f32x4 v = red[(w * NW) * 64 + lane];
  for (int i = 1; i < NW; ++i) v += red[(w * NW + i) * 64 + lane];
  const int n = tile * kTileN + r;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int m = 4 * kb + q;
    if (m < M) store_y<false>(a, (long)m * a.ldy + n, v[q]);
  }
}

inline unsigned blocks_for(long threads, int per) {
  return (unsigned)((threads + per - 1) / per);
}

// (waves, chunks per wave, tile slots) shapes: four waves below 16 chunks of
// K, eight up to 64 chunks, sixteen up to 128.
#define QMM_FMT_SHAPES(X)                                                                     \
  X(4, 2, 1) X(4, 2, 2) X(4, 2, 3) X(4, 4, 1) X(4, 4, 2) X(4, 4, 3) X(8, 2, 1) X(8, 2, 2)     \
  X(8, 2, 3) X(8, 4, 1) X(8, 4, 2) X(8, 4, 3) X(8, 5, 1) X(8, 5, 2) X(8, 5, 3) X(8, 8, 1)     \
  X(8, 8, 2) X(8, 8, 3) X(16, 8, 1) X(16, 8, 2)

template <int BITS, int GS>
hipError_t fmt_dispatch(int nw, int cpw, int tm, const LaunchArgs& a, int grid, size_t lds,
                        hipStream_t st) {
#define QMM_GO(W, C, T)                                                                       \
  if constexpr (fmt_regs_fit(BITS, GS, W, C, T)) {                                               \
    if (nw == W && cpw == C && tm == T) {                                                     \
      auto* kfn = &fmt_kernel<BITS, GS, W, C, T>;                                             \
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kfn),                  \
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds); \
      if (e != hipSuccess) return e;                                                          \
      kfn<<<grid, W * 64, lds, st>>>(a);                                                      \
      return hipGetLastError();                                                               \
    }                                                                                         \
  }
  QMM_FMT_SHAPES(QMM_GO)
#undef QMM_GO
  return hipErrorInvalidValue;
}

}  // namespace

bool fmt_format(int bits, int group_size) {
  if (group_size != 32 && group_size != 64 && group_size != 128) return false;
  return bits == 2 || bits == 8 || ((bits == 3 || bits == 4) && group_size == 32);
}

bool fmt_shape(int bits, int group_size, int nC, int tm, int* nw, int* cpw) {
  int best_w = 0, best_c = 0;
#define QMM_PICK(W, C, T)                                                                    \
  if (T == tm && (nC < 16) == (W == 4) && W * C >= nC &&                                     \
      fmt_regs_fit(bits, group_size, W, C, T) && (best_c == 0 || C < best_c)) {                 \
    best_w = W;                                                                             \
    best_c = C;                                                                             \
  }
  QMM_FMT_SHAPES(QMM_PICK)
#undef QMM_PICK
  *nw = best_w;
  *cpw = best_c;
  return best_c > 0;
}

int fmt_rows(long K) {
  const long r = (long)kMaxLdsBytes / (K * 2);
  return (int)std::min(r, 16L);
}

size_t fmt_lds_bytes(int nw, int tm, int M, int K) {
  return std::max((size_t)std::min(M, 16) * K * 2, (size_t)tm * nw * 64 * 16);
}

hipError_t launch_fmt(int bits, int group_size, int nw, int cpw, int tm, const LaunchArgs& a,
                      int grid, size_t lds_bytes, hipStream_t st) {
#define QMM_FMT(B, GS)        \
  if (bits == B && group_size == GS) \
    return fmt_dispatch<B, GS>(nw, cpw, tm, a, grid, lds_bytes, st);
  QMM_FMT(2, 32) QMM_FMT(2, 64) QMM_FMT(2, 128) QMM_FMT(8, 32) QMM_FMT(8, 64) QMM_FMT(8, 128)
  QMM_FMT(3, 32) QMM_FMT(4, 32)
#undef QMM_FMT
  return hipErrorInvalidValue;
}

hipError_t launch_repack_fmt(int bits, int group_size, const uint32_t* w, const void* scales,
                             const void* biases, uint32_t* codes, void* sb, int N, int K,
                             hipStream_t st) {
  const unsigned grid = blocks_for((long)(N / kTileN) * (K / kChunkK) * 64, 256);
  const uint16_t* s = static_cast<const uint16_t*>(scales);
  const uint16_t* bb = static_cast<const uint16_t*>(biases);
  uint16_t* d = static_cast<uint16_t*>(sb);
  switch (bits) {
    case 2: repack_fmt_kernel<2><<<grid, 256, 0, st>>>(w, s, bb, codes, d, N, K, group_size); break;
    case 3: repack_fmt_kernel<3><<<grid, 256, 0, st>>>(w, s, bb, codes, d, N, K, group_size); break;
    case 4: repack_fmt_kernel<4><<<grid, 256, 0, st>>>(w, s, bb, codes, d, N, K, group_size); break;
    case 8: repack_fmt_kernel<8><<<grid, 256, 0, st>>>(w, s, bb, codes, d, N, K, group_size); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_debug_unpack_fmt(int bits, const uint32_t* codes, uint8_t* out, int N, int K,
                                   hipStream_t st) {
  const unsigned grid = blocks_for((long)(N / kTileN) * (K / kChunkK) * 64, 256);
  switch (bits) {
    case 2: debug_unpack_fmt_kernel<2><<<grid, 256, 0, st>>>(codes, out, N, K); break;
    case 3: debug_unpack_fmt_kernel<3><<<grid, 256, 0, st>>>(codes, out, N, K); break;
    case 4: debug_unpack_fmt_kernel<4><<<grid, 256, 0, st>>>(codes, out, N, K); break;
    case 8: debug_unpack_fmt_kernel<8><<<grid, 256, 0, st>>>(codes, out, N, K); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace qmm
