// qmm_formats.h -- weight-format policies of the matrix-core kernels: how a
// lane loads its codes of one block (16 rows x 128 columns), turns them into
// 16 pairs of bf16 B-operand values, which 16-byte activation vector is its A
// fragment of each of the block's four 16x16x32 products ("steps"), and the
// per-group factors that turn the products into s * sum(q x) + b * sum(x).
// The streaming and resident kernels are written once over these policies.
// Not installed.
//
// [P1] = page "@mlx-bun/inference 0.0.0-stage -> 1.0.0": affine-split-mma.ts
// (MLX affine weights, w = s * q + b per group); affine3-rows.ts header (the
// factored sum_g s * sum(q x) + b * sum(x)).  [P3] = page "mlx-bun 0.0.4",
// fused-decode-kernel.ts: widths 4 and 8 and group sizes 32, 64 and 128 of
// affine-quantized tensors.
//
// NativeFmt<BITS, ST>: 3- and 4-bit codes in the native layout of
// qmm_device.h (groups of 64; a group of 128 repacked as two halves with the
// same scale and bias).  Step t = 2g' + h covers, for lane quarter kg,
// columns 64g' + 16kg + 8h + 0..7 of the chunk: two steps per group.
//
// StepFmt<BITS, GS>: 2- and 8-bit codes (groups of 32, 64, 128) and 3- and
// 4-bit codes with groups of 32 in the step layout, bf16 scales and biases.
// Block (tile t, chunk c) has index t*nC + c and holds 64 lanes x BITS words;
// lane l = (r = l & 15, kb = l >> 4) holds the 32 codes e = 8s + i of row
// 16t + r at columns
//     k = 128c + 32s + 8kb + i,   s = 0..3 (step), i = 0..7,
// exactly its B operand of step s; a group of 32, 64 or 128 columns is 1, 2
// or 4 whole steps.  Code e is half h = e & 1 of pair p = e >> 1:
//   4-bit: pair p in word p >> 2, field u = p & 3: bits 4u (h = 0), 16+4u;
//   2-bit: pair p in word p >> 3, field u = p & 7: bits 2u (h = 0), 16+2u;
//   3-bit: the two low bits of the codes as the 2-bit layout in words 0 and
//          1, bit 2 of pair p's codes in word 2 at bits p (h = 0) and 16+p;
//   8-bit: code e in byte e & 3 of word e >> 2; the lane's words 0..3 and
//          4..7 are two 16-byte vectors, each contiguous over the 64 lanes.
// A wave reads 512, 768, 1024 or 2 x 1024 contiguous bytes per block.  For
// 2, 3 and 4 bits one and-or per pair makes bf16 values 128 + q (0x4300 | q)
// and the offset goes with the group's sum of x:
//     sum_k (s q_k + b) x_k = s * sum_k (128 + q_k) x_k + (b - 128 s) * sum_k x_k;
// 8-bit codes go through byte-to-float conversions and a packed bf16
// conversion (integers up to 256 are bf16 values), offset 0.  Scales and
// biases: block b holds 16 rows x (Gc scales, then Gc biases), Gc = 128/GS.
#pragma once

#include "qmm_device.h"

namespace qmm {

template <int BITS, typename ST>
struct NativeFmt {
  static constexpr int kBits = BITS;
  static constexpr int kGroups = 2;      // groups per chunk
  static constexpr int kSpg = 2;         // steps per group
  static constexpr int kGroupVecs = 8;   // 16-byte activation vectors per group
  static constexpr int kCodeLoads = 1;   // vector-memory instructions per block, counted low
  static constexpr int kSbElems = 4;     // scale/bias elements per (row, block)
  using St = ST;
  using Sb = SBPair<ST>;
  using Masks = PairMasks;
  __device__ static __forceinline__ Masks masks() { return pair_mask_vgpr<BITS>(); }
  __device__ static __forceinline__ void load(const uint32_t* __restrict__ codes, long blk,
                                              int lane, uint32_t* w) {
    const uint32_t* p = codes + blk * 64 * BITS + lane * BITS;
#pragma unroll
    for (int q = 0; q < BITS; ++q) w[q] = __builtin_nontemporal_load(p + q);
  }
  __device__ static __forceinline__ void unpack(const uint32_t* w, uint32_t* P, const Masks& k) {
    unpack_pairs<BITS>(w, P, k);
  }
  // 16-byte vector of a row's 128-value chunk slice that is lane quarter
  // kg's A fragment of step t
  __device__ static __forceinline__ int a_vec(int t, int kg) { return 8 * (t >> 1) + 2 * kg + (t & 1); }
  __device__ static __forceinline__ Affine affine(int g, const Sb& sb) {
    return group_affine<BITS>(g, sb.s(g), sb.b(g));
  }
  // every built shape of the streaming and resident kernels
  static constexpr bool stream_fits(int, int) { return true; }
  static constexpr bool resident_fits(int, int, int) { return true; }
};

// Chunks of weight loads a wave of the resident kernel keeps in flight (its
// ring of weight registers).
constexpr int kResidentRing = 2;

typedef uint32_t u32x2 __attribute__((__vector_size__(8)));
typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));

// Mask constants of the step-layout pair extraction: the or-value 0x43004300
// in a VGPR, the field masks in SGPRs (an and-or takes no literal here).
struct StepMasks {
  uint32_t orv, m2, m4, b2;  // 0x43004300, 0x00030003, 0x000F000F, 0x00040004
};

// The GC scales and GC biases of one (row, block), raw bf16 words.
template <int GC>
struct StepSb {
  uint32_t raw[GC];  // bf16 values 0..GC-1 scales, GC..2GC-1 biases
  __device__ __forceinline__ void load(const uint16_t* p) {
    if constexpr (GC == 4) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(p);
      raw[0] = v[0];
      raw[1] = v[1];
      raw[2] = v[2];
      raw[3] = v[3];
    } else if constexpr (GC == 2) {
      const u32x2 v = *reinterpret_cast<const u32x2*>(p);
      raw[0] = v[0];
      raw[1] = v[1];
    } else {
      raw[0] = *reinterpret_cast<const uint32_t*>(p);
    }
  }
  __device__ __forceinline__ float value(int i) const {
    const uint32_t v = raw[i >> 1];
    return __uint_as_float((i & 1) ? (v & 0xFFFF0000u) : (v << 16));
  }
  __device__ __forceinline__ float s(int g) const { return value(g); }
  __device__ __forceinline__ float b(int g) const { return value(GC + g); }
};

template <int BITS, int GS>
struct StepFmt {
  static_assert(GS == 32 || GS == 64 || GS == 128, "MLX affine group sizes");
  static constexpr int kBits = BITS;
  static constexpr int kGroups = kChunkK / GS;
  static constexpr int kSpg = GS / 32;
  static constexpr int kGroupVecs = GS / 8;
  static constexpr int kCodeLoads = BITS == 8 ? 2 : 1;
  static constexpr int kSbElems = 2 * kGroups;
  static constexpr float kOffset = BITS == 8 ? 0.f : 128.f;  // value = offset + q
  using St = uint16_t;
  using Sb = StepSb<kGroups>;
  using Masks = StepMasks;

  __device__ static __forceinline__ Masks masks() {
    Masks k{};
    asm volatile("v_mov_b32 %0, %1" : "=v"(k.orv) : "s"(0x43004300u));
    if constexpr (BITS == 4) k.m4 = opaque_sgpr(0x000F000Fu);
    if constexpr (BITS == 2 || BITS == 3) k.m2 = opaque_sgpr(0x00030003u);
    if constexpr (BITS == 3) k.b2 = opaque_sgpr(0x00040004u);
    return k;
  }
  // word j of a lane in its block
  __device__ static __forceinline__ long word(long blk, int lane, int j) {
    if constexpr (BITS == 8)
      return blk * 64 * 8 + (j >> 2) * 256 + lane * 4 + (j & 3);
    else
      return blk * 64 * BITS + lane * BITS + j;
  }
  __device__ static __forceinline__ void load(const uint32_t* __restrict__ codes, long blk,
                                              int lane, uint32_t* w) {
    if constexpr (BITS == 2) {
      const u32x2 v =
          __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(codes + word(blk, lane, 0)));
      w[0] = v[0];
      w[1] = v[1];
    } else if constexpr (BITS == 3) {
      const uint32_t* p = codes + word(blk, lane, 0);
#pragma unroll
      for (int q = 0; q < 3; ++q) w[q] = __builtin_nontemporal_load(p + q);
    } else {
#pragma unroll
      for (int i = 0; i < BITS / 4; ++i) {
        const u32x4 v = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4*>(codes + word(blk, lane, 4 * i)));
        w[4 * i] = v[0];
        w[4 * i + 1] = v[1];
        w[4 * i + 2] = v[2];
        w[4 * i + 3] = v[3];
      }
    }
  }
  __device__ static __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    const bf16x2_v v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
  }
  // pair p (codes 2p, 2p+1) as two bf16 values
  __device__ static __forceinline__ uint32_t pair(const uint32_t* w, int p, const Masks& k) {
    if constexpr (BITS == 4) {
      return and_or(w[p >> 2] >> (4 * (p & 3)), k.m4, k.orv);
    } else if constexpr (BITS == 2) {
      return and_or(w[p >> 3] >> (2 * (p & 7)), k.m2, k.orv);
    } else if constexpr (BITS == 3) {
      const uint32_t lo = and_or(w[p >> 3] >> (2 * (p & 7)), k.m2, k.orv);
      const uint32_t hi = p >= 2 ? w[2] >> (p - 2) : w[2] << (2 - p);
      return (hi & k.b2) | lo;
    } else {
      // byte-to-float conversions (v_cvt_f32_ubyteN), one packed bf16 conversion
      const uint32_t v = w[p >> 1] >> (16 * (p & 1));
      return pack_bf16((float)(v & 0xFFu), (float)((v >> 8) & 0xFFu));
    }
  }
  // inverse of pair() for one code: OR code q of lane code e into w
  __device__ static __forceinline__ void place(uint32_t* w, int e, uint32_t q) {
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
  __device__ static __forceinline__ void unpack(const uint32_t* w, uint32_t* P, const Masks& k) {
#pragma unroll
    for (int p = 0; p < 16; ++p) P[p] = pair(w, p, k);
  }
  __device__ static __forceinline__ int a_vec(int t, int kb) { return 4 * t + kb; }
  __device__ static __forceinline__ Affine affine(int g, const Sb& sb) {
    const float s = sb.s(g);
    return Affine{s, sb.b(g) - kOffset * s};
  }
  // Shapes whose weight registers (codes and scale/bias words of every
  // chunk and tile slot a wave holds at once: the resident kernel's ring
  // holds kResidentRing chunks, the streaming kernel all of its chunks)
  // leave room for the rest without spilling: 128 words with up to 8 waves
  // (two per SIMD); with 16 waves (128 registers each) 72, and 56 for the
  // streaming kernel, whose waves also hold their activation slices in
  // registers.
  static constexpr bool resident_fits(int nw, int cpw, int tm) {
    return (cpw < kResidentRing ? cpw : kResidentRing) * tm * (BITS + kGroups) <=
           (nw >= 16 ? 72 : 128);
  }
  static constexpr bool stream_fits(int nw, int cpw) {
    return cpw * (BITS + kGroups) <= (nw >= 16 ? 56 : 128);
  }
};

// Step-layout formats that have kernels: 2- and 8-bit codes with any MLX
// group size, 3- and 4-bit codes with groups of 32.
#define QMM_STEP_FORMATS(X) X(2, 32) X(2, 64) X(2, 128) X(8, 32) X(8, 64) X(8, 128) X(3, 32) X(4, 32)

}  // namespace qmm
