// qmm_wide.hip -- the wide kernel for 65..128 activation rows (weights
// dequantized once to bf16 in registers).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "qmm_device.h"

namespace qmm {

// ---------------------------------------------------------------------------
// Wide kernel for 65..128 activation rows (the compute/bandwidth crossover).
// At 128 rows the per-group epilogue of the factored dequant (two FMAs per
// output and group) would cost more vector instructions than the weights
// themselves, so here every weight is dequantized once, in registers, to
// bf16 (w = s*q + b, rounded to nearest even; 4-bit codes converted exactly
// to f32 two at a time by dequant4_exact, 3-bit ones from the unpacked pairs
// and group factors) and the MFMAs accumulate y directly over all of K: no
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
// One B fragment of bf16 weights w = s*q + b from 4-bit word j of the
// native layout (pair t = field t: codes at bits 4t and 16+4t).  The word's
// nibble planes hold one code per byte; a byte below 16 read as an OCP e4m3
// value is exactly q * 2^-9, so one conversion scaled by 2^9 gives two exact
// codes as f32: plane lo = fields 0 and 2, plane hi = fields 1 and 3, byte
// halves 0 / 1 = the low / high code of the pair.
typedef float f32x2_w __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u32x4 dequant4_exact(uint32_t w, float s, float b, uint32_t nib) {
  const uint32_t lo = w & nib, hi = (w >> 4) & nib;
  const f32x2_w l0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(lo, 512.0f, false);
  const f32x2_w l1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(lo, 512.0f, true);
  const f32x2_w h0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hi, 512.0f, false);
  const f32x2_w h1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hi, 512.0f, true);
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  auto pk = [&](float qa, float qb) {
    const bf16x2_t v = {(__bf16)fmaf(s, qa, b), (__bf16)fmaf(s, qb, b)};
    return __builtin_bit_cast(uint32_t, v);
  };
  return u32x4{pk(l0[0], l1[0]), pk(h0[0], h1[0]), pk(l0[1], l1[1]), pk(h0[1], h1[1])};
}

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
    const uint32_t nib = opaque_sgpr(0x0F0F0F0Fu);  // 4-bit: one code per byte
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
        uint32_t Wg[TW][2];  // 4-bit: the words of group gp
#pragma unroll
        for (int i = 0; i < TW; ++i) {
          if constexpr (BITS == 4) {
            Wg[i][0] = W[i][2 * gp];
            Wg[i][1] = W[i][2 * gp + 1];
            f[i] = Affine{SBv[i].s(gp), SBv[i].b(gp)};
          } else {
            unpack_pairs<BITS>(W[i], P[i], mask_v);
            f[i] = group_affine<BITS>(gp, SBv[i].s(gp), SBv[i].b(gp));
          }
        }
        if (gp == 1 && j + 1 < NS) load(j + 1);  // the raw words are unpacked
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int q = 2 * gp + h;
          u32x4 B[TW];
#pragma unroll
          for (int i = 0; i < TW; ++i) {
            if constexpr (BITS == 4) {
              B[i] = dequant4_exact(Wg[i][h], f[i].sc, f[i].bp, nib);
              continue;
            }
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
        if (m < M) store_y<false>(a, (long)m * a.ldy + n, v[q]);
      }
    }
  }
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

}  // namespace qmm
