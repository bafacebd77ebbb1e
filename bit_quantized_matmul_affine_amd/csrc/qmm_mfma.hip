// qmm_mfma.hip -- the blocked matrix-core kernel (any row count up to 64 per
// pass, optional K split across workgroups) and the vector-ALU kernel (f32
// activations, and bf16 where forced).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "qmm_device.h"

namespace qmm {

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
          if (m < a.M) store_y<false>(a, (long)m * a.ldy + n, acc[nt][mt][q]);
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
        if (m < a.M) store_y<X_F32>(a, (long)m * a.ldy + n, acc[nt][m]);
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

}  // namespace qmm
