// qmm_stream.hip -- the streaming matrix-core kernel for 1..4 activation rows.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "qmm_device.h"

namespace qmm {

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

// Timing build: the wait for chunk j's weights (two loads per later chunk
// outstanding); j is a constant once the caller's loop is unrolled.
template <int CPW, int J = 0>
__device__ __forceinline__ void stamp_chunk(int j) {
  if constexpr (J < CPW) {
    if (j == J)
      stamp_wait<(CPW - 1 - J) * 2>();
    else
      stamp_chunk<CPW, J + 1>(j);
  }
}

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
  WaveStamps ts(a, (long)blockIdx.x * NW + w);  // timing build only
  ts.mark(0);
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
  ts.mark(1);

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
  ts.mark(2);

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

  ts.mark(3);
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
    stamp_chunk<CPW>(j);  // timing build: wait for chunk j's weights, then
    ts.mark(4 + j);       // stamp their arrival
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

  ts.mark(12);
  // 4. add the NW partial tiles in wave order and store rows < M
  f32x4* red = reinterpret_cast<f32x4*>(lds + (size_t)NW * a.M * (ROWB + CPW * 8));  // [NW-1][64]
  if (w > 0) red[(w - 1) * 64 + lane] = acc;
  __syncthreads();
  ts.mark(13);
  if (w != 0) {
    ts.flush(lane);
    return;
  }
#pragma unroll
  for (int i = 1; i < NW; ++i) acc += red[(i - 1) * 64 + lane];
  const int n = tile * kTileN + r;
#pragma unroll
  for (int q = 0; q < MQ; ++q) {
    const int m = 4 * kg + q;
    if (m < a.M) store_y<false>(a, (long)m * a.ldy + n, acc[q]);
  }
  ts.mark(14);
  ts.flush(lane);
}

size_t stream_lds_bytes(int nw, int cpw, int M) {
  return (size_t)nw * M * (cpw * 256 + kStreamRowPad + cpw * 8) + (size_t)(nw - 1) * 64 * 16;
}
bool stream_fits(int nw, int cpw, int M, size_t max_lds) {
  return M >= 1 && M <= kStreamMaxRows && stream_lds_bytes(nw, cpw, M) <= max_lds;
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

}  // namespace qmm
