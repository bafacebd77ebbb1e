// qmm_stream.hip -- the streaming matrix-core kernel for 1..4 activation rows.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "qmm_formats.h"

namespace qmm {

// ---------------------------------------------------------------------------
// Streaming MFMA kernel for short activation blocks (at most 4 rows), over a
// weight-format policy F (qmm_formats.h).  One
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
// VALU = true is the vector-ALU form of step 3: per activation row, lane
// (r, kg) takes the dot products of its B-operand pairs with the same A
// fragments through v_dot2_f32_bf16, scales each group's dot by s, and lanes
// kg = 0 add b' * (the group's sum of x); the four lane quarters of a row are
// added by cross-lane swaps before the fold, and output row m comes from the
// lanes kg = 0 of column r.
// XS = true takes the group sums of x from a.xsums (qmm_run_sums: written by
// the residual add + RMS norm that produced x) instead of forming them from
// the slices: loaded with the slices, stored to the same LDS area.
// LDS per wave: rows x (CPW*256 + 16) bytes of slices (the 16-byte pad puts
// consecutive rows on different banks) and rows x CPW x F::kGroups group sums.
// ---------------------------------------------------------------------------
constexpr int kStreamRowPad = 16;
// Sum over each aligned group of L (4, 8 or 16) lanes: swap neighbours,
// pairs, half rows, rows.
template <int L>
__device__ __forceinline__ float dpp_sum(float s) {
  s += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, s), 0xB1, 0xF, 0xF, true));
  s += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, s), 0x4E, 0xF, 0xF, true));
  if constexpr (L >= 8)
    s += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, s), 0x141, 0xF, 0xF, true));
  if constexpr (L >= 16)
    s += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, s), 0x140, 0xF, 0xF, true));
  return s;
}

// The G floats at p (G = 1, 2 or 4) in one load.
template <int G>
__device__ __forceinline__ void load_floats(const float* p, float* v) {
  if constexpr (G == 4) {
    const float4 f = *reinterpret_cast<const float4*>(p);
    v[0] = f.x;
    v[1] = f.y;
    v[2] = f.z;
    v[3] = f.w;
  } else if constexpr (G == 2) {
    const float2 f = *reinterpret_cast<const float2*>(p);
    v[0] = f.x;
    v[1] = f.y;
  } else {
    v[0] = *p;
  }
}

// Vectors of 16 bytes per lane for rows (<= MQ) x CPW slices of 128 values.
template <int MQ, int CPW>
struct StreamXL { static constexpr int value = (MQ * CPW * 16 + 63) / 64; };

// Timing build: the wait for chunk j's weights (LPC loads per later chunk
// outstanding); j is a constant once the caller's loop is unrolled.
template <int CPW, int LPC, int J = 0>
__device__ __forceinline__ void stamp_chunk(int j) {
  if constexpr (J < CPW) {
    if (j == J)
      stamp_wait<(CPW - 1 - J) * LPC>();
    else
      stamp_chunk<CPW, LPC, J + 1>(j);
  }
}

template <typename F, int NW, int CPW, int MQ, bool VALU = false, bool XS = false>
__global__ void __launch_bounds__(NW * 64) stream_kernel(LaunchArgs a) {
  constexpr int BITS = F::kBits, GC = F::kGroups, SPG = F::kSpg;
  using ST = typename F::St;
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
                (size_t)w * a.M * CPW * GC;                                    // [M][CPW][GC]

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
  // XS: the given group sums of this wave's entries (row m, slot j, group g)
  // in the LDS order of the sums, (m * CPW + j) * GC + g
  constexpr int XSL = XS ? (MQ * CPW * GC + 63) / 64 : 1;
  const int ns = a.M * CPW * GC;
  float xsv[XSL];
  if constexpr (XS) {
#pragma unroll
    for (int i = 0; i < XSL; ++i) {
      const int e = min(lane + 64 * i, ns - 1);
      const int m = e / (CPW * GC), j = (e / GC) % CPW, g = e % GC;
      const int c = min(w + j * NW, clast);
      xsv[i] = a.xsums[(long)(GC * c + g) * a.xsums_ld + m];
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  ts.mark(1);

  // weight loads of every slot; slots past `count` re-read the last chunk
  const ST* sbase = sbp + ((long)tile * nC * kTileN + r) * F::kSbElems;
  uint32_t W[CPW][BITS];
  typename F::Sb SBv[CPW];
#pragma unroll
  for (int j = 0; j < CPW; ++j) {
    const int c = min(w + j * NW, clast);
    F::load(a.codes, (long)tile * nC + c, lane, W[j]);
    SBv[j].load(sbase + (long)c * kTileN * F::kSbElems);
    __builtin_amdgcn_sched_barrier(0);  // chunk j's loads issue before chunk j+1's
  }
  __builtin_amdgcn_sched_barrier(0);
  ts.mark(2);

  // 2. slices and their group sums to this wave's LDS area.  The lanes
  //    holding one (row, slot, group) are an aligned group of F::kGroupVecs;
  //    lanes whose vector index is past the end hold a repeated vector and
  //    write no sum.
  const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
#pragma unroll
  for (int i = 0; i < XL; ++i) {
    *reinterpret_cast<u32x4*>(xw + xo[i]) = xv[i];
    if constexpr (XS) continue;
    // (each element is copied out first: a bit cast of a vector subscript
    // compiles to element 0 here)
    float s = 0.f;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t xd = xv[i][d], od = ones[d];
      s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, xd),
                                          __builtin_bit_cast(bf16x2, od), s, false);
    }
    s = dpp_sum<F::kGroupVecs>(s);
    const int v = lane + 64 * i;
    if (v < nv && (lane & (F::kGroupVecs - 1)) == 0) {
      const int m = v / (CPW * 16), rem = v - m * (CPW * 16);
      xsum[(m * CPW + (rem >> 4)) * GC + (rem & 15) / F::kGroupVecs] = s;
    }
  }
  if constexpr (XS) {
#pragma unroll
    for (int i = 0; i < XSL; ++i)
      if (lane + 64 * i < ns) xsum[lane + 64 * i] = xsv[i];
  }
  // other lanes of this wave read what these lanes wrote: keep the compiler
  // from moving the reads above the writes (LDS runs a wave's accesses in order)
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  ts.mark(3);
  // 3. compute in load order; rows past the last one read the last row
  //    (never stored)
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  const typename F::Masks mask_v = F::masks();
  f32x4 acc = zero;
  if constexpr (!VALU) {
    const unsigned char* xrow = xw + min(r, a.M - 1) * ROWB;
    const float* srow[MQ];
#pragma unroll
    for (int q = 0; q < MQ; ++q) srow[q] = xsum + min(4 * kg + q, a.M - 1) * CPW * GC;
#pragma unroll
    for (int j = 0; j < CPW; ++j) {
      const bool live = j < count;
      stamp_chunk<CPW, F::kCodeLoads + 1>(j);  // timing build: wait for chunk j's
      ts.mark(4 + j);                          // weights, then stamp their arrival
      u32x4 A[4];
#pragma unroll
      for (int t = 0; t < 4; ++t)
        A[t] = *reinterpret_cast<const u32x4*>(xrow + 256 * j + 16 * F::a_vec(t, kg));
      float ex[MQ][GC];
#pragma unroll
      for (int q = 0; q < MQ; ++q) load_floats<GC>(srow[q] + GC * j, ex[q]);
      uint32_t P[16];
      F::unpack(W[j], P, mask_v);
#pragma unroll
      for (int g = 0; g < GC; ++g) {
        f32x4 dd = zero;
#pragma unroll
        for (int u = 0; u < SPG; ++u) {
          const int t = g * SPG + u;
          const u32x4 B = {P[4 * t], P[4 * t + 1], P[4 * t + 2], P[4 * t + 3]};
          dd = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, A[t]),
                                                       __builtin_bit_cast(bf16x8, B), dd, 0, 0, 0);
        }
        const Affine af = F::affine(g, SBv[j]);
        const float sc = af.sc, bp = af.bp;
#pragma unroll
        for (int q = 0; q < MQ; ++q) {
          const float v = fmaf(sc, dd[q], fmaf(bp, ex[q][g], acc[q]));
          acc[q] = live ? v : acc[q];
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    // rows q < MQ (rows past the last one read the last row, never stored)
    const unsigned char* xrow[MQ];
    const float* srow[MQ];
#pragma unroll
    for (int q = 0; q < MQ; ++q) {
      xrow[q] = xw + min(q, a.M - 1) * ROWB;
      srow[q] = xsum + min(q, a.M - 1) * CPW * GC;
    }
    const float bias_lane = kg == 0 ? 1.f : 0.f;  // one quarter adds each group's bias term
#pragma unroll
    for (int j = 0; j < CPW; ++j) {
      const bool live = j < count;
      stamp_chunk<CPW, F::kCodeLoads + 1>(j);
      ts.mark(4 + j);
      uint32_t P[16];
      F::unpack(W[j], P, mask_v);
#pragma unroll
      for (int q = 0; q < MQ; ++q) {
        u32x4 A[4];
#pragma unroll
        for (int t = 0; t < 4; ++t)
          A[t] = *reinterpret_cast<const u32x4*>(xrow[q] + 256 * j + 16 * F::a_vec(t, kg));
        float ex[GC];
        load_floats<GC>(srow[q] + GC * j, ex);
#pragma unroll
        for (int g = 0; g < GC; ++g) {
          float dot = 0.f;
#pragma unroll
          for (int u = 0; u < SPG; ++u) {
            const int t = g * SPG + u;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const uint32_t xa = A[t][i];  // (copied out: see the slice sums above)
              dot = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, P[4 * t + i]),
                                                    __builtin_bit_cast(bf16x2, xa), dot, false);
            }
          }
          const Affine af = F::affine(g, SBv[j]);
          const float v = fmaf(af.sc, dot, fmaf(af.bp * bias_lane, ex[g], acc[q]));
          acc[q] = live ? v : acc[q];
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // add the four lane quarters of each row: lanes l, l^16, l^32, l^48
#pragma unroll
    for (int q = 0; q < MQ; ++q) {
      acc[q] += __shfl_xor(acc[q], 16);
      acc[q] += __shfl_xor(acc[q], 32);
    }
  }

  ts.mark(12);
  // 4. add the NW partial tiles in wave order and store rows < M
  // [NW-1][64] after every wave's slices and group sums (stream_lds_bytes)
  f32x4* red = reinterpret_cast<f32x4*>(lds + (size_t)NW * a.M * (ROWB + CPW * 4 * GC));
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
    // the matrix-core form holds rows 4kg + q, the vector-ALU form rows q (every quarter)
    const int m = VALU ? q : 4 * kg + q;
    if (m < a.M && (!VALU || kg == 0)) store_y<false>(a, (long)m * a.ldy + n, acc[q]);
  }
  ts.mark(14);
  ts.flush(lane);
}

size_t stream_lds_bytes(int nw, int cpw, int M, int groups) {
  return (size_t)nw * M * (cpw * 256 + kStreamRowPad + cpw * 4 * groups) +
         (size_t)(nw - 1) * 64 * 16;
}
bool stream_fits(int nw, int cpw, int M, int groups, size_t max_lds) {
  return M >= 1 && M <= kStreamMaxRows && stream_lds_bytes(nw, cpw, M, groups) <= max_lds;
}

template <typename F, int MQ, bool VALU, bool XS>
static hipError_t stream_dispatch_mq(int nw, int cpw, const LaunchArgs& a, size_t lds,
                                     hipStream_t st) {
  const unsigned grid = (unsigned)(a.N / kTileN);
#define QMM_STREAM(NWV, CPWV)                                                                \
  if constexpr (F::stream_fits(NWV, CPWV)) {                                                 \
    if (nw == NWV && cpw == CPWV) {                                                          \
      auto* kfn = &stream_kernel<F, NWV, CPWV, MQ, VALU, XS>;                                          \
      if (lds > 64 * 1024) {                                                                 \
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kfn),               \
                                           hipFuncAttributeMaxDynamicSharedMemorySize,       \
                                           (int)lds);                                        \
        if (e != hipSuccess) return e;                                                       \
      }                                                                                      \
      kfn<<<grid, NWV * 64, lds, st>>>(a);                                                   \
      return hipGetLastError();                                                              \
    }                                                                                        \
  }
  QMM_STREAM(4, 2) QMM_STREAM(4, 4) QMM_STREAM(8, 4) QMM_STREAM(8, 5) QMM_STREAM(8, 8)
  QMM_STREAM(16, 8)
#undef QMM_STREAM
  return hipErrorInvalidValue;
}

template <typename F, bool VALU, bool XS>
static hipError_t stream_dispatch_xs(int nw, int cpw, const LaunchArgs& a, size_t lds,
                                     hipStream_t st) {
  if (a.M == 1) return stream_dispatch_mq<F, 1, VALU, XS>(nw, cpw, a, lds, st);
  if (a.M == 2) return stream_dispatch_mq<F, 2, VALU, XS>(nw, cpw, a, lds, st);
  return stream_dispatch_mq<F, 4, VALU, XS>(nw, cpw, a, lds, st);
}

// The matrix-core form takes given group sums (a.xsums); the vector-ALU form
// always forms its own.
template <typename F, bool VALU = false>
static hipError_t stream_dispatch(int nw, int cpw, const LaunchArgs& a, size_t lds,
                                  hipStream_t st) {
  if (!VALU && a.xsums) return stream_dispatch_xs<F, false, true>(nw, cpw, a, lds, st);
  return stream_dispatch_xs<F, VALU, false>(nw, cpw, a, lds, st);
}

bool stream_step_fits(int bits, int group_size, int nw, int cpw) {
#define QMM_FIT(B, GS) \
  if (bits == B && group_size == GS) return StepFmt<B, GS>::stream_fits(nw, cpw);
  QMM_STEP_FORMATS(QMM_FIT)
#undef QMM_FIT
  return false;
}

hipError_t launch_stream(int bits, int step_gs, bool sb_f32, int nw, int cpw, const LaunchArgs& a,
                         size_t lds_bytes, hipStream_t st) {
  if (step_gs) {
#define QMM_STEP(B, GS)                 \
  if (bits == B && step_gs == GS) \
    return stream_dispatch<StepFmt<B, GS>>(nw, cpw, a, lds_bytes, st);
    QMM_STEP_FORMATS(QMM_STEP)
#undef QMM_STEP
    return hipErrorInvalidValue;
  }
  if (bits == 3)
    return sb_f32 ? stream_dispatch<NativeFmt<3, float>>(nw, cpw, a, lds_bytes, st)
                  : stream_dispatch<NativeFmt<3, uint16_t>>(nw, cpw, a, lds_bytes, st);
  return sb_f32 ? stream_dispatch<NativeFmt<4, float>>(nw, cpw, a, lds_bytes, st)
                : stream_dispatch<NativeFmt<4, uint16_t>>(nw, cpw, a, lds_bytes, st);
}

hipError_t launch_stream_valu(int bits, bool sb_f32, int nw, int cpw, const LaunchArgs& a,
                              size_t lds_bytes, hipStream_t st) {
  if (bits == 3)
    return sb_f32 ? stream_dispatch<NativeFmt<3, float>, true>(nw, cpw, a, lds_bytes, st)
                  : stream_dispatch<NativeFmt<3, uint16_t>, true>(nw, cpw, a, lds_bytes, st);
  return sb_f32 ? stream_dispatch<NativeFmt<4, float>, true>(nw, cpw, a, lds_bytes, st)
                : stream_dispatch<NativeFmt<4, uint16_t>, true>(nw, cpw, a, lds_bytes, st);
}

}  // namespace qmm
