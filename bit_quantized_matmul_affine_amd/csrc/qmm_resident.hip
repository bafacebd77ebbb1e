// qmm_resident.hip -- the resident matrix-core kernel (up to 16 activation
// rows held in LDS) and the fused gate/up projection pair built on it.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "qmm_formats.h"

namespace qmm {

// ---------------------------------------------------------------------------
// Resident MFMA kernel for blocks of up to 16 activation rows whose whole
// activation block fits in LDS (rows*K*2 <= 160 KB), over a weight-format
// policy F (qmm_formats.h).  Workgroup g owns the
// TM tiles g, g+G, g+2G, ... (G = grid size); its NW wavefronts split K:
// wave w takes chunks w, w+NW, ... (at most CPW) of every one of those tiles,
// so each activation fragment it reads, and each group sum it forms, serves
// TM tiles.  Order of work in a wave:
//   1. LDS-direct loads (no registers) of the activation slices of its
//      chunks, then the weight loads of its first two chunks (TM tiles each);
//   2. a wait for its own activation slices only (loads retire in issue
//      order, so the weights stay in flight); no barrier;
//   3. per chunk, in arrival order: the A fragments and the group sums
//      (all-ones MFMA), then per tile: unpack, MFMA, per-group scale; then
//      the weight loads of the chunk two ahead go out into the registers
//      this chunk's words and scales leave (a two-chunk ring: with every
//      chunk's loads issued up front, a compute unit's queue of weight
//      requests held back its later waves' activation loads);
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

// Timing build: the wait for chunk j's weights (LPC loads outstanding per
// chunk issued after it: the ring holds chunks j .. j+RD-1); j is a
// constant once the caller's loop is unrolled.
template <int CPW, int LPC, int RD, int J = 0>
__device__ __forceinline__ void stamp_chunk(int j) {
  if constexpr (J < CPW) {
    if (j == J)
      stamp_wait<((J + RD < CPW ? J + RD : CPW) - 1 - J) * LPC>();
    else
      stamp_chunk<CPW, LPC, RD, J + 1>(j);
  }
}

// XS = true: the group sums of x come from a.xsums (qmm_run_sums; written by
// the residual add + RMS norm that produced x) in place of the all-ones
// products: per chunk and group, lane (r, kb) loads the sums of rows
// 4kb .. 4kb+3 (one 16-byte load, issued with the chunk's weights).
template <typename F, int NW, int CPW, int TM, bool GU = false, bool XS = false>
__global__ void __launch_bounds__(NW * 64) resident_kernel(LaunchArgs a) {
  constexpr int BITS = F::kBits, GC = F::kGroups, SPG = F::kSpg;
  constexpr int LPT = F::kCodeLoads + 1;  // loads per (chunk, tile slot)
  constexpr int LPC = TM * LPT + (XS ? GC : 0);  // loads per chunk
  using ST = typename F::St;
  constexpr int TMH = GU ? TM / 2 : TM;  // distinct tiles per workgroup
  static_assert(!GU || TM % 2 == 0, "gate/up slots come in pairs");
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, kg = lane >> 4;
  const int G = gridDim.x, g = blockIdx.x;
  const int nT = a.N / kTileN, nC = a.K / kChunkK;
  WaveStamps ts(a, (long)blockIdx.x * NW + w);  // timing build only
  ts.mark(0);
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

  // 1b. the weight loads of the ring's first chunks, chunk-major
  int tl[TM];
#pragma unroll
  for (int t = 0; t < TM; ++t) {
    const int tile = g + (t % TMH) * G;
    tl[t] = tile < nT ? tile : g;
  }
  const ST* __restrict__ sbp2 = reinterpret_cast<const ST*>(a.sb2);
  constexpr int RD = CPW < kResidentRing ? CPW : kResidentRing;
  // chunk j's words, scales and given sums in ring slot j % RD
  uint32_t W[RD][TM][BITS];
  typename F::Sb SBv[RD][TM];
  f32x4 exv[XS ? RD : 1][GC];
  auto issue = [&](int j) {  // j is a constant once the callers are unrolled
    const int d = j % RD;
    const int c = min(w + j * NW, clast);
    if constexpr (XS) {
#pragma unroll
      for (int g = 0; g < GC; ++g)
        exv[d][g] = *reinterpret_cast<const f32x4*>(a.xsums + (long)(GC * c + g) * a.xsums_ld +
                                                    4 * kg);
    }
#pragma unroll
    for (int t = 0; t < TM; ++t) {
      const bool second = GU && t >= TMH;  // compile-time once unrolled
      const long blk = (long)tl[t] * nC + c;
      F::load(second ? a.codes2 : a.codes, blk, lane, W[d][t]);
      SBv[d][t].load((second ? sbp2 : sbp) + (blk * kTileN + r) * F::kSbElems);
    }
  };
#pragma unroll
  for (int j = 0; j < RD; ++j) {
    issue(j);
    __builtin_amdgcn_sched_barrier(0);  // chunk j's loads issue before chunk j+1's
  }
  ts.mark(1);

  // 2. this wave's activation slices have landed once at most its weight
  //    loads (LPC per chunk in the ring, counted low) are outstanding.  The
  //    wait also drains the LDS counter: until it does, the compiler counts
  //    the LDS-direct loads as pending on both counters and may turn later
  //    weight waits into full ones (vmcnt(0)).
  wait_vm_lds<(RD * LPC < 63 ? RD * LPC : 63)>();
  ts.mark(2);

  // 3. compute in load order; rows past the last one read the last row
  //    (never stored)
  const int xm = min(r, M - 1);
  const int sw = xm & 15;
  const typename F::Masks mask_v = F::masks();
  const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  f32x4 acc[TM];
#pragma unroll
  for (int t = 0; t < TM; ++t) acc[t] = zero;
#pragma unroll
  for (int j = 0; j < CPW; ++j) {
    const bool live = j < count;
    const int c = min(w + j * NW, clast);
    const int d = j % RD;
    stamp_chunk<CPW, LPC, RD>(j);  // timing build: wait for chunk j's weights,
    ts.mark(3 + j);                // then stamp their arrival
    const u32x4* xrow = reinterpret_cast<const u32x4*>(lds + (size_t)c * M * 256) + xm * 16;
    u32x4 A[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) A[q] = xrow[F::a_vec(q, kg) ^ sw];
    __builtin_amdgcn_sched_barrier(0);
    f32x4 ex[GC];
#pragma unroll
    for (int g = 0; g < GC; ++g) {
      if constexpr (XS) {
        ex[g] = exv[d][g];
      } else {
        f32x4 e = zero;
#pragma unroll
        for (int u = 0; u < SPG; ++u)
          e = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, A[g * SPG + u]),
                                                      __builtin_bit_cast(bf16x8, ones), e, 0, 0, 0);
        ex[g] = e;
      }
    }
#pragma unroll
    for (int t = 0; t < TM; ++t) {
      uint32_t P[16];
      F::unpack(W[d][t], P, mask_v);
#pragma unroll
      for (int g = 0; g < GC; ++g) {
        f32x4 dd = zero;
#pragma unroll
        for (int u = 0; u < SPG; ++u) {
          const int st = g * SPG + u;
          const u32x4 B = {P[4 * st], P[4 * st + 1], P[4 * st + 2], P[4 * st + 3]};
          dd = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, A[st]),
                                                       __builtin_bit_cast(bf16x8, B), dd, 0, 0, 0);
        }
        const Affine af = F::affine(g, SBv[d][t]);
        const float sc = live ? af.sc : 0.f, bp = live ? af.bp : 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[t][q] = fmaf(sc, dd[q], fmaf(bp, ex[g][q], acc[t][q]));
      }
    }
    if (j + RD < CPW) issue(j + RD);  // into the slot chunk j leaves
    __builtin_amdgcn_sched_barrier(0);
  }

  ts.mark(12);
  // 4. add the NW partial tiles of each tile in wave order (slices are dead)
  __syncthreads();
  ts.mark(13);
  f32x4* red = reinterpret_cast<f32x4*>(lds);  // [TM][NW][64]
#pragma unroll
  for (int t = 0; t < TM; ++t) red[(t * NW + w) * 64 + lane] = acc[t];
  __syncthreads();
  if (w >= TMH || g + w * G >= nT) {
    ts.flush(lane);
    return;
  }
  const int tile = g + w * G;
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
    if (m < M) store_y<false>(a, (long)m * a.ldy + n, v[q]);
  }
  ts.mark(14);
  ts.flush(lane);
}

// (waves, chunks per wave, tile slots) shapes of the resident kernel.  The
// 16-wave shapes cover 65..128 chunks (K up to 16384, a few rows): 10.3 us
// against 10.7 us for the streaming kernel on the 4-bit 15360 -> 3840
// projection at 4 rows (eight waves of 15 chunks: 11.6 us).
#define QMM_RESIDENT_SHAPES(X)                                                               \
  X(4, 2, 1) X(4, 2, 2) X(4, 2, 3) X(4, 2, 4) X(4, 4, 1) X(4, 4, 2) X(4, 4, 3) X(4, 4, 4)     \
  X(8, 4, 1) X(8, 4, 2) X(8, 4, 3) X(8, 4, 4) X(8, 5, 1) X(8, 5, 2) X(8, 5, 3) X(8, 5, 4)     \
  X(8, 8, 1) X(8, 8, 2) X(16, 8, 1) X(16, 8, 2)

// Step-layout formats: the built shapes whose weight registers fit.
template <typename F>
static bool resident_pick(int nC, int tm, int* nw, int* cpw) {
  // the fewest chunks per wave that cover K: four waves below 16 chunks
  int best_w = 0, best_c = 0;
#define QMM_PICK(W, C, T)                                                                  \
  if (T == tm && (nC < 16) == (W == 4) && W * C >= nC && F::resident_fits(W, C, T) &&     \
      (best_c == 0 || C < best_c)) {                                                      \
    best_w = W;                                                                           \
    best_c = C;                                                                           \
  }
  QMM_RESIDENT_SHAPES(QMM_PICK)
#undef QMM_PICK
  *nw = best_w;
  *cpw = best_c;
  return best_c > 0;
}

bool resident_shape(int bits, int step_gs, int nC, int tm, int* nw, int* cpw) {
  if (step_gs) {
#define QMM_STEP(B, GS) \
  if (bits == B && step_gs == GS) return resident_pick<StepFmt<B, GS>>(nC, tm, nw, cpw);
    QMM_STEP_FORMATS(QMM_STEP)
#undef QMM_STEP
    *nw = *cpw = 0;
    return false;
  }
  return resident_pick<NativeFmt<4, uint16_t>>(nC, tm, nw, cpw);
}

int resident_rows(int M) { return std::min(M, 16); }

size_t resident_lds_bytes(int nw, int tm, int M, int K) {
  return std::max((size_t)resident_rows(M) * K * 2, (size_t)tm * nw * 64 * 16);
}

// Shapes built with given group sums: eight waves or fewer, and at most 48
// registers of sums (4 * GC per chunk of the ring); other shapes form their
// own sums.
template <typename F, bool XS>
constexpr bool resident_built(int nw, int cpw, int tm) {
  return F::resident_fits(nw, cpw, tm) &&
         (!XS || (nw <= 8 && (cpw < kResidentRing ? cpw : kResidentRing) * F::kGroups * 4 <= 48));
}

template <typename F>
static bool resident_xs_shape(int nw, int cpw, int tm) {
#define QMM_HAS(W, C, T) \
  if (nw == W && cpw == C && tm == T) return resident_built<F, true>(W, C, T);
  QMM_RESIDENT_SHAPES(QMM_HAS)
#undef QMM_HAS
  return false;
}

template <typename F, bool XS>
static hipError_t resident_dispatch_xs(int nw, int cpw, int tm, const LaunchArgs& a, int grid,
                                       size_t lds, hipStream_t st) {
#define QMM_GO(W, C, T)                                                                       \
  if constexpr (resident_built<F, XS>(W, C, T)) {                                             \
    if (nw == W && cpw == C && tm == T) {                                                     \
      auto* kfn = &resident_kernel<F, W, C, T, false, XS>;                                               \
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kfn),                  \
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds); \
      if (e != hipSuccess) return e;                                                          \
      kfn<<<grid, W * 64, lds, st>>>(a);                                                      \
      return hipGetLastError();                                                               \
    }                                                                                         \
  }
  QMM_RESIDENT_SHAPES(QMM_GO)
#undef QMM_GO
  return hipErrorInvalidValue;
}

template <typename F>
static hipError_t resident_dispatch(int nw, int cpw, int tm, const LaunchArgs& a, int grid,
                                    size_t lds, hipStream_t st) {
  if (a.xsums && resident_xs_shape<F>(nw, cpw, tm))
    return resident_dispatch_xs<F, true>(nw, cpw, tm, a, grid, lds, st);
  LaunchArgs b = a;
  b.xsums = nullptr;
  return resident_dispatch_xs<F, false>(nw, cpw, tm, b, grid, lds, st);
}

hipError_t launch_resident(int bits, int step_gs, bool sb_f32, int nw, int cpw, int tm,
                           const LaunchArgs& a, int grid, size_t lds_bytes, hipStream_t st) {
  if (step_gs) {
#define QMM_STEP(B, GS)                \
  if (bits == B && step_gs == GS) \
    return resident_dispatch<StepFmt<B, GS>>(nw, cpw, tm, a, grid, lds_bytes, st);
    QMM_STEP_FORMATS(QMM_STEP)
#undef QMM_STEP
    return hipErrorInvalidValue;
  }
  if (bits == 3)
    return sb_f32 ? resident_dispatch<NativeFmt<3, float>>(nw, cpw, tm, a, grid, lds_bytes, st)
                  : resident_dispatch<NativeFmt<3, uint16_t>>(nw, cpw, tm, a, grid, lds_bytes, st);
  return sb_f32 ? resident_dispatch<NativeFmt<4, float>>(nw, cpw, tm, a, grid, lds_bytes, st)
                : resident_dispatch<NativeFmt<4, uint16_t>>(nw, cpw, tm, a, grid, lds_bytes, st);
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
    auto* kfn = &resident_kernel<NativeFmt<BITS, ST>, W, C, 2 * P, true>;                              \
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

}  // namespace qmm
