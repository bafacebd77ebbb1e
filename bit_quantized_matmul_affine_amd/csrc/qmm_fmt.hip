// qmm_fmt.hip -- the one-time loader (MLX layout -> step layout) and the test
// decoder of the other affine formats: 2- and 8-bit weights with groups of
// 32, 64 or 128 values, 3- and 4-bit weights with groups of 32 (the layout
// and its B operands: StepFmt in qmm_formats.h).  Their products run on the
// streaming and resident kernels.
//
// [P1] = page "@mlx-bun/inference 0.0.0-stage -> 1.0.0": affine-split-mma.ts
// (MLX's LSB-first packing of the codes of a row, scales and biases per
// group); [P3] = page "mlx-bun 0.0.4", fused-decode-kernel.ts (widths 4 and 8,
// groups of 32, 64 and 128).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "qmm_formats.h"

namespace qmm {

namespace {

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

// One thread per (block, lane): the lane's 32 codes and, for kb = 0, its
// row's scales and biases of the block.
template <int BITS, int GS>
__global__ void __launch_bounds__(256) repack_fmt_kernel(const uint32_t* __restrict__ w,
                                                         const uint16_t* __restrict__ scales,
                                                         const uint16_t* __restrict__ biases,
                                                         uint32_t* __restrict__ codes,
                                                         uint16_t* __restrict__ sb, int N, int K) {
  using F = StepFmt<BITS, GS>;
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
    F::place(out, e, mlx_code_any<BITS>(row, (long)kChunkK * c + 32 * (e >> 3) + 8 * kb + (e & 7)));
#pragma unroll
  for (int j = 0; j < BITS; ++j) codes[F::word(blk, lane, j)] = out[j];
  if (kb == 0) {
    constexpr int Gc = F::kGroups;
    const int G = K / GS;
    uint16_t* d = sb + (blk * kTileN + r) * F::kSbElems;
#pragma unroll
    for (int q = 0; q < Gc; ++q) {
      d[q] = scales[(long)n * G + (long)Gc * c + q];
      d[Gc + q] = biases[(long)n * G + (long)Gc * c + q];
    }
  }
}

// Test decoder: the codes as the kernels' B operands see them (value minus
// the offset), written to out[n*K + k].
template <int BITS>
__global__ void __launch_bounds__(256) debug_unpack_fmt_kernel(const uint32_t* __restrict__ codes,
                                                               uint8_t* __restrict__ out, int N,
                                                               int K) {
  using F = StepFmt<BITS, 32>;  // the code layout does not depend on the group size
  const long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const int nC = K / kChunkK, nT = N / kTileN;
  if (gid >= (long)nT * nC * 64) return;
  const int lane = (int)(gid & 63);
  const long blk = gid >> 6;
  const int c = (int)(blk % nC), tile = (int)(blk / nC);
  const int r = lane & 15, kb = lane >> 4, n = tile * kTileN + r;
  uint32_t w[BITS], P[16];
#pragma unroll
  for (int j = 0; j < BITS; ++j) w[j] = codes[F::word(blk, lane, j)];
  F::unpack(w, P, F::masks());
#pragma unroll
  for (int p = 0; p < 16; ++p) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int e = 2 * p + h;
      const float val = bf16_to_f32(h ? P[p] >> 16 : P[p] & 0xFFFFu) - F::kOffset;
      out[(long)n * K + (long)kChunkK * c + 32 * (e >> 3) + 8 * kb + (e & 7)] = (uint8_t)val;
    }
  }
}

inline unsigned blocks_for(long threads, int per) {
  return (unsigned)((threads + per - 1) / per);
}

}  // namespace

bool fmt_format(int bits, int group_size) {
#define QMM_IS(B, GS) \
  if (bits == B && group_size == GS) return true;
  QMM_STEP_FORMATS(QMM_IS)
#undef QMM_IS
  return false;
}

int fmt_rows(long K) {
  const long r = (long)kMaxLdsBytes / (K * 2);
  return (int)std::min(r, 16L);
}

hipError_t launch_repack_fmt(int bits, int group_size, const uint32_t* w, const void* scales,
                             const void* biases, uint32_t* codes, void* sb, int N, int K,
                             hipStream_t st) {
  const unsigned grid = blocks_for((long)(N / kTileN) * (K / kChunkK) * 64, 256);
  const uint16_t* s = static_cast<const uint16_t*>(scales);
  const uint16_t* bb = static_cast<const uint16_t*>(biases);
  uint16_t* d = static_cast<uint16_t*>(sb);
#define QMM_REPACK(B, GS)                                                            \
  if (bits == B && group_size == GS) {                                               \
    repack_fmt_kernel<B, GS><<<grid, 256, 0, st>>>(w, s, bb, codes, d, N, K);        \
    return hipGetLastError();                                                        \
  }
  QMM_STEP_FORMATS(QMM_REPACK)
#undef QMM_REPACK
  return hipErrorInvalidValue;
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
