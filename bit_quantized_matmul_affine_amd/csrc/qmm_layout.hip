// qmm_layout.hip -- the one-time loader (MLX layout -> native layout), the
// test decoder of the native layout, and the HBM read probe.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "qmm_device.h"

namespace qmm {

// ---------------------------------------------------------------------------
// One-time loader and the test decoder.
// ---------------------------------------------------------------------------

template <int BITS, typename ST>
__global__ void __launch_bounds__(256) repack_kernel(const uint32_t* __restrict__ w,
                                                     const ST* __restrict__ scales,
                                                     const ST* __restrict__ biases,
                                                     uint32_t* __restrict__ codes,
                                                     ST* __restrict__ sb, int N, int K,
                                                     int gs) {
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
    // the groups of the chunk's two 64-value halves (one group of 128 serves both)
    const int G = K / gs;
    const long g0 = (long)n * G + (long)kChunkK * c / gs, g1 = (long)n * G + (kChunkK * c + 64) / gs;
    ST* e = sb + (blk * kTileN + r) * 4;
    e[0] = scales[g0];
    e[1] = scales[g1];
    e[2] = biases[g0];
    e[3] = biases[g1];
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

hipError_t launch_repack(int bits, int gs, bool sb_f32, const uint32_t* w, const void* scales,
                         const void* biases, uint32_t* codes, void* sb, int N, int K,
                         hipStream_t st) {
  const long threads = (long)(N / kTileN) * (K / kChunkK) * 64;
  const unsigned grid = blocks_for(threads, 256);
  if (bits == 3 && !sb_f32)
    repack_kernel<3, uint16_t><<<grid, 256, 0, st>>>(w, (const uint16_t*)scales, (const uint16_t*)biases, codes, (uint16_t*)sb, N, K, gs);
  else if (bits == 3)
    repack_kernel<3, float><<<grid, 256, 0, st>>>(w, (const float*)scales, (const float*)biases, codes, (float*)sb, N, K, gs);
  else if (!sb_f32)
    repack_kernel<4, uint16_t><<<grid, 256, 0, st>>>(w, (const uint16_t*)scales, (const uint16_t*)biases, codes, (uint16_t*)sb, N, K, gs);
  else
    repack_kernel<4, float><<<grid, 256, 0, st>>>(w, (const float*)scales, (const float*)biases, codes, (float*)sb, N, K, gs);
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

hipError_t launch_probe(const void* buf, size_t bytes, uint32_t* sink, int grid, hipStream_t st) {
  probe_kernel<<<grid, 256, 0, st>>>(reinterpret_cast<const u32x4*>(buf), (long)(bytes / 16), sink);
  return hipGetLastError();
}

}  // namespace qmm
