// qmm_generic.hip -- the affine format variants: bits 2, 3, 4, 8 with groups
// of 32, 64 or 128 values ("@mlx-bun/inference 0.0.0-stage -> 1.0.0" page,
// affine-split-mma.ts: MLX affine weights, w = s * q + b per group; the
// hot-path kernels are built for 3- and 4-bit group-64 weights, the other
// MLX widths and group sizes run here).
//
// The weights stay in MLX's layout: row n is K*bits/32 uint32 words, codes
// packed least significant bits first (a 3-bit code may straddle two
// words); scales and biases are two planes [N, K/gs] (scales, then biases).
//
// gfx950 design (a vector-ALU kernel for the decode regime): a workgroup of
// four waves owns 8 rows of W, each wave 2 of them; lane l takes the
// 32-value slices k0 = 32 l, 32 l + 2048, ... of K (a slice lies in one
// group because every group size is a multiple of 32, and is `bits` whole
// words).  Per slice a lane loads its activation slices of up to MR rows
// (f32 in registers, with their sums), then for each of its 4 W rows the
// slice's words, scale and bias, converts the 32 codes to floats (one
// v_cvt_f32_ubyteN per code for 2-, 4- and 8-bit codes, on byte planes of
// the word) and accumulates s * sum q x + b * sum x.  Lanes are added by a
// fixed butterfly: the result is bitwise reproducible.  Measured at 1 row of
// 5120 -> 10240: two W rows per wave (eight per workgroup) beat four (more
// waves hide the load latency of each slice pass); the offset-128 bf16 pair
// form of 2- and 4-bit codes with v_dot2_f32_bf16 was slower here than the
// byte-plane conversion, the kernel being bound by load latency, not by its
// vector instructions.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qmm_internal.h"

namespace qmm {

namespace {

constexpr int kGenThreads = 256;
constexpr int kGenRowsPerWave = 2;
constexpr int kGenSlice = 32;  // values per lane slice

// f32 -> bf16 bits, round to nearest even (NaN stays a quiet NaN).
__device__ __forceinline__ uint16_t to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint32_t opaque(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

// The `bits` words of a lane's 32-value slice.
template <int BITS>
__device__ __forceinline__ void load_slice(const uint32_t* __restrict__ p, uint32_t* w) {
  if constexpr (BITS == 2) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    w[0] = v.x;
    w[1] = v.y;
  } else if constexpr (BITS == 3) {
    w[0] = p[0];
    w[1] = p[1];
    w[2] = p[2];
  } else {
#pragma unroll
    for (int i = 0; i < BITS / 4; ++i) {
      const uint4 v = reinterpret_cast<const uint4*>(p)[i];
      w[4 * i] = v.x;
      w[4 * i + 1] = v.y;
      w[4 * i + 2] = v.z;
      w[4 * i + 3] = v.w;
    }
  }
}

// Codes 0..31 of a slice as floats, in K order.
template <int BITS>
__device__ __forceinline__ void decode_slice(const uint32_t* w, float* c) {
  if constexpr (BITS == 3) {
    // code i sits at bit 3i of the 96-bit little-endian stream
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const int b = 3 * i, j = b >> 5, s = b & 31;
      uint32_t v = w[j] >> s;
      if (s > 29) v |= w[j + 1] << (32 - s);
      c[i] = (float)(v & 7u);
    }
  } else {
    // byte plane t of word j holds codes (32/BITS) j + (8/BITS) byte + t
    constexpr int PER = 32 / BITS, PLANES = 8 / BITS;
    constexpr uint32_t MASK = BITS == 8 ? 0xFFFFFFFFu : (BITS == 4 ? 0x0F0F0F0Fu : 0x03030303u);
#pragma unroll
    for (int j = 0; j < BITS; ++j) {
#pragma unroll
      for (int t = 0; t < PLANES; ++t) {
        const uint32_t plane = BITS == 8 ? w[j] : opaque((w[j] >> (BITS * t)) & MASK);
#pragma unroll
        for (int byte = 0; byte < 4; ++byte)
          c[PER * j + PLANES * byte + t] = (float)((plane >> (8 * byte)) & 0xFFu);
      }
    }
  }
}

template <bool XF>
__device__ __forceinline__ void load_x_slice(const void* x, long idx, float* v) {
  if constexpr (XF) {
    const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + idx);
#pragma unroll
    for (int i = 0; i < kGenSlice / 4; ++i) {
      const float4 f = p[i];
      v[4 * i] = f.x;
      v[4 * i + 1] = f.y;
      v[4 * i + 2] = f.z;
      v[4 * i + 3] = f.w;
    }
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(x) + idx);
#pragma unroll
    for (int i = 0; i < kGenSlice / 8; ++i) {
      const uint4 u = p[i];
      const uint32_t d[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[8 * i + 2 * e] = __uint_as_float(d[e] << 16);
        v[8 * i + 2 * e + 1] = __uint_as_float(d[e] & 0xFFFF0000u);
      }
    }
  }
}

template <bool SF>
__device__ __forceinline__ float load_sb(const void* sb, long idx) {
  if constexpr (SF) return reinterpret_cast<const float*>(sb)[idx];
  return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(sb)[idx] << 16);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

template <int BITS, bool XF, bool SF, int MR>
__global__ void __launch_bounds__(kGenThreads) generic_kernel(LaunchArgs a, int gs_shift) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int K = a.K, N = a.N, M = a.M;
  const int G = K >> gs_shift;
  const int rw = K * BITS / 32;  // words per W row
  const int n0 = blockIdx.x * (4 * kGenRowsPerWave) + wave * kGenRowsPerWave;
  const long plane = (long)N * G;  // biases follow the scales
  float acc[kGenRowsPerWave][MR];
#pragma unroll
  for (int j = 0; j < kGenRowsPerWave; ++j)
#pragma unroll
    for (int m = 0; m < MR; ++m) acc[j][m] = 0.f;
  for (int k0 = lane * kGenSlice; k0 < K; k0 += 64 * kGenSlice) {
    float xv[MR][kGenSlice], xs[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      load_x_slice<XF>(a.x, (long)min(m, M - 1) * a.ldx + k0, xv[m]);
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < kGenSlice; ++i) s += xv[m][i];
      xs[m] = s;
    }
    const int g = k0 >> gs_shift;
#pragma unroll
    for (int j = 0; j < kGenRowsPerWave; ++j) {
      const int n = n0 + j;
      uint32_t w[BITS];
      load_slice<BITS>(a.codes + (long)n * rw + k0 / 32 * BITS, w);
      const float s = load_sb<SF>(a.sb, (long)n * G + g);
      const float b = load_sb<SF>(a.sb, plane + (long)n * G + g);
      float c[kGenSlice];
      decode_slice<BITS>(w, c);
#pragma unroll
      for (int m = 0; m < MR; ++m) {
        float d = 0.f;
#pragma unroll
        for (int i = 0; i < kGenSlice; ++i) d = fmaf(c[i], xv[m][i], d);
        acc[j][m] = fmaf(s, d, fmaf(b, xs[m], acc[j][m]));
      }
    }
  }
#pragma unroll
  for (int j = 0; j < kGenRowsPerWave; ++j)
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      const float v = wave_sum(acc[j][m]);
      if (lane == 0 && m < M) {
        const long idx = (long)m * a.ldy + n0 + j;
        if (XF || a.y_f32)
          reinterpret_cast<float*>(a.y)[idx] = v;
        else
          reinterpret_cast<uint16_t*>(a.y)[idx] = to_bf16(v);
      }
    }
}

template <int BITS>
hipError_t generic_dispatch(bool xf, bool sf, int mr, const LaunchArgs& a, int gs_shift,
                            hipStream_t st) {
  const int grid = a.N / (4 * kGenRowsPerWave);
#define QMM_GEN(XF, SF, MR)                                                           \
  if (xf == XF && sf == SF && mr == MR) {                                             \
    generic_kernel<BITS, XF, SF, MR><<<grid, kGenThreads, 0, st>>>(a, gs_shift);      \
    return hipGetLastError();                                                         \
  }
  QMM_GEN(false, false, 1) QMM_GEN(false, false, 2) QMM_GEN(false, true, 1)
  QMM_GEN(false, true, 2) QMM_GEN(true, false, 1) QMM_GEN(true, false, 2)
  QMM_GEN(true, true, 1) QMM_GEN(true, true, 2)
#undef QMM_GEN
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_generic(int bits, int group_size, bool x_f32, bool sb_f32, int rows,
                          const LaunchArgs& a, hipStream_t st) {
  const int gs_shift = group_size == 32 ? 5 : (group_size == 64 ? 6 : 7);
  const int mr = rows <= 1 ? 1 : 2;
  switch (bits) {
    case 2: return generic_dispatch<2>(x_f32, sb_f32, mr, a, gs_shift, st);
    case 3: return generic_dispatch<3>(x_f32, sb_f32, mr, a, gs_shift, st);
    case 4: return generic_dispatch<4>(x_f32, sb_f32, mr, a, gs_shift, st);
    case 8: return generic_dispatch<8>(x_f32, sb_f32, mr, a, gs_shift, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qmm
