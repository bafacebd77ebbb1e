// qmm_norm.hip -- residual add + RMS normalization producing the activations
// a projection consumes (page "@mlx-bun/inference 0.0.0-stage -> 1.0.0",
// diffend npm page 53, residual-rms-norm.ts).
//
// For each row of D values, with T the storage type (bf16 or f32) and R the
// rounding to T:
//   residual[i]   = R(x[i] + update[i])                (f32 sum, rounded)
//   inv           = 1 / sqrt(sum_i residual[i]^2 / D + eps)   (f32)
//   normalized[i] = R(weight[i] * R(residual[i] * inv))
// The roundings sit where an add followed by an RMS norm in T would put them:
// the residual sum is rounded before it is squared, the normalized value
// before the weight multiplies it, and the weighted product is stored in T.
//
// With group sums (GL > 0 lanes per group of 8*GL values) the kernel also
// writes, per row m and group g, the f32 sum of the group's stored
// normalized values to sums[g * ld + m]: the per-group sum of x that the
// projection's factored form needs for the bias term (the same page's
// affine3-rows.ts header: s * sum(q x) + b * sum(x)), formed here while the
// values are in registers.  Each thread adds its 8 values in order, then the
// GL threads of a group add their partial sums by lane swaps (fixed order).
//
// gfx950 design: one workgroup of 256 threads per row; each thread owns
// 8-value vectors (16 bytes of bf16) spread over the row.  The rounded
// residuals stay in registers between the two passes (no second read); the
// sum of squares is reduced by lane exchanges within each wave and 4 LDS
// words across the waves.  HBM-bound: 2 reads and 2 writes of D values per
// row, plus the weight vector (cached).  Loading the weight vectors with the
// row instead (ahead of the reduction) measured no faster at 4 rows and
// slower at 16384 (more registers per thread).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qmm_internal.h"

namespace qmm {

namespace {

constexpr int kNormThreads = 256;
constexpr int kNormMaxVecs = 8;  // vectors of 8 values per thread: D <= 16384

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u) return (u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;  // round to nearest, ties to even
}

template <bool BF16>
struct Vec8 {
  float v[8];
  __device__ __forceinline__ void load(const void* base, long i8) {
    if constexpr (BF16) {
      const uint4 w = reinterpret_cast<const uint4*>(base)[i8];
      const uint32_t d[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[2 * e] = bf16_bits_to_f32(d[e] & 0xFFFFu);
        v[2 * e + 1] = bf16_bits_to_f32(d[e] >> 16);
      }
    } else {
      const float4 a = reinterpret_cast<const float4*>(base)[2 * i8];
      const float4 b = reinterpret_cast<const float4*>(base)[2 * i8 + 1];
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
      v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
  }
  __device__ __forceinline__ void store(void* base, long i8) const {
    if constexpr (BF16) {
      uint4 w;
      w.x = f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16);
      w.y = f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16);
      w.z = f32_to_bf16_bits(v[4]) | (f32_to_bf16_bits(v[5]) << 16);
      w.w = f32_to_bf16_bits(v[6]) | (f32_to_bf16_bits(v[7]) << 16);
      reinterpret_cast<uint4*>(base)[i8] = w;
    } else {
      reinterpret_cast<float4*>(base)[2 * i8] = make_float4(v[0], v[1], v[2], v[3]);
      reinterpret_cast<float4*>(base)[2 * i8 + 1] = make_float4(v[4], v[5], v[6], v[7]);
    }
  }
};

template <bool BF16>
__device__ __forceinline__ float round_t(float v) {
  if constexpr (BF16) return bf16_bits_to_f32(f32_to_bf16_bits(v));
  return v;
}

// Sum over the 64 lanes of a wave, then over the 4 waves through LDS.
__device__ __forceinline__ float block_sum(float s, float* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = s;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < kNormThreads / 64; ++i) t += red[i];  // fixed order
  return t;
}

template <bool BF16, int NV, int GL>
__global__ void __launch_bounds__(kNormThreads) residual_rms_norm_kernel(
    const void* __restrict__ x, const void* __restrict__ update, const void* __restrict__ weight,
    void* __restrict__ residual, void* __restrict__ normalized, int D, float eps,
    float* __restrict__ sums, int ld) {
  __shared__ float red[kNormThreads / 64];
  const int row = blockIdx.x;
  const int nv = D / 8;  // 8-value vectors per row
  const long base = (long)row * nv;
  Vec8<BF16> r[NV];
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int v = threadIdx.x + j * kNormThreads;
    if (v < nv) {
      Vec8<BF16> a, b;
      a.load(x, base + v);
      b.load(update, base + v);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        r[j].v[e] = round_t<BF16>(a.v[e] + b.v[e]);
        acc = fmaf(r[j].v[e], r[j].v[e], acc);
      }
      r[j].store(residual, base + v);
    }
  }
  const float ss = block_sum(acc, red);
  const float inv = 1.0f / sqrtf(ss / (float)D + eps);
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int v = threadIdx.x + j * kNormThreads;
    float gsum = 0.f;
    if (v < nv) {
      Vec8<BF16> wv, o;
      wv.load(weight, v);  // L2-resident after the first rows
#pragma unroll
      for (int e = 0; e < 8; ++e) o.v[e] = wv.v[e] * round_t<BF16>(r[j].v[e] * inv);
      o.store(normalized, base + v);  // rounded to T by the store
      if constexpr (GL > 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) gsum += round_t<BF16>(o.v[e]);  // the stored values
      }
    }
    if constexpr (GL > 0) {
      // every lane takes part in the swaps; a group lies wholly below or
      // above the row's end (D is a multiple of the group size)
      if (j * kNormThreads < nv) {  // block-uniform
#pragma unroll
        for (int off = 1; off < GL; off <<= 1) gsum += __shfl_xor(gsum, off);
        if (v < nv && (v & (GL - 1)) == 0) sums[(long)(v / GL) * ld + row] = gsum;
      }
    }
  }
}

template <bool BF16, int GL>
hipError_t norm_dispatch(const void* x, const void* u, const void* w, void* res, void* out,
                         int rows, int D, float eps, float* sums, int ld, hipStream_t st) {
  const int nv = D / 8;
  const int per = (nv + kNormThreads - 1) / kNormThreads;
#define QMM_NV(N)                                                                         \
  if (per <= N) {                                                                         \
    residual_rms_norm_kernel<BF16, N, GL><<<rows, kNormThreads, 0, st>>>(x, u, w, res, out, D, \
                                                                        eps, sums, ld);   \
    return hipGetLastError();                                                             \
  }
  QMM_NV(1) QMM_NV(2) QMM_NV(4) QMM_NV(8)
#undef QMM_NV
  return hipErrorInvalidValue;
}

template <bool BF16>
hipError_t norm_dispatch_gs(const void* x, const void* u, const void* w, void* res, void* out,
                            int rows, int D, float eps, float* sums, int group_size, int ld,
                            hipStream_t st) {
  if (!sums) return norm_dispatch<BF16, 0>(x, u, w, res, out, rows, D, eps, nullptr, 0, st);
  if (group_size == 32) return norm_dispatch<BF16, 4>(x, u, w, res, out, rows, D, eps, sums, ld, st);
  if (group_size == 64) return norm_dispatch<BF16, 8>(x, u, w, res, out, rows, D, eps, sums, ld, st);
  if (group_size == 128)
    return norm_dispatch<BF16, 16>(x, u, w, res, out, rows, D, eps, sums, ld, st);
  return hipErrorInvalidValue;
}

}  // namespace

bool residual_rms_norm_supported(long D) {
  return D >= 8 && D % 8 == 0 && D / 8 <= (long)kNormThreads * kNormMaxVecs;
}

hipError_t launch_residual_rms_norm(bool bf16, const void* x, const void* update,
                                    const void* weight, void* residual, void* normalized,
                                    int rows, int D, float eps, float* sums, int group_size,
                                    int sums_ld, hipStream_t st) {
  if (bf16)
    return norm_dispatch_gs<true>(x, update, weight, residual, normalized, rows, D, eps, sums,
                                  group_size, sums_ld, st);
  return norm_dispatch_gs<false>(x, update, weight, residual, normalized, rows, D, eps, sums,
                                 group_size, sums_ld, st);
}

}  // namespace qmm
