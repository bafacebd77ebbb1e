// qmm_internal.h -- declarations shared by the C-ABI front end (qmm_api.cpp)
// and the HIP kernels (qmm_*.hip).  Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmm {

// Kernel-native tiling.  One wavefront multiplies a block of 16 rows of W by
// 128 columns (two quantization groups) per step.
constexpr int kTileN = 16;
constexpr int kChunkK = 128;
constexpr int kWaves = 4;            // wavefronts per workgroup
constexpr int kBlockThreads = 64 * kWaves;
constexpr int kMaxMfmaRows = 64;     // rows per MFMA launch (4 tiles of 16)
constexpr int kMaxGemvRows = 8;      // rows per vector-ALU launch

struct LaunchArgs {
  const void* x;          // [M, K] activations (x_dtype)
  const uint32_t* codes;  // native packed codes
  const void* sb;         // native packed scales/biases (sb_dtype)
  void* y;                // [M, N] output (x_dtype)
  float* part;            // [S, M, N] split-K partials (S > 1)
  uint32_t* tickets;      // one counter per tile block (S > 1)
  int M, N, K;
  int S;                  // K splits
  int nTB;                // tile blocks (kWaves * ntw tiles each)
  int ldx, ldy;           // row strides of x and y in elements
  const uint32_t* codes2; // fused gate/up: the up projection's codes (codes = gate)
  const void* sb2;        // fused gate/up: the up projection's scales/biases
  int y_f32;              // 1: y is f32 whatever x's dtype (QMM_FLAG_F32_OUT)
  const float* xsums;     // null, or the group sums of x: [K/group][xsums_ld] (qmm_run_sums)
  int xsums_ld;
};

// All launchers return hipSuccess or the launch error.
// Native layout (3- and 4-bit codes, groups of 64 or 128 values): a group of
// 128 gives both 64-value halves of a chunk its scale and bias.
hipError_t launch_repack(int bits, int group_size, bool sb_f32, const uint32_t* w,
                         const void* scales, const void* biases, uint32_t* codes, void* sb, int N,
                         int K, hipStream_t st);
hipError_t launch_debug_unpack(int bits, const uint32_t* codes, uint8_t* out, int N, int K,
                               hipStream_t st);
hipError_t launch_mfma(int bits, bool sb_f32, int mt, int ntw, int wk, const LaunchArgs& a,
                       hipStream_t st);
hipError_t launch_gemv(int bits, bool x_f32, bool sb_f32, int mr, int ntw, const LaunchArgs& a,
                       size_t lds_bytes, hipStream_t st);
// The streaming and resident kernels run the native layout (step_gs = 0:
// 3- and 4-bit codes, bf16 or f32 scales) and the step layout of the other
// formats (step_gs = the group size; bf16 scales; see fmt_format).
hipError_t launch_stream(int bits, int step_gs, bool sb_f32, int nw, int cpw, const LaunchArgs& a,
                         size_t lds_bytes, hipStream_t st);
// The streaming kernel's vector-ALU form (v_dot2_f32_bf16 on the same
// operands, lane quarters added by cross-lane swaps) on the native layout.
hipError_t launch_stream_valu(int bits, bool sb_f32, int nw, int cpw, const LaunchArgs& a,
                              size_t lds_bytes, hipStream_t st);
// Rows the streaming kernel takes per launch (its waves stage every row of
// their own chunks' activation slices in registers on the way to LDS).
constexpr int kStreamMaxRows = 4;
// LDS of the streaming kernel with `groups` quantization groups per chunk.
size_t stream_lds_bytes(int nw, int cpw, int M, int groups);
// Whether M rows fit the streaming kernel (M <= kStreamMaxRows and at most
// max_lds bytes of LDS for NW waves of at most cpw chunks).
bool stream_fits(int nw, int cpw, int M, int groups, size_t max_lds);
// Whether the streaming kernel is built for a step-layout format at this
// (waves, chunks per wave): the wave's weight registers must fit.
bool stream_step_fits(int bits, int group_size, int nw, int cpw);
hipError_t launch_resident(int bits, int step_gs, bool sb_f32, int nw, int cpw, int tm,
                           const LaunchArgs& a, int grid, size_t lds_bytes, hipStream_t st);
// Resident kernel: the built (waves, chunks per wave) for `tm` tile slots
// that covers nC chunks of K (false if none does), and its dynamic LDS bytes
// for M rows (the activation block, reused for the partial tiles).
bool resident_shape(int bits, int step_gs, int nC, int tm, int* nw, int* cpw);
// Rows of LDS a block of M rows takes (M, at most 16 per launch).
int resident_rows(int M);
size_t resident_lds_bytes(int nw, int tm, int M, int K);
constexpr int kResidentMaxSlots = 4;
// Residual add + RMS normalization (qmm_norm.hip): D a multiple of 8, at most
// 16384.
// Format variants (bits 2, 3, 4, 8; groups of 32, 64, 128) on MLX's own
// layout: codes as given, scales then biases as two [N, K/gs] planes; up to
// kGenericMaxRows activation rows per launch; N a multiple of 16.
constexpr int kGenericMaxRows = 2;
hipError_t launch_generic(int bits, int group_size, bool x_f32, bool sb_f32, int rows,
                          const LaunchArgs& a, hipStream_t st);

// Step layout of the other formats (qmm_formats.h, qmm_fmt.hip): 2- and
// 8-bit codes with groups of 32, 64 or 128, 3- and 4-bit codes with groups of
// 32; bf16 activations and bf16 scales/biases.  They run on the streaming
// and resident kernels; the resident kernel takes fmt_rows(K) rows per
// launch (at most 16, their activation block in one compute unit's LDS).
bool fmt_format(int bits, int group_size);
int fmt_rows(long K);
hipError_t launch_repack_fmt(int bits, int group_size, const uint32_t* w, const void* scales,
                             const void* biases, uint32_t* codes, void* sb, int N, int K,
                             hipStream_t st);
hipError_t launch_debug_unpack_fmt(int bits, const uint32_t* codes, uint8_t* out, int N, int K,
                                   hipStream_t st);

// Decode attention over an affine-quantized KV cache: kAttnBlock cached rows
// per workgroup of the block kernel; partial outputs [H, G, D] and
// (max, sum) pairs [H, G, 2] of G = ceil(N / kAttnBlock) blocks in the
// workspace when G > 1.
constexpr int kAttnBlock = 256;
constexpr int kAttnMaxBlocks = 8192;  // merge weights in LDS: 32 KB
struct AttnArgs {
  const void* q;         // bf16 [H, D]
  const uint32_t* kw;    // [KV, N, D*bits/32]
  const void* ks;        // bf16 [KV, N, D/GS]
  const void* kb;
  const uint32_t* vw;
  const void* vs;
  const void* vb;
  void* out;             // bf16 [H, D]
  float* opart;          // [H, G, D]
  float* stats;          // [H, G, 2]
  int H, KV, N, GS, G;
};
bool attention_supported(int D, int rep);
hipError_t launch_attention(int bits, int D, int rep, const AttnArgs& a, hipStream_t st);

bool residual_rms_norm_supported(long D);
// sums: null, or the per-(group, row) sums of the stored normalized values
// at sums[g * sums_ld + row] for groups of group_size (32, 64, 128) values.
hipError_t launch_residual_rms_norm(bool bf16, const void* x, const void* update,
                                    const void* weight, void* residual, void* normalized,
                                    int rows, int D, float eps, float* sums, int group_size,
                                    int sums_ld, hipStream_t st);
// Fused gate/up through the resident kernel: tile pairs per workgroup (1 or
// 2) that are built for cq chunks, and the launch.
bool gate_up_shape(int nC, int pairs, int* nw, int* cpw);
hipError_t launch_gate_up(int bits, bool sb_f32, int nw, int cpw, int pairs, const LaunchArgs& a,
                          int grid, size_t lds_bytes, hipStream_t st);
// Slab kernel: tile slots per workgroup, slices of K built for `mt` row tiles
// (0 if none covers nC chunks), dynamic LDS bytes.
constexpr int kSlabTiles = 3;
int slab_slices(int mt, int nC);
size_t slab_lds_bytes(int mt);
// Wide kernel: 65..128 activation rows per launch (up to kWideRowTiles tiles
// of 16 rows; 6 tiles for up to 96 rows, else 8), weights dequantized to bf16
// in registers, 8 W tiles per workgroup, K in slices of 256 (K a multiple of
// 256).
constexpr int kWideRowTiles = 8;
constexpr int kWideTiles = 8;
size_t wide_lds_bytes(int mt);
bool wide_fits(int nC);
hipError_t launch_wide(int bits, bool sb_f32, int mt, const LaunchArgs& a, int grid,
                       size_t lds_bytes, hipStream_t st);
// Split slab kernel: K cut into S (1 or 2) parts across workgroups, TW (2 or
// 3) W tiles per compute wave, NSLOT tile slots; partial tiles of S = 2 go
// through the workspace (tickets, then the part area).
bool split_slab_shape(int mt, int tw, int nC, int S, int* ns, int* nslot);
size_t split_slab_lds_bytes(int mt);
size_t split_slab_part_bytes(int mt, int tw, int nslot, int groups, int S);
hipError_t launch_split_slab(int bits, bool sb_f32, int mt, int ns, int tw, const LaunchArgs& a,
                             int grid, size_t lds_bytes, hipStream_t st);
hipError_t launch_slab(int bits, bool sb_f32, int mt, int ns, const LaunchArgs& a, int grid,
                       size_t lds_bytes, hipStream_t st);
constexpr size_t kMaxLdsBytes = 160 * 1024;
hipError_t launch_probe(const void* buf, size_t bytes, uint32_t* sink, int grid, hipStream_t st);

// Bytes of LDS the vector-ALU kernel needs for `mr` rows over `kslice` columns.
size_t gemv_lds_bytes(bool x_f32, int mr, int kslice);


}  // namespace qmm
