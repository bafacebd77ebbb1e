// qmm_api.cpp -- the C ABI of include/qmm.h: argument validation, launch
// planning and dispatch.  All validation happens on the host before any HIP
// call.
//
// [P1] = page "@mlx-bun/inference 0.0.0-stage -> 1.0.0" (diffend npm page 53).
//   * affineSplitMmaEligible(): eligibility is a separate predicate (affine,
//     group 64, bits 3 or 4, shape multiples, at least one row) -> here the
//     QMM_ERR_UNSUPPORTED status, raised in qmm_create.
//   * affineSplitMma(): throws when there are no rows -> QMM_ERR_INVALID_ARG
//     from qmm_run for rows < 1.
//   * affineSplitMmaPlan(): the launch shape is a small value chosen from the
//     output width N -> here plan_config(), which also looks at the row count
//     and the chip's 256 compute units.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>

#include "../../include/qmm.h"
#include "qmm_internal.h"

namespace {

thread_local std::string g_err;

qmm_status fail(qmm_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

struct Cfg {
  int variant;  // QMM_VARIANT_GEMV or QMM_VARIANT_MFMA
  int rows_per_launch;
  int tile_rows;  // mt (MFMA, 16-row tiles of x) or mr (GEMV rows)
  int ntw;        // W tiles per wavefront
  int wk;         // wavefronts of a workgroup that split K (MFMA)
  int S;          // K splits across workgroups
  int nTB;        // tile blocks
  size_t lds;     // dynamic LDS bytes (GEMV, STREAM, RESIDENT, SLAB)
  int grid;       // RESIDENT, SLAB: workgroups
  int cpw;        // RESIDENT: chunks of K per wave; SLAB: slices per workgroup
  bool split;     // SLAB: the split slab kernel (ntw = tiles per wave, wk = tile slots)
  bool valu_stream;  // GEMV: the streaming kernel's vector-ALU form (wk = waves, ntw = chunks
                     // per wave)
};

}  // namespace

struct qmm_plan {
  qmm_desc d;
  int nT, nC;
  int force_variant;  // from QMM_FORCE_VARIANT, 0 = none
  int env_ntw, env_splitk, env_kwaves;
  mutable std::atomic<uint64_t> launches[8];
  bool generic;  // other formats on MLX's own layout and the vector-ALU kernel
  bool fmt;      // other formats on the step layout: streaming and resident kernels
  int step_gs;   // fmt: the group size (selects the step-layout kernels); else 0
  int groups;    // quantization groups per 128-value chunk in the kernels' layout
  mutable std::atomic<int> last_variant, last_ntw, last_splitk, last_grid;
  int cus;      // compute units of the device current at qmm_create
  bool f32_out; // QMM_FLAG_F32_OUT: y is f32 whatever x_dtype
};

namespace {

constexpr int kMinBlocks = 512;   // two workgroups per compute unit

// Compute units of the current device (queried once per device).
int device_cus() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = cached[dev].load();
  if (v <= 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        v <= 0)
      v = 256;
    cached[dev] = v;
  }
  return v;
}
constexpr size_t kMaxGemvLds = 64 * 1024;

int env_int(const char* name) {
  const char* v = getenv(name);
  return v ? atoi(v) : 0;
}

int round_up_pow2(int v, int cap) {
  int p = 1;
  while (p < v && p < cap) p <<= 1;
  return p;
}

size_t ticket_bytes(const qmm_plan* p) {
  return ((size_t)p->nT * 4 + 255) / 256 * 256;
}

// Pick the kernel family.  Vector-ALU for f32 activations (the MFMA path takes
// bf16 operands) and, for bf16, wherever it is measured faster.
bool stream_shape(const qmm_plan* p, int* nw, int* cpw) {
  const int nC = p->nC;
  // (waves, chunks per wave): four waves for short K, eight from 16 chunks
  const int opts[][2] = {{4, 2}, {4, 4}, {8, 4}, {8, 5}, {8, 8}, {16, 8}};
  for (const auto& o : opts) {
    if (nC < 16 && o[0] != 4) continue;
    if (nC >= 16 && o[0] == 4) continue;
    if (nC <= o[0] * o[1]) {
      *nw = o[0];
      *cpw = o[1];
      return true;
    }
  }
  return false;
}

// Rows the resident kernel takes per launch: 16 for the native layout (the
// family is chosen only where they fit), for the step layout as many as fit
// one compute unit's LDS (it is their only family beyond the streaming one).
int resident_launch_rows(const qmm_plan* p) { return p->fmt ? qmm::fmt_rows(p->d.K) : 16; }

// Whether a block of `rows` (<= 16) rows fits the resident kernel's LDS.
bool resident_fits(const qmm_plan* p, int rows) {
  int nw, cpw;
  const int r = std::min(qmm::resident_rows(rows), resident_launch_rows(p));
  return r >= 1 && (size_t)r * p->d.K * 2 <= qmm::kMaxLdsBytes &&
         qmm::resident_shape(p->d.bits, p->step_gs, p->nC, 1, &nw, &cpw);
}

bool slab_fits(const qmm_plan* p) {
  return qmm::slab_slices(1, p->nC) > 0 && qmm::slab_slices(2, p->nC) > 0 &&
         qmm::slab_slices(4, p->nC) > 0;
}

// LDS the streaming kernel may stage activations in: 64 KB keeps two or more
// of its workgroups per compute unit; when the tiles fit in one pass over the
// compute units anyway, a workgroup may take a whole unit's LDS.
size_t stream_max_lds(const qmm_plan* p) {
  return p->nT <= p->cus ? qmm::kMaxLdsBytes : (size_t)64 * 1024;
}

// Whether the streaming kernel takes a block of `rows` rows (at most
// kStreamMaxRows) of this plan.
bool stream_ok(const qmm_plan* p, int rows) {
  int nw, cpw;
  return stream_shape(p, &nw, &cpw) &&
         qmm::stream_fits(nw, cpw, rows, p->groups, stream_max_lds(p)) &&
         (!p->fmt || qmm::stream_step_fits(p->d.bits, p->d.group_size, nw, cpw));
}

int pick_variant(const qmm_plan* p, int rows, int forced) {
  if (p->generic) return QMM_VARIANT_GENERIC;
  if (p->d.x_dtype == QMM_F32) return QMM_VARIANT_GEMV;
  if (forced) return forced;
  if (p->fmt) {
    // the step layout runs on the streaming and resident kernels only
    if (p->force_variant == QMM_VARIANT_STREAM || p->force_variant == QMM_VARIANT_RESIDENT)
      return p->force_variant;
    return rows <= 2 && stream_ok(p, rows) ? QMM_VARIANT_STREAM : QMM_VARIANT_RESIDENT;
  }
  if (p->force_variant) return p->force_variant;
  // Measured on the 3-bit 5120->10240 sweep and the 4-bit MLP shapes: the
  // streaming kernel for one or two rows; the resident kernel up to 16 rows
  // while the activation block fits one compute unit's LDS; the streaming
  // kernel up to 4 rows beyond that; then the slab kernel where it is built
  // for this K; else MFMA.
  const bool streams = stream_ok(p, rows);
  if (rows <= 2 && streams) return QMM_VARIANT_STREAM;
  if (rows <= 16 && resident_fits(p, rows)) return QMM_VARIANT_RESIDENT;
  if (streams) return QMM_VARIANT_STREAM;
  // more than 64 rows: the wide kernel (bf16 weights, no per-group epilogue)
  // where its grid (eight W tiles per workgroup) fills at least half the
  // compute units; else 64-row blocks on the slab or MFMA kernels (3-bit
  // 5120->10240 at 128 rows, 80 workgroups: 41.6 us wide against about 36 us
  // as two 64-row split slab launches; 4-bit 8192->28672, 224 workgroups:
  // 85 against 155 us)
  if (rows > qmm::kMaxMfmaRows && qmm::wide_fits(p->nC) &&
      2 * ((p->nT + qmm::kWideTiles - 1) / qmm::kWideTiles) >= p->cus)
    return QMM_VARIANT_WIDE;
  if (slab_fits(p)) return QMM_VARIANT_SLAB;
  return QMM_VARIANT_MFMA;
}

// Launch shape for one launch of `rows` rows (rows <= rows_per_launch).
// ntw_req / wk_req / s_req: 0 = choose here.
Cfg plan_config(const qmm_plan* p, int rows, int variant, int ntw_req, int wk_req, int s_req) {
  Cfg c{};
  c.variant = variant;
  const int nT = p->nT, nC = p->nC;
  auto pow2_floor = [](int v) { return v >= 4 ? 4 : (v >= 2 ? 2 : 1); };
  int tiles_per_block;
  if (variant == QMM_VARIANT_RESIDENT) {
    // as few tile slots as fill every compute unit once (fewer where no
    // built shape covers this K with that many); more tiles than slots x
    // compute units take a second pass
    c.rows_per_launch = resident_launch_rows(p);
    c.tile_rows = 1;
    const int g = std::min(p->cus, nT);
    const int r = std::min(rows, c.rows_per_launch);
    int tm = std::min(qmm::kResidentMaxSlots, (nT + g - 1) / g);
    // four slots per unit: two workgroups of two slots each keep twice the
    // waves per unit at the same tiles per unit (measured faster) where two
    // activation blocks fit its LDS
    if (tm == 4 && 2 * (size_t)qmm::resident_rows(r) * p->d.K * 2 <= qmm::kMaxLdsBytes) tm = 2;
    if (ntw_req) tm = std::max(1, std::min(ntw_req, qmm::kResidentMaxSlots));
    int nw = 0, cpw = 0;
    while (tm > 1 && !qmm::resident_shape(p->d.bits, p->step_gs, nC, tm, &nw, &cpw)) --tm;
    qmm::resident_shape(p->d.bits, p->step_gs, nC, tm, &nw, &cpw);
    c.ntw = tm;
    c.cpw = cpw;
    c.wk = nw;
    c.grid = (nT + tm - 1) / tm;
    c.nTB = c.grid;
    c.S = 1;
    c.lds = qmm::resident_lds_bytes(nw, tm, r, (int)p->d.K);
    return c;
  }
  if (variant == QMM_VARIANT_WIDE) {
    c.rows_per_launch = 16 * qmm::kWideRowTiles;
    // 65..96 rows in six row tiles: no MFMAs or A-fragment reads for a
    // seventh and eighth tile of padding rows
    c.tile_rows = std::min(rows, c.rows_per_launch) <= 96 ? 6 : qmm::kWideRowTiles;
    c.ntw = qmm::kWideTiles;
    c.wk = 1;
    c.S = 1;
    c.nTB = (nT + qmm::kWideTiles - 1) / qmm::kWideTiles;
    c.grid = c.nTB;
    c.lds = qmm::wide_lds_bytes(c.tile_rows);
    return c;
  }
  if (variant == QMM_VARIANT_GENERIC) {
    c.rows_per_launch = qmm::kGenericMaxRows;
    c.tile_rows = std::min(rows, qmm::kGenericMaxRows);
    c.ntw = 1;
    c.wk = 1;
    c.S = 1;
    c.nTB = nT;
    c.grid = (int)(p->d.N / 8);  // eight W rows per workgroup
    return c;
  }
  if (variant == QMM_VARIANT_SLAB) {
    c.rows_per_launch = qmm::kMaxMfmaRows;
    const int r = std::min(rows, qmm::kMaxMfmaRows);
    c.tile_rows = r <= 16 ? 1 : (r <= 32 ? 2 : 4);
    // the split slab kernel (ntw = 2 W tiles per compute wave, splitk = 2 K
    // parts) by default for 33..64 rows, where the slab kernel's compute units
    // each take in the whole activation block (measured 19.8 against 23 us at
    // 64 rows of the 3-bit 5120x10240 workload; at 32 rows the slab kernel is
    // faster, 12.5 against 13.6 us); ntw = 1 forces the slab kernel
    const int tw = ntw_req ? ntw_req : (c.tile_rows == 4 ? 2 : 1);
    const int S = s_req ? s_req : 2;
    int ns = 0, nslot = 0;
    // 33..48 rows: the split form in three row tiles (48 rows) where it is
    // built, instead of four with a fourth computed for nothing
    if (c.tile_rows == 4 && r <= 48 && tw >= 2 && qmm::split_slab_shape(3, tw, nC, S, &ns, &nslot))
      c.tile_rows = 3;
    if (c.tile_rows >= 2 && tw >= 2 && qmm::split_slab_shape(c.tile_rows, tw, nC, S, &ns, &nslot)) {
      c.split = true;
      c.ntw = tw;
      c.wk = nslot;
      c.cpw = ns;
      c.S = S;
      c.nTB = (nT + tw * nslot - 1) / (tw * nslot);
      c.grid = c.nTB * S;
      c.lds = qmm::split_slab_lds_bytes(c.tile_rows);
      return c;
    }
    c.cpw = qmm::slab_slices(c.tile_rows, nC);
    c.ntw = qmm::kSlabTiles;
    c.wk = 4;
    c.grid = (nT + qmm::kSlabTiles - 1) / qmm::kSlabTiles;
    c.nTB = c.grid;
    c.S = 1;
    c.lds = qmm::slab_lds_bytes(c.tile_rows);
    return c;
  }
  if (variant == QMM_VARIANT_GEMV && p->d.x_dtype == QMM_BF16 && !p->fmt &&
      stream_ok(p, std::min(rows, qmm::kStreamMaxRows))) {
    // bf16 activations: the streaming kernel's structure, vector-ALU products
    c.valu_stream = true;
    c.rows_per_launch = qmm::kStreamMaxRows;
    c.tile_rows = 1;
    int nw = 8, cpw = 8;
    stream_shape(p, &nw, &cpw);
    c.wk = nw;
    c.ntw = cpw;
    c.nTB = nT;
    c.lds = qmm::stream_lds_bytes(nw, cpw, std::min(rows, qmm::kStreamMaxRows), p->groups);
    c.S = 1;
    return c;
  }
  if (variant == QMM_VARIANT_STREAM) {
    c.rows_per_launch = qmm::kStreamMaxRows;
    c.tile_rows = 1;
    int nw = 8, cpw = 8;
    stream_shape(p, &nw, &cpw);
    c.wk = nw;
    c.ntw = cpw;  // chunks per wave for this family
    c.nTB = nT;
    const int r = std::min(rows, qmm::kStreamMaxRows);
    c.lds = qmm::stream_lds_bytes(nw, cpw, r, p->groups);
    c.S = 1;
    return c;
  }
  if (variant == QMM_VARIANT_MFMA) {
    c.rows_per_launch = qmm::kMaxMfmaRows;
    const int r = std::min(rows, qmm::kMaxMfmaRows);
    c.tile_rows = round_up_pow2((r + 15) / 16, 4);
    // defaults (measured on the 3-bit 5120->10240 workload): K split over
    // the workgroup's four waves; two W tiles per wave once the activation
    // block is long enough for the reuse to pay
    int ntw = r <= 1 ? 1 : 2, wk = c.tile_rows <= 2 ? 4 : 2;
    if (ntw_req) ntw = ntw_req;
    if (wk_req) wk = wk_req;
    c.ntw = std::min(pow2_floor(ntw), c.tile_rows <= 1 ? 4 : 2);
    c.wk = pow2_floor(wk);
    tiles_per_block = (qmm::kWaves / c.wk) * c.ntw;
  } else {
    c.rows_per_launch = qmm::kMaxGemvRows;
    const int r = std::min(rows, qmm::kMaxGemvRows);
    c.tile_rows = round_up_pow2(r, 8);
    int ntw = 1;
    if (ntw_req) ntw = ntw_req;
    const int cap = c.tile_rows == 1 ? 4 : (c.tile_rows <= 4 ? 2 : 1);
    c.ntw = std::min(pow2_floor(ntw), cap);
    c.wk = 1;
    tiles_per_block = qmm::kWaves * c.ntw;
  }
  c.nTB = (nT + tiles_per_block - 1) / tiles_per_block;
  int S;
  if (s_req) {
    S = s_req;
  } else {
    // A K split across workgroups needs a device-scope release per workgroup
    // (an L2 write-back on this chip), which costs more than it gains unless
    // the grid would otherwise leave most compute units idle.
    S = c.nTB >= kMinBlocks / 8 ? 1 : (kMinBlocks / 8 + c.nTB - 1) / c.nTB;
    // partial sums cost S*rows*N*8 bytes of traffic: keep S*rows bounded
    const int r = std::min(rows, c.rows_per_launch);
    S = std::min(S, std::max(1, 64 / std::max(1, r)));
    S = std::min(S, std::max(1, nC / (2 * c.wk)));
  }
  S = std::max(1, std::min(S, nC));
  if (variant == QMM_VARIANT_GEMV) {
    const bool xf = p->d.x_dtype == QMM_F32;
    // the activation slice of one split must fit the LDS budget
    while (S < nC && qmm::gemv_lds_bytes(xf, c.tile_rows, ((nC + S - 1) / S) * qmm::kChunkK) > kMaxGemvLds) ++S;
    c.lds = qmm::gemv_lds_bytes(xf, c.tile_rows, ((nC + S - 1) / S) * qmm::kChunkK);
  }
  c.S = S;
  return c;
}

size_t cfg_workspace(const qmm_plan* p, const Cfg& c, int rows) {
  if (c.S <= 1) return 0;
  if (c.split)
    return ticket_bytes(p) + qmm::split_slab_part_bytes(c.tile_rows, c.ntw, c.wk, c.nTB, c.S);
  const int r = std::min(rows, c.rows_per_launch);
  return ticket_bytes(p) + (size_t)c.S * r * p->d.N * sizeof(float);
}

// The family of one row block of a call in several blocks: a choice left to
// the library is remade for a block shorter than the call's blocks (a
// 65-row call on the slab family: one 64-row block, then one row on the
// streaming kernel; a 129-row call on the wide kernel: one 128-row block,
// then one row on the streaming kernel); a forced family runs every block.
int block_variant(const qmm_plan* p, int call_variant, bool chosen, int rows, int rb) {
  if (!chosen || rb == rows || p->force_variant) return call_variant;
  if (call_variant == QMM_VARIANT_WIDE && rb <= qmm::kMaxMfmaRows)
    return pick_variant(p, rb, QMM_VARIANT_AUTO);
  if (call_variant != QMM_VARIANT_SLAB && call_variant != QMM_VARIANT_MFMA) return call_variant;
  return pick_variant(p, rb, QMM_VARIANT_AUTO);
}

// Largest workspace any row block of a `rows`-row call needs (blocks of a
// call run one after another on the stream and share the workspace).
size_t call_workspace(const qmm_plan* p, int rows, int variant, bool chosen, int ntw, int wk,
                      int s) {
  const Cfg c = plan_config(p, rows, variant, ntw, wk, s);
  size_t need = 0;
  for (int r0 = 0; r0 < rows; r0 += c.rows_per_launch) {
    const int rb = std::min(c.rows_per_launch, rows - r0);
    const int vb = block_variant(p, variant, chosen, rows, rb);
    need = std::max(need, cfg_workspace(p, plan_config(p, rb, vb, ntw, wk, s), rb));
  }
  return need;
}

bool aligned(const void* ptr, size_t a) { return ((uintptr_t)ptr % a) == 0; }

qmm_status check_plan(const qmm_plan* p) {
  if (!p) return fail(QMM_ERR_INVALID_ARG, "plan is NULL");
  return QMM_OK;
}

qmm_status hip_fail(hipError_t e, const char* what) {
  return fail(e == hipErrorNoDevice ? QMM_ERR_NO_DEVICE : QMM_ERR_HIP, "%s: %s", what,
              hipGetErrorString(e));
}

// Values per group of the group sums the plan's kernels use: 64 on the
// native layout (a group of 128 is stored as two halves), else the plan's
// group size.
int sum_group(const qmm_plan* p) { return p->fmt || p->generic ? p->d.group_size : 64; }

qmm_status run_impl(const qmm_plan* p, int variant_req, int ntw_req, int wk_req, int s_req,
                    const void* x,
                    const void* codes, const void* sb, void* y, int32_t rows, void* ws,
                    size_t ws_bytes, void* stream, const float* xsums = nullptr,
                    int32_t xsums_ld = 0) {
  if (qmm_status st = check_plan(p)) return st;
  if (rows < 1 || rows > p->d.max_rows)
    return fail(QMM_ERR_INVALID_ARG, "rows=%d outside 1..max_rows=%d", rows, p->d.max_rows);
  if (xsums && (!aligned(xsums, 16) || xsums_ld % 16 != 0 || xsums_ld < (rows + 15) / 16 * 16))
    return fail(QMM_ERR_INVALID_ARG,
                "x_sums must be 16-byte aligned with sums_ld a multiple of 16 and at least rows "
                "rounded up to 16 (rows=%d, sums_ld=%d)", rows, xsums_ld);
  if (!x || !codes || !sb || !y) return fail(QMM_ERR_INVALID_ARG, "NULL data pointer");
  if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(sb, 16) || !aligned(y, 4))
    return fail(QMM_ERR_INVALID_ARG, "x, codes and sb must be 16-byte aligned, y 4-byte aligned");
  if (variant_req < QMM_VARIANT_AUTO || variant_req > QMM_VARIANT_WIDE)
    return fail(QMM_ERR_INVALID_ARG, "unknown variant %d", variant_req);
  if (p->generic && variant_req != QMM_VARIANT_AUTO && variant_req != QMM_VARIANT_GENERIC)
    return fail(QMM_ERR_UNSUPPORTED,
                "bits=%d group_size=%d with f32 activations or scales run only on the "
                "vector-ALU kernel of MLX's layout (QMM_VARIANT_GENERIC)",
                p->d.bits, p->d.group_size);
  if (p->fmt && variant_req != QMM_VARIANT_AUTO && variant_req != QMM_VARIANT_STREAM &&
      variant_req != QMM_VARIANT_RESIDENT)
    return fail(QMM_ERR_UNSUPPORTED,
                "bits=%d group_size=%d run on the streaming and resident kernels only",
                p->d.bits, p->d.group_size);
  if (!p->generic && variant_req == QMM_VARIANT_GENERIC)
    return fail(QMM_ERR_UNSUPPORTED,
                "QMM_VARIANT_GENERIC is the vector-ALU kernel of plans that keep MLX's layout "
                "(formats without a matrix-core path, or f32 activations or scales)");
  if ((variant_req == QMM_VARIANT_MFMA || variant_req == QMM_VARIANT_STREAM ||
       variant_req == QMM_VARIANT_RESIDENT || variant_req == QMM_VARIANT_SLAB ||
       variant_req == QMM_VARIANT_WIDE) &&
      p->d.x_dtype != QMM_BF16)
    return fail(QMM_ERR_UNSUPPORTED, "the MFMA kernels take bf16 activations");
  if (variant_req == QMM_VARIANT_STREAM && !stream_ok(p, std::min(rows, qmm::kStreamMaxRows)))
    return fail(QMM_ERR_UNSUPPORTED,
                "the streaming kernel needs K <= 16384, its activation slices to fit its LDS "
                "budget and, for the step layout, its weight registers to fit");
  if (variant_req == QMM_VARIANT_RESIDENT && !resident_fits(p, std::min(rows, 16)))
    return fail(QMM_ERR_UNSUPPORTED,
                "the resident kernel needs K <= 16384 and rows*K*2 bytes of activations (rows "
                "capped at 16) to fit one compute unit's 160 KB of LDS");
  if (variant_req == QMM_VARIANT_WIDE && !qmm::wide_fits(p->nC))
    return fail(QMM_ERR_UNSUPPORTED, "the wide kernel needs K to be a multiple of 256 (K=%lld)",
                (long long)p->d.K);
  if (variant_req == QMM_VARIANT_SLAB && !slab_fits(p))
    return fail(QMM_ERR_UNSUPPORTED, "the slab kernel is built for K = 5120 and 8192 (K=%lld)",
                (long long)p->d.K);
  if (ntw_req < 0 || ntw_req > 8 || s_req < 0 || wk_req < 0 || wk_req > 8)
    return fail(QMM_ERR_INVALID_ARG, "ntw must be 0..8, kwaves 0..8 and splitk >= 0");
  const int ntw_eff = ntw_req ? ntw_req : p->env_ntw;
  const int wk_eff = wk_req ? wk_req : p->env_kwaves;
  const int s_eff = s_req ? s_req : p->env_splitk;
  const int variant = pick_variant(p, rows, variant_req);
  const bool chosen = variant_req == QMM_VARIANT_AUTO;
  const Cfg c = plan_config(p, rows, variant, ntw_eff, wk_eff, s_eff);
  const size_t need = call_workspace(p, rows, variant, chosen, ntw_eff, wk_eff, s_eff);
  if (need > 0) {
    if (!ws || ws_bytes < need)
      return fail(QMM_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                  ws ? ws_bytes : (size_t)0);
    if (!aligned(ws, 256)) return fail(QMM_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  }
  const bool xf = p->d.x_dtype == QMM_F32, sf = p->d.sb_dtype == QMM_F32;
  const size_t xe = xf ? 4 : 2, ye = (xf || p->f32_out) ? 4 : 2;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  for (int r0 = 0; r0 < rows; r0 += c.rows_per_launch) {
    const int rb = std::min(c.rows_per_launch, rows - r0);
    const int vb = block_variant(p, variant, chosen, rows, rb);
    const Cfg cb = plan_config(p, rb, vb, ntw_eff, wk_eff, s_eff);
    qmm::LaunchArgs a{};
    a.x = static_cast<const char*>(x) + (size_t)r0 * p->d.K * xe;
    a.codes = static_cast<const uint32_t*>(codes);
    a.sb = sb;
    a.y = static_cast<char*>(y) + (size_t)r0 * p->d.N * ye;
    a.y_f32 = p->f32_out ? 1 : 0;
    // given group sums: the matrix-core streaming kernel (rows < rb only),
    // and the resident kernel where its reads stay inside x_sums: it reads
    // rows r0 .. r0+15 of every group, 16 bytes at a time, which sums_ld
    // (a multiple of 16, at least rows rounded up to 16) covers when r0 is a
    // multiple of 16
    const bool takes_sums = (vb == QMM_VARIANT_STREAM) ||
                            (vb == QMM_VARIANT_RESIDENT && r0 % 16 == 0);
    a.xsums = xsums && takes_sums ? xsums + r0 : nullptr;
    a.xsums_ld = xsums_ld;
    a.tickets = static_cast<uint32_t*>(ws);
    a.part = ws ? reinterpret_cast<float*>(static_cast<char*>(ws) + ticket_bytes(p)) : nullptr;
    a.M = rb;
    a.N = (int)p->d.N;
    a.K = (int)p->d.K;
    a.S = cb.S;
    a.nTB = cb.nTB;
    a.ldx = (int)p->d.K;
    a.ldy = (int)p->d.N;
    if (cb.S > 1 && cfg_workspace(p, cb, rb) > ws_bytes)
      return fail(QMM_ERR_WORKSPACE, "workspace too small for a %d-row block", rb);
    hipError_t e;
    if (vb == QMM_VARIANT_GENERIC)
      e = qmm::launch_generic(p->d.bits, p->d.group_size, xf, sf, rb, a, st);
    else if (vb == QMM_VARIANT_WIDE)
      e = qmm::launch_wide(p->d.bits, sf, cb.tile_rows, a, cb.grid, cb.lds, st);
    else if (vb == QMM_VARIANT_SLAB && cb.split)
      e = qmm::launch_split_slab(p->d.bits, sf, cb.tile_rows, cb.cpw, cb.ntw, a, cb.grid, cb.lds,
                                 st);
    else if (vb == QMM_VARIANT_SLAB)
      e = qmm::launch_slab(p->d.bits, sf, cb.tile_rows, cb.cpw, a, cb.grid, cb.lds, st);
    else if (vb == QMM_VARIANT_RESIDENT)
      e = qmm::launch_resident(p->d.bits, p->step_gs, sf, cb.wk, cb.cpw, cb.ntw, a, cb.grid,
                               cb.lds, st);
    else if (vb == QMM_VARIANT_STREAM)
      e = qmm::launch_stream(p->d.bits, p->step_gs, sf, cb.wk, cb.ntw, a, cb.lds, st);
    else if (vb == QMM_VARIANT_MFMA)
      e = qmm::launch_mfma(p->d.bits, sf, cb.tile_rows, cb.ntw, cb.wk, a, st);
    else if (cb.valu_stream)
      e = qmm::launch_stream_valu(p->d.bits, sf, cb.wk, cb.ntw, a, cb.lds, st);
    else
      e = qmm::launch_gemv(p->d.bits, xf, sf, cb.tile_rows, cb.ntw, a, cb.lds, st);
    if (e != hipSuccess) return hip_fail(e, "kernel launch");
    p->launches[vb].fetch_add(1);
    p->last_variant = vb;
    p->last_ntw = cb.ntw;
    p->last_splitk = cb.S;
    p->last_grid = (vb == QMM_VARIANT_RESIDENT || vb == QMM_VARIANT_SLAB)
                       ? cb.grid : cb.nTB * cb.S;
  }
  if (getenv("QMM_LOG"))
    fprintf(stderr, "qmm: rows=%d variant=%d ntw=%d kwaves=%d splitk=%d grid=%d\n", rows,
            variant, c.ntw, c.wk, c.S, c.nTB * c.S);
  return QMM_OK;
}

}  // namespace

namespace qmm {
qmm_status set_error(qmm_status st, const char* msg) { return fail(st, "%s", msg); }
}  // namespace qmm

extern "C" {

qmm_status qmm_create(const qmm_desc* d, qmm_plan** out) {
  if (!out) return fail(QMM_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (!d) return fail(QMM_ERR_INVALID_ARG, "desc is NULL");
  const int b = d->bits;
  if (b != 2 && b != 3 && b != 4 && b != 5 && b != 6 && b != 8)
    return fail(QMM_ERR_INVALID_ARG, "bits=%d is not an MLX affine width", b);
  if (d->group_size != 32 && d->group_size != 64 && d->group_size != 128)
    return fail(QMM_ERR_INVALID_ARG, "group_size=%d is not an MLX affine group size", d->group_size);
  if (d->K <= 0 || d->N <= 0) return fail(QMM_ERR_INVALID_ARG, "K and N must be positive");
  if (d->K % d->group_size != 0)
    return fail(QMM_ERR_INVALID_ARG, "K=%lld is not a multiple of the group size", (long long)d->K);
  if (d->max_rows < 1) return fail(QMM_ERR_INVALID_ARG, "max_rows must be >= 1");
  if ((d->x_dtype != QMM_F32 && d->x_dtype != QMM_BF16) ||
      (d->sb_dtype != QMM_F32 && d->sb_dtype != QMM_BF16))
    return fail(QMM_ERR_INVALID_ARG, "unknown dtype");
  if ((d->flags & ~(uint32_t)QMM_FLAG_F32_OUT) != 0)
    return fail(QMM_ERR_INVALID_ARG, "flags=0x%x: only QMM_FLAG_F32_OUT is defined", d->flags);
  if (b != 2 && b != 3 && b != 4 && b != 8)
    return fail(QMM_ERR_UNSUPPORTED, "bits=%d: 2, 3, 4 and 8 are implemented", b);
  if (d->K % qmm::kChunkK != 0)
    return fail(QMM_ERR_UNSUPPORTED, "K=%lld: must be a multiple of %d", (long long)d->K, qmm::kChunkK);
  if (d->N % qmm::kTileN != 0)
    return fail(QMM_ERR_UNSUPPORTED, "N=%lld: must be a multiple of %d", (long long)d->N, qmm::kTileN);
  if (d->K > (1LL << 24) || d->N > (1LL << 24) || (int64_t)d->max_rows * d->K > (1LL << 31) ||
      (int64_t)d->max_rows * d->N > (1LL << 31))
    return fail(QMM_ERR_UNSUPPORTED, "shape exceeds 32-bit indexing");
  qmm_plan* p = new (std::nothrow) qmm_plan();
  if (!p) return fail(QMM_ERR_INVALID_ARG, "out of host memory");
  p->d = *d;
  p->nT = (int)(d->N / qmm::kTileN);
  p->nC = (int)(d->K / qmm::kChunkK);
  // 3- and 4-bit codes with groups of 64 or 128: the native layout; the
  // other formats with bf16 activations and scales: the step layout where
  // its kernel covers K; else MLX's layout on the vector-ALU kernel
  const bool native = (b == 3 || b == 4) && (d->group_size == 64 || d->group_size == 128);
  int fnw = 0, fcpw = 0;
  p->fmt = !native && d->x_dtype == QMM_BF16 && d->sb_dtype == QMM_BF16 &&
           qmm::fmt_format(b, d->group_size) && qmm::fmt_rows(d->K) >= 1 &&
           qmm::resident_shape(b, d->group_size, p->nC, 1, &fnw, &fcpw);
  p->generic = !native && !p->fmt;
  p->step_gs = p->fmt ? d->group_size : 0;
  p->groups = p->fmt ? qmm::kChunkK / d->group_size : 2;
  p->force_variant = 0;
  if (const char* v = getenv("QMM_FORCE_VARIANT")) {
    if (!strcmp(v, "gemv")) p->force_variant = QMM_VARIANT_GEMV;
    if (!strcmp(v, "mfma")) p->force_variant = QMM_VARIANT_MFMA;
    if (!strcmp(v, "stream")) p->force_variant = QMM_VARIANT_STREAM;
    if (!strcmp(v, "resident")) p->force_variant = QMM_VARIANT_RESIDENT;
    if (!strcmp(v, "slab")) p->force_variant = QMM_VARIANT_SLAB;
  }
  p->env_ntw = env_int("QMM_NTW");
  p->env_splitk = env_int("QMM_SPLITK");
  p->env_kwaves = env_int("QMM_KWAVES");
  for (auto& l : p->launches) l = 0;
  p->last_variant = 0;
  p->last_ntw = 0;
  p->last_splitk = 0;
  p->last_grid = 0;
  p->cus = device_cus();
  p->f32_out = (d->flags & QMM_FLAG_F32_OUT) != 0;
  *out = p;
  return QMM_OK;
}

void qmm_destroy(qmm_plan* p) { delete p; }

qmm_status qmm_packed_bytes(const qmm_plan* p, size_t* codes_bytes, size_t* sb_bytes) {
  if (qmm_status st = check_plan(p)) return st;
  if (!codes_bytes || !sb_bytes) return fail(QMM_ERR_INVALID_ARG, "NULL output pointer");
  *codes_bytes = (size_t)p->d.N * p->d.K * p->d.bits / 8;
  // the native layout holds a scale and a bias per 64 values (a group of
  // 128 gives both halves its pair)
  const int64_t per = (p->generic || p->fmt) ? p->d.group_size : 64;
  *sb_bytes = (size_t)2 * p->d.N * (p->d.K / per) * (p->d.sb_dtype == QMM_F32 ? 4 : 2);
  return QMM_OK;
}

qmm_status qmm_prepack(const qmm_plan* p, const uint32_t* w, const void* scales,
                       const void* biases, void* codes_out, void* sb_out, void* stream) {
  if (qmm_status st = check_plan(p)) return st;
  if (!w || !scales || !biases || !codes_out || !sb_out)
    return fail(QMM_ERR_INVALID_ARG, "NULL pointer");
  if (!aligned(w, 4) || !aligned(codes_out, 16) || !aligned(sb_out, 16) ||
      !aligned(scales, p->d.sb_dtype == QMM_F32 ? 4 : 2) ||
      !aligned(biases, p->d.sb_dtype == QMM_F32 ? 4 : 2))
    return fail(QMM_ERR_INVALID_ARG, "misaligned pointer");
  if (p->generic) {
    // MLX's layout as it is: the codes, then the scales and biases as planes
    const size_t cb = (size_t)p->d.N * p->d.K * p->d.bits / 8;
    const size_t pb = (size_t)p->d.N * (p->d.K / p->d.group_size) * (p->d.sb_dtype == QMM_F32 ? 4 : 2);
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    hipError_t e = hipMemcpyAsync(codes_out, w, cb, hipMemcpyDeviceToDevice, st);
    if (e == hipSuccess) e = hipMemcpyAsync(sb_out, scales, pb, hipMemcpyDeviceToDevice, st);
    if (e == hipSuccess)
      e = hipMemcpyAsync(static_cast<char*>(sb_out) + pb, biases, pb, hipMemcpyDeviceToDevice, st);
    if (e != hipSuccess) return hip_fail(e, "prepack copy");
    return QMM_OK;
  }
  hipError_t e;
  if (p->fmt)
    e = qmm::launch_repack_fmt(p->d.bits, p->d.group_size, w, scales, biases,
                               static_cast<uint32_t*>(codes_out), sb_out, (int)p->d.N,
                               (int)p->d.K, reinterpret_cast<hipStream_t>(stream));
  else
    e = qmm::launch_repack(p->d.bits, p->d.group_size, p->d.sb_dtype == QMM_F32, w, scales,
                           biases, static_cast<uint32_t*>(codes_out), sb_out, (int)p->d.N,
                           (int)p->d.K, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "repack launch");
  return QMM_OK;
}

size_t qmm_workspace_bytes_ex(const qmm_plan* p, int32_t variant, int32_t ntw, int32_t kwaves,
                              int32_t splitk, int32_t rows) {
  if (!p || rows < 1) return 0;
  const int v = pick_variant(p, rows, variant);
  return call_workspace(p, rows, v, variant == QMM_VARIANT_AUTO, ntw ? ntw : p->env_ntw,
                        kwaves ? kwaves : p->env_kwaves, splitk ? splitk : p->env_splitk);
}

size_t qmm_workspace_bytes(const qmm_plan* p, int32_t rows) {
  if (!p || rows < 1) return 0;
  size_t need = qmm_workspace_bytes_ex(p, QMM_VARIANT_AUTO, 0, 0, 0, rows);
  if (p->d.x_dtype == QMM_BF16 && !p->fmt) {
    need = std::max(need, qmm_workspace_bytes_ex(p, QMM_VARIANT_GEMV, 0, 0, 0, rows));
    need = std::max(need, qmm_workspace_bytes_ex(p, QMM_VARIANT_MFMA, 0, 0, 0, rows));
  }
  return need;
}

qmm_status qmm_run(const qmm_plan* p, const void* x, const void* codes, const void* sb, void* y,
                   int32_t rows, void* ws, size_t ws_bytes, void* stream) {
  return run_impl(p, QMM_VARIANT_AUTO, 0, 0, 0, x, codes, sb, y, rows, ws, ws_bytes, stream);
}

qmm_status qmm_run_sums(const qmm_plan* p, const void* x, const float* x_sums, int32_t sums_ld,
                        const void* codes, const void* sb, void* y, int32_t rows, void* ws,
                        size_t ws_bytes, void* stream) {
  if (!x_sums) return fail(QMM_ERR_INVALID_ARG, "x_sums is NULL (use qmm_run)");
  return run_impl(p, QMM_VARIANT_AUTO, 0, 0, 0, x, codes, sb, y, rows, ws, ws_bytes, stream,
                  x_sums, sums_ld);
}

int32_t qmm_sum_group(const qmm_plan* p) { return p ? sum_group(p) : 0; }

qmm_status qmm_run_ex(const qmm_plan* p, int32_t variant, int32_t ntw, int32_t kwaves,
                      int32_t splitk, const void* x, const void* codes, const void* sb, void* y,
                      int32_t rows, void* ws, size_t ws_bytes, void* stream) {
  return run_impl(p, variant, ntw, kwaves, splitk, x, codes, sb, y, rows, ws, ws_bytes, stream);
}

qmm_status qmm_run_gate_up(const qmm_plan* p, const void* x, const void* gate_codes,
                           const void* gate_sb, const void* up_codes, const void* up_sb, void* h,
                           int32_t rows, int32_t tile_pairs, void* stream) {
  if (qmm_status st = check_plan(p)) return st;
  if (rows < 1 || rows > p->d.max_rows)
    return fail(QMM_ERR_INVALID_ARG, "rows=%d outside 1..max_rows=%d", rows, p->d.max_rows);
  if (!x || !gate_codes || !gate_sb || !up_codes || !up_sb || !h)
    return fail(QMM_ERR_INVALID_ARG, "NULL data pointer");
  if (!aligned(x, 16) || !aligned(gate_codes, 16) || !aligned(gate_sb, 16) ||
      !aligned(up_codes, 16) || !aligned(up_sb, 16) || !aligned(h, 4))
    return fail(QMM_ERR_INVALID_ARG, "x, codes and sb must be 16-byte aligned, h 4-byte aligned");
  if (p->d.x_dtype != QMM_BF16)
    return fail(QMM_ERR_UNSUPPORTED, "the fused gate/up kernel takes bf16 activations");
  if (p->generic || p->fmt)
    return fail(QMM_ERR_UNSUPPORTED,
                "the fused gate/up kernel takes 3- and 4-bit weights with groups of 64 or 128");
  if (p->f32_out)
    return fail(QMM_ERR_UNSUPPORTED, "the fused gate/up output is bf16 by definition (no QMM_FLAG_F32_OUT)");
  if (tile_pairs < 0 || tile_pairs > 2)
    return fail(QMM_ERR_INVALID_ARG, "tile_pairs must be 0 (plan's choice), 1 or 2");
  const int nT = p->nT, nC = p->nC;
  const int r_max = std::min(rows, 16);
  int nw = 0, cpw = 0;
  if ((size_t)qmm::resident_rows(r_max) * p->d.K * 2 > qmm::kMaxLdsBytes ||
      !qmm::gate_up_shape(nC, 1, &nw, &cpw))
    return fail(QMM_ERR_UNSUPPORTED,
                "the fused gate/up kernel needs K <= 8192 and rows*K*2 bytes of activations "
                "(rows capped at 16 per pass) to fit one compute unit's 160 KB of LDS");
  // one tile pair per workgroup (measured faster than two on the MLP shapes:
  // 17.6 against 18.4 us for 3840 -> 15360 at 4 rows)
  int pairs = tile_pairs ? tile_pairs : 1;
  if (!qmm::gate_up_shape(nC, pairs, &nw, &cpw)) pairs = 1;
  qmm::gate_up_shape(nC, pairs, &nw, &cpw);
  const bool sf = p->d.sb_dtype == QMM_F32;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  for (int r0 = 0; r0 < rows; r0 += 16) {
    const int rb = std::min(16, rows - r0);
    qmm::LaunchArgs a{};
    a.x = static_cast<const char*>(x) + (size_t)r0 * p->d.K * 2;
    a.codes = static_cast<const uint32_t*>(gate_codes);
    a.sb = gate_sb;
    a.codes2 = static_cast<const uint32_t*>(up_codes);
    a.sb2 = up_sb;
    a.y = static_cast<char*>(h) + (size_t)r0 * p->d.N * 2;
    a.M = rb;
    a.N = (int)p->d.N;
    a.K = (int)p->d.K;
    a.S = 1;
    a.ldx = (int)p->d.K;
    a.ldy = (int)p->d.N;
    const int grid = (nT + pairs - 1) / pairs;
    a.nTB = grid;
    const size_t lds = qmm::resident_lds_bytes(nw, 2 * pairs, rb, (int)p->d.K);
    if (hipError_t e = qmm::launch_gate_up(p->d.bits, sf, nw, cpw, pairs, a, grid, lds, st))
      return hip_fail(e, "kernel launch");
    p->launches[QMM_VARIANT_RESIDENT].fetch_add(1);
    p->last_variant = QMM_VARIANT_RESIDENT;
    p->last_ntw = 2 * pairs;
    p->last_splitk = 1;
    p->last_grid = grid;
  }
  return QMM_OK;
}

qmm_status qmm_residual_rms_norm(const void* x, const void* update, const void* weight,
                                 void* residual, void* normalized, int32_t rows, int64_t D,
                                 float eps, int32_t dtype, void* stream) {
  return qmm_residual_rms_norm_ex(x, update, weight, residual, normalized, nullptr, 64, 0, rows,
                                  D, eps, dtype, stream);
}

qmm_status qmm_residual_rms_norm_ex(const void* x, const void* update, const void* weight,
                                    void* residual, void* normalized, float* group_sums,
                                    int32_t group_size, int32_t sums_ld, int32_t rows, int64_t D,
                                    float eps, int32_t dtype, void* stream) {
  if (!x || !update || !weight || !residual || !normalized)
    return fail(QMM_ERR_INVALID_ARG, "NULL data pointer");
  if (group_sums) {
    if (group_size != 32 && group_size != 64 && group_size != 128)
      return fail(QMM_ERR_INVALID_ARG, "group_size=%d: 32, 64 or 128", group_size);
    if (D % group_size != 0)
      return fail(QMM_ERR_INVALID_ARG, "D=%lld is not a multiple of group_size=%d", (long long)D,
                  group_size);
    if (sums_ld < rows || !aligned(group_sums, 4))
      return fail(QMM_ERR_INVALID_ARG, "sums_ld=%d must be >= rows=%d, group_sums 4-byte aligned",
                  sums_ld, rows);
  }
  if (!aligned(x, 16) || !aligned(update, 16) || !aligned(weight, 16) || !aligned(residual, 16) ||
      !aligned(normalized, 16))
    return fail(QMM_ERR_INVALID_ARG, "every buffer must be 16-byte aligned");
  if (rows < 1) return fail(QMM_ERR_INVALID_ARG, "rows=%d must be >= 1", rows);
  if (dtype != QMM_BF16 && dtype != QMM_F32)
    return fail(QMM_ERR_INVALID_ARG, "dtype must be QMM_BF16 or QMM_F32");
  if (!(eps >= 0.f) || !std::isfinite(eps))
    return fail(QMM_ERR_INVALID_ARG, "eps must be finite and >= 0");
  if (!qmm::residual_rms_norm_supported(D))
    return fail(QMM_ERR_UNSUPPORTED, "D=%lld: a multiple of 8 from 8 to 16384 is supported",
                (long long)D);
  if (hipError_t e = qmm::launch_residual_rms_norm(dtype == QMM_BF16, x, update, weight, residual,
                                                   normalized, rows, (int)D, eps, group_sums,
                                                   group_size, sums_ld,
                                                   reinterpret_cast<hipStream_t>(stream)))
    return hip_fail(e, "kernel launch");
  return QMM_OK;
}

size_t qmm_attention_workspace_bytes(int32_t H, int64_t N, int32_t D) {
  if (H < 1 || N < 1 || D < 1) return 0;
  const int64_t G = (N + qmm::kAttnBlock - 1) / qmm::kAttnBlock;
  if (G <= 1) return 0;
  return (size_t)H * G * (D + 2) * sizeof(float);
}

qmm_status qmm_decode_attention(const void* q, const uint32_t* k_words, const void* k_scales,
                                const void* k_biases, const uint32_t* v_words,
                                const void* v_scales, const void* v_biases, void* out, int32_t H,
                                int32_t KV, int64_t N, int32_t D, int32_t bits,
                                int32_t group_size, void* workspace, size_t workspace_bytes,
                                void* stream) {
  if (!q || !k_words || !k_scales || !k_biases || !v_words || !v_scales || !v_biases || !out)
    return fail(QMM_ERR_INVALID_ARG, "NULL data pointer");
  if (!aligned(k_words, 16) || !aligned(v_words, 16) || !aligned(q, 4) || !aligned(out, 4) ||
      !aligned(k_scales, 2) || !aligned(k_biases, 2) || !aligned(v_scales, 2) ||
      !aligned(v_biases, 2))
    return fail(QMM_ERR_INVALID_ARG, "code words must be 16-byte aligned, q and out 4-byte aligned");
  if (H < 1 || KV < 1 || H % KV != 0)
    return fail(QMM_ERR_INVALID_ARG, "H=%d must be a positive multiple of KV=%d", H, KV);
  if (N < 1) return fail(QMM_ERR_INVALID_ARG, "N=%lld: the cache must hold a row", (long long)N);
  if (bits != 4 && bits != 8) return fail(QMM_ERR_UNSUPPORTED, "bits=%d: 4 and 8 are supported", bits);
  if (group_size != 32 && group_size != 64 && group_size != 128)
    return fail(QMM_ERR_UNSUPPORTED, "group_size=%d: 32, 64 and 128 are supported", group_size);
  const int rep = H / KV;
  if (!qmm::attention_supported(D, rep))
    return fail(QMM_ERR_UNSUPPORTED,
                "D=%d with %d query heads per KV head: D in {128, 256, 512}, heads per KV head "
                "in {1, 2, 4, 8}, their product <= 1024", D, rep);
  if (N > (int64_t)qmm::kAttnMaxBlocks * qmm::kAttnBlock || (int64_t)KV * N > (1LL << 31))
    return fail(QMM_ERR_UNSUPPORTED, "N=%lld: at most %d cached rows per head are supported",
                (long long)N, qmm::kAttnMaxBlocks * qmm::kAttnBlock);
  const int64_t G = (N + qmm::kAttnBlock - 1) / qmm::kAttnBlock;
  const size_t need = qmm_attention_workspace_bytes(H, N, D);
  if (need > 0) {
    if (!workspace || workspace_bytes < need)
      return fail(QMM_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                  workspace ? workspace_bytes : (size_t)0);
    if (!aligned(workspace, 16)) return fail(QMM_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  }
  qmm::AttnArgs a{};
  a.q = q;
  a.kw = k_words;
  a.ks = k_scales;
  a.kb = k_biases;
  a.vw = v_words;
  a.vs = v_scales;
  a.vb = v_biases;
  a.out = out;
  a.opart = need ? static_cast<float*>(workspace) : nullptr;
  a.stats = need ? static_cast<float*>(workspace) + (size_t)H * G * D : nullptr;
  a.H = H;
  a.KV = KV;
  a.N = (int)N;
  a.GS = group_size;
  a.G = (int)G;
  if (hipError_t e = qmm::launch_attention(bits, D, rep, a, reinterpret_cast<hipStream_t>(stream)))
    return hip_fail(e, "attention launch");
  return QMM_OK;
}

qmm_status qmm_debug_unpack(const qmm_plan* p, const void* codes, uint8_t* out, void* stream) {
  if (qmm_status st = check_plan(p)) return st;
  if (p->generic)
    return fail(QMM_ERR_UNSUPPORTED, "the vector-ALU kernel keeps MLX's layout: nothing to unpack");
  if (!codes || !out) return fail(QMM_ERR_INVALID_ARG, "NULL pointer");
  if (!aligned(codes, 4)) return fail(QMM_ERR_INVALID_ARG, "misaligned codes");
  const uint32_t* cw = static_cast<const uint32_t*>(codes);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = p->fmt ? qmm::launch_debug_unpack_fmt(p->d.bits, cw, out, (int)p->d.N, (int)p->d.K, st)
                        : qmm::launch_debug_unpack(p->d.bits, cw, out, (int)p->d.N, (int)p->d.K, st);
  if (e != hipSuccess) return hip_fail(e, "debug unpack launch");
  return QMM_OK;
}

qmm_status qmm_get_stats(const qmm_plan* p, qmm_stats* out) {
  if (qmm_status st = check_plan(p)) return st;
  if (!out) return fail(QMM_ERR_INVALID_ARG, "out is NULL");
  for (int i = 0; i < 8; ++i) out->launches[i] = p->launches[i].load();
  out->last_variant = p->last_variant;
  out->last_ntw = p->last_ntw;
  out->last_splitk = p->last_splitk;
  out->last_grid = p->last_grid;
  return QMM_OK;
}

const char* qmm_last_error(void) { return g_err.c_str(); }

qmm_status qmm_hbm_probe(const void* buf, size_t bytes, uint32_t* sink, int32_t grid,
                         void* stream) {
  if (!buf || !sink) return fail(QMM_ERR_INVALID_ARG, "NULL pointer");
  if (bytes == 0 || bytes % 16 != 0 || !aligned(buf, 16))
    return fail(QMM_ERR_INVALID_ARG, "bytes must be a positive multiple of 16, buf 16-byte aligned");
  if (grid < 0) return fail(QMM_ERR_INVALID_ARG, "grid must be >= 0");
  hipError_t e = qmm::launch_probe(buf, bytes, sink, grid ? grid : 4096,
                                   reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "probe launch");
  return QMM_OK;
}

}  // extern "C"
