/*
 * qmm.h -- C ABI of libqmm: y = x . W^T over MLX-style affine group-quantized
 * weights on AMD MI355X (gfx950).
 *
 * The operation.  [P1] = page "@mlx-bun/inference 0.0.0-stage -> 1.0.0"
 * (diffend npm page 53).
 *   - affine-split-mma.ts, header comment: matmul over MLX affine 3- or 4-bit,
 *     group-64 weights, y = x . W^T, for any number of activation rows; the
 *     row count is read at run time with one pipeline per projection shape.
 *   - affine-split-mma.ts, HEADER comment and helper affine_unit; affine3-mma.ts
 *     helper affine_q3; affine4-mma.ts helper affine_q4: codes are `bits`-bit
 *     fields of MLX's LSB-first bit stream of uint32 words, a 3-bit field may
 *     straddle two words, a 4-bit field never does.
 *   - affine3-mma.ts / affine4-mma.ts kernel bodies: row n of w starts at byte
 *     n*K*bits/8; scale and bias of (row n, group g) sit at n*(K/gs)+g; the
 *     weight is scale*q + bias.  The hot path is the pages' 3- and 4-bit,
 *     group-64 format; width 8 and group sizes 32 and 128 (which the pages
 *     name for their affine KV cache, "mlx-bun 0.0.4" page,
 *     fused-decode-kernel.ts) and MLX's width 2 run on the same matrix-core
 *     kernels through a second layout (qmm_desc).
 *   - affine-split-mma.ts, affineSplitMma(): x [..., K] times W^T gives
 *     [..., N] in x's dtype; it borrows its inputs and throws when there are
 *     no rows.  affineSplitMmaEligible(): a separate yes/no predicate (affine,
 *     group 64, bits 3 or 4, shape rules) under which the caller falls back.
 * So for rows m < M and outputs n < N, with gs the group size:
 *     y[m][n] = sum_k x[m][k] * (scale[n][k/gs] * q(n,k) + bias[n][k/gs]).
 * Beside it: the fused gate/up projection pair (qmm_run_gate_up), residual
 * add + RMS normalization (qmm_residual_rms_norm, and with the per-group
 * sums of its output for the projection, qmm_residual_rms_norm_ex and
 * qmm_run_sums) and decode attention over an affine-quantized KV cache
 * (qmm_decode_attention).
 * Summation order is the kernels' own (not bit-identical to any other
 * implementation); each kernel is deterministic run to run.
 *
 * Memory.  Every pointer argument that names data is a DEVICE pointer
 * (hipMalloc'd or a framework's device allocation) owned by the caller and
 * only borrowed until the enqueued work completes.  `stream` is a
 * hipStream_t (NULL = the default stream).  qmm_run and qmm_prepack only
 * enqueue work: they never synchronize and never allocate device memory.
 *
 * Errors.  Every entry point validates its arguments on the host before any
 * HIP call and returns a negative qmm_status on failure, with a message for
 * qmm_last_error().  QMM_ERR_INVALID_ARG: the format or an argument is wrong
 * (the page's "throw").  QMM_ERR_UNSUPPORTED: a valid format that no kernel
 * here covers (the page's "not eligible": the caller should fall back).
 */
#ifndef QMM_H_
#define QMM_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QMM_OK = 0,
  QMM_ERR_INVALID_ARG = -1,
  QMM_ERR_UNSUPPORTED = -2,
  QMM_ERR_HIP = -3,
  QMM_ERR_WORKSPACE = -4,
  QMM_ERR_NO_DEVICE = -5
} qmm_status;

/* Element types of x/y and of scales/biases. */
typedef enum { QMM_F32 = 0, QMM_BF16 = 1 } qmm_dtype;

/* Kernel families (qmm_run picks one; qmm_run_ex can force one). */
typedef enum {
  QMM_VARIANT_AUTO = 0,
  QMM_VARIANT_GEMV = 1,   /* vector-ALU kernels: for bf16 activations the streaming kernel's
                             structure with v_dot2_f32_bf16 products (1..4 rows per launch);
                             for f32 activations (the default for them) a kernel staging the
                             activations of its K split in LDS, 1..8 rows per pass */
  QMM_VARIANT_MFMA = 2,   /* blocked matrix-core kernel (bf16 in, f32 accumulate), 1..64 rows
                             per pass; bf16 activations only */
  QMM_VARIANT_STREAM = 3, /* matrix-core kernel for 1..4 rows per launch (more rows run as
                             blocks of 4): one workgroup per 16 rows of W, each wave stages
                             the activations of its own chunks and issues all its weight
                             loads up front; K <= 16384; bf16 activations; also runs the
                             other formats (default for 1..2 rows) */
  QMM_VARIANT_RESIDENT = 4, /* matrix-core kernel for 1..16 rows whose activation block fits in
                               one compute unit's LDS (rows*K*2 <= 160 KB, K <= 16384): one
                               workgroup holds up to four 16-row tiles of W, each wave takes
                               a share of K for all of them; bf16 activations; also runs the
                               other formats (default from 3 rows, as many rows per launch as
                               fit the LDS, at most 16) */
  QMM_VARIANT_SLAB = 5      /* matrix-core kernel for 17..64 rows per pass: one workgroup per
                               compute unit owning three 16-row tiles of W, activations streamed
                               through an LDS ring in slices of 512 columns by loader waves;
                               for 33..64 rows its split form: six tiles per workgroup, K cut
                               in two across workgroups, partial tiles added through the
                               workspace, 48-row blocks at 33..48 rows and 64-row blocks
                               above (ntw = 1 forces the unsplit form, ntw = 2 with
                               splitk = 2 the split one at 17..32 rows too);
                               built for K = 5120 and 8192; bf16 activations */,
  QMM_VARIANT_GENERIC = 6   /* vector-ALU kernel for the other formats (bits 2 and 8, and 3 or
                               4 with groups of 32) with f32 activations or f32 scales, on
                               MLX's own layout; 1..2 rows per pass; the only family such
                               plans run on */,
  QMM_VARIANT_WIDE = 7      /* matrix-core kernel for 65..128 rows per pass (the default above
                               64 rows where N/128 workgroups fill at least half the compute
                               units; 96-row blocks up to 96 rows, else 128): eight 16-row
                               tiles of W per workgroup, each weight
                               dequantized once to bf16 in registers (rounded to nearest
                               even) and the matrix cores accumulating over all of K;
                               K a multiple of 256; bf16 activations */
} qmm_variant;

/* qmm_desc.flags.  QMM_FLAG_F32_OUT: y is written as f32 [rows, N] whatever
 * x_dtype (the f32 sums before the output rounding), so that a test can judge
 * the accumulation apart from the rounding to bf16 (the pages fix no output
 * tolerance: "@mlx-bun/inference 0.0.0-stage -> 1.0.0" page,
 * affine-split-mma.ts header comment, results are not bit-identical to
 * MLX's).  qmm_run_gate_up rejects such plans (its output is bf16 by
 * definition). */
#define QMM_FLAG_F32_OUT 1u

/* Shape and format of one projection.  bits: 2, 3, 4 or 8 (5 and 6 are
 * UNSUPPORTED).  group_size: 32, 64 or 128.  3- and 4-bit weights with groups
 * of 64 or 128 run on every family in the native layout (a group of 128 as
 * two halves of 64 with the same scale and bias); the other formats with
 * bf16 activations and bf16 scales run on QMM_VARIANT_STREAM and
 * QMM_VARIANT_RESIDENT in the step layout (codes placed as the matrix cores'
 * operands of 32-column steps, so a group of 32, 64 or 128 is whole steps)
 * where a built shape covers K (K <= 16384; 8-bit codes with groups of 32 or
 * 64 up to K = 8192); with f32 activations or scales, or beyond those K, on
 * QMM_VARIANT_GENERIC in MLX's layout.  K: multiple of 128.  N: multiple of
 * 16.
 * max_rows: the largest row count qmm_run will be given (>= 1).
 * x_dtype: dtype of x and y.  sb_dtype: dtype of scales and biases.
 * flags: 0 or QMM_FLAG_F32_OUT (other bits: QMM_ERR_INVALID_ARG). */
typedef struct {
  int32_t bits;
  int32_t group_size;
  int64_t K;
  int64_t N;
  int32_t max_rows;
  int32_t x_dtype;
  int32_t sb_dtype;
  uint32_t flags;
} qmm_desc;

typedef struct qmm_plan qmm_plan;

typedef struct {
  uint64_t launches[8];   /* indexed by qmm_variant: kernels run per family */
  int32_t last_variant;   /* family of the last qmm_run */
  int32_t last_ntw;       /* output tiles (16 rows of W each) per wavefront */
  int32_t last_splitk;    /* K splits folded through the workspace */
  int32_t last_grid;      /* workgroups launched */
} qmm_stats;

/* Validate `desc` and build a plan (host state only; no device memory).
 * The plan records the compute-unit count of the device current at this
 * call (256 when no device answers), so that qmm_run validates and plans
 * without any HIP query.  Returns QMM_OK and *out, or an error and
 * *out = NULL. */
qmm_status qmm_create(const qmm_desc* desc, qmm_plan** out);

/* Free a plan.  NULL is allowed. */
void qmm_destroy(qmm_plan* plan);

/* Bytes of the two buffers of the kernel-native weight layout written by
 * qmm_prepack: packed codes (exactly N*K*bits/8, the MLX byte count) and
 * packed scales+biases (2*N*(K/group_size) elements of sb_dtype; for 3- and
 * 4-bit groups of 128, 2*N*(K/64): each group's pair is stored for both of
 * its halves). */
qmm_status qmm_packed_bytes(const qmm_plan* plan, size_t* codes_bytes, size_t* sb_bytes);

/* One-time weight loader: MLX layout -> kernel-native layout.
 *   w       uint32 [N, K*bits/32]  (MLX packed words, row-major)
 *   scales  sb_dtype [N, K/group_size]
 *   biases  sb_dtype [N, K/group_size]
 *   codes_out, sb_out: buffers of qmm_packed_bytes().
 * In the native layout (3- and 4-bit, groups of 64 or 128) and the step
 * layout (the other formats, bf16 activations and scales) the 16 rows x 128
 * columns of W that one wavefront multiplies are contiguous, and each lane's
 * codes are ordered so that the unpack to bf16 pairs is a shift and one
 * and-or per pair (8-bit codes: byte conversions).  Plans on MLX's layout
 * (f32 activations or scales of the other formats) copy the codes as they
 * are and store the scales, then the biases.  Enqueued on `stream`; the
 * inputs may be freed once it completes. */
qmm_status qmm_prepack(const qmm_plan* plan, const uint32_t* w, const void* scales,
                       const void* biases, void* codes_out, void* sb_out, void* stream);

/* Device workspace that qmm_run needs for `rows` rows (split-K partial sums
 * and per-tile tickets).  0 means none.  The workspace must be zero-filled
 * before its first use (a ticket counts the workgroups of one tile block that
 * have stored their partials, and the one that finds the count complete does
 * the fold; a count that does not start at zero cannot be told apart from
 * one in progress).  The kernel re-arms every ticket it used to zero before
 * it ends, so a completed qmm_run leaves the workspace ready for the next call
 * of any plan; there is no separate clearing launch.  Calls that overlap in
 * time must not share a workspace. */
size_t qmm_workspace_bytes(const qmm_plan* plan, int32_t rows);

/* y[rows, N] = x[rows, K] . W^T with W given in the native layout.  Rows
 * beyond one launch of the chosen family run as consecutive row blocks on
 * `stream`; a shorter last block runs on the family chosen for its own row
 * count.  Every argument is validated before the first HIP call.
 *   x: x_dtype [rows, K] row-contiguous, 16-byte aligned;
 *   y: x_dtype [rows, N] (f32 with QMM_FLAG_F32_OUT) row-contiguous, 4-byte
 *   aligned; only rows < `rows` are written;
 *   workspace: >= qmm_workspace_bytes(plan, rows) bytes (may be NULL when
 *   that is 0).
 * 1 <= rows <= max_rows, else QMM_ERR_INVALID_ARG (the page's "no rows"). */
qmm_status qmm_run(const qmm_plan* plan, const void* x, const void* codes, const void* sb,
                   void* y, int32_t rows, void* workspace, size_t workspace_bytes,
                   void* stream);

/* qmm_run with a forced kernel family and launch shape, for tests and
 * measurement (a forced family runs every row block).  ntw: tiles of 16 rows of W per wavefront (1, 2, 4; for the
 * RESIDENT family: tiles a workgroup holds at once, 1..4; for SLAB: 1 = the
 * unsplit form, 2 = the split form where it is built for this K and splitk,
 * else the unsplit form); kwaves: wavefronts of a workgroup that split K
 * between them (1, 2, 4; MFMA family only); splitk: workgroups that split K,
 * folded through the workspace (>= 1; SLAB's split form: 2).  Each may be 0
 * for the plan's choice. */
qmm_status qmm_run_ex(const qmm_plan* plan, int32_t variant, int32_t ntw, int32_t kwaves,
                      int32_t splitk, const void* x, const void* codes, const void* sb,
                      void* y, int32_t rows, void* workspace, size_t workspace_bytes,
                      void* stream);

/* Values per group of the group sums qmm_run_sums takes for this plan: 64
 * for 3- and 4-bit weights (a group of 128 is stored as two halves of 64 with
 * the same scale and bias), else the plan's group size.  0 for NULL. */
int32_t qmm_sum_group(const qmm_plan* plan);

/* qmm_run with the per-group sums of x given (the bias term of the factored
 * form sum_g s * sum(q x) + b * sum(x), page "@mlx-bun/inference 0.0.0-stage
 * -> 1.0.0", affine3-rows.ts header), as qmm_residual_rms_norm_ex writes
 * them while it produces x: x_sums f32 [K / qmm_sum_group(plan)][sums_ld],
 * element (g, m) the sum of x[m][g*G .. (g+1)*G) for G = qmm_sum_group(plan),
 * 16-byte aligned, sums_ld a multiple of 16 and >= rows rounded up to 16
 * (entries of rows >= `rows` are read and never affect y).  The streaming
 * and resident kernels use them in place of forming them (the resident
 * kernel where its shape has the registers for them and for row blocks
 * starting at a multiple of 16); the other families, and the vector-ALU
 * forms, form their own.  Otherwise as qmm_run;
 * QMM_ERR_INVALID_ARG for a NULL x_sums or a sums_ld outside these rules. */
qmm_status qmm_run_sums(const qmm_plan* plan, const void* x, const float* x_sums,
                        int32_t sums_ld, const void* codes, const void* sb, void* y,
                        int32_t rows, void* workspace, size_t workspace_bytes, void* stream);

/* Fused gate/up projections of a gated MLP with a SiLU-times-up epilogue
 * ("mlx-bun 0.4.0 -> 1.0.0" page, trellis-shared-m.ts, its gate/up kernel:
 * both projections of one activation row block, then sigmoid, SiLU and
 * product; applied here to affine weights):
 *   gate = x . Wg^T, up = x . Wu^T (f32 sums, as qmm_run), then
 *   h = bf16( bf16( bf16(gate) * bf16(sigmoid(bf16(gate))) ) * bf16(up) )
 * element by element, every intermediate rounded to bf16 round-to-nearest-
 * even as the unfused chain of bf16 operations would.  Wg and Wu share the
 * plan's shape (bits, K, N, group size 64) and are both in the native layout
 * of qmm_prepack.  x and h: bf16 [rows, K] and [rows, N], row-contiguous.
 * Every activation row block of up to 16 rows is read once for both
 * projections.  tile_pairs: 16-column tiles of each projection per
 * workgroup (1 or 2; 0 = the plan's choice, 1).  No workspace.
 * Errors: QMM_ERR_UNSUPPORTED for f32 activations, or when 16 rows x K bf16
 * activations (fewer if rows < 16) exceed 160 KB or K > 8192;
 * QMM_ERR_INVALID_ARG for NULL or misaligned pointers and rows outside
 * 1..max_rows; QMM_ERR_HIP for launch failures. */
qmm_status qmm_run_gate_up(const qmm_plan* plan, const void* x, const void* gate_codes,
                           const void* gate_sb, const void* up_codes, const void* up_sb,
                           void* h, int32_t rows, int32_t tile_pairs, void* stream);

/* Residual add + RMS normalization producing the activations a projection
 * consumes ("@mlx-bun/inference 0.0.0-stage -> 1.0.0" page, residual-rms-
 * norm.ts).  Per row of D values, T = dtype (QMM_BF16 or QMM_F32), R = round
 * to T (nearest, ties to even):
 *   residual[i]   = R(x[i] + update[i])
 *   normalized[i] = R(weight[i] * R(residual[i] / sqrt(mean_i residual^2 + eps)))
 * with the sum of squares and the scaling in f32.  x, update, residual and
 * normalized: T [rows, D] row-contiguous; weight: T [D]; all 16-byte aligned;
 * residual and normalized must not overlap the inputs.  D: a multiple of 8,
 * 8..16384 (else QMM_ERR_UNSUPPORTED); rows >= 1, eps finite and >= 0 (else
 * QMM_ERR_INVALID_ARG).  Enqueued on `stream`; no plan, no workspace. */
qmm_status qmm_residual_rms_norm(const void* x, const void* update, const void* weight,
                                 void* residual, void* normalized, int32_t rows, int64_t D,
                                 float eps, int32_t dtype, void* stream);

/* qmm_residual_rms_norm that also writes, when group_sums is not NULL, the
 * sum of every group of group_size (32, 64, 128) stored normalized values:
 * group_sums[g * sums_ld + m] = sum over i in [g*group_size, (g+1)*group_size)
 * of normalized[m][i] as stored (each thread adds its 8 values in order, the
 * threads of a group add their partial sums by lane swaps in a fixed order;
 * f32).  These are the sums qmm_run_sums takes for the projection that reads
 * `normalized` (group_size = qmm_sum_group of its plan; sums_ld as that call
 * needs).  Errors as qmm_residual_rms_norm, plus QMM_ERR_INVALID_ARG for a
 * group size other than 32, 64, 128, D not a multiple of it, sums_ld < rows
 * or a misaligned group_sums. */
qmm_status qmm_residual_rms_norm_ex(const void* x, const void* update, const void* weight,
                                    void* residual, void* normalized, float* group_sums,
                                    int32_t group_size, int32_t sums_ld, int32_t rows, int64_t D,
                                    float eps, int32_t dtype, void* stream);

/* Decode attention over an affine-quantized KV cache ("mlx-bun 0.0.4" page,
 * fused-decode-kernel.ts): one query row per head, head h attending to all N
 * cached rows of KV head h / (H / KV).  Keys and values are stored like MLX
 * affine weights: k_words/v_words uint32 [KV, N, D*bits/32], codes packed
 * along D least significant bits first; k_scales, k_biases, v_scales,
 * v_biases bf16 [KV, N, D/group_size]; value = scale * code + bias.
 *   score[h, n] = bf16(q[h] . k[kv, n])      (no extra scale: q arrives scaled)
 *   out[h]      = bf16(sum_n e^score[h, n] v[kv, n] / sum_n e^score[h, n])
 * with every sum in f32.  q, out: bf16 [H, D]; all buffers device memory,
 * row-contiguous, borrowed until the enqueued work completes; code words
 * 16-byte aligned.  The cache is split into blocks of 256 rows whose partial
 * results are merged in block order (bitwise reproducible).  workspace: >=
 * qmm_attention_workspace_bytes(H, N, D) bytes (none when N <= 256; no
 * zero-fill needed).  Errors: QMM_ERR_INVALID_ARG for NULL or misaligned
 * pointers, N < 1 or H not a multiple of KV; QMM_ERR_UNSUPPORTED for bits
 * other than 4 and 8, group sizes other than 32, 64, 128, D outside
 * {128, 256, 512} or H/KV outside {1, 2, 4, 8} or D * H/KV > 1024, or N
 * above 2^21 rows;
 * QMM_ERR_WORKSPACE for a missing or short workspace; QMM_ERR_HIP for launch
 * failures.  Enqueued on `stream`. */
size_t qmm_attention_workspace_bytes(int32_t H, int64_t N, int32_t D);
qmm_status qmm_decode_attention(const void* q, const uint32_t* k_words, const void* k_scales,
                                const void* k_biases, const uint32_t* v_words,
                                const void* v_scales, const void* v_biases, void* out, int32_t H,
                                int32_t KV, int64_t N, int32_t D, int32_t bits,
                                int32_t group_size, void* workspace, size_t workspace_bytes,
                                void* stream);

/* The largest workspace qmm_run_noalloc holds on a device. */
#define QMM_NOALLOC_MAX_WORKSPACE (8u << 20)

/* qmm_run for callers that cannot allocate device memory: code under HIP
 * graph capture, serving loops and harnesses that forbid hipMalloc.  Same
 * arguments and results as qmm_run, without the workspace: the split-K
 * workspace (ticket words, then partial tiles) comes from a device array of
 * QMM_NOALLOC_MAX_WORKSPACE bytes that the library holds on every device it
 * runs on until the process ends.  It allocates nothing (no hipMalloc,
 * hipFree or allocating library call).  Errors: those of qmm_run, and
 * QMM_ERR_WORKSPACE, before any HIP call, when the call needs more workspace
 * than the array holds (qmm_workspace_bytes_ex(plan, QMM_VARIANT_AUTO, 0, 0,
 * 0, rows) > QMM_NOALLOC_MAX_WORKSPACE; the 3-bit 5120 -> 10240 projection
 * at 64 rows needs 5.3 MB).  All calls on one device share that device's array, which
 * keeps the last call's contents: calls that overlap in time on one device
 * (two streams, two host threads) race, and the caller must order them.
 * The array's ticket words start at zero, and every completed call leaves
 * them at zero. */
qmm_status qmm_run_noalloc(const qmm_plan* plan, const void* x, const void* codes,
                           const void* sb, void* y, int32_t rows, void* stream);

/* Workspace needed by qmm_run_ex with the same variant/ntw/kwaves/splitk. */
size_t qmm_workspace_bytes_ex(const qmm_plan* plan, int32_t variant, int32_t ntw,
                              int32_t kwaves, int32_t splitk, int32_t rows);

/* Test hook: decode the native or step layout with the compute kernels' own
 * unpack and write the codes q(n,k) as uint8 [N, K] (device buffer);
 * QMM_ERR_UNSUPPORTED for plans that keep MLX's layout. */
qmm_status qmm_debug_unpack(const qmm_plan* plan, const void* codes, uint8_t* codes_nk,
                            void* stream);

/* Launch counters of a plan (host memory). */
qmm_status qmm_get_stats(const qmm_plan* plan, qmm_stats* out);

/* Message of the last failed call on this thread ("" if none). */
const char* qmm_last_error(void);

/* Measurement hook: stream-read `bytes` (multiple of 16) of device memory at
 * `buf` and write one uint32 per workgroup to `sink` (`grid` entries;
 * grid = 0 picks 4096).  Used to measure the achievable HBM read rate. */
qmm_status qmm_hbm_probe(const void* buf, size_t bytes, uint32_t* sink, int32_t grid,
                         void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QMM_H_ */
