/*
 * w4a16.h -- C ABI of libw4a16.so, the MI355X (gfx950) W4A16 group-quantized projection.
 *
 * Operation (every compute entry point):
 *
 *     y[m, n] = bf16( sum_k x[m, k] * w[n, k] ),   w[n, k] = s[n, k/128] * q[n, k] + b[n, k/128]
 *
 * a "quantized linear" projection of bf16 activations by 4-bit affine weights with one bf16
 * scale and one bf16 bias per 128 reduction values of each output column, fp32 accumulation,
 * and one rounding of the result to bf16.  Sources: tiny-llm book, "Week 2 Day 6: SIMD-Matrix
 * Prefill" -- opening scope list (four-bit weights, group size 128, BF16 activations,
 * quantization parameters and output, FP32 matrix accumulators), Task 1 (matvec for M <= 8,
 * tiled matrix kernel for M > 8, 16-bit result dtype), Task 3 (one scale and bias per 128
 * reduction values, cast once at the final store); "Route affine qmv_wide by bit-width and
 * batch size #5" (affine group dequantization reused across the M input rows).
 *
 * Layouts (all row-major, contiguous; the pages leave these open and this library fixes them):
 *   x       bf16  [M, K]      bit patterns passed as uint16_t
 *   wq      u32   [N, K/8]    code q[n, 8j+i] in bits 4i..4i+3 of wq[n, j] (low nibble first)
 *   scales  bf16  [N, K/128]
 *   biases  bf16  [N, K/128]
 *   y       bf16  [M, N]      overwritten, never accumulated into
 *
 * Ownership: every pointer is caller-owned device memory (for example torch tensors).  The
 * library allocates nothing on the compute paths, keeps no pointer after a call returns and
 * only enqueues work on `stream` (a hipStream_t; NULL = the null stream).  Buffers must stay
 * alive until that work completes; y must not overlap any input.  Calls are asynchronous:
 * a fault during execution surfaces when the caller synchronizes the stream.
 *
 * Preconditions checked on the host (a violation returns an error status, never launches):
 *   1 <= M, N <= 2^31 - 1;  1 <= K <= 2^20;  K % 128 == 0;  group == 128;
 *   x, wq, workspace 16-byte aligned;  scales, biases, y 2-byte aligned;
 *   the output's bytes disjoint from every input's (by address range; the workspace is not
 *   compared and must not overlap any other buffer).
 *
 * Errors are returned as status codes (never exceptions); w4a16_status_string() names them.
 * A case outside what an entry point serves is an error of its own (W4A16_ERR_UNSUPPORTED),
 * never a silently different computation: the convention of raising NotImplementedError for
 * unsupported cases in "MLX Metal Kernels v0.20.0", Known limitations (continuation prefill).
 * Thread safety: stateless apart from a per-device cache of the compute-unit count, the
 * per-device scratch of w4a16_linear_noalloc and the per-thread request of
 * w4a16_time_next_launch.
 */
#ifndef W4A16_H
#define W4A16_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define W4A16_ABI_VERSION 1
#define W4A16_GROUP 128

enum w4a16_status {
    W4A16_OK = 0,
    W4A16_ERR_NULL = 1,        /* a required pointer is NULL                                  */
    W4A16_ERR_SHAPE = 2,       /* a size outside the limits above, or K % 128 != 0           */
    W4A16_ERR_GROUP = 3,       /* group != 128                                                */
    W4A16_ERR_ALIGN = 4,       /* a pointer violates the alignment stated above               */
    W4A16_ERR_WORKSPACE = 5,   /* a forced split_k > 1 has too little workspace               */
    W4A16_ERR_UNSUPPORTED = 6, /* valid arguments this entry point does not serve (qmv, M > 8)*/
    W4A16_ERR_LAUNCH = 7,      /* the HIP runtime rejected a launch                           */
    W4A16_ERR_DEVICE = 8,      /* the device could not be queried                             */
    W4A16_ERR_OVERLAP = 9      /* an output shares bytes with an input                        */
};

enum w4a16_path {
    W4A16_PATH_AUTO = 0,       /* dispatch: M <= 8 -> qmv ("Week 2 Day 6", Task 1), 8 < M <= 32
                                  -> skinny, M > 32 -> qmm                                       */
    W4A16_PATH_QMV = 1,        /* wavefront matvec for decode rows                                */
    W4A16_PATH_QMM = 2,        /* MFMA-tiled matrix path for prefill rows                         */
    W4A16_PATH_SKINNY = 3,     /* 8 < M <= 32 under AUTO (any M <= 32 when asked for): the matvec
                                  kernels up to 16 rows, 32-row MFMA tiles with deterministic
                                  split-K above (the small-batch regime 8 < rows <= 32 that
                                  "Feature Request: Metal prefill speedup (~68%) on M5 Max",
                                  Related work, names for skinny tiles + deterministic split-K)  */
    W4A16_PATH_GATE_UP = 4,    /* reported by w4a16_gate_up_plan only: the fused gate / up tiles  */
    W4A16_PATH_W4A8 = 5,       /* reported by w4a8_plan only: int8-activation tiles               */
    W4A16_PATH_GROUPED = 6,    /* reported by w4a16_grouped_plan only: one tile launch over the
                                  column tiles of every projection                                */
    W4A16_PATH_PER_PROJECTION = 7 /* reported by w4a16_grouped_plan only: one w4a16_linear dispatch
                                  per projection                                                  */
};

/* Launch plan chosen by the dispatch policy (filled by w4a16_plan). */
typedef struct w4a16_plan {
    int32_t path;              /* W4A16_PATH_QMV, _QMM or _SKINNY                          */
    int32_t tile_m;            /* rows per workgroup tile, or 16 for the matvec kernels     */
    int32_t tile_n;            /* output columns per workgroup                              */
    int32_t tile_k;            /* reduction values per pipeline step (one group = 128)     */
    int32_t grid_x;            /* workgroups along N                                        */
    int32_t grid_y;            /* workgroups along M                                        */
    int32_t grid_z;            /* split-K slices (qmm) or 1                                 */
    int32_t block_threads;     /* threads per workgroup                                     */
    int32_t split_k;           /* S: number of K slices (1 = unsplit)                       */
    int32_t k_waves;           /* waves of one workgroup that split K (1 = none): qmv waves
                                  over groups; qmm tiles with two waves per column strip  */
    int32_t num_cus;           /* compute units the plan was made for                       */
    int32_t variant;           /* kernel instance index (diagnostic); qmm and gate / up plans
                                  add 10 when they run the exact-code form (see qmm_w4a16)    */
    uint64_t workspace_bytes;  /* the exact-code form's activation group sums, then the fp32
                                  partials when split_k > 1 (S * M * N * 4; twice that for
                                  the gate / up pair)                                         */
} w4a16_plan_t;

/* ABI version of the loaded library (W4A16_ABI_VERSION). */
int w4a16_abi_version(void);

/* Static, NUL-terminated name of a status code ("W4A16_OK", ...); unknown codes give "unknown". */
const char* w4a16_status_string(int status);

/*
 * Kernel timestamps for measurement (the per-launch device time that the roofline fraction of a
 * projection is computed from).  Arms a request on the calling host thread: the next
 * contraction kernel that this thread launches through any entry point below (a tile or matvec
 * kernel; not the group-sum pre-pass of the exact-code form nor a split-K slice sum) is launched
 * with hipExtLaunchKernel, which sets start_event / stop_event to that kernel's execution start
 * and end (so hipEventElapsedTime over them gives the kernel's own duration, without the launch
 * overhead and the end-of-kernel system-scope cache flush that events recorded on the stream
 * around the call also span).  The launch consumes the request; an entry point that returns an
 * error before launching leaves it armed.  start_event and stop_event are hipEvent_t handles
 * created by the caller (either may be null); passing two nulls cancels the request.  A launch
 * into a stream under HIP graph capture consumes the request without timing (the kernel is
 * captured as a plain launch and the events are left as they were).  Returns W4A16_OK.
 */
int w4a16_time_next_launch(void* start_event, void* stop_event);

/*
 * Dispatch policy ("Week 2 Day 6", Task 1 for the M threshold; Task 5 and "Benchmark Analysis:
 * Identify Under-Filled Prefill Shapes" for splitting K only when the tile grid under-fills the
 * GPU).  path: W4A16_PATH_AUTO / _QMV / _QMM / _SKINNY.  split_k: 0 = policy, 1 = never split, S > 1 =
 * exactly S slices (clamped to the number of groups).  num_cus: compute units to plan for;
 * 0 = query the current device.  Pure host arithmetic; `out` is caller-owned.
 * Returns W4A16_OK, _ERR_NULL, _ERR_SHAPE, _ERR_GROUP, _ERR_UNSUPPORTED (qmv with M > 8,
 * skinny with M > 32, unknown path) or _ERR_DEVICE.
 */
int w4a16_plan(int64_t M, int64_t N, int64_t K, int32_t group, int32_t path, int32_t split_k,
               int32_t num_cus, w4a16_plan_t* out);

/*
 * Workspace bytes w4a16_linear needs for this shape under the policy (0 when the plan needs
 * neither group sums nor partials).  num_cus as in w4a16_plan.  Returns 0 for invalid shapes.
 */
uint64_t w4a16_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t group, int32_t num_cus);

/*
 * Decode-row matvec, 1 <= M <= 8 ("Week 2 Day 6", Task 1: the Day 3 matvec serves M <= 8;
 * "Route affine qmv_wide ...": a dequantized group is reused across the M rows).  Needs no
 * workspace.  M > 8 returns W4A16_ERR_UNSUPPORTED.  The kernel family follows w4a16_plan: up
 * to 4 rows below 32k columns (at 1 and 2 rows up to 128 groups, at 3 and 4 up to 80) and 5 to
 * 8 rows below 16k columns up to 64 groups the burst kernel, whose waves issue all of their
 * loads at once; wider heads the persistent wide kernel.
 */
int qmv_w4a16(const uint16_t* x, const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
              uint16_t* y, int64_t M, int64_t N, int64_t K, int32_t group, void* stream);

/*
 * Tiled matrix path for any M >= 1 ("Week 2 Day 6", "From a Matvec to a Cooperative Tile",
 * Tasks 2 and 3), with optional split-K (Task 5: a temporary buffer and a second launch).
 * split_k: 0 = policy, 1 = off, S > 1 = forced (clamped to the number of groups).
 *
 * Two forms of the same product (both within the parity tolerance, integer cases identical):
 * tiles of up to 96 rows (M <= 1024) dequantize each weight to bf16 in registers; the 128-row
 * tiles (M > 1024) multiply the raw codes on the matrix core, scale each group's fp32 product
 * once and add sum_g b * X from the activations' per-group sums, which a first launch writes
 * to the start of `workspace` (bf16 [M, 2G rounded up to 16], padded to 256 bytes).
 *
 * `workspace` (16-byte aligned) holds, in order, those group sums (exact-code form only) and,
 * when the plan splits, S * M * N fp32 partials; w4a16_plan().workspace_bytes is the total.
 * The slices are summed in slice order, so results are deterministic.  With too little
 * workspace the call drops the exact-code form, then (under the policy) the split, both of
 * which compute the same result; a forced S > 1 without room for its partials returns
 * W4A16_ERR_WORKSPACE.
 */
int qmm_w4a16(const uint16_t* x, const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
              uint16_t* y, int64_t M, int64_t N, int64_t K, int32_t group, int32_t split_k,
              void* workspace, size_t workspace_bytes, void* stream);

/*
 * The quantized-linear entry point: dispatch by M (qmv for M <= 8, the skinny path for
 * 8 < M <= 32, qmm beyond, each with the policy's split).  Same arguments and errors as
 * qmm_w4a16 with split_k = 0.
 */
int w4a16_linear(const uint16_t* x, const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                 uint16_t* y, int64_t M, int64_t N, int64_t K, int32_t group,
                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * Allocation-free variant of w4a16_linear, for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same dispatch
 * and arguments as w4a16_linear, without a workspace argument, plus split_k as for qmm_w4a16
 * (0 = policy, 1 = off, S > 1 = forced).  The split-K partials and the exact-code form's group
 * sums live in a device array of W4A16_NOALLOC_SCRATCH_BYTES inside the library, one per GPU,
 * kept until the process ends; the call allocates nothing and calls no allocating routine.
 * Under the policy the plan is fitted to that scratch exactly as w4a16_linear fits it to a short
 * workspace (same result); a forced split_k whose partials (S * M * N * 4 bytes) exceed it returns
 * W4A16_ERR_WORKSPACE.  The first call on a device resolves that device's scratch address
 * (W4A16_ERR_DEVICE if it cannot).  The scratch keeps the last call's contents; every value a
 * call reads from it is written earlier in the same call, so nothing needs clearing.  Calls that
 * overlap on one GPU (concurrent streams or host threads) share the scratch and race: the
 * caller must order them.  Other preconditions and errors as w4a16_linear.
 */
#define W4A16_NOALLOC_SCRATCH_BYTES (32u << 20)
int w4a16_linear_noalloc(const uint16_t* x, const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                         uint16_t* y, int64_t M, int64_t N, int64_t K, int32_t group, int32_t split_k, void* stream);

/*
 * Projections of one input in one call, for projections that read the same activations (the
 * query, key and value projections of an attention layer):
 *
 *     y_p = x . dequant(Wq_p)^T,   p = 0 .. count - 1,   1 <= count <= W4A16_MAX_GROUPED,
 *
 * each with the layouts above: x [M, K] shared, wq[p] uint32 [N[p], K / 8], scales[p] and
 * biases[p] bf16 [N[p], K / 128], y[p] bf16 [M, N[p]].  The pointer arrays and N are host
 * memory; the buffers they point to are device memory owned by the caller.
 *
 * "Week 2 Day 6: SIMD-Matrix Prefill", Benchmark Analysis (Identify Under-Filled Prefill
 * Shapes) and the paragraph before it: a short, narrow key / value projection has too few result
 * tiles to occupy the GPU, and splitting K adds a temporary buffer and another launch.  Here,
 * with more than 32 rows, the projections' 128-column tiles form one grid of one launch (the
 * tile form the qmm policy takes for M rows and the summed tile columns, never split; a
 * projection's last tile may be ragged), so the key and value tiles run beside the query tiles.
 * With at most 32 rows, or count = 1, every projection runs its own w4a16_linear dispatch.
 * Results equal those of w4a16_linear per projection within the tolerance stated at qmm_w4a16
 * (bit for bit where both take the same tile form).
 *
 * Workspace: w4a16_grouped_plan().workspace_bytes (the exact-code form's group sums of x, shared
 * by the projections; or the largest per-projection workspace); with too little the call drops
 * the exact-code form (same result within the tolerance).  Errors as w4a16_linear for every
 * projection, plus: count outside 1 .. W4A16_MAX_GROUPED -> W4A16_ERR_SHAPE; a null pointer
 * array -> W4A16_ERR_NULL; an output sharing bytes with any input or another output ->
 * W4A16_ERR_OVERLAP.  All validation happens before any launch.
 */
#define W4A16_MAX_GROUPED 4
int w4a16_linear_grouped(const uint16_t* x, int32_t count, const uint32_t* const* wq,
                         const uint16_t* const* scales, const uint16_t* const* biases, uint16_t* const* y,
                         const int64_t* N, int64_t M, int64_t K, int32_t group, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * Plan of w4a16_linear_grouped: path W4A16_PATH_GROUPED with the one launch's tiles (grid_x =
 * the summed column tiles, split_k = 1), or W4A16_PATH_PER_PROJECTION (the first projection's
 * plan), or, for count = 1, w4a16_plan's plan; workspace_bytes as above.  num_cus as in
 * w4a16_plan.  Pure host arithmetic.  Returns W4A16_OK, _ERR_NULL, _ERR_SHAPE, _ERR_GROUP or
 * _ERR_DEVICE.
 */
int w4a16_grouped_plan(int32_t count, const int64_t* N, int64_t M, int64_t K, int32_t group, int32_t num_cus,
                       w4a16_plan_t* out);

/*
 * Fused gate / up projection pair with SwiGLU (the SwiGLU fused into the mat-mat, and gate / up
 * computed together with the GLU in the mat-mat epilogue, named by "Feature Request: Metal
 * prefill speedup (~68%) on M5 Max": feature list and Related work):
 *
 *     h[m, n] = bf16( silu(g[m, n]) * u[m, n] ),   silu(z) = z / (1 + e^-z),
 *     g = x . dequant(Wq_gate)^T,  u = x . dequant(Wq_up)^T   (fp32, never rounded to bf16)
 *
 * One tile kernel reads each activation fragment once for both projections and writes only h.
 * Both weight sets have the layouts above with the same N and K; h is bf16 [M, N].  Any M >= 1:
 * 32-row tiles up to 32 rows; above, 64-row tiles in the exact-code form described at
 * qmm_w4a16 (codes on the matrix core, the bias term from the activations' group sums), or,
 * when the workspace has no room for the group sums, dequantizing tiles (64 rows up to ~1k,
 * 128 beyond; same result within the tolerance).  Unsplit grids that 96-row tiles cover in
 * fewer rounds of tiles per compute unit (at most two) run dequantizing 96-row tiles.  split_k as for qmm_w4a16.  Workspace
 * (w4a16_gate_up_plan().workspace_bytes): [group sums, exact-code form][gate partials][up
 * partials], the partials 2 * S * M * N fp32 of a split plan, summed in slice order before the
 * SiLU, so results are deterministic.  Same preconditions, ownership and errors as qmm_w4a16
 * (every pointer checked for null and alignment; h overlapping x or either weight set returns
 * W4A16_ERR_OVERLAP).
 */
int w4a16_gate_up_swiglu(const uint16_t* x, const uint32_t* wq_gate, const uint16_t* scales_gate,
                         const uint16_t* biases_gate, const uint32_t* wq_up, const uint16_t* scales_up,
                         const uint16_t* biases_up, uint16_t* h, int64_t M, int64_t N, int64_t K, int32_t group,
                         int32_t split_k, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Launch plan of w4a16_gate_up_swiglu (path = W4A16_PATH_GATE_UP): tiles, split and workspace
 * bytes.  split_k and num_cus as in w4a16_plan.  Pure host arithmetic.  Returns W4A16_OK,
 * _ERR_NULL, _ERR_SHAPE, _ERR_GROUP or _ERR_DEVICE.
 */
int w4a16_gate_up_plan(int64_t M, int64_t N, int64_t K, int32_t group, int32_t split_k, int32_t num_cus,
                       w4a16_plan_t* out);

/* Kernel choice of qmv_affine ("Route affine qmv_wide by bit-width and batch size #5"). */
enum w4a16_qmv_mode {
    W4A16_QMV_POLICY = 0,      /* route by (bits, M) as measured on MI355X                         */
    W4A16_QMV_AMORTIZED = 1,   /* row-amortized: one unpacked group feeds all M rows (matrix core)  */
    W4A16_QMV_PER_ROW = 2,     /* per-row dot products, M <= 2                                      */
    W4A16_QMV_FAMILIES = 3,    /* bits = 4 only: the kernel families and policy of qmv_w4a16        */
    W4A16_QMV_BURST = 4        /* M <= 8: every wave issues all of its loads at once; up to 4 rows
                                  4 K slices in the matrix core's spare rows (below 32k columns, at
                                  most 128 groups; beyond 160 blocks of 16 columns or 64 groups only
                                  up to 2 rows), else 16-column blocks (3 to 8 rows below 16k
                                  columns, at most 80 groups up to 4 rows and 64 beyond)          */
};

/*
 * Affine matvec for decode rows (1 <= M <= 8) at bits = 1, 2, 3, 4 or 8 per code, routed by
 * (bits, M) between a per-row kernel and a row-amortized one ("Route affine qmv_wide by
 * bit-width and batch size #5" routes 1-bit and small M per row and larger M row-amortized).
 * Measured on MI355X the row-amortized kernel leads the per-row one at every width and M, and
 * the burst form leads both where it applies, so the policy takes the burst form there and the
 * row-amortized kernel elsewhere; at bits = 4 the policy is qmv_w4a16's.  Layouts as above with wq uint32 [N, K * bits / 32]:
 * a row's words are one bit stream, lowest bits first (stream bit t = bit t % 32 of word t / 32),
 * element k in stream bits bits*k .. bits*k + bits - 1 -- at 1, 2, 4 and 8 bits element
 * (32/bits)*j + i in bits bits*i .. of word j, at 3 bits codes 10 and 21 of every 32 straddle a
 * word; scales and biases bf16 [N, K/128]; w = s * q + b.  mode: enum w4a16_qmv_mode.  Needs no
 * workspace.  Same preconditions, ownership and errors as qmv_w4a16; bits outside {1, 2, 3, 4, 8},
 * M > 8, an unknown mode, the per-row mode with M > 2, W4A16_QMV_FAMILIES with bits != 4, or
 * W4A16_QMV_BURST outside its shapes return W4A16_ERR_UNSUPPORTED.
 */
int qmv_affine(const uint16_t* x, const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
               uint16_t* y, int64_t M, int64_t N, int64_t K, int32_t group, int32_t bits, int32_t mode,
               void* stream);

/*
 * Plan of qmv_affine (path = W4A16_PATH_QMV; variant = the chosen enum w4a16_qmv_mode; with
 * W4A16_QMV_FAMILIES the tile and grid fields are those of w4a16_plan's matvec plan).  num_cus
 * as in w4a16_plan.  Pure host arithmetic.  Errors as qmv_affine, plus W4A16_ERR_NULL for `out`;
 * W4A16_QMV_FAMILIES with bits != 4 returns W4A16_ERR_UNSUPPORTED.
 */
int qmv_affine_plan(int64_t M, int64_t N, int64_t K, int32_t group, int32_t bits, int32_t mode,
                    int32_t num_cus, w4a16_plan_t* out);

/*
 * W4A8: the same 4-bit affine weights with int8 activations on the int8 matrix cores (the int8
 * mat-mat for large batches that "Feature Request: Metal prefill speedup (~68%) on M5 Max (NAX /
 * tensor API kernels)" lists in its feature list and Related work; the page gives no recipe).
 * Reading taken: each activation row m is quantized symmetrically, all in fp32,
 *
 *     a = max_k |x[m, k]|,  inv = 127 / a,  sx[m] = a / 127   (correctly rounded; a = 0 gives 0),
 *     xq[m, k] = clamp(rint(x[m, k] * inv), -127, 127)         (product rounded to fp32, ties even),
 *
 * and the projection uses sx * xq in place of x:  y[m, n] = bf16( sum_k sx[m] xq[m, k] w[n, k] ),
 * computed as sx[m] * (sum_g s[n, g] P[m, n, g] + sum_g b[n, g] X[m, g]) with the exact integer
 * group products P = sum_{k in g} xq q and group sums X = sum_{k in g} xq.  Inputs must be finite.
 *
 * Activation buffers (made by w4a8_quantize_rows, read by qmm_w4a8; caller-owned device memory):
 *   xq    int8 [M, K], 16-byte aligned: each aligned run of 8 values k0..k7 is stored in the
 *         order k0 k2 k4 k6 k1 k3 k5 k7 (the order of the kernel's code operand)
 *   sx    fp32 [M], 4-byte aligned
 *   xsum  bf16 [M, w4a8_xsum_cols(K)], 16-byte aligned: xsum[m, 2g] + xsum[m, 2g + 1] = X[m, g]
 *         exactly (the multiple of 128 and the remainder 0..127), zeros beyond 2G
 */

/* Columns of xsum for a given K: 2 * K / 128 rounded up to a multiple of 16 (0 for invalid K). */
int64_t w4a8_xsum_cols(int64_t K);

/*
 * Quantize the rows of x (bf16 [M, K]) into xq, sx and xsum as described above.  One launch on
 * `stream`.  Errors: W4A16_ERR_NULL, _ERR_SHAPE (M < 1, K outside the limits), _ERR_GROUP,
 * _ERR_ALIGN, _ERR_LAUNCH.
 */
int w4a8_quantize_rows(const uint16_t* x, int8_t* xq, float* sx, uint16_t* xsum, int64_t M, int64_t K, int32_t group,
                       void* stream);

/*
 * Launch plan of qmm_w4a8 (path = W4A16_PATH_W4A8): 32-row tiles up to 32 rows, 64 up to ~1k,
 * 128 beyond; the split rule of qmm_w4a16.  64-row grids of at most one work unit (tile x
 * slice) per compute unit run eight waves per tile, two per 32-column block (k_waves = 2,
 * block_threads = 512).  workspace_bytes = the fp32 partials (S * M * N * 4) when the plan
 * splits.  split_k and num_cus as in w4a16_plan.  Pure host arithmetic.
 */
int w4a8_plan(int64_t M, int64_t N, int64_t K, int32_t group, int32_t split_k, int32_t num_cus, w4a16_plan_t* out);

/*
 * int8-activation tile path for any M >= 1 over buffers from w4a8_quantize_rows; weights, y,
 * split_k, workspace and errors as for qmm_w4a16 (the slices are summed in slice order).
 */
int qmm_w4a8(const int8_t* xq, const float* sx, const uint16_t* xsum, const uint32_t* wq, const uint16_t* scales,
             const uint16_t* biases, uint16_t* y, int64_t M, int64_t N, int64_t K, int32_t group, int32_t split_k,
             void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes of w4a8_linear: the three activation buffers plus the policy's partials. */
uint64_t w4a8_linear_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t group, int32_t num_cus);

/*
 * One-call W4A8 projection of bf16 x: w4a8_quantize_rows into the start of `workspace` (256-byte
 * aligned, at least w4a8_linear_workspace_bytes), then qmm_w4a8 under the policy with the rest
 * of the workspace for partials (a policy split without room falls back to S = 1).  Same
 * preconditions and errors as qmm_w4a16; a missing or short workspace returns
 * W4A16_ERR_WORKSPACE, a misaligned one W4A16_ERR_ALIGN.
 *
 * Nothing routes to this path by itself: the caller chooses it.  Measured on MI355X (each call
 * alone, weights from HBM) against the W4A16 entry points on the same shapes: at 512 rows it is
 * within 3% of them on the 2560 -> 9728 gate and up projections (ahead or behind from run to
 * run) and slower on the narrower ones (q 2560 -> 4096 by 21%, k and v 2560 -> 1024 by 28-30%,
 * o 4096 -> 2560 by 16-19%, down 9728 -> 2560 by 6-7%): the per-group int32 -> fp32 conversion and scaling of the group products costs about as
 * much vector-ALU time as the int8 matrix rate saves.  At 4096 rows it is slightly faster.
 */
int w4a8_linear(const uint16_t* x, const uint32_t* wq, const uint16_t* scales, const uint16_t* biases, uint16_t* y,
                int64_t M, int64_t N, int64_t K, int32_t group, void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* W4A16_H */
