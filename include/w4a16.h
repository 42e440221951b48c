/*
 * w4a16.h -- C ABI of the MI355X (gfx950) W4A16 weight-only GEMM library.
 *
 * The operation. W4A16 keeps the weights of a linear layer in 4-bit integer
 * storage and the activations in 16-bit floating point (kongchang.com page,
 * section "What Exactly Is This Stack"). One decode step reads every weight
 * matrix once and multiplies it by the activation rows of all streams of the
 * batch, so extra rows add arithmetic but almost no bytes (ai.satyajit.si page,
 * section "One weight read, shared by every stream", the t_step equation and
 * the paragraph before it); with speculation each stream adds its verified
 * positions as further rows (same page, section "Speculation spends the same
 * arithmetic"). The 4-bit checkpoint is group-wise integer, one scale per group
 * of weights (same page, section "What one more stream costs on this model").
 * This library computes, for M activation rows,
 *
 *     y[m][n] = sum_k x[m][k] * q[n][k] * s[n][k / group]      (0 <= m < M, 0 <= n < N)
 *
 * with x bf16, q a signed 4-bit code in -8..7, s an fp16 scale, fp32
 * accumulation and a bf16 result rounded to nearest even.
 *
 * Packed format (the pages leave it open; this is the library's definition).
 *   Words: word j of output column n holds the codes of k = 8j..8j+7 as
 *   4-bit two's complement (q & 0xF); the code of k = 8j+i sits in nibble
 *   (i/2) + 4*(i%2), i.e. bits 4*((i/2) + 4*(i%2)) .. +3: even k in nibbles
 *   0..3, odd k in nibbles 4..7, so that nibbles v and v+4 become the two
 *   bf16 halves of one operand register. Device arrangement (what w4a16_pack
 *   writes and the kernels read): columns in blocks of 16, the last block
 *   padded with zero codes and zero scales; blocks = ceil(N/16), G = K/group,
 *   wpl = group/32.
 *   qweight : uint32 [blocks][G][64][wpl]. Tile (b, t) covers 16 columns x one
 *             group; its entry (l, w) is word t*(group/8) + (l/16)*wpl + w
 *             of column 16b + (l%16). A tile is exactly the MFMA B operands of
 *             its group for one wavefront, and a block's K range is contiguous.
 *   scales  : fp16 [blocks][G][16]; entry (b, t, c) = s[16b + c][t].
 *   x       : bf16 [M][K] row-major, contiguous.   y : bf16 [M][N] row-major.
 *
 * Ownership and threading. The caller owns every buffer. The library keeps no
 * per-call state, allocates no memory, never synchronizes, and may be called
 * from several host threads at once. GEMM calls are asynchronous on `stream`
 * (NULL = the device's default stream); the pointers must stay valid until the
 * work on `stream` completes. `y` must not overlap any input.
 *
 * Errors. Every check happens on the host before any launch; a failed call
 * launches nothing and leaves no state behind, so the next call is unaffected.
 */
#ifndef W4A16_H
#define W4A16_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

struct ihipStream_t; /* hipStream_t is `struct ihipStream_t*` */

typedef enum {
  W4A16_OK = 0,
  W4A16_ERR_INVALID_ARG = 1, /* null pointer, negative size, size mismatch, code out of -8..7 */
  W4A16_ERR_UNSUPPORTED = 2, /* shape outside the supported set (see w4a16_gemm) */
  W4A16_ERR_MISALIGNED = 3,  /* a device pointer is not 16-byte aligned */
  W4A16_ERR_LAUNCH = 4,      /* the HIP runtime refused the kernel launch */
  W4A16_ERR_TOO_LARGE = 5    /* needs more scratch than w4a16_gemm_noalloc's static array */
} w4a16_status;

/* Kernel paths; W4A16_PATH_AUTO lets the M-dispatch heuristic choose. */
typedef enum {
  W4A16_PATH_AUTO = 0,
  W4A16_PATH_SKINNY = 1, /* workgroups of 16-64 rows x 32-80 columns over all of K, waves split K */
  W4A16_PATH_LARGE = 2   /* workgroups of 32-128 rows x 256 columns over all of K, LDS-staged
                            activation tiles, waves split N */
} w4a16_path;

/* Bytes of the packed weights, ceil(N/16)*16*K/2, and of the packed scales,
 * ceil(N/16)*16*(K/group)*2. The pages fix no format; these sizes are the
 * library's own: N is padded up to whole 16-column blocks (the width of one
 * MFMA tile), so for N % 16 != 0 they exceed the unpadded N*K/2 and
 * N*(K/group)*2, and every buffer handed to a GEMM call must hold the padded
 * size. Return 0 for negative sizes, K not a multiple of 32, or a group that is
 * not a multiple of 32 or does not divide K. */
size_t w4a16_qweight_bytes(int N, int K);
size_t w4a16_scales_bytes(int N, int K, int group);

/*
 * Host-side packing into the packed format above (the library's own format:
 * the pages name 4-bit weights with group-wise scales, kongchang.com page,
 * section "What Exactly Is This Stack", but no layout). Pure and
 * deterministic; no device involvement.
 *   q          : host int8 [N][K], each code in -8..7 (read only)
 *   scales_in  : host fp16 bit patterns [N][K/group], row n = output column n
 *   qweight_out: host, w4a16_qweight_bytes(N, K) bytes, device arrangement above
 *   scales_out : host, w4a16_scales_bytes(N, K, group) bytes, device arrangement above
 * Requires N >= 0, K >= 0, group > 0, group % 32 == 0, K % group == 0.
 * Returns W4A16_OK, or W4A16_ERR_INVALID_ARG (nothing written) for a null
 * pointer with a non-empty shape, a bad shape, or any code outside -8..7.
 * Scale values are copied bit for bit; they are not inspected.
 */
int w4a16_pack(const int8_t* q, const uint16_t* scales_in, uint32_t* qweight_out,
               uint16_t* scales_out, int N, int K, int group);

/*
 * y = x . dequant(qweight, scales) on the GPU, overwriting y (no bias, no beta):
 * the W4A16 product of kongchang.com, section "What Exactly Is This Stack"
 * (4-bit weights, 16-bit activations), with the weights read once and shared
 * by all M rows (ai.satyajit.si, section "One weight read, shared by every
 * stream"). Needs no workspace: every kernel behind it reduces within a
 * workgroup, so calls on different streams may overlap.
 *   x       : device bf16 [M][K]
 *   qweight, scales : device copies of what w4a16_pack wrote for (N, K, group)
 *   y       : device bf16 [M][N]
 * All four pointers must be 16-byte aligned device addresses of the current
 * device. Supported shapes: M >= 0, N >= 1, K >= 1, group in {32, 64, 128, 256},
 * K % group == 0; N needs no rounding (ragged column tiles are masked).
 * Above 1,048,560 rows (65,535 row tiles of 16) only the tile engine runs,
 * which needs group 32, 64 or 128 and packed weights below 4 GB; other shapes
 * of that many rows return W4A16_ERR_UNSUPPORTED before any launch.
 * M == 0 returns W4A16_OK and launches nothing.
 * Returns W4A16_OK, W4A16_ERR_INVALID_ARG, W4A16_ERR_UNSUPPORTED,
 * W4A16_ERR_MISALIGNED or W4A16_ERR_LAUNCH.
 */
int w4a16_gemm(const void* x, const void* qweight, const void* scales, void* y, int M, int N,
               int K, int group, struct ihipStream_t* stream);

/* As w4a16_gemm, with the kernel path forced (W4A16_PATH_*; the M-dispatch
 * choice is the library's own, the pages give none); every path gives a result
 * within the same tolerance of the exact product. W4A16_PATH_LARGE runs the
 * plain kernel where the tile engine cannot (group 256, packed weights of 4 GB
 * or more), and W4A16_PATH_SKINNY the tile engine above 1,048,560 rows. */
int w4a16_gemm_ex(const void* x, const void* qweight, const void* scales, void* y, int M,
                  int N, int K, int group, int path, struct ihipStream_t* stream);

/*
 * Workspace of the streaming entry points below (the library's own; the pages
 * describe the product, not its scheduling), for M activation rows and
 * `total_columns` output columns (the sum of N over the problems of a call):
 * for M <= 16, per-block counters, one swap slot per output value and fp32
 * partial sums per workgroup; for M > 16, per-tile counters and partial sums.
 * For 52,224 columns (one layer's four projections): 0.6 MB at M = 1, 10 MB
 * at M = 16, 21 to 84 MB for M > 16. Device memory owned by the caller,
 * 256-byte aligned, zero-filled once before its first use; every call leaves
 * every byte of it at zero again (counters, slots and partial sums), so one
 * workspace serves any sequence of calls of any kind (any M, any problems,
 * planned or not) without clearing, as long as it is large enough for each.
 * One workspace must not serve two calls that can run at the same time.
 * Returns 0 for M < 0 or total_columns < 0.
 */
size_t w4a16_workspace_bytes(int M, long long total_columns);

/*
 * As w4a16_gemm (same operation, same citations), using a workspace (see
 * w4a16_workspace_bytes(M, N)). For
 * M <= 16 this runs the streaming kernel: a persistent grid whose waves split
 * the packed weights into equal contiguous runs, combining the column blocks
 * cut between waves through the workspace. For larger M (group 32, 64 or
 * 128) a persistent grid of MFMA workgroups splits the (tile, k-tile) work
 * evenly, combining the tiles cut between workgroups through the workspace.
 * Both sum parts in a fixed order, so results are deterministic. Group 256 at
 * M > 16 runs the kernels of w4a16_gemm and does not use the workspace; so
 * does any problem above 16 rows for which the library's time models put
 * w4a16_gemm's kernels ahead of the stream-K schedule (most shapes below a
 * few hundred rows; the exceptions are few, deep 256-column tiles), and the
 * result is then that of w4a16_gemm, bit for bit.
 * Extra errors: W4A16_ERR_INVALID_ARG for a null or too small workspace
 * (checked only when a streaming kernel runs), W4A16_ERR_MISALIGNED for a
 * workspace that is not 256-byte aligned.
 */
int w4a16_gemm_ws(const void* x, const void* qweight, const void* scales, void* y, int M, int N,
                  int K, int group, void* workspace, size_t workspace_bytes,
                  struct ihipStream_t* stream);

/*
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. The same
 * GEMM and kernels as w4a16_gemm_ws, with the library's own static device
 * array of W4A16_NOALLOC_SCRATCH_BYTES (96 MiB; each GPU the library runs on
 * holds one until the process ends) in place of the caller's workspace. It
 * allocates nothing and frees nothing. Arguments, validation and results as
 * for w4a16_gemm; a shape whose workspace w4a16_workspace_bytes(M, N) exceeds
 * the array returns W4A16_ERR_TOO_LARGE before anything runs (for example
 * M <= 16 with N above about 1.4 million columns). The first call on a device
 * clears the array once, with one fill kernel on `stream`; every call leaves
 * its counters and slots at zero for the next. All calls on one GPU share
 * that GPU's array: calls that can overlap on one GPU (different streams or
 * host threads without ordering between them) race and give wrong results,
 * so the caller orders them.
 */
#define W4A16_NOALLOC_SCRATCH_BYTES ((size_t)96 << 20)
int w4a16_gemm_noalloc(const void* x, const void* qweight, const void* scales, void* y, int M,
                       int N, int K, int group, struct ihipStream_t* stream);

/* One GEMM of a grouped call: y[M][N] = x[M][K] . dequant(qweight, scales). */
typedef struct w4a16_problem {
  const void* x;
  const void* qweight;
  const void* scales;
  void* y;
  int N;
  int K;
} w4a16_problem;

/*
 * Several GEMMs that share M and the group size, in one launch (for example
 * the four projections of one layer: one weight stream and one launch instead
 * of four; the step time of ai.satyajit.si, section "One weight read, shared
 * by every stream", is per step, not per matrix). `problems` is host memory read during the call; count is
 * 1..W4A16_MAX_PROBLEMS. The workspace is sized by
 * w4a16_workspace_bytes(M, sum of N). Each problem is validated as in
 * w4a16_gemm; with group 256 at M > 16 the problems run one after another on
 * `stream` without the workspace. A call of one problem runs as w4a16_gemm_ws
 * (which may take w4a16_gemm's kernels above 16 rows).
 */
#define W4A16_MAX_PROBLEMS 8
int w4a16_gemm_grouped(const w4a16_problem* problems, int count, int M, int group,
                       void* workspace, size_t workspace_bytes, struct ihipStream_t* stream);

/*
 * Planned calls: many GEMMs sharing M and the group size in ONE launch, with
 * their descriptors in device memory, so that a whole step (for example the
 * four projections of every layer of a stack: 256 GEMMs) pays one launch ramp
 * and one tail instead of one per layer; the step time of ai.satyajit.si,
 * section "One weight read, shared by every stream", is per step. The GEMMs of
 * one plan are independent of each other (no output feeds an input). The
 * planning is the library's own; the pages give none.
 *
 * w4a16_plan_bytes: bytes of the plan of `count` problems (1..4096), or 0.
 *
 * w4a16_plan_build: writes the plan of `count` problems (host memory,
 *   read during the call; each validated as in w4a16_gemm) at M >= 1 rows and
 *   `group` into `plan` (host memory, plan_bytes >= w4a16_plan_bytes(count)):
 *   each problem's descriptor and place in one persistent stream-K launch,
 *   sized for the current device's compute units, with a checksum. Pure host
 *   code. M <= 16 takes the streaming kernel (any supported group); M > 16 the
 *   MFMA tile engine, which needs group 32, 64 or 128 and packed weights and
 *   activations of each problem below 4 GB (else W4A16_ERR_UNSUPPORTED).
 *   Returns W4A16_OK, W4A16_ERR_INVALID_ARG, W4A16_ERR_UNSUPPORTED or
 *   W4A16_ERR_MISALIGNED; on an error the plan holds nothing usable.
 *
 * w4a16_plan_workspace_bytes: workspace bytes of a built plan (0 if `plan` is
 *   not one). The workspace follows the rules of w4a16_workspace_bytes:
 *   caller-owned device memory, 256-byte aligned, zero-filled once before its
 *   first use, left with zero counters by every call, one call at a time.
 *
 * w4a16_gemm_planned: runs every GEMM of the plan in one launch on `stream`.
 *   `plan` is the host plan, `plan_dev` a byte copy of it in device memory
 *   (16-byte aligned) that the caller made (for example once, when the
 *   buffers of the plan are allocated); the kernels read the descriptors from
 *   plan_dev. A device copy whose checksum differs from the host plan's makes
 *   the launch do nothing. The buffers the plan names must stay valid while
 *   calls run. Asynchronous; allocates nothing. Returns W4A16_OK,
 *   W4A16_ERR_INVALID_ARG (not a plan, null or too small workspace),
 *   W4A16_ERR_MISALIGNED or W4A16_ERR_LAUNCH.
 */
#define W4A16_PLAN_MAX_PROBLEMS 4096
size_t w4a16_plan_bytes(int count);
int w4a16_plan_build(const w4a16_problem* problems, int count, int M, int group, void* plan,
                     size_t plan_bytes);
size_t w4a16_plan_workspace_bytes(const void* plan);
int w4a16_gemm_planned(const void* plan, const void* plan_dev, void* workspace,
                       size_t workspace_bytes, struct ihipStream_t* stream);

/*
 * W4A8: the activations quantized to int8 with one scale per row, times the
 * same packed 4-bit weights, on the int8 MFMA. Once the rows' arithmetic
 * rather than the weight stream bounds a step, cheaper arithmetic is what
 * raises the rate (ai.satyajit.si page, section "What one more stream costs
 * on this model"); the int8 product does twice the multiply-adds per cycle
 * of the bf16 one. Intended for large M (hundreds of rows and more); any
 * M >= 1 is computed correctly.
 *
 * w4a8_quantize: x (device bf16 [M][K]) -> xq (device int8 [M][K]) and sx
 * (device fp32 [M]). For row m, in fp32 with round to nearest even:
 *   a = max_k |x[m][k]|,  sx[m] = a / 127,
 *   xq[m][k] = x[m][k] * (127 / a) rounded to the nearest integer (ties to
 *              even) and clamped to [-127, 127];  a row of zeros gives codes 0
 *              and sx[m] = 0. Inputs must be finite.
 * Arrangement of xq: row-major, each aligned block of 16 k stored in the
 * order in which the MFMA consumes two packed weight words: byte j of block
 * b holds the code of k = 16b + o[j], o = 0,4,1,5,2,6,3,7,8,12,9,13,10,14,11,15.
 * Requires M >= 0, K >= 16, K % 16 == 0; every pointer a 16-byte aligned
 * device address. M == 0 returns W4A16_OK and launches nothing.
 */
int w4a8_quantize(const void* x, void* xq, void* sx, int M, int K, struct ihipStream_t* stream);

/*
 * w4a8_gemm: y[m][n] = sx[m] * sum_t s[n][t] * sum_{k in group t} xq[m][k] * q[n][k],
 * with xq and sx as w4a8_quantize writes them, qweight and scales as
 * w4a16_pack writes them, the integer sums exact (int32), the scaling in fp32
 * and y (device bf16 [M][N]) rounded to nearest even. group 64 or 128,
 * K % group == 0, N >= 1; other shapes return W4A16_ERR_UNSUPPORTED. Every
 * pointer a 16-byte aligned device address; y overlaps no input. Errors and
 * asynchrony as for w4a16_gemm; no workspace.
 */
int w4a8_gemm(const void* xq, const void* sx, const void* qweight, const void* scales, void* y,
              int M, int N, int K, int group, struct ihipStream_t* stream);

/* One quantization of a grouped call: x (bf16 [M][K]) -> xq, sx, as w4a8_quantize. */
typedef struct w4a8_quantize_problem {
  const void* x;
  void* xq;
  void* sx;
  int K;
} w4a8_quantize_problem;

/*
 * Several quantizations sharing M in one launch (for example the inputs of a
 * layer's projections). `problems` is host memory read during the call;
 * count is 1..W4A16_MAX_PROBLEMS; each problem is validated as in
 * w4a8_quantize, and every result equals that of w4a8_quantize.
 */
int w4a8_quantize_grouped(const w4a8_quantize_problem* problems, int count, int M,
                          struct ihipStream_t* stream);

/* One GEMM of a grouped W4A8 call: y[M][N] from xq, sx ([M][K], [M]) and the
 * packed weights, as w4a8_gemm. */
typedef struct w4a8_problem {
  const void* xq;
  const void* sx;
  const void* qweight;
  const void* scales;
  void* y;
  int N;
  int K;
} w4a8_problem;

/*
 * Several W4A8 GEMMs sharing M and the group size in one launch, so that the
 * small projections of a layer do not leave compute units idle and the
 * deepest-K problems start first. `problems` is host memory read during the
 * call; count is 1..W4A16_MAX_PROBLEMS; each problem is validated as in
 * w4a8_gemm, and every result equals that of w4a8_gemm. No workspace.
 */
int w4a8_gemm_grouped(const w4a8_problem* problems, int count, int M, int group,
                      struct ihipStream_t* stream);

/* The path W4A16_PATH_AUTO picks for this shape (an M-dispatch heuristic on
 * host integers), or -1 for a shape w4a16_gemm does not take. */
int w4a16_select_path(int M, int N, int K, int group);

/* The kernel form w4a16_gemm_ex runs for this shape on `path` (the library's
 * own choice, from time models of its kernels; the pages give none): writes the
 * workgroup's output tile (*rows x *cols) and its waves, and returns the path
 * that runs (W4A16_PATH_AUTO resolved), or -1 (nothing written) for an
 * unsupported shape, a bad path or a null output pointer. Host arithmetic only,
 * for tests and profiles. */
int w4a16_select_form(int M, int N, int K, int group, int path, int* rows, int* cols, int* waves);

/* Static text for a status code; never NULL. */
const char* w4a16_status_string(int status);

/*
 * Measurement aid, not part of the GEMM: reads `bytes` of device memory at
 * `buf` once, in the access pattern of the small-M weight stream (a persistent
 * grid of two 8-wave workgroups per compute unit, each wave one contiguous run
 * of non-temporal 16-byte loads), and nothing else. Its rate over the packed
 * weights of a step is the practical ceiling of the bandwidth-ceiling equation
 * (ai.satyajit.si page, section "One weight read, shared by every stream") on
 * this chip, against which the streaming kernels are judged.
 *   buf  : device, 16-byte aligned, bytes % 16 == 0 (bytes == 0: no launch)
 *   sink : device, 4-byte aligned, at least 8,192 bytes (2,048 uint32); the
 *          probe writes one 32-bit wrapping sum per workgroup into its first
 *          words, so over a zero-filled sink the wrapping sum of all sink words
 *          equals that of every 32-bit word of the buffer.
 * Asynchronous on `stream`; allocates nothing. Returns W4A16_OK,
 * W4A16_ERR_INVALID_ARG, W4A16_ERR_MISALIGNED or W4A16_ERR_LAUNCH.
 */
int w4a16_read_probe(const void* buf, size_t bytes, void* sink, size_t sink_bytes,
                     struct ihipStream_t* stream);

/* Library version: major * 10000 + minor * 100 + patch. */
int w4a16_version(void);

#ifdef __cplusplus
}
#endif

#endif /* W4A16_H */
