/*
 * qint4.h -- C ABI of libqint4.so: group-affine 4-bit weight dequantisation
 * fused into matrix-vector and small-M matrix products, for AMD MI355X
 * (gfx950, CDNA4).
 *
 * Sources, cited by page title and passage:
 *   [FFAI #14] thewafflehaus/FFAI pull 14, "feat(everything-bagel): clean
 *              migration of PR #9 + #10 onto updated dev".
 *   [FFAI #9]  thewafflehaus/FFAI pull 9, "Everything Bagel".
 *   [ds4 #844] antirez/ds4 pull 844, "Ornith 1.5 + Qwen 3.8 27B hybrid runtime
 *              + DFlash speculative decoding on Metal".
 *
 * ---------------------------------------------------------------------------
 * Weight format (shared by every entry point)
 * ---------------------------------------------------------------------------
 * A matrix W has n_out rows and k_in input columns.  Each weight is a 4-bit
 * code q in 0..15 with an affine map per group of `group_size` consecutive
 * input columns of a row:
 *
 *     w[o][k] = scale[o][k / group_size] * q[o][k] + bias[o][k / group_size]
 *
 * ([FFAI #14], commit "dequantGemvInt4Two/Three/Four": the int4 GEMV takes
 * a packed weight with its scales and biases, in_dim and group_size.)
 *
 *   codes   uint32 [n_experts][n_out][k_in/8], row-major, eight codes per
 *           word along k_in ([FFAI #14], commit adding the packed-width
 *           precondition: in_dim = packed width * 8).  Code k of a row is
 *           (codes[k/8] >> (4*(k%8))) & 15, least significant nibble first.
 *   scales  [n_experts][n_out][k_in/group_size], float32 or bfloat16
 *   biases  same shape and dtype as scales
 *
 * A stack of experts ([FFAI #14], expert-indexed GEMV commit: a stacked
 * [nExperts, outDim, inDim/8] u32 tensor) is the same layout with
 * n_experts > 1; expert e starts at codes + e*n_out*k_in/8 and
 * scales/biases + e*n_out*(k_in/group_size).
 *
 * ---------------------------------------------------------------------------
 * Conventions
 * ---------------------------------------------------------------------------
 * - Every data pointer is DEVICE memory of the current HIP device, owned by
 *   the caller.  The library never allocates, frees or keeps a pointer.
 * - `stream` is a hipStream_t (NULL = the null stream).  Every call only
 *   enqueues work on it and returns; there is no host synchronisation.
 * - Arguments are validated before anything is enqueued.  On failure the
 *   call returns a non-zero qint4_status, writes nothing to device memory,
 *   and qint4_last_error() names the offending values.  No call aborts.
 * - Faults inside a kernel surface at the caller's next synchronisation.
 * - Requirements common to all entry points:
 *     group_size in {32, 64, 128};  k_in % group_size == 0;
 *     n_out >= 1;  k_in >= group_size;
 *     codes 16-byte aligned; activations 16-byte aligned;
 *     scales/biases aligned to their element size;
 *     the current device is a gfx950 GPU.
 * - Outputs must not overlap any input (checked on the address ranges).
 * - Calls are reentrant; concurrent calls on different streams need
 *   separate outputs and workspaces.
 */
#ifndef QINT4_H
#define QINT4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QINT4_ABI_VERSION 1
#define QINT4_MULTI_MAX 8   /* most projections one qgemv_int4_multi call takes */
#define QINT4_TOPK_MAX 8    /* most experts one moe_gather_qgemv_int4 call combines */

/* Element types (passed as int32_t). */
enum { QINT4_F32 = 0, QINT4_BF16 = 1 };

/* Epilogues of qgemv_int4_multi (passed as int32_t). */
enum {
  QINT4_EPI_NONE = 0,        /* ys[i] = W_i x                                  */
  QINT4_EPI_SWIGLU_PAIR = 1  /* n == 2: ys[0] = silu(W_0 x) * (W_1 x)          */
};

/* Status codes. */
typedef enum qint4_status {
  QINT4_OK = 0,
  QINT4_ERR_NULL = 1,       /* a required pointer is NULL                      */
  QINT4_ERR_SHAPE = 2,      /* sizes inconsistent or outside the supported set */
  QINT4_ERR_DTYPE = 3,      /* unsupported element-type combination            */
  QINT4_ERR_ALIGN = 4,      /* a pointer or leading dimension is misaligned    */
  QINT4_ERR_ALIAS = 5,      /* an output overlaps an input                     */
  QINT4_ERR_WORKSPACE = 6,  /* workspace NULL or smaller than required         */
  QINT4_ERR_DEVICE = 7,     /* no current gfx950 device                        */
  QINT4_ERR_LAUNCH = 8,     /* the HIP runtime rejected a kernel launch        */
  QINT4_ERR_VALUE = 9       /* a scalar argument is outside its valid range    */
} qint4_status;

/* One packed matrix, or a stack of n_experts matrices of the same shape. */
typedef struct qint4_matrix {
  const uint32_t *codes;    /* device, [n_experts][n_out][k_in/8]                */
  const void *scales;       /* device, [n_experts][n_out][k_in/group_size]       */
  const void *biases;       /* device, same shape/dtype as scales                */
  int64_t n_out;            /* rows (outputs)                                    */
  int64_t k_in;             /* input columns                                     */
  int32_t group_size;       /* 32, 64 or 128                                     */
  int32_t n_experts;        /* 1 for a plain matrix                              */
  int32_t sb_dtype;         /* QINT4_F32 or QINT4_BF16                           */
  int32_t reserved;         /* must be 0                                         */
} qint4_matrix;

/*
 * qgemv_int4 -- y = W x, one decode token (T = 1).
 *
 * [FFAI #14], commits on the dequant_gemv_int4 family: one output per row of
 * the packed matrix, the input vector shared by all rows.
 *
 *   w       matrix (n_experts must be 1)
 *   x       device [k_in], dtype x_dtype (QINT4_F32 or QINT4_BF16)
 *   y       device [n_out], dtype y_dtype (QINT4_F32 or QINT4_BF16);
 *           every element is overwritten (bf16: round to nearest even from
 *           the float32 accumulator)
 * Accumulation is float32.  Float32 activations enter the products scaled by
 * up to 2^24 (exactly, by powers of two), so activations of magnitude 2^104
 * or more overflow to inf; as do scales of that size in the prefill GEMMs'
 * dequantisation.  Returns QINT4_OK or an error status.
 */
qint4_status qgemv_int4(const qint4_matrix *w, const void *x, int32_t x_dtype,
                        void *y, int32_t y_dtype, void *stream);

/*
 * qgemv_int4_multi -- n projections of ONE shared input in ONE launch.
 *
 * [FFAI #14], batched QKV / batched-4 qgemv commits: the q, k, v (or four
 * GDN input) projections share one input and run as one kernel launch that
 * reads the input once; all packed widths must match the leading matrix
 * (the precondition added in the packed-width commit, whose error names the
 * mismatched widths).  SwiGLU pairing: [FFAI #9], commit fusing silu(gate) *
 * up into one swiglu step.
 *
 *   n        1..QINT4_MULTI_MAX matrices; all share k_in, group_size and
 *            sb_dtype; each has n_experts == 1
 *   ws       host array [n] of matrix descriptors
 *   x        device [k_in], dtype x_dtype
 *   ys       host array of device output pointers:
 *              QINT4_EPI_NONE:        [n], ys[i] is [ws[i].n_out]
 *              QINT4_EPI_SWIGLU_PAIR: n == 2, ws[0] (gate) and ws[1] (up)
 *                                     have equal n_out, ys[0] is
 *                                     h = silu(gate x) * (up x), [n_out],
 *                                     computed in float32
 *   y_dtype  element type of every output
 *   epilogue QINT4_EPI_NONE or QINT4_EPI_SWIGLU_PAIR
 */
qint4_status qgemv_int4_multi(int32_t n, const qint4_matrix *ws, const void *x,
                              int32_t x_dtype, void *const *ys, int32_t y_dtype,
                              int32_t epilogue, void *stream);

/*
 * qgemv_int4_smallm -- qgemv_int4_multi for T = 1..QINT4_SMALLM_MAX activation
 * rows at once (small-M products: a few decode tokens, or the tokens of a
 * speculative-verify round, against the same weights).
 *
 * [ds4 #844], PR body and the commit on small speculative-verify rounds: a
 * fused gate/up SwiGLU for 1..8 rows, and 2..9-token verify rounds that
 * cannot fill a 32-row matrix-multiply tile; and its batched-vs-sequential
 * contract: row t of a T-row call equals a T = 1 call of this function on
 * row t, bit for bit.  Every code load and its nibble decode is shared by the
 * T rows.  The per-group form is that of qgemv_int4_multi,
 *   s * (sum (128 + q) x - 128 sum x) + b sum x,
 * but with bf16 activations, group_size 32, 64 or 128 and k_in a multiple of
 * 512 up to 8192 (stored outputs or the gate/up pair), the inner sums come
 * from MFMA for every T: those results agree with qgemv_int4_multi's to the
 * rounding of float32 sums, not bit for bit.  Other calls run the
 * qgemv_int4_multi arithmetic per row.
 *
 *   T        1..QINT4_SMALLM_MAX (16); T > 1 needs x_dtype QINT4_BF16.  Up
 *            to 16 rows share one weight stream on the MFMA form (8 where the
 *            16 staged rows would not fit in LDS: k_in above 4096 or so, two
 *            launches), 8 per launch on the other form
 *   x        device [T][ldx], row t at x + t * ldx elements, 16-byte aligned;
 *            ldx >= k_in, ldx % 8 == 0 when T > 1
 *   ys       as in qgemv_int4_multi, each output [T][n_out] (row-major)
 *   other arguments as in qgemv_int4_multi
 */
#define QINT4_SMALLM_MAX 16
qint4_status qgemv_int4_smallm(int32_t n, const qint4_matrix *ws, const void *x,
                               int32_t x_dtype, int64_t T, int64_t ldx, void *const *ys,
                               int32_t y_dtype, int32_t epilogue, void *stream);

/*
 * rms_norm_qgemv_int4 -- qgemv_int4_multi of the RMS-normalised input, in
 * the same single launch:
 *
 *   ys[i] = W_i xn,   xn[k] = x[k] * gamma[k] / sqrt(mean_k(x[k]^2) + eps)
 *
 * (SWIGLU_PAIR: ys[0] = silu(W_0 xn) * (W_1 xn)).
 *
 * [FFAI #14], commit wrapping the RMSNorm-fused qgemv: the normalised
 * activation is fed straight into the int4 dequant GEMV instead of a norm
 * launch followed by a GEMV launch, saving the round trip of the normalised
 * vector through memory (used for the final norm + LM head, and for any
 * pre-norm -> int4 projection).  [ds4 #844], commit unifying the norm
 * kernels: the normaliser is 1 / sqrt(mean + eps).
 *
 * The normalised vector is never rounded: the kernel stages x * gamma in
 * float32 (exact for bf16 inputs), reduces sum(x^2) in float32, and scales
 * the float32 row sums by 1 / sqrt(sum / k_in + eps) -- the same value, since
 * the norm is one scalar per input row.
 *
 *   gamma   device [k_in], dtype x_dtype, 16-byte aligned (the norm weight)
 *   eps     finite, > 0 (QINT4_ERR_VALUE otherwise)
 *   other arguments as in qgemv_int4_multi (one activation row)
 */
qint4_status rms_norm_qgemv_int4(int32_t n, const qint4_matrix *ws, const void *x,
                                 int32_t x_dtype, const void *gamma, float eps,
                                 void *const *ys, int32_t y_dtype, int32_t epilogue,
                                 void *stream);

/*
 * Bytes of device workspace one moe_gather_qgemv_int4 call needs with the
 * down-projection stack `down` (host descriptor; only its k_in, the expert
 * intermediate width inter, is read) and `top_k` kept experts: the float32
 * SwiGLU intermediates, one row of inter per kept expert.  0 when down is NULL
 * or its k_in or top_k is outside the range the call accepts.
 */
size_t moe_gather_qgemv_int4_workspace_bytes(const qint4_matrix *down, int32_t top_k);

/*
 * moe_gather_qgemv_int4 -- one token through a top-K mixture of experts.
 *
 *   out = residual + sum_{k < top_k} wts[k] * W_down[ids[k]] h_k,
 *   h_k = silu(W_gate[ids[k]] x) * (W_up[ids[k]] x)
 *
 * [FFAI #14]: the expert-indexed GEMV reads the expert id on the device and
 * selects that slab of the stacked tensor (no host readback); the router
 * writes [k] u32 ids and [k] weights; the chain8 commit fuses SwiGLU, the
 * expert-indexed down GEMV and the weighted accumulate
 * acc[i] = sum_k w_k out_k[i]; the scalar-FMA commit defines the 8-way
 * scalar FMA chain out[i] = base[i] + sum_k scalar_k value_k[i].
 *
 *   gate, up  stacks [E][inter][hidden]; down stack [E][hidden][inter];
 *             all three with the same n_experts E, group_size and sb_dtype
 *   x         device [hidden], dtype act_dtype
 *   ids       device uint32 [top_k]; an id >= E contributes nothing (ids are
 *             device data and are not checked on the host)
 *   wts       device float32 [top_k]
 *   top_k     1..QINT4_TOPK_MAX
 *   residual  device [hidden], dtype act_dtype, or NULL for none
 *   out       device [hidden], dtype act_dtype; every element overwritten
 *   act_dtype QINT4_F32 or QINT4_BF16
 *   workspace device scratch of at least
 *             moe_gather_qgemv_int4_workspace_bytes(down, top_k) bytes,
 *             16-byte aligned; contents on entry are ignored, contents on
 *             return are unspecified.  One workspace per concurrent call.
 * Two kernel launches on `stream` (gate/up + SwiGLU, then down + combine).
 */
qint4_status moe_gather_qgemv_int4(const qint4_matrix *gate, const qint4_matrix *up,
                                   const qint4_matrix *down, const void *x,
                                   const uint32_t *ids, const float *wts, int32_t top_k,
                                   const void *residual, void *out, int32_t act_dtype,
                                   void *workspace, size_t workspace_bytes, void *stream);

/*
 * moe_gather_qgemv_int4_noalloc -- moe_gather_qgemv_int4 without a workspace
 * argument, for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.
 *
 * Same arguments (less the workspace), result and launches as
 * moe_gather_qgemv_int4.  The float32 SwiGLU intermediates go to a static
 * device array inside the library, QINT4_NOALLOC_SCRATCH_BYTES on each GPU it
 * runs on (held until the process ends); its address is looked up once per
 * device, on the first call there.  The call allocates nothing.
 *
 *   top_k * inter * 4 <= QINT4_NOALLOC_SCRATCH_BYTES, else QINT4_ERR_WORKSPACE
 *   (nothing is launched).
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents; a call reads only what it wrote earlier in the same call.  Calls
 * that overlap on one GPU (unordered streams) race on the array: order them,
 * or give each its own workspace through moe_gather_qgemv_int4.
 */
#define QINT4_NOALLOC_SCRATCH_BYTES (1u << 20)
qint4_status moe_gather_qgemv_int4_noalloc(const qint4_matrix *gate, const qint4_matrix *up,
                                           const qint4_matrix *down, const void *x,
                                           const uint32_t *ids, const float *wts, int32_t top_k,
                                           const void *residual, void *out, int32_t act_dtype,
                                           void *stream);

/*
 * moe_route_gather_qgemv_int4 -- moe_router_topk followed by
 * moe_gather_qgemv_int4 for one token, with the routing done inside the
 * gate/up launch: every wave of that launch ranks the token's logits itself
 * (exactly as moe_router_topk does), so the router's separate launch and its
 * dependency gap disappear.  ids and wts are written by the gate/up launch
 * and read by the down launch; on return (after the stream work) they hold
 * the same values moe_router_topk would have written, and out equals the
 * two-call result bit for bit.
 *
 * [FFAI #14], GPU MoE router commit (router output threaded straight into the
 * expert-indexed GEMV); the other passages as for moe_gather_qgemv_int4.
 *
 *   logits        device [n_experts], dtype logits_dtype (QINT4_F32 or
 *                 QINT4_BF16), element-aligned; n_experts = the stacks'
 *                 n_experts, top_k <= n_experts <= 256
 *   ids, wts      device uint32 [top_k] / float32 [top_k], OUTPUTS, written
 *   other arguments as in moe_gather_qgemv_int4
 */
qint4_status moe_route_gather_qgemv_int4(const qint4_matrix *gate, const qint4_matrix *up,
                                         const qint4_matrix *down, const void *x,
                                         const void *logits, int32_t logits_dtype, int32_t top_k,
                                         const void *residual, void *out, int32_t act_dtype,
                                         uint32_t *ids, float *wts, void *workspace,
                                         size_t workspace_bytes, void *stream);

/*
 * Bytes of device workspace one moe_prefill_qgemm_int4 call needs (0 for
 * invalid sizes: T * top_k must be in [1, 2^24], n_experts <= 4096).
 */
size_t moe_prefill_qgemm_int4_workspace_bytes(int64_t T, int32_t top_k, int32_t n_experts,
                                              int64_t hidden, int64_t inter);

/*
 * moe_prefill_qgemm_int4 -- T tokens through a top-K mixture of experts at
 * once (prefill), on bf16 matrix cores:
 *
 *   out[t] = residual[t] + sum_{k < top_k} wts[t][k] * W'_down[e] h_tk,
 *   h_tk   = silu(W'_gate[e] x[t]) * (W'_up[e] x[t]),   e = ids[t][k]
 *
 * where W' are the weights dequantised in float32 and rounded to bfloat16
 * (nearest even), as in qgemm_int4_padT; accumulation is float32 and h is
 * carried between the two products to float32 accuracy (two bf16 planes).
 *
 * [FFAI #9], batched MoE commits: the T * top_k (token, slot) rows are fanned
 * into one GEMM per gate / up / down, sorted by expert id so that a row tile
 * shares one expert's weights, with CSR expert offsets built from the sorted
 * ids, and a scatter-sum unpermutes the rows afterwards.  [FFAI #14]: the
 * chain8 weighted combine and the residual add.  Here the sort runs on the
 * device, so ids produced by moe_router_topk are used without a host read.
 *
 *   gate, up  stacks [E][inter][hidden]; down [E][hidden][inter]; shared E
 *             (<= 4096), group_size and sb_dtype
 *   x         device bf16 [T][ldx], 16-byte aligned; ldx >= hidden, ldx % 8 == 0
 *   T         tokens, 1 <= T * top_k <= 2^24
 *   ids       device uint32 [T][top_k]; an id >= E contributes nothing
 *   wts       device float32 [T][top_k]
 *   top_k     1..QINT4_TOPK_MAX
 *   residual  device [T][hidden] of out_dtype, 16-byte aligned, or NULL
 *   out       device [T][hidden], dtype out_dtype (QINT4_F32 or QINT4_BF16),
 *             16-byte aligned; fully overwritten
 *   workspace device scratch, 256-byte aligned, at least
 *             moe_prefill_qgemm_int4_workspace_bytes(T, top_k, E, hidden,
 *             inter) bytes; contents on entry ignored, on return unspecified
 * Four kernel launches on `stream` (sort, gate/up, down, combine).
 */
qint4_status moe_prefill_qgemm_int4(const qint4_matrix *gate, const qint4_matrix *up,
                                    const qint4_matrix *down, const void *x, int64_t T, int64_t ldx,
                                    const uint32_t *ids, const float *wts, int32_t top_k,
                                    const void *residual, void *out, int32_t out_dtype,
                                    void *workspace, size_t workspace_bytes, void *stream);

/*
 * qgemm_int4_padT -- prefill: Y[t][o] = sum_k bf16(w[o][k]) * X[t][k], t < T.
 *
 * [FFAI #9], dequantGemmDynamicM commit: T is padded up to a multiple of 32
 * with zero rows, the dequant GEMM runs on the padded block, and the first T
 * rows are kept.  Here the padding is virtual: rows t >= T are read as zero
 * inside the kernel and never written, so X and Y need only T rows.  The
 * weights are dequantised in float32 and rounded to bfloat16 (nearest even)
 * in LDS, then multiplied on bf16 MFMA with float32 accumulation.
 * [FFAI #14], commit adding the outDim guard: the GEMM tile needs
 * n_out % 32 == 0.
 *
 *   w     matrix (n_experts == 1), n_out % 32 == 0
 *   x     device bf16 [T][ldx], ldx >= k_in, ldx % 8 == 0
 *   T     rows of x and y, T >= 1
 *   y     device [T][ldy], dtype y_dtype (QINT4_F32 or QINT4_BF16),
 *         ldy >= n_out; rows < T fully overwritten, nothing else written
 */
qint4_status qgemm_int4_padT(const qint4_matrix *w, const void *x, int64_t T, int64_t ldx,
                             void *y, int64_t ldy, int32_t y_dtype, void *stream);

/*
 * qgemm_int4_padT_ws -- qgemm_int4_padT with a scratch workspace, the same
 * product and arguments, the same bf16 weight rounding; only the summation
 * order over k differs.
 *
 * For T <= 64 the product is a weight stream with too few 16-row tiles to
 * occupy the GPU (a 17408-row matrix has 1088); with a workspace the K range
 * is cut into slices summed by different workgroups into float32 partial
 * planes, which a second kernel adds into y.  Same citations as
 * qgemm_int4_padT (the T-padding driver; the outDim guard).
 *
 *   workspace        device scratch, 256-byte aligned, or NULL; contents on
 *                    entry ignored, on return unspecified; must not overlap
 *                    w, x or y.  Calls that share a workspace must be
 *                    ordered (one stream), as for any output buffer.
 *   workspace_bytes  its size.  The call uses at most this much and never
 *                    fails for want of space: a smaller (or NULL) workspace
 *                    means fewer slices (none: the plain kernel).
 * One or two kernel launches on `stream`.
 */
qint4_status qgemm_int4_padT_ws(const qint4_matrix *w, const void *x, int64_t T, int64_t ldx,
                                void *y, int64_t ldy, int32_t y_dtype, void *workspace,
                                size_t workspace_bytes, void *stream);

/*
 * qgemm_int4_padT_multi -- the prefill GEMM of n matrices that share one
 * activation block, in ONE launch:
 *
 *   Y_i[t][o] = sum_k bf16(w_i[o][k]) * X[t][k],   t < T,  i < n
 *
 * [FFAI #14], batched QKV and batched-4 qgemv commits: the q/k/v (or four)
 * projections of one input run as one kernel whose M > 1 path writes three
 * (four) separate outputs; [FFAI #9], dequantGemmDynamicM commit: T padded
 * to a multiple of 32 with zero rows, the first T rows kept (virtual here, as
 * in qgemm_int4_padT).  The weights are dequantised and rounded to bf16 as in
 * qgemm_int4_padT and multiplied on bf16 MFMA with float32 accumulation; each
 * output tile belongs to one matrix, and the tiles of all matrices are one
 * grid, so the launch reads X once per token tile and weight tile pair.
 *
 *   n       1..QINT4_MULTI_MAX matrices; equal k_in, group_size and sb_dtype;
 *           n_experts == 1; n_out % 32 == 0 each
 *   ws      host array [n] of matrix descriptors
 *   x       device bf16 [T][ldx], 16-byte aligned; ldx >= k_in, ldx % 8 == 0
 *   T       rows of x and of every output, T >= 1
 *   ys      host array [n] of device outputs, ys[i] is [T][ldys[i]] of y_dtype
 *           (QINT4_F32 or QINT4_BF16); rows < T fully overwritten, columns
 *           >= n_out and rows >= T never written
 *   ldys    host array [n] of row strides (>= n_out), or NULL for n_out each
 * One kernel launch on `stream`; no workspace.
 */
qint4_status qgemm_int4_padT_multi(int32_t n, const qint4_matrix *ws, const void *x, int64_t T,
                                   int64_t ldx, void *const *ys, const int64_t *ldys,
                                   int32_t y_dtype, void *stream);

/*
 * Workspace bytes with which qgemm_int4_padT_ws runs its full K split for a
 * T x n_out x k_in product on the current device; 0 when it uses none (T > 64
 * or a shape that does not split).  Depends on the current device's compute
 * unit count; 0 when no usable device is current.
 */
size_t qgemm_int4_padT_workspace_bytes(int64_t T, int64_t n_out, int64_t k_in);

/*
 * moe_router_topk -- top-K expert routing of n_tokens rows of router logits,
 * on the device, producing the ids / wts that moe_gather_qgemv_int4 reads.
 *
 * [FFAI #14], GPU MoE router commit: a row of logits [n_experts] becomes
 * [k] u32 expert indices plus [k] weights, a batched form handles one row
 * per token in one dispatch, and the index buffer is threaded straight into
 * the expert-indexed GEMV with no host readback.  [FFAI #9], top-K
 * partial-sort commit: selection order (value desc, index asc).
 *
 * Per row: p = softmax(logits); the top_k largest p are kept, equal values
 * going to the smaller expert index; ids[k] are their expert indices in that
 * order and wts[k] = p_k / (sum of the kept p), i.e. a softmax over the kept
 * logits, computed in float32.  NaN logits rank below every number; a row
 * whose kept logits are all -inf gets weights 1/top_k.
 *
 *   logits    device [n_tokens][n_experts], dtype logits_dtype (QINT4_F32 or
 *             QINT4_BF16), element-aligned
 *   n_tokens  >= 1
 *   n_experts top_k..4096
 *   top_k     1..QINT4_TOPK_MAX
 *   ids       device uint32 [n_tokens][top_k], fully overwritten
 *   wts       device float32 [n_tokens][top_k], fully overwritten
 * One kernel launch on `stream`.
 */
qint4_status moe_router_topk(const void *logits, int32_t logits_dtype, int64_t n_tokens,
                             int32_t n_experts, int32_t top_k, uint32_t *ids, float *wts,
                             void *stream);

/*
 * quantize_int4 -- the offline int4 group-affine quantiser: float weights
 * [n_rows][k_in] -> codes, scales and biases in the format above.
 *
 * [ds4 #844], PR body (verification list): the 4-bit group-64 affine type
 * derives its codes from the serialised bf16 scale/bias.  The pages give no
 * other rule; this is the plain min/max affine quantiser.  Per group:
 *
 *   s = (max w - min w) / 15,  b = min w           (float32)
 *   s', b' = the stored values (sb_dtype bf16: rounded to nearest even)
 *   q = clamp(rint((w - b') / s'), 0, 15)          (float32, ties to even;
 *                                                   q = 0 where s' == 0)
 *
 *   w         device [n_rows][k_in], dtype w_dtype (QINT4_F32 or QINT4_BF16),
 *             16-byte aligned; values must be finite and their per-group
 *             range finite in float32 (otherwise the codes are unspecified)
 *   n_rows    rows (n_experts * n_out for an expert stack; the layouts match)
 *   k_in      multiple of group_size, group_size in {32, 64, 128}
 *   codes     device uint32 [n_rows][k_in/8], 16-byte aligned, overwritten
 *   scales,   device [n_rows][k_in/group_size], dtype sb_dtype, overwritten
 *   biases
 * One kernel launch per 2 GiB of weights, on `stream`.
 */
qint4_status quantize_int4(const void *w, int32_t w_dtype, int64_t n_rows, int64_t k_in,
                           int32_t group_size, int32_t sb_dtype, uint32_t *codes, void *scales,
                           void *biases, void *stream);

/* ---------------------------------------------------------------------------
 * Launch plans (host only)
 * ---------------------------------------------------------------------------
 * qint4_plan_qgemv, qint4_plan_moe_gather -- the launches a GEMV-family call
 * with these shapes makes, planned by the same code the call runs, without
 * touching device memory or launching anything.  For tests and tuning: a
 * planner change that moves a shape to another kernel form shows here.
 *
 * The persistent GEMV kernels (QINT4_FORM_RING) deal tasks of rows_per_task
 * rows round-robin to grid * waves waves; `lanes` lanes cover one row, and a
 * step is one 16-byte code load per lane.  Each wave keeps a ring of loads in
 * flight: ring_depth 0 is the streaming ring, refilled while it is consumed;
 * 1, 2 or 4 is a ring filled once, taken when no wave has more steps than
 * that.  The small-M MFMA kernels (QINT4_FORM_MFMA) run one 16-row tile per
 * workgroup, its K range split over `waves` waves.  The activation-stationary
 * kernel (QINT4_FORM_XS: qgemv_int4 / qgemv_int4_multi at T = 1 on one to
 * eight matrices with stored outputs, k_in from 2048 to 32768 and at least
 * 5120 * 5120 codes in all, or on the gate/up pair with at least 2^25 codes;
 * rms_norm_qgemv_int4 alike) gives
 * lane j of a row group of wave w the 32-code chunk lanes * w + j of its
 * rows, whose activations it holds in registers; a workgroup's `waves` waves
 * cover k_in.  Each matrix owns a range of the `grid` workgroups, and its
 * workgroup b of G takes rows b, b + G, ... (the pair: a contiguous block
 * of rows per workgroup) (tasks: rows of all matrices;
 * rows_per_task: rows per wave step; busiest_wave_steps: rows of the busiest
 * workgroup; ring_depth: rows in flight per wave).  ([FFAI #9], the note on
 * T=1 decode negative results, structural conclusion: decode is bound by the
 * bandwidth of the expert weight gather; the plan keeps enough loads in
 * flight on every CU.)
 *
 *   call       QINT4_CALL_QGEMV (qgemv_int4, qgemv_int4_multi),
 *              QINT4_CALL_RMS_NORM (rms_norm_qgemv_int4) or
 *              QINT4_CALL_SMALLM (qgemv_int4_smallm)
 *   n, n_outs  the call's matrix count and the n_out of each (host array)
 *   k_in, group_size, x_dtype, T, epilogue   as the call takes them
 *              (T = 1 except for QINT4_CALL_SMALLM)
 *   hidden, inter, top_k, group_size, act_dtype   as moe_gather_qgemv_int4
 *              takes them; routed != 0: moe_route_gather_qgemv_int4 (the
 *              gate/up launch ranks the logits); residual != 0: a residual row
 *   n_cu       compute units to plan for; 0 = the current device's (which must
 *              then be a gfx950 GPU)
 *   form       host: the one form every launch of the call takes
 *   forms      host [2]: the gate/up launch, then the down launch
 * Returns QINT4_ERR_SHAPE / _DTYPE / _VALUE / _NULL for arguments the call
 * itself would reject on these grounds.
 */
enum { QINT4_FORM_RING = 0, QINT4_FORM_MFMA = 1, QINT4_FORM_XS = 2 };
enum { QINT4_CALL_QGEMV = 0, QINT4_CALL_RMS_NORM = 1, QINT4_CALL_SMALLM = 2 };

typedef struct qint4_gemv_form {
  int32_t kernel;              /* QINT4_FORM_RING, QINT4_FORM_MFMA or QINT4_FORM_XS  */
  int32_t tokens;              /* token template: most activation rows per launch    */
  int64_t launches;            /* launches the call makes                            */
  int64_t grid;                /* workgroups per launch                              */
  int64_t tasks;               /* ring: tasks; MFMA: 16-row tiles; XS: rows          */
  int32_t waves;               /* waves per workgroup                                */
  int32_t lanes;               /* ring, XS: lanes per row (XS: per wave slice)       */
  int32_t rows_per_task;       /* ring                                               */
  int32_t steps_per_task;      /* ring                                               */
  int64_t busiest_wave_steps;  /* ring: steps of the busiest wave; XS: its rows      */
  int32_t ring_depth;          /* ring: 0 streaming; 1, 2 or 4 one pass; XS: rows in */
                               /* flight per wave                                    */
  int32_t reserved;
} qint4_gemv_form;

qint4_status qint4_plan_qgemv(int32_t call, int32_t n, const int64_t *n_outs, int64_t k_in,
                              int32_t group_size, int32_t x_dtype, int64_t T, int32_t epilogue,
                              int32_t n_cu, qint4_gemv_form *form);

qint4_status qint4_plan_moe_gather(int64_t hidden, int64_t inter, int32_t top_k,
                                   int32_t group_size, int32_t act_dtype, int32_t routed,
                                   int32_t residual, int32_t n_cu, qint4_gemv_form *forms);

/* Static description of a status code. */
const char *qint4_status_string(int32_t status);

/* Detail of the calling thread's last failed call ("" if none). */
const char *qint4_last_error(void);

/* QINT4_ABI_VERSION of the loaded library. */
int32_t qint4_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QINT4_H */
