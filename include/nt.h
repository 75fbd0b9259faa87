/*
 * nt.h - C ABI of the fused row-reduction library for AMD MI355X (gfx950).
 *
 * Three memory-bound row operations over a dense row-major [M, N] matrix,
 * each one HIP launch sequence on the caller's stream:
 *
 *   nt_softmax_rows    y = exp(x - max(x)) / sum(exp(x - max(x)))  per row
 *   nt_layernorm_rows  y = (x - mean) * rstd * gamma + beta, plus mean, rstd
 *   nt_rmsnorm_rows    y = x / sqrt(mean(x^2) + eps) * weight
 *
 * Definitions follow the public pages this library implements:
 *  - softmax: "Portable Triton Kernels" (Hugging Face kernel-builder
 *    triton-kernels skill), "Safe Softmax Pattern" and "Reference Kernel:
 *    Softmax"; stanleyjacob.dev Triton guide, Part II "Worked example: fused
 *    softmax" (load the row once, shift by its max, exp, sum, divide, store
 *    once).  Rows too wide to hold on chip use the online max/denominator
 *    rescaling of "Triton: Block-Level GPU Programming Without CUDA", section
 *    "How Flash Attention Uses Triton".
 *  - RMSNorm: "Portable Triton Kernels", "Reference Kernel: RMSNorm".
 *  - LayerNorm: named in "Rebuilding Triton and Helion from Scratch in 4,000
 *    Lines of Python" ("Memory-bound kernels", "deuteron") without a formula;
 *    this library uses the biased variance sum((x-mean)^2)/N with eps added
 *    inside the square root.
 *
 * Conventions common to every entry point
 * ---------------------------------------
 *  Layout     x and y are dense row-major [M, N] arrays of element type `dt`
 *             with row stride N (contiguous rows).  y has the same type as x.
 *  Vectors    gamma, beta and weight are length-N arrays of type `dt`.  NULL
 *             means the identity (gamma = 1, beta = 0, weight = 1).
 *  Stats      mean and rstd are float arrays of length M; NULL means "do not
 *             write".
 *  Pointers   device (or device-accessible) addresses.  Each must be aligned
 *             to the element size (mean/rstd to 4 bytes, workspace to 8);
 *             16-byte alignment is NOT required (misaligned rows are handled).
 *  eps        must be finite and >= 0; it is added inside the square root.
 *  Shapes     M == 0 is a no-op returning NT_OK.  M < 0, N <= 0,
 *             N > INT32_MAX, or M*N overflowing int64 returns NT_ERR_SHAPE.
 *             Any row width is accepted: rows too wide to hold on chip take
 *             the split online path (softmax, needs a workspace) or a looped
 *             kernel that reads the row twice (LayerNorm, RMSNorm).
 *  Ownership  the caller allocates and owns every buffer, including the
 *             workspace (which need not be zeroed).  The library allocates and
 *             frees no device memory and keeps no pointer after returning.
 *  Stream     `stream` is a hipStream_t passed as void* (NULL = null stream).
 *             Work is enqueued and the call returns without synchronizing;
 *             results are valid once the stream reaches that point, and the
 *             inputs must stay alive until then.
 *  Errors     argument errors are returned synchronously, before anything is
 *             enqueued.  A failed launch returns NT_ERR_HIP: the status is
 *             the one the launch call itself returned; the library neither
 *             reads nor clears the thread's last HIP error, so an error left
 *             by an earlier, unrelated HIP call is not reported as this
 *             call's and stays for its owner to read.
 *  Aliasing   y == x (in place) is allowed.  y partly overlapping x, and a
 *             workspace overlapping x or y, return NT_ERR_ALIAS (checked from
 *             the addresses and sizes, before anything is enqueued).  Any
 *             overlap of y with the parameters or the stats is undefined.
 *  Numerics   inputs are widened to fp32 and reduced in fp32 (LayerNorm keeps
 *             its two row sums and its per-element affine step in fp64); the
 *             result is rounded to `dt` once, round-to-nearest-even.  The
 *             reduction order is fixed, so results are bitwise repeatable
 *             for a given shape, type and device.
 *  Threads    every entry point is thread-safe.  Global state: a cache of
 *             per-device properties (compute units, each kernel's occupancy;
 *             filled on first use, then read-only), an atomic call counter
 *             that tags the split path's workspace records, the tuning
 *             overrides of nt_set_override (atomics, read once from the
 *             environment at load), and the device scratch array of
 *             nt_softmax_rows_noalloc.  The per-call path reads the
 *             environment never and queries device attributes only on the
 *             first call on each device.
 */
#ifndef NT_H
#define NT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The enumerations are int-sized in C.  Compiled as C++ they get int as a
 * fixed underlying type, so that any int a caller passes (an unknown dtype
 * or op code) is a valid value of the parameter and is rejected with a
 * status, not undefined behaviour; the ABI is the same. */
#ifdef __cplusplus
#define NT_ENUM enum : int
#else
#define NT_ENUM enum
#endif

typedef NT_ENUM { NT_F32 = 0, NT_F16 = 1, NT_BF16 = 2 } nt_dtype;

typedef NT_ENUM {
    NT_OK = 0,
    NT_ERR_NULL = 1,       /* a required pointer is NULL                       */
    NT_ERR_SHAPE = 2,      /* M < 0, N <= 0, N > INT32_MAX, or M*N overflows   */
    NT_ERR_DTYPE = 3,      /* dt is not one of nt_dtype                        */
    NT_ERR_EPS = 4,        /* eps is negative, infinite or NaN                 */
    NT_ERR_ALIGN = 5,      /* a pointer is not aligned to its element size     */
    NT_ERR_WORKSPACE = 6,  /* workspace smaller than nt_softmax_workspace_bytes
                              (or nt_norm_workspace_bytes)                    */
    NT_ERR_HIP = 7,        /* the HIP runtime reported a launch error          */
    NT_ERR_ALIAS = 8,      /* an output overlaps a buffer it may not overlap   */
    NT_ERR_SCALE = 9,      /* causal softmax: scale is not finite and > 0      */
    NT_ERR_OVERRIDE = 10   /* nt_set_override: unknown name or malformed value */
} nt_status;

/*
 * Bytes of device workspace nt_softmax_rows needs for this shape: 0 when each
 * row fits on chip (single pass), else 16 bytes per (row, row chunk) for the
 * per-chunk running max and denominator of the split online path, plus 16
 * bytes for the record tag of a call captured into a graph.  Returns 0 for
 * invalid arguments.  The contents need not be initialized and are
 * overwritten; two calls in flight at once must not share a workspace, and a
 * workspace overlapping x or y is NT_ERR_ALIAS.
 */
size_t nt_softmax_workspace_bytes(int64_t M, int64_t N, nt_dtype dt);

/*
 * Row softmax.  y[r, j] = exp(x[r, j] - m_r) / sum_k exp(x[r, k] - m_r) with
 * m_r = max_k x[r, k].  -inf entries contribute exactly 0 (a row of -inf only
 * yields NaN, as the formula does).  Rows that fit on chip are read once and
 * written once; wider rows take the split path, which needs `workspace` of at
 * least nt_softmax_workspace_bytes(M, N, dt) bytes (may be NULL when that is
 * 0): each workgroup takes one chunk of a row, computes its max and
 * denominator, merges those of the row's chunks, and writes its chunk.  Up to
 * 128 chunks per row this is one kernel that reads x once (the workgroups of a
 * row exchange their pairs through the workspace; a pair that does not arrive
 * within a bounded wait is recomputed from x, so the result does not depend on
 * scheduling); wider rows and in-place calls use two kernels and read x
 * twice.  Either way the results are bitwise the same.  The exchanged records
 * carry a tag unique to the call; a call made while the stream is being
 * captured into a graph reads its tag from a word in the 16 workspace bytes
 * after the records (nt_plan_launch's workspace_bytes - 16), which a
 * one-thread kernel captured ahead of it advances, so every replay of the
 * graph tags its records afresh.
 */
nt_status nt_softmax_rows(int64_t M, int64_t N, nt_dtype dt,
                          const void *x, void *y,
                          void *workspace, size_t workspace_bytes,
                          void *stream);

/*
 * nt_softmax_rows without a workspace argument, for callers that cannot
 * allocate device memory (code under graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the split path's records go to a device
 * array inside the library, NT_NOALLOC_SCRATCH_BYTES (1 MiB) per device,
 * which each device the library runs on holds until the process ends.  The
 * result is bitwise that of nt_softmax_rows.  Shapes whose workspace
 * (nt_softmax_workspace_bytes) exceeds the array return NT_ERR_WORKSPACE
 * before anything is enqueued; rows that fit on chip need none.  The call
 * allocates and frees nothing; the first call on a device looks the array's
 * address up once (NT_ERR_HIP if that fails).  Every call on a device
 * shares its array, so calls that overlap in time on one device (other
 * streams, other threads) race and must not be made; calls ordered on one
 * stream are fine.  Other arguments, checks and errors as nt_softmax_rows.
 */
#define NT_NOALLOC_SCRATCH_BYTES (1u << 20)
nt_status nt_softmax_rows_noalloc(int64_t M, int64_t N, nt_dtype dt, const void *x, void *y, void *stream);

/*
 * Causal, scaled softmax of attention-score rows.  Row r holds the scores of
 * query q = r mod `queries` (rows of several heads follow one another) against
 * N keys; key k is visible to it iff k <= q + offset (offset 0: square causal
 * attention, the diagonal kept; offset N - queries aligns the last query with
 * the last key).  Over the visible keys
 *   y[r, k] = exp(scale*x[r, k] - m) / sum_k' exp(scale*x[r, k'] - m),
 * m the max of scale*x over them, and y[r, k] = 0 at masked keys, whose x is
 * never read (it may hold anything).  The result is the plain softmax of the
 * row with its masked scores at -inf ("Portable Triton Kernels", "Safe
 * Softmax Pattern": a -inf entry contributes exactly nothing), computed
 * while reading only the visible part of each row: for square causal rows
 * about half the bytes of nt_softmax_rows.
 *
 * scale must be finite and > 0 (NT_ERR_SCALE); queries >= 1 and offset >= 0
 * (NT_ERR_SHAPE).  Layout, dtypes, alignment, workspace (sized by
 * nt_softmax_workspace_bytes for rows too wide to hold on chip), in-place
 * calls and errors as nt_softmax_rows.
 */
nt_status nt_softmax_causal_rows(int64_t M, int64_t N, nt_dtype dt, float scale,
                                 int64_t queries, int64_t offset,
                                 const void *x, void *y,
                                 void *workspace, size_t workspace_bytes,
                                 void *stream);

/*
 * LayerNorm over each row.  mean_r = sum_j x[r, j] / N,
 * var_r = sum_j (x[r, j] - mean_r)^2 / N (biased), rstd_r = 1/sqrt(var_r + eps),
 * y[r, j] = (x[r, j] - mean_r) * rstd_r * gamma[j] + beta[j].
 * mean and rstd (fp32, length M) are written when non-NULL.
 */
nt_status nt_layernorm_rows(int64_t M, int64_t N, nt_dtype dt, float eps,
                            const void *x, const void *gamma, const void *beta,
                            void *y, float *mean, float *rstd, void *stream);

/*
 * RMSNorm over each row.  inv_r = 1/sqrt(sum_j x[r, j]^2 / N + eps),
 * y[r, j] = x[r, j] * inv_r * weight[j].
 */
nt_status nt_rmsnorm_rows(int64_t M, int64_t N, nt_dtype dt, float eps,
                          const void *x, const void *weight, void *y,
                          void *stream);

/*
 * The norms with a workspace, for a few rows too wide for one pass.  There
 * the plain entry points stream each row twice with one workgroup, so M
 * rows keep at most M compute units busy.  With a workspace the row is cut
 * into chunks, one workgroup each, and every chunk's partial sums
 * (LayerNorm: sum(x - p) and sum((x - p)^2) around the row's first element
 * p, RMSNorm: sum(x^2); in fp64) go through the workspace.  Up to 128 chunks
 * per row this is one pass: the row's workgroups exchange their sums as
 * tagged records, each keeping its chunk in registers, and a record that
 * does not arrive within a bounded wait is recomputed from x by the waiting
 * workgroup (so the result never depends on scheduling; captured into a
 * graph, the tag comes from the workspace as for the softmax).  Beyond that,
 * or in place (y == x), two kernels: the
 * first writes the sums, the second combines them and writes the outputs,
 * reading x a second time.  Both forms combine a row's sums in the same
 * fixed order and give the same bits.  The statistics are those of the
 * definitions above, summed in another order than the one-workgroup
 * kernels' (results within the same tolerances, not necessarily bitwise
 * equal to them; repeated calls are bitwise equal).  This is the split
 * softmax's scheme ("How Flash Attention Uses Triton") applied to the
 * norms' sums.
 *
 * nt_norm_workspace_bytes(op, M, N, dt): bytes the split needs (32 per row
 * chunk, 8 per row, 16 for a captured call's tag) for op NT_OP_LAYERNORM or NT_OP_RMSNORM, 0 when the
 * plain plan is used (rows that fit one pass, or enough rows to fill the
 * GPU) or for invalid arguments.
 *
 * nt_layernorm_rows_ws / nt_rmsnorm_rows_ws take the plain entry points'
 * arguments, with their conventions and checks, plus `workspace` and
 * `workspace_bytes`: NULL runs the plain plan; otherwise workspace must be
 * 8-byte aligned (NT_ERR_ALIGN) and hold nt_norm_workspace_bytes(op, M, N, dt)
 * bytes (NT_ERR_WORKSPACE).  Contents need not be initialized; two calls in
 * flight at once must not share a workspace; a workspace overlapping x or y
 * is NT_ERR_ALIAS (overlapping the parameters is undefined).  In place
 * (y == x) is allowed.  The override NT_COOP=0 (nt_set_override) selects
 * the two kernels throughout.
 */
size_t nt_norm_workspace_bytes(int op, int64_t M, int64_t N, nt_dtype dt);

nt_status nt_layernorm_rows_ws(int64_t M, int64_t N, nt_dtype dt, float eps,
                               const void *x, const void *gamma, const void *beta,
                               void *y, float *mean, float *rstd,
                               void *workspace, size_t workspace_bytes, void *stream);

nt_status nt_rmsnorm_rows_ws(int64_t M, int64_t N, nt_dtype dt, float eps,
                             const void *x, const void *weight, void *y,
                             void *workspace, size_t workspace_bytes, void *stream);

/*
 * Fused residual add + norm: the step right before a norm in a residual
 * block, in one pass.  h = x + residual, rounded once to `dt` (the updated
 * residual stream), and the norm of that stored h:
 *
 *   nt_add_layernorm_rows  h, y = LayerNorm(h) as nt_layernorm_rows, mean, rstd
 *   nt_add_rmsnorm_rows    h, y = RMSNorm(h) as nt_rmsnorm_rows
 *
 * The pages list fused add + norm among the kernel patterns of "Portable
 * Triton Kernels" (References) and give fusion's point in "Triton:
 * Block-Level GPU Programming Without CUDA" (read each input once, write each
 * result once); no formula is printed.  The reading here: fusing changes no
 * bit, h is what an add kernel would store and y is bitwise what the plain
 * norm entry point computes from that h.  Traffic: x and residual read once,
 * h and y written once (against an extra write and read of h unfused).
 *
 * x, residual, h and y are [M, N] arrays of `dt` with the conventions above;
 * gamma, beta, weight, mean and rstd as in the plain norms.  residual and h
 * must be non-NULL (NT_ERR_NULL) and lie at the same address modulo 16 as x
 * (NT_ERR_ALIGN); y may have any element-aligned address.  h may be x or
 * residual (in place); y may be x or residual; any other overlap of h or y
 * with x, the residual or each other (y == h included) is NT_ERR_ALIAS.
 */
nt_status nt_add_layernorm_rows(int64_t M, int64_t N, nt_dtype dt, float eps,
                                const void *x, const void *residual,
                                const void *gamma, const void *beta,
                                void *h, void *y, float *mean, float *rstd,
                                void *stream);

nt_status nt_add_rmsnorm_rows(int64_t M, int64_t N, nt_dtype dt, float eps,
                              const void *x, const void *residual,
                              const void *weight, void *h, void *y,
                              void *stream);

/*
 * Tuning overrides, for tests and launch-shape sweeps (not needed in normal
 * use).  `name` is one of the NT_* settings below, each read once from the
 * environment variable of the same name when the library is loaded; `value`
 * is its new value, or NULL to restore the value read at load.  Returns
 * NT_ERR_OVERRIDE for an unknown name or a malformed value (nothing
 * changes), NT_ERR_NULL for a NULL name.  The settings are process-wide and
 * apply to calls planned after the change; change them only while no other
 * thread is calling the library.
 *   NT_FORCE_PATH      "split" (softmax: the split path at any width) or
 *                      "looped" (norms: the looped kernel at any width)
 *   NT_FORCE_SHAPE     "W,K": single-pass shape, ignored where it does not
 *                      fit the row or is not built
 *   NT_SPLIT_SHAPE     "W,K": chunk shape of the split softmax
 *   NT_COOP            "0": the two-kernel split forms throughout;
 *                      "rows1" / "rows2": the cooperative softmax with one /
 *                      two rows per workgroup where it is used
 *   NT_COOP_SPIN       polls (0..65536, default 1024) of a cooperative
 *                      kernel before it recomputes a missing record
 *   NT_PERSISTENT      "0" never, "1" where it pays (default), "always"
 *   NT_PERSIST_GRID    workgroups of the persistent norm kernel (> 0)
 *   NT_NORM_SPLIT_ROWS rows below which a wide norm row is split (>= 0)
 *   NT_DEBUG           "1": print each plan to stderr
 */
nt_status nt_set_override(const char *name, const char *value);

/*
 * Attention forward with the online softmax ("Triton: Block-Level GPU
 * Programming Without CUDA", section "How Flash Attention Uses Triton": the
 * loop over key/value tiles that carries the running max and denominator
 * and rescales the accumulator, never writing the scores out):
 *   o[b, i, :] = sum_j w_j v[b, j, :] / sum_j w_j,
 *   w_j = exp(s_j - max_j s_j),  s_j = scale * sum_c q[b, i, c] k[b, j, c],
 * over the keys j visible to query i: all Lk keys, or when `causal` is 1
 * only j <= i + offset (offset 0: square causal attention, the diagonal
 * kept; Lk - Lq aligns the last query with the last key).
 *
 * q is [BH, Lq, D], k and v [BH, Lk, D], o [BH, Lq, D]: dense row-major
 * arrays of `dt`, NT_F16 or NT_BF16 (else NT_ERR_DTYPE), each 16-byte
 * aligned (NT_ERR_ALIGN), none NULL (NT_ERR_NULL).  D is 64 or 128; Lk >= 1,
 * Lq >= 0, BH >= 0, offset >= 0, causal 0 or 1 (else NT_ERR_SHAPE).  scale
 * must be finite and > 0 (NT_ERR_SCALE); 1/sqrt(D) is the usual choice.
 * BH == 0 or Lq == 0 is a no-op.  o must not overlap q, k or v
 * (NT_ERR_ALIAS).  Errors are returned before anything is enqueued; the
 * work is enqueued on `stream`.
 *
 * Numerics: q.k on the matrix cores with fp32 accumulation, the softmax in
 * fp32, the weights kept to 16 significant bits (each split into two 16-bit
 * parts) for the weights-times-values product, accumulated in fp32; o is
 * rounded once to `dt`.  An output is within one unit in the last place of
 * the exact result plus 2^-12 times the size of the terms it sums
 * (sum_j w_j |v_j| / sum_j w_j).  Results are bitwise repeatable.
 */
nt_status nt_attention_fwd(int64_t BH, int64_t Lq, int64_t Lk, int64_t D, nt_dtype dt, float scale, int causal,
                           int64_t offset, const void *q, const void *k, const void *v, void *o, void *stream);

/* Static, human-readable name of a status code. */
const char *nt_status_string(nt_status s);

/*
 * Launch plan introspection (host only; touches no device).  Describes the
 * kernels the library would launch for an operation on this shape, when
 * every pointer is 16-byte aligned (`aligned16` != 0) or not, with every
 * parameter vector present.
 */
typedef NT_ENUM {
    NT_OP_SOFTMAX = 0,
    NT_OP_LAYERNORM = 1,
    NT_OP_RMSNORM = 2,
    NT_OP_ADD_LAYERNORM = 3,  /* nt_add_layernorm_rows */
    NT_OP_ADD_RMSNORM = 4,    /* nt_add_rmsnorm_rows   */
    NT_OP_SOFTMAX_CAUSAL = 5, /* nt_softmax_causal_rows */
    NT_OP_LAYERNORM_WS = 6,   /* nt_layernorm_rows_ws with a workspace */
    NT_OP_RMSNORM_WS = 7      /* nt_rmsnorm_rows_ws with a workspace   */
} nt_op;

typedef struct {
    int32_t split;            /* 0: single pass, row held on chip; 1: split online softmax
                                 (per-chunk workgroups and a workspace); 2: looped norm
                                 kernel (one workgroup streams a wide row twice); 3: split
                                 norm (per-chunk workgroups, partial sums in a workspace) */
    int32_t waves_per_row;    /* 64-lane waves cooperating on one row (or one chunk)    */
    int32_t chunks_per_lane;  /* 16-byte chunks each lane holds                         */
    int32_t rows_per_block;   /* rows one workgroup processes side by side              */
    int32_t threads_per_block;
    int32_t aligned;          /* 1 when the 16-byte-aligned variant is used             */
    int32_t persistent;       /* 1: norm kernel with parameters held in registers across
                                 rows; `grid` below is then k workgroups per compute unit
                                 (k from the row's bytes), capped at launch by how many
                                 fit on the device at once                                */
    int32_t cooperative;      /* split path: 1 when one kernel does both phases (x read once;
                                 the workgroups of a row exchange their partial results
                                 through the workspace), 2 when it does so for two rows
                                 per workgroup (softmax; rows_per_block 2); 0: two
                                 kernels, x read twice.  In-place calls (y == x) always
                                 use the two kernels                                     */
    int64_t grid;             /* workgroups per launch                                  */
    int64_t row_chunks;       /* split paths: chunks per row (0 otherwise)              */
    int64_t workspace_bytes;  /* split paths: workspace size (0 otherwise)              */
} nt_plan;

nt_status nt_plan_launch(nt_op op, int64_t M, int64_t N, nt_dtype dt,
                         int aligned16, nt_plan *out);

#undef NT_ENUM

#ifdef __cplusplus
}
#endif

#endif /* NT_H */
