/*
 * drgg.h -- C ABI of the MI355X (gfx950) ragged BF16 grouped GEMM library
 * (libdrgg.so).
 *
 * The operation (flashinfer PR #8258, "run the split k512 wgrad tail whole
 * on the least-loaded clusters on sm_107a", opening summary paragraph): a
 * grouped GEMM for mixture-of-experts training whose E experts own
 * contiguous, ragged token ranges.  Three programs, all accumulating in FP32:
 *
 *   forward          Y  = X W^T     Y[t,:]  = X[t,:] W[e(t)]^T
 *   data gradient    dX = G W       dX[t,:] = G[t,:] W[e(t)]
 *   weight gradient  dW = G^T X     dW[e]   = sum over e's tokens of G[t,:]^T X[t,:]
 *
 * The dense projection GEMM (flashinfer PR #8363, "run the deterministic
 * program at the sm_107a token counts its new plans win", Summary) is the
 * E = 1 case with group_offsets = {0, M}.
 *
 * Shapes (all row-major and contiguous, BF16 unless stated):
 *   X [M, K]     activations / layer input       (M = total tokens)
 *   W [E, N, K]  expert weights, nn.Linear [out, in] layout per expert
 *   G [M, N]     output gradient
 *   Y [M, N], dX [M, K], dW [E, N, K]   outputs, BF16 or FP32
 *   group_offsets  int32 [E + 1] on the DEVICE: o[0] = 0, non-decreasing,
 *                  o[E] = M; expert e owns tokens o[e] .. o[e+1]-1.
 *
 * Variants (PR #8258 summary):
 *   deterministic != 0  bitwise reproducible from run to run, independent of
 *                       the CU count and of the work-to-CU mapping.  The
 *                       weight gradient cuts an expert's token range into
 *                       chunks by a rule that depends only on the problem
 *                       (never on the device), writes one FP32 partial per
 *                       chunk and folds the partials in chunk order before a
 *                       single rounding.
 *   deterministic == 0  routed by default to the deterministic program (whose
 *                       result is a valid non-deterministic result): on
 *                       gfx950 it was the faster one at every measured shape.
 *                       With DRGG_KNOB_NONDET = 1 the split program runs:
 *                       the weight gradient cuts an expert's token range into
 *                       chunks of whole 512-token units (the deterministic
 *                       chunk lengths rounded up); the pieces of a tile cut
 *                       into several chunks add their FP32 partials into an
 *                       FP32 tile sum with atomic adds, and a per-tile ticket
 *                       picks the last arrival, which reads and clears the sum
 *                       and writes the output tile (a piece that finds every
 *                       other piece already done adds its own partial in
 *                       registers instead).  The summation order of a split
 *                       tile can differ from run to run.  Forward and
 *                       data gradient have no split and are identical in both
 *                       modes (PR #8363, Summary: the dense non-deterministic
 *                       forward and input gradient are the deterministic
 *                       programs).
 *
 * Conventions for every entry point:
 *   * Pointers are device pointers unless a comment says "host".
 *   * The caller owns every buffer, including outputs and the workspace; the
 *     library allocates no device memory on any call path.
 *   * Calls are asynchronous on `stream` (NULL = the default stream) and do
 *     not synchronise; group_offsets is read only by the kernels.  Calls are
 *     capturable into a HIP graph.
 *   * Argument checks run on the host before anything is enqueued; on any
 *     error nothing is enqueued and the status says why
 *     (drgg_status_string).  By default the offsets are not checked on the
 *     host (they live on the device and the call does not synchronise); the
 *     kernels clamp every offset into [0, M] so that no access leaves the
 *     buffers, and the result for invalid offsets is unspecified.  With the
 *     debug check on (environment DRGG_CHECK_OFFSETS=1, or
 *     DRGG_KNOB_CHECK_OFFSETS), a grouped call first copies the offsets to
 *     the host synchronously and returns DRGG_ESHAPE unless o[0] = 0, they
 *     are non-decreasing and o[E] = M; nothing of the computation is
 *     enqueued then.  The check cannot be graph-captured (it synchronises),
 *     which is why it is off by default; this follows the fail-closed
 *     precedent of flashinfer PR #7516 (#7632 commit body: a program that
 *     cannot run raises and says why rather than launching).
 *   * Alignment: every pointer 16-byte aligned; N and K multiples of 8.
 *   * Limits: 1 <= E <= 1024, 0 <= M < 2^31, 8 <= N, K <= 2^22, and every
 *     buffer size below 2^62 bytes (checked in 64-bit arithmetic).
 */
#ifndef DRGG_H
#define DRGG_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DRGG_ABI_VERSION 1

typedef enum {
    DRGG_BF16 = 0,
    DRGG_FP32 = 1
} drgg_dtype;

typedef enum {
    DRGG_OP_FWD = 0,
    DRGG_OP_DGRAD = 1,
    DRGG_OP_WGRAD = 2
} drgg_op;

typedef enum {
    DRGG_OK = 0,
    DRGG_EINVAL = 1,        /* null pointer, bad enum value, E out of range   */
    DRGG_ESHAPE = 2,        /* negative or too large dimension; offsets that
                               fail the debug check                           */
    DRGG_EALIGN = 3,        /* pointer not 16-byte aligned, N or K not % 8    */
    DRGG_EOVERFLOW = 4,     /* a size product overflows 64-bit arithmetic     */
    DRGG_EWORKSPACE = 5,    /* workspace missing or smaller than required; a
                               split-program workspace that is not zero (debug
                               check)                                         */
    DRGG_EUNSUPPORTED = 6,  /* no program for this device or combination      */
    DRGG_EDEVICE = 7        /* HIP error while querying the device or launching */
} drgg_status;

/*
 * Forward: Y[t,n] = sum_k X[t,k] * W[e(t),n,k], FP32 accumulation, one
 * rounding to out_dtype.  X [M,K] BF16, W [E,N,K] BF16, Y [M,N] out_dtype.
 * Rows of Y are written only for tokens 0..M-1 (all of them, since the
 * experts' ranges cover [0, M)).  No workspace is needed (workspace may be
 * NULL with workspace_bytes = 0).
 */
drgg_status grouped_gemm_fwd(const void *X, const void *W, const int32_t *group_offsets,
                             int32_t E, int64_t M, int64_t N, int64_t K,
                             drgg_dtype out_dtype, int deterministic, void *Y,
                             void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Data gradient: dX[t,k] = sum_n G[t,n] * W[e(t),n,k].  G [M,N] BF16,
 * W [E,N,K] BF16, dX [M,K] out_dtype.  The workspace is optional: when the
 * experts average at least 3072 tokens (M >= 3072 * E) and the workspace has
 * at least grouped_gemm_workspace_size(DRGG_OP_DGRAD, ...) bytes (E*N*K*2,
 * rounded up to 256; 16-byte aligned), W is first transposed into it
 * (W^T [E,K,N]) and the product runs with both operands
 * reduction-contiguous, which is faster at those token counts; otherwise
 * (fewer tokens per expert, a smaller workspace, or NULL) W is read
 * transposed by the kernel, and the workspace size is 0 below that count.
 * The results are bitwise the same either way.  The workspace needs no
 * initialisation and holds W^T after a call that used it.
 */
drgg_status grouped_gemm_dgrad(const void *G, const void *W, const int32_t *group_offsets,
                               int32_t E, int64_t M, int64_t N, int64_t K,
                               drgg_dtype out_dtype, int deterministic, void *dX,
                               void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Weight gradient: dW[e,n,k] = sum_{t = o[e]}^{o[e+1]-1} G[t,n] * X[t,k];
 * experts without tokens get dW[e] = +0.  X [M,K] BF16, G [M,N] BF16,
 * dW [E,N,K] out_dtype.
 * Workspace: at least grouped_gemm_workspace_size(DRGG_OP_WGRAD, ...) bytes.
 *   deterministic != 0: FP32 chunk partials and a small per-expert table
 *     that the chunk kernel writes for the ordered fold; no initialisation
 *     needed.  None (size 0, the pointer may be null) when no expert can be
 *     cut into chunks (M at most the plan's chunk_max).
 *   deterministic == 0, routed (the default): as deterministic != 0.
 *   deterministic == 0, split program (DRGG_KNOB_NONDET = 1): FP32 tile sums
 *     and tickets that must be zero before the first call
 *     (drgg_workspace_init); every call leaves them zero again.  A buffer
 *     that served a deterministic (or routed) call holds partials afterwards
 *     and must be zeroed again before a split-program call; with the debug
 *     check on (environment DRGG_CHECK_WORKSPACE=1, or
 *     DRGG_KNOB_CHECK_WORKSPACE) a split-program call copies the workspace to
 *     the host first and returns DRGG_EWORKSPACE if any byte is set.
 *   Two calls in flight at once must not share a workspace.
 */
drgg_status grouped_gemm_wgrad(const void *X, const void *G, const int32_t *group_offsets,
                               int32_t E, int64_t M, int64_t N, int64_t K,
                               drgg_dtype out_dtype, int deterministic, void *dW,
                               void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * The weight gradient for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): grouped_gemm_wgrad with the same arguments minus the
 * workspace, which comes from a fixed array in device memory that the
 * library holds per device (64 MiB, allocated when the library's kernels are
 * loaded on that device and held until the process ends).  Same programs,
 * same results: the deterministic variant is bitwise that of
 * grouped_gemm_wgrad.  A problem whose workspace
 * (grouped_gemm_workspace_size) exceeds 64 MiB gets DRGG_EWORKSPACE with
 * nothing enqueued.  The call allocates nothing: before a split-program call
 * it clears the part of the array the tile sums and tickets use with a fill
 * kernel on `stream`.  Every call on one device shares that device's array,
 * and it keeps the last call's contents: calls that overlap on one device
 * (on different streams, or from different threads) race on it and must be
 * serialised by the caller.
 */
drgg_status grouped_gemm_wgrad_noalloc(const void *X, const void *G, const int32_t *group_offsets,
                                       int32_t E, int64_t M, int64_t N, int64_t K,
                                       drgg_dtype out_dtype, int deterministic, void *dW,
                                       hipStream_t stream);

/*
 * Batched projection GEMM: the projection family also covers batched
 * products (PR #8363, Summary; its #8438 commit body names batched "MLA head
 * rows"), read here as B independent products of one shape -- batch b has
 * its own weight W[b] and T token rows -- with the token-major buffers
 * addressed through element strides, so that a head-interleaved activation
 * [T, H, K] (MLA's per-head projections, batch = head) is used in place:
 *
 *   row t of batch b of a token-major buffer = base + b*batch + t*row
 *   (elements; each row is contiguous: K values for X and dX, N for G and Y)
 *
 * W [B, N, K] and dW [B, N, K] are contiguous.  Same programs, rounding and
 * determinism as the grouped calls; the result is bitwise that of the
 * grouped call on the same rows laid out contiguously with
 * group_offsets = {0, T, 2T, ..., B*T}.  Strides: row >= the row length,
 * batch >= 0, both multiples of 8, row <= 2^22 (DRGG_ESHAPE / DRGG_EALIGN
 * otherwise); an output's rows must not overlap: its batches either stacked
 * (batch >= (T-1)*row + row length) or interleaved (row >= (B-1)*batch +
 * row length, batch >= row length), else DRGG_ESHAPE.  B in 1..1024,
 * B*T <= 2^31-1.  Workspace: as for the grouped call with E = B,
 * M = B*T (grouped_gemm_workspace_size); the forward needs none.
 */
typedef struct {
    int32_t B;                 /* batches */
    int64_t T;                 /* token rows per batch */
    int64_t N, K;              /* output features, input features */
    int64_t a_row, a_batch;    /* fwd, wgrad: X; dgrad: G */
    int64_t b_row, b_batch;    /* wgrad: G (unused otherwise) */
    int64_t o_row, o_batch;    /* fwd: Y; dgrad: dX (unused for wgrad) */
} drgg_batched;

drgg_status batched_gemm_fwd(const void *X, const void *W, const drgg_batched *shape,
                             drgg_dtype out_dtype, void *Y, hipStream_t stream);
drgg_status batched_gemm_dgrad(const void *G, const void *W, const drgg_batched *shape,
                               drgg_dtype out_dtype, void *dX, void *workspace,
                               size_t workspace_bytes, hipStream_t stream);
drgg_status batched_gemm_wgrad(const void *X, const void *G, const drgg_batched *shape,
                               drgg_dtype out_dtype, int deterministic, void *dW,
                               void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * FP32 router GEMM out[m,n] = sum_k X[m,k] * Wr[n,k] computed on BF16 MFMA
 * as a BF16x3 split (PR #8363, Summary: the family's router GEMM has 256
 * experts and emulates FP32 with three BF16 products): each FP32 operand
 * value v is split into
 * hi = bf16(v), lo = bf16(v - hi) (round to nearest even) and every product
 * is taken as hi*hi + hi*lo + lo*hi with FP32 accumulation.
 * X [M,K] FP32, Wr [N,K] FP32, out [M,N] FP32.  K must be a multiple of 8,
 * N a multiple of 4 (DRGG_EALIGN otherwise), both at most 2^22 and
 * M < 2^31 (DRGG_ESHAPE otherwise).  Deterministic (one fixed order).
 */
drgg_status router_gemm_fp32_bf16x3(const float *X, const float *Wr, int64_t M, int64_t N,
                                    int64_t K, float *out, hipStream_t stream);

/*
 * The same FP32 router GEMM (the same BF16x3 products, PR #8363, Summary),
 * in the program drgg_router_split picks from (M, N, K): when the single-pass
 * program's 128x128 tiles alone fill 256 workgroups (or K > 2^21) that
 * program runs, as router_gemm_fp32_bf16x3; otherwise the sliced program:
 * 256x256 output tiles with the reduction cut into ks slices of kq values,
 * slice 0 summed into `out`, slices 1 .. ks-1 into the workspace, and a second
 * kernel adding them to `out` in slice order.  Deterministic either way (a
 * function of M, N, K; the sliced result is not bitwise the single-pass one,
 * whose sum runs over all of K in one chain).  Arguments and limits as
 * router_gemm_fp32_bf16x3; `workspace` is a DEVICE buffer of at least
 * router_workspace_size bytes, 16-byte aligned (may be NULL when that size is
 * 0), owned by the caller and overwritten; calls that share one workspace
 * must not overlap.  DRGG_EWORKSPACE if it is missing or too small,
 * DRGG_EALIGN if misaligned.
 */
drgg_status router_gemm_fp32_bf16x3_ws(const float *X, const float *Wr, int64_t M, int64_t N,
                                       int64_t K, float *out, void *workspace,
                                       size_t workspace_bytes, hipStream_t stream);

/*
 * Workspace bytes (to *bytes, a HOST pointer) of router_gemm_fp32_bf16x3_ws:
 * (ks - 1) * M * N * 4 for the sliced program, else 0 (PR #8363, Summary,
 * the router GEMM).  Shape errors as router_gemm_fp32_bf16x3.
 */
drgg_status router_workspace_size(int64_t M, int64_t N, int64_t K, size_t *bytes);

/*
 * The program router_gemm_fp32_bf16x3_ws runs (host only, HOST pointers):
 * *ks = 0 (and *kq = K) for the single-pass program, which runs when
 * ceil(M/128) * ceil(N/128) >= 256 or K > 2^21; else *ks slices of *kq values
 * (a multiple of 32; the last slice may be shorter), with
 * ceil(M/256) * ceil(N/256) * ks workgroups reaching 256 where K allows (at
 * most 8 slices, none shorter than 256 values).
 */
drgg_status drgg_router_split(int64_t M, int64_t N, int64_t K, int64_t *ks, int64_t *kq);

/*
 * Workspace bytes (written to *bytes, a HOST pointer) that a call with these
 * arguments needs; they do not depend on the CU count (cu_count is accepted
 * for symmetry with drgg_plan and ignored).  0 bytes for fwd; for dgrad the
 * optional W^T buffer (0 when the experts average fewer than 3072 tokens);
 * for wgrad the buffers of the variant's reduction:
 * the deterministic variant's per-chunk FP32 partials, folded in a fixed
 * order, or the split program's shared FP32 tile sums and per-tile tickets
 * (flashinfer PR #8258, Summary: the split tail adds FP32 partial tiles into
 * a shared sum, and a per-tile ticket picks the last arrival).  The caller
 * allocates it (the library allocates nothing).
 */
drgg_status grouped_gemm_workspace_size(drgg_op op, int32_t E, int64_t M, int64_t N, int64_t K,
                                        drgg_dtype out_dtype, int deterministic, int cu_count,
                                        size_t *bytes);

/* Zero a workspace on `stream` with a fill kernel (capturable): needed once
 * before its first split-program weight-gradient call, because the tile
 * sums and tickets of PR #8258's split tail (Summary) start at zero and the
 * last arrival on each tile clears them again. */
drgg_status drgg_workspace_init(void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * The plan a call would use, for inspection (HOST only, touches no GPU when
 * cu_count > 0).  Fields are written to *out (a host pointer).  The output
 * tile is 256x256 unless the call is too small to fill the CUs with it: a
 * forward or data gradient with at most half a wave of 256x256 tiles (even
 * with every group's rows packed), or whose groups average fewer than 128
 * tokens, takes 128x128, one with between one and
 * one and a half waves (both operands reduction-contiguous) 128x256; a
 * deterministic weight gradient none of whose groups can be cut into chunks
 * takes 128x128 up to 32 tiles of 256x256 and 128x256 up to 128, one with
 * chunks 128x128 up to 128 work items (tiles x chunks); outputs of
 * at most 128 columns take 128x128 and weight gradients with N <= 64 64x256.
 * The results do not depend on the tile.
 */
typedef struct {
    int32_t tile_m, tile_n, tile_k;   /* output tile and reduction step        */
    int32_t mfma_m, mfma_n, mfma_k;   /* MFMA instruction shape               */
    int64_t grid;                     /* workgroups launched (persistent)     */
    int64_t chunk_max;                /* wgrad det: longest token chunk; 0 otherwise */
    int64_t unit;                     /* wgrad split program: token units; 0 otherwise */
    int64_t max_partials;             /* wgrad det: partial slots reserved     */
    size_t workspace_bytes;
} drgg_plan_info;

drgg_status drgg_plan(drgg_op op, int32_t E, int64_t M, int64_t N, int64_t K,
                      drgg_dtype out_dtype, int deterministic, int cu_count, drgg_plan_info *out);

/*
 * The chunk rule of the deterministic weight gradient (HOST): the token count
 * of each chunk of an expert with T tokens is returned in *chunk_len (host),
 * and the number of chunks in *chunks.  chunk_max comes from drgg_plan.
 * Mirrors exactly what the device computes.
 */
drgg_status drgg_wgrad_chunking(int64_t T, int64_t chunk_max, int64_t *chunk_len, int64_t *chunks);

/*
 * Test knobs (process-wide; not thread-safe; 0 restores the default):
 *   DRGG_KNOB_TILE        force the output tile of fwd/dgrad/det-wgrad:
 *                         1 = 256x256, 2 = 128x128, 3 = 256x128, 4 = 128x256
 *   DRGG_KNOB_GRID        force the workgroup count of the persistent kernels
 *                         (every program)
 *   DRGG_KNOB_REVERSE     1 = walk the work items in reverse order
 *   DRGG_KNOB_NONDET      1 = a non-deterministic weight gradient runs the
 *                         split program (atomic tile sums) instead of being
 *                         routed to the deterministic one; the workspace
 *                         size and plan follow the program chosen
 *   DRGG_KNOB_TIMING      1 = record a HIP event on the stream before every
 *                         kernel launch of a call and after its last launch
 *                         (read back with drgg_timing_read)
 *   DRGG_KNOB_CHECK_OFFSETS    1 = the synchronous offsets check described
 *                         above (0 = as the environment says)
 *   DRGG_KNOB_CHECK_WORKSPACE  1 = the split program's zero-workspace check
 *                         (0 = as the environment says)
 *   DRGG_KNOB_DELAY_SEED  n > 0: the split program's tail pieces sleep a
 *                         bounded, seeded time (under 50 000 cycles) before
 *                         adding their partial, so that the arrivals at a
 *                         tile's ticket come in other orders (race testing)
 *   DRGG_KNOB_SPLIT_REPORT  a 16-byte aligned DEVICE address of four int32
 *                         where the split program writes {slack placement
 *                         taken (0/1), tail tiles of the banded walk, banded
 *                         walk taken (0/1), grid}; 0 = off
 *   DRGG_KNOB_DGRAD_WT    1 = the data gradient transposes W into its
 *                         workspace at every size (0 = only when the experts
 *                         average at least 3072 tokens)
 * None of them changes the arithmetic of the deterministic variant.
 */
enum { DRGG_KNOB_TILE = 1, DRGG_KNOB_GRID = 2, DRGG_KNOB_REVERSE = 3, DRGG_KNOB_TIMING = 4,
       DRGG_KNOB_NONDET = 5, DRGG_KNOB_CHECK_OFFSETS = 6, DRGG_KNOB_CHECK_WORKSPACE = 7,
       DRGG_KNOB_DELAY_SEED = 8, DRGG_KNOB_SPLIT_REPORT = 9, DRGG_KNOB_DGRAD_WT = 10 };
drgg_status drgg_set_knob(int knob, int64_t value);

/*
 * Route table of the non-deterministic weight gradient (HOST only).  A call
 * with deterministic == 0 runs the deterministic program unless its point
 * (E, M, N, K, out_dtype), matched exactly, is in this table; then it runs
 * the split program (atomic FP32 tile sums and tickets, its workspace zeroed
 * as described at grouped_gemm_wgrad; the batched weight gradient's point is
 * E = B, M = B*T).  The entries come from a calibration on the device that
 * will run them: the package's calibrate module measures both programs at a
 * point and keeps the split one only where it passes the selection rule of
 * PR #8363 (Summary; restated as three conditions in its #8438 commit body):
 * faster in every run at the op level (one-sided paired sign test p < 0.05,
 * median ratio < 0.99) in eager launches and graph replays, at most 3 %
 * slower next to a kernel holding 8, 16 or 32 compute units, and the
 * backward and checkpointed step at most 1.3 % slower.  DRGG_KNOB_NONDET = 1
 * overrides the table (split program everywhere).
 *   drgg_route_split   add a point (no-op if present; DRGG_EUNSUPPORTED when
 *                      256 points are stored; shape checks as for the calls)
 *   drgg_route_clear   remove every point
 *   drgg_route_count   number of points stored
 * Thread-safe; a change applies to calls planned afterwards.
 */
drgg_status drgg_route_split(int32_t E, int64_t M, int64_t N, int64_t K, drgg_dtype out_dtype);
/* Calibration aid for the co-run condition: occupies `cus` compute units
 * (one workgroup with a whole CU's LDS each) for `microseconds` on `stream`,
 * then exits.  cus in 1..4096, microseconds in 0..10^6, else DRGG_EINVAL. */
drgg_status drgg_hold_cus(int cus, int64_t microseconds, hipStream_t stream);
drgg_status drgg_route_clear(void);
int drgg_route_count(void);

/*
 * With DRGG_KNOB_TIMING on: the number of kernels the most recent call
 * launched, and for kernel i (0-based, launch order) its name (*kernel, a
 * static string) and duration in milliseconds (*ms), both HOST pointers.
 * drgg_timing_read waits for that kernel to finish.
 */
int drgg_timing_count(void);
drgg_status drgg_timing_read(int i, const char **kernel, float *ms);

/*
 * The deterministic weight gradient's plan for these group offsets (HOST
 * only; group_offsets is a HOST array [E + 1]; the kernel makes the same
 * choice on the device).  Experts cut into chunks run either every output
 * tile as chunk items ("all-split"), or the tiles of their first 256-row
 * bands whole, in full waves on their share of 256 reference workgroups,
 * and only the remaining tiles -- the tail -- as chunk items ("tail-only";
 * flashinfer PR #8258, Summary: only the tail's K range is split).  The
 * kernel takes the tail-only plan when its planned walk is not slower on 256
 * reference workgroups; the choice depends on the problem only.  Writes
 * *tail_only (HOST) = 1 for the tail-only plan, and, if row0 (HOST, E
 * entries) is given, the first dW row of each expert that comes from folded
 * partials (0 for all rows).  DRGG_EINVAL for null pointers or E, N, K out
 * of range.
 */
drgg_status drgg_wgrad_tail_plan(const int32_t *group_offsets, int32_t E, int64_t N, int64_t K,
                                 int *tail_only, int32_t *row0);

/*
 * The split program's walk (HOST only; group_offsets is a HOST array
 * [E + 1]; the kernel makes the same choice on the device) for a grid of
 * `grid` workgroups and the output tile `tile` (a DRGG_KNOB_TILE value, 0 =
 * the default).  Banded walk: each expert's whole tiles first, in full
 * waves on its share of the grid, then its remaining tiles, the tail, either
 * whole or cut into chunks of 512-token units (an expert's tail is cut only
 * when the tail-split rule of drgg_tailsplit_units allows it on its share).
 * Slack placement (flashinfer PR #8258, Summary): the workgroups are ranked
 * by the load of their first-pass tiles, and if the i-th tail tile fits
 * whole on the i-th least-loaded workgroup for every i (within the largest
 * load plus one tail share, a chunk of that expert) the whole tail runs that
 * way, with no tile sums and no tickets.  All-split walk: every tile of an
 * expert cut into chunks runs as chunk items.  The banded walk runs when its
 * estimated time on the grid is not above the all-split walk's.  Writes
 * *slack (HOST) = 1 when the tail is placed whole, *tail_tiles (HOST) = the
 * number of tail tiles of the banded walk, and *banded_walk (HOST, may be
 * NULL) = 1 when the banded walk runs.  DRGG_EINVAL for null pointers or bad
 * arguments.
 */
drgg_status drgg_wgrad_split_plan(const int32_t *group_offsets, int32_t E, int64_t N, int64_t K, int tile,
                                  int64_t grid, int *slack, int64_t *tail_tiles, int *banded_walk);

/*
 * The tail-split rule of a persistent schedule (HOST only; flashinfer
 * PR #7516, #7632 commit body, its tail-split routing test): `tiles` equal
 * output tiles on `workers` persistent workers run in full waves plus a
 * partial last wave of tail = tiles mod workers tiles; when
 * 2 * tail <= workers each tail tile is cut in two along the reduction
 * (2 * tail half units), otherwise every tile stays whole.  Writes
 * out[0..3] = (tiles, units handed out, tiles run whole, pieces per tail
 * tile) to a HOST array of four.  DRGG_EINVAL for a null out, tiles < 0 or
 * workers < 1.
 */
drgg_status drgg_tailsplit_units(int64_t tiles, int64_t workers, int64_t *out);

/* Text of a status code, with the HIP error name and text appended for
 * DRGG_EDEVICE (the fail-closed precedent of PR #7516, #7632 commit body:
 * an error names what failed and why). */
const char *drgg_status_string(drgg_status status);
int drgg_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DRGG_H */
