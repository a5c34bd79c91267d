/*
 * libdora: the DoRA forward hot path on AMD Instinct MI355X (gfx950).
 *
 * DoRA writes an adapted weight as W' = m * (W + sBA) / ||W + sBA||_row
 * ("Scaling DoRA: High-Rank Adaptation via Factored Norms and Fused Kernels",
 * summary on alanhou.org, "The Problem"). This library computes the two
 * pieces of that forward pass that dominate its cost:
 *
 *   dora_factored_norm  the row norm ||W + sBA||_row without forming BA,
 *                       through ||W||^2 + 2s<W,BA> + s^2||BA||^2 with
 *                       U = W A^T and G = A A^T ("DoRA优化技术解析：从内存瓶颈到
 *                       高效实现", cyqw.cn, §1.2, §1.2.1, §5.1 Algorithm 1),
 *                       and optionally g = m / max(wnorm, eps) (same page,
 *                       §1.2.2);
 *   dora_compose        the stable magnitude compose
 *                       (g - 1) * base + g * (s * lora) in one pass
 *                       (same page, §2.1, §2.1.1, §5.2);
 *   dora_compose_backward
 *                       its gradients d_base, d_lora and dg (dm) in one
 *                       pass plus a deterministic column reduction (same
 *                       page, §4.2, §5.2, §6.1 Table 9).
 *
 * Conventions shared by every entry point:
 *   - Matrices are dense, row-major and contiguous. Layouts follow LoRA:
 *     W [d_out, d_in], A [r, d_in], B [d_out, r]; activations [T, d_out].
 *   - Device pointers are device memory the caller owns (e.g. torch
 *     tensors). The library allocates nothing and never frees or retains
 *     a pointer. Its only host state is the device address of the
 *     dora_factored_norm_noalloc scratch array on each GPU, looked up once
 *     per GPU and never changed.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     All work is enqueued asynchronously on it; results are valid once
 *     the stream has reached that point. Calls enqueue kernels only (no
 *     memset, copy, allocation or host synchronisation; counters a call
 *     needs are cleared by one of its own kernels), so a sequence of calls
 *     can be captured into a HIP graph and replayed; a replay depends on
 *     nothing an earlier call left in the workspace.
 *   - Errors: arguments are checked on the host before any launch. A
 *     failed check returns a non-zero dora_status and enqueues nothing.
 *     A HIP launch error returns DORA_ERR_HIP. No exception crosses this
 *     ABI and no call aborts the process.
 *   - Results are bitwise reproducible from run to run for the same
 *     arguments: reductions use a fixed order and no floating-point
 *     atomics.
 */
#ifndef DORA_H_
#define DORA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dora_status {
  DORA_OK = 0,
  DORA_ERR_INVALID_ARG = 1,       /* null pointer, negative size, bad alias  */
  DORA_ERR_UNSUPPORTED_DTYPE = 2, /* dtype code not in dora_dtype            */
  DORA_ERR_BUDGET = 3,            /* workspace needed exceeds the budget     */
  DORA_ERR_WORKSPACE = 4,         /* workspace pointer too small / misaligned */
  DORA_ERR_HIP = 5                /* a HIP runtime or launch call failed     */
} dora_status;

typedef enum dora_dtype {
  DORA_BF16 = 0, /* bfloat16 storage, fp32 arithmetic */
  DORA_F32 = 1,  /* binary32 storage and arithmetic   */
  DORA_F16 = 2   /* binary16 storage, fp32 arithmetic (accumulation in fp32;
                    G = A A^T, which may exceed binary16's range, is held as
                    bf16 hi + lo or in fp32) */
} dora_dtype;

/* Human-readable name of a status code (static string, never NULL). */
const char* dora_status_string(int status);

/* Library version as major*10000 + minor*100 + patch. */
int dora_version(void);

/*
 * Chunk width of the factored norm's d_in loop, as the cyqw.cn page defines
 * it (§5.1 Algorithm 1, step 1): the fp32 chunk buffer [d_out, cs] must fit
 * `budget_bytes`, aligned to 64 elements. cs = min(d_in, max(64,
 * 64 * floor(floor(budget / (4 d_out)) / 64))); cs = d_in when d_out or
 * d_in is 0. Host only; never touches the GPU.
 * Returns DORA_ERR_INVALID_ARG for negative sizes or cs == NULL.
 */
dora_status dora_norm_chunk_size(int64_t d_out, int64_t d_in, size_t budget_bytes,
                                 int64_t* cs);

/*
 * Bytes of device workspace dora_factored_norm needs for this shape.
 * The planner picks the most parallel split whose workspace fits
 * `budget_bytes`; the same arguments always give the same plan.
 * s == 0 or r == 0 needs no workspace (the cross and Gram terms are
 * skipped, cyqw.cn §5.1 notes). Host only; never touches the GPU.
 * Returns DORA_ERR_BUDGET if even the least parallel plan does not fit,
 * DORA_ERR_INVALID_ARG for negative sizes or ws_bytes == NULL,
 * DORA_ERR_UNSUPPORTED_DTYPE for an unknown dtype.
 */
dora_status dora_norm_workspace_size(int64_t d_out, int64_t d_in, int64_t r, int dtype,
                                     float s, size_t budget_bytes, size_t* ws_bytes);

/*
 * The plan dora_factored_norm would use, for diagnostics and benchmarks.
 * Fills info[0 .. n_info-1] with, in order: mode (0 nothing to do, 1 row
 * sum of squares only, 2 factored, 3 dense fused; in mode 3 the factored
 * fields describe the fallback used when the pointers do not allow aligned
 * 16-byte loads), W-pass column tile width, W-pass column
 * tiles, Gram-pass column tile width, Gram-pass column tiles, streaming and
 * general kernel configuration of the W pass, the same of the Gram pass,
 * d_in granule (elements), granules over d_in, d_in ranges of the W pass,
 * d_in ranges of the Gram pass, workspace bytes, W-pass grid and Gram-pass
 * grid of the streaming kernel, its LDS bytes in the W pass, the rows of
 * its W-pass tile, and 1 if the streaming W pass computes G itself (no
 * separate Gram pass; gram grid and ranges then do not apply), else 0,
 * 1 if the streaming Gram pass computes only the tiles on and above the
 * diagonal of G, else 0, and 1 if the streaming W pass also runs the Gram
 * term (B G) . B in its own accumulators (every dtype when G is not
 * folded in; no separate Gram-term pass), else 0, the index of the W
 * pass among the call's launches (see dora_factored_norm_marked), and 1 if
 * every operand tile of the streaming kernel spans less than 2^31 bytes
 * (its 32-bit buffer offsets; otherwise the general kernel runs), else 0,
 * and in mode 3 the dense pass's row tiles (64 rows) and column tiles (128
 * columns of d_in), else 0 and 0, and the d_in range groups of the
 * streaming W pass's die grid (the dies as range groups by row groups, so
 * that B's rows of a row tile are fetched by that many dies instead of one
 * die per range), 0 where it keeps the plain order; the streaming fields
 * apply when W, A and B allow aligned 16-byte loads.
 * Entries past the last field are set to -1.
 * Before returning it replays the plan on the host and checks that the
 * d_in ranges tile d_in exactly, every grid fits and every partial sum the
 * kernels write lies inside its workspace region; DORA_ERR_INVALID_ARG if
 * not. Host only; never touches the GPU.
 */
dora_status dora_norm_plan_info(int64_t d_out, int64_t d_in, int64_t r, int dtype, float s,
                                size_t budget_bytes, int64_t* info, int n_info);

/*
 * Factored row norm and magnitude scale (cyqw.cn §1.2, §1.2.1, §1.2.2,
 * §5.1 Algorithm 1; alanhou.org "Factored Norm").
 *
 *   wnorm[j] = sqrt(max(base[j] + 2s*cross[j] + s^2*ba[j], 0))
 *     base[j]  = sum_k W[j,k]^2
 *     cross[j] = sum_l B[j,l] * U[j,l],      U = W A^T   [d_out, r]
 *     ba[j]    = sum_l (B G)[j,l] * B[j,l],  G = A A^T   [r, r]
 *   g[j]     = m[j] / max(wnorm[j], eps)      (only if m != NULL)
 *
 * Inputs W, A, B are device pointers of storage type `dtype`; all
 * accumulation is fp32. U never leaves the matrix-core accumulators; BA is
 * never formed.
 *
 * Where r >= d_out, or r > d_in with d_out <= 4096 (bf16 and fp16, d_in
 * and r multiples of 8, plan mode 3), the Gram matrix or the Gram term
 * would cost more than B A itself, and the call computes the same wnorm
 * by its definition instead: a dense fused pass forms each 64 x 128 tile
 * of W + s B A in the matrix-core accumulators, squares it and keeps only
 * its row sums (cyqw.cn §1.1), and a second launch adds each row's tile
 * sums in a fixed order and takes the root. No tile of B A leaves the
 * chip; the workspace is the larger of the two paths' (the factored path
 * runs instead when W, A or B is not 16-byte aligned).
 *
 * wnorm (and g) are fp32 [d_out] device arrays written by the call. m is
 * an fp32 [d_out] device array or NULL (then g is not written and may be
 * NULL). A NaN in the inputs propagates to wnorm and g.
 *
 * `workspace` must hold at least dora_norm_workspace_size(...) bytes
 * (256-byte aligned) for the same (d_out, d_in, r, dtype, s, budget);
 * it may be NULL when that size is 0. Its contents on entry are ignored.
 *
 * Sizes may be 0: d_out == 0 does nothing; d_in == 0 gives wnorm = 0;
 * r == 0 or s == 0 gives wnorm = ||W||_row.
 *
 * Errors: DORA_ERR_INVALID_ARG (negative size, non-finite s or eps, eps <= 0,
 * required pointer NULL, output overlapping an input), DORA_ERR_UNSUPPORTED_DTYPE,
 * DORA_ERR_BUDGET (plan does not fit budget_bytes), DORA_ERR_WORKSPACE
 * (workspace_bytes too small or pointer misaligned), DORA_ERR_HIP.
 */
dora_status dora_factored_norm(const void* W, const void* A, const void* B, int dtype,
                               int64_t d_out, int64_t d_in, int64_t r, float s,
                               size_t budget_bytes, void* workspace, size_t workspace_bytes,
                               float* wnorm, const float* m, float eps, float* g,
                               void* stream);

/*
 * dora_factored_norm with timing marks: the same computation, arguments,
 * results and errors, and in addition HIP events recorded on `stream`
 * between the call's launches, so that a caller (a benchmark, a profiler)
 * can time each kernel of the norm on its own. events[0 .. n_events-1] are
 * hipEvent_t handles the caller created and owns; the call records
 * events[0] before its first launch and events[i] after its i-th launch,
 * for i < n_events (at most 8 are used); null entries are skipped (each
 * recorded event adds a little time between launches, so a caller that
 * times one launch passes only the two events around it). Nothing is kept
 * after the call returns. Launches of one call, in order:
 *   G not folded in: Gram pass, gram_reduce (fp16: which also splits B
 *     into bf16 hi + lo for the W pass), W pass with the Gram term (and
 *     the assembly when the W pass runs in one round of at most 256
 *     workgroups with at most 16 partials per row), assembly otherwise;
 *   G folded into the W pass (plan field gram_folded): W pass with G,
 *     gram_reduce, (fp16: widening of B,) Gram term (+ assembly with
 *     several Gram-term tiles);
 *   dense fused (plan mode 3): dense pass, assembly;
 *   s == 0, r == 0 or d_in == 0: one row-sum launch.
 * (These are the streaming-path launches, used when W, A and B allow
 * aligned 16-byte loads; plan field w_launch is the W pass's index i, which
 * lies between events[i] and events[i+1].)
 * Errors: those of dora_factored_norm, and DORA_ERR_INVALID_ARG for
 * n_events < 0 or events NULL with n_events > 0.
 */
dora_status dora_factored_norm_marked(const void* W, const void* A, const void* B, int dtype,
                                      int64_t d_out, int64_t d_in, int64_t r, float s,
                                      size_t budget_bytes, void* workspace, size_t workspace_bytes,
                                      float* wnorm, const float* m, float eps, float* g,
                                      void* stream, void* const* events, int n_events);

/*
 * Bytes of the device scratch array behind dora_factored_norm_noalloc: the
 * largest norm workspace that entry point can use (32 MiB per GPU).
 */
#define DORA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/*
 * dora_factored_norm for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation, arguments, results and errors, except
 * that there is no workspace argument. The workspace is a library-owned
 * array of DORA_NOALLOC_SCRATCH_BYTES in device memory, one per GPU, held
 * until the process ends; the call allocates nothing (no hipMalloc, no
 * library allocator). The plan is made under min(budget_bytes,
 * DORA_NOALLOC_SCRATCH_BYTES); a shape whose least parallel plan needs more
 * returns DORA_ERR_BUDGET before anything is enqueued. With the same plan
 * the results are bitwise those of dora_factored_norm. The scratch keeps
 * the last call's partial sums; every call overwrites what it reads, so
 * nothing needs clearing between calls. All calls on one GPU share its
 * scratch: calls that overlap in time on one GPU (on different streams, or
 * from different threads without ordering) race and give wrong results;
 * order them, e.g. on one stream. The first call on each GPU looks up the
 * array's device address (hipGetSymbolAddress, that GPU current); later
 * calls reuse it.
 */
dora_status dora_factored_norm_noalloc(const void* W, const void* A, const void* B, int dtype,
                                       int64_t d_out, int64_t d_in, int64_t r, float s,
                                       size_t budget_bytes, float* wnorm, const float* m, float eps,
                                       float* g, void* stream);

/*
 * g[j] = m[j] / max(wnorm[j], eps), fp32, on the device (cyqw.cn §1.2.2:
 * the magnitude division is kept apart from the fused kernels). A NaN
 * wnorm gives a NaN g. g may alias m or wnorm exactly.
 * Errors: DORA_ERR_INVALID_ARG (NULL pointer with d_out > 0, negative
 * d_out, eps not finite or <= 0), DORA_ERR_HIP.
 */
dora_status dora_magnitude_scale(const float* m, const float* wnorm, float eps,
                                 int64_t d_out, float* g, void* stream);

/*
 * out[j] = wnorm[j] rounded to the storage type `dtype` (round to nearest
 * even; DORA_F32 copies): the cast with which Algorithm 1 returns the norm
 * (cyqw.cn §5.1, step 7). dora_factored_norm keeps wnorm and g in fp32;
 * callers that want the pages' input-dtype norm apply this to its wnorm.
 * wnorm: fp32 [n] device array; out: [n] device array of `dtype`, owned by
 * the caller, not overlapping wnorm. Asynchronous on `stream`.
 * Errors: DORA_ERR_INVALID_ARG (negative n, NULL pointer with n > 0,
 * misaligned or overlapping pointers), DORA_ERR_UNSUPPORTED_DTYPE,
 * DORA_ERR_HIP.
 */
dora_status dora_norm_to_dtype(const float* wnorm, int64_t n, int dtype, void* out, void* stream);

/*
 * Stable magnitude compose (cyqw.cn §2.1, §2.1.1, §5.2):
 *
 *   out[t,j] = (g[j] - 1) * base[t,j] + g[j] * (s * lora[t,j])
 *
 * base, lora and out are [T, d_out] device arrays of storage type `dtype`;
 * g is an fp32 [d_out] device array. Arithmetic is fp32: s*lora is formed
 * first, then one fused multiply-add g*(s*lora) + (g-1)*base, rounded once
 * to the output type (round-to-nearest-even). One pass: base, lora and g
 * are read once and out is written once.
 * The result is the delta the DoRA layer adds to its base output.
 *
 * out may alias base or lora exactly (in-place); partial overlap is
 * rejected. T == 0 or d_out == 0 does nothing.
 * Errors: DORA_ERR_INVALID_ARG (NULL pointer with T*d_out > 0, negative
 * size, non-finite s, partial overlap), DORA_ERR_UNSUPPORTED_DTYPE,
 * DORA_ERR_HIP.
 */
dora_status dora_compose(const void* base, const void* lora, const float* g, float s,
                         int dtype, int64_t T, int64_t d_out, void* out, void* stream);

/*
 * DoRA layer output: the compose delta added to the base projection
 * (cyqw.cn §2.1.1: the layer returns base + delta; "Scaling DoRA",
 * alanhou.org, "The Problem": the adapted weight is m * V / ||V||_row with
 * V = W + sBA, so y = x V'^T = g * (base + s * lora) with base = x W^T,
 * lora = x A^T B^T):
 *
 *   y[t,j] = base[t,j] + ((g[j] - 1) * base[t,j] + g[j] * (s * lora[t,j]))
 *
 * Same arguments, layout, ownership and errors as dora_compose, with y in
 * place of out. The delta is formed in fp32 exactly as dora_compose forms
 * it, base is added in fp32, and y is rounded once to the storage type, in
 * the same single pass (base and lora read once, y written once).
 */
dora_status dora_layer_output(const void* base, const void* lora, const float* g, float s,
                              int dtype, int64_t T, int64_t d_out, void* y, void* stream);

/*
 * Workspace bytes dora_compose_backward needs to produce dg for a [T, d_out]
 * problem (at most 256 * d_out * 4). Host only. DORA_ERR_INVALID_ARG for
 * negative sizes or ws_bytes == NULL.
 */
dora_status dora_compose_backward_workspace_size(int64_t T, int64_t d_out, size_t* ws_bytes);

/*
 * Backward of the stable compose (cyqw.cn §4.2, §5.2, §6.1 Table 9 report
 * this fused backward; its formulas are the plain derivative of
 * delta = (g - 1) * base + g * (s * lora) with the row norm detached):
 *
 *   d_base[t,j] = (g[j] - 1) * dy[t,j]               (fp32, RNE to dtype)
 *   d_lora[t,j] = g[j] * (s * dy[t,j])               (fp32, RNE to dtype)
 *   dg[j]       = sum_t dy[t,j] * (base[t,j] + s * lora[t,j])     (fp32)
 *   dm[j]       = dg[j] / max(wnorm[j], eps)   (g = m / max(wnorm, eps))
 *
 * dy, base, lora, d_base, d_lora: device [T, d_out] row-major of `dtype`.
 * g, wnorm, dg, dm: fp32 [d_out] device arrays. Any of d_base, d_lora, dg
 * may be NULL to skip that output; with dg == NULL (magnitude frozen) base
 * and lora are not read and may be NULL. dm requires dg, wnorm and eps > 0.
 * dg is summed in fp32 in a fixed order (each thread's rows in increasing
 * order, then row blocks in increasing order): reproducible for a fixed
 * shape, no atomics. Outputs overlap no input and no other output.
 * `workspace` (256-byte aligned, dora_compose_backward_workspace_size bytes)
 * is needed only when dg != NULL; its contents on entry are ignored.
 * Asynchronous on `stream`.
 *
 * Errors: DORA_ERR_INVALID_ARG (negative size, non-finite s, bad eps,
 * missing or misaligned pointer, overlapping buffers),
 * DORA_ERR_UNSUPPORTED_DTYPE, DORA_ERR_WORKSPACE, DORA_ERR_HIP.
 */
dora_status dora_compose_backward(const void* dy, const void* base, const void* lora, const float* g,
                                  float s, int dtype, int64_t T, int64_t d_out, void* d_base,
                                  void* d_lora, float* dg, const float* wnorm, float eps, float* dm,
                                  void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DORA_H_ */
