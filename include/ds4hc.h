/*
 * ds4hc.h -- C ABI of libds4hc.so, the MI355X (gfx950) implementation of the
 * DeepSeek-V4 hyper-connection (HC) op.
 *
 * The op, as the lucebox pages describe it:
 *   - lucebox PR #496 "feat(ds4): add DSpark speculative runtime +
 *     optimizations", PR body: a fused DS4 hyper-connection op
 *     (GGML_OP_DS4_HC) with a register-resident Sinkhorn kernel.
 *   - lucebox-hub PR #494 "fix(ds4): keep ROCmFPX generation byte-safe":
 *     "HC-pre" as a decode cost centre (comment with the timing breakdown);
 *     commit notes on the HC fn matvecs, hc_post and the GPU HC pre-mix;
 *     the comment on the Sinkhorn kernel specialised for NHC = 4; and the
 *     direct HC-pre API left out of that PR.
 *   - lucebox PR #507 "correct layer-split HC handoff and per-device state",
 *     Summary/Implementation: the full HC state flows between layers, the HC
 *     fn weights are held as F16 per device, and HC scratch must be per
 *     device (a shared scratch buffer was a bug there).
 *
 * Definitions (n = n_hc streams, d features, K = n*d, m = 2n + n*n):
 *   X[t]      state of token t: n streams x d features, row-major
 *             (flattened index k = i*d + c).
 *   r         = sqrt(sum_k X[t]_k^2 / K + rms_eps)
 *   z_j       = sum_k W[j][k] * X[t]_k / r + bias[j]             (fn matvec)
 *   pre_i     = 1/(1+exp(-z_i)),  post_i = 1/(1+exp(-z_{n+i}))  (gates)
 *   H         = Sinkhorn of Z[i][j] = z_{2n+i*n+j}: M = exp(Z - rowmax(Z)),
 *               then sinkhorn_iters x (divide rows by their sums, then
 *               columns by their sums).
 *   layer_in[c] = sum_i pre_i * X[i][c]                           (pre-mix)
 *   X'[i][c]    = sum_j H[i][j] * X[j][c] + post_i * layer_out[c]  (hc_post)
 *   coeffs[t] = pre[0..n) | post[0..n) | H row-major [n*n]  (m floats)
 *
 * Conventions for every entry point:
 *   - All array pointers are DEVICE pointers on the calling thread's current
 *     HIP device, dense row-major with the shapes given. Alignment: the
 *     state-typed arrays (X, X_out, layer_in, layer_out and their _share
 *     forms) and W must be 16-byte aligned, since the kernels move them in
 *     16-byte vectors; the float32 arrays (bias, coeffs, coeffs_prev, logits,
 *     partials, logits_res, H) and the workspace need 4-byte alignment only.
 *     A pointer that misses its alignment is DS4HC_ERR_INVALID_ARG.
 *   - The caller owns every buffer; the library allocates no device memory.
 *     Its only global state is a per-device cache of the compute-unit count
 *     (looked up on a device's first call, read-only after, atomically
 *     published), a thread-local slot holding the last HIP error text, and
 *     the fixed scratch array of ds4hc_post_pre_noalloc (below) with its
 *     per-device address cache. Every other entry point is re-entrant and
 *     thread-safe.
 *   - Work is enqueued on `stream` (0 = the default stream) and the call
 *     returns without waiting. Faults during execution surface at the
 *     caller's next synchronisation of that stream.
 *   - Arguments are validated on the host before any HIP call. A rejected
 *     call enqueues nothing.
 *   - State dtype (X, layer_in, layer_out, X_out): float32 or bfloat16.
 *     Coefficients, logits and bias are float32; W is IEEE float16.
 *     Arithmetic is float32 with one round-to-nearest-even at each store.
 *     The Sinkhorn normalises by multiplying with the hardware reciprocal
 *     of each row or column sum (within 1 ulp of 1/sum) rather than by a
 *     correctly rounded division, and clamps each entry of H to at most 1
 *     (a NaN stays NaN); H is within a few float32 ulps of the divided result.
 *   - Every path is deterministic: no floating-point atomics, fixed
 *     reduction orders. Repeated calls on equal inputs give equal bits.
 *   - T = 0 returns DS4HC_OK once the scalar arguments are valid, without
 *     looking at any pointer (zero-size buffers may be NULL); nothing runs.
 *   - Supported on the GPU: n_hc in {1, 2, 4}; d > 0 with d % 8 == 0;
 *     0 <= T <= 2^24; sinkhorn_iters in [0, 1000].
 */
#ifndef DS4HC_H
#define DS4HC_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DS4HC_ABI_VERSION 1

typedef enum {
    DS4HC_OK = 0,
    DS4HC_ERR_INVALID_ARG = 1, /* null/misaligned pointer, bad shape, small workspace, overlap */
    DS4HC_ERR_UNSUPPORTED = 2, /* valid for the op, not supported by this GPU library */
    DS4HC_ERR_HIP = 3          /* a HIP launch failed; see ds4hc_last_hip_error() */
} ds4hc_status;

typedef enum {
    DS4HC_F32 = 0,  /* state stored as IEEE float32 */
    DS4HC_BF16 = 1  /* state stored as bfloat16 (uint16 bit patterns) */
} ds4hc_dtype;

/* Operation constants. Defaults: rms_eps = 1e-6f, sinkhorn_iters = 20. */
typedef struct {
    int32_t n_hc;           /* streams n: 1, 2 or 4 on the GPU */
    int32_t d;              /* features per stream, d % 8 == 0 */
    float rms_eps;          /* added to the mean square inside the sqrt, >= 0 */
    int32_t sinkhorn_iters; /* row-then-column normalisation rounds, 0..1000 */
    uint32_t flags;         /* DS4HC_FLAG_* */
} ds4hc_params;

/* Every path is deterministic already; the flag is accepted and changes nothing. */
#define DS4HC_FLAG_DETERMINISTIC 1u
/* Force one kernel path (all compute the same op; forcing more than one is
 * invalid). The default for HC-pre and fused is the cheapest by a cost model
 * in T and the row length K = n * d, fitted to measured times of every path
 * (at d = 4096 float32: split-K through T = 519, the tile kernel above):
 *   ROWRES  one token per workgroup, row kept in registers, VALU matvec;
 *   TILE    persistent, one workgroup per CU striding over tiles of four
 *           tokens, rows kept in registers, MFMA matvec;
 *   SPLITK  partials over column chunks into the workspace (4 tokens per
 *           workgroup below T = 32, 16 from T = 32), then a combining
 *           kernel. */
#define DS4HC_FLAG_FORCE_ROWRES 2u
#define DS4HC_FLAG_FORCE_SPLITK 4u
#define DS4HC_FLAG_FORCE_TILE 8u

/*
 * ds4hc_pre -- HC-pre: RMS statistic, fn matvec, sigmoid gates, Sinkhorn and
 * the pre-mix ("HC-pre" and the GPU "HC pre-mix", lucebox-hub PR #494).
 *   X          [T, n, d]  state dtype       (read)
 *   W_f16      [m, n*d]   float16 bits      (read)
 *   bias       [m]        float32           (read)
 *   layer_in   [T, d]     state dtype       (written)
 *   coeffs     [T, m]     float32           (written: pre | post | H)
 *   logits_opt [T, m]     float32 or NULL   (written: raw z, for debugging)
 *   workspace  device scratch of at least ds4hc_workspace_bytes(p, T, dtype)
 *              bytes (may be NULL when that is 0); contents need not be set
 *              and are overwritten. Calls that share one workspace must be
 *              ordered on one stream.
 * Outputs must not overlap inputs or each other.
 */
ds4hc_status ds4hc_pre(const ds4hc_params *p, int64_t T, ds4hc_dtype dtype, const void *X,
                       const uint16_t *W_f16, const float *bias, void *layer_in, float *coeffs,
                       float *logits_opt, void *workspace, size_t workspace_bytes,
                       hipStream_t stream);

/*
 * ds4hc_sinkhorn -- the register-resident Sinkhorn micro-kernel alone (the
 * NHC = 4 template kernel of lucebox-hub PR #494's comment on its 95 us ->
 * 5.3 us fix), on arbitrary residual logits.
 *   logits_res [T, n, n] float32 (read), H [T, n, n] float32 (written).
 * n_hc in {1, 2, 4}; iters in [0, 1000]. H may not overlap logits_res.
 */
ds4hc_status ds4hc_sinkhorn(int64_t T, int32_t n_hc, int32_t iters, const float *logits_res,
                            float *H, hipStream_t stream);

/*
 * ds4hc_post -- hc_post (lucebox-hub PR #494 commit notes): the post update
 * X' = H.X + post (x) layer_out from coefficients written by ds4hc_pre.
 *   X [T, n, d] state (read), coeffs [T, m] float32 (read),
 *   layer_out [T, d] state (read), X_out [T, n, d] state (written).
 * X_out may be exactly X (in-place update); any other overlap is invalid.
 */
ds4hc_status ds4hc_post(const ds4hc_params *p, int64_t T, ds4hc_dtype dtype, const void *X,
                        const float *coeffs, const void *layer_out, void *X_out,
                        hipStream_t stream);

/*
 * ds4hc_fused -- the whole op (GGML_OP_DS4_HC of lucebox PR #496) in one
 * call, for a layer_out that does not depend on this call's layer_in.
 * Arguments as in ds4hc_pre and ds4hc_post; coeffs_opt may be NULL.
 * X_out may be exactly X; layer_in must not overlap X, X_out or layer_out.
 */
ds4hc_status ds4hc_fused(const ds4hc_params *p, int64_t T, ds4hc_dtype dtype, const void *X,
                         const uint16_t *W_f16, const float *bias, const void *layer_out,
                         void *layer_in, float *coeffs_opt, void *X_out, void *workspace,
                         size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes ds4hc_pre / ds4hc_fused need for these arguments (0 when
 * the chosen path needs none). Pure function; 0 for invalid arguments. It takes
 * the state dtype because the path, and below T = 32 the split-K column-chunk
 * width (16 or 32 lanes x one 16-byte vector) and hence the number of partial
 * sums, depend on it. */
size_t ds4hc_workspace_bytes(const ds4hc_params *p, int64_t T, ds4hc_dtype dtype);

/*
 * ds4hc_post_pre -- one decode-chain step: the post update of site l followed
 * by HC-pre of site l+1, the two halves the pages run back to back on the GPU
 * with no host round trip between them ("hc_post" and "HC-pre", lucebox-hub
 * PR #494, comment on the GPU HC pre-mix and hc_post). With
 *   X' = H_l . X + post_l (x) layer_out_l            (coefficients from site l)
 * it writes X_out = X' and, for site l+1 on X' (as stored, in the state dtype):
 * layer_in = pre-mix, coeffs = pre | post | H, logits_opt = raw z.
 *   X            [T, n, d]  state dtype  (read)  state before site l's post
 *   coeffs_prev  [T, m]     float32      (read)  site l's coefficients
 *   layer_out    [T, d]     state dtype  (read)  site l's layer output
 *   W_f16_next   [m, n*d]   float16 bits (read)  site l+1's fn weight
 *   bias_next    [m]        float32      (read)
 *   X_out        [T, n, d]  state dtype  (written; may be exactly X)
 *   layer_in     [T, d]     state dtype  (written)
 *   coeffs       [T, m]     float32      (written; must not overlap coeffs_prev)
 *   workspace    >= ds4hc_post_pre_workspace_bytes(p, T, dtype) bytes
 * X' is bitwise what ds4hc_post writes. For T <= 160 (or DS4HC_FLAG_FORCE_SPLITK)
 * the state is read once: a split-K kernel over column chunks applies the post
 * update, stores X' and accumulates site l+1's partial projections, then a
 * combining kernel finishes site l+1. Otherwise it runs the post kernel, then
 * HC-pre on the path ds4hc_pre would take (or the forced one). Errors as for
 * ds4hc_fused.
 */
ds4hc_status ds4hc_post_pre(const ds4hc_params *p, int64_t T, ds4hc_dtype dtype, const void *X,
                            const float *coeffs_prev, const void *layer_out,
                            const uint16_t *W_f16_next, const float *bias_next, void *X_out,
                            void *layer_in, float *coeffs, float *logits_opt, void *workspace,
                            size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes ds4hc_post_pre needs for these arguments (0 if none or invalid). */
size_t ds4hc_post_pre_workspace_bytes(const ds4hc_params *p, int64_t T, ds4hc_dtype dtype);

/*
 * ds4hc_post_pre_noalloc -- ds4hc_post_pre for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc. Same arguments, semantics, kernels and results (bit
 * for bit) as ds4hc_post_pre, without the workspace: the split-K partial sums
 * go to a file-scope device array of DS4HC_NOALLOC_SCRATCH_BYTES bytes that
 * every device the library runs on holds until the process ends. The call
 * allocates nothing; on a device's first call it looks up the array's device
 * address (hipGetSymbolAddress) and keeps it.
 * Limit: a call whose ds4hc_post_pre_workspace_bytes(p, T, dtype) exceeds
 * DS4HC_NOALLOC_SCRATCH_BYTES returns DS4HC_ERR_UNSUPPORTED and enqueues
 * nothing (n = 4: T * P * 100 bytes with P = ceil(d / (16 * V)) column chunks
 * where that is at most 64, else ceil(d / (32 * V)); V = 4 for float32 and 8
 * for bfloat16 state; d = 4096 float32 fits every T of the one-pass path).
 * All calls on one device share that device's array, and the kernels
 * overwrite every byte they read before reading it (nothing must start at
 * zero). Calls that overlap on one device race on the array: order them on
 * one stream.
 */
#define DS4HC_NOALLOC_SCRATCH_BYTES (2u << 20)
ds4hc_status ds4hc_post_pre_noalloc(const ds4hc_params *p, int64_t T, ds4hc_dtype dtype,
                                    const void *X, const float *coeffs_prev, const void *layer_out,
                                    const uint16_t *W_f16_next, const float *bias_next,
                                    void *X_out, void *layer_in, float *coeffs, float *logits_opt,
                                    hipStream_t stream);

/*
 * Split over d (one GPU's share of the columns of every stream; the exchange
 * point of a tensor-parallel split, shown on one GPU). The op's only coupling
 * across columns is the 2n + n^2 fn dot products and the sum of squares of
 * each token row, so a share can emit those partial sums, the shares exchange
 * them ([T, m + 1] floats per share: an all-gather), and each share finishes
 * its own columns. p->d is the share's width d_s (d_s % 8 == 0).
 *
 * ds4hc_partials -- per token, over the share's columns:
 *   partials[t][j] = sum_k W_share[j][k] x_share[k]  (j < m, unnormalised)
 *   partials[t][m] = sum_k x_share[k]^2
 *   X_share   [T, n, d_s]    state dtype   (read)
 *   W_share   [m, n * d_s]   float16 bits  (read) W's columns i*d + share, per stream i
 *   partials  [T, m + 1]     float32       (written)
 *   workspace >= ds4hc_partials_workspace_bytes(p, T, dtype) bytes (0 for
 *               T > 160: a streamed kernel, 16 tokens per workgroup, writes the
 *               partials directly; split-K chunks below, or when forced)
 */
ds4hc_status ds4hc_partials(const ds4hc_params *p, int64_t T, ds4hc_dtype dtype, const void *X_share,
                            const uint16_t *W_share, float *partials, void *workspace,
                            size_t workspace_bytes, hipStream_t stream);
size_t ds4hc_partials_workspace_bytes(const ds4hc_params *p, int64_t T, ds4hc_dtype dtype);

/*
 * ds4hc_combine -- sums the G shares' partials [G, T, m + 1] in share order
 * (deterministic; every share that combines the same partials gets bitwise the
 * same coefficients), then z = dots / r + bias with r over all n * d_total
 * columns, the gates, the Sinkhorn, and pass 2 on this share: layer_in_share
 * = pre-mix, X_out_share = H . X_share + post (x) layer_out_share (may be
 * exactly X_share). coeffs_opt [T, m] may be NULL. d_total >= p->d.
 */
ds4hc_status ds4hc_combine(const ds4hc_params *p, int32_t d_total, int64_t T, ds4hc_dtype dtype,
                           int32_t G, const float *partials, const float *bias, const void *X_share,
                           const void *layer_out_share, void *layer_in_share, float *coeffs_opt,
                           void *X_out_share, hipStream_t stream);

/* Static, human-readable name of a status code. */
const char *ds4hc_status_string(ds4hc_status s);

/* Text of the last HIP error seen by a ds4hc call on this thread ("" if none). */
const char *ds4hc_last_hip_error(void);

/* DS4HC_ABI_VERSION of the loaded library. */
int ds4hc_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DS4HC_H */
