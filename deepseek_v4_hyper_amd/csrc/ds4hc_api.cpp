// ds4hc_api.cpp -- the C ABI declared in include/ds4hc.h: host-side argument
// validation, choice between the row-resident and split-K paths, and launch.
//
// Nothing here touches the GPU until every argument has been checked, so all
// rejections are free of side effects. The library allocates no device memory:
// per-device scratch is the caller's workspace argument, except for
// ds4hc_post_pre_noalloc, whose scratch is a fixed device array with one copy
// per device. (lucebox PR #507 "correct layer-split HC handoff and per-device
// state" fixed a bug where an HC scratch buffer was shared across devices;
// scratch that is the caller's, or a device-resident array looked up per
// device, cannot have it.)
#include "ds4hc.h"

#include <algorithm>
#include <math.h>
#include <stdio.h>
#include <string.h>

#include "hc_launch.hpp"

namespace {

// T at or below which the one-pass chain step and the split-K partials of the
// split over d are the defaults.
constexpr int64_t SPLITK_MAX_T = 160;
constexpr int64_t MAX_T = int64_t(1) << 24;
constexpr int MAX_ITERS = 1000;
constexpr uint64_t MAX_WORK_ITEMS = 0xFFFFFFFFull;  // HSA dispatch grid size is 32-bit
// The streamed partials kernel forms 32-bit byte offsets up to 64 * n * d_s;
// longer share rows take split-K (ds4hc::STREAM_K_MAX).
constexpr uint64_t STREAM_MAX_K = (uint64_t)ds4hc::STREAM_K_MAX;
constexpr uint32_t FORCE_FLAGS =
    DS4HC_FLAG_FORCE_ROWRES | DS4HC_FLAG_FORCE_TILE | DS4HC_FLAG_FORCE_SPLITK;
constexpr uint32_t KNOWN_FLAGS = DS4HC_FLAG_DETERMINISTIC | FORCE_FLAGS;

thread_local char g_last_hip_error[256] = "";

ds4hc_status hip_fail(hipError_t e) {
    snprintf(g_last_hip_error, sizeof g_last_hip_error, "%s: %s", hipGetErrorName(e),
             hipGetErrorString(e));
    return DS4HC_ERR_HIP;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

struct Range {
    const void *p;
    uint64_t bytes;
};

bool overlap(Range a, Range b) {
    if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
    return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

int state_bytes(ds4hc_dtype dt) { return dt == DS4HC_F32 ? 4 : 2; }
int vec_elems(ds4hc_dtype dt) { return dt == DS4HC_F32 ? 4 : 8; }

// Checks shared by pre / post / fused on the op constants.
ds4hc_status check_params(const ds4hc_params *p, int64_t T, ds4hc_dtype dt) {
    if (!p) return DS4HC_ERR_INVALID_ARG;
    if (dt != DS4HC_F32 && dt != DS4HC_BF16) return DS4HC_ERR_INVALID_ARG;
    if (T < 0 || p->n_hc < 1 || p->d <= 0 || p->d % 8 != 0) return DS4HC_ERR_INVALID_ARG;
    if (!(p->rms_eps >= 0.f) || !isfinite(p->rms_eps)) return DS4HC_ERR_INVALID_ARG;
    if (p->sinkhorn_iters < 0) return DS4HC_ERR_INVALID_ARG;
    if (p->flags & ~KNOWN_FLAGS) return DS4HC_ERR_INVALID_ARG;
    const uint32_t force = p->flags & FORCE_FLAGS;
    if (force & (force - 1)) return DS4HC_ERR_INVALID_ARG;  // more than one path forced
    if (p->n_hc != 1 && p->n_hc != 2 && p->n_hc != 4) return DS4HC_ERR_UNSUPPORTED;
    if (p->sinkhorn_iters > MAX_ITERS || T > MAX_T) return DS4HC_ERR_UNSUPPORTED;
    return DS4HC_OK;
}

struct Plan {
    int path;              // ds4hc::PATH_*
    int P;                 // split-K chunks
    uint64_t ws_bytes;     // workspace needed
};

// Path for HC-pre / fused: split-K for small T (the fn weight dominates the
// bytes and must be spread over many CUs), the one-token VALU kernel for
// middling T, the persistent MFMA tile kernel for large T (measured on MI355X
// at n = 4: 141.5 us against 258 us for the VALU kernel at T = 4096, d = 4096
// float32, and 557 us against 1333 us at T = 16384, d = 7168 bfloat16), then
// the VALU kernel, then split-K where a row is too long for either.
// Default path of HC-pre / fused: the cheapest by a cost model fitted to
// sweeps of every path on MI355X (graph-replayed ds4hc_fused, n = 4: f32
// d = 4096 and bf16 d = 7168 over T = 1 .. 2048, f32 d = 256, 1024, 2048 and
// bf16 d = 256 over T = 1 .. 256), in microseconds with K = n * d and sb the
// state's bytes per element:
//   split-K       6 + (3.9e-7 + 6.75e-7 * sb) * T * K, at least 6.9 (T = 1)
//                 or 8.6 (two kernels' latency); fitted where it meets the
//                 tile kernel (it is concave in T above ~300)
//                                                        (swept up to T = 1024)
//   row-resident  16 + 1.6e-4 * K, + 6 * (T - 192) / 64 for 192 < T <= 256
//                 (one token per CU)
//   tile          32.3 + 2.6e-4 * (K - 16384) from K = 16384, 5 + 1.65e-3 * K
//                 below (a tile's weight stream)         (flat while T <= 1024)
// Beyond those ranges the tile kernel where it fits. Measured points (split-K
// streams its partials from T = 32):
// f32 d = 4096: split-K 12.5 / 18.9 / 29.5 / 32.0 / 43.0 us at T = 128 / 256 /
// 448 / 512 / 768 against tile 31.4 / 32.4 / 32.5 / 32.7 / 33.4.
// bf16 d = 7168: split-K 14.7 / 22.1 / 26.5 / 31.8 / 32.9 / 44.6 at T = 128 /
// 256 / 320 / 448 / 512 / 768 against row-resident 19.6 / 26.0 / 34.5 / - and
// tile 35.3 - 36.9 / 37.9.
// f32 d = 256: tile 6.6 / 7.1 / 7.5 us at T = 1 / 4 / 256 against split-K
// 6.8 / 8.5 / 9.2; d = 1024: split-K 7.0 / 8.8 against tile 8.6 / 10.9.
int default_path(int64_t T, int64_t K, int sb, bool fits_rowres, bool fits_tile) {
    constexpr double NONE = 1e30;
    const double k = (double)K, t = (double)T;
    const double splitk = T <= 1024 ? std::max(6.0 + (3.9e-7 + 6.75e-7 * sb) * t * k, T == 1 ? 6.9 : 8.6) : NONE;
    const double rowres = fits_rowres && T <= 256 ? 16.0 + 1.6e-4 * k + (T > 192 ? 6.0 * (t - 192.0) / 64.0 : 0.0) : NONE;
    const double tile = !fits_tile ? NONE : K >= 16384 ? 32.3 + 2.6e-4 * (k - 16384.0) : 5.0 + 1.65e-3 * k;
    if (splitk <= rowres && splitk <= tile && splitk < NONE) return ds4hc::PATH_SPLITK;
    if (rowres <= tile && rowres < NONE) return ds4hc::PATH_ROWRES;
    if (fits_tile) return ds4hc::PATH_TILE;
    return fits_rowres ? ds4hc::PATH_ROWRES : ds4hc::PATH_SPLITK;
}

// Returns UNSUPPORTED if a forced path cannot take the shape or a launch
// would not fit.
ds4hc_status make_plan(const ds4hc_params *p, int64_t T, ds4hc_dtype dt, Plan *out) {
    const int n = p->n_hc, d = p->d, m = 2 * n + n * n;
    const bool fits_rowres = ds4hc::rowres_chunks(d, dt) <= ds4hc::rowres_max_chunks(n, dt);
    const bool fits_tile = ds4hc::tile_steps(d, dt) <= ds4hc::tile_max_steps();
    const uint32_t force = p->flags & FORCE_FLAGS;
    int path;
    if (force == DS4HC_FLAG_FORCE_ROWRES) {
        if (!fits_rowres) return DS4HC_ERR_UNSUPPORTED;
        path = ds4hc::PATH_ROWRES;
    } else if (force == DS4HC_FLAG_FORCE_TILE) {
        if (!fits_tile) return DS4HC_ERR_UNSUPPORTED;
        path = ds4hc::PATH_TILE;
    } else if (force == DS4HC_FLAG_FORCE_SPLITK) {
        path = ds4hc::PATH_SPLITK;
    } else {
        path = default_path(T, (int64_t)n * d, state_bytes(dt), fits_rowres, fits_tile);
    }
    Plan pl{path, 0, 0};
    if (path == ds4hc::PATH_ROWRES) {
        if ((uint64_t)T * 256u > MAX_WORK_ITEMS) return DS4HC_ERR_UNSUPPORTED;
    } else if (path == ds4hc::PATH_TILE) {
        // persistent grid: at most one workgroup per CU, whatever T is
    } else {
        // partials grid (token groups, P): 4 tokens by 64 threads per group on
        // the column-chunk kernel, 16 by 512 on the streamed one; finish grid
        // (T, column blocks)
        const bool streamed = ds4hc::splitk_streams(T, (int64_t)n * d);
        pl.P = streamed ? ds4hc::stream_chunks(T, n * d) : ds4hc::colchunk_chunks(d, dt);
        const uint64_t tg_threads = streamed ? (uint64_t)(T + 15) / 16 * 512u : (uint64_t)(T + 3) / 4 * 64u;
        const uint64_t cb = (uint64_t)(d + 64 * vec_elems(dt) - 1) / (64 * vec_elems(dt));
        if (tg_threads > MAX_WORK_ITEMS || pl.P > 0xFFFF || (uint64_t)T * 64u > MAX_WORK_ITEMS || cb > 0xFFFFu)
            return DS4HC_ERR_UNSUPPORTED;
        pl.ws_bytes = (uint64_t)pl.P * (uint64_t)T * (uint64_t)(m + 1) * sizeof(float);
    }
    *out = pl;
    return DS4HC_OK;
}

ds4hc_status run_hc(bool fused, const ds4hc_params *p, int64_t T, ds4hc_dtype dt, const void *X,
                    const uint16_t *W, const float *bias, const void *layer_out, void *layer_in,
                    float *coeffs, float *logits, void *X_out, void *workspace,
                    size_t workspace_bytes, hipStream_t stream) {
    ds4hc_status st = check_params(p, T, dt);
    if (st != DS4HC_OK || T == 0) return st;  // zero tokens: nothing is read or written
    if (!X || !W || !bias || !layer_in) return DS4HC_ERR_INVALID_ARG;
    if (!fused && !coeffs) return DS4HC_ERR_INVALID_ARG;
    if (fused && (!layer_out || !X_out)) return DS4HC_ERR_INVALID_ARG;
    if (!aligned(X, 16) || !aligned(W, 16) || !aligned(layer_in, 16) || !aligned(bias, 4) ||
        (coeffs && !aligned(coeffs, 4)) || (logits && !aligned(logits, 4)) ||
        (fused && (!aligned(layer_out, 16) || !aligned(X_out, 16))) ||
        (workspace && !aligned(workspace, 4)))
        return DS4HC_ERR_INVALID_ARG;

    Plan pl;
    st = make_plan(p, T, dt, &pl);
    if (st != DS4HC_OK) return st;
    if (pl.ws_bytes > 0 && (!workspace || workspace_bytes < pl.ws_bytes))
        return DS4HC_ERR_INVALID_ARG;

    const int n = p->n_hc, d = p->d, m = 2 * n + n * n;
    const uint64_t sb = (uint64_t)state_bytes(dt), K = (uint64_t)n * d, uT = (uint64_t)T;
    const Range rX{X, uT * K * sb}, rW{W, (uint64_t)m * K * 2}, rb{bias, (uint64_t)m * 4};
    const Range rlo{fused ? layer_out : nullptr, uT * d * sb};
    const Range rli{layer_in, uT * d * sb}, rc{coeffs, uT * m * 4}, rz{logits, uT * m * 4};
    const Range rXo{fused ? X_out : nullptr, uT * K * sb};
    const Range rws{pl.ws_bytes ? workspace : nullptr, pl.ws_bytes};
    // Outputs must not overlap any other buffer, except that X_out may be exactly X.
    const Range all[] = {rX, rW, rb, rlo, rli, rc, rz, rXo, rws};
    constexpr int FIRST_OUT = 4, N_ALL = 9;
    for (int a = FIRST_OUT; a < N_ALL; ++a) {
        for (int b = 0; b < N_ALL; ++b) {
            if (a == b) continue;
            const bool in_place = (a == 7 && b == 0) && X_out == X;
            if (!in_place && overlap(all[a], all[b])) return DS4HC_ERR_INVALID_ARG;
        }
    }

    ds4hc::FusedArgs a{n, d, (int)dt, p->sinkhorn_iters, T, p->rms_eps, X, W, bias, layer_out,
                       layer_in, coeffs, logits, X_out, static_cast<float *>(workspace)};
    const hipError_t e = ds4hc::launch_hc(a, fused, pl.path, stream);
    return e == hipSuccess ? DS4HC_OK : hip_fail(e);
}

// Plan for post(l) + pre(l+1): one pass over the state for small T (split-K
// over column chunks; also when split-K is forced), else post then the pre
// path make_plan picks (or the forced one).
struct PostPrePlan {
    bool one_pass;
    Plan pre;          // pre path when !one_pass
    uint64_t ws_bytes;
};

ds4hc_status make_post_pre_plan(const ds4hc_params *p, int64_t T, ds4hc_dtype dt, PostPrePlan *out) {
    const uint32_t force = p->flags & FORCE_FLAGS;
    PostPrePlan pp{};
    pp.one_pass = force == DS4HC_FLAG_FORCE_SPLITK || (force == 0 && T <= SPLITK_MAX_T);
    if (pp.one_pass) {
        const int m = 2 * p->n_hc + p->n_hc * p->n_hc;
        const uint64_t P2 = (uint64_t)ds4hc::colchunk_chunks(p->d, dt);
        const uint64_t tg = (uint64_t)(T + 3) / 4;
        if (tg * 64u > MAX_WORK_ITEMS || P2 > 0xFFFFu || (uint64_t)T * 64u > MAX_WORK_ITEMS)
            return DS4HC_ERR_UNSUPPORTED;
        pp.ws_bytes = P2 * (uint64_t)T * (uint64_t)(m + 1) * sizeof(float);
    } else {
        const ds4hc_status st = make_plan(p, T, dt, &pp.pre);
        if (st != DS4HC_OK) return st;
        const uint64_t cb = (uint64_t)(p->d + 64 * vec_elems(dt) - 1) / (64 * vec_elems(dt));
        if (cb > 0xFFFFu || (uint64_t)T * 64u > MAX_WORK_ITEMS) return DS4HC_ERR_UNSUPPORTED;
        pp.ws_bytes = pp.pre.ws_bytes;
    }
    *out = pp;
    return DS4HC_OK;
}

// ds4hc_post_pre and its variant that allocates nothing: the same validation,
// plan and kernels; with `noalloc` the workspace is the library's device-resident
// scratch array instead of the caller's buffer.
ds4hc_status post_pre_impl(const ds4hc_params *p, int64_t T, ds4hc_dtype dtype, const void *X,
                           const float *coeffs_prev, const void *layer_out,
                           const uint16_t *W_f16_next, const float *bias_next, void *X_out,
                           void *layer_in, float *coeffs, float *logits_opt, void *workspace,
                           size_t workspace_bytes, bool noalloc, hipStream_t stream) {
    ds4hc_status st = check_params(p, T, dtype);
    if (st != DS4HC_OK || T == 0) return st;
    if (!X || !coeffs_prev || !layer_out || !W_f16_next || !bias_next || !X_out || !layer_in ||
        !coeffs)
        return DS4HC_ERR_INVALID_ARG;
    if (!aligned(X, 16) || !aligned(layer_out, 16) || !aligned(W_f16_next, 16) ||
        !aligned(X_out, 16) || !aligned(layer_in, 16) || !aligned(coeffs_prev, 4) ||
        !aligned(bias_next, 4) || !aligned(coeffs, 4) || (logits_opt && !aligned(logits_opt, 4)) ||
        (workspace && !aligned(workspace, 4)))
        return DS4HC_ERR_INVALID_ARG;
    PostPrePlan pp;
    st = make_post_pre_plan(p, T, dtype, &pp);
    if (st != DS4HC_OK) return st;
    if (noalloc) {
        // the static array has a fixed size: larger needs are refused, not allocated
        if (pp.ws_bytes > ds4hc::NOALLOC_SCRATCH_BYTES) return DS4HC_ERR_UNSUPPORTED;
        workspace = nullptr;
        workspace_bytes = 0;
    } else if (pp.ws_bytes > 0 && (!workspace || workspace_bytes < pp.ws_bytes)) {
        return DS4HC_ERR_INVALID_ARG;
    }

    const int n = p->n_hc, d = p->d, m = 2 * n + n * n;
    const uint64_t sb = (uint64_t)state_bytes(dtype), K = (uint64_t)n * d, uT = (uint64_t)T;
    const Range rX{X, uT * K * sb}, rcp{coeffs_prev, uT * m * 4}, rlo{layer_out, uT * d * sb};
    const Range rW{W_f16_next, (uint64_t)m * K * 2}, rb{bias_next, (uint64_t)m * 4};
    const Range rXo{X_out, uT * K * sb}, rli{layer_in, uT * d * sb}, rc{coeffs, uT * m * 4};
    const Range rz{logits_opt, uT * m * 4}, rws{pp.ws_bytes ? workspace : nullptr, pp.ws_bytes};
    // Outputs must not overlap any other buffer, except that X_out may be exactly X.
    const Range all[] = {rX, rcp, rlo, rW, rb, rXo, rli, rc, rz, rws};
    constexpr int FIRST_OUT = 5, N_ALL = 10;
    for (int a = FIRST_OUT; a < N_ALL; ++a) {
        for (int b = 0; b < N_ALL; ++b) {
            if (a == b) continue;
            const bool in_place = ((a == 5 && b == 0) || (a == 0 && b == 5)) && X_out == X;
            if (!in_place && overlap(all[a], all[b])) return DS4HC_ERR_INVALID_ARG;
        }
    }
    if (noalloc && pp.ws_bytes > 0) {
        // every argument is valid: now the device address of the scratch array
        // (a symbol lookup on the device's first call, no allocation)
        const hipError_t e = ds4hc::noalloc_scratch(&workspace);
        if (e != hipSuccess) return hip_fail(e);
    }
    ds4hc::FusedArgs a{n, d, (int)dtype, p->sinkhorn_iters, T, p->rms_eps, X, W_f16_next, bias_next,
                       layer_out, layer_in, coeffs, logits_opt, X_out, static_cast<float *>(workspace)};
    const hipError_t e = ds4hc::launch_post_pre(a, coeffs_prev, pp.one_pass, pp.pre.path, stream);
    return e == hipSuccess ? DS4HC_OK : hip_fail(e);
}

}  // namespace

extern "C" {

ds4hc_status ds4hc_post_pre(const ds4hc_params *p, int64_t T, ds4hc_dtype dtype, const void *X,
                            const float *coeffs_prev, const void *layer_out,
                            const uint16_t *W_f16_next, const float *bias_next, void *X_out,
                            void *layer_in, float *coeffs, float *logits_opt, void *workspace,
                            size_t workspace_bytes, hipStream_t stream) {
    return post_pre_impl(p, T, dtype, X, coeffs_prev, layer_out, W_f16_next, bias_next, X_out,
                         layer_in, coeffs, logits_opt, workspace, workspace_bytes, false, stream);
}

ds4hc_status ds4hc_post_pre_noalloc(const ds4hc_params *p, int64_t T, ds4hc_dtype dtype,
                                    const void *X, const float *coeffs_prev, const void *layer_out,
                                    const uint16_t *W_f16_next, const float *bias_next,
                                    void *X_out, void *layer_in, float *coeffs, float *logits_opt,
                                    hipStream_t stream) {
    return post_pre_impl(p, T, dtype, X, coeffs_prev, layer_out, W_f16_next, bias_next, X_out,
                         layer_in, coeffs, logits_opt, nullptr, 0, true, stream);
}

}  // extern "C"

namespace {

// Split-over-d partials: for large T the streamed 16-token kernel, else split-K
// chunks of the share (workspace) summed into [T][m+1]; FORCE_TILE takes the
// tile kernel's partials mode.
ds4hc_status make_partials_plan(const ds4hc_params *p, int64_t T, ds4hc_dtype dt, Plan *out) {
    const int n = p->n_hc, d = p->d, m = 2 * n + n * n;
    const uint32_t force = p->flags & FORCE_FLAGS;
    if (force == DS4HC_FLAG_FORCE_ROWRES) return DS4HC_ERR_UNSUPPORTED;
    const bool fits_tile = ds4hc::tile_steps(d, dt) <= ds4hc::tile_max_steps();
    Plan pl{ds4hc::PATH_SPLITK, 0, 0};
    if (force == DS4HC_FLAG_FORCE_TILE) {
        if (!fits_tile) return DS4HC_ERR_UNSUPPORTED;
        pl.path = ds4hc::PATH_TILE;
    } else if (force == 0 && T > SPLITK_MAX_T && (uint64_t)n * d <= STREAM_MAX_K) {
        if ((uint64_t)(T + 15) / 16 * 512u > MAX_WORK_ITEMS) return DS4HC_ERR_UNSUPPORTED;
        pl.path = ds4hc::PATH_STREAM;
    } else {
        pl.P = ds4hc::colchunk_chunks(d, dt);
        const uint64_t tg = (uint64_t)(T + 3) / 4;
        if (tg * 64u > MAX_WORK_ITEMS || pl.P > 0xFFFF || (uint64_t)T * 64u > MAX_WORK_ITEMS)
            return DS4HC_ERR_UNSUPPORTED;
        pl.ws_bytes = (uint64_t)pl.P * (uint64_t)T * (uint64_t)(m + 1) * sizeof(float);
    }
    *out = pl;
    return DS4HC_OK;
}

}  // namespace

extern "C" {

ds4hc_status ds4hc_partials(const ds4hc_params *p, int64_t T, ds4hc_dtype dtype, const void *X_share,
                            const uint16_t *W_share, float *partials, void *workspace,
                            size_t workspace_bytes, hipStream_t stream) {
    ds4hc_status st = check_params(p, T, dtype);
    if (st != DS4HC_OK || T == 0) return st;
    if (!X_share || !W_share || !partials) return DS4HC_ERR_INVALID_ARG;
    if (!aligned(X_share, 16) || !aligned(W_share, 16) || !aligned(partials, 4) ||
        (workspace && !aligned(workspace, 4)))
        return DS4HC_ERR_INVALID_ARG;
    Plan pl;
    st = make_partials_plan(p, T, dtype, &pl);
    if (st != DS4HC_OK) return st;
    if (pl.ws_bytes > 0 && (!workspace || workspace_bytes < pl.ws_bytes)) return DS4HC_ERR_INVALID_ARG;
    const int n = p->n_hc, d = p->d, m = 2 * n + n * n;
    const uint64_t sb = (uint64_t)state_bytes(dtype), K = (uint64_t)n * d, uT = (uint64_t)T;
    const Range rX{X_share, uT * K * sb}, rW{W_share, (uint64_t)m * K * 2};
    const Range rP{partials, uT * (m + 1) * 4}, rws{pl.ws_bytes ? workspace : nullptr, pl.ws_bytes};
    if (overlap(rP, rX) || overlap(rP, rW) || overlap(rP, rws) || overlap(rws, rX) || overlap(rws, rW))
        return DS4HC_ERR_INVALID_ARG;
    ds4hc::FusedArgs a{n, d, (int)dtype, p->sinkhorn_iters, T, p->rms_eps, X_share, W_share, nullptr,
                       nullptr, nullptr, nullptr, partials, nullptr, static_cast<float *>(workspace)};
    const hipError_t e = ds4hc::launch_partials(a, pl.path, stream);
    return e == hipSuccess ? DS4HC_OK : hip_fail(e);
}

size_t ds4hc_partials_workspace_bytes(const ds4hc_params *p, int64_t T, ds4hc_dtype dtype) {
    if (check_params(p, T, dtype) != DS4HC_OK) return 0;
    Plan pl;
    if (make_partials_plan(p, T, dtype, &pl) != DS4HC_OK) return 0;
    return (size_t)pl.ws_bytes;
}

ds4hc_status ds4hc_combine(const ds4hc_params *p, int32_t d_total, int64_t T, ds4hc_dtype dtype,
                           int32_t G, const float *partials, const float *bias, const void *X_share,
                           const void *layer_out_share, void *layer_in_share, float *coeffs_opt,
                           void *X_out_share, hipStream_t stream) {
    ds4hc_status st = check_params(p, T, dtype);
    if (st != DS4HC_OK) return st;
    if (d_total < p->d || d_total % 8 != 0 || G < 1 || G > 0xFFFF) return DS4HC_ERR_INVALID_ARG;
    if (T == 0) return DS4HC_OK;
    if (!partials || !bias || !X_share || !layer_out_share || !layer_in_share || !X_out_share)
        return DS4HC_ERR_INVALID_ARG;
    if (!aligned(X_share, 16) || !aligned(layer_out_share, 16) || !aligned(layer_in_share, 16) ||
        !aligned(X_out_share, 16) || !aligned(partials, 4) || !aligned(bias, 4) ||
        (coeffs_opt && !aligned(coeffs_opt, 4)))
        return DS4HC_ERR_INVALID_ARG;
    const int n = p->n_hc, d = p->d, m = 2 * n + n * n;
    const uint64_t sb = (uint64_t)state_bytes(dtype), K = (uint64_t)n * d, uT = (uint64_t)T;
    const uint64_t cb = (uint64_t)(d + 64 * vec_elems(dtype) - 1) / (64 * vec_elems(dtype));
    if (cb > 0xFFFFu || uT * 64u > MAX_WORK_ITEMS) return DS4HC_ERR_UNSUPPORTED;
    const Range rP{partials, (uint64_t)G * uT * (m + 1) * 4}, rb{bias, (uint64_t)m * 4};
    const Range rX{X_share, uT * K * sb}, rlo{layer_out_share, uT * d * sb};
    const Range rli{layer_in_share, uT * d * sb}, rc{coeffs_opt, uT * m * 4}, rXo{X_out_share, uT * K * sb};
    const Range all[] = {rP, rb, rX, rlo, rli, rc, rXo};
    constexpr int FIRST_OUT = 4, N_ALL = 7;
    for (int a = FIRST_OUT; a < N_ALL; ++a) {
        for (int b = 0; b < N_ALL; ++b) {
            if (a == b) continue;
            const bool in_place = ((a == 6 && b == 2) || (a == 2 && b == 6)) && X_out_share == X_share;
            if (!in_place && overlap(all[a], all[b])) return DS4HC_ERR_INVALID_ARG;
        }
    }
    ds4hc::FusedArgs a{n, d, (int)dtype, p->sinkhorn_iters, T, p->rms_eps, X_share, nullptr, bias,
                       layer_out_share, layer_in_share, coeffs_opt, nullptr, X_out_share, nullptr};
    const hipError_t e = ds4hc::launch_combine(a, d_total, G, partials, stream);
    return e == hipSuccess ? DS4HC_OK : hip_fail(e);
}

size_t ds4hc_post_pre_workspace_bytes(const ds4hc_params *p, int64_t T, ds4hc_dtype dtype) {
    if (check_params(p, T, dtype) != DS4HC_OK) return 0;
    PostPrePlan pp;
    if (make_post_pre_plan(p, T, dtype, &pp) != DS4HC_OK) return 0;
    return (size_t)pp.ws_bytes;
}

ds4hc_status ds4hc_pre(const ds4hc_params *p, int64_t T, ds4hc_dtype dtype, const void *X,
                       const uint16_t *W_f16, const float *bias, void *layer_in, float *coeffs,
                       float *logits_opt, void *workspace, size_t workspace_bytes,
                       hipStream_t stream) {
    return run_hc(false, p, T, dtype, X, W_f16, bias, nullptr, layer_in, coeffs, logits_opt,
                  nullptr, workspace, workspace_bytes, stream);
}

ds4hc_status ds4hc_fused(const ds4hc_params *p, int64_t T, ds4hc_dtype dtype, const void *X,
                         const uint16_t *W_f16, const float *bias, const void *layer_out,
                         void *layer_in, float *coeffs_opt, void *X_out, void *workspace,
                         size_t workspace_bytes, hipStream_t stream) {
    return run_hc(true, p, T, dtype, X, W_f16, bias, layer_out, layer_in, coeffs_opt, nullptr,
                  X_out, workspace, workspace_bytes, stream);
}

ds4hc_status ds4hc_post(const ds4hc_params *p, int64_t T, ds4hc_dtype dtype, const void *X,
                        const float *coeffs, const void *layer_out, void *X_out,
                        hipStream_t stream) {
    ds4hc_status st = check_params(p, T, dtype);
    if (st != DS4HC_OK || T == 0) return st;
    if (!X || !coeffs || !layer_out || !X_out) return DS4HC_ERR_INVALID_ARG;
    if (!aligned(X, 16) || !aligned(layer_out, 16) || !aligned(X_out, 16) || !aligned(coeffs, 4))
        return DS4HC_ERR_INVALID_ARG;
    const int n = p->n_hc, d = p->d, m = 2 * n + n * n;
    const uint64_t sb = (uint64_t)state_bytes(dtype), uT = (uint64_t)T, K = (uint64_t)n * d;
    const Range rXo{X_out, uT * K * sb};
    if (X_out != X && overlap(rXo, Range{X, uT * K * sb})) return DS4HC_ERR_INVALID_ARG;
    if (overlap(rXo, Range{coeffs, uT * m * 4}) || overlap(rXo, Range{layer_out, uT * d * sb}))
        return DS4HC_ERR_INVALID_ARG;
    const uint64_t cb = (uint64_t)(d + 64 * vec_elems(dtype) - 1) / (64 * vec_elems(dtype));
    if (cb > 0xFFFFu || uT * 64u > MAX_WORK_ITEMS) return DS4HC_ERR_UNSUPPORTED;  // grid (T, cb)
    const hipError_t e = ds4hc::launch_post(n, (int)dtype, d, T, X, coeffs, layer_out, X_out, stream);
    return e == hipSuccess ? DS4HC_OK : hip_fail(e);
}

ds4hc_status ds4hc_sinkhorn(int64_t T, int32_t n_hc, int32_t iters, const float *logits_res,
                            float *H, hipStream_t stream) {
    if (T < 0 || n_hc < 1 || iters < 0) return DS4HC_ERR_INVALID_ARG;
    if (n_hc != 1 && n_hc != 2 && n_hc != 4) return DS4HC_ERR_UNSUPPORTED;
    if (iters > MAX_ITERS || T > MAX_T) return DS4HC_ERR_UNSUPPORTED;
    if (T == 0) return DS4HC_OK;
    if (!logits_res || !H || !aligned(logits_res, 4) || !aligned(H, 4)) return DS4HC_ERR_INVALID_ARG;
    const uint64_t bytes = (uint64_t)T * n_hc * n_hc * 4;
    if (overlap(Range{logits_res, bytes}, Range{H, bytes})) return DS4HC_ERR_INVALID_ARG;
    const hipError_t e = ds4hc::launch_sinkhorn(n_hc, iters, T, logits_res, H, stream);
    return e == hipSuccess ? DS4HC_OK : hip_fail(e);
}

size_t ds4hc_workspace_bytes(const ds4hc_params *p, int64_t T, ds4hc_dtype dtype) {
    if (check_params(p, T, dtype) != DS4HC_OK) return 0;
    Plan pl;
    if (make_plan(p, T, dtype, &pl) != DS4HC_OK) return 0;
    return (size_t)pl.ws_bytes;
}

const char *ds4hc_status_string(ds4hc_status s) {
    switch (s) {
    case DS4HC_OK: return "DS4HC_OK";
    case DS4HC_ERR_INVALID_ARG: return "DS4HC_ERR_INVALID_ARG";
    case DS4HC_ERR_UNSUPPORTED: return "DS4HC_ERR_UNSUPPORTED";
    case DS4HC_ERR_HIP: return "DS4HC_ERR_HIP";
    }
    return "DS4HC_UNKNOWN_STATUS";
}

const char *ds4hc_last_hip_error(void) { return g_last_hip_error; }

int ds4hc_abi_version(void) { return DS4HC_ABI_VERSION; }

}  // extern "C"
