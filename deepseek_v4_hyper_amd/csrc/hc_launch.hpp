// hc_launch.hpp -- internal interface between the C ABI (ds4hc_api.cpp) and
// the kernels (hc_kernels.hip). Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>
#include <utility>

namespace ds4hc {

// Arguments of one HC-pre / fused call after host-side validation.
struct FusedArgs {
    int n, d, dt, iters;
    int64_t T;
    float eps;
    const void *X;
    const uint16_t *W;
    const float *bias;
    const void *layer_out;  // fused only
    void *layer_in;
    float *coeffs;          // may be null
    float *logits;          // may be null
    void *X_out;            // fused only
    float *ws;              // split-K workspace
};

// Kernel paths for HC-pre / fused.
enum : int { PATH_ROWRES = 0, PATH_TILE = 1, PATH_SPLITK = 2, PATH_STREAM = 3 };  // STREAM: partials only

int rowres_chunks(int d, int dt);
int rowres_max_chunks(int n, int dt);
int tile_steps(int d, int dt);
int tile_max_steps();
hipError_t launch_hc(const FusedArgs &a, bool fused, int path, hipStream_t s);
hipError_t launch_post(int n, int dt, int d, int64_t T, const void *X, const float *coeffs,
                       const void *layer_out, void *X_out, hipStream_t s);
hipError_t launch_sinkhorn(int n, int iters, int64_t T, const float *Z, float *H, hipStream_t s);
// post(l) + pre(l+1): one pass (split-K chunks over columns, then the combining
// kernel) or post then pre on `path`. a.X = X_l, a.layer_out = layer_out_l,
// a.X_out = X_{l+1}, a.W/bias/layer_in/coeffs/logits = site l+1.
// Split over d: a.X / a.W = one column share (a.d = its width), partial sums to
// a.logits as [T][m + 1]; path PATH_TILE or PATH_SPLITK (workspace a.ws).
hipError_t launch_partials(const FusedArgs &a, int path, hipStream_t s);
// Combine G shares' partials [G][T][m + 1] in share order, then gates, Sinkhorn
// and pass 2 on the share a.X (width a.d) of a row n * d_total long.
hipError_t launch_combine(const FusedArgs &a, int d_total, int G, const float *partials,
                          hipStream_t s);
// Split-K column chunks (HC-pre, the one-pass chain step, the split over d at
// small T): lanes per chunk (16 or 32) and the number of chunks.
int colchunk_lanes(int d, int dt);
int colchunk_chunks(int d, int dt);
// Split-K of HC-pre / fused for T >= SPLITK_STREAM_MIN_T takes the streamed
// 16-token partials over column chunks of stream_chunk_cols(T, K) columns of
// the flattened row (K = n * d): stream_chunks(T, K) of them.
// Rows up to STREAM_K_MAX columns keep the streamed kernel's 32-bit offsets
// (16 token rows of float32) in range.
constexpr int64_t SPLITK_STREAM_MIN_T = 32;
constexpr int64_t STREAM_K_MAX = int64_t(1) << 24;
inline bool splitk_streams(int64_t T, int64_t K) { return T >= SPLITK_STREAM_MIN_T && K <= STREAM_K_MAX; }
int stream_chunk_cols(int64_t T, int K);
int stream_chunks(int64_t T, int K);
// Bytes of the device-resident scratch array behind ds4hc_post_pre_noalloc,
// and its address on the current device (looked up once per device).
constexpr size_t NOALLOC_SCRATCH_BYTES = size_t(2) << 20;
hipError_t noalloc_scratch(void **ptr);
hipError_t launch_post_pre(const FusedArgs &a, const float *coeffs_prev, bool one_pass, int path,
                           hipStream_t s);

// hipLaunchKernel with the kernel's own parameter types, so the launch status
// comes back directly instead of through the thread's sticky last-error slot.
template <typename... KArgs, std::size_t... I>
hipError_t launch_tuple(void (*kern)(KArgs...), dim3 grid, dim3 block, hipStream_t s,
                        std::tuple<KArgs...> &tup, std::index_sequence<I...>) {
    void *argv[sizeof...(KArgs) + 1] = {(void *)&std::get<I>(tup)..., nullptr};
    return hipLaunchKernel(reinterpret_cast<const void *>(kern), grid, block, argv, 0, s);
}

template <typename... KArgs, typename... Args>
hipError_t launch_kernel(void (*kern)(KArgs...), dim3 grid, dim3 block, hipStream_t s,
                         Args... args) {
    static_assert(sizeof...(KArgs) == sizeof...(Args), "kernel argument count");
    std::tuple<KArgs...> tup(static_cast<KArgs>(args)...);
    return launch_tuple(kern, grid, block, s, tup, std::index_sequence_for<KArgs...>{});
}

}  // namespace ds4hc
