// hc_kernels.hip -- HIP kernels of the DeepSeek-V4 hyper-connection op for
// MI355X (gfx950) and their host-side launchers.
//
// Two paths compute the same op (see ds4hc.h for its definition):
//
//  * row-resident (large T): one 256-thread workgroup per token. The token's
//    n*d state is loaded once from HBM into registers, the RMS statistic and
//    the m = 2n + n*n fn dot products are accumulated from it, reduced in a
//    fixed order, the gates and the register-resident Sinkhorn run in one
//    wavefront, and the pre-mix and post update are computed from the same
//    registers. X is read once and X' written once: the HBM-bound minimum.
//
//  * split-K (small T, decode and speculative verify): the fn weight (m*K
//    float16, 768 KiB at d = 4096) dominates the bytes, so K is cut into
//    chunks and many workgroups each read one chunk of W for all tokens,
//    writing fixed-order partial sums to a caller workspace. A second kernel
//    combines them in chunk order, runs gates + Sinkhorn, and does the
//    pre-mix / post update column-parallel. The pages' decode runs these HC
//    sites 86 times per token (lucebox-hub PR #494, Sinkhorn comment), so
//    this path is about latency, not bandwidth.
//
// Arithmetic: float32 everywhere, f16 weights widened exactly, one RNE
// rounding at each store of a bf16 state. No floating-point atomics.
#include "hc_device.hpp"
#include "hc_launch.hpp"

#include <tuple>
#include <utility>

namespace ds4hc {

constexpr int ROWRES_THREADS = 256;
constexpr int ROWRES_WAVES = ROWRES_THREADS / 64;
constexpr int SPLITK_TOKENS = 4;   // tokens per partials workgroup

enum : int { MODE_PRE = 0, MODE_FUSED = 1 };

// Largest number of column chunks (256*V columns each) a row-resident
// instance keeps in registers without spilling to scratch on gfx950.
constexpr int rowres_cap(int n, int dt) { return n == 4 ? (dt == DT_F32 ? 7 : 5) : 8; }

// ---------------------------------------------------------------------------
// Row-resident kernel: one workgroup per token.
// Thread `tid` owns, for every stream i and column chunk q < CQ, the V
// consecutive columns c0 = (q*256 + tid)*V .. c0+V-1 (valid while c0 < d).
// ---------------------------------------------------------------------------
template <int N, int DT, int CQ, int MODE>
__global__ __launch_bounds__(ROWRES_THREADS) void hc_rowres_kernel(
    int d, float eps, int iters, const void *__restrict__ X, const uint16_t *__restrict__ W,
    const float *__restrict__ bias, const void *__restrict__ layer_out, void *__restrict__ layer_in,
    float *__restrict__ coeffs, float *__restrict__ logits, void *X_out) {
    constexpr int V = StateVec<DT>::V;
    constexpr int M = n_logits(N);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const size_t t = blockIdx.x;
    const size_t K = (size_t)N * d;
    const size_t xrow = t * K;

    __shared__ float red[ROWRES_WAVES][M + 1];
    __shared__ float tot[M + 1];
    __shared__ float cf[M];

    // ---- load the row (and layer_out) once ----
    StateVec<DT> xv[N][CQ];
    StateVec<DT> lov[CQ];
#pragma unroll
    for (int q = 0; q < CQ; ++q) {
        const int c0 = (q * ROWRES_THREADS + tid) * V;
        const bool ok = c0 < d;
#pragma unroll
        for (int i = 0; i < N; ++i)
            xv[i][q] = ok ? load_vec<DT>(X, xrow + (size_t)i * d + c0) : zero_vec<DT>();
        if constexpr (MODE == MODE_FUSED)
            lov[q] = ok ? load_vec<DT>(layer_out, t * d + c0) : zero_vec<DT>();
    }

    // ---- sum of squares and the m fn dot products ----
    float acc[M];
#pragma unroll
    for (int j = 0; j < M; ++j) acc[j] = 0.f;
    float ss = 0.f;
#pragma unroll
    for (int q = 0; q < CQ; ++q) {
        const int c0 = (q * ROWRES_THREADS + tid) * V;
        if (c0 < d) {
#pragma unroll
            for (int i = 0; i < N; ++i) {
                float x[V];
#pragma unroll
                for (int e = 0; e < V; ++e) {
                    x[e] = vec_get<DT>(xv[i][q], e);
                    ss = fmaf(x[e], x[e], ss);
                }
                const uint16_t *wk = W + (size_t)i * d + c0;
#pragma unroll
                for (int j = 0; j < M; ++j) {
                    const HalfVec<V> w = load_half_vec<V>(wk + (size_t)j * K);
#pragma unroll
                    for (int e = 0; e < V; ++e) acc[j] = fmaf(half_get<V>(w, e), x[e], acc[j]);
                }
            }
        }
    }

    // ---- fixed-order block reduction of the M+1 partials ----
#pragma unroll
    for (int j = 0; j < M; ++j) acc[j] = wave_sum(acc[j]);
    ss = wave_sum(ss);
    if (lane == 0) {
#pragma unroll
        for (int j = 0; j < M; ++j) red[wave][j] = acc[j];
        red[wave][M] = ss;
    }
    __syncthreads();
    if (tid <= M) {
        float s = red[0][tid];
#pragma unroll
        for (int w = 1; w < ROWRES_WAVES; ++w) s += red[w][tid];
        tot[tid] = s;
    }
    __syncthreads();

    // ---- logits, gates, Sinkhorn (wave 0) ----
    if (wave == 0) {
        const float r = sqrtf(tot[M] / (float)K + eps);
        float z = 0.f;
        if (lane < M) {
            z = tot[lane] / r + bias[lane];
            if (logits) logits[t * M + lane] = z;
            if (lane < 2 * N) {
                const float g = logistic(z);
                cf[lane] = g;
                if (coeffs) coeffs[t * M + lane] = g;
            }
        }
        // Residual logits z_{2N + l} moved to lane l of every N*N group.
        const int src = 2 * N + (lane % (N * N));
        const float zr = __shfl(z, src, 64);
        const float h = sinkhorn_lane<N>(zr, iters);
        if (lane < N * N) {
            cf[2 * N + lane] = h;
            if (coeffs) coeffs[t * M + 2 * N + lane] = h;
        }
    }
    __syncthreads();

    // ---- pre-mix and post update from the registers ----
    float pre[N], post[N], H[N][N];
#pragma unroll
    for (int i = 0; i < N; ++i) {
        pre[i] = cf[i];
        post[i] = cf[N + i];
#pragma unroll
        for (int j = 0; j < N; ++j) H[i][j] = cf[2 * N + i * N + j];
    }
#pragma unroll
    for (int q = 0; q < CQ; ++q) {
        const int c0 = (q * ROWRES_THREADS + tid) * V;
        if (c0 >= d) continue;
        float x[N][V];
#pragma unroll
        for (int i = 0; i < N; ++i)
#pragma unroll
            for (int e = 0; e < V; ++e) x[i][e] = vec_get<DT>(xv[i][q], e);
        float li[V];
#pragma unroll
        for (int e = 0; e < V; ++e) {
            float s = pre[0] * x[0][e];
#pragma unroll
            for (int i = 1; i < N; ++i) s = fmaf(pre[i], x[i][e], s);
            li[e] = s;
        }
        store_vec<DT>(layer_in, t * d + c0, li);
        if constexpr (MODE == MODE_FUSED) {
            float lo[V];
#pragma unroll
            for (int e = 0; e < V; ++e) lo[e] = vec_get<DT>(lov[q], e);
#pragma unroll
            for (int i = 0; i < N; ++i) {
                float o[V];
#pragma unroll
                for (int e = 0; e < V; ++e) {
                    float s = H[i][0] * x[0][e];
#pragma unroll
                    for (int j = 1; j < N; ++j) s = fmaf(H[i][j], x[j][e], s);
                    o[e] = fmaf(post[i], lo[e], s);
                }
                store_vec<DT>(X_out, xrow + (size_t)i * d + c0, o);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Split-K partials: grid (ceil(T / SPLITK_TOKENS), P chunks), one wavefront.
// Chunk p covers flattened columns [p*64*V, (p+1)*64*V) of K; lane l owns V
// consecutive columns. Writes ws[p][t][0..M) = partial dots, ws[p][t][M] =
// partial sum of squares.
// ---------------------------------------------------------------------------
template <int N, int DT>
__global__ __launch_bounds__(64) void hc_partials_kernel(int d, int T, const void *__restrict__ X,
                                                         const uint16_t *__restrict__ W,
                                                         float *__restrict__ ws) {
    constexpr int V = StateVec<DT>::V;
    constexpr int M = n_logits(N);
    const int lane = threadIdx.x;
    const size_t K = (size_t)N * d;
    const size_t k0 = ((size_t)blockIdx.y * 64 + lane) * V;
    const bool ok = k0 < K;
    const int tbase = blockIdx.x * SPLITK_TOKENS;

    HalfVec<V> w[M];
#pragma unroll
    for (int j = 0; j < M; ++j) {
        if (ok)
            w[j] = load_half_vec<V>(W + (size_t)j * K + k0);
        else
            w[j].raw = {};
    }

#pragma unroll
    for (int tt = 0; tt < SPLITK_TOKENS; ++tt) {
        const int t = tbase + tt;
        if (t >= T) break;  // uniform across the wavefront
        const StateVec<DT> xv = ok ? load_vec<DT>(X, (size_t)t * K + k0) : zero_vec<DT>();
        float acc[M + 1];
#pragma unroll
        for (int j = 0; j <= M; ++j) acc[j] = 0.f;
#pragma unroll
        for (int e = 0; e < V; ++e) {
            const float x = vec_get<DT>(xv, e);
            acc[M] = fmaf(x, x, acc[M]);
#pragma unroll
            for (int j = 0; j < M; ++j) acc[j] = fmaf(half_get<V>(w[j], e), x, acc[j]);
        }
#pragma unroll
        for (int j = 0; j <= M; ++j) acc[j] = wave_sum(acc[j]);
        if (lane <= M) {
            float v = acc[0];
#pragma unroll
            for (int j = 1; j <= M; ++j)
                if (lane == j) v = acc[j];
            ws[((size_t)blockIdx.y * T + t) * (M + 1) + lane] = v;
        }
    }
}

// ---------------------------------------------------------------------------
// Split-K finish: grid (T, ceil(d / (64*V))), one wavefront. Combines the P
// partials of token t in chunk order, computes logits, gates and Sinkhorn,
// then the pre-mix (and post update) of 64*V columns.
// ---------------------------------------------------------------------------
template <int N, int DT, int MODE>
__global__ __launch_bounds__(64) void hc_finish_kernel(
    int d, int T, int P, float eps, int iters, const void *__restrict__ X,
    const float *__restrict__ bias, const float *__restrict__ ws, const void *__restrict__ layer_out,
    void *__restrict__ layer_in, float *__restrict__ coeffs, float *__restrict__ logits, void *X_out) {
    constexpr int V = StateVec<DT>::V;
    constexpr int M = n_logits(N);
    const int lane = threadIdx.x;
    const size_t t = blockIdx.x;
    const size_t K = (size_t)N * d;
    __shared__ float cf[M];

    float tot = 0.f;
    if (lane <= M) {
        const float *p = ws + t * (M + 1) + lane;
        const size_t stride = (size_t)T * (M + 1);
        for (int c = 0; c < P; ++c) tot += p[(size_t)c * stride];
    }
    const float ssum = __shfl(tot, M, 64);
    const float r = sqrtf(ssum / (float)K + eps);
    float z = 0.f;
    if (lane < M) z = tot / r + bias[lane];
    const bool writer = blockIdx.y == 0;
    if (lane < 2 * N) {
        const float g = logistic(z);
        cf[lane] = g;
        if (writer && coeffs) coeffs[t * M + lane] = g;
    }
    if (writer && logits && lane < M) logits[t * M + lane] = z;
    const float zr = __shfl(z, 2 * N + (lane % (N * N)), 64);
    const float h = sinkhorn_lane<N>(zr, iters);
    if (lane < N * N) {
        cf[2 * N + lane] = h;
        if (writer && coeffs) coeffs[t * M + 2 * N + lane] = h;
    }
    __syncthreads();

    const int c0 = (blockIdx.y * 64 + lane) * V;
    if (c0 >= d) return;
    float x[N][V];
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const StateVec<DT> v = load_vec<DT>(X, t * K + (size_t)i * d + c0);
#pragma unroll
        for (int e = 0; e < V; ++e) x[i][e] = vec_get<DT>(v, e);
    }
    float li[V];
#pragma unroll
    for (int e = 0; e < V; ++e) {
        float s = cf[0] * x[0][e];
#pragma unroll
        for (int i = 1; i < N; ++i) s = fmaf(cf[i], x[i][e], s);
        li[e] = s;
    }
    store_vec<DT>(layer_in, t * d + c0, li);
    if constexpr (MODE == MODE_FUSED) {
        const StateVec<DT> lv = load_vec<DT>(layer_out, t * d + c0);
#pragma unroll
        for (int i = 0; i < N; ++i) {
            float o[V];
#pragma unroll
            for (int e = 0; e < V; ++e) {
                float s = cf[2 * N + i * N] * x[0][e];
#pragma unroll
                for (int j = 1; j < N; ++j) s = fmaf(cf[2 * N + i * N + j], x[j][e], s);
                o[e] = fmaf(cf[N + i], vec_get<DT>(lv, e), s);
            }
            store_vec<DT>(X_out, t * K + (size_t)i * d + c0, o);
        }
    }
}

// ---------------------------------------------------------------------------
// Post update alone: grid (T, ceil(d / (64*V))), one wavefront.
// ---------------------------------------------------------------------------
template <int N, int DT>
__global__ __launch_bounds__(64) void hc_post_kernel(int d, const void *X,
                                                     const float *__restrict__ coeffs,
                                                     const void *__restrict__ layer_out, void *X_out) {
    constexpr int V = StateVec<DT>::V;
    constexpr int M = n_logits(N);
    const int lane = threadIdx.x;
    const size_t t = blockIdx.x;
    const size_t K = (size_t)N * d;
    __shared__ float cf[M];
    if (lane < M) cf[lane] = coeffs[t * M + lane];
    __syncthreads();
    const int c0 = (blockIdx.y * 64 + lane) * V;
    if (c0 >= d) return;
    float x[N][V];
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const StateVec<DT> v = load_vec<DT>(X, t * K + (size_t)i * d + c0);
#pragma unroll
        for (int e = 0; e < V; ++e) x[i][e] = vec_get<DT>(v, e);
    }
    const StateVec<DT> lv = load_vec<DT>(layer_out, t * d + c0);
#pragma unroll
    for (int i = 0; i < N; ++i) {
        float o[V];
#pragma unroll
        for (int e = 0; e < V; ++e) {
            float s = cf[2 * N + i * N] * x[0][e];
#pragma unroll
            for (int j = 1; j < N; ++j) s = fmaf(cf[2 * N + i * N + j], x[j][e], s);
            o[e] = fmaf(cf[N + i], vec_get<DT>(lv, e), s);
        }
        store_vec<DT>(X_out, t * K + (size_t)i * d + c0, o);
    }
}

// ---------------------------------------------------------------------------
// Sinkhorn alone: 64 / (N*N) matrices per wavefront.
// ---------------------------------------------------------------------------
template <int N>
__global__ __launch_bounds__(64) void hc_sinkhorn_kernel(int T, int iters,
                                                         const float *__restrict__ Z,
                                                         float *__restrict__ H) {
    constexpr int NN = N * N;
    const int lane = threadIdx.x;
    const size_t t = (size_t)blockIdx.x * (64 / NN) + lane / NN;
    const int e = lane % NN;
    const bool ok = t < (size_t)T;
    const float z = ok ? Z[t * NN + e] : 0.f;
    const float h = sinkhorn_lane<N>(z, iters);
    if (ok) H[t * NN + e] = h;
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
template <int N, int DT, int MODE>
static hipError_t launch_rowres_n(int cq, const FusedArgs &a, hipStream_t s) {
    const dim3 grid((unsigned)a.T), block(ROWRES_THREADS);
    constexpr int CAP = rowres_cap(N, DT);
#define DS4HC_ROWRES_CASE(CQ)                                                                    \
    case CQ:                                                                                     \
        if constexpr (CQ <= CAP)                                                                 \
            return launch_kernel(hc_rowres_kernel<N, DT, CQ, MODE>, grid, block, s, a.d, a.eps,  \
                                 a.iters, a.X, a.W, a.bias, a.layer_out, a.layer_in, a.coeffs,   \
                                 a.logits, a.X_out);                                             \
        else                                                                                     \
            return hipErrorInvalidValue;
    switch (cq) {
        DS4HC_ROWRES_CASE(1)
        DS4HC_ROWRES_CASE(2)
        DS4HC_ROWRES_CASE(3)
        DS4HC_ROWRES_CASE(4)
        DS4HC_ROWRES_CASE(5)
        DS4HC_ROWRES_CASE(6)
        DS4HC_ROWRES_CASE(7)
        DS4HC_ROWRES_CASE(8)
    default:
        return hipErrorInvalidValue;
    }
#undef DS4HC_ROWRES_CASE
}

template <int N, int DT, int MODE>
static hipError_t launch_splitk_n(const FusedArgs &a, hipStream_t s) {
    constexpr int V = StateVec<DT>::V;
    const int P = splitk_chunks(N, a.d, DT);
    const dim3 g1((unsigned)((a.T + SPLITK_TOKENS - 1) / SPLITK_TOKENS), (unsigned)P);
    hipError_t e = launch_kernel(hc_partials_kernel<N, DT>, g1, dim3(64), s, a.d, (int)a.T, a.X,
                                 a.W, a.ws);
    if (e != hipSuccess) return e;
    const dim3 g2((unsigned)a.T, (unsigned)((a.d + 64 * V - 1) / (64 * V)));
    return launch_kernel(hc_finish_kernel<N, DT, MODE>, g2, dim3(64), s, a.d, (int)a.T, P, a.eps,
                         a.iters, a.X, a.bias, (const float *)a.ws, a.layer_out, a.layer_in,
                         a.coeffs, a.logits, a.X_out);
}

template <int N>
static hipError_t dispatch_dt(int dt, bool fused, bool rowres, int cq, const FusedArgs &a,
                              hipStream_t s) {
    if (dt == DT_F32) {
        if (rowres)
            return fused ? launch_rowres_n<N, DT_F32, MODE_FUSED>(cq, a, s)
                         : launch_rowres_n<N, DT_F32, MODE_PRE>(cq, a, s);
        return fused ? launch_splitk_n<N, DT_F32, MODE_FUSED>(a, s)
                     : launch_splitk_n<N, DT_F32, MODE_PRE>(a, s);
    }
    if (rowres)
        return fused ? launch_rowres_n<N, DT_BF16, MODE_FUSED>(cq, a, s)
                     : launch_rowres_n<N, DT_BF16, MODE_PRE>(cq, a, s);
    return fused ? launch_splitk_n<N, DT_BF16, MODE_FUSED>(a, s)
                 : launch_splitk_n<N, DT_BF16, MODE_PRE>(a, s);
}

int rowres_chunks(int d, int dt) {
    const int V = dt == DT_F32 ? 4 : 8;
    return (d + ROWRES_THREADS * V - 1) / (ROWRES_THREADS * V);
}

int rowres_max_chunks(int n, int dt) { return rowres_cap(n, dt); }

int splitk_chunks(int n, int d, int dt) {
    const int V = dt == DT_F32 ? 4 : 8;
    const long K = (long)n * d;
    return (int)((K + 64 * V - 1) / (64 * V));
}

hipError_t launch_hc(const FusedArgs &a, bool fused, bool rowres, hipStream_t s) {
    const int cq = rowres_chunks(a.d, a.dt);
    switch (a.n) {
    case 1: return dispatch_dt<1>(a.dt, fused, rowres, cq, a, s);
    case 2: return dispatch_dt<2>(a.dt, fused, rowres, cq, a, s);
    case 4: return dispatch_dt<4>(a.dt, fused, rowres, cq, a, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_post(int n, int dt, int d, int64_t T, const void *X, const float *coeffs,
                       const void *layer_out, void *X_out, hipStream_t s) {
    const int V = dt == DT_F32 ? 4 : 8;
    const dim3 grid((unsigned)T, (unsigned)((d + 64 * V - 1) / (64 * V)));
#define DS4HC_POST(NN, DD) \
    launch_kernel(hc_post_kernel<NN, DD>, grid, dim3(64), s, d, X, coeffs, layer_out, X_out)
    if (dt == DT_F32) {
        switch (n) {
        case 1: return DS4HC_POST(1, DT_F32);
        case 2: return DS4HC_POST(2, DT_F32);
        case 4: return DS4HC_POST(4, DT_F32);
        }
    } else {
        switch (n) {
        case 1: return DS4HC_POST(1, DT_BF16);
        case 2: return DS4HC_POST(2, DT_BF16);
        case 4: return DS4HC_POST(4, DT_BF16);
        }
    }
#undef DS4HC_POST
    return hipErrorInvalidValue;
}

hipError_t launch_sinkhorn(int n, int iters, int64_t T, const float *Z, float *H, hipStream_t s) {
    const int per = 64 / (n * n);
    const dim3 grid((unsigned)((T + per - 1) / per));
    switch (n) {
    case 1: return launch_kernel(hc_sinkhorn_kernel<1>, grid, dim3(64), s, (int)T, iters, Z, H);
    case 2: return launch_kernel(hc_sinkhorn_kernel<2>, grid, dim3(64), s, (int)T, iters, Z, H);
    case 4: return launch_kernel(hc_sinkhorn_kernel<4>, grid, dim3(64), s, (int)T, iters, Z, H);
    }
    return hipErrorInvalidValue;
}

}  // namespace ds4hc
