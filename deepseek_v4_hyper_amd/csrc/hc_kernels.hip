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
// MFMA tile kernel: two tokens per 256-thread workgroup, rows kept in
// registers, the fn matvec on v_mfma_f32_4x4x4_16b_f16.
//
// The fn projection z = W . x~ (x~ = x / r) is a [24 x K] . [K x 2] product
// per workgroup. One 4x4x4_16b instruction is 16 independent 4x4x4 products
// (block b = lane / 4): A_b = 4 rows of W x 4 consecutive k, B_b = 4 k x 4
// columns, where the columns are (token 0 hi, token 0 lo, token 1 hi,
// token 1 lo). x~ is split exactly into f16 hi + lo (hi = f16(x~),
// lo = f16(x~ - hi)), so hi + lo carries x~ to ~2^-23 relative and the
// products are exact; accumulation is fp32. |x~| <= sqrt(K), so f16 cannot
// overflow. Lane 4b + 2t + p holds V state elements of token t (p = 0 the
// first, p = 1 the second V of block b's 2V columns); a quad DPP swap hands
// each lane the hi or lo half its column needs from its partner.
//
// Column step j of wave w covers STEP = 32*V columns of every stream:
// columns (w + 4j)*STEP + b*2V + p*V .. +V-1, so every lane holds all n
// streams of its columns and the post update needs no data exchange.
// ---------------------------------------------------------------------------
// Opaque register barrier: the compiler must assume the packed vector changed,
// so it re-derives float32 values from it instead of keeping unpacked copies of
// a whole register-resident row live across phases (which spills to scratch).
template <int DT>
__device__ __forceinline__ void launder(StateVec<DT> &v) {
    asm volatile("" : "+v"(v.raw.x), "+v"(v.raw.y), "+v"(v.raw.z), "+v"(v.raw.w));
}

// Word 3 of a gfx9-family buffer resource descriptor (32-bit data format,
// raw addressing); loads at or past num_records return zero.
constexpr int BUFFER_RSRC_WORD3 = 0x00020000;
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef unsigned int uint2_t __attribute__((ext_vector_type(2)));

constexpr int TILE_TOKENS = 2;
constexpr int TILE_THREADS = 256;
constexpr int TILE_WAVES = TILE_THREADS / 64;

// Opaque register barrier on a 4 x f16 value: later uses see these exact bits.
__device__ __forceinline__ void pin_half4(half4_t &v) {
    uint2_t u = __builtin_bit_cast(uint2_t, v);
    asm volatile("" : "+v"(u.x), "+v"(u.y));
    v = __builtin_bit_cast(half4_t, u);
}

// Exchange a 4 x f16 value with the partner lane (lane ^ 1) of the quad.
__device__ __forceinline__ half4_t quad_swap(half4_t v) {
    uint2_t u = __builtin_bit_cast(uint2_t, v);
    u.x = (unsigned)__builtin_amdgcn_mov_dpp((int)u.x, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
    u.y = (unsigned)__builtin_amdgcn_mov_dpp((int)u.y, 0xB1, 0xF, 0xF, false);
    return __builtin_bit_cast(half4_t, u);
}

// Sub-block sb (4 consecutive float16) of a packed W slice, as an MFMA operand.
template <int V>
__device__ __forceinline__ half4_t half_sub4(const HalfVec<V> &h, int sb) {
    uint2_t u;
    if constexpr (V == 4) {
        u.x = h.raw.x;
        u.y = h.raw.y;
    } else {
        u.x = sb == 0 ? h.raw.x : h.raw.z;
        u.y = sb == 0 ? h.raw.y : h.raw.w;
    }
    return __builtin_bit_cast(half4_t, u);
}

template <int N, int DT, int CS, int MODE>
__global__ __launch_bounds__(TILE_THREADS, 2) void hc_tile_kernel(
    int d, int T, float eps, int iters, const void *__restrict__ X, const uint16_t *__restrict__ W,
    const float *__restrict__ bias, const void *__restrict__ layer_out, void *__restrict__ layer_in,
    float *__restrict__ coeffs, float *__restrict__ logits, void *X_out) {
    constexpr int V = StateVec<DT>::V;
    constexpr int M = n_logits(N);
    constexpr int G = (M + 3) / 4;  // groups of 4 W rows
    constexpr int SB = V / 4;       // 4-element sub-blocks per lane vector
    constexpr int STEP = 32 * V;    // columns per step
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // readfirstlane makes the wave index (and every offset built from it) a
    // scalar the compiler can put in the buffer loads' scalar offset field.
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int blk = lane >> 2;
    const int t = (lane >> 1) & 1;
    const int p = lane & 1;
    const int row4 = lane & 3;
    const size_t tok = (size_t)blockIdx.x * TILE_TOKENS + t;
    const bool tok_ok = tok < (size_t)T;
    const size_t K = (size_t)N * d;

    __shared__ float ssr[TILE_WAVES][TILE_TOKENS];
    __shared__ float zred[TILE_WAVES][4][G * 4];
    __shared__ float zs[TILE_TOKENS][M];
    __shared__ float cf[TILE_TOKENS][M];

    // ---- phase 1: the two rows into registers, sum of squares ----
    StateVec<DT> xv[N][CS];
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < CS; ++j) {
        const int c0 = (wave + TILE_WAVES * j) * STEP + blk * 2 * V + p * V;
        const bool ok = tok_ok && c0 < d;
#pragma unroll
        for (int i = 0; i < N; ++i)
            xv[i][j] = ok ? load_vec<DT>(X, tok * K + (size_t)i * d + c0) : zero_vec<DT>();
    }
#pragma unroll
    for (int j = 0; j < CS; ++j)
#pragma unroll
        for (int i = 0; i < N; ++i)
#pragma unroll
            for (int e = 0; e < V; ++e) {
                const float x = vec_get<DT>(xv[i][j], e);
                ss = fmaf(x, x, ss);
            }
    ss += __shfl_xor(ss, 1, 64);
    ss += __shfl_xor(ss, 4, 64);
    ss += __shfl_xor(ss, 8, 64);
    ss += __shfl_xor(ss, 16, 64);
    ss += __shfl_xor(ss, 32, 64);
    if (lane == 0 || lane == 2) ssr[wave][t] = ss;
    __syncthreads();
    float sst = ssr[0][t];
#pragma unroll
    for (int w = 1; w < TILE_WAVES; ++w) sst += ssr[w][t];
    const float inv_r = 1.0f / sqrtf(sst / (float)K + eps);

    // ---- phase 2: fn matvec on MFMA ----
    const __amdgpu_buffer_rsrc_t wrsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(W), (short)0, (int)((size_t)M * K * 2), BUFFER_RSRC_WORD3);
    // W row 4g + row4 of every group through one descriptor: a per-lane byte
    // offset plus a wave-uniform offset per (group, stream, step). Padding rows
    // (>= M, when M % 4 != 0) fall past the end of W and read as zero.
    const int w_voff = (int)((row4 * K + blk * 2 * V) * 2);
#pragma unroll
    for (int j = 0; j < CS; ++j)
#pragma unroll
        for (int i = 0; i < N; ++i) launder<DT>(xv[i][j]);
    float4_t acc[G];
#pragma unroll
    for (int g = 0; g < G; ++g) acc[g] = (float4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < CS; ++j) {
        const int cs = wave + TILE_WAVES * j;
        if (cs * STEP >= d) break;  // wave-uniform
        const int cb = cs * STEP + blk * 2 * V;  // first column of block b
        const bool e_ok = cb < d, o_ok = cb + V < d;
#pragma unroll
        for (int i = 0; i < N; ++i) {
            // A operands: W rows 4g + row4, columns cb .. cb + 2V - 1 of stream i
            HalfVec<V> we[G], wo[G];
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const int soff = (int)((4 * g * K + (size_t)i * d + (size_t)cs * STEP) * 2);
                if constexpr (V == 4) {
                    uint4 u = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(wrsrc, w_voff, soff, 0));
                    if (!e_ok) u = make_uint4(0u, 0u, 0u, 0u);
                    we[g].raw = make_uint2(u.x, u.y);
                    wo[g].raw = make_uint2(u.z, u.w);
                } else {
                    uint4 a = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(wrsrc, w_voff, soff, 0));
                    uint4 b = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(wrsrc, w_voff + 16, soff, 0));
                    if (!e_ok) a = make_uint4(0u, 0u, 0u, 0u);
                    if (!o_ok) b = make_uint4(0u, 0u, 0u, 0u);
                    we[g].raw = a;
                    wo[g].raw = b;
                }
            }
            half4_t hi[SB], lo[SB], rcv[SB];
#pragma unroll
            for (int sb = 0; sb < SB; ++sb) {
                float xt[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    xt[e] = vec_get<DT>(xv[i][j], 4 * sb + e) * inv_r;
                    hi[sb][e] = (_Float16)xt[e];
                }
                // lo must be formed from the very bits the MFMA consumes as hi:
                // left free, the compiler rounds x~ to f16 twice with two
                // instructions that break ties differently, and hi + lo misses
                // x~ by one f16 ulp on exact ties.
                pin_half4(hi[sb]);
#pragma unroll
                for (int e = 0; e < 4; ++e) lo[sb][e] = (_Float16)(xt[e] - (float)hi[sb][e]);
                rcv[sb] = quad_swap(p ? hi[sb] : lo[sb]);
            }
#pragma unroll
            for (int sb = 0; sb < SB; ++sb) {
                const half4_t be = p ? rcv[sb] : hi[sb];  // block columns cb + 4sb ..
                const half4_t bo = p ? lo[sb] : rcv[sb];  // block columns cb + V + 4sb ..
#pragma unroll
                for (int g = 0; g < G; ++g)
                    acc[g] = __builtin_amdgcn_mfma_f32_4x4x4f16(half_sub4<V>(we[g], sb), be,
                                                                acc[g], 0, 0, 0);
#pragma unroll
                for (int g = 0; g < G; ++g)
                    acc[g] = __builtin_amdgcn_mfma_f32_4x4x4f16(half_sub4<V>(wo[g], sb), bo,
                                                                acc[g], 0, 0, 0);
            }
        }
    }

    // layer_out for the post update: issued now, consumed after the reductions
    // and the Sinkhorn, whose latency it hides.
    StateVec<DT> lov[CS];
    if constexpr (MODE == MODE_FUSED) {
#pragma unroll
        for (int j = 0; j < CS; ++j) {
            const int c0 = (wave + TILE_WAVES * j) * STEP + blk * 2 * V + p * V;
            lov[j] = (tok_ok && c0 < d) ? load_vec<DT>(layer_out, tok * d + c0) : zero_vec<DT>();
        }
    }

    // ---- phase 3: sum the 16 blocks, then the waves, in a fixed order ----
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float v = acc[g][r];
            v += __shfl_xor(v, 4, 64);
            v += __shfl_xor(v, 8, 64);
            v += __shfl_xor(v, 16, 64);
            v += __shfl_xor(v, 32, 64);
            if (lane < 4) zred[wave][lane][4 * g + r] = v;
        }
    __syncthreads();
    if (tid < TILE_TOKENS * M) {
        const int tt = tid / M, row = tid % M;
        float s = zred[0][2 * tt][row] + zred[0][2 * tt + 1][row];
#pragma unroll
        for (int w = 1; w < TILE_WAVES; ++w) s += zred[w][2 * tt][row] + zred[w][2 * tt + 1][row];
        const float z = s + bias[row];
        zs[tt][row] = z;
        const size_t tk = (size_t)blockIdx.x * TILE_TOKENS + tt;
        if (logits && tk < (size_t)T) logits[tk * M + row] = z;
    }
    __syncthreads();

    // ---- phase 4: gates and Sinkhorn for both tokens (wave 0) ----
    if (wave == 0) {
        constexpr int NN = N * N;
        const int grp = lane / NN, e = lane % NN, tt = grp & 1;
        const float h = sinkhorn_lane<N>(zs[tt][2 * N + e], iters);
        const size_t tk = (size_t)blockIdx.x * TILE_TOKENS + tt;
        if (grp < TILE_TOKENS) {
            cf[tt][2 * N + e] = h;
            if (coeffs && tk < (size_t)T) coeffs[tk * M + 2 * N + e] = h;
        }
        if (lane < TILE_TOKENS * 2 * N) {
            const int gt = lane / (2 * N), idx = lane % (2 * N);
            const float gv = logistic(zs[gt][idx]);
            cf[gt][idx] = gv;
            const size_t gk = (size_t)blockIdx.x * TILE_TOKENS + gt;
            if (coeffs && gk < (size_t)T) coeffs[gk * M + idx] = gv;
        }
    }
    __syncthreads();

    // ---- phase 5: pre-mix and post update from the registers ----
#pragma unroll
    for (int j = 0; j < CS; ++j)
#pragma unroll
        for (int i = 0; i < N; ++i) launder<DT>(xv[i][j]);
    float pre[N], post[N], H[N][N];
#pragma unroll
    for (int i = 0; i < N; ++i) {
        pre[i] = cf[t][i];
        post[i] = cf[t][N + i];
#pragma unroll
        for (int j = 0; j < N; ++j) H[i][j] = cf[t][2 * N + i * N + j];
    }
#pragma unroll
    for (int j = 0; j < CS; ++j) {
        const int c0 = (wave + TILE_WAVES * j) * STEP + blk * 2 * V + p * V;
        if (!tok_ok || c0 >= d) continue;
        float x[N][V];
#pragma unroll
        for (int i = 0; i < N; ++i)
#pragma unroll
            for (int e = 0; e < V; ++e) x[i][e] = vec_get<DT>(xv[i][j], e);
        float li[V];
#pragma unroll
        for (int e = 0; e < V; ++e) {
            float s = pre[0] * x[0][e];
#pragma unroll
            for (int i = 1; i < N; ++i) s = fmaf(pre[i], x[i][e], s);
            li[e] = s;
        }
        store_vec<DT>(layer_in, tok * d + c0, li);
        if constexpr (MODE == MODE_FUSED) {
#pragma unroll
            for (int i = 0; i < N; ++i) {
                float o[V];
#pragma unroll
                for (int e = 0; e < V; ++e) {
                    float s = H[i][0] * x[0][e];
#pragma unroll
                    for (int jj = 1; jj < N; ++jj) s = fmaf(H[i][jj], x[jj][e], s);
                    o[e] = fmaf(post[i], vec_get<DT>(lov[j], e), s);
                }
                store_vec<DT>(X_out, tok * K + (size_t)i * d + c0, o);
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
static hipError_t launch_tile_n(int cs, const FusedArgs &a, hipStream_t s) {
    const dim3 grid((unsigned)((a.T + TILE_TOKENS - 1) / TILE_TOKENS)), block(TILE_THREADS);
#define DS4HC_TILE_CASE(CS)                                                                      \
    case CS:                                                                                     \
        return launch_kernel(hc_tile_kernel<N, DT, CS, MODE>, grid, block, s, a.d, (int)a.T,     \
                             a.eps, a.iters, a.X, a.W, a.bias, a.layer_out, a.layer_in,          \
                             a.coeffs, a.logits, a.X_out);
    switch (cs) {
        DS4HC_TILE_CASE(1)
        DS4HC_TILE_CASE(2)
        DS4HC_TILE_CASE(3)
        DS4HC_TILE_CASE(4)
        DS4HC_TILE_CASE(5)
        DS4HC_TILE_CASE(6)
        DS4HC_TILE_CASE(7)
        DS4HC_TILE_CASE(8)
    default:
        return hipErrorInvalidValue;
    }
#undef DS4HC_TILE_CASE
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

template <int N, int DT, int MODE>
static hipError_t dispatch_path(int path, const FusedArgs &a, hipStream_t s) {
    switch (path) {
    case PATH_ROWRES: return launch_rowres_n<N, DT, MODE>(rowres_chunks(a.d, DT), a, s);
    case PATH_TILE: return launch_tile_n<N, DT, MODE>(tile_steps(a.d, DT), a, s);
    case PATH_SPLITK: return launch_splitk_n<N, DT, MODE>(a, s);
    }
    return hipErrorInvalidValue;
}

template <int N>
static hipError_t dispatch_dt(int dt, bool fused, int path, const FusedArgs &a, hipStream_t s) {
    if (dt == DT_F32)
        return fused ? dispatch_path<N, DT_F32, MODE_FUSED>(path, a, s)
                     : dispatch_path<N, DT_F32, MODE_PRE>(path, a, s);
    return fused ? dispatch_path<N, DT_BF16, MODE_FUSED>(path, a, s)
                 : dispatch_path<N, DT_BF16, MODE_PRE>(path, a, s);
}

int rowres_chunks(int d, int dt) {
    const int V = dt == DT_F32 ? 4 : 8;
    return (d + ROWRES_THREADS * V - 1) / (ROWRES_THREADS * V);
}

int rowres_max_chunks(int n, int dt) { return rowres_cap(n, dt); }

int tile_steps(int d, int dt) {
    const int V = dt == DT_F32 ? 4 : 8;
    const int steps = (d + 32 * V - 1) / (32 * V);
    return (steps + TILE_WAVES - 1) / TILE_WAVES;
}

int tile_max_steps() { return 8; }

int splitk_chunks(int n, int d, int dt) {
    const int V = dt == DT_F32 ? 4 : 8;
    const long K = (long)n * d;
    return (int)((K + 64 * V - 1) / (64 * V));
}

hipError_t launch_hc(const FusedArgs &a, bool fused, int path, hipStream_t s) {
    switch (a.n) {
    case 1: return dispatch_dt<1>(a.dt, fused, path, a, s);
    case 2: return dispatch_dt<2>(a.dt, fused, path, a, s);
    case 4: return dispatch_dt<4>(a.dt, fused, path, a, s);
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
