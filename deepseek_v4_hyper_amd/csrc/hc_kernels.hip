// hc_kernels.hip -- HIP kernels of the DeepSeek-V4 hyper-connection op for
// MI355X (gfx950) and their host-side launchers.
//
// Three paths compute the same op (see ds4hc.h for its definition); the
// library picks one with a cost model in T and the row length K = n*d, fitted
// to measured sweeps of every path (default_path in ds4hc_api.cpp), and flags
// can force any of them:
//
//  * tile (large T): a persistent MFMA kernel, one 512-thread workgroup per
//    CU striding over tiles of four tokens. A tile's rows live in registers,
//    so X is read once and X' written once; the fn matvec runs on
//    v_mfma_f32_4x4x4_16b_f16 with W streamed from L2 through per-wave LDS
//    rings, and the drained rings stage half of the next tile's rows.
//
//  * row-resident (mid-size T where the cost model puts it, or rows too long
//    for the tile kernel):
//    one 256-thread workgroup per token; the token's n*d state is loaded once
//    into registers, the RMS statistic and the m = 2n + n*n fn dot products
//    are accumulated from it on the VALU, reduced in a fixed order, the gates
//    and the register-resident Sinkhorn run in one wavefront, and the pre-mix
//    and post update are computed from the same registers.
//
//  * split-K (small T: decode and speculative verify): the fn weight (m*K
//    float16, 768 KiB at d = 4096) dominates the bytes, so K is cut into
//    chunks and many workgroups each read one chunk of W for all tokens,
//    writing fixed-order partial sums to a caller workspace. A second kernel
//    combines them in chunk order, runs gates + Sinkhorn, and does the
//    pre-mix / post update column-parallel. The pages' decode runs these HC
//    sites 86 times per token (lucebox-hub PR #494, Sinkhorn comment), so
//    this path is about latency, not bandwidth.
//
// Also here: the one-pass decode-chain step (post of one site and the split-K
// part of the next), the two halves of the split over d (partial sums of a
// column share; their share-order combine), the post update alone and the
// Sinkhorn alone.
//
// Arithmetic: float32 accumulation with f16 weights widened exactly; the tile
// kernel's products are exact (the scaled state split into f16 hi + lo; hi
// alone for a bfloat16 state, exact to 2^-38 of the lane's largest value); the
// Sinkhorn multiplies by the hardware reciprocal of each sum; one RNE rounding
// at each store of a bf16 state. No floating-point atomics.
#include "hc_device.hpp"
#include "hc_launch.hpp"

#include <atomic>

#include <tuple>
#include <type_traits>
#include <utility>

namespace ds4hc {

constexpr int ROWRES_THREADS = 256;
constexpr int ROWRES_WAVES = ROWRES_THREADS / 64;
constexpr int SPLITK_TOKENS = 4;   // tokens per partials workgroup

// MODE_PARTIALS (tile kernel only): write each token's unnormalised fn dots
// and sum of squares, [T][m + 1] through the logits pointer, for one share of
// the columns; no gates, Sinkhorn or pass 2 (the split-over-d exchange point).
enum : int { MODE_PRE = 0, MODE_FUSED = 1, MODE_PARTIALS = 2 };

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
        const float h = sinkhorn_lane_dpp<N>(zr, iters);
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
// MFMA tile kernel: persistent, one 512-thread workgroup per CU striding over
// tiles of four tokens; the tile's rows are kept in registers and the fn
// matvec runs on v_mfma_f32_4x4x4_16b_f16.
//
// The fn projection of a tile is a [m x K] . [K x 4] product. One
// 4x4x4_16b instruction is 16 independent 4x4x4 products (block b = lane/4):
// A_b = 4 rows of W x 4 consecutive k, B_b = those 4 k x the 4 tokens. Lane
// 4b + t supplies token t's B column and W row t of the group's A. The lane's
// x, scaled by a power of two 2^S that puts its largest |x| in [2^13, 2^14)
// (so f16 cannot overflow), is split exactly into f16 hi + lo (hi = f16(x~),
// lo = f16(x~ - hi)); hi and lo are two MFMAs on the same A accumulating into
// one result, so hi + lo carries x~ to ~2^-23 relative, products are exact and
// accumulation is fp32; 2^-S and 1/r are applied to the reduced sums. For a
// bfloat16 state hi alone carries x~ (lo is skipped; see the projection).
// Each W element fetched from L2 feeds all four tokens.
//
// W (the same for every tile) streams from L2 through a ring of unit-sized
// slots in LDS, one ring per wave, filled by direct buffer->LDS loads that
// run RING - 1 units ahead of the MFMAs. The ring drains at the end of each
// projection, and its LDS then takes the next tile's rows of the first STAGED
// column steps straight from HBM, so those loads run during the reductions
// and the Sinkhorn, while the registers still hold the current tile. Pass 2
// moves the staged rows into each column step's registers as soon as the
// post update has consumed them, restarts the ring for the next tile, and
// loads the remaining steps' rows from HBM into their registers.
//
// Column step j of wave w covers STEP = 16*V columns of every stream:
// columns (w + 8j)*STEP + b*V .. +V-1 for token t = lane % 4, so every lane
// holds all n streams of its columns and the post update needs no exchange.
// ---------------------------------------------------------------------------
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef unsigned int uint2_t __attribute__((ext_vector_type(2)));

constexpr int TILE_TOKENS = 4;
constexpr int TILE_THREADS = 512;
constexpr int TILE_WAVES = TILE_THREADS / 64;

// Opaque register barrier on a 4 x f16 value: later uses see these exact bits.
__device__ __forceinline__ void pin_half4(half4_t &v) {
    uint2_t u = __builtin_bit_cast(uint2_t, v);
    asm volatile("" : "+v"(u.x), "+v"(u.y));
    v = __builtin_bit_cast(half4_t, u);
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

// A byte offset past any buffer this library describes: loads through it
// return zero and stores through it are dropped. Masking by offset keeps
// every load and store unconditional (no branches around memory operations,
// which would make the compiler drain all outstanding loads at the joins).
constexpr int OOB_OFFSET = 0x7FFFFFF0;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             BUFFER_RSRC_WORD3);
}

// Cache policy of the state stream: every row of X and layer_out is read once
// and every output written once, so both go non-temporal (the nt bit), which
// leaves L2 to the weight that every tile reads again. Measured on MI355X:
// prefill 180.6 -> 171.7 us, stress 707.6 -> 694.8 us against the default policy.
constexpr int CPOL_STREAM = 2;

// 16-byte state vector through a buffer descriptor (zero past num_records).
template <int DT>
__device__ __forceinline__ StateVec<DT> buf_load_vec(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    const uint4 u = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, CPOL_STREAM));
    StateVec<DT> v;
    if constexpr (DT == DT_F32)
        v.raw = make_float4(__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z),
                            __uint_as_float(u.w));
    else
        v.raw = u;
    return v;
}

// Store V float32 values as one 16-byte state vector (one RNE rounding for bf16);
// stores past num_records are dropped. The whole offset goes in the vector
// offset and the scalar offset is the constant 0: with an SGPR scalar offset
// the compiler assumes the 128-bit store-data hazard cannot occur and lets
// the next VALU instruction overwrite the data VGPRs at once, and on gfx950
// that corrupted the first dword of the stored vector.
template <int DT>
__device__ __forceinline__ void buf_store_vec(__amdgpu_buffer_rsrc_t r, int voff, const float *f) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    u32x4 u;
    if constexpr (DT == DT_F32) {
        u = (u32x4){__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                    __float_as_uint(f[3])};
    } else {
        u = (u32x4){f32x2_to_bf16x2_bits(f[0], f[1]), f32x2_to_bf16x2_bits(f[2], f[3]),
                    f32x2_to_bf16x2_bits(f[4], f[5]), f32x2_to_bf16x2_bits(f[6], f[7])};
    }
    __builtin_amdgcn_raw_buffer_store_b128(u, r, voff, 0, CPOL_STREAM);
}

// Per-wave ring of weight units in LDS, filled by direct buffer->LDS loads.
constexpr int TILE_RING_BYTES = 18 * 1024;  // per wave; 8 waves -> 144 KiB of the 160 KiB LDS

// Issue one direct buffer->LDS load of 16 bytes per lane: lane l's bytes land
// at lds_base + 16*l. Written as inline assembly so the compiler does not
// track it: its conservative handling of LDS DMA would drain every load in
// flight before each LDS read. Completion is waited for explicitly with
// wait_vm_at_most() before the data is read.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rsrc, uint32_t lds_base,
                                          int voff, int soff) {
    // M0 holds the LDS destination; one wait state must separate its write
    // from an LDS-DMA load that reads it. M0 is reserved to the compiler, so
    // the asm saves and restores it rather than declaring it clobbered.
    uint32_t saved_m0;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %2, %3, %4 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved_m0)
        : "s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(voff), "s"(rsrc), "s"(soff)
        : "memory");
}

// The same load with the non-temporal cache policy, for state rows (read once).
__device__ __forceinline__ void lds_dma16_nt(__amdgpu_buffer_rsrc_t rsrc, uint32_t lds_base,
                                             int voff, int soff) {
    uint32_t saved_m0;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %2, %3, %4 offen nt lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved_m0)
        : "s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(voff), "s"(rsrc), "s"(soff)
        : "memory");
}

// Wait until at most n vector-memory operations of this wave are outstanding.
// Vector memory operations complete in issue order, so every operation older
// than the last n is then complete.
template <int n>
__device__ __forceinline__ void wait_vm_at_most() {
    static_assert(n >= 0 && n < 64, "vmcnt range");
    // s_waitcnt encoding (gfx9): vmcnt[3:0] | expcnt[6:4] = 7 | lgkmcnt[11:8] = 15 | vmcnt[5:4] at [15:14]
    constexpr int enc = (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14);
    asm volatile("s_waitcnt %0" : : "n"(enc) : "memory");
}

// Calls f(std::integral_constant<int, I>) for I = B .. E - 1, in order.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// Loads a wave of the tile kernel has issued after the weight loads of unit u
// when it reaches unit u's wait, at least (U units per tile, a ring of RING
// slots, LOADS loads per unit; the ring is refilled only with units of the
// same tile and started afresh for every tile):
//  * u < RING: loaded by the tile's prologue, followed by the prologue's
//    later units and the refills issued at units 0 .. u - 1 (unit v refills
//    unit v + RING while that is < U);
//  * u >= RING: loaded as the refill at unit u - RING, followed by the
//    refills issued at units u - RING + 1 .. u - 1 that exist.
// Capped at 63, the most the counter holds.
constexpr int tile_unit_wait(int u, int U, int RING, int LOADS) {
    const int after = u < RING ? LOADS * (RING - 1 - u) + LOADS * (u < U - RING ? u : U - RING)
                               : LOADS * (RING - 1 < U - 1 - u ? RING - 1 : U - 1 - u);
    return after < 63 ? after : 63;
}

// wait_vm_at_most<(S - 1 - j) * P>() for a step j < S that is a constant only
// after loop unrolling (the S comparisons fold to the one wait).
template <int S, int P, int J = 0>
__device__ __forceinline__ void wait_vm_for_step(int j) {
    if constexpr (J < S) {
        if (j == J)
            wait_vm_at_most<(S - 1 - J) * P>();
        else
            wait_vm_for_step<S, P, J + 1>(j);
    }
}

// Wave priority (s_setprio takes an immediate): 3 while a wave issues loads of
// the state stream, otherwise `base` (0 or 1).
__device__ __forceinline__ void set_wave_prio(bool high, bool base) {
    if (high)
        __builtin_amdgcn_s_setprio(3);
    else if (base)
        __builtin_amdgcn_s_setprio(1);
    else
        __builtin_amdgcn_s_setprio(0);
}

// Sum over the 16 lanes of a DPP row that share lane % 4 (blocks of a row):
// rotations by 4 and 8 lanes.
__device__ __forceinline__ float row_sum_by4(float v) {
    v += dpp_mov<0x124>(v);  // row_ror:4
    v += dpp_mov<0x128>(v);  // row_ror:8
    return v;
}

// Sum over the 64 lanes that share lane % 4: rotations within each 16-lane
// row, then the gfx950 row swaps (rows 0<->1, 2<->3, then halves), which move
// data between rows in the VALU instead of through the LDS crossbar.
__device__ __forceinline__ float wave_sum_by4(float v) {
    v = row_sum_by4(v);
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Largest biased float32 exponent among the N*V values of column step j,
// from the raw bits (magnitudes compare as unsigned integers); NaN and Inf
// give 255.
template <int DT, int N, int CS>
__device__ __forceinline__ int max_biased_exponent(const StateVec<DT> (&xv)[N][CS], int j) {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const uint32_t w[4] = {__builtin_bit_cast(uint32_t, xv[i][j].raw.x),
                               __builtin_bit_cast(uint32_t, xv[i][j].raw.y),
                               __builtin_bit_cast(uint32_t, xv[i][j].raw.z),
                               __builtin_bit_cast(uint32_t, xv[i][j].raw.w)};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if constexpr (DT == DT_F32) {
                m = max(m, w[q] & 0x7FFFFFFFu);
            } else {
                m = max(m, (w[q] & 0x7FFFu) << 16);
                m = max(m, w[q] & 0x7FFF0000u);
            }
        }
    }
    return (int)(m >> 23);
}

template <int N, int DT, int CS, int MODE>
__global__ __launch_bounds__(TILE_THREADS, 1) void hc_tile_kernel(
    int d, int T, float eps, int iters, const void *__restrict__ X, const uint16_t *__restrict__ W,
    const float *__restrict__ bias, const void *__restrict__ layer_out, void *__restrict__ layer_in,
    float *__restrict__ coeffs, float *__restrict__ logits, void *X_out) {
    constexpr int V = StateVec<DT>::V;
    constexpr int M = n_logits(N);
    constexpr int G = (M + 3) / 4;   // groups of 4 W rows
    constexpr int SB = V / 4;        // 4-element k-blocks per lane vector
    constexpr int STEP = 16 * V;     // columns per step
    constexpr int U = CS * N;        // (column step, stream) units per wave and tile
    constexpr int ROWB = STEP * 2;   // bytes of one W row within a unit
    constexpr int UNIT = 4 * G * ROWB;
    constexpr int LOADS = (UNIT + 1023) / 1024;  // 16-byte-per-lane loads per unit
    constexpr int SLOT = LOADS * 1024;
    constexpr int RING_FIT = TILE_RING_BYTES / SLOT;
    // At most U slots: the ring then always holds consecutive units of one
    // tile or the next, which is what the refill below assumes.
    constexpr int RING_CAP = RING_FIT > 8 ? 8 : RING_FIT;
    constexpr int RING = RING_CAP < U ? RING_CAP : U;
    constexpr int SBYTES = DT == DT_F32 ? 4 : 2;
    static_assert(RING >= 1 && RING * SLOT <= TILE_RING_BYTES, "weight ring");
    // Column steps of the next tile's rows staged in this wave's ring area
    // while the ring is idle (one 1 KiB load per stream and step).
    constexpr int STAGE_FIT = RING * SLOT / (N * 1024);
    constexpr int STAGED = STAGE_FIT < CS ? STAGE_FIT : CS;
    static_assert(STAGED >= 1, "staging area");

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // readfirstlane makes the wave index (and every offset built from it) a
    // scalar the compiler can put in the buffer loads' scalar offset field.
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const size_t K = (size_t)N * d;
    const int ntiles = (T + TILE_TOKENS - 1) / TILE_TOKENS;

    __shared__ __attribute__((aligned(16))) unsigned char wring[TILE_WAVES][RING][SLOT];
    __shared__ float ssr[TILE_WAVES][TILE_TOKENS];
    __shared__ float zred[TILE_WAVES][TILE_TOKENS][G * 4];
    __shared__ float zs[TILE_TOKENS][M];
    __shared__ float cf[TILE_TOKENS][M];

    // ---- weight units: unit u = (column step u / N of this wave, stream u % N).
    // Load q of a unit: lane l fetches bytes [p, p+16) of the unit's [4G rows][STEP
    // columns] f16 block, p = 1024 q + 16 l: row p / ROWB, byte p % ROWB of the
    // row's slice. ROWB divides 1024, so the column is the same for every q
    // and load q is row offset q * 1024 / ROWB further down. Rows at or past M
    // lie past the end of W, so the buffer descriptor turns them into zeros.
    static_assert(1024 % ROWB == 0, "weight unit rows");
    constexpr int QROWS = 1024 / ROWB;
    const __amdgpu_buffer_rsrc_t wrsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(W), (short)0, (int)((size_t)M * K * 2), BUFFER_RSRC_WORD3);
    const int row_bytes = (int)(K * 2);
    const uint32_t ring_base = (uint32_t)(uintptr_t)&wring[wave][0][0];
    auto unit_step = [&](int u) { return wave + TILE_WAVES * (u / N); };
    // wlane = this lane's offset within a unit's first load, wcol its column.
    auto issue_unit = [&](int u, int slot, int dd, int wlane, int wcol) {
        const int soff = ((u % N) * dd + unit_step(u) * STEP) * 2;
        const bool ok = wcol < dd - unit_step(u) * STEP;
#pragma unroll
        for (int q = 0; q < LOADS; ++q) {
            const int voff = ok ? wlane + q * QROWS * row_bytes : OOB_OFFSET;
            lds_dma16(wrsrc, ring_base + (uint32_t)(slot * SLOT + q * 1024), voff, soff);
        }
    };
    // Bank swizzle of a slot: row r's bytes sit at r * ROWB + (c ^ wswz(r)).
    // A unit read has lane 4b + t read row 4g + t at the same column for
    // every t; with 128-byte rows (float32 state) rows t and t + 2, with
    // 256-byte rows (bfloat16) all four rows would share banks (64 banks of
    // 4 bytes). Exchanging row halves (quarters) by row makes each read
    // conflict-free; the arithmetic is unchanged.
    static_assert(ROWB == 128 || ROWB == 256, "weight row pitch");
    auto wswz = [](int r) { return ROWB == 128 ? ((r >> 1) & 1) * 64 : (r & 3) * 64; };
    // lane l's direct load puts the unit's bytes for slot offset 16 l (+ 1024 q)
    auto lane_wlane = [&](int ln) {
        const int r = 16 * ln / ROWB;
        return r * row_bytes + (((16 * ln) % ROWB) ^ wswz(r));
    };
    auto lane_wcol = [&](int ln) { return (((16 * ln) % ROWB) ^ wswz(16 * ln / ROWB)) / 2; };

    // the first tile's first RING units, before anything else
#pragma unroll
    for (int u = 0; u < RING; ++u) issue_unit(u, u, d, lane_wlane(lane), lane_wcol(lane));

    auto tile_rsrc = [&](const void *base, size_t row_elems, int tile) {
        const size_t tile0 = (size_t)tile * TILE_TOKENS;
        const size_t ntok = min((size_t)TILE_TOKENS, (size_t)T - tile0);
        return make_rsrc((const char *)base + tile0 * row_elems * SBYTES,
                         (uint32_t)(ntok * row_elems * SBYTES));
    };

    // ---- the first tile's rows into registers ----
    StateVec<DT> xv[N][CS];
    {
        const __amdgpu_buffer_rsrc_t xr = tile_rsrc(X, K, blockIdx.x);
        const int bv = (lane >> 2) * V;
        const int x_voff = ((lane & 3) * (int)K + bv) * SBYTES;
#pragma unroll
        for (int j = 0; j < CS; ++j) {
            const int cs = wave + TILE_WAVES * j;
            const int voff = bv < d - cs * STEP ? x_voff : OOB_OFFSET;
#pragma unroll
            for (int i = 0; i < N; ++i) xv[i][j] = buf_load_vec<DT>(xr, voff, (i * d + cs * STEP) * SBYTES);
        }
    }

    // bias of the logit row this thread finishes in every tile, loaded once
    // (a load inside the loop would make the compiler drain every load in flight)
    const float bias_row = MODE != MODE_PARTIALS && tid < TILE_TOKENS * M ? bias[tid % M] : 0.f;

    for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        const bool has_next = tile + (int)gridDim.x < ntiles;
        const size_t tile0 = (size_t)tile * TILE_TOKENS;
        // Every per-lane offset and mask below is the same for every tile.
        // Re-deriving them here from values hidden from the optimiser keeps it
        // from hoisting them out of the loop into registers that stay live for
        // the whole kernel (they are a few integer operations per tile).
        int dl = d, ln = lane;
        asm volatile("" : "+s"(dl));  // (separate statements: an asm with any
        asm volatile("" : "+v"(ln));  //  vector output counts as divergent)
        const int tid_l = wave * 64 + ln;
        const int blk = ln >> 2;
        const int t = ln & 3;  // token of this lane's B column; also its A row in the group
        const int bv = blk * V;  // this lane's first column within a column step
        const int x_voff = (t * (int)K + bv) * SBYTES;
        const int d_voff = (t * dl + bv) * SBYTES;
        const int wlane = lane_wlane(ln), wcol = lane_wcol(ln);
        const int wread = t * ROWB + ((bv * 2) ^ wswz(t));  // byte of row t's slice read by this lane

        // ---- phase 2: fn matvec on MFMA, weights from the LDS ring ----
        // The projection runs on the raw rows and is normalised afterwards
        // (z = (W . x) / r), so it does not wait for the whole tile to arrive:
        // unit u needs only its own column step, and the rows of the next
        // tile stream in while the MFMAs of its first units run. The f16
        // split needs x scaled into f16 range: each lane keeps its own
        // power-of-two scale 2^S, lowered (and its accumulators rescaled,
        // exactly) when a column step brings a larger value. A lane's accumulators
        // only ever hold its own B column (its token, its columns), so no
        // other lane needs to agree on S. The sum of squares accumulates in
        // the same pass.
        float4_t acc[G];
#pragma unroll
        for (int g = 0; g < G; ++g) acc[g] = (float4_t){0.f, 0.f, 0.f, 0.f};
        int S = 140;  // |x| * 2^S < 2^14 for every x seen so far
        float ss = 0.f;
        static_for<0, U>([&](auto uc) {
            constexpr int u = decltype(uc)::value;
            constexpr int slot = u % RING;
            // Unit u's loads are complete once no more vector-memory loads
            // are outstanding than were issued after them (loads complete in
            // issue order): see tile_unit_wait. Anything else issued since
            // only makes this stricter.
            wait_vm_at_most<tile_unit_wait(u, U, RING, LOADS)>();
            HalfVec<V> w[G];
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const unsigned char *src = &wring[wave][slot][4 * g * ROWB + wread];
                if constexpr (V == 4)
                    w[g].raw = *reinterpret_cast<const uint2 *>(src);
                else
                    w[g].raw = *reinterpret_cast<const uint4 *>(src);
            }
            // Scale updates. For a float32 state, two per tile: at unit 0 from
            // the staged column steps, at the first unit of the other steps from
            // those (whose rows have in practice all arrived by then, as that
            // unit's weight refill queues behind them): prefill 147.4 -> 146.1
            // us on MI355X, the same bits. For bfloat16 that form made the
            // instance spill registers, so it updates at every column step.
            constexpr bool TWO_SCALES = DT == DT_F32;
            if constexpr (TWO_SCALES ? (u == 0 || u == STAGED * N) : (u % N == 0)) {
                constexpr int j0 = TWO_SCALES ? (u == 0 ? 0 : STAGED) : u / N;
                constexpr int j1 = TWO_SCALES ? (u == 0 ? STAGED : CS) : u / N + 1;
                int eb = 0;
#pragma unroll
                for (int j = j0; j < j1; ++j) eb = max(eb, max_biased_exponent<DT, N>(xv, j));
                // 2^(140 - eb) puts the largest |x| in [2^13, 2^14); for Inf or
                // NaN the scale is tiny and Inf stays Inf, NaN stays NaN.
                const int s_new = min(S, 140 - eb);
                // Rescale unconditionally (by 2^0 when nothing changed): a
                // branch here fragments the unrolled loop and costs registers.
                // At unit 0 the accumulators are still zero.
                if constexpr (u != 0) {
#pragma unroll
                    for (int g = 0; g < G; ++g)
#pragma unroll
                        for (int r = 0; r < 4; ++r) acc[g][r] = __builtin_amdgcn_ldexpf(acc[g][r], s_new - S);
                }
                S = s_new;
            }
            const StateVec<DT> &xvu = xv[u % N][u / N];
            float xr[V];
#pragma unroll
            for (int e = 0; e < V; ++e) {
                xr[e] = vec_get<DT>(xvu, e);
                ss = fmaf(xr[e], xr[e], ss);
            }
            half4_t hi[SB], lo[SB];
#pragma unroll
            for (int sb = 0; sb < SB; ++sb) {
                float xt[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    xt[e] = __builtin_amdgcn_ldexpf(xr[4 * sb + e], S);
                    hi[sb][e] = (_Float16)xt[e];
                }
                // A bfloat16 x has 8 significant bits, which f16 holds exactly
                // down to 2^-17 (its subnormals included); the lane's largest
                // scaled value is at least 2^13, so hi misses x~ only for values
                // more than 2^30 below it, by at most 2^-25 = 2^-38 of it. lo is
                // then zero or negligible, and its MFMAs are skipped (stress
                // workload: the same bits, 618.2 -> 605.9 us on MI355X).
                if constexpr (DT == DT_F32) {
                    // lo must be formed from the very bits the MFMA consumes as
                    // hi: left free, the compiler rounds x~ to f16 twice with two
                    // instructions that break ties differently, and hi + lo
                    // misses x~ by one f16 ulp on exact ties.
                    pin_half4(hi[sb]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) lo[sb][e] = (_Float16)(xt[e] - (float)hi[sb][e]);
                }
            }
#pragma unroll
            for (int sb = 0; sb < SB; ++sb)
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    const half4_t a = half_sub4<V>(w[g], sb);
                    acc[g] = __builtin_amdgcn_mfma_f32_4x4x4f16(a, hi[sb], acc[g], 0, 0, 0);
                    if constexpr (DT == DT_F32)
                        acc[g] = __builtin_amdgcn_mfma_f32_4x4x4f16(a, lo[sb], acc[g], 0, 0, 0);
                }
            // Refill this slot, once this wave's reads of it are done, with
            // unit u + RING of this tile. The ring is not carried into the next
            // tile: it holds the next tile's rows in between (below).
            if constexpr (u + RING < U) {
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                issue_unit(u + RING, slot, dl, wlane, wcol);
            }
        });

        // layer_out for the post update: issued now, consumed after the reductions
        // and the Sinkhorn, whose latency it hides.
        // Issue priority. The CU's vector-memory stream serves waves in
        // priority order, then by age, so the older wave of each SIMD (0..3)
        // used to get its whole pass 2 through first, and waves 4..7 - the
        // tile's critical path - finished pass 2 and their projection ~9 us
        // later. Every load of the state stream (layer_out, staged and HBM rows
        // of the next tile) is issued at priority 3, so loads overtake queued
        // stores, and waves 4..7 run pass 2 at priority 1. Prefill 146.6 ->
        // 140.7 us, stress 598.3 -> 554.6 us on MI355X, the same bits.
        const bool late_wave = wave >= TILE_WAVES / 2;
        StateVec<DT> lov[CS];
        if constexpr (MODE == MODE_FUSED) {
            const __amdgpu_buffer_rsrc_t lr = tile_rsrc(layer_out, (size_t)d, tile);
            set_wave_prio(true, false);
#pragma unroll
            for (int j = 0; j < CS; ++j) {
                const int cs = wave + TILE_WAVES * j;
                const int voff = bv < dl - cs * STEP ? d_voff : OOB_OFFSET;
                lov[j] = buf_load_vec<DT>(lr, voff, cs * STEP * SBYTES);
            }
            set_wave_prio(false, false);
        }

        // The ring has drained. Its LDS takes the next tile's rows of the
        // first STAGED column steps, by direct loads that stream in during the
        // reductions and the Sinkhorn; the registers still hold this tile.
        // (Past the last tile the loads return zeros that go unused.)
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's ring reads are done
        {
            const __amdgpu_buffer_rsrc_t xs = tile_rsrc(X, K, has_next ? tile + (int)gridDim.x : tile);
            set_wave_prio(true, false);
#pragma unroll
            for (int j = 0; j < STAGED; ++j) {
                const int cs = wave + TILE_WAVES * j;
                const int voff = bv < dl - cs * STEP && has_next ? x_voff : OOB_OFFSET;
#pragma unroll
                for (int i = 0; i < N; ++i)
                    lds_dma16_nt(xs, ring_base + (uint32_t)((j * N + i) * 1024), voff,
                                 (i * dl + cs * STEP) * SBYTES);
            }
            set_wave_prio(false, false);
        }

        // ---- phase 3: undo each lane's scale, sum the 16 blocks (DPP within
        // rows, then across rows), then the waves; normalise by 1/r ----
        ss = wave_sum_by4(ss);
        float zsum[G][4];
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int r = 0; r < 4; ++r) zsum[g][r] = wave_sum_by4(__builtin_amdgcn_ldexpf(acc[g][r], -S));
        if (ln < TILE_TOKENS) {
            ssr[wave][ln] = ss;
#pragma unroll
            for (int g = 0; g < G; ++g)
#pragma unroll
                for (int r = 0; r < 4; ++r) zred[wave][ln][4 * g + r] = zsum[g][r];
        }
        __syncthreads();
        if (tid_l < TILE_TOKENS * M) {
            const int tt = tid_l / M, row = tid_l % M;
            float sst = ssr[0][tt];
#pragma unroll
            for (int w = 1; w < TILE_WAVES; ++w) sst += ssr[w][tt];
            const float inv_r = 1.0f / sqrtf(sst / (float)K + eps);
            float s = zred[0][tt][row];
#pragma unroll
            for (int w = 1; w < TILE_WAVES; ++w) s += zred[w][tt][row];
            const size_t tk = tile0 + tt;
            if constexpr (MODE == MODE_PARTIALS) {
                if (tk < (size_t)T) {
                    logits[tk * (M + 1) + row] = s;
                    if (row == 0) logits[tk * (M + 1) + M] = sst;
                }
            } else {
                const float z = s * inv_r + bias_row;
                zs[tt][row] = z;
                if (logits && tk < (size_t)T) logits[tk * M + row] = z;
            }
        }
        __syncthreads();

        const __amdgpu_buffer_rsrc_t lir = tile_rsrc(layer_in, (size_t)d, tile);
        // ---- phase 4: gates and Sinkhorn for the four tokens (wave 0). For a
        // float32 state the other waves compute their pre gates themselves (the
        // same function on the same logits, so the same bits) and store the
        // pre-mix meanwhile: prefill 153.4 -> 150.9 us on MI355X. (For bfloat16
        // the extra unpacking made that instance spill registers.)
        constexpr bool EARLY_PREMIX = MODE != MODE_PARTIALS && DT == DT_F32;
        if (EARLY_PREMIX && wave != 0) {
            float pre_w[N];
#pragma unroll
            for (int i = 0; i < N; ++i) pre_w[i] = logistic(zs[t][i]);
#pragma unroll
            for (int j = 0; j < CS; ++j) {
                const int cs = wave + TILE_WAVES * j;
                float li[V];
#pragma unroll
                for (int e = 0; e < V; ++e) {
                    float s = pre_w[0] * vec_get<DT>(xv[0][j], e);
#pragma unroll
                    for (int i = 1; i < N; ++i) s = fmaf(pre_w[i], vec_get<DT>(xv[i][j], e), s);
                    li[e] = s;
                }
                buf_store_vec<DT>(lir, bv < dl - cs * STEP ? d_voff + cs * STEP * SBYTES : OOB_OFFSET, li);
            }
        }
        if (MODE != MODE_PARTIALS && wave == 0) {
            constexpr int NN = N * N;
            const int grp = ln / NN, e = ln % NN, tt = grp % TILE_TOKENS;
            const float h = sinkhorn_lane_dpp<N>(zs[tt][2 * N + e], iters);
            const size_t tk = tile0 + tt;
            if (grp < TILE_TOKENS) {
                cf[tt][2 * N + e] = h;
                if (coeffs && tk < (size_t)T) coeffs[tk * M + 2 * N + e] = h;
            }
            if (ln < TILE_TOKENS * 2 * N) {
                const int gt = ln / (2 * N), idx = ln % (2 * N);
                const float gv = logistic(zs[gt][idx]);
                cf[gt][idx] = gv;
                const size_t gk = tile0 + gt;
                if (coeffs && gk < (size_t)T) coeffs[gk * M + idx] = gv;
            }
        }
        __syncthreads();

        // ---- phase 5: pre-mix and post update from the registers; the next
        // tile's rows are loaded into each step's registers as soon as they are free ----
        float pre[N], post[N], H[N][N];
#pragma unroll
        for (int i = 0; i < N; ++i) {
            pre[i] = cf[t][i];
            post[i] = cf[t][N + i];
#pragma unroll
            for (int j = 0; j < N; ++j) H[i][j] = cf[t][2 * N + i * N + j];
        }
#pragma unroll
        for (int j = 0; j < CS; ++j)
#pragma unroll
            for (int i = 0; i < N; ++i) launder<DT>(xv[i][j]);
        const __amdgpu_buffer_rsrc_t xor_ = tile_rsrc(X_out, K, tile);
        set_wave_prio(false, late_wave);
        const __amdgpu_buffer_rsrc_t xnext = tile_rsrc(X, K, has_next ? tile + (int)gridDim.x : tile);
#pragma unroll
        for (int j = 0; j < CS; ++j) {
            const int cs = wave + TILE_WAVES * j;
            const bool col_ok = bv < dl - cs * STEP;
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
            // (with EARLY_PREMIX, waves 1..7 stored theirs during the Sinkhorn)
            if (MODE != MODE_PARTIALS && (!EARLY_PREMIX || wave == 0))
                buf_store_vec<DT>(lir, col_ok ? d_voff + cs * STEP * SBYTES : OOB_OFFSET, li);
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
                    buf_store_vec<DT>(xor_, col_ok ? x_voff + (i * d + cs * STEP) * SBYTES : OOB_OFFSET, o);
                }
            }
            if (j < STAGED) {
                // Staged rows: step j's loads are complete once no more loads
                // are outstanding than the staged loads issued after them
                // (loads complete in issue order; stores since only add).
                wait_vm_for_step<STAGED, N>(j);
#pragma unroll
                for (int i = 0; i < N; ++i) {
                    const unsigned char *src = &wring[wave][0][0] + (j * N + i) * 1024 + 16 * ln;
                    if constexpr (DT == DT_F32)
                        xv[i][j].raw = *reinterpret_cast<const float4 *>(src);
                    else
                        xv[i][j].raw = *reinterpret_cast<const uint4 *>(src);
                }
                if (j == STAGED - 1) {
                    // the staged rows are in registers: the next tile's first
                    // RING weight units go into the ring
                    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
                    for (int u = 0; u < RING; ++u) issue_unit(u, u, dl, wlane, wcol);
                }
            } else {
                // (zeros past the last tile: no branch around the loads)
                const int voff = col_ok && has_next ? x_voff : OOB_OFFSET;
                set_wave_prio(true, late_wave);
#pragma unroll
                for (int i = 0; i < N; ++i) xv[i][j] = buf_load_vec<DT>(xnext, voff, (i * dl + cs * STEP) * SBYTES);
                set_wave_prio(false, late_wave);
            }
        }
        set_wave_prio(false, false);
    }
    // no load into this workgroup's LDS may still be in flight when it ends
    wait_vm_at_most<0>();
}

// ---------------------------------------------------------------------------
// Sum of p[c * stride] over chunks c = 0 .. P-1, added in ascending c, with PB
// loads in flight at a time. A last batch shorter than PB reads the final chunk
// again in its unused slots (every load is in bounds and none waits on
// another) and skips those slots in the sum. Loading the remainder one chunk
// at a time instead serialised it: 28 chunks at d = 7168 bf16 were 28
// dependent trips past L2.
// ---------------------------------------------------------------------------
template <int PB>
__device__ __forceinline__ float sum_chunks(const float *__restrict__ p, size_t stride, int P) {
    float tot = 0.f;
    int c = 0;
    for (; c + PB <= P; c += PB) {
        float v[PB];
#pragma unroll
        for (int k = 0; k < PB; ++k) v[k] = p[(size_t)(c + k) * stride];
#pragma unroll
        for (int k = 0; k < PB; ++k) tot += v[k];
    }
    if (c < P) {
        const int last = P - 1 - c;  // < PB
        float v[PB];
#pragma unroll
        for (int k = 0; k < PB; ++k) v[k] = p[(size_t)(c + min(k, last)) * stride];
#pragma unroll
        for (int k = 0; k < PB; ++k)
            if (k <= last) tot += v[k];
    }
    return tot;
}

// ---------------------------------------------------------------------------
// Streamed partials: grid (ceil(T / 16), column chunks), 512 threads. For the
// split over d at large T one chunk holds the whole share row; split-K from
// T = 32 takes chunks of KC columns (multiples of 256) of the row, each
// chunk's sums to its slice of the workspace. With no pass 2 the rows need not
// stay on chip, so a workgroup takes 16 tokens and streams their rows, and
// its chunk of the weight, through its CU once (the tile kernel's partials
// mode streams the weight once per 4 tokens, the column-chunk kernel once per
// 4). The chunk (K = n * d_s columns for the split over d) is cut into k-steps
// of 32 columns; wave w takes the w-th of eight contiguous runs of steps.
// Lane l holds token l % 16 and columns 8 (l / 16) .. + 7 of a step: 32 bytes
// of its token's row (16 for bfloat16) and 16 bytes of each of its W rows,
// through buffer descriptors (rows past T or M and columns past K read zeros).
// The fn dots are float32 MFMAs, v_mfma_f32_16x16x4_f32 with A = W (row
// 16 b + l % 16 of block b, converted from f16 exactly) and B = x (token
// l % 16), one instruction per column of the lane's eight: D[row][token]
// gains the products of four columns, one per lane group. The sum of squares
// is a per-lane VALU chain. A wave keeps one batch of SP_BATCH steps in flight
// while it uses the other. Each wave's sums go to LDS and are added in wave
// order (and lane-group order for the sum of squares), so the result does not
// depend on timing.
//
// Measured on the prefill share (T = 4096, K = 4096, float32): the same loads
// with the steps interleaved over the waves read the share at 4.2 TB/s against
// 6.0 with contiguous runs (a token row is then read in 64-byte pieces
// scattered over all the waves); 8-byte W loads per lane (16 columns per
// step) left the load side alone at 22.7 us. The state loads keep the default
// cache policy: the two 16-byte loads of a float32 lane each cover half of the
// token's 128-byte line, and with the streaming (nt) policy the pass took 20.3
// against 17.7 us. One step per batch: 17.0 us; two 17.7, four 23.
// ---------------------------------------------------------------------------
constexpr int SP_TOKENS = 16;
constexpr int SP_WAVES = 8;
constexpr int SP_BATCH = 1;  // k-steps of 32 columns per register batch (two batches)

template <int N, int DT>
__global__ __launch_bounds__(SP_WAVES * 64) void hc_stream_partials_kernel(int K, int KC, int T,
                                                                           const void *__restrict__ X,
                                                                           const uint16_t *__restrict__ W,
                                                                           float *__restrict__ out) {
    constexpr int M = n_logits(N);
    constexpr int RB = (M + 15) / 16;  // 16-row blocks of W
    static_assert((M + 1) * SP_TOKENS <= SP_WAVES * 64, "one thread per output of the final sum");
    typedef float f4_t __attribute__((ext_vector_type(4)));
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int tok = lane & 15, grp = lane >> 4;
    const int t0 = blockIdx.x * SP_TOKENS;
    const int ntok = min(SP_TOKENS, T - t0);
    constexpr int SB = DT == DT_F32 ? 4 : 2;
    // Buffer loads: tokens past T (past this group's rows) and W rows past M
    // lie past their descriptor's end, and columns past the chunk's end take
    // OOB_OFFSET, so all of them read zeros with no branch or select.
    const __amdgpu_buffer_rsrc_t xr = make_rsrc((const char *)X + (size_t)t0 * K * SB, (uint32_t)((size_t)ntok * K * SB));
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(W, (uint32_t)((size_t)M * K * 2));
    // column chunk blockIdx.y: columns [kbase, kend) of the flattened row,
    // its sums to out[blockIdx.y][T][M + 1] (one chunk of all K columns for
    // the split over d)
    const int kbase = blockIdx.y * KC;
    const int kend = min(K, kbase + KC);
    out += (size_t)blockIdx.y * T * (M + 1);
    const int nsteps = (kend - kbase + 31) / 32;
    const int per = (nsteps + SP_WAVES - 1) / SP_WAVES;
    const int first = wave * per;
    const int mine = max(0, min(per, nsteps - first));
    __shared__ float red[SP_WAVES][M + 4][SP_TOKENS];

    // Two batches of SP_BATCH steps in registers: while one is used, the
    // other's loads are in flight. The batches swap roles every half of the
    // loop, so the batch being used was always issued before the one in
    // flight, on the way into the loop as on the way round it.
    struct Batch {
        StateVec<DT> x[SP_BATCH][8 / StateVec<DT>::V];
        uint4 w[SP_BATCH][RB];
    };
    // steps i .. i + SP_BATCH - 1 of this wave (steps past its last read zeros)
    auto fetch = [&](Batch &bt, int i) {
#pragma unroll
        for (int j = 0; j < SP_BATCH; ++j) {
            const int k = kbase + (first + i + j) * 32 + 8 * grp;
            const bool ok = i + j < mine && k < kend;
            // (offsets pinned in a register: given the constant OOB_OFFSET in
            // one arm, the compiler otherwise branches between two loads)
            int xo = ok ? (tok * K + k) * SB : OOB_OFFSET;
            asm volatile("" : "+v"(xo));
#pragma unroll
            for (int h = 0; h < 8 / StateVec<DT>::V; ++h) {
                const uint4 u = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xr, xo, 16 * h, 0));
                if constexpr (DT == DT_F32)
                    bt.x[j][h].raw = make_float4(__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z),
                                                 __uint_as_float(u.w));
                else
                    bt.x[j][h].raw = u;
            }
#pragma unroll
            for (int b = 0; b < RB; ++b) {
                int wo = ok ? ((16 * b + tok) * K + k) * 2 : OOB_OFFSET;
                asm volatile("" : "+v"(wo));
                bt.w[j][b] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(wr, wo, 0, 0));
            }
        }
    };

    f4_t acc[RB];
#pragma unroll
    for (int b = 0; b < RB; ++b) acc[b] = f4_t{0.f, 0.f, 0.f, 0.f};
    float ss = 0.f;
    auto use = [&](const Batch &bt) {
#pragma unroll
        for (int j = 0; j < SP_BATCH; ++j) {
            float xf[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                constexpr int V = StateVec<DT>::V;
                xf[e] = vec_get<DT>(bt.x[j][e / V], e % V);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) ss = fmaf(xf[e], xf[e], ss);
#pragma unroll
            for (int e = 0; e < 8; ++e)
#pragma unroll
                for (int b = 0; b < RB; ++b) {
                    HalfVec<8> hv;
                    hv.raw = bt.w[j][b];
                    acc[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(half_get<8>(hv, e), xf[e], acc[b], 0, 0, 0);
                }
        }
    };

    // (scheduling barriers keep each batch's loads issued as a block, ahead
    // of the use of the other batch)
    Batch A, Bn;
    fetch(A, 0);
    for (int i0 = 0; i0 < mine; i0 += 2 * SP_BATCH) {
        __builtin_amdgcn_sched_barrier(0);
        fetch(Bn, i0 + SP_BATCH);
        __builtin_amdgcn_sched_barrier(0);
        use(A);
        __builtin_amdgcn_sched_barrier(0);
        fetch(A, i0 + 2 * SP_BATCH);
        __builtin_amdgcn_sched_barrier(0);
        use(Bn);
    }

    // D layout: lane l holds rows 4 (l / 16) + r of its block, token l % 16
#pragma unroll
    for (int b = 0; b < RB; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * b + 4 * grp + r;
            if (row < M) red[wave][row][tok] = acc[b][r];
        }
    red[wave][M + grp][tok] = ss;
    __syncthreads();
    const int tid = threadIdx.x;
    if (tid < (M + 1) * SP_TOKENS) {
        const int j = tid / SP_TOKENS, tk = tid % SP_TOKENS;
        float v = 0.f;
        if (j < M) {
#pragma unroll
            for (int w = 0; w < SP_WAVES; ++w) v += red[w][j][tk];
        } else {
#pragma unroll
            for (int w = 0; w < SP_WAVES; ++w)
#pragma unroll
                for (int g = 0; g < 4; ++g) v += red[w][M + g][tk];
        }
        if (t0 + tk < T) out[(size_t)(t0 + tk) * (M + 1) + j] = v;
    }
}

// ---------------------------------------------------------------------------
// Split-over-d partials for small T: the split-K chunk partials of one column
// share summed in chunk order into out[t][0..M] (dots, then sum of squares).
// Grid (T), one wavefront.
// ---------------------------------------------------------------------------
template <int N>
__global__ __launch_bounds__(64) void hc_chunk_sum_kernel(int T, int P, const float *__restrict__ ws,
                                                          float *__restrict__ out) {
    constexpr int M = n_logits(N);
    const int lane = threadIdx.x;
    const size_t t = blockIdx.x;
    if (lane > M) return;
    out[t * (M + 1) + lane] = sum_chunks<32>(ws + t * (M + 1) + lane, (size_t)T * (M + 1), P);
}

// ---------------------------------------------------------------------------
// Split-K partials over column chunks: grid (ceil(T / SPLITK_TOKENS), P), one
// wavefront. With L lanes per column chunk (16 or 32), chunk p covers columns
// [p*L*V, (p+1)*L*V) of every stream: lane l = L g + c holds the V columns
// p*L*V + c*V .. of all n streams, and the 64 / L lane groups g hold the same
// columns and split the M fn rows (rows g*RPW ..), so each lane sums only its
// group's rows over 16 or 32 lanes. Writes the partial dots and the partial
// sum of squares to ws[p][t][0..M]; the finish kernel (or the chunk sum of the
// split over d) adds them in chunk order.
//
// POST = false: the partials of X itself (split-K HC-pre, and the split over
// d at small T). POST = true: the one-pass chain step; a lane first applies
// the previous site's post update X' = H.X + post (x) layer_out to its columns
// (same operation order as hc_post_kernel, so X' is bitwise what ds4hc_post
// writes), group 0 stores X', and the partials are those of X' as stored
// (rounded to the state type).
//
// At decode sizes the pass is latency-bound: narrower chunks spread W over
// more CUs and give each lane fewer loads, but add partials for the finish
// kernel to combine. colchunk_lanes() takes 16 lanes while that gives at most
// 64 chunks, else 32. Graph-replayed ds4hc_post_pre at T = 1, 16 against 32
// lanes: d = 4096 fp32 6.2 / 6.7 us, d = 7168 bf16 8.0 / 8.3 us, d = 7168 fp32
// (112 chunks at 16 lanes) 8.0 / 7.7 us. For HC-pre this layout replaced
// chunks of 64 lanes over the flattened row, each lane summing all M + 1
// values over the whole wave per token: ds4hc_fused at T = 4, d = 4096 fp32
// 11.4 -> 7.7 us, at T = 1 7.4 -> 6.1 us.
// ---------------------------------------------------------------------------

// Sum over the L lanes of a column chunk (every lane gets the total): within
// each 16-lane DPP row, then across row pairs by the gfx950 row swap when a
// chunk spans two rows.
template <int L>
__device__ __forceinline__ float chunk_sum(float v) {
    static_assert(L == 16 || L == 32, "chunk of one or two DPP rows");
    v += dpp_mov<0x128>(v);  // row_ror:8
    v += dpp_mov<0x124>(v);  // row_ror:4
    v += dpp_mov<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp_mov<0xB1>(v);   // quad_perm [1,0,3,2]
    if constexpr (L == 32) {
        const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    }
    return v;
}

template <int N, int DT, int L, bool POST>
__global__ __launch_bounds__(64) void hc_colchunk_partials_kernel(
    int d, int T, const void *__restrict__ X, const float *__restrict__ coeffs_prev,
    const void *__restrict__ layer_out, const uint16_t *__restrict__ W, void *X_out,
    float *__restrict__ ws) {
    constexpr int V = StateVec<DT>::V;
    constexpr int M = n_logits(N);
    constexpr int RG = 64 / L;                 // row groups
    constexpr int RPW = (M + RG - 1) / RG;     // fn rows per group
    const int lane = threadIdx.x;
    const int grp = lane / L, cl = lane % L;
    const int row0 = grp * RPW;
    const bool ss_group = grp == RG - 1;
    const size_t K = (size_t)N * d;
    const int c0 = (blockIdx.y * L + cl) * V;
    const bool ok = c0 < d;
    const int cs = ok ? c0 : 0;                // in-bounds column for every lane
    const int tbase = blockIdx.x * SPLITK_TOKENS;

    // The (next site's) weights for this lane's rows and columns, loaded once
    // for all tokens of the group and first of all: they do not depend on the
    // post update, so their round trip overlaps that of the state and the
    // previous coefficients instead of following it (T = 1, d = 4096: the
    // weight loads used to be issued only after the post update, itself after
    // four dependent loads of the coefficients). Rows past M (last group when 4
    // does not divide M) read row M - 1 and are never stored; lanes past d read
    // column 0 and use zero weights.
    HalfVec<V> w[N][RPW];
#pragma unroll
    for (int i = 0; i < N; ++i)
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
            const int j = min(row0 + r, M - 1);
            w[i][r] = load_half_vec<V>(W + (size_t)j * K + (size_t)i * d + cs);
            if (!ok) w[i][r].raw = {};
        }

#pragma unroll
    for (int tt = 0; tt < SPLITK_TOKENS; ++tt) {
        const int t = tbase + tt;
        if (t >= T) break;  // uniform across the wavefront
        // (the previous site's coefficients,) the state (and layer_out): all
        // loads issued together, before the first store
        float cp[M];
        StateVec<DT> lv;
        if constexpr (POST) {
#pragma unroll
            for (int j = 0; j < M; ++j) cp[j] = coeffs_prev[(size_t)t * M + j];
        }
        StateVec<DT> xin[N];
#pragma unroll
        for (int i = 0; i < N; ++i) xin[i] = load_vec<DT>(X, (size_t)t * K + (size_t)i * d + cs);
        if constexpr (POST) lv = load_vec<DT>(layer_out, (size_t)t * d + cs);
        float x[N][V];
        float acc[RPW + 1];
#pragma unroll
        for (int j = 0; j <= RPW; ++j) acc[j] = 0.f;
        if constexpr (!POST) {
            // lanes past d contribute zeros
#pragma unroll
            for (int i = 0; i < N; ++i)
#pragma unroll
                for (int e = 0; e < V; ++e) x[i][e] = ok ? vec_get<DT>(xin[i], e) : 0.f;
        }
#pragma unroll
        for (int i = 0; i < N && POST; ++i) {
            float o[V];
#pragma unroll
            for (int e = 0; e < V; ++e) {
                float s = cp[2 * N + i * N] * vec_get<DT>(xin[0], e);
#pragma unroll
                for (int j = 1; j < N; ++j) s = fmaf(cp[2 * N + i * N + j], vec_get<DT>(xin[j], e), s);
                o[e] = fmaf(cp[N + i], vec_get<DT>(lv, e), s);
            }
            // (the row groups read X in the same instruction: group 0's
            // store cannot overtake another group's load)
            if (ok && grp == 0) store_vec<DT>(X_out, (size_t)t * K + (size_t)i * d + c0, o);
            // the next site sees X' as stored (rounded to the state type);
            // lanes past d contribute zeros
#pragma unroll
            for (int e = 0; e < V; ++e) {
                float v;
                if constexpr (DT == DT_F32)
                    v = o[e];
                else
                    v = bf16_lo(f32_to_bf16_bits(o[e]));
                x[i][e] = ok ? v : 0.f;
            }
        }
#pragma unroll
        for (int i = 0; i < N; ++i) {
#pragma unroll
            for (int r = 0; r < RPW; ++r)
#pragma unroll
                for (int e = 0; e < V; ++e) acc[r] = fmaf(half_get<V>(w[i][r], e), x[i][e], acc[r]);
#pragma unroll
            for (int e = 0; e < V; ++e) acc[RPW] = fmaf(x[i][e], x[i][e], acc[RPW]);
        }
#pragma unroll
        for (int j = 0; j <= RPW; ++j) acc[j] = chunk_sum<L>(acc[j]);
        float *out = ws + ((size_t)blockIdx.y * T + t) * (M + 1);
        if (cl < RPW && row0 + cl < M) {
            float v = acc[0];
#pragma unroll
            for (int j = 1; j < RPW; ++j)
                if (cl == j) v = acc[j];
            out[row0 + cl] = v;
        }
        if (ss_group && cl == L - 1) out[M] = acc[RPW];
    }
}

// ---------------------------------------------------------------------------
// Split-K finish: grid (T, ceil(d / (64*V))), one wavefront. Combines the P
// partials of token t in chunk order (PB loads in flight: 64 takes the 64
// chunks of the decode pre at d = 4096 fp32 in one round, 8.08 -> 7.95 us at
// T = 1; the one-pass chain step, with 32 chunks, is 0.2 us slower with the
// larger batch's registers and keeps 32), computes logits, gates and Sinkhorn,
// then the pre-mix (and post update) of 64*V columns.
// ---------------------------------------------------------------------------
template <int N, int DT, int MODE, int PB = 64>
__global__ __launch_bounds__(64) void hc_finish_kernel(
    int d, int kfull, int T, int P, float eps, int iters, const void *__restrict__ X,
    const float *__restrict__ bias, const float *__restrict__ ws, const void *__restrict__ layer_out,
    void *__restrict__ layer_in, float *__restrict__ coeffs, float *__restrict__ logits, void *X_out) {
    constexpr int V = StateVec<DT>::V;
    constexpr int M = n_logits(N);
    const int lane = threadIdx.x;
    const size_t t = blockIdx.x;
    const size_t K = (size_t)N * d;
    __shared__ float cf[M];

    // This lane's columns of X (and layer_out) for pass 2, loaded first: at
    // decode sizes the kernel is latency-bound, and these loads then overlap
    // the partial sums and the Sinkhorn instead of following them.
    const int c0 = (blockIdx.y * 64 + lane) * V;
    const bool col_ok = c0 < d;
    StateVec<DT> xs[N], lvs;
    if (col_ok) {
#pragma unroll
        for (int i = 0; i < N; ++i) xs[i] = load_vec<DT>(X, t * K + (size_t)i * d + c0);
        if constexpr (MODE == MODE_FUSED) lvs = load_vec<DT>(layer_out, t * d + c0);
    }

    // the partials were written by other CUs: each batch is a trip past this
    // XCD's L2
    float tot = 0.f;
    if (lane <= M) tot = sum_chunks<PB>(ws + t * (M + 1) + lane, (size_t)T * (M + 1), P);
    const float ssum = __shfl(tot, M, 64);
    const float r = sqrtf(ssum / (float)kfull + eps);  // kfull: all n*d columns, also when X is a share
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
    const float h = sinkhorn_lane_dpp<N>(zr, iters);
    if (lane < N * N) {
        cf[2 * N + lane] = h;
        if (writer && coeffs) coeffs[t * M + 2 * N + lane] = h;
    }
    __syncthreads();

    if (!col_ok) return;
    float x[N][V];
#pragma unroll
    for (int i = 0; i < N; ++i)
#pragma unroll
        for (int e = 0; e < V; ++e) x[i][e] = vec_get<DT>(xs[i], e);
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
#pragma unroll
        for (int i = 0; i < N; ++i) {
            float o[V];
#pragma unroll
            for (int e = 0; e < V; ++e) {
                float s = cf[2 * N + i * N] * x[0][e];
#pragma unroll
                for (int j = 1; j < N; ++j) s = fmaf(cf[2 * N + i * N + j], x[j][e], s);
                o[e] = fmaf(cf[N + i], vec_get<DT>(lvs, e), s);
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
    const float h = sinkhorn_lane_dpp<N>(z, iters);
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

// Compute units of the current device, looked up once per device.
static hipError_t device_cu_count(int *cus) {
    static std::atomic<int> cache[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < 64) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) {
            *cus = c;
            return hipSuccess;
        }
    }
    int c = 0;
    e = hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (c <= 0) return hipErrorInvalidDevice;
    if (dev >= 0 && dev < 64) cache[dev].store(c, std::memory_order_relaxed);
    *cus = c;
    return hipSuccess;
}

// Scratch of the entry point that allocates nothing (ds4hc_post_pre_noalloc):
// a file-scope device array, one copy on every device the library runs on,
// held until the process ends. In host code `scratch` names a host-side
// stand-in, not device memory: kernels and copies get the address that
// hipGetSymbolAddress returns for the current device, looked up once per
// device and kept.
static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

hipError_t noalloc_scratch(void **ptr) {
    static std::atomic<void *> cache[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    void *p = cache[dev].load(std::memory_order_acquire);
    if (!p) {
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        cache[dev].store(p, std::memory_order_release);
    }
    *ptr = p;
    return hipSuccess;
}

template <int N, int DT, int MODE>
static hipError_t launch_tile_n(int cs, const FusedArgs &a, hipStream_t s) {
    // Persistent: one workgroup per compute unit (the weight ring takes most
    // of a CU's LDS, so no second one would fit), each striding over tiles.
    int cus = 0;
    const hipError_t e = device_cu_count(&cus);
    if (e != hipSuccess) return e;
    const int64_t ntiles = (a.T + TILE_TOKENS - 1) / TILE_TOKENS;
    const dim3 grid((unsigned)(ntiles < cus ? ntiles : cus)), block(TILE_THREADS);
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

// Column-chunk partials of X (POST = false) into the workspace: P chunks of L lanes.
template <int N, int DT, int L>
static hipError_t launch_colchunk_pre(const FusedArgs &a, int P, hipStream_t s) {
    const dim3 g1((unsigned)((a.T + SPLITK_TOKENS - 1) / SPLITK_TOKENS), (unsigned)P);
    return launch_kernel(hc_colchunk_partials_kernel<N, DT, L, false>, g1, dim3(64), s, a.d, (int)a.T, a.X,
                         (const float *)nullptr, (const void *)nullptr, a.W, (void *)nullptr, a.ws);
}

// Split-K HC-pre / fused: the column-chunk partials, then the finish kernel,
// which sums the P partials (PB = 64 in flight for the up to 64 chunks of
// 16-lane chunking, 32 otherwise) and runs gates, Sinkhorn and pass 2.
template <int N, int DT, int MODE, int L>
static hipError_t launch_splitk_nl(const FusedArgs &a, hipStream_t s) {
    constexpr int V = StateVec<DT>::V;
    const int P = colchunk_chunks(a.d, DT);
    hipError_t e = launch_colchunk_pre<N, DT, L>(a, P, s);
    if (e != hipSuccess) return e;
    const dim3 g2((unsigned)a.T, (unsigned)((a.d + 64 * V - 1) / (64 * V)));
    return launch_kernel(hc_finish_kernel<N, DT, MODE, L == 16 ? 64 : 32>, g2, dim3(64), s, a.d, N * a.d,
                         (int)a.T, P, a.eps, a.iters, a.X, a.bias, (const float *)a.ws, a.layer_out,
                         a.layer_in, a.coeffs, a.logits, a.X_out);
}

// Split-K where splitk_streams(T, K): the streamed 16-token MFMA partials
// over stream_chunks column chunks (the weight read once per 16 tokens instead
// of once per 4), then the same finish kernel.
template <int N, int DT, int MODE>
static hipError_t launch_splitk_stream(const FusedArgs &a, hipStream_t s) {
    constexpr int V = StateVec<DT>::V;
    const int K = N * a.d;
    const int P = stream_chunks(a.T, K);
    const int KC = stream_chunk_cols(a.T, K);
    const dim3 g1((unsigned)((a.T + SP_TOKENS - 1) / SP_TOKENS), (unsigned)P);
    hipError_t e = launch_kernel(hc_stream_partials_kernel<N, DT>, g1, dim3(SP_WAVES * 64), s, K, KC, (int)a.T,
                                 a.X, a.W, (float *)a.ws);
    if (e != hipSuccess) return e;
    const dim3 g2((unsigned)a.T, (unsigned)((a.d + 64 * V - 1) / (64 * V)));
    return launch_kernel(hc_finish_kernel<N, DT, MODE, 64>, g2, dim3(64), s, a.d, K, (int)a.T, P, a.eps,
                         a.iters, a.X, a.bias, (const float *)a.ws, a.layer_out, a.layer_in, a.coeffs, a.logits,
                         a.X_out);
}

template <int N, int DT, int MODE>
static hipError_t launch_splitk_n(const FusedArgs &a, hipStream_t s) {
    if (splitk_streams(a.T, (int64_t)N * a.d)) return launch_splitk_stream<N, DT, MODE>(a, s);
    return colchunk_lanes(a.d, DT) == 16 ? launch_splitk_nl<N, DT, MODE, 16>(a, s)
                                         : launch_splitk_nl<N, DT, MODE, 32>(a, s);
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
    const int steps = (d + 16 * V - 1) / (16 * V);
    return (steps + TILE_WAVES - 1) / TILE_WAVES;
}

int tile_max_steps() { return 8; }

hipError_t launch_hc(const FusedArgs &a, bool fused, int path, hipStream_t s) {
    switch (a.n) {
    case 1: return dispatch_dt<1>(a.dt, fused, path, a, s);
    case 2: return dispatch_dt<2>(a.dt, fused, path, a, s);
    case 4: return dispatch_dt<4>(a.dt, fused, path, a, s);
    default: return hipErrorInvalidValue;
    }
}

// The finish kernel sums the P2 chunk partials (PB = 64 in flight for the up
// to 64 chunks of 16-lane chunking, 32 otherwise); the pre-mix reads X' back
// from X_out, with no post update there, 64 * V columns per workgroup.
template <int N, int DT, int L>
static hipError_t launch_post_pre_nl(const FusedArgs &a, const float *coeffs_prev, hipStream_t s) {
    constexpr int V = StateVec<DT>::V;
    const int P2 = colchunk_chunks(a.d, DT);
    const dim3 g1((unsigned)((a.T + SPLITK_TOKENS - 1) / SPLITK_TOKENS), (unsigned)P2);
    hipError_t e = launch_kernel(hc_colchunk_partials_kernel<N, DT, L, true>, g1, dim3(64), s, a.d, (int)a.T,
                                 a.X, coeffs_prev, a.layer_out, a.W, a.X_out, a.ws);
    if (e != hipSuccess) return e;
    const dim3 g2((unsigned)a.T, (unsigned)((a.d + 64 * V - 1) / (64 * V)));
    return launch_kernel(hc_finish_kernel<N, DT, MODE_PRE, L == 16 ? 64 : 32>, g2, dim3(64), s, a.d, N * a.d,
                         (int)a.T, P2, a.eps, a.iters, (const void *)a.X_out, a.bias, (const float *)a.ws,
                         (const void *)nullptr, a.layer_in, a.coeffs, a.logits, (void *)nullptr);
}

template <int N, int DT>
static hipError_t launch_post_pre_n(const FusedArgs &a, const float *coeffs_prev, hipStream_t s) {
    return colchunk_lanes(a.d, DT) == 16 ? launch_post_pre_nl<N, DT, 16>(a, coeffs_prev, s)
                                         : launch_post_pre_nl<N, DT, 32>(a, coeffs_prev, s);
}

int colchunk_lanes(int d, int dt) {
    const int V = dt == DT_F32 ? 4 : 8;
    return (d + 16 * V - 1) / (16 * V) <= 64 ? 16 : 32;
}

// Column chunks of the streamed split-K partials: about 512 workgroups (two
// per CU) over ceil(T / 16) token groups, each chunk a multiple of 256
// columns (one 32-column step per wave), at most 64 chunks.
int stream_chunk_cols(int64_t T, int K) {
    const int64_t groups = (T + SP_TOKENS - 1) / SP_TOKENS;
    int64_t want = (512 + groups - 1) / groups;
    if (want < 1) want = 1;
    if (want > 64) want = 64;
    int64_t kc = (K + want - 1) / want;
    kc = (kc + 255) / 256 * 256;
    return (int)kc;
}

int stream_chunks(int64_t T, int K) {
    const int kc = stream_chunk_cols(T, K);
    return (K + kc - 1) / kc;
}

int colchunk_chunks(int d, int dt) {
    const int V = dt == DT_F32 ? 4 : 8;
    const int L = colchunk_lanes(d, dt);
    return (d + L * V - 1) / (L * V);
}

hipError_t launch_post_pre(const FusedArgs &a, const float *coeffs_prev, bool one_pass, int path,
                           hipStream_t s) {
    if (!one_pass) {
        // post then pre on X' (two passes over the state)
        hipError_t e = launch_post(a.n, a.dt, a.d, a.T, a.X, coeffs_prev, a.layer_out, a.X_out, s);
        if (e != hipSuccess) return e;
        FusedArgs b = a;
        b.X = a.X_out;
        b.layer_out = nullptr;
        return launch_hc(b, false, path, s);
    }
#define DS4HC_PP(NN)                                                                             \
    return a.dt == DT_F32 ? launch_post_pre_n<NN, DT_F32>(a, coeffs_prev, s)                     \
                          : launch_post_pre_n<NN, DT_BF16>(a, coeffs_prev, s)
    switch (a.n) {
    case 1: DS4HC_PP(1);
    case 2: DS4HC_PP(2);
    case 4: DS4HC_PP(4);
    }
#undef DS4HC_PP
    return hipErrorInvalidValue;
}

template <int N, int DT>
static hipError_t launch_partials_n(const FusedArgs &a, int path, hipStream_t s) {
    if (path == PATH_TILE) return launch_tile_n<N, DT, MODE_PARTIALS>(tile_steps(a.d, DT), a, s);
    if (path == PATH_STREAM)
        return launch_kernel(hc_stream_partials_kernel<N, DT>,
                             dim3((unsigned)((a.T + SP_TOKENS - 1) / SP_TOKENS)), dim3(SP_WAVES * 64), s,
                             N * a.d, N * a.d, (int)a.T, a.X, a.W, a.logits);
    const int P = colchunk_chunks(a.d, DT);
    const hipError_t e = colchunk_lanes(a.d, DT) == 16 ? launch_colchunk_pre<N, DT, 16>(a, P, s)
                                                       : launch_colchunk_pre<N, DT, 32>(a, P, s);
    if (e != hipSuccess) return e;
    return launch_kernel(hc_chunk_sum_kernel<N>, dim3((unsigned)a.T), dim3(64), s, (int)a.T, P,
                         (const float *)a.ws, a.logits);
}

hipError_t launch_partials(const FusedArgs &a, int path, hipStream_t s) {
#define DS4HC_PA(NN)                                                                             \
    return a.dt == DT_F32 ? launch_partials_n<NN, DT_F32>(a, path, s)                            \
                          : launch_partials_n<NN, DT_BF16>(a, path, s)
    switch (a.n) {
    case 1: DS4HC_PA(1);
    case 2: DS4HC_PA(2);
    case 4: DS4HC_PA(4);
    }
#undef DS4HC_PA
    return hipErrorInvalidValue;
}

template <int N, int DT>
static hipError_t launch_combine_n(const FusedArgs &a, int d_total, int G, const float *partials,
                                   hipStream_t s) {
    constexpr int V = StateVec<DT>::V;
    const dim3 g2((unsigned)a.T, (unsigned)((a.d + 64 * V - 1) / (64 * V)));
    return launch_kernel(hc_finish_kernel<N, DT, MODE_FUSED>, g2, dim3(64), s, a.d, N * d_total,
                         (int)a.T, G, a.eps, a.iters, a.X, a.bias, partials, a.layer_out,
                         a.layer_in, a.coeffs, a.logits, a.X_out);
}

hipError_t launch_combine(const FusedArgs &a, int d_total, int G, const float *partials,
                          hipStream_t s) {
#define DS4HC_CO(NN)                                                                             \
    return a.dt == DT_F32 ? launch_combine_n<NN, DT_F32>(a, d_total, G, partials, s)             \
                          : launch_combine_n<NN, DT_BF16>(a, d_total, G, partials, s)
    switch (a.n) {
    case 1: DS4HC_CO(1);
    case 2: DS4HC_CO(2);
    case 4: DS4HC_CO(4);
    }
#undef DS4HC_CO
    return hipErrorInvalidValue;
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
