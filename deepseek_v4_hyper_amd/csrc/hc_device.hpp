// hc_device.hpp -- device-side building blocks of the HC op for gfx950
// (wave64). Storage types, 16-byte vector loads/stores, wavefront
// reductions and the register-resident Sinkhorn.
//
// The Sinkhorn follows the design point of lucebox-hub PR #494 "fix(ds4):
// keep ROCmFPX generation byte-safe" (comment on the Sinkhorn kernel
// specialised for NHC = 4): the generic kernel spilled its matrix to scratch
// memory (95 us per launch), the unrolled NHC = 4 kernel kept it in registers
// (5.3 us). Here one lane holds one matrix entry, so the whole n x n matrix
// lives in n*n lanes of a wavefront and row/column sums are lane shuffles.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ds4hc {

enum : int { DT_F32 = 0, DT_BF16 = 1 };

constexpr int n_logits(int n) { return 2 * n + n * n; }

// One 16-byte vector of state elements: 4 float32 or 8 bfloat16.
template <int DT> struct StateVec;
template <> struct StateVec<DT_F32> {
    static constexpr int V = 4;
    float4 raw;
};
template <> struct StateVec<DT_BF16> {
    static constexpr int V = 8;
    uint4 raw;
};

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

// float32 -> bfloat16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

// Two float32 -> one word of two bfloat16 (a in the low half), each rounded to
// nearest even: the same bits as two f32_to_bf16_bits, but one
// v_cvt_pk_bf16_f32 instead of two conversions, a shift and an or.
__device__ __forceinline__ uint32_t f32x2_to_bf16x2_bits(float a, float b) {
    typedef float f2_t __attribute__((ext_vector_type(2)));
    typedef __bf16 b2_t __attribute__((ext_vector_type(2)));
    const f2_t f = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, b2_t));
}

__device__ __forceinline__ float f16_lo(uint32_t u) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(u & 0xFFFFu));
}
__device__ __forceinline__ float f16_hi(uint32_t u) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(u >> 16));
}

template <int DT>
__device__ __forceinline__ StateVec<DT> load_vec(const void *base, size_t elem_off) {
    StateVec<DT> v;
    if constexpr (DT == DT_F32)
        v.raw = *reinterpret_cast<const float4 *>(static_cast<const float *>(base) + elem_off);
    else
        v.raw = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(base) + elem_off);
    return v;
}

template <int DT>
__device__ __forceinline__ StateVec<DT> zero_vec() {
    StateVec<DT> v;
    if constexpr (DT == DT_F32)
        v.raw = make_float4(0.f, 0.f, 0.f, 0.f);
    else
        v.raw = make_uint4(0u, 0u, 0u, 0u);
    return v;
}

// Element e of a vector, widened to float32 (exact).
template <int DT>
__device__ __forceinline__ float vec_get(const StateVec<DT> &v, int e) {
    if constexpr (DT == DT_F32) {
        return e == 0 ? v.raw.x : e == 1 ? v.raw.y : e == 2 ? v.raw.z : v.raw.w;
    } else {
        const uint32_t w = e < 2 ? v.raw.x : e < 4 ? v.raw.y : e < 6 ? v.raw.z : v.raw.w;
        return (e & 1) ? bf16_hi(w) : bf16_lo(w);
    }
}

// Store V float32 values as one 16-byte vector of the state type (one RNE rounding).
template <int DT>
__device__ __forceinline__ void store_vec(void *base, size_t elem_off, const float *f) {
    if constexpr (DT == DT_F32) {
        *reinterpret_cast<float4 *>(static_cast<float *>(base) + elem_off) =
            make_float4(f[0], f[1], f[2], f[3]);
    } else {
        uint4 u;
        u.x = f32x2_to_bf16x2_bits(f[0], f[1]);
        u.y = f32x2_to_bf16x2_bits(f[2], f[3]);
        u.z = f32x2_to_bf16x2_bits(f[4], f[5]);
        u.w = f32x2_to_bf16x2_bits(f[6], f[7]);
        *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(base) + elem_off) = u;
    }
}

// W row slice of V float16 values (8 or 16 bytes), kept packed.
template <int V> struct HalfVec;
template <> struct HalfVec<4> { uint2 raw; };
template <> struct HalfVec<8> { uint4 raw; };

template <int V>
__device__ __forceinline__ HalfVec<V> load_half_vec(const uint16_t *p) {
    HalfVec<V> h;
    if constexpr (V == 4)
        h.raw = *reinterpret_cast<const uint2 *>(p);
    else
        h.raw = *reinterpret_cast<const uint4 *>(p);
    return h;
}

template <int V>
__device__ __forceinline__ float half_get(const HalfVec<V> &h, int e) {
    uint32_t w;
    if constexpr (V == 4)
        w = e < 2 ? h.raw.x : h.raw.y;
    else
        w = e < 2 ? h.raw.x : e < 4 ? h.raw.y : e < 6 ? h.raw.z : h.raw.w;
    return (e & 1) ? f16_hi(w) : f16_lo(w);
}

// Lane exchange by DPP control CTRL (only quad permutations and row rotations
// are used: every lane has a valid source). bound_ctrl is set so that the
// compiler folds the move into the instruction that consumes it (v_add_f32
// with a DPP source operand, one instruction instead of two on the serial
// chains of the reductions and the Sinkhorn); with every source valid it
// changes no value.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    static_assert((CTRL >= 0x00 && CTRL <= 0xFF) || (CTRL >= 0x121 && CTRL <= 0x12F),
                  "quad permutations and row rotations only");
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

// Sum over the 64 lanes of a wavefront, entirely in the VALU: quad butterflies
// (lane ^ 1, lane ^ 2), then the quads of a 16-lane row (rotations by 8, then
// 4), then the gfx950 row swaps (rows 0<->1 and 2<->3, then the halves). Each
// step adds the same two partial sums in every lane that receives them, so
// every lane ends with the same bits.
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp_mov<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp_mov<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp_mov<0x128>(v);  // row_ror:8
    v += dpp_mov<0x124>(v);  // row_ror:4
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Register-resident Sinkhorn. Lanes form groups of N*N; lane l of a group
// holds Z[i][j] with i = (l % N^2) / N, j = l % N. All 64 lanes must call it.
// Returns H[i][j] after: M = exp(Z - rowmax Z), then `iters` x (divide by row
// sums, then by column sums). The lane exchanges are DPP (no LDS crossbar
// traffic): row reductions (over j) are xor butterflies inside a quad; column
// reductions (over i) for n = 4 rotate the 16-lane row by 8 and then 4 lanes.
// Every lane of a row (column) ends with the same sum bits.
//
// Each normalisation multiplies by the hardware reciprocal of the sum
// (v_rcp_f32, within 1 ulp) instead of dividing: the 40 normalisations of a
// 20-iteration Sinkhorn are one serial chain, and the IEEE division sequence
// (scale, reciprocal, Newton steps, fix-up) made up most of its latency. The
// error stays a few float32 ulps of each entry; sums of powers of two (the
// uniform and permutation cases) are still exact. A product with the
// reciprocal can exceed 1 by an ulp where an entry is its whole row or column
// sum (a quotient cannot), so the result is clamped to 1; the comparison keeps
// NaN as NaN. No contraction here: fused into the next sum, a lane's own
// product would enter it unrounded while its partners' entered rounded, and
// the lanes of a row or column would no longer hold the same sum bits.
template <int N>
__device__ __forceinline__ float sinkhorn_lane_dpp(float z, int iters) {
#pragma clang fp contract(off)
    static_assert(N == 1 || N == 2 || N == 4, "n_hc");
    if constexpr (N == 1) {
        float m = expf(z - z);
        for (int it = 0; it < iters; ++it) {
            m = m * __builtin_amdgcn_rcpf(m);
            m = m * __builtin_amdgcn_rcpf(m);
        }
        return m;
    } else {
        constexpr int XOR1 = 0xB1, XOR2 = 0x4E, ROR4 = 0x124, ROR8 = 0x128;
        float mx = z;
        mx = fmaxf(mx, dpp_mov<XOR1>(mx));
        if constexpr (N == 4) mx = fmaxf(mx, dpp_mov<XOR2>(mx));
        float m = expf(z - mx);
        for (int it = 0; it < iters; ++it) {
            float rs = m + dpp_mov<XOR1>(m);
            if constexpr (N == 4) rs = rs + dpp_mov<XOR2>(rs);
            m = m * __builtin_amdgcn_rcpf(rs);
            float cs;
            if constexpr (N == 4) {
                // rows i and i+2 first: then every lane of a column adds the
                // same two partial sums, so all four hold identical bits.
                cs = m + dpp_mov<ROR8>(m);
                cs = cs + dpp_mov<ROR4>(cs);
            } else {
                cs = m + dpp_mov<XOR2>(m);
            }
            m = m * __builtin_amdgcn_rcpf(cs);
        }
        return m > 1.0f ? 1.0f : m;
    }
}

__device__ __forceinline__ float logistic(float v) { return 1.0f / (1.0f + expf(-v)); }

}  // namespace ds4hc
