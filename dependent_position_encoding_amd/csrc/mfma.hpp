// mfma.hpp -- gfx950 matrix-core helpers (v_mfma_f32_32x32x16_bf16).
//
// Operand layouts of the 32x32x16 bf16 instruction (lane l, h = l / 32):
//   A (32 x 16): lane holds row l % 32, k = 8h .. 8h+7
//   B (16 x 32): lane holds column l % 32, k = 8h .. 8h+7
//   C (32 x 32): lane holds column l % 32, register r = 4i + j holds
//                row 8i + 4h + j.
// A C tile read back as a B operand (the next product contracts over the C
// tile's rows) therefore sees its rows in the order "swap bits 2 and 3
// within each group of 16": k-slot s <-> row swap23(s).  Operands that are
// contracted against such a B are stored with the same permutation.
#pragma once
#include <hip/hip_runtime.h>

namespace pa {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ inline f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__host__ __device__ constexpr int swap23(int x) {
    return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1);
}

// C-tile register r of lane half h -> tile row.
__device__ constexpr int crow(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// 8 consecutive values as a bf16 operand; for float input also the residual
// lo = bf16(x - hi), so that hi + lo carries ~16 mantissa bits.
__device__ inline void ld8(const __bf16* p, bf16x8& hi, bf16x8& lo) {
    hi = *reinterpret_cast<const bf16x8*>(p);
    (void)lo;
}
__device__ inline void ld8(const float* p, bf16x8& hi, bf16x8& lo) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        hi[e] = (__bf16)a[e];
        lo[e] = (__bf16)(a[e] - (float)hi[e]);
        hi[e + 4] = (__bf16)b[e];
        lo[e + 4] = (__bf16)(b[e] - (float)hi[e + 4]);
    }
}

template <typename T> struct is_f32 { static constexpr bool value = false; };
template <> struct is_f32<float> { static constexpr bool value = true; };

// acc += A[m0:m0+32, 0:K] * Bn[n0:n0+32, 0:K]^T with A row-major (stride
// lda) and Bn holding B transposed (row n = column n of B, stride ldb), both
// in LDS.  float operands are split into bf16 hi + lo and the three
// significant partial products are accumulated (lo * lo is dropped), which
// gives close to fp32 accuracy; bf16 operands are exact and used once.
template <int K, typename TA, typename TB>
__device__ inline void tile_mm(f32x16& acc, const TA* A, int lda, const TB* Bn, int ldb,
                               int m0, int n0, int lane) {
    const int r = lane & 31, h = lane >> 5;
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += 16) {
        bf16x8 ah, al, bh, bl;
        ld8(A + (m0 + r) * lda + k0 + 8 * h, ah, al);
        ld8(Bn + (n0 + r) * ldb + k0 + 8 * h, bh, bl);
        acc = mfma32(ah, bh, acc);
        if constexpr (is_f32<TB>::value) acc = mfma32(ah, bl, acc);
        if constexpr (is_f32<TA>::value) acc = mfma32(al, bh, acc);
    }
}

// acc += A B for operands split into bf16 hi + lo parts: the three partial
// products that matter (lo * lo dropped), smallest first.
__device__ inline f32x16 mfma_split(const bf16x8& ah, const bf16x8& al, const bf16x8& bh,
                                    const bf16x8& bl, f32x16 acc) {
    acc = mfma32(ah, bl, acc);
    acc = mfma32(al, bh, acc);
    return mfma32(ah, bh, acc);
}

// float32 operands split three ways (hi + mid + lo, 8 mantissa bits each):
// acc += A * Bn^T with the six partial products that matter at fp32
// precision, smallest first.  Used where a long chain of d x d products must
// stay at fp32 accuracy.
__device__ inline void ld8_3(const float* p, bf16x8& hi, bf16x8& mid, bf16x8& lo) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float x = e < 4 ? a[e] : b[e - 4];
        hi[e] = (__bf16)x;
        const float r = x - (float)hi[e];
        mid[e] = (__bf16)r;
        lo[e] = (__bf16)(r - (float)mid[e]);
    }
}

template <int K>
__device__ inline void tile_mm_f32(f32x16& acc, const float* A, int lda, const float* Bn, int ldb,
                                   int m0, int n0, int lane) {
    const int r = lane & 31, h = lane >> 5;
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += 16) {
        bf16x8 ah, am, al, bh, bm, bl;
        ld8_3(A + (m0 + r) * lda + k0 + 8 * h, ah, am, al);
        ld8_3(Bn + (n0 + r) * ldb + k0 + 8 * h, bh, bm, bl);
        acc = mfma32(am, bm, acc);
        acc = mfma32(al, bh, acc);
        acc = mfma32(ah, bl, acc);
        acc = mfma32(am, bh, acc);
        acc = mfma32(ah, bm, acc);
        acc = mfma32(ah, bh, acc);
    }
}

// The two halves of a wave hold different key rows of the same query
// column (C layout).  v_permlane32_swap on two copies of x leaves x[lane] in
// one result and x[lane ^ 32] in the other, so these reduce over the pair
// without going through LDS.
__device__ inline float pair_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float pair_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Sum of the 32 bf16 probabilities a lane feeds to P.V (four bf16x8 operand
// registers), by paired dot products against ones with fp32 accumulation:
// the normaliser then adds exactly the weights the value product uses.
__device__ inline float sum_bf16x32(const bf16x8 (&p)[4]) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 one = {(__bf16)1.f, (__bf16)1.f};
    float s[2] = {0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < 4; ++kc)
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
            const bf16x2 two = {p[kc][e], p[kc][e + 1]};
            s[kc & 1] = __builtin_amdgcn_fdot2_f32_bf16(two, one, s[kc & 1], false);
        }
    return s[0] + s[1];
}

__device__ inline f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int e = 0; e < 16; ++e) z[e] = 0.f;
    return z;
}

}  // namespace pa
