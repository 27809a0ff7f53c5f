// common.hpp -- small device/host helpers shared by the libpath_attn kernels.
// gfx950 only: 64-lane wavefronts, bf16 stored as raw 16-bit patterns.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// bf16 storage type: raw bits.  Conversions are explicit so the rounding is
// visible: float -> bf16 rounds to nearest even; NaN stays NaN.
struct bf16 {
    uint16_t bits;
};

__host__ __device__ inline float bf16_to_f32(bf16 x) {
    union { uint32_t u; float f; } c;
    c.u = (uint32_t)x.bits << 16;
    return c.f;
}

__host__ __device__ inline bf16 f32_to_bf16(float f) {
    union { uint32_t u; float f; } c;
    c.f = f;
    uint32_t u = c.u;
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) {
        bf16 r; r.bits = (uint16_t)((u >> 16) | 0x40u); return r;   // quiet NaN
    }
    u += 0x7fffu + ((u >> 16) & 1u);                                // nearest even
    bf16 r; r.bits = (uint16_t)(u >> 16); return r;
}

template <typename T> __device__ inline float to_f32(T x);
template <> __device__ inline float to_f32<float>(float x) { return x; }
template <> __device__ inline float to_f32<bf16>(bf16 x) { return bf16_to_f32(x); }

template <typename T> __device__ inline T from_f32(float x);
template <> __device__ inline float from_f32<float>(float x) { return x; }
template <> __device__ inline bf16 from_f32<bf16>(float x) { return f32_to_bf16(x); }

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

}  // namespace pa
