// Small device helpers shared by the QEvict kernels.
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qv {

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16, round to nearest even (finite inputs)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// float64 -> bf16 with a single round-to-nearest-even from the exact value:
// truncate to fp32, mark inexactness in the last bit (round to odd), then round
// fp32 -> bf16.  Round-to-odd with >= 2 spare bits makes the second rounding exact.
__device__ __forceinline__ uint16_t f64_to_bf16(double x) {
    float f = __double2float_rz(x);
    uint32_t u = __float_as_uint(f);
    if ((double)f != x) u |= 1u;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// largest fp16 value <= x / smallest fp16 value >= x, computed exactly in fp64
// (11 significant bits, subnormal quantum 2^-24).
__device__ __forceinline__ double fp16_round_down(double x) {
    if (x == 0.0) return 0.0;
    int e;
    frexp(x, &e);
    int q = e - 11 < -24 ? -24 : e - 11;
    return ldexp(floor(ldexp(x, -q)), q);
}
__device__ __forceinline__ double fp16_round_up(double x) {
    if (x == 0.0) return 0.0;
    int e;
    frexp(x, &e);
    int q = e - 11 < -24 ? -24 : e - 11;
    return ldexp(ceil(ldexp(x, -q)), q);
}
// bits of an fp16-representable double
__device__ __forceinline__ uint16_t fp16_bits_exact(double x) { return __half_as_ushort(__float2half((float)x)); }
__device__ __forceinline__ float fp16_bits_to_f32(uint16_t b) { return __half2float(__ushort_as_half(b)); }

template <typename T>
__device__ __forceinline__ T wave_xor(T v, int mask) {
    return __shfl_xor(v, mask, 64);
}

}  // namespace qv
