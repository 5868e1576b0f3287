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

// x from lane (lane ^ M), M a power of two: DPP quad permutes for 1 and 2,
// ds_swizzle (bit mode, within 32 lanes) for 4..16, ds_bpermute for 32.
template <int M>
__device__ __forceinline__ float xor_lane(float x) {
    const int v = __float_as_int(x);
    if constexpr (M == 1) return __int_as_float(__builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false));
    else if constexpr (M == 2) return __int_as_float(__builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false));
    else if constexpr (M < 32) return __int_as_float(__builtin_amdgcn_ds_swizzle(v, 0x1F | (M << 10)));
    else return __shfl_xor(x, 32, 64);
}

// sum / max over the lanes that differ in bits [log2 LO, log2 HI)
template <int LO, int HI>
__device__ __forceinline__ float lanes_sum(float x) {
    if constexpr (LO < HI) {
        x += xor_lane<LO>(x);
        return lanes_sum<LO * 2, HI>(x);
    } else {
        return x;
    }
}
template <int LO, int HI>
__device__ __forceinline__ float lanes_max(float x) {
    if constexpr (LO < HI) {
        x = fmaxf(x, xor_lane<LO>(x));
        return lanes_max<LO * 2, HI>(x);
    } else {
        return x;
    }
}

}  // namespace qv
