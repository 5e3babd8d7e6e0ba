// moe_device.h -- device-side helpers shared by the libmoe kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- bf16 bits

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float(((uint32_t)h) << 16);
}

// fp32 -> bf16 with gfx950's converter (v_cvt_pk_bf16_f32, two values per
// instruction): round to nearest even, NaN stays NaN.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return (uint16_t)(pack_bf16x2(f, 0.0f) & 0xffffu);
}

// ---------------------------------------------------------------- E4M3FN
//
// OCP E4M3FN: sign, 4 exponent bits (bias 7), 3 mantissa bits; largest finite
// 448; smallest normal 2^-6; subnormals m * 2^-9.  Encoding of values already
// clamped to [-448, 448] with gfx950's converter (v_cvt_pk_fp8_f32: OCP
// E4M3, round to nearest even, subnormals kept, the sign kept on zero).
__device__ __forceinline__ uint32_t e4m3_encode4(float a, float b, float c, float d) {
    int r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    r = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
    return (uint32_t)r;
}
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v, 0.0f, 0, false) & 0xffu;
}

__device__ __forceinline__ float e4m3_decode(uint32_t c) {
    uint32_t e = (c >> 3) & 0xfu, m = c & 7u;
    float v = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
    return (c & 0x80u) ? -v : v;
}

// quantise one value with its tile scale: clamp(v/scale) to +-448, nearest-even
__device__ __forceinline__ uint32_t quant_e4m3(float v, float scale) {
    if (scale == 0.0f) return 0u;
    float t = v / scale;                    // IEEE fp32 divide
    t = fminf(fmaxf(t, -448.0f), 448.0f);
    return e4m3_encode(t);
}

// ---------------------------------------------------------------- misc

__host__ __device__ constexpr int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace moe

namespace moe {

// inclusive prefix sum over a 256-thread block; every thread must call it
__device__ __forceinline__ int32_t block_incl_scan_256(int32_t v, int32_t* sh_wave4) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int32_t u = __shfl_up(v, o, 64);
        if (lane >= o) v += u;
    }
    if (lane == 63) sh_wave4[w] = v;
    __syncthreads();
    int32_t add = 0;
    for (int i = 0; i < w; ++i) add += sh_wave4[i];
    __syncthreads();
    return v + add;
}

}  // namespace moe
