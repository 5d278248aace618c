// Device helpers shared by the gfx950 kernels of libbase_layer.so.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define BASE_DEV __device__ __forceinline__

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));

namespace base {

constexpr int kWave = 64;

// bf16 <-> fp32 by bit manipulation (bf16 is the top half of an fp32).
BASE_DEV float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// fp32 -> bf16, round to nearest, ties to even; NaN stays a quiet NaN.
BASE_DEV uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return uint16_t(u >> 16);
}

// Order-preserving maps of floats to unsigned integers: a < b  <=>  key(a) < key(b)
// (for non-NaN values).
BASE_DEV uint32_t f32_key(float f) {
    uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
BASE_DEV float f32_unkey(uint32_t k) {
    uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
    return __uint_as_float(u);
}
BASE_DEV unsigned long long f64_key(double d) {
    unsigned long long u = (unsigned long long)__double_as_longlong(d);
    return (u & 0x8000000000000000ull) ? ~u : (u | 0x8000000000000000ull);
}

BASE_DEV bool is_finite_f32(float f) { return (__float_as_uint(f) & 0x7f800000u) != 0x7f800000u; }

// Wave-wide reductions (64 lanes) through shuffles.
BASE_DEV float wave_max_f32(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}
BASE_DEV float wave_min_f32(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fminf(v, __shfl_xor(v, o, kWave));
    return v;
}
BASE_DEV int wave_sum_i32(int v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}
BASE_DEV double shfl_xor_f64(double v, int o) {
    long long x = __double_as_longlong(v);
    int lo = int(x & 0xffffffff), hi = int(x >> 32);
    lo = __shfl_xor(lo, o, kWave);
    hi = __shfl_xor(hi, o, kWave);
    return __longlong_as_double((long long)(((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo));
}
BASE_DEV double shfl_f64(double v, int src) {
    long long x = __double_as_longlong(v);
    int lo = int(x & 0xffffffff), hi = int(x >> 32);
    lo = __shfl(lo, src, kWave);
    hi = __shfl(hi, src, kWave);
    return __longlong_as_double((long long)(((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo));
}
BASE_DEV double wave_min_f64(double v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmin(v, shfl_xor_f64(v, o));
    return v;
}

// Exact GELU x * Phi(x) = x/2 * (1 + erf(x / sqrt 2)), fp32.
BASE_DEV float gelu_erf(float x) { return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f)); }

BASE_DEV float sigmoid_f32(float x) { return 1.0f / (1.0f + expf(-x)); }

}  // namespace base
