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

// address spaces for the direct global -> LDS loads (global_load_lds)
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

// ---- DPP cross-lane moves (a few cycles, no LDS crossbar). Lanes whose
// source is outside the row keep their own value.
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <- 7-i within 8
constexpr int kDppMirror = 0x140;     // lane i <- 15-i within 16
constexpr int kDppWaveShl1 = 0x130;   // lane i <- i+1 across the wave (lane 63: old value)
constexpr int kDppWaveShr1 = 0x138;   // lane i <- i-1 across the wave (lane 0: old value)
constexpr int kDppRowBcast0 = 0x150;  // every lane <- lane 0 of its row of 16
constexpr int kDppBcast15 = 0x142;    // row r <- lane 15 of row r-1 (rows in the row mask)
constexpr int kDppBcast31 = 0x143;    // rows 2, 3 <- lane 31 (rows in the row mask)

template <int CTRL>
BASE_DEV int dpp_i32(int v) {
    return __builtin_amdgcn_update_dpp(v, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
BASE_DEV double dpp_f64(double v) {
    long long x = __double_as_longlong(v);
    int lo = dpp_i32<CTRL>((int)(x & 0xffffffff));
    int hi = dpp_i32<CTRL>((int)(x >> 32));
    return __longlong_as_double((long long)(((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo));
}
// rows outside ROW_MASK keep v
template <int CTRL, int ROW_MASK>
BASE_DEV int dpp_rows_i32(int v) {
    return __builtin_amdgcn_update_dpp(v, v, CTRL, ROW_MASK, 0xF, false);
}
template <int CTRL, int ROW_MASK>
BASE_DEV double dpp_rows_f64(double v) {
    long long x = __double_as_longlong(v);
    int lo = dpp_rows_i32<CTRL, ROW_MASK>((int)(x & 0xffffffff));
    int hi = dpp_rows_i32<CTRL, ROW_MASK>((int)(x >> 32));
    return __longlong_as_double((long long)(((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo));
}
BASE_DEV int readlane_i32(int v, int l) { return __builtin_amdgcn_readlane(v, l); }
BASE_DEV double readlane_f64(double v, int l) {
    long long x = __double_as_longlong(v);
    int lo = __builtin_amdgcn_readlane((int)(x & 0xffffffff), l);
    int hi = __builtin_amdgcn_readlane((int)(x >> 32), l);
    return __longlong_as_double((long long)(((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo));
}
BASE_DEV int first_lane_i32(int v) { return __builtin_amdgcn_readfirstlane(v); }

// (value, index) pairs: a replaces b if larger, or equal with a lower index.
BASE_DEV void argmax_merge(double& v, int& i, double ov, int oi) {
    if (ov > v || (ov == v && oi < i)) { v = ov; i = oi; }
}
// Wave-wide argmax (lowest index among equal maxima); result is uniform.
BASE_DEV void wave_argmax_f64(double& v, int& i) {
    argmax_merge(v, i, dpp_f64<kDppXor1>(v), dpp_i32<kDppXor1>(i));
    argmax_merge(v, i, dpp_f64<kDppXor2>(v), dpp_i32<kDppXor2>(i));
    argmax_merge(v, i, dpp_f64<kDppHalfMirror>(v), dpp_i32<kDppHalfMirror>(i));
    argmax_merge(v, i, dpp_f64<kDppMirror>(v), dpp_i32<kDppMirror>(i));
    double bv = readlane_f64(v, 0);
    int bi = readlane_i32(i, 0);
    argmax_merge(bv, bi, readlane_f64(v, 16), readlane_i32(i, 16));
    argmax_merge(bv, bi, readlane_f64(v, 32), readlane_i32(i, 32));
    argmax_merge(bv, bi, readlane_f64(v, 48), readlane_i32(i, 48));
    v = bv;
    i = bi;
}
// Wave-wide max: reduce within each row of 16, then carry the row maxima up
// with row broadcasts; lane 63 ends with the maximum (returned uniform).
BASE_DEV double wave_max_f64(double v) {
    v = fmax(v, dpp_f64<kDppXor1>(v));
    v = fmax(v, dpp_f64<kDppXor2>(v));
    v = fmax(v, dpp_f64<kDppHalfMirror>(v));
    v = fmax(v, dpp_f64<kDppMirror>(v));
    v = fmax(v, dpp_rows_f64<kDppBcast15, 0xA>(v));
    v = fmax(v, dpp_rows_f64<kDppBcast31, 0xC>(v));
    return readlane_f64(v, 63);
}
BASE_DEV int wave_min_i32(int v) {
    v = min(v, dpp_i32<kDppXor1>(v));
    v = min(v, dpp_i32<kDppXor2>(v));
    v = min(v, dpp_i32<kDppHalfMirror>(v));
    v = min(v, dpp_i32<kDppMirror>(v));
    v = min(v, dpp_rows_i32<kDppBcast15, 0xA>(v));
    v = min(v, dpp_rows_i32<kDppBcast31, 0xC>(v));
    return readlane_i32(v, 63);
}

// Exact GELU x * Phi(x) = x/2 * (1 + erf(x / sqrt 2)), fp32.
BASE_DEV float gelu_erf(float x) { return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f)); }

BASE_DEV float sigmoid_f32(float x) { return 1.0f / (1.0f + expf(-x)); }

}  // namespace base
