// Layer norm of the grouped token rows, the first step of each feed-forward
// block of an expert (BASE layers, sec. 4.1: layer norm, projection up,
// activation, projection back, residual connection).
//
// One wave per row, grid-stride; statistics in fp32 with the population
// variance (mean first, then the centred sum of squares). For bf16 rows of up
// to 8192 elements the row stays in registers (R chunks of 8 values per lane),
// so HBM sees one read and one write of the row and the three passes cost no
// extra loads; other rows (fp32, or longer) are read three times, the second
// and third reads served from the caches.
#include "common.h"
#include "internal.h"

namespace base {

namespace {

BASE_DEV float wave_sum_f32(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

BASE_DEV void unpack8(const uint4 u, float (&f)[8]) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        f[2 * q] = __uint_as_float(w[q] << 16);
        f[2 * q + 1] = __uint_as_float(w[q] & 0xffff0000u);
    }
}

// bf16 rows held in registers: lane l owns the 8-element chunks l, l + 64,
// ..., l + 64 (R - 1) (chunk c covers columns 8c .. 8c + 7; D % 8 == 0 and
// D <= 512 R). gamma / beta rows are read as float4 (16-byte aligned).
template <int R>
__global__ __launch_bounds__(256) void layernorm_bf16_reg_kernel(
    const uint16_t* __restrict__ x, int gather, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ assign, const float* __restrict__ gamma,
    const float* __restrict__ beta, float eps, uint16_t* __restrict__ Y, int64_t T, int64_t E,
    int64_t D) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int64_t nw = ((int64_t)gridDim.x * blockDim.x) >> 6;
    const int nc = (int)(D / 8);
    const float inv_d = 1.0f / (float)D;
    for (int64_t r = wave; r < T; r += nw) {
        const int64_t t = perm[r];
        const int64_t src = gather ? t : r;
        int64_t e = assign[t];
        // an id outside [0, E) (a rejected given assignment, which the call
        // reports as unbalanced) reads expert 0's parameters
        if (e < 0 || e >= E) e = 0;
        const uint4* row = (const uint4*)(x + src * D);
        float v[R][8];
#pragma unroll
        for (int j = 0; j < R; ++j) {
            const int c = lane + 64 * j;
            const uint4 u = c < nc ? row[c] : make_uint4(0u, 0u, 0u, 0u);
            unpack8(u, v[j]);
        }
        float sum = 0.0f;
#pragma unroll
        for (int j = 0; j < R; ++j)
#pragma unroll
            for (int i = 0; i < 8; ++i) sum += v[j][i];
        const float mean = wave_sum_f32(sum) * inv_d;
        float ss = 0.0f;
#pragma unroll
        for (int j = 0; j < R; ++j) {
            if (lane + 64 * j < nc) {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float a = v[j][i] - mean;
                    ss = fmaf(a, a, ss);
                }
            }
        }
        const float rstd = 1.0f / sqrtf(wave_sum_f32(ss) * inv_d + eps);
        uint4* out = (uint4*)(Y + r * D);
        const float4* g4 = gamma ? (const float4*)(gamma + e * D) : nullptr;
        const float4* b4 = beta ? (const float4*)(beta + e * D) : nullptr;
#pragma unroll
        for (int j = 0; j < R; ++j) {
            const int c = lane + 64 * j;
            if (c < nc) {
                float y[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) y[i] = (v[j][i] - mean) * rstd;
                if (g4) {
                    const float4 ga = g4[2 * c], gb = g4[2 * c + 1];
                    y[0] *= ga.x; y[1] *= ga.y; y[2] *= ga.z; y[3] *= ga.w;
                    y[4] *= gb.x; y[5] *= gb.y; y[6] *= gb.z; y[7] *= gb.w;
                }
                if (b4) {
                    const float4 ba = b4[2 * c], bb = b4[2 * c + 1];
                    y[0] += ba.x; y[1] += ba.y; y[2] += ba.z; y[3] += ba.w;
                    y[4] += bb.x; y[5] += bb.y; y[6] += bb.z; y[7] += bb.w;
                }
                uint32_t o[4];
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    o[q] = (uint32_t)f32_to_bf16(y[2 * q]) | ((uint32_t)f32_to_bf16(y[2 * q + 1]) << 16);
                out[c] = make_uint4(o[0], o[1], o[2], o[3]);
            }
        }
    }
}

template <int DT>  // 0 fp32, 1 bf16
__global__ __launch_bounds__(256) void layernorm_kernel(const void* x, int gather,
                                                         const int32_t* perm,
                                                         const int32_t* assign,
                                                         const float* gamma, const float* beta,
                                                         float eps, void* Y, int64_t T, int64_t E,
                                                         int64_t D) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int64_t nw = ((int64_t)gridDim.x * blockDim.x) >> 6;
    for (int64_t r = wave; r < T; r += nw) {
        const int64_t t = perm[r];
        const int64_t src = gather ? t : r;
        // an id outside [0, E) (a rejected given assignment) reads expert 0's
        // parameters; the call reports the assignment as unbalanced anyway
        int64_t e = assign[t];
        if (e < 0 || e >= E) e = 0;
        const float* ga = gamma ? gamma + e * D : nullptr;
        const float* be = beta ? beta + e * D : nullptr;
        float sum = 0.0f, ss = 0.0f;
        if (DT == 1) {
            // 8 bf16 (16 bytes) per lane and chunk; D % 8 == 0
            const uint4* row = (const uint4*)((const uint16_t*)x + src * D);
            const int64_t nc = D / 8;
            for (int64_t c = lane; c < nc; c += 64) {
                const uint4 u = row[c];
                const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    sum += __uint_as_float(w[q] << 16) + __uint_as_float(w[q] & 0xffff0000u);
            }
            const float mean = wave_sum_f32(sum) / (float)D;
            for (int64_t c = lane; c < nc; c += 64) {
                const uint4 u = row[c];
                const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float a = __uint_as_float(w[q] << 16) - mean;
                    const float b = __uint_as_float(w[q] & 0xffff0000u) - mean;
                    ss = fmaf(a, a, fmaf(b, b, ss));
                }
            }
            const float rstd = 1.0f / sqrtf(wave_sum_f32(ss) / (float)D + eps);
            uint4* out = (uint4*)((uint16_t*)Y + r * D);
            for (int64_t c = lane; c < nc; c += 64) {
                const uint4 u = row[c];
                const uint32_t w[4] = {u.x, u.y, u.z, u.w};
                uint32_t o[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int64_t d = c * 8 + 2 * q;
                    float a = (__uint_as_float(w[q] << 16) - mean) * rstd;
                    float b = (__uint_as_float(w[q] & 0xffff0000u) - mean) * rstd;
                    if (ga) { a *= ga[d]; b *= ga[d + 1]; }
                    if (be) { a += be[d]; b += be[d + 1]; }
                    o[q] = (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
                }
                out[c] = make_uint4(o[0], o[1], o[2], o[3]);
            }
        } else {
            const float* row = (const float*)x + src * D;
            for (int64_t d = lane; d < D; d += 64) sum += row[d];
            const float mean = wave_sum_f32(sum) / (float)D;
            for (int64_t d = lane; d < D; d += 64) {
                const float a = row[d] - mean;
                ss = fmaf(a, a, ss);
            }
            const float rstd = 1.0f / sqrtf(wave_sum_f32(ss) / (float)D + eps);
            float* out = (float*)Y + r * D;
            for (int64_t d = lane; d < D; d += 64) {
                float a = (row[d] - mean) * rstd;
                if (ga) a *= ga[d];
                if (be) a += be[d];
                out[d] = a;
            }
        }
    }
}

}  // namespace

hipError_t launch_layernorm(const void* x, int gather, const int32_t* perm, const int32_t* assign,
                            const float* gamma, const float* beta, double eps, void* Y, int64_t T,
                            int64_t E, int64_t D, int dt, hipStream_t st) {
    if (T <= 0) return hipSuccess;
    int64_t blocks = (T + 3) / 4;  // 4 waves per block, one row each
    if (blocks > 65536) blocks = 65536;
    const bool a16 = ((uintptr_t)gamma & 15u) == 0 && ((uintptr_t)beta & 15u) == 0;
    if (dt != 0 && a16 && D <= 8192) {
        const int nc = (int)(D / 8);
        const int R = nc <= 64 ? 1 : nc <= 128 ? 2 : nc <= 256 ? 4 : nc <= 512 ? 8 : 16;
        const float fe = (float)eps;
        const uint16_t* xb = (const uint16_t*)x;
        uint16_t* yb = (uint16_t*)Y;
        const dim3 g((unsigned)blocks), b(256);
        switch (R) {
        case 1: hipLaunchKernelGGL(layernorm_bf16_reg_kernel<1>, g, b, 0, st, xb, gather, perm, assign, gamma, beta, fe, yb, T, E, D); break;
        case 2: hipLaunchKernelGGL(layernorm_bf16_reg_kernel<2>, g, b, 0, st, xb, gather, perm, assign, gamma, beta, fe, yb, T, E, D); break;
        case 4: hipLaunchKernelGGL(layernorm_bf16_reg_kernel<4>, g, b, 0, st, xb, gather, perm, assign, gamma, beta, fe, yb, T, E, D); break;
        case 8: hipLaunchKernelGGL(layernorm_bf16_reg_kernel<8>, g, b, 0, st, xb, gather, perm, assign, gamma, beta, fe, yb, T, E, D); break;
        default: hipLaunchKernelGGL(layernorm_bf16_reg_kernel<16>, g, b, 0, st, xb, gather, perm, assign, gamma, beta, fe, yb, T, E, D); break;
        }
        return hipGetLastError();
    }
    if (dt == 0)
        hipLaunchKernelGGL(layernorm_kernel<0>, dim3((unsigned)blocks), dim3(256), 0, st, x, gather,
                           perm, assign, gamma, beta, (float)eps, Y, T, E, D);
    else
        hipLaunchKernelGGL(layernorm_kernel<1>, dim3((unsigned)blocks), dim3(256), 0, st, x, gather,
                           perm, assign, gamma, beta, (float)eps, Y, T, E, D);
    return hipGetLastError();
}

}  // namespace base
