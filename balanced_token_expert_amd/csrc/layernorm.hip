// Layer norm of the grouped token rows, the first step of each feed-forward
// block of an expert (BASE layers, sec. 4.1: layer norm, projection up,
// activation, projection back, residual connection).
//
// One wave per row, grid-stride. The row is read three times (sum, centred
// sum of squares, output); the second and third reads hit the CU's L1/L2, so
// HBM sees one read and one write of the row. Statistics in fp32 with the
// population variance.
#include "common.h"
#include "internal.h"

namespace base {

namespace {

BASE_DEV float wave_sum_f32(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
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
    if (blocks > 4096) blocks = 4096;
    if (dt == 0)
        hipLaunchKernelGGL(layernorm_kernel<0>, dim3((unsigned)blocks), dim3(256), 0, st, x, gather,
                           perm, assign, gamma, beta, (float)eps, Y, T, E, D);
    else
        hipLaunchKernelGGL(layernorm_kernel<1>, dim3((unsigned)blocks), dim3(256), 0, st, x, gather,
                           perm, assign, gamma, beta, (float)eps, Y, T, E, D);
    return hipGetLastError();
}

}  // namespace base
