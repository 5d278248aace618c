// Small kernels of the layer's backward pass (base_layer_backward). The
// assignment is held fixed: the affinities that chose the experts carry no
// gradient, and the centroids learn through the sigmoid gate only (BASE
// Layers sec. 3.1; the released code scores tokens under no_grad). With the
// logit l = h_t . w_e of a token's expert and g = sigma(l):
//   dl = g (1 - g) dg,  dg = dy . c (eq. 1) or dy . (c - h_t) (convex blend),
//   dh_t gets dl w_e,  dw_e = sum over its tokens of dl h_t.
// The expert products (and dy . c, accumulated in their epilogue as
// V . act(Z), V = W2^T dy) live in gemm.hip.
#include <initializer_list>

#include "common.h"
#include "internal.h"

namespace base {

namespace {

BASE_DEV float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

// one wave per row; 16-byte pieces when the row allows, else 4-byte words
__global__ __launch_bounds__(256) void gather2_kernel(const char* h, const char* dy,
                                                      const int32_t* perm, char* Xg, char* dYg,
                                                      int64_t T, int64_t rowbytes, int wide) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int64_t nw = ((int64_t)gridDim.x * blockDim.x) >> 6;
    for (int64_t r = wave; r < T; r += nw) {
        const int64_t t = perm[r];
        if (wide) {
            const int64_t n = rowbytes >> 4;
            const uint4* a = (const uint4*)(h + t * rowbytes);
            const uint4* b = (const uint4*)(dy + t * rowbytes);
            uint4* x = (uint4*)(Xg + r * rowbytes);
            uint4* y = (uint4*)(dYg + r * rowbytes);
            for (int64_t c = lane; c < n; c += 64) {
                x[c] = a[c];
                y[c] = b[c];
            }
        } else {
            const int64_t n = rowbytes >> 2;
            const uint32_t* a = (const uint32_t*)(h + t * rowbytes);
            const uint32_t* b = (const uint32_t*)(dy + t * rowbytes);
            uint32_t* x = (uint32_t*)(Xg + r * rowbytes);
            uint32_t* y = (uint32_t*)(dYg + r * rowbytes);
            for (int64_t c = lane; c < n; c += 64) {
                x[c] = a[c];
                y[c] = b[c];
            }
        }
    }
}

BASE_DEV int64_t group_of(const int32_t* goff, int64_t E, int64_t r) {
    int64_t lo = 0, hi = E;  // goff[lo] <= r < goff[hi]
    while (hi - lo > 1) {
        const int64_t mid = (lo + hi) >> 1;
        if (goff[mid] <= r) lo = mid;
        else hi = mid;
    }
    return lo;
}

template <int DT>
BASE_DEV float ld_elem(const void* p, int64_t i) {
    return DT ? bf16_to_f32(((const uint16_t*)p)[i]) : ((const float*)p)[i];
}

// one wave per grouped row
template <int DT>
__global__ __launch_bounds__(256) void gate_grad_kernel(const float* part, int64_t nparts,
                                                        const void* Xg, const void* dYg,
                                                        const int32_t* perm, const int32_t* goff,
                                                        const float* s, int mix, float* dl,
                                                        int64_t T, int64_t E, int64_t D) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int64_t nw = ((int64_t)gridDim.x * blockDim.x) >> 6;
    for (int64_t r = wave; r < T; r += nw) {
        float dg = 0.0f;
        for (int64_t j = lane; j < nparts; j += 64) dg += part[r * nparts + j];
        if (mix) {
            // convex blend: y = g c + (1 - g) x, so dg also holds -dy . x
            for (int64_t d = lane; d < D; d += 64)
                dg -= ld_elem<DT>(dYg, r * D + d) * ld_elem<DT>(Xg, r * D + d);
        }
        dg = wave_sum(dg);
        if (lane == 0) {
            const int64_t e = group_of(goff, E, r);
            const float g = sigmoid_f32(s[(int64_t)perm[r] * E + e]);
            dl[r] = g * (1.0f - g) * dg;
        }
    }
}

// block (x, e): columns 256 x .. 256 x + 255 of dw[e]. Wave w sums the
// rows goff[e] + w, + 4, ...; lane l owns columns 4 l .. 4 l + 3 (one 8-byte
// bf16 or 16-byte fp32 load per row), so each wave streams whole 512-byte
// (1 KB) row pieces. The four waves' sums meet in LDS in a fixed order.
template <int DT>
__global__ __launch_bounds__(256) void centroid_grad_kernel(const float* dl, const void* Xg,
                                                            const int32_t* goff, void* dw,
                                                            int64_t D, int vec) {
    __shared__ float red[4][256];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t e = blockIdx.y;
    const int64_t d0 = (int64_t)blockIdx.x * 256 + 4 * lane;
    const int64_t r0 = goff[e], r1 = goff[e + 1];
    float a[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (d0 < D) {
        if (vec) {  // d0 + 3 < D: D % 4 == 0 (fp32) or D % 8 == 0 (bf16)
#pragma unroll 4
            for (int64_t r = r0 + wv; r < r1; r += 4) {
                const float c = dl[r];
                float x[4];
                if (DT) {
                    const uint2 u = *(const uint2*)((const uint16_t*)Xg + r * D + d0);
                    x[0] = __uint_as_float(u.x << 16);
                    x[1] = __uint_as_float(u.x & 0xffff0000u);
                    x[2] = __uint_as_float(u.y << 16);
                    x[3] = __uint_as_float(u.y & 0xffff0000u);
                } else {
                    const float4 v = *(const float4*)((const float*)Xg + r * D + d0);
                    x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) a[i] = fmaf(c, x[i], a[i]);
            }
        } else {
            for (int64_t r = r0 + wv; r < r1; r += 4) {
                const float c = dl[r];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (d0 + i < D) a[i] = fmaf(c, ld_elem<DT>(Xg, r * D + d0 + i), a[i]);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wv][4 * lane + i] = a[i];
    __syncthreads();
    if (wv == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t d = d0 + i;
            if (d >= D) continue;
            const int j = 4 * lane + i;
            const float v = (red[0][j] + red[1][j]) + (red[2][j] + red[3][j]);
            if (DT) ((uint16_t*)dw)[e * D + d] = f32_to_bf16(v);
            else ((float*)dw)[e * D + d] = v;
        }
    }
}

// ---- experts of sec. 4.1 layer-norm blocks (x_{n+1} = x_n + W2 act(W1 LN(x_n)))

template <int DT>
BASE_DEV void st_elem(void* p, int64_t i, float v) {
    if (DT) ((uint16_t*)p)[i] = f32_to_bf16(v);
    else ((float*)p)[i] = v;
}

// one wave per grouped row: the blocks' upstream dX = g dy (fp32 copy in dXa,
// operand copy in dXo) and the gate-logit gradient dl = g (1 - g) dg with
// dg = dy . x_N (residual) or dy . (x_N - x_0) (convex)
template <int DT>
__global__ __launch_bounds__(256) void block_gate_kernel(const void* X0, const void* XN,
                                                         const void* dYg, const int32_t* perm,
                                                         const int32_t* goff, const float* s,
                                                         int mix, float* dXa, void* dXo,
                                                         float* dl, int64_t T, int64_t E,
                                                         int64_t D) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int64_t nw = ((int64_t)gridDim.x * blockDim.x) >> 6;
    for (int64_t r = wave; r < T; r += nw) {
        const int64_t e = group_of(goff, E, r);
        const float g = sigmoid_f32(s[(int64_t)perm[r] * E + e]);
        float dg = 0.0f;
        for (int64_t d = lane; d < D; d += 64) {
            const int64_t i = r * D + d;
            const float dy = ld_elem<DT>(dYg, i);
            const float x = ld_elem<DT>(XN, i) - (mix ? ld_elem<DT>(X0, i) : 0.0f);
            dg = fmaf(dy, x, dg);
            dXa[i] = g * dy;
            st_elem<DT>(dXo, i, g * dy);
        }
        dg = wave_sum(dg);
        if (lane == 0) dl[r] = g * (1.0f - g) * dg;
    }
}

// one wave per grouped row r of expert e: the layer-norm backward of
// y = (x - mean) rstd gamma_e + beta_e (population variance, fp32
// statistics): with xh = (x - mean) rstd and q = dY gamma_e,
// dx = rstd (q - mean(q) - xh mean(q xh)); dXa[r] += dx, dXo[r] = dXa[r];
// the row's mean and rstd go to stats (for the gamma / beta gradients)
template <int DT>
__global__ __launch_bounds__(256) void ln_backward_kernel(const void* X, const void* dY,
                                                          const float* gamma, const int32_t* goff,
                                                          float eps, float* dXa, void* dXo,
                                                          float* stats, int64_t T, int64_t E,
                                                          int64_t D) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int64_t nw = ((int64_t)gridDim.x * blockDim.x) >> 6;
    const float inv_d = 1.0f / (float)D;
    for (int64_t r = wave; r < T; r += nw) {
        const int64_t e = group_of(goff, E, r);
        const float* ga = gamma ? gamma + e * D : nullptr;
        float sum = 0.0f;
        for (int64_t d = lane; d < D; d += 64) sum += ld_elem<DT>(X, r * D + d);
        const float mean = wave_sum(sum) * inv_d;
        float ss = 0.0f;
        for (int64_t d = lane; d < D; d += 64) {
            const float c = ld_elem<DT>(X, r * D + d) - mean;
            ss = fmaf(c, c, ss);
        }
        const float rstd = 1.0f / sqrtf(wave_sum(ss) * inv_d + eps);
        float m1 = 0.0f, m2 = 0.0f;
        for (int64_t d = lane; d < D; d += 64) {
            const float xh = (ld_elem<DT>(X, r * D + d) - mean) * rstd;
            const float q = ld_elem<DT>(dY, r * D + d) * (ga ? ga[d] : 1.0f);
            m1 += q;
            m2 = fmaf(q, xh, m2);
        }
        m1 = wave_sum(m1) * inv_d;
        m2 = wave_sum(m2) * inv_d;
        for (int64_t d = lane; d < D; d += 64) {
            const int64_t i = r * D + d;
            const float xh = (ld_elem<DT>(X, i) - mean) * rstd;
            const float q = ld_elem<DT>(dY, i) * (ga ? ga[d] : 1.0f);
            const float v = dXa[i] + rstd * (q - m1 - xh * m2);
            dXa[i] = v;
            st_elem<DT>(dXo, i, v);
        }
        if (lane == 0) {
            stats[2 * r] = mean;
            stats[2 * r + 1] = rstd;
        }
    }
}

// block (x, e): columns 256 x .. + 255 of dgamma[e] = sum over the expert's
// rows of dY (x - mean) rstd and dbeta[e] = sum of dY (fp32). Wave w takes
// rows goff[e] + w, + 4, ...; the waves' sums meet in LDS in a fixed order.
template <int DT>
__global__ __launch_bounds__(256) void ln_param_grad_kernel(const void* X, const void* dY,
                                                            const float* stats,
                                                            const int32_t* goff, float* dgamma,
                                                            float* dbeta, int64_t D) {
    __shared__ float red[2][4][256];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t e = blockIdx.y;
    const int64_t d0 = (int64_t)blockIdx.x * 256 + 4 * lane;
    const int64_t r0 = goff[e], r1 = goff[e + 1];
    float ag[4] = {0.0f, 0.0f, 0.0f, 0.0f}, ab[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int64_t r = r0 + wv; r < r1; r += 4) {
        const float mean = stats[2 * r], rstd = stats[2 * r + 1];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t d = d0 + i;
            if (d < D) {
                const float dy = ld_elem<DT>(dY, r * D + d);
                ag[i] = fmaf(dy, (ld_elem<DT>(X, r * D + d) - mean) * rstd, ag[i]);
                ab[i] += dy;
            }
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        red[0][wv][4 * lane + i] = ag[i];
        red[1][wv][4 * lane + i] = ab[i];
    }
    __syncthreads();
    if (wv == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t d = d0 + i;
            if (d >= D) continue;
            const int j = 4 * lane + i;
            if (dgamma)
                dgamma[e * D + d] = (red[0][0][j] + red[0][1][j]) + (red[0][2][j] + red[0][3][j]);
            if (dbeta)
                dbeta[e * D + d] = (red[1][0][j] + red[1][1][j]) + (red[1][2][j] + red[1][3][j]);
        }
    }
}

// one wave per grouped row: dh[perm[r]] = dXa[r] + c dYg[r] + dl[r] w_e with
// c = 1 (residual) or 1 - g (convex)
template <int DT>
__global__ __launch_bounds__(256) void finish_dh_kernel(const float* dXa, const void* dYg,
                                                        const float* dl, const void* w,
                                                        const int32_t* perm, const int32_t* goff,
                                                        const float* s, int mix, void* dh,
                                                        int64_t T, int64_t E, int64_t D) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int64_t nw = ((int64_t)gridDim.x * blockDim.x) >> 6;
    for (int64_t r = wave; r < T; r += nw) {
        const int64_t e = group_of(goff, E, r);
        const int64_t t = perm[r];
        const float g = sigmoid_f32(s[t * E + e]);
        const float c = mix ? 1.0f - g : 1.0f;
        const float l = dl[r];
        for (int64_t d = lane; d < D; d += 64) {
            const float v = dXa[r * D + d] + c * ld_elem<DT>(dYg, r * D + d) +
                            l * ld_elem<DT>(w, e * D + d);
            st_elem<DT>(dh, t * D + d, v);
        }
    }
}

// ---- 16-byte forms of the row kernels (D a multiple of 8, every row and
// vector 16-byte aligned): a lane moves 8 consecutive elements at a time

// elements i .. i + 7 as fp32: one 16-byte load of bf16, or two of fp32
template <int DT>
BASE_DEV void ld8(const void* p, int64_t i, float (&v)[8]) {
    if (DT) {
        const uint4 u = *(const uint4*)((const uint16_t*)p + i);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            v[2 * k] = __uint_as_float(w[k] << 16);
            v[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
        }
    } else {
        const float4 a = *(const float4*)((const float*)p + i);
        const float4 b = *(const float4*)((const float*)p + i + 4);
        v[0] = a.x, v[1] = a.y, v[2] = a.z, v[3] = a.w;
        v[4] = b.x, v[5] = b.y, v[6] = b.z, v[7] = b.w;
    }
}

template <int DT>
BASE_DEV void st8(void* p, int64_t i, const float (&v)[8]) {
    if (DT) {
        uint4 u;
        u.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
        u.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
        u.z = (uint32_t)f32_to_bf16(v[4]) | ((uint32_t)f32_to_bf16(v[5]) << 16);
        u.w = (uint32_t)f32_to_bf16(v[6]) | ((uint32_t)f32_to_bf16(v[7]) << 16);
        *(uint4*)((uint16_t*)p + i) = u;
    } else {
        *(float4*)((float*)p + i) = make_float4(v[0], v[1], v[2], v[3]);
        *(float4*)((float*)p + i + 4) = make_float4(v[4], v[5], v[6], v[7]);
    }
}

// block_gate_kernel, 8 elements per lane step
template <int DT>
__global__ __launch_bounds__(256) void block_gate_vec_kernel(const void* X0, const void* XN,
                                                             const void* dYg,
                                                             const int32_t* perm,
                                                             const int32_t* goff, const float* s,
                                                             int mix, float* dXa, void* dXo,
                                                             float* dl, int64_t T, int64_t E,
                                                             int64_t D) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int64_t nw = ((int64_t)gridDim.x * blockDim.x) >> 6;
    for (int64_t r = wave; r < T; r += nw) {
        const int64_t e = group_of(goff, E, r);
        const float g = sigmoid_f32(s[(int64_t)perm[r] * E + e]);
        float dg = 0.0f;
        for (int64_t d = 8 * lane; d < D; d += 512) {
            const int64_t i = r * D + d;
            float dy[8], x[8], x0[8], o[8];
            ld8<DT>(dYg, i, dy);
            ld8<DT>(XN, i, x);
            if (mix) {
                ld8<DT>(X0, i, x0);
#pragma unroll
                for (int k = 0; k < 8; ++k) x[k] -= x0[k];
            }
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                dg = fmaf(dy[k], x[k], dg);
                o[k] = g * dy[k];
            }
            st8<0>(dXa, i, o);
            st8<DT>(dXo, i, o);
        }
        dg = wave_sum(dg);
        if (lane == 0) dl[r] = g * (1.0f - g) * dg;
    }
}

// ln_backward_kernel with the row in registers: D <= 512 R, lane j holds
// elements 8 (j + 64 c) .. + 7 for c < R
template <int DT, int R>
__global__ __launch_bounds__(256) void ln_backward_vec_kernel(const void* X, const void* dY,
                                                              const float* gamma,
                                                              const int32_t* goff, float eps,
                                                              float* dXa, void* dXo,
                                                              float* stats, int64_t T, int64_t E,
                                                              int64_t D) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int64_t nw = ((int64_t)gridDim.x * blockDim.x) >> 6;
    const float inv_d = 1.0f / (float)D;
    for (int64_t r = wave; r < T; r += nw) {
        const int64_t e = group_of(goff, E, r);
        float x[R][8], q[R][8];
        float sum = 0.0f;
#pragma unroll
        for (int c = 0; c < R; ++c) {
            const int64_t d = 8 * (lane + 64 * c);
            if (d < D) {
                ld8<DT>(X, r * D + d, x[c]);
                ld8<DT>(dY, r * D + d, q[c]);
                if (gamma) {
                    float gm[8];
                    ld8<0>(gamma, e * D + d, gm);
#pragma unroll
                    for (int k = 0; k < 8; ++k) q[c][k] *= gm[k];
                }
#pragma unroll
                for (int k = 0; k < 8; ++k) sum += x[c][k];
            }
        }
        const float mean = wave_sum(sum) * inv_d;
        float ss = 0.0f;
#pragma unroll
        for (int c = 0; c < R; ++c)
            if (8 * (lane + 64 * c) < D) {
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    x[c][k] -= mean;
                    ss = fmaf(x[c][k], x[c][k], ss);
                }
            }
        const float rstd = 1.0f / sqrtf(wave_sum(ss) * inv_d + eps);
        float m1 = 0.0f, m2 = 0.0f;
#pragma unroll
        for (int c = 0; c < R; ++c)
            if (8 * (lane + 64 * c) < D) {
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    x[c][k] *= rstd;  // xh
                    m1 += q[c][k];
                    m2 = fmaf(q[c][k], x[c][k], m2);
                }
            }
        m1 = wave_sum(m1) * inv_d;
        m2 = wave_sum(m2) * inv_d;
#pragma unroll
        for (int c = 0; c < R; ++c) {
            const int64_t d = 8 * (lane + 64 * c);
            if (d < D) {
                float v[8];
                ld8<0>(dXa, r * D + d, v);
#pragma unroll
                for (int k = 0; k < 8; ++k) v[k] += rstd * (q[c][k] - m1 - x[c][k] * m2);
                st8<0>(dXa, r * D + d, v);
                st8<DT>(dXo, r * D + d, v);
            }
        }
        if (lane == 0) {
            stats[2 * r] = mean;
            stats[2 * r + 1] = rstd;
        }
    }
}

// ln_param_grad_kernel with 8 columns per lane: block (x, e) sums columns
// 512 x .. + 511; wave w takes rows goff[e] + w, + 4, ...; the waves' sums
// meet in LDS in a fixed order
template <int DT>
__global__ __launch_bounds__(256) void ln_param_grad_vec_kernel(const void* X, const void* dY,
                                                                const float* stats,
                                                                const int32_t* goff,
                                                                float* dgamma, float* dbeta,
                                                                int64_t D) {
    __shared__ float red[2][4][512];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t e = blockIdx.y;
    const int64_t d0 = (int64_t)blockIdx.x * 512 + 8 * lane;
    const int64_t r0 = goff[e], r1 = goff[e + 1];
    float ag[8], ab[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) ag[k] = ab[k] = 0.0f;
    if (d0 < D) {
        for (int64_t r = r0 + wv; r < r1; r += 4) {
            const float mean = stats[2 * r], rstd = stats[2 * r + 1];
            float dy[8], x[8];
            ld8<DT>(dY, r * D + d0, dy);
            ld8<DT>(X, r * D + d0, x);
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                ag[k] = fmaf(dy[k], (x[k] - mean) * rstd, ag[k]);
                ab[k] += dy[k];
            }
        }
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        red[0][wv][8 * lane + k] = ag[k];
        red[1][wv][8 * lane + k] = ab[k];
    }
    __syncthreads();
    if (wv == 0 && d0 < D) {
        float og[8], ob[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int j = 8 * lane + k;
            og[k] = (red[0][0][j] + red[0][1][j]) + (red[0][2][j] + red[0][3][j]);
            ob[k] = (red[1][0][j] + red[1][1][j]) + (red[1][2][j] + red[1][3][j]);
        }
        if (dgamma) st8<0>(dgamma, e * D + d0, og);
        if (dbeta) st8<0>(dbeta, e * D + d0, ob);
    }
}

// finish_dh_kernel, 8 elements per lane step
template <int DT>
__global__ __launch_bounds__(256) void finish_dh_vec_kernel(const float* dXa, const void* dYg,
                                                            const float* dl, const void* w,
                                                            const int32_t* perm,
                                                            const int32_t* goff, const float* s,
                                                            int mix, void* dh, int64_t T,
                                                            int64_t E, int64_t D) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int64_t nw = ((int64_t)gridDim.x * blockDim.x) >> 6;
    for (int64_t r = wave; r < T; r += nw) {
        const int64_t e = group_of(goff, E, r);
        const int64_t t = perm[r];
        const float g = sigmoid_f32(s[t * E + e]);
        const float c = mix ? 1.0f - g : 1.0f;
        const float l = dl[r];
        for (int64_t d = 8 * lane; d < D; d += 512) {
            float a[8], dy[8], we[8];
            ld8<0>(dXa, r * D + d, a);
            ld8<DT>(dYg, r * D + d, dy);
            ld8<DT>(w, e * D + d, we);
#pragma unroll
            for (int k = 0; k < 8; ++k) a[k] += c * dy[k] + l * we[k];
            st8<DT>(dh, t * D + d, a);
        }
    }
}

// every row of these D-wide buffers starts 16-byte aligned
bool rows16(int64_t D, std::initializer_list<const void*> ptrs) {
    if (D % 8) return false;
    for (const void* p : ptrs)
        if (p && ((uintptr_t)p & 15)) return false;
    return true;
}

unsigned row_blocks(int64_t T) {
    int64_t b = (T + 3) / 4;  // 4 waves of 64 per block, one row each
    return (unsigned)(b > 65536 ? 65536 : b);
}

}  // namespace

hipError_t launch_gather2(const void* h, const void* dy, const int32_t* perm, void* Xg,
                          void* dYg, int64_t T, int64_t D, int dt, hipStream_t st) {
    if (T <= 0) return hipSuccess;
    const int64_t rowbytes = D * (dt ? 2 : 4);
    // 16-byte pieces when every row start is 16-byte aligned
    const int wide = (rowbytes & 15) == 0 && (((uintptr_t)h | (uintptr_t)dy | (uintptr_t)Xg |
                                               (uintptr_t)dYg) & 15) == 0;
    hipLaunchKernelGGL(gather2_kernel, dim3(row_blocks(T)), dim3(256), 0, st, (const char*)h,
                       (const char*)dy, perm, (char*)Xg, (char*)dYg, T, rowbytes, wide);
    return hipGetLastError();
}

hipError_t launch_gate_grad(const float* part, int64_t nparts, const void* Xg, const void* dYg,
                            const int32_t* perm, const int32_t* goff, const float* s, int mix,
                            float* dl, int64_t T, int64_t E, int64_t D, int dt, hipStream_t st) {
    if (T <= 0) return hipSuccess;
    if (dt)
        hipLaunchKernelGGL(gate_grad_kernel<1>, dim3(row_blocks(T)), dim3(256), 0, st, part,
                           nparts, Xg, dYg, perm, goff, s, mix, dl, T, E, D);
    else
        hipLaunchKernelGGL(gate_grad_kernel<0>, dim3(row_blocks(T)), dim3(256), 0, st, part,
                           nparts, Xg, dYg, perm, goff, s, mix, dl, T, E, D);
    return hipGetLastError();
}

hipError_t launch_block_gate(const void* X0, const void* XN, const void* dYg, const int32_t* perm,
                             const int32_t* goff, const float* s, int mix, float* dXa, void* dXo,
                             float* dl, int64_t T, int64_t E, int64_t D, int dt, hipStream_t st) {
    if (T <= 0) return hipSuccess;
    if (rows16(D, {X0, XN, dYg, dXa, dXo})) {
        if (dt)
            hipLaunchKernelGGL(block_gate_vec_kernel<1>, dim3(row_blocks(T)), dim3(256), 0, st,
                               X0, XN, dYg, perm, goff, s, mix, dXa, dXo, dl, T, E, D);
        else
            hipLaunchKernelGGL(block_gate_vec_kernel<0>, dim3(row_blocks(T)), dim3(256), 0, st,
                               X0, XN, dYg, perm, goff, s, mix, dXa, dXo, dl, T, E, D);
        return hipGetLastError();
    }
    if (dt)
        hipLaunchKernelGGL(block_gate_kernel<1>, dim3(row_blocks(T)), dim3(256), 0, st, X0, XN,
                           dYg, perm, goff, s, mix, dXa, dXo, dl, T, E, D);
    else
        hipLaunchKernelGGL(block_gate_kernel<0>, dim3(row_blocks(T)), dim3(256), 0, st, X0, XN,
                           dYg, perm, goff, s, mix, dXa, dXo, dl, T, E, D);
    return hipGetLastError();
}

hipError_t launch_ln_backward(const void* X, const void* dY, const float* gamma,
                              const int32_t* goff, double eps, float* dXa, void* dXo,
                              float* stats, int64_t T, int64_t E, int64_t D, int dt,
                              hipStream_t st) {
    if (T <= 0) return hipSuccess;
    if (D <= 4096 && rows16(D, {X, dY, gamma, dXa, dXo})) {
        const int R = D <= 512 ? 1 : D <= 1024 ? 2 : D <= 2048 ? 4 : 8;
#define BASE_LNB(DTV, RV)                                                                     \
    hipLaunchKernelGGL((ln_backward_vec_kernel<DTV, RV>), dim3(row_blocks(T)), dim3(256), 0, st, \
                       X, dY, gamma, goff, (float)eps, dXa, dXo, stats, T, E, D)
        if (dt) {
            if (R == 1) BASE_LNB(1, 1);
            else if (R == 2) BASE_LNB(1, 2);
            else if (R == 4) BASE_LNB(1, 4);
            else BASE_LNB(1, 8);
        } else {
            if (R == 1) BASE_LNB(0, 1);
            else if (R == 2) BASE_LNB(0, 2);
            else if (R == 4) BASE_LNB(0, 4);
            else BASE_LNB(0, 8);
        }
#undef BASE_LNB
        return hipGetLastError();
    }
    if (dt)
        hipLaunchKernelGGL(ln_backward_kernel<1>, dim3(row_blocks(T)), dim3(256), 0, st, X, dY,
                           gamma, goff, (float)eps, dXa, dXo, stats, T, E, D);
    else
        hipLaunchKernelGGL(ln_backward_kernel<0>, dim3(row_blocks(T)), dim3(256), 0, st, X, dY,
                           gamma, goff, (float)eps, dXa, dXo, stats, T, E, D);
    return hipGetLastError();
}

hipError_t launch_ln_param_grad(const void* X, const void* dY, const float* stats,
                                const int32_t* goff, float* dgamma, float* dbeta, int64_t E,
                                int64_t D, int dt, hipStream_t st) {
    if (!dgamma && !dbeta) return hipSuccess;
    if (rows16(D, {X, dY, dgamma, dbeta})) {
        const dim3 g8((unsigned)((D + 511) / 512), (unsigned)E);
        if (dt)
            hipLaunchKernelGGL(ln_param_grad_vec_kernel<1>, g8, dim3(256), 0, st, X, dY, stats,
                               goff, dgamma, dbeta, D);
        else
            hipLaunchKernelGGL(ln_param_grad_vec_kernel<0>, g8, dim3(256), 0, st, X, dY, stats,
                               goff, dgamma, dbeta, D);
        return hipGetLastError();
    }
    const dim3 grid((unsigned)((D + 255) / 256), (unsigned)E);
    if (dt)
        hipLaunchKernelGGL(ln_param_grad_kernel<1>, grid, dim3(256), 0, st, X, dY, stats, goff,
                           dgamma, dbeta, D);
    else
        hipLaunchKernelGGL(ln_param_grad_kernel<0>, grid, dim3(256), 0, st, X, dY, stats, goff,
                           dgamma, dbeta, D);
    return hipGetLastError();
}

hipError_t launch_finish_dh(const float* dXa, const void* dYg, const float* dl, const void* w,
                            const int32_t* perm, const int32_t* goff, const float* s, int mix,
                            void* dh, int64_t T, int64_t E, int64_t D, int dt, hipStream_t st) {
    if (T <= 0) return hipSuccess;
    if (rows16(D, {dXa, dYg, w, dh})) {
        if (dt)
            hipLaunchKernelGGL(finish_dh_vec_kernel<1>, dim3(row_blocks(T)), dim3(256), 0, st,
                               dXa, dYg, dl, w, perm, goff, s, mix, dh, T, E, D);
        else
            hipLaunchKernelGGL(finish_dh_vec_kernel<0>, dim3(row_blocks(T)), dim3(256), 0, st,
                               dXa, dYg, dl, w, perm, goff, s, mix, dh, T, E, D);
        return hipGetLastError();
    }
    if (dt)
        hipLaunchKernelGGL(finish_dh_kernel<1>, dim3(row_blocks(T)), dim3(256), 0, st, dXa, dYg,
                           dl, w, perm, goff, s, mix, dh, T, E, D);
    else
        hipLaunchKernelGGL(finish_dh_kernel<0>, dim3(row_blocks(T)), dim3(256), 0, st, dXa, dYg,
                           dl, w, perm, goff, s, mix, dh, T, E, D);
    return hipGetLastError();
}

hipError_t launch_centroid_grad(const float* dl, const void* Xg, const int32_t* goff, void* dw,
                                int64_t E, int64_t D, int dt, hipStream_t st) {
    const dim3 grid((unsigned)((D + 255) / 256), (unsigned)E);
    // whole 4-column pieces load as one vector when every row start allows
    const int vec = dt ? (D % 8 == 0 && ((uintptr_t)Xg & 7) == 0)
                       : (D % 4 == 0 && ((uintptr_t)Xg & 15) == 0);
    if (dt)
        hipLaunchKernelGGL(centroid_grad_kernel<1>, grid, dim3(256), 0, st, dl, Xg, goff, dw, D,
                           vec);
    else
        hipLaunchKernelGGL(centroid_grad_kernel<0>, grid, dim3(256), 0, st, dl, Xg, goff, dw, D,
                           vec);
    return hipGetLastError();
}

}  // namespace base
