// Small kernels of the layer's backward pass (base_layer_backward). The
// assignment is held fixed: the affinities that chose the experts carry no
// gradient, and the centroids learn through the sigmoid gate only (BASE
// Layers sec. 3.1; the released code scores tokens under no_grad). With the
// logit l = h_t . w_e of a token's expert and g = sigma(l):
//   dl = g (1 - g) dg,  dg = dy . c (eq. 1) or dy . (c - h_t) (convex blend),
//   dh_t gets dl w_e,  dw_e = sum over its tokens of dl h_t.
// The expert products (and dy . c, accumulated in their epilogue as
// V . act(Z), V = W2^T dy) live in gemm.hip.
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
