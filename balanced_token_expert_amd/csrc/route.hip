// Score sanitizing scan, greedy routing and the stable expert grouping.
//
//  scan      one pass over s: smallest finite score and the number of NaN/inf
//            scores. The released BASE code replaces non-finite affinities by
//            the smallest finite one before solving; consumers apply that
//            replacement on the fly from this summary.
//  greedy    test-time routing of "BASE Layers" sec. 3.2.2: a_t = argmax_e
//            s[t][e], lowest expert id among equal scores. One wave per row.
//  perm      fig. 2's sort_by_expert: token ids grouped by expert, ascending
//            within each group (a stable counting sort): per-chunk histograms,
//            a scan, then ranks from bit-sliced wave ballots.
#include "common.h"
#include "internal.h"

namespace base {

constexpr int32_t kStatusUnbalanced = -8;

__global__ void scan_init_kernel(ScoreScan* scan) {
    if (threadIdx.x == 0) {
        scan->min_key = 0xffffffffu;
        scan->nonfinite = 0;
    }
}

__global__ __launch_bounds__(256) void scan_scores_kernel(const float* s, int64_t n, ScoreScan* scan) {
    __shared__ uint32_t wmin[4], wbad[4];
    uint32_t kmin = 0xffffffffu;
    uint32_t bad = 0;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t n4 = n / 4;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
        float4 v = ((const float4*)s)[i];
        float a[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (is_finite_f32(a[q])) kmin = min(kmin, f32_key(a[q]));
            else ++bad;
        }
    }
    for (int64_t i = n4 * 4 + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        float a = s[i];
        if (is_finite_f32(a)) kmin = min(kmin, f32_key(a));
        else ++bad;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o, 64));
        bad += (uint32_t)__shfl_xor((int)bad, o, 64);
    }
    // one atomic per block, and only when it can lower the minimum (many
    // blocks hitting one address serialise at the L2)
    const int wv = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) { wmin[wv] = kmin; wbad[wv] = bad; }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int q = 1; q < (int)(blockDim.x >> 6); ++q) { kmin = min(kmin, wmin[q]); bad += wbad[q]; }
        if (kmin < __hip_atomic_load(&scan->min_key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
            atomicMin(&scan->min_key, kmin);
        if (bad) atomicAdd(&scan->nonfinite, bad);
    }
}

__global__ void stats_reset_kernel(AucStatsDev* st) {
    if (threadIdx.x == 0) {
        st->status = 0;
        st->phases = 0;
        for (int q = 0; q < 16; ++q) { st->bids[q] = 0; st->rounds[q] = 0; st->tail[q] = 0; }
    }
}

hipError_t launch_stats_reset(AucStatsDev* st, hipStream_t s) {
    hipLaunchKernelGGL(stats_reset_kernel, dim3(1), dim3(64), 0, s, st);
    return hipGetLastError();
}

hipError_t launch_scan_init(ScoreScan* scan, hipStream_t st) {
    hipLaunchKernelGGL(scan_init_kernel, dim3(1), dim3(64), 0, st, scan);
    return hipGetLastError();
}

hipError_t launch_scan_scores(const float* s, int64_t n, ScoreScan* scan, hipStream_t st) {
    int64_t blocks = (n / 4 + 255) / 256;
    if (blocks < 1) blocks = 1;
    if (blocks > 1024) blocks = 1024;
    hipLaunchKernelGGL(scan_scores_kernel, dim3((unsigned)blocks), dim3(256), 0, st, s, n, scan);
    return hipGetLastError();
}

// ---------------------------------------------------------------- greedy

// 16 lanes per token (4 tokens per wave): lane j of a token's group reads
// experts j, j + 16, ... (with VEC, 4 consecutive experts from 4 j, 4 j + 64,
// ...), keeps the largest value and its lowest index, and the group merges
// its 16 candidates with xor shuffles (larger value, then lower index, wins).
template <bool VEC>
__global__ __launch_bounds__(256) void greedy_kernel(const float* s, int64_t T, int64_t E,
                                                     const ScoreScan* scan, int32_t* assign) {
    const int lane = threadIdx.x & 63, sub = lane & 15;
    const int64_t grp = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 4;
    const int64_t ngrp = ((int64_t)gridDim.x * blockDim.x) >> 4;
    const bool fix = scan->nonfinite != 0;
    const float repl = scan->min_key == 0xffffffffu ? 0.0f : f32_unkey(scan->min_key);
    // every group of the wave runs the same number of iterations, so the
    // shuffles below always see all 64 lanes active
    const int64_t iters = (T + ngrp - 1) / ngrp;
    for (int64_t it = 0; it < iters; ++it) {
        const int64_t t = grp + it * ngrp;
        float best = 0.0f;
        int bi = 0x7fffffff;
        auto take = [&](float v, int e) {
            if (fix && !is_finite_f32(v)) v = repl;
            if (bi == 0x7fffffff || v > best) { best = v; bi = e; }
        };
        if (t < T) {
            const float* row = s + t * E;
            if (VEC) {
                for (int64_t e = 4 * sub; e < E; e += 64) {
                    const float4 v = *(const float4*)(row + e);
                    take(v.x, (int)e);
                    take(v.y, (int)e + 1);
                    take(v.z, (int)e + 2);
                    take(v.w, (int)e + 3);
                }
            } else {
                for (int64_t e = sub; e < E; e += 16) take(row[e], (int)e);
            }
        }
#pragma unroll
        for (int o = 8; o > 0; o >>= 1) {
            const float ov = __shfl_xor(best, o, 64);
            const int oi = __shfl_xor(bi, o, 64);
            if (oi != 0x7fffffff && (bi == 0x7fffffff || ov > best || (ov == best && oi < bi))) {
                best = ov;
                bi = oi;
            }
        }
        if (sub == 0 && t < T) assign[t] = bi;
    }
}

hipError_t launch_greedy(const float* s, int64_t T, int64_t E, const ScoreScan* scan,
                         int32_t* assign, int32_t* /*counts*/, hipStream_t st) {
    int64_t blocks = (T + 15) / 16;  // 16 tokens per 256-thread block at once
    if (blocks > 8192) blocks = 8192;
    if (E % 64 == 0 && ((uintptr_t)s & 15) == 0)
        hipLaunchKernelGGL(greedy_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, st, s, T, E,
                           scan, assign);
    else
        hipLaunchKernelGGL(greedy_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, st, s, T, E,
                           scan, assign);
    return hipGetLastError();
}

// ---------------------------------------------------------------- perm

constexpr int kPermChunk = 512;  // tokens per block (128 blocks at 65536 tokens)
constexpr int kPermThreads = 256;
constexpr int kScanLds = 32768;  // per-block counts the scan stages in LDS (128 KB)

size_t perm_ws_bytes(int64_t T, int64_t E) {
    int64_t nb = (T + kPermChunk - 1) / kPermChunk;
    return (size_t)(2 * nb * E + E) * sizeof(int32_t) + 256;
}

BASE_DEV int clamp_id(int32_t a, int64_t E) { return (a < 0 || a >= E) ? 0 : a; }

// block b: counts of its chunk per expert -> cnt[b*E + e]
__global__ __launch_bounds__(kPermThreads) void perm_hist_kernel(const int32_t* assign, int64_t T,
                                                                 int64_t E, int32_t* cnt,
                                                                 int32_t* status) {
    extern __shared__ int32_t hist[];
    for (int64_t e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
    __syncthreads();
    const int64_t t0 = (int64_t)blockIdx.x * kPermChunk;
    const int64_t t1 = min(T, t0 + kPermChunk);
    bool bad = false;
    for (int64_t t = t0 + threadIdx.x; t < t1; t += blockDim.x) {
        int32_t a = assign[t];
        if (a < 0 || a >= E) bad = true;
        atomicAdd(&hist[clamp_id(a, E)], 1);
    }
    if (bad && status) *status = kStatusUnbalanced;
    __syncthreads();
    for (int64_t e = threadIdx.x; e < E; e += blockDim.x) cnt[blockIdx.x * E + e] = hist[e];
}

// one block: base[b*E+e] = offsets[e] + sum_{b'<b} cnt[b'*E+e], i.e. the
// exclusive prefix sum of the counts taken in (expert, block) order; then
// offsets[e] = base[e] (block 0), counts[e] = offsets[e+1] - offsets[e]. Each
// thread sums a contiguous run of that order, the runs' sums are scanned
// across the block (wave prefix sums, then the 16 wave totals), and each
// thread writes its run's bases.
__global__ __launch_bounds__(1024) void perm_scan_kernel(const int32_t* cnt, int64_t nb, int64_t E,
                                                         int64_t T, int32_t* base, int32_t* offsets,
                                                         int32_t* counts, int64_t want_k,
                                                         int32_t* status) {
    __shared__ int32_t wsum[16];
    __shared__ int32_t sc[kScanLds];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t n = nb * E;
    // the counts come into LDS with coalesced loads when they fit, so the two
    // strided passes below read LDS instead of waiting on L2 per element
    const bool staged = n <= kScanLds;
    if (staged) {
        for (int64_t j = tid; j < n; j += blockDim.x) sc[j] = cnt[j];
        __syncthreads();
    }
    auto get = [&](int64_t j) -> int32_t { return staged ? sc[j] : cnt[j]; };
    const int64_t per = (n + 1023) / 1024;
    const int64_t i0 = min(n, (int64_t)tid * per), i1 = min(n, i0 + per);
    // i = e nb + b; the run starts at (e0, b0) and steps b, then e
    const int64_t e0 = i0 / nb, b0 = i0 % nb;
    int32_t own = 0;
    {
        int64_t e = e0, b = b0;
        for (int64_t i = i0; i < i1; ++i) {
            own += get(b * E + e);
            if (++b == nb) { b = 0; ++e; }
        }
    }
    int32_t v = own;  // inclusive prefix over the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int32_t u = __shfl_up(v, o, 64);
        if (lane >= o) v += u;
    }
    if (lane == 63) wsum[wave] = v;
    __syncthreads();
    if (wave == 0) {
        int32_t x = lane < 16 ? wsum[lane] : 0;
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) {
            const int32_t u = __shfl_up(x, o, 64);
            if (lane >= o) x += u;
        }
        if (lane < 16) wsum[lane] = x;
    }
    __syncthreads();
    int32_t run = v - own + (wave > 0 ? wsum[wave - 1] : 0);
    {
        int64_t e = e0, b = b0;
        for (int64_t i = i0; i < i1; ++i) {
            const int64_t j = b * E + e;
            const int32_t c = get(j);
            base[j] = run;
            run += c;
            if (++b == nb) { b = 0; ++e; }
        }
    }
    __syncthreads();
    for (int64_t e = tid; e < E; e += blockDim.x) {
        const int32_t off = base[e];
        const int32_t next = e + 1 < E ? base[e + 1] : (int32_t)T;
        if (offsets) offsets[e] = off;
        if (counts) counts[e] = next - off;
        if (want_k > 0 && next - off != want_k && status) *status = kStatusUnbalanced;
    }
    if (tid == 0 && offsets) offsets[E] = (int32_t)T;
}

// block b: stable placement of its chunk. Tokens are taken 256 at a time in
// order; within a wave, equal-expert lanes are found with one ballot per bit
// of the expert id, and the rank of a lane is the number of equal lanes below
// it. Waves of a batch are ordered through per-wave counts in LDS.
__global__ __launch_bounds__(kPermThreads) void perm_scatter_kernel(const int32_t* assign, int64_t T,
                                                                    int64_t E, const int32_t* base,
                                                                    int32_t* perm) {
    extern __shared__ int32_t sm[];
    int32_t* running = sm;            // E
    int32_t* wcnt = sm + E;           // 4 * E
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int64_t e = threadIdx.x; e < E; e += blockDim.x) running[e] = base[blockIdx.x * E + e];
    int nbits = 0;
    while ((1ll << nbits) < E) ++nbits;
    const int64_t t0 = (int64_t)blockIdx.x * kPermChunk;
    const int64_t t1 = min(T, t0 + kPermChunk);
    for (int64_t tb = t0; tb < t1; tb += kPermThreads) {
        for (int64_t i = threadIdx.x; i < 4 * E; i += blockDim.x) wcnt[i] = 0;
        __syncthreads();
        const int64_t t = tb + threadIdx.x;
        const bool valid = t < t1;
        const int e = valid ? clamp_id(assign[t], E) : 0;
        unsigned long long same = __ballot(valid);
        for (int j = 0; j < nbits; ++j) {
            const bool bit = (e >> j) & 1;
            const unsigned long long b = __ballot(valid && bit);
            same &= bit ? b : ~b;
        }
        if (!valid) same = 0;
        const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
        const int rank = __popcll(same & below);
        const bool last = valid && ((same >> lane) == 1ull);  // highest equal lane
        if (last) wcnt[wave * E + e] = rank + 1;
        __syncthreads();
        if (valid) {
            int pos = running[e] + rank;
            for (int w = 0; w < wave; ++w) pos += wcnt[w * E + e];
            perm[pos] = (int32_t)t;
        }
        __syncthreads();
        for (int64_t x = threadIdx.x; x < E; x += blockDim.x)
            running[x] += wcnt[x] + wcnt[E + x] + wcnt[2 * E + x] + wcnt[3 * E + x];
        __syncthreads();
    }
}

hipError_t launch_perm(const int32_t* assign, int64_t T, int64_t E, int32_t* perm,
                       int32_t* offsets, int32_t* counts, int64_t want_k, int32_t* status,
                       void* ws, hipStream_t st) {
    const int64_t nb = (T + kPermChunk - 1) / kPermChunk;
    int32_t* cnt = (int32_t*)ws;
    int32_t* base = cnt + nb * E;
    hipLaunchKernelGGL(perm_hist_kernel, dim3((unsigned)nb), dim3(kPermThreads), E * sizeof(int32_t),
                       st, assign, T, E, cnt, status);
    hipLaunchKernelGGL(perm_scan_kernel, dim3(1), dim3(1024), 0, st, cnt, nb, E, T, base, offsets,
                       counts, want_k, status);
    hipLaunchKernelGGL(perm_scatter_kernel, dim3((unsigned)nb), dim3(kPermThreads),
                       5 * E * sizeof(int32_t), st, assign, T, E, base, perm);
    return hipGetLastError();
}

}  // namespace base
