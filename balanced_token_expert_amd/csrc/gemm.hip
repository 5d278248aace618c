// Dense products of the BASE layer on gfx950.
//
// Three products share one "NT" kernel shape, C[m][n] = sum_k A[m][k] B[n][k]
// with K contiguous in both operands:
//   affinity  s = h w^T                       ("BASE Layers" sec. 3.1, fig. 2)
//   FFN1      H_e = act(X_e W1_e^T), X_e[i] = h[perm[e*k+i]]   (gather fused
//             into the A-tile loads: fig. 2's expert sort costs no pass)
//   FFN2      Y_e = H_e W2_e^T with the epilogue of eq. 1:
//             out[t] = sigmoid(s[t][e]) * Y_e[i] + h[t], t = perm[e*k+i]
//             (fig. 2's inverse sort fused into the stores)
//
// bf16 path: 64-wide waves issue v_mfma_f32_32x32x16_bf16 with fp32
// accumulation. The expert products use 256 x 256 tiles fed through a
// 4-stage LDS pipeline of direct global->LDS loads (gemm_dma.h); the affinity
// uses a register-staged, double-buffered 128-row tile. The block -> tile map
// keeps the tiles that share a weight tile on one XCD (consecutive logical
// tiles land on the same L2).
// fp32 path: a plain LDS-tiled FMA kernel (exact fp32 products).
#include "common.h"
#include "internal.h"

namespace base {

enum { KIND_AFF = 0, KIND_FFN1 = 1, KIND_FFN2 = 2,
       // backward products of the layer, per expert group (grouped rows):
       KIND_BZ = 3,  // Z = X W1^T; stores Z and gate * act(Z)
       KIND_BV = 4,  // V = dY W2 (W2 read k-major); stores dZ = gate V act'(Z)
                     // and per-row partial sums of V act(Z)
       KIND_BX = 5,  // dX = dZ W1 (W1 read k-major); dh[t] = dX + c dY + dl w_e
       KIND_BW = 6   // dW_g = P_g^T Q_g over the group's rows (both k-major)
};

struct GemmParams {
    const void* A;          // bf16 bits or fp32, rows of length K
    const void* B;          // N x K per group
    int64_t M, N, K;        // M = rows per group
    int64_t groups;
    const int32_t* perm;    // FFN1: A row map; FFN2: output row map
    int64_t b_gstride;      // elements between consecutive groups' B
    float* s_out;           // AFF: M x N fp32
    ScoreScan* scan;        // AFF: min finite key / non-finite count
    void* H;                // FFN1 output, (groups*M) x N
    int act;                // 0 relu, 1 gelu
    const float* s_in;      // FFN2: gate scores, rows of length E
    int64_t E;
    const void* h;          // FFN2: residual rows (length N)
    void* out;              // FFN2: output rows (length N)
    // ragged groups (null: every group has M rows): group g owns rows
    // [goff[g], goff[g+1]) and the blocks [gblk[g], gblk[g+1]) of the launch
    const int32_t* goff;
    const int32_t* gblk;
    // FFN2 epilogue of the layer variants (see Ffn2Epi); epi_general == 0 is
    // eq. 1's y = sigmoid(s) C + h, scattered to out
    int epi_general, epi_gate, epi_keep, epi_res;
    const void* xr;
    void* xo;
    // backward products. An operand "read k-major" is stored as rows of k
    // with M (or N) contiguous: element (m, k) at A[k * lda + m] (B: ldb).
    int64_t lda, ldb;
    const int32_t* kgoff;   // BW: group g sums rows [kgoff[g], kgoff[g+1]) (null: K each)
    const void* zin;        // BV: saved pre-activations Z, grouped rows of length N
    void* gu;               // BZ: gate * act(Z), grouped rows
    const void* dyg;        // BX: grouped upstream gradient rows (length N)
    const void* wc;         // BX: centroids, E x N
    const float* dl;        // BX: gate-logit gradient of each grouped row
    float* part;            // BV: partial sums of V . act(Z), nparts per grouped row
    int64_t nparts;
    int mix;                // BX: 0 residual (c = 1), 1 convex (c = 1 - gate)
    int a_bytes;            // persistent FFN1 with gathered rows: bytes of h (< 2^31)
};

// The tile a block computes: group g, tile (tm, tn), and the group's rows
// row0 .. row0 + rows - 1 (in the grouped row order of A / H).
struct Tile {
    int64_t g, tm, tn, row0, rows;
};
template <int BM, int BN>
BASE_DEV bool locate_tile(const GemmParams& p, int64_t lid, Tile& t) {
    const int64_t ntn = (p.N + BN - 1) / BN;
    if (!p.goff) {
        const int64_t ntm = (p.M + BM - 1) / BM;
        t.g = lid / (ntm * ntn);
        if (t.g >= p.groups) return false;
        const int64_t rr = lid % (ntm * ntn);
        t.tn = rr / ntm;  // M tiles fastest: they share B
        t.tm = rr % ntm;
        t.row0 = t.g * p.M;
        t.rows = p.M;
        return true;
    }
    if (lid >= p.gblk[p.groups]) return false;
    int64_t lo = 0, hi = p.groups;  // the last group whose blocks start at or before lid
    while (hi - lo > 1) {
        const int64_t mid = (lo + hi) >> 1;
        if (p.gblk[mid] <= lid) lo = mid;
        else hi = mid;
    }
    t.g = lo;
    t.row0 = p.goff[lo];
    t.rows = p.goff[lo + 1] - p.goff[lo];
    const int64_t ntm = (t.rows + BM - 1) / BM;
    const int64_t local = lid - p.gblk[lo];
    t.tn = local / ntm;
    t.tm = local % ntm;
    return true;
}

// gblk[g] = blocks of groups 0..g-1 for BM-row tiles and ntn column tiles
// (one workgroup of 1024 threads; groups <= 1024)
__global__ __launch_bounds__(1024) void group_blocks_kernel(const int32_t* goff, int64_t groups,
                                                            int64_t bm, int64_t ntn, int32_t* gblk) {
    __shared__ int32_t sc[1024];
    const int g = threadIdx.x;
    const int32_t own = (g < groups) ? (int32_t)(((goff[g + 1] - goff[g]) + bm - 1) / bm * ntn) : 0;
    sc[g] = own;
    __syncthreads();
    for (int o = 1; o < 1024; o <<= 1) {
        const int32_t v = (g >= o) ? sc[g - o] : 0;
        __syncthreads();
        sc[g] += v;
        __syncthreads();
    }
    if (g < groups) gblk[g + 1] = sc[g];
    if (g == 0) gblk[0] = 0;
}

// Physical block id -> logical tile id such that each XCD (blocks are dealt
// round-robin to the 8 XCDs) receives a contiguous run of logical tiles.
BASE_DEV int64_t xcd_logical(int64_t pid, int64_t nblk) {
    int64_t x = pid & 7, slot = pid >> 3;
    int64_t per = nblk >> 3, rem = nblk & 7;
    return x * per + (x < rem ? x : rem) + slot;
}

BASE_DEV float apply_act(float v, int act) { return act ? gelu_erf(v) : fmaxf(v, 0.0f); }

template <int Kind, int TM, int TN>
BASE_DEV void store_tile(const GemmParams& p, f32x16_t (&acc)[TM][TN], const Tile& tl, int64_t mw,
                         int64_t nw, int lane);

// ---------------------------------------------------------------- bf16 MFMA

template <int Kind, int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(WM* WN * 64) void gemm_bf16_kernel(GemmParams p) {
    constexpr int BK = 64, LDK = BK + 8;
    constexpr int NT = WM * WN * 64;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int TM = WTM / 32, TN = WTN / 32;
    constexpr int CA = BM * (BK / 8) / NT;   // 16-byte A chunks per thread
    constexpr int CB = BN * (BK / 8) / NT;
    static_assert(TM >= 1 && TN >= 1 && CA >= 1 && CB >= 1, "tile shape");
    static_assert((BM * (BK / 8)) % NT == 0 && (BN * (BK / 8)) % NT == 0, "tile shape");

    __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * LDK];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * LDK];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    Tile tl;
    if (!locate_tile<BM, BN>(p, xcd_logical(blockIdx.x, gridDim.x), tl)) return;
    const int64_t g = tl.g;
    const int64_t m0 = tl.tm * BM, n0 = tl.tn * BN;

    const uint16_t* A = (const uint16_t*)p.A;
    const uint16_t* B = (const uint16_t*)p.B + g * p.b_gstride;

    // rows this thread stages (fixed over the K loop)
    const uint16_t* arow[CA];
    const uint16_t* brow[CB];
    int akc[CA], bkc[CB], ar[CA], br[CB];
#pragma unroll
    for (int j = 0; j < CA; ++j) {
        int c = tid + j * NT;
        ar[j] = c >> 3;
        akc[j] = (c & 7) * 8;
        int64_t m = m0 + ar[j];
        arow[j] = nullptr;
        if (m < tl.rows) {
            int64_t src;
            if (Kind == KIND_FFN1) src = p.perm[tl.row0 + m];
            else if (Kind == KIND_FFN2) src = tl.row0 + m;
            else src = m;
            arow[j] = A + src * p.K;
        }
    }
#pragma unroll
    for (int j = 0; j < CB; ++j) {
        int c = tid + j * NT;
        br[j] = c >> 3;
        bkc[j] = (c & 7) * 8;
        int64_t n = n0 + br[j];
        brow[j] = (n < p.N) ? B + n * p.K : nullptr;
    }

    uint4 ra[CA], rb[CB];
    auto load_regs = [&](int64_t k0) {
#pragma unroll
        for (int j = 0; j < CA; ++j) {
            int64_t kk = k0 + akc[j];
            ra[j] = (arow[j] && kk < p.K) ? *(const uint4*)(arow[j] + kk) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < CB; ++j) {
            int64_t kk = k0 + bkc[j];
            rb[j] = (brow[j] && kk < p.K) ? *(const uint4*)(brow[j] + kk) : make_uint4(0, 0, 0, 0);
        }
    };
    auto store_lds = [&](int buf) {
#pragma unroll
        for (int j = 0; j < CA; ++j) *(uint4*)&As[buf][ar[j] * LDK + akc[j]] = ra[j];
#pragma unroll
        for (int j = 0; j < CB; ++j) *(uint4*)&Bs[buf][br[j] * LDK + bkc[j]] = rb[j];
    };

    f32x16_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int64_t nk = (p.K + BK - 1) / BK;
    load_regs(0);
    store_lds(0);
    __syncthreads();
    const int frow = lane & 31, fk = (lane >> 5) * 8;
    for (int64_t kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) load_regs((kt + 1) * BK);
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            bf16x8_t af[TM], bfr[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i)
                af[i] = *(const bf16x8_t*)&As[buf][(wm * WTM + i * 32 + frow) * LDK + kk * 16 + fk];
#pragma unroll
            for (int j = 0; j < TN; ++j)
                bfr[j] = *(const bf16x8_t*)&Bs[buf][(wn * WTN + j * 32 + frow) * LDK + kk * 16 + fk];
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < nk) store_lds(buf ^ 1);
        __syncthreads();
    }

    store_tile<Kind, TM, TN>(p, acc, tl, m0 + wm * WTM, n0 + wn * WTN, lane);
}

#include "gemm_dma.h"

// ---- epilogue of one wave's TM x TN block of 32x32 MFMA tiles, whose first
// output row and column are mw and nw. acc[i][j][r] is C[row][col] with
//   row = mw + i*32 + (r/4)*8 + (lane/32)*4 + r%4,  col = nw + j*32 + lane%32
template <int Kind, int TM, int TN>
BASE_DEV void store_tile(const GemmParams& p, f32x16_t (&acc)[TM][TN], const Tile& tl, int64_t mw,
                         int64_t nw, int lane) {
    const int64_t g = tl.g;
    uint32_t kmin = 0xffffffffu;
    int nonfin = 0;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int64_t m = mw + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
            if (m >= tl.rows) continue;
            int64_t t = 0;
            float gate = 0.0f;
            if (Kind == KIND_FFN2) {
                t = p.perm[tl.row0 + m];
                gate = sigmoid_f32(p.s_in[t * p.E + g]);
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int64_t n = nw + j * 32 + (lane & 31);
                if (n >= p.N) continue;
                const float v = acc[i][j][r];
                if (Kind == KIND_AFF) {
                    p.s_out[m * p.N + n] = v;
                    if (is_finite_f32(v)) kmin = min(kmin, f32_key(v));
                    else ++nonfin;
                } else if (Kind == KIND_FFN1) {
                    ((uint16_t*)p.H)[(tl.row0 + m) * p.N + n] = f32_to_bf16(apply_act(v, p.act));
                } else {
                    const float res = bf16_to_f32(((const uint16_t*)p.h)[t * p.N + n]);
                    ((uint16_t*)p.out)[t * p.N + n] = f32_to_bf16(gate * v + res);
                }
            }
        }
    }
    if (Kind == KIND_AFF) {
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o, 64));
            nonfin += __shfl_xor(nonfin, o, 64);
        }
        if (lane == 0 && p.scan) {
            if (kmin != 0xffffffffu &&
                kmin < __hip_atomic_load(&p.scan->min_key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
                atomicMin(&p.scan->min_key, kmin);
            if (nonfin) atomicAdd(&p.scan->nonfinite, (uint32_t)nonfin);
        }
    }
}

// ---------------------------------------------------------------- fp32 FMA

template <int Kind>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmParams p) {
    constexpr int BM = 64, BN = 64, BK = 16;
    __shared__ float As[BK][BM + 4];
    __shared__ float Bs[BK][BN + 4];
    const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
    Tile tl;
    if (!locate_tile<BM, BN>(p, blockIdx.x, tl)) return;
    const int64_t g = tl.g;
    const int64_t m0 = tl.tm * BM, n0 = tl.tn * BN;
    const float* A = (const float*)p.A;
    const float* B = (const float*)p.B + g * p.b_gstride;

    // staging: 64 rows x 16 k per tile, 4 elements per thread
    const int lr = tid >> 2, lk = (tid & 3) * 4;
    const float* arow = nullptr;
    {
        int64_t m = m0 + lr;
        if (m < tl.rows) {
            int64_t src = (Kind == KIND_FFN1 && p.perm) ? p.perm[tl.row0 + m]
                        : (Kind == KIND_FFN1 || Kind == KIND_FFN2) ? tl.row0 + m : m;
            arow = A + src * p.K;
        }
    }
    const float* brow = (n0 + lr < p.N) ? B + (n0 + lr) * p.K : nullptr;

    float acc[4][4] = {};
    for (int64_t k0 = 0; k0 < p.K; k0 += BK) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            int64_t kk = k0 + lk + q;
            As[lk + q][lr] = (arow && kk < p.K) ? arow[kk] : 0.0f;
            Bs[lk + q][lr] = (brow && kk < p.K) ? brow[kk] : 0.0f;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < BK; ++kk) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }
    uint32_t kmin = 0xffffffffu;
    int nonfin = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t m = m0 + ty * 4 + i;
        if (m >= tl.rows) continue;
        int64_t t = 0;
        float gate = 0.0f;
        if (Kind == KIND_FFN2) {
            t = p.perm[tl.row0 + m];
            gate = (p.epi_general && p.epi_gate) ? 1.0f : sigmoid_f32(p.s_in[t * p.E + g]);
        }
        const float c2 = (!p.epi_general || p.epi_keep == 0) ? 1.0f
                         : (p.epi_keep == 1 ? 1.0f - gate : 0.0f);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t n = n0 + tx * 4 + j;
            if (n >= p.N) continue;
            const float v = acc[i][j];
            if (Kind == KIND_AFF) {
                p.s_out[m * p.N + n] = v;
                if (is_finite_f32(v)) kmin = min(kmin, f32_key(v));
                else ++nonfin;
            } else if (Kind == KIND_FFN1) {
                ((float*)p.H)[(tl.row0 + m) * p.N + n] = apply_act(v, p.act);
            } else if (!p.epi_general) {
                ((float*)p.out)[t * p.N + n] = gate * v + ((const float*)p.h)[t * p.N + n];
            } else {
                const float ht = (c2 != 0.0f || p.epi_res == 1) ? ((const float*)p.h)[t * p.N + n] : 0.0f;
                const float r = p.epi_res == 1 ? ht
                              : (p.epi_res == 2 ? ((const float*)p.xr)[(tl.row0 + m) * p.N + n] : 0.0f);
                const float y = fmaf(gate, r + v, c2 * ht);
                if (p.xo) ((float*)p.xo)[(tl.row0 + m) * p.N + n] = y;
                else ((float*)p.out)[t * p.N + n] = y;
            }
        }
    }
    if (Kind == KIND_AFF) {
        const int lane = tid & 63;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o, 64));
            nonfin += __shfl_xor(nonfin, o, 64);
        }
        if (lane == 0 && p.scan) {
            if (kmin != 0xffffffffu &&
                kmin < __hip_atomic_load(&p.scan->min_key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
                atomicMin(&p.scan->min_key, kmin);
            if (nonfin) atomicAdd(&p.scan->nonfinite, (uint32_t)nonfin);
        }
    }
}

// fp32 backward products: 64 x 64 tiles, exact fp32 FMAs, the epilogues of
// the bf16 path with fp32 storage. Operands read k-major are staged with M
// (N) contiguous, so both layouts load coalesced.
template <int Kind>
__global__ __launch_bounds__(256) void gemm_f32_bwd_kernel(GemmParams p) {
    constexpr int BM = 64, BN = 64, BK = 16;
    constexpr bool AT = Kind == KIND_BW;
    constexpr bool BT = Kind == KIND_BV || Kind == KIND_BX || Kind == KIND_BW;
    __shared__ float As[BK][BM + 4];
    __shared__ float Bs[BK][BN + 4];
    const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
    Tile tl;
    if (!locate_tile<BM, BN>(p, blockIdx.x, tl)) return;
    const int64_t g = tl.g;
    const int64_t m0 = tl.tm * BM, n0 = tl.tn * BN;
    const float* A = (const float*)p.A;
    const float* B = (const float*)p.B + g * p.b_gstride;
    int64_t kbeg = 0, Kc = p.K;
    if (Kind == KIND_BW) {
        kbeg = p.kgoff ? p.kgoff[g] : g * p.K;
        Kc = p.kgoff ? p.kgoff[g + 1] - kbeg : p.K;
    }
    // k-major staging: thread -> (k = tid / 16, 4 consecutive m / n);
    // m/n-major staging: thread -> (row = tid / 4, 4 consecutive k)
    const int lr = tid >> 2, lk = (tid & 3) * 4;
    const int tk = tid >> 4, tc = (tid & 15) * 4;
    float acc[4][4] = {};
    for (int64_t k0 = 0; k0 < Kc; k0 += BK) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (AT) {
                const int64_t k = k0 + tk, m = m0 + tc + q;
                As[tk][tc + q] = (k < Kc && m < tl.rows) ? A[(kbeg + k) * p.lda + m] : 0.0f;
            } else {
                const int64_t k = k0 + lk + q, m = m0 + lr;
                As[lk + q][lr] = (k < Kc && m < tl.rows) ? A[(tl.row0 + m) * p.K + k] : 0.0f;
            }
            if (BT) {
                const int64_t k = k0 + tk, n = n0 + tc + q;
                Bs[tk][tc + q] = (k < Kc && n < p.N) ? B[(kbeg + k) * p.ldb + n] : 0.0f;
            } else {
                const int64_t k = k0 + lk + q, n = n0 + lr;
                Bs[lk + q][lr] = (k < Kc && n < p.N) ? B[n * p.K + k] : 0.0f;
            }
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < BK; ++kk) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t m = m0 + ty * 4 + i;
        const bool rowok = m < tl.rows;
        const int64_t row = tl.row0 + m;
        int64_t t = 0;
        float gate = 0.0f;
        if (Kind != KIND_BW && rowok) {
            t = p.perm[row];
            gate = p.epi_gate ? 1.0f : sigmoid_f32(p.s_in[t * p.E + g]);
        }
        float psum = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t n = n0 + tx * 4 + j;
            if (!rowok || n >= p.N) continue;
            const float v = acc[i][j];
            if (Kind == KIND_BZ) {
                ((float*)p.H)[row * p.N + n] = v;
                ((float*)p.gu)[row * p.N + n] = gate * apply_act(v, p.act);
            } else if (Kind == KIND_BV) {
                const float z = ((const float*)p.zin)[row * p.N + n];
                const float u = apply_act(z, p.act);
                const float du = p.act ? 0.5f * (1.0f + erff(z * 0.70710678118654752f)) +
                                             z * expf(-0.5f * z * z) * 0.39894228040143268f
                                       : (z > 0.0f ? 1.0f : 0.0f);
                psum = fmaf(v, u, psum);
                ((float*)p.H)[row * p.N + n] = gate * v * du;
            } else if (Kind == KIND_BX && p.xo) {
                ((float*)p.xo)[row * p.N + n] = v;
            } else if (Kind == KIND_BX) {
                const float cx = p.mix ? 1.0f - gate : 1.0f;
                ((float*)p.out)[t * p.N + n] =
                    fmaf(p.dl[row], ((const float*)p.wc)[g * p.N + n],
                         fmaf(cx, ((const float*)p.dyg)[row * p.N + n], v));
            } else {
                ((float*)p.H)[row * p.N + n] = v;
            }
        }
        if (Kind == KIND_BV) {
            // the 16 threads of a row are 16 consecutive lanes
#pragma unroll
            for (int o = 8; o > 0; o >>= 1) psum += __shfl_xor(psum, o, 64);
            if (tx == 0 && rowok) p.part[row * p.nparts + tl.tn] = psum;
        }
    }
}

// ---------------------------------------------------------------- launchers

template <int Kind, int BM, int BN, int WM, int WN>
static hipError_t run_bf16(const GemmParams& p, hipStream_t st) {
    const int64_t tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN) * p.groups;
    if (tiles <= 0) return hipSuccess;
    if (tiles > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gemm_bf16_kernel<Kind, BM, BN, WM, WN>), dim3((unsigned)tiles),
                       dim3(WM * WN * 64), 0, st, p);
    return hipGetLastError();
}

// Blocks to launch for BM x BN tiles: exact for equal groups; for ragged
// groups the block map is built on the device first and the launch covers
// its upper bound (ceil(rows/BM) + groups column-tile rows; the rest exit).
template <int BM, int BN>
static int64_t grid_blocks(const GemmParams& p, int32_t* gblk, int64_t rows_total,
                           hipStream_t st) {
    const int64_t ntn = (p.N + BN - 1) / BN;
    if (!p.goff) return ((p.M + BM - 1) / BM) * ntn * p.groups;
    hipLaunchKernelGGL(group_blocks_kernel, dim3(1), dim3(1024), 0, st, p.goff, p.groups,
                       (int64_t)BM, ntn, gblk);
    return ((rows_total + BM - 1) / BM + p.groups) * ntn;
}

template <int Kind, int BN, int WM, int WN, bool GEN = false>
static hipError_t run_dma64(const GemmParams& p, int32_t* gblk, int64_t rows_total, hipStream_t st) {
    const int64_t tiles = grid_blocks<256, BN>(p, gblk, rows_total, st);
    if (tiles <= 0) return hipSuccess;
    if (tiles > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gemm_bf16_dma64_kernel<Kind, BN, WM, WN, GEN>), dim3((unsigned)tiles),
                       dim3(WM * WN * 64), 0, st, p);
    return hipGetLastError();
}

// Persistent launch of the backward products: one block per CU (a block
// holds 128 KB of LDS stages and 512 threads of 256 registers, so a CU runs
// one at a time), a multiple of 8 so every XCD gets the same number.
static int64_t cu_count() {
    static int n = 0;
    if (n == 0) {
        int dev = 0, c = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
            c > 0)
            n = c;
        else
            n = 256;
    }
    return n;
}

// The persistent kernel addresses a step's operands with 32-bit offsets:
// widths up to 2^20 and, for rows gathered through perm, all of h below 2^31
// bytes. Larger problems take the one-tile-per-block kernel.
static bool pers_fits(int64_t K, int64_t N, int64_t gathered_bytes) {
    const int64_t lim = int64_t(1) << 20;
    return K <= lim && N <= lim && gathered_bytes < (int64_t(1) << 31);
}

template <int Kind, bool GEN = false, bool GATHER = false>
static hipError_t run_pers(const GemmParams& p, int32_t* gblk, int64_t rows_total,
                           hipStream_t st) {
    const int64_t tiles = grid_blocks<256, 256>(p, gblk, rows_total, st);
    if (tiles <= 0) return hipSuccess;
    if (tiles > 0x7fffffffLL) return hipErrorInvalidValue;
    int64_t grid = (cu_count() + 7) / 8 * 8;
    const int64_t t8 = (tiles + 7) / 8 * 8;
    if (grid > t8) grid = t8;
    hipLaunchKernelGGL((gemm_bf16_pers_kernel<Kind, 4, 2, GEN, GATHER>), dim3((unsigned)grid),
                       dim3(512), 0, st, p, tiles);
    return hipGetLastError();
}

template <int Kind>
static hipError_t run_f32_bwd(const GemmParams& p, int32_t* gblk, int64_t rows_total,
                              hipStream_t st) {
    const int64_t tiles = grid_blocks<64, 64>(p, gblk, rows_total, st);
    if (tiles <= 0) return hipSuccess;
    if (tiles > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(gemm_f32_bwd_kernel<Kind>, dim3((unsigned)tiles), dim3(256), 0, st, p);
    return hipGetLastError();
}

template <int Kind>
static hipError_t run_f32(const GemmParams& p, int32_t* gblk, int64_t rows_total, hipStream_t st) {
    const int64_t tiles = grid_blocks<64, 64>(p, gblk, rows_total, st);
    if (tiles <= 0) return hipSuccess;
    if (tiles > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(gemm_f32_kernel<Kind>, dim3((unsigned)tiles), dim3(256), 0, st, p);
    return hipGetLastError();
}

hipError_t launch_affinity(const void* h, const void* w, float* s, int64_t T, int64_t E,
                           int64_t D, int dt, ScoreScan* scan, hipStream_t st) {
    GemmParams p = {};
    p.A = h; p.B = w; p.M = T; p.N = E; p.K = D; p.groups = 1;
    p.s_out = s; p.scan = scan;
    if (dt == 0) return run_f32<KIND_AFF>(p, nullptr, T, st);
    if (E <= 64) return run_bf16<KIND_AFF, 128, 64, 2, 2>(p, st);
    return run_bf16<KIND_AFF, 128, 128, 2, 2>(p, st);
}

hipError_t launch_ffn1(const void* h, const int32_t* perm, const void* W1, void* H, int64_t E,
                       int64_t k, int64_t D, int64_t F, int dt, int act, const int32_t* goff,
                       int32_t* gblk, int64_t rows_total, hipStream_t st) {
    GemmParams p = {};
    p.A = h; p.B = W1; p.M = k; p.N = F; p.K = D; p.groups = E;
    p.perm = perm; p.b_gstride = F * D; p.H = H; p.act = act;
    p.goff = goff; p.gblk = gblk;
    if (dt == 0) return run_f32<KIND_FFN1>(p, gblk, rows_total, st);
    const int64_t hb = perm ? rows_total * D * 2 : 0;
    if (pers_fits(D, F, hb)) {
        p.a_bytes = (int)hb;
        return perm ? run_pers<KIND_FFN1, false, true>(p, gblk, rows_total, st)
                    : run_pers<KIND_FFN1>(p, gblk, rows_total, st);
    }
    return run_dma64<KIND_FFN1, 256, 4, 2>(p, gblk, rows_total, st);
}

hipError_t launch_ffn2(const void* H, const int32_t* perm, const void* W2, const float* s,
                       const void* h, void* out, int64_t E, int64_t k, int64_t D, int64_t F,
                       int dt, const int32_t* goff, int32_t* gblk, int64_t rows_total,
                       hipStream_t st) {
    GemmParams p = {};
    p.A = H; p.B = W2; p.M = k; p.N = D; p.K = F; p.groups = E;
    p.perm = perm; p.b_gstride = D * F; p.s_in = s; p.E = E; p.h = h; p.out = out;
    p.goff = goff; p.gblk = gblk;
    if (dt == 0) return run_f32<KIND_FFN2>(p, gblk, rows_total, st);
    if (pers_fits(F, D, 0)) return run_pers<KIND_FFN2>(p, gblk, rows_total, st);
    return run_dma64<KIND_FFN2, 256, 4, 2>(p, gblk, rows_total, st);
}

hipError_t launch_ffn2_ex(const void* H, const int32_t* perm, const void* W2, const float* s,
                          const void* h, void* out, int64_t E, int64_t k, int64_t D, int64_t F,
                          int dt, const int32_t* goff, int32_t* gblk, int64_t rows_total,
                          const Ffn2Epi& epi, hipStream_t st) {
    GemmParams p = {};
    p.A = H; p.B = W2; p.M = k; p.N = D; p.K = F; p.groups = E;
    p.perm = perm; p.b_gstride = D * F; p.s_in = s; p.E = E; p.h = h; p.out = out;
    p.goff = goff; p.gblk = gblk;
    p.epi_general = 1;
    p.epi_gate = epi.gate;
    p.epi_keep = epi.keep;
    p.epi_res = epi.res;
    p.xr = epi.xr;
    p.xo = epi.xo;
    if (dt == 0) return run_f32<KIND_FFN2>(p, gblk, rows_total, st);
    if (pers_fits(F, D, 0)) return run_pers<KIND_FFN2, true>(p, gblk, rows_total, st);
    return run_dma64<KIND_FFN2, 256, 4, 2, true>(p, gblk, rows_total, st);
}

// ---- backward products (ragged groups: group e owns rows goff[e] ..
// goff[e+1]-1 of the grouped order; T = goff[E])

int64_t bwd_nparts(int64_t F, int dt) { return dt == 0 ? (F + 63) / 64 : (F + 255) / 256 * 2; }

hipError_t launch_bwd_z(const void* Xg, const void* W1, const int32_t* perm, const float* s,
                        void* Z, void* gU, int64_t T, int64_t E, int64_t D, int64_t F, int dt,
                        int act, const int32_t* goff, int32_t* gblk, int gate_one,
                        hipStream_t st) {
    GemmParams p = {};
    p.epi_gate = gate_one;
    p.A = Xg; p.B = W1; p.M = T / E; p.N = F; p.K = D; p.groups = E;
    p.perm = perm; p.b_gstride = F * D; p.s_in = s; p.E = E; p.H = Z; p.gu = gU; p.act = act;
    p.goff = goff; p.gblk = gblk;
    if (dt == 0) return run_f32_bwd<KIND_BZ>(p, gblk, T, st);
    return run_pers<KIND_BZ>(p, gblk, T, st);
}

hipError_t launch_bwd_v(const void* dYg, const void* W2, const int32_t* perm, const float* s,
                        const void* Z, void* dZ, float* part, int64_t T, int64_t E, int64_t D,
                        int64_t F, int dt, int act, const int32_t* goff, int32_t* gblk,
                        int gate_one, hipStream_t st) {
    GemmParams p = {};
    p.epi_gate = gate_one;
    p.A = dYg; p.B = W2; p.M = T / E; p.N = F; p.K = D; p.groups = E;
    p.perm = perm; p.b_gstride = D * F; p.ldb = F; p.s_in = s; p.E = E; p.zin = Z; p.H = dZ;
    p.part = part; p.nparts = bwd_nparts(F, dt); p.act = act;
    p.goff = goff; p.gblk = gblk;
    if (dt == 0) return run_f32_bwd<KIND_BV>(p, gblk, T, st);
    return run_pers<KIND_BV>(p, gblk, T, st);
}

hipError_t launch_bwd_x(const void* dZ, const void* W1, const int32_t* perm, const float* s,
                        const void* dYg, const void* w, const float* dl, int mix, void* dh,
                        int64_t T, int64_t E, int64_t D, int64_t F, int dt, const int32_t* goff,
                        int32_t* gblk, void* grouped_out, hipStream_t st) {
    GemmParams p = {};
    p.xo = grouped_out;
    p.A = dZ; p.B = W1; p.M = T / E; p.N = D; p.K = F; p.groups = E;
    p.perm = perm; p.b_gstride = F * D; p.ldb = D; p.s_in = s; p.E = E; p.dyg = dYg; p.wc = w;
    p.dl = dl; p.mix = mix; p.out = dh;
    p.goff = goff; p.gblk = gblk;
    if (dt == 0) return run_f32_bwd<KIND_BX>(p, gblk, T, st);
    return run_pers<KIND_BX>(p, gblk, T, st);
}

hipError_t launch_bwd_w(const void* P, const void* Q, int64_t M, int64_t N, int64_t E,
                        const int32_t* goff, void* dW, int dt, hipStream_t st) {
    GemmParams p = {};
    p.A = P; p.B = Q; p.M = M; p.N = N; p.K = 0; p.groups = E;
    p.lda = M; p.ldb = N; p.kgoff = goff; p.H = dW;
    if (dt == 0) return run_f32_bwd<KIND_BW>(p, nullptr, 0, st);
    return run_pers<KIND_BW>(p, nullptr, 0, st);
}

}  // namespace base
