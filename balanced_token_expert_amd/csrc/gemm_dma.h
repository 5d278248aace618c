// bf16 MFMA GEMM fed by direct global -> LDS loads (included by gemm.hip,
// inside namespace base).
//
// 256 x BN output tile per workgroup of WM x WN waves; K steps of 32 held in
// 4 LDS stages that global_load_lds (16 bytes per lane) fills three K steps
// ahead of the MFMAs, so about 96 KB per CU are in flight -- enough to cover
// HBM latency without registers. Each stage is its own LDS object and the
// K loop is unrolled by the stage count, so the compiler can tell the stage
// being read from the stages being filled and keeps its LDS reads free of
// waits on the loads in flight; the loop waits explicitly for the one K step
// it is about to use. A row of a stage is 4 chunks of 16 bytes; chunk c of
// row r sits at position c ^ ((r >> 2) & 3), so a fragment read (32 rows x
// one chunk per half wave) touches 16 different bank groups. Lanes whose row
// or K range lies outside the operand load a 16-byte block of zeros.

constexpr int kDmaStageBytes = (256 + 256) * 32 * 2;
__shared__ __attribute__((aligned(16))) char g_stage0[kDmaStageBytes];
__shared__ __attribute__((aligned(16))) char g_stage1[kDmaStageBytes];
__shared__ __attribute__((aligned(16))) char g_stage2[kDmaStageBytes];
__shared__ __attribute__((aligned(16))) char g_stage3[kDmaStageBytes];

__device__ __attribute__((aligned(16))) uint4 g_zero16;

template <int S>
BASE_DEV char* dma_stage() {
    return S == 0 ? g_stage0 : (S == 1 ? g_stage1 : (S == 2 ? g_stage2 : g_stage3));
}

BASE_DEV void dma16(const void* src, char* dst) {
    __builtin_amdgcn_global_load_lds((glb_void_t*)src, (lds_void_t*)dst, 16, 0, 0);
}

template <int N>
BASE_DEV void wait_vmcnt() {
    if (N == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    else if (N == 3) asm volatile("s_waitcnt vmcnt(3)" ::: "memory");
    else if (N == 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    else if (N == 6) asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
    else if (N == 8) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    else if (N == 12) asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
    else if (N == 16) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// LAG = 0: a wave reads a K step's fragments right after the barrier that
// makes the step ready, then issues its MFMAs (2 waves per SIMD hide each
// other's LDS latency). LAG = 1: fragments are read one K step ahead of the
// MFMAs that use them (two register sets), for one wave per SIMD with a
// large sub-tile.
template <int Kind, int BN, int WM, int WN, int LAG>
__global__ __launch_bounds__(WM* WN * 64) void gemm_bf16_dma_kernel(GemmParams p) {
    constexpr int BM = 256, BK = 32, S = 4, NT = WM * WN * 64;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int TM = WTM / 32, TN = WTN / 32;
    constexpr int A_BYTES = BM * BK * 2;
    constexpr int AI = BM * (BK / 8) / NT;  // DMA instructions per wave per stage: A
    constexpr int BI = BN * (BK / 8) / NT;  //                                      B
    constexpr int PER = AI + BI;
    static_assert(AI >= 1 && BI >= 1 && TM >= 1 && TN >= 1, "tile shape");
    static_assert(A_BYTES + BN * BK * 2 <= kDmaStageBytes, "stage size");

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    Tile tl;
    if (!locate_tile<BM, BN>(p, xcd_logical(blockIdx.x, gridDim.x), tl)) return;
    const int64_t g = tl.g;
    const int64_t m0 = tl.tm * BM, n0 = tl.tn * BN;
    const uint16_t* A = (const uint16_t*)p.A;
    const uint16_t* B = (const uint16_t*)p.B + g * p.b_gstride;

    // this lane's DMA sources (row pointer + chunk offset, or null)
    const uint16_t* asrc[AI];
    const uint16_t* bsrc[BI];
    int akc[AI], bkc[BI];
#pragma unroll
    for (int j = 0; j < AI; ++j) {
        const int slot = (wave * AI + j) * 64 + lane;
        const int row = slot >> 2, c = (slot & 3) ^ ((row >> 2) & 3);
        akc[j] = c * 8;
        const int64_t m = m0 + row;
        asrc[j] = nullptr;
        if (m < tl.rows) {
            int64_t src;
            if (Kind == KIND_FFN1) src = p.perm[tl.row0 + m];
            else if (Kind == KIND_FFN2) src = tl.row0 + m;
            else src = m;
            asrc[j] = A + src * p.K + c * 8;
        }
    }
#pragma unroll
    for (int j = 0; j < BI; ++j) {
        const int slot = (wave * BI + j) * 64 + lane;
        const int row = slot >> 2, c = (slot & 3) ^ ((row >> 2) & 3);
        bkc[j] = c * 8;
        const int64_t n = n0 + row;
        bsrc[j] = (n < p.N) ? B + n * p.K + c * 8 : nullptr;
    }
    const void* zero = (const void*)&g_zero16;
    auto issue = [&](int64_t kt, char* st) {
        const int64_t k0 = kt * BK;
#pragma unroll
        for (int j = 0; j < AI; ++j) {
            const void* src = (asrc[j] && k0 + akc[j] < p.K) ? (const void*)(asrc[j] + k0) : zero;
            dma16(src, st + (wave * AI + j) * 1024);
        }
#pragma unroll
        for (int j = 0; j < BI; ++j) {
            const void* src = (bsrc[j] && k0 + bkc[j] < p.K) ? (const void*)(bsrc[j] + k0) : zero;
            dma16(src, st + A_BYTES + (wave * BI + j) * 1024);
        }
    };

    // fragment byte offsets inside a stage: [kk][tile]
    int fa[2][TM], fb[2][TN];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        const int c = 2 * kk + (lane >> 5);
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int row = wm * WTM + i * 32 + (lane & 31);
            fa[kk][i] = (row * 4 + (c ^ ((row >> 2) & 3))) * 16;
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int row = wn * WTN + j * 32 + (lane & 31);
            fb[kk][j] = A_BYTES + (row * 4 + (c ^ ((row >> 2) & 3))) * 16;
        }
    }

    f32x16_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    auto load_frags = [&](const char* st, bf16x8_t (&fa_)[2][TM], bf16x8_t (&fb_)[2][TN]) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
            for (int i = 0; i < TM; ++i) fa_[kk][i] = *(const bf16x8_t*)(st + fa[kk][i]);
#pragma unroll
            for (int j = 0; j < TN; ++j) fb_[kk][j] = *(const bf16x8_t*)(st + fb[kk][j]);
        }
    };
    auto mfmas = [&](const bf16x8_t (&fa_)[2][TM], const bf16x8_t (&fb_)[2][TN]) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa_[kk][i], fb_[kk][j],
                                                                         acc[i][j], 0, 0, 0);
    };
    const int64_t nk = (p.K + BK - 1) / BK;
    // wait for K step kt (the loads of the steps issued after it may stay in
    // flight) and for every wave's reads of the stage about to be refilled
    auto ready = [&](int64_t kt) {
        const int64_t rest = nk - 1 - kt;  // K steps issued after kt (at most S - 2)
        if (rest >= 2) wait_vmcnt<2 * PER>();
        else if (rest == 1) wait_vmcnt<PER>();
        else wait_vmcnt<0>();
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // reads of the stage refilled next
        __builtin_amdgcn_s_barrier();
    };

    if (nk > 0) issue(0, dma_stage<0>());
    if (nk > 1) issue(1, dma_stage<1>());
    if (nk > 2) issue(2, dma_stage<2>());
    if (LAG == 0) {
        // both 16-deep halves' fragments are read up front so the second
        // half's reads overlap the first half's MFMAs
        bf16x8_t af[2][TM], bfr[2][TN];
        auto compute = [&](const char* st) {
            load_frags(st, af, bfr);
            mfmas(af, bfr);
        };
        for (int64_t kt = 0; kt < nk; kt += S) {
            ready(kt);
            if (kt + 3 < nk) issue(kt + 3, dma_stage<3>());
            compute(dma_stage<0>());
            if (kt + 1 < nk) {
                ready(kt + 1);
                if (kt + 4 < nk) issue(kt + 4, dma_stage<0>());
                compute(dma_stage<1>());
            }
            if (kt + 2 < nk) {
                ready(kt + 2);
                if (kt + 5 < nk) issue(kt + 5, dma_stage<1>());
                compute(dma_stage<2>());
            }
            if (kt + 3 < nk) {
                ready(kt + 3);
                if (kt + 6 < nk) issue(kt + 6, dma_stage<2>());
                compute(dma_stage<3>());
            }
        }
    } else {
        // step kt: make step kt+1 ready, refill kt's stage with step kt+4,
        // read step kt+1's fragments, then the MFMAs of step kt
        bf16x8_t a0[2][TM], b0[2][TN], a1[2][TM], b1[2][TN];
        if (nk > 0) {
            ready(0);
            load_frags(dma_stage<0>(), a0, b0);
        }
        for (int64_t kt = 0; kt < nk; kt += S) {
            if (kt + 1 < nk) {
                ready(kt + 1);
                if (kt + 4 < nk) issue(kt + 4, dma_stage<0>());
                load_frags(dma_stage<1>(), a1, b1);
            }
            mfmas(a0, b0);
            if (kt + 1 >= nk) break;
            if (kt + 2 < nk) {
                ready(kt + 2);
                if (kt + 5 < nk) issue(kt + 5, dma_stage<1>());
                load_frags(dma_stage<2>(), a0, b0);
            }
            mfmas(a1, b1);
            if (kt + 2 >= nk) break;
            if (kt + 3 < nk) {
                ready(kt + 3);
                if (kt + 6 < nk) issue(kt + 6, dma_stage<2>());
                load_frags(dma_stage<3>(), a1, b1);
            }
            mfmas(a0, b0);
            if (kt + 3 >= nk) break;
            if (kt + 4 < nk) {
                ready(kt + 4);
                if (kt + 7 < nk) issue(kt + 7, dma_stage<3>());
                load_frags(dma_stage<0>(), a0, b0);
            }
            mfmas(a1, b1);
        }
    }
    store_tile<Kind, TM, TN>(p, acc, tl, m0 + wm * WTM, n0 + wn * WTN, lane);
}
