// bf16 MFMA GEMM fed by direct global -> LDS loads (included by gemm.hip,
// inside namespace base). Used for both expert products.
//
// 256 x BN output tile per workgroup of WM x WN waves; K steps of 64 held in
// two LDS stages of 64 KB that global_load_lds (16 bytes per lane) fills one
// step ahead of the MFMAs. A stage row is 128 bytes, so the 8 lanes that fill
// one row read a whole 128-byte line: half the L2 requests of 32-deep stages
// for the same bytes (an L2-resident DMA probe moved 27 TB/s this way against
// 16 TB/s with 64-byte row pieces; in the GEMM the 64-deep stages beat four
// 32-deep stages with three steps of lead by about 9 %). Each stage is its
// own LDS object and the K loop is unrolled by the stage count, so the
// compiler can tell the stage being read from the stage being filled; the
// loop waits explicitly for the step it is about to use. Chunk c of row r
// sits at position c ^ swz8(r), which keeps the fragment reads (32 rows x one
// chunk per half wave) free of LDS bank conflicts. Lanes whose row or K range
// lies outside the operand load a 16-byte block of zeros.
//
// Operands of the backward products may be stored "k-major" instead (rows of
// k with M or N contiguous, e.g. W2 read as W2^T, or token rows summed over
// in a weight gradient). Such a stage holds 64 k-rows of 256 values (512
// bytes, 32 chunks; chunk c of row r at c ^ swz_t(r)), filled by the same
// 16-byte DMA, and its fragments come from two ds_read_b64_tr_b16 per
// 32 x 16 fragment: within each 16-lane group, the lane that supplies row
// r0 + j, columns 4a .. 4a+3 hands element b of them to lane 4a + b, so lane
// l ends up with 4 consecutive k of column l % 32 (rows 8 (l / 32) .. + 3 and
// + 4 .. + 7 over the two reads), the layout the MFMA takes.
//
// The MFMAs take the weight fragment as their first operand, so each
// accumulator holds C transposed: a lane owns one output row and runs of 4
// consecutive columns. The epilogue then writes 8-byte pieces of rows and
// needs one gate and one token index per row per lane.

__device__ __attribute__((aligned(16))) uint4 g_zero16;

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));

BASE_DEV void dma16(const void* src, char* dst) {
    __builtin_amdgcn_global_load_lds((glb_void_t*)src, (lds_void_t*)dst, 16, 0, 0);
}

// The same 16-byte DMA through a raw buffer descriptor: a byte offset at or
// past the descriptor's size (kOob included) loads zeros.
typedef __amdgpu_buffer_rsrc_t buf_rsrc_t;
constexpr uint32_t kOob = 0x80000000u;
// The arguments are uniform; readfirstlane tells the compiler so, which keeps
// the descriptor in scalar registers (else each load gets a waterfall loop).
BASE_DEV buf_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = (uint64_t)base;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    const uint32_t n = __builtin_amdgcn_readfirstlane(bytes);
    void* b = (void*)(((uint64_t)hi << 32) | lo);
    // 0x00020000: the descriptor word 3 of raw dword buffers on gfx9
    return __builtin_amdgcn_make_buffer_rsrc(b, 0, (int)n, 0x00020000);
}
BASE_DEV void dma16_buf(buf_rsrc_t r, uint32_t voff, char* dst) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)dst, 16, (int)voff, 0, 0, 0);
}

// s_waitcnt through the builtin rather than inline asm, so that the
// compiler's own wait insertion knows which loads have completed; with an
// opaque wait it assumes the stage about to be read may still be in flight
// and drains every outstanding DMA first.
// gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8.
template <int N>
BASE_DEV void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (((N >> 4) & 3) << 14) | (7 << 4) | (15 << 8));
}

BASE_DEV void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4)); }

// GELU(x) = x/2 (1 + erf(x / sqrt 2)) with erf from Abramowitz & Stegun,
// Handbook of Mathematical Functions, formula 7.1.26 (|error| <= 1.5e-7):
// erf(z) = 1 - P(u) e^(-z^2), u = 1 / (1 + p z), z >= 0. Written so that the
// negative side uses P(u) e^(-z^2) = 1 - erf(z) directly, without
// cancellation. Two transcendental instructions (rcp, exp2) and 12 FMA-class
// ones. The result is rounded to bf16 afterwards (relative error up to
// 2^-8), far above the formula's error.
BASE_DEV float gelu_as7126(float x) {
    const float z = fabsf(x) * 0.70710678118654752f;
    const float u = __builtin_amdgcn_rcpf(fmaf(0.3275911f, z, 1.0f));
    float q = fmaf(u, 1.061405429f, -1.453152027f);
    q = fmaf(u, q, 1.421413741f);
    q = fmaf(u, q, -0.284496736f);
    q = fmaf(u, q, 0.254829592f);
    q *= u;
    const float tail = q * __builtin_amdgcn_exp2f(-(z * z) * 1.44269504088896341f);  // 1 - erf(z)
    const float two_phi = x >= 0.0f ? 2.0f - tail : tail;  // 1 + erf(x / sqrt 2)
    return 0.5f * x * two_phi;
}

// Epilogue for one wave's TM x TN block of transposed 32x32 accumulators:
// acc[i][j][4q + c] is C[row][col] with
//   row = mw + i*32 + lane%32,  col = nw + j*32 + 8q + 4*(lane/32) + c.
// FFN1: H[row0 + row][col] = act(C) (bf16). FFN2 (eq. 1): for token
// t = perm[row0 + row], out[t][col] = bf16(gate * C + h[t][col]), with the
// row's gate sigma(s[t][g]) and t loaded before the K loop.
template <int Kind, int TM, int TN, bool FULL>
BASE_DEV void dma_epilogue_rows(const GemmParams& p, f32x16_t (&acc)[TM][TN], const Tile& tl,
                                int64_t mw, int64_t nw, int lane, const int32_t (&trow)[TM],
                                const float (&gate)[TM]) {
    // FULL: every row and column of the wave's block exists and N % 4 == 0,
    // so no piece needs a bounds check and all pieces are 8-byte aligned
    const bool vec = FULL || (p.N & 3) == 0;
    const int64_t cb = nw + 4 * (lane >> 5);
    if (Kind == KIND_FFN1) {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int64_t m = mw + i * 32 + (lane & 31);
            if (!FULL && m >= tl.rows) continue;
            uint16_t* hrow = (uint16_t*)p.H + (tl.row0 + m) * p.N;
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int64_t n = cb + j * 32 + 8 * q;
                    f32x4_t y;
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const float v = acc[i][j][4 * q + c];
                        y[c] = p.act ? gelu_as7126(v) : fmaxf(v, 0.0f);
                    }
                    if (vec) {
                        if (FULL || n < p.N)
                            *(bf16x4_t*)(hrow + n) = __builtin_convertvector(y, bf16x4_t);
                    } else {
#pragma unroll
                        for (int c = 0; c < 4; ++c)
                            if (n + c < p.N) hrow[n + c] = f32_to_bf16(y[c]);
                    }
                }
        }
    } else {
        // all residual pieces of the lane are loaded first (one latency)
        bf16x4_t res[TM][TN][4];
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int64_t m = mw + i * 32 + (lane & 31);
            const uint16_t* hrow = (const uint16_t*)p.h + (int64_t)trow[i] * p.N;
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int64_t n = cb + j * 32 + 8 * q;
                    if (FULL || (m < tl.rows && vec && n < p.N))
                        res[i][j][q] = *(const bf16x4_t*)(hrow + n);
                }
        }
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int64_t m = mw + i * 32 + (lane & 31);
            if (!FULL && m >= tl.rows) continue;
            const int64_t t = trow[i];
            const uint16_t* hrow = (const uint16_t*)p.h + t * p.N;
            uint16_t* orow = (uint16_t*)p.out + t * p.N;
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int64_t n = cb + j * 32 + 8 * q;
                    if (vec) {
                        if (!FULL && n >= p.N) continue;
                        const f32x4_t r = __builtin_convertvector(res[i][j][q], f32x4_t);
                        f32x4_t y;
#pragma unroll
                        for (int c = 0; c < 4; ++c) y[c] = fmaf(gate[i], acc[i][j][4 * q + c], r[c]);
                        *(bf16x4_t*)(orow + n) = __builtin_convertvector(y, bf16x4_t);
                    } else {
#pragma unroll
                        for (int c = 0; c < 4; ++c)
                            if (n + c < p.N)
                                orow[n + c] = f32_to_bf16(
                                    fmaf(gate[i], acc[i][j][4 * q + c], bf16_to_f32(hrow[n + c])));
                    }
                }
        }
    }
}

// FFN2 epilogue of the layer variants (same accumulator layout as above):
// y = g (R + C) + c2 h[t] with the choices of GemmParams' epi_* fields,
// written to out[t] or to the grouped row xo[row0 + row].
template <int TM, int TN>
BASE_DEV void dma_epilogue_general(const GemmParams& p, f32x16_t (&acc)[TM][TN], const Tile& tl,
                                   int64_t mw, int64_t nw, int lane, const int32_t (&trow)[TM],
                                   const float (&gate)[TM]) {
    const bool vec = (p.N & 3) == 0;
    const int64_t cb = nw + 4 * (lane >> 5);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int64_t m = mw + i * 32 + (lane & 31);
        if (m >= tl.rows) continue;
        const int64_t t = trow[i];
        const float g = gate[i];
        const float c2 = p.epi_keep == 0 ? 1.0f : (p.epi_keep == 1 ? 1.0f - g : 0.0f);
        const bool need_h = c2 != 0.0f || p.epi_res == 1;
        const uint16_t* hrow = (const uint16_t*)p.h + t * p.N;
        const uint16_t* rrow = (p.epi_res == 2) ? (const uint16_t*)p.xr + (tl.row0 + m) * p.N : hrow;
        uint16_t* orow = p.xo ? (uint16_t*)p.xo + (tl.row0 + m) * p.N : (uint16_t*)p.out + t * p.N;
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t n = cb + j * 32 + 8 * q;
                if (vec) {
                    if (n >= p.N) continue;
                    f32x4_t hv = {0.0f, 0.0f, 0.0f, 0.0f}, rv = {0.0f, 0.0f, 0.0f, 0.0f};
                    if (need_h) hv = __builtin_convertvector(*(const bf16x4_t*)(hrow + n), f32x4_t);
                    if (p.epi_res == 1) rv = hv;
                    else if (p.epi_res == 2)
                        rv = __builtin_convertvector(*(const bf16x4_t*)(rrow + n), f32x4_t);
                    f32x4_t y;
#pragma unroll
                    for (int c = 0; c < 4; ++c) y[c] = fmaf(g, rv[c] + acc[i][j][4 * q + c], c2 * hv[c]);
                    *(bf16x4_t*)(orow + n) = __builtin_convertvector(y, bf16x4_t);
                } else {
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        if (n + c >= p.N) continue;
                        const float hv = need_h ? bf16_to_f32(hrow[n + c]) : 0.0f;
                        const float rv = p.epi_res == 1 ? hv
                                         : (p.epi_res == 2 ? bf16_to_f32(rrow[n + c]) : 0.0f);
                        orow[n + c] = f32_to_bf16(fmaf(g, rv + acc[i][j][4 * q + c], c2 * hv));
                    }
                }
            }
    }
}

template <int Kind, int TM, int TN>
BASE_DEV void dma_epilogue(const GemmParams& p, f32x16_t (&acc)[TM][TN], const Tile& tl,
                           int64_t mw, int64_t nw, int lane, const int32_t (&trow)[TM],
                           const float (&gate)[TM]) {
    if ((p.N & 3) == 0 && nw + TN * 32 <= p.N && mw + TM * 32 <= tl.rows)
        dma_epilogue_rows<Kind, TM, TN, true>(p, acc, tl, mw, nw, lane, trow, gate);
    else
        dma_epilogue_rows<Kind, TM, TN, false>(p, acc, tl, mw, nw, lane, trow, gate);
}

constexpr int kDma64StageBytes = (256 + 256) * 64 * 2;
__shared__ __attribute__((aligned(16))) char g_d64_0[kDma64StageBytes];
__shared__ __attribute__((aligned(16))) char g_d64_1[kDma64StageBytes];

template <int S>
BASE_DEV char* dma64_stage() {
    return S == 0 ? g_d64_0 : g_d64_1;
}

// 8 chunks of 16 bytes per row: rows 2 apart differ in bits 1..3 of the row,
// so 16 consecutive rows (one ds_read_b128 pass) hit 16 distinct bank groups.
BASE_DEV int swz8(int r) { return (r >> 1) & 7; }

// k-major stages (32 chunks per row): the rows one transpose read touches,
// r0 + 0..3 (first half wave) and r0 + 8..11 (second half), land in distinct
// 64-byte bank groups.
BASE_DEV int swz_t(int r) { return ((r & 3) << 2) | ((r & 8) << 1); }

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

// 32 x 16 fragment of a k-major stage: rows k .. k+3 and k+4 .. k+7 from the
// lane's address (the second read 4 rows = 2048 bytes further)
BASE_DEV bf16x8_t tr_frag(const char* a) {
    const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)a);
    const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(a + 4 * 512));
    const s16x8_t v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8_t, v);
}

// GELU (the A&S 7.1.26 form above) and its derivative Phi(x) + x phi(x),
// sharing the exp: e^(-z^2) with z = |x| / sqrt 2 is e^(-x^2 / 2).
BASE_DEV void gelu_grad_as7126(float x, float& u, float& du) {
    const float z = fabsf(x) * 0.70710678118654752f;
    const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, z, 1.0f));
    float q = fmaf(t, 1.061405429f, -1.453152027f);
    q = fmaf(t, q, 1.421413741f);
    q = fmaf(t, q, -0.284496736f);
    q = fmaf(t, q, 0.254829592f);
    q *= t;
    const float ex = __builtin_amdgcn_exp2f(-(z * z) * 1.44269504088896341f);
    const float tail = q * ex;
    const float two_phi = x >= 0.0f ? 2.0f - tail : tail;
    u = 0.5f * x * two_phi;
    du = fmaf(x * ex, 0.39894228040143268f, 0.5f * two_phi);
}

BASE_DEV void act_grad(float x, int act, float& u, float& du) {
    if (act) {
        gelu_grad_as7126(x, u, du);
    } else {
        u = fmaxf(x, 0.0f);
        du = x > 0.0f ? 1.0f : 0.0f;
    }
}

// Staged stores of 32 rows (set i) of a wave's 64 x 128 output block (bf16):
// out[j][q] holds row 32 i + lane % 32, columns 32 j + 8 q + 4 (lane / 32)
// .. + 3. Written directly, each store instruction puts 16 bytes into each
// of 32 rows, and HBM writes of outputs with long rows ran 1.7-2.4x the
// bytes stored (lines left L2 partly written). Here the 32 rows go through
// the wave's 4 KB of LDS one 64-column half at a time (16-byte chunk c of
// row r at chunk c ^ (r % 8): one write instruction covers 32 rows in the
// fewest bank cycles) and come back as whole 128-byte row pieces: each store
// instruction writes 8 rows x 128 bytes, i.e. whole lines. The code has no
// divergent branch: every lane takes part in every LDS exchange, and the
// stores go through a buffer descriptor of the block (dst: its row 0,
// column 0; rows ld elements apart; its size ends at the last row that
// exists), so rows past the block and columns at or past ncols are dropped
// by the descriptor's bound (an exec-masked LDS exchange here once had a
// read moved inside the masked region by the compiler).
__shared__ __attribute__((aligned(16))) char g_epi[8 * 4096];

typedef int i32x4_t __attribute__((ext_vector_type(4)));

// val(j, q) gives out[j][q] (computed just before its half is staged, so
// only half a row set of packed values is live at a time).
constexpr int kCpolNT = 2;  // buffer-instruction cache policy: non-temporal

template <int TN, class Val>
BASE_DEV void store_rows_staged(char* lds, int lane, int i, Val&& val, buf_rsrc_t dst, int64_t ld,
                                int64_t ncols) {
    static_assert(TN == 4, "128 columns per wave");
    const int lr = lane & 31;
#pragma unroll
    for (int jh = 0; jh < 2; ++jh) {
        uint2 o[2][4];
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
            for (int q = 0; q < 4; ++q) o[jj][q] = val(2 * jh + jj, q);
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                *(uint2*)(lds + lr * 128 + (((4 * jj + q) ^ (lr & 7)) << 4) + 8 * (lane >> 5)) =
                    o[jj][q];
        // one wave owns the buffer and its LDS operations run in order
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int r = 8 * s + (lane >> 3), c = lane & 7;
            const uint4 v = *(const uint4*)(lds + r * 128 + ((c ^ (r & 7)) << 4));
            const int64_t col = 64 * jh + 8 * c;
            const uint32_t off = col < ncols ? (uint32_t)(((32 * i + r) * ld + col) * 2) : kOob;
            // non-temporal: these outputs (GBs, read by a later launch) would
            // otherwise evict the operand panels neighbouring tiles re-read
            // from L2 (cache-policy bit NT)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4_t, v), dst, (int)off, 0,
                                                   kCpolNT);
        }
    }
}

BASE_DEV uint2 pack_bf16x4(f32x4_t y) {
    return __builtin_bit_cast(uint2, __builtin_convertvector(y, bf16x4_t));
}

// Descriptor of a wave's block of grouped rows of length ld: its row 0,
// column 0, sized to end at its last existing row (the launcher keeps
// 64 ld * 2 below 2^31).
BASE_DEV buf_rsrc_t block_rsrc(const void* base, const Tile& tl, int64_t mw, int64_t nw,
                               int64_t ld) {
    const int64_t vr = tl.rows - mw < 0 ? 0 : (tl.rows - mw > 64 ? 64 : tl.rows - mw);
    return make_rsrc((const uint16_t*)base + (tl.row0 + mw) * ld + nw, (uint32_t)(vr * ld * 2));
}

// Epilogue of the weight gradients: plain bf16 rows of dW, stored through
// LDS in whole row pieces (store_rows_staged). Large workload: dW2 3.83 ->
// 3.08 ms and dW1 3.51 -> 3.19 ms against direct 8-byte stores.
template <int TM, int TN>
BASE_DEV void dma_epilogue_bw(const GemmParams& p, f32x16_t (&acc)[TM][TN], const Tile& tl,
                              int64_t mw, int64_t nw, int lane) {
    char* lds = g_epi + (threadIdx.x >> 6) * 4096;
    const buf_rsrc_t dst = block_rsrc(p.H, tl, mw, nw, p.N);
#pragma unroll
    for (int i = 0; i < TM; ++i)
        store_rows_staged<TN>(
            lds, lane, i,
            [&](int j, int q) {
                f32x4_t y;
#pragma unroll
                for (int c = 0; c < 4; ++c) y[c] = acc[i][j][4 * q + c];
                return pack_bf16x4(y);
            },
            dst, p.N, p.N - nw);
}

// The recomputation of Z: stores Z and g act(Z) with the same staged stores
// (large workload: 3.17 -> 2.63 ms). V -> dZ keeps direct stores: holding
// the Z values it reads beside the staged ones spilled registers and made it
// a third slower.
template <int TM, int TN>
BASE_DEV void dma_epilogue_z(const GemmParams& p, f32x16_t (&acc)[TM][TN], const Tile& tl,
                             int64_t mw, int64_t nw, int lane, const float (&gate)[TM]) {
    char* lds = g_epi + (threadIdx.x >> 6) * 4096;
    const buf_rsrc_t zr = block_rsrc(p.H, tl, mw, nw, p.N);
    const buf_rsrc_t ur = block_rsrc(p.gu, tl, mw, nw, p.N);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const float g = gate[i];
        store_rows_staged<TN>(
            lds, lane, i,
            [&](int j, int q) {
                f32x4_t y;
#pragma unroll
                for (int c = 0; c < 4; ++c) y[c] = acc[i][j][4 * q + c];
                return pack_bf16x4(y);
            },
            zr, p.N, p.N - nw);
        store_rows_staged<TN>(
            lds, lane, i,
            [&](int j, int q) {
                f32x4_t gu;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    float u, du;
                    act_grad(acc[i][j][4 * q + c], p.act, u, du);
                    gu[c] = g * u;
                }
                return pack_bf16x4(gu);
            },
            ur, p.N, p.N - nw);
    }
}

// Epilogue of the backward products (accumulator layout as above; rows are
// grouped rows, or output rows of dW for BW). wpart: this wave's column of
// the BV partial sums.
template <int Kind, int TM, int TN>
BASE_DEV void dma_epilogue_bwd(const GemmParams& p, f32x16_t (&acc)[TM][TN], const Tile& tl,
                               int64_t mw, int64_t nw, int lane, const int32_t (&trow)[TM],
                               const float (&gate)[TM], int64_t wpart) {
    const int64_t cb = nw + 4 * (lane >> 5);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int64_t m = mw + i * 32 + (lane & 31);
        const bool rowok = m < tl.rows;
        const int64_t row = tl.row0 + m;
        const float g = gate[i];
        float psum = 0.0f;
        float cx = 1.0f, dlr = 0.0f;
        if (Kind == KIND_BX && rowok) {
            cx = p.mix ? 1.0f - g : 1.0f;
            dlr = p.dl[row];
        }
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t n = cb + j * 32 + 8 * q;
                // N % 8 == 0: a run of 4 is wholly inside or outside
                if (!rowok || n >= p.N) continue;
                f32x4_t y;
#pragma unroll
                for (int c = 0; c < 4; ++c) y[c] = acc[i][j][4 * q + c];
                if (Kind == KIND_BZ) {
                    f32x4_t gu;
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        float u, du;
                        act_grad(y[c], p.act, u, du);
                        gu[c] = g * u;
                    }
                    *(bf16x4_t*)((uint16_t*)p.H + row * p.N + n) = __builtin_convertvector(y, bf16x4_t);
                    *(bf16x4_t*)((uint16_t*)p.gu + row * p.N + n) = __builtin_convertvector(gu, bf16x4_t);
                } else if (Kind == KIND_BV) {
                    const f32x4_t z = __builtin_convertvector(
                        *(const bf16x4_t*)((const uint16_t*)p.zin + row * p.N + n), f32x4_t);
                    f32x4_t dz;
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        float u, du;
                        act_grad(z[c], p.act, u, du);
                        psum = fmaf(y[c], u, psum);
                        dz[c] = g * y[c] * du;
                    }
                    *(bf16x4_t*)((uint16_t*)p.H + row * p.N + n) = __builtin_convertvector(dz, bf16x4_t);
                } else if (Kind == KIND_BX && p.xo) {
                    // plain grouped rows (the input gradient of a layer-norm block)
                    *(bf16x4_t*)((uint16_t*)p.xo + row * p.N + n) = __builtin_convertvector(y, bf16x4_t);
                } else if (Kind == KIND_BX) {
                    const f32x4_t d = __builtin_convertvector(
                        *(const bf16x4_t*)((const uint16_t*)p.dyg + row * p.N + n), f32x4_t);
                    const f32x4_t wv = __builtin_convertvector(
                        *(const bf16x4_t*)((const uint16_t*)p.wc + tl.g * p.N + n), f32x4_t);
                    f32x4_t o;
#pragma unroll
                    for (int c = 0; c < 4; ++c) o[c] = fmaf(dlr, wv[c], fmaf(cx, d[c], y[c]));
                    *(bf16x4_t*)((uint16_t*)p.out + (int64_t)trow[i] * p.N + n) =
                        __builtin_convertvector(o, bf16x4_t);
                } else {
                    *(bf16x4_t*)((uint16_t*)p.H + row * p.N + n) = __builtin_convertvector(y, bf16x4_t);
                }
            }
        if (Kind == KIND_BV) {
            psum += __shfl_xor(psum, 32, 64);
            if (lane < 32 && rowok) p.part[row * p.nparts + wpart] = psum;
        }
    }
}

// GEN: the FFN2 epilogue of the layer variants instead of eq. 1's
template <int Kind, int BN, int WM, int WN, bool GEN = false>
__global__ __launch_bounds__(WM* WN * 64) void gemm_bf16_dma64_kernel(GemmParams p) {
    static_assert(Kind != KIND_AFF, "expert products only");
    // operands read k-major (see above): A for the weight gradients, B for
    // every backward product but the recomputation of Z
    constexpr bool AT = Kind == KIND_BW;
    constexpr bool BT = Kind == KIND_BV || Kind == KIND_BX || Kind == KIND_BW;
    constexpr bool ROWTOK = Kind == KIND_FFN2 || Kind == KIND_BZ || Kind == KIND_BV ||
                            Kind == KIND_BX;  // rows need their token and gate
    static_assert(!BT || BN == 256, "k-major stages are 256 wide");
    constexpr bool BWD = Kind >= KIND_BZ;
    constexpr int BM = 256, BK = 64, NT = WM * WN * 64;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int TM = WTM / 32, TN = WTN / 32;
    constexpr int ROWB = BK * 2;            // bytes of a stage row
    constexpr int CPR = ROWB / 16;          // 16-byte chunks per row
    constexpr int A_BYTES = BM * ROWB;
    constexpr int AI = BM * CPR / NT;       // DMA instructions per wave per stage: A
    constexpr int BI = BN * CPR / NT;       //                                      B
    static_assert(AI >= 1 && BI >= 1 && TM >= 1 && TN >= 1, "tile shape");
    static_assert(A_BYTES + BN * ROWB <= kDma64StageBytes, "stage size");

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    Tile tl;
    if (!locate_tile<BM, BN>(p, xcd_logical(blockIdx.x, gridDim.x), tl)) return;
    const int64_t g = tl.g;
    const int64_t m0 = tl.tm * BM, n0 = tl.tn * BN;
    const uint16_t* A = (const uint16_t*)p.A;
    const uint16_t* B = (const uint16_t*)p.B + g * p.b_gstride;
    // the K range: a weight gradient sums its group's rows
    int64_t kbeg = 0, Kc = p.K;
    if (Kind == KIND_BW) {
        kbeg = p.kgoff ? p.kgoff[g] : g * p.K;
        Kc = p.kgoff ? p.kgoff[g + 1] - kbeg : p.K;
    }

    int32_t trow[TM];
    float gate[TM];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        trow[i] = 0;
        gate[i] = 0.0f;
        const int64_t m = m0 + wm * WTM + i * 32 + (lane & 31);
        if (ROWTOK && m < tl.rows) {
            trow[i] = p.perm[tl.row0 + m];
            gate[i] = (GEN && p.epi_gate) ? 1.0f : sigmoid_f32(p.s_in[(int64_t)trow[i] * p.E + g]);
        }
    }

    // forward products, per DMA slot: source of the stage's first step
    // (null: zeros) and its k offset inside a step
    const uint16_t* asrc[BWD ? 1 : AI];
    const uint16_t* bsrc[BWD ? 1 : BI];
    int akc[BWD ? 1 : AI], bkc[BWD ? 1 : BI];
    // backward products (every operand row grouped, none gathered): the
    // slots load through a buffer descriptor rebuilt each step, so a slot's
    // source is a 32-bit byte offset (one register) and the descriptor's
    // bound turns rows past the operand, and k-rows past the step's window,
    // into zeros; a column block past M / N carries an out-of-range marker.
    uint32_t aoff[BWD ? AI : 1], boff[BWD ? BI : 1];
    // the k of slot j inside a step: k-major operands the row, others the
    // chunk's first k
    auto slot_k = [&](bool kmaj, int wj) -> int {
        const int slot = wj * 64 + lane;
        if (kmaj) return slot >> 5;
        return (((slot % CPR) ^ swz8(slot / CPR)) * 8);
    };
    if constexpr (BWD) {
#pragma unroll
        for (int j = 0; j < AI; ++j) {
            const int slot = (wave * AI + j) * 64 + lane;
            if (AT) {
                const int row = slot >> 5, c = (slot & 31) ^ swz_t(row);
                aoff[j] = (m0 + 8 * c < tl.rows) ? (uint32_t)(row * p.lda + 8 * c) * 2u : kOob;
            } else {
                const int row = slot / CPR, c = (slot % CPR) ^ swz8(row);
                aoff[j] = (uint32_t)(row * p.K + c * 8) * 2u;
            }
        }
#pragma unroll
        for (int j = 0; j < BI; ++j) {
            const int slot = (wave * BI + j) * 64 + lane;
            if (BT) {
                const int row = slot >> 5, c = (slot & 31) ^ swz_t(row);
                boff[j] = (n0 + 8 * c < p.N) ? (uint32_t)(row * p.ldb + 8 * c) * 2u : kOob;
            } else {
                const int row = slot / CPR, c = (slot % CPR) ^ swz8(row);
                boff[j] = (uint32_t)(row * p.K + c * 8) * 2u;
            }
        }
    } else {
        // expert products of the forward pass: a pointer per slot (A rows
        // may be gathered through perm)
#pragma unroll
        for (int j = 0; j < AI; ++j) {
            const int slot = (wave * AI + j) * 64 + lane;
            const int row = slot / CPR, c = (slot % CPR) ^ swz8(row);
            akc[j] = c * 8;
            const int64_t m = m0 + row;
            asrc[j] = nullptr;
            if (m < tl.rows) {
                const int64_t src = (Kind == KIND_FFN1 && p.perm) ? p.perm[tl.row0 + m] : tl.row0 + m;
                asrc[j] = A + src * p.K + c * 8;
            }
        }
#pragma unroll
        for (int j = 0; j < BI; ++j) {
            const int slot = (wave * BI + j) * 64 + lane;
            const int row = slot / CPR, c = (slot % CPR) ^ swz8(row);
            bkc[j] = c * 8;
            const int64_t n = n0 + row;
            bsrc[j] = (n < p.N) ? B + n * p.K + c * 8 : nullptr;
        }
    }
    // 32-bit copies of the sizes the backward descriptors are built from
    const int kc32 = (int)Kc, k32 = (int)p.K, lda32 = (int)p.lda, ldb32 = (int)p.ldb;
    const int rows32 = (int)tl.rows, m032 = (int)m0, n32 = (int)p.N, n032 = (int)n0;
    const void* zero = (const void*)&g_zero16;
    auto issue = [&](int64_t kt, char* st) {
        const int64_t k0 = kt * BK;
        if constexpr (BWD) {
            // descriptors of this step: k-major operands cover the step's
            // (up to) 64 k-rows from column m0 / n0 on; the others the tile's
            // valid rows from k0 on (their k tail is masked per slot)
            // 32-bit min / max only (the launcher keeps every size below
            // 2^21): branches here would merge paths inside the K loop and
            // cost the compiler its tracking of which stage the DMAs write
            const int k0i = (int)k0;
            const int kv = min(max(kc32 - k0i, 0), BK);
            int an, bn;
            const uint16_t *ab, *bb;
            if (AT) {
                ab = A + (kbeg + k0) * p.lda + m0;
                an = max(kv * lda32 + (rows32 - m032) - lda32, 0);
            } else {
                ab = A + (tl.row0 + m0) * p.K + k0;
                an = max(min(rows32 - m032, BM) * k32 - k0i, 0);
            }
            if (BT) {
                bb = B + (kbeg + k0) * p.ldb + n0;
                bn = max(kv * ldb32 + (n32 - n032) - ldb32, 0);
            } else {
                bb = B + n0 * p.K + k0;
                bn = max(min(n32 - n032, BN) * k32 - k0i, 0);
            }
            an *= 2;
            bn *= 2;
            const buf_rsrc_t ra = make_rsrc(ab, (uint32_t)an), rb = make_rsrc(bb, (uint32_t)bn);
#pragma unroll
            for (int j = 0; j < AI; ++j) {
                uint32_t v = aoff[j];
                if (!AT && k0 + slot_k(false, wave * AI + j) >= Kc) v = kOob;
                dma16_buf(ra, v, st + (wave * AI + j) * 1024);
            }
#pragma unroll
            for (int j = 0; j < BI; ++j) {
                uint32_t v = boff[j];
                if (!BT && k0 + slot_k(false, wave * BI + j) >= Kc) v = kOob;
                dma16_buf(rb, v, st + A_BYTES + (wave * BI + j) * 1024);
            }
            return;
        }
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

    // A lane's fragment rows all share bits 1..3 (they differ by multiples of
    // 32 rows), hence one swizzle term; fragment i / j then sits a fixed
    // number of bytes after the lane's first row.
    const int sx = swz8(lane & 31);
    const int arow0 = (wm * WTM + (lane & 31)) * ROWB;
    const int brow0 = A_BYTES + (wn * WTN + (lane & 31)) * ROWB;
    // k-major fragments: the lane's byte offset for the wave's first
    // fragment (first row, chunk and byte within it). Fragment i starts 4 i
    // chunks further; the swizzle XORs chunk bits 2..4 and leaves bits 0..1
    // (the lane's place inside the fragment), so its offset is the first one
    // XOR 64 i bytes.
    int atoff = 0, btoff = 0;
    {
        const int r0 = 8 * (lane >> 5) + ((lane & 15) >> 2);
        const int sw = swz_t(r0);
        const int low = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
        const int byte = r0 * 512 + 8 * (lane & 1);
        static_assert(WTM % 32 == 0 && WTN % 32 == 0 && BM == 256, "fragment chunk bits");
        if (AT) atoff = byte + (((((wm * WTM) >> 3) ^ sw) | low) << 4);
        if (BT) btoff = A_BYTES + byte + (((((wn * WTN) >> 3) ^ sw) | low) << 4);
    }

    f32x16_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // K steps of 64, padded to an even count (zero blocks past K)
    const int64_t nk = ((Kc + 2 * BK - 1) / (2 * BK)) * 2;
    // wait for the step about to be read (the only one in flight) and for
    // every wave's reads of the stage refilled next
    auto ready = [&]() {
        wait_vmcnt<0>();
        wait_lgkmcnt0();
        __builtin_amdgcn_s_barrier();
    };

    bf16x8_t a0[TM], b0[TN], a1[TM], b1[TN];
    // sub-step s (16 deep) of the stage at st: chunk 2s + lane/32
    auto load_sub = [&](const char* st, int s, bf16x8_t (&fa_)[TM], bf16x8_t (&fb_)[TN]) {
        const int co = ((2 * s + (lane >> 5)) ^ sx) * 16;
#pragma unroll
        for (int i = 0; i < TM; ++i)
            fa_[i] = AT ? tr_frag(st + (atoff ^ (64 * i)) + 16 * s * 512)
                        : *(const bf16x8_t*)(st + arow0 + co + i * 32 * ROWB);
#pragma unroll
        for (int j = 0; j < TN; ++j)
            fb_[j] = BT ? tr_frag(st + (btoff ^ (64 * j)) + 16 * s * 512)
                        : *(const bf16x8_t*)(st + brow0 + co + j * 32 * ROWB);
    };
    auto mfma_sub = [&](const bf16x8_t (&fa_)[TM], const bf16x8_t (&fb_)[TN]) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb_[j], fa_[i], acc[i][j], 0, 0, 0);
    };
    // step kt in stage `cur`, kt+1 in `next` (issued one step earlier); the
    // fragments of sub-step s+1 are read while sub-step s is multiplied
    auto step = [&](int64_t kt, char* cur, char* next) {
        load_sub(cur, 1, a1, b1);
        __builtin_amdgcn_sched_barrier(0);
        mfma_sub(a0, b0);
        load_sub(cur, 2, a0, b0);
        __builtin_amdgcn_sched_barrier(0);
        mfma_sub(a1, b1);
        load_sub(cur, 3, a1, b1);
        __builtin_amdgcn_sched_barrier(0);
        mfma_sub(a0, b0);
        ready();
        issue(kt + 2, cur);
        load_sub(next, 0, a0, b0);
        __builtin_amdgcn_sched_barrier(0);
        mfma_sub(a1, b1);
    };

    issue(0, dma64_stage<0>());
    issue(1, dma64_stage<1>());
    ready();
    load_sub(dma64_stage<0>(), 0, a0, b0);
    for (int64_t kt = 0; kt < nk; kt += 2) {
        step(kt, dma64_stage<0>(), dma64_stage<1>());
        step(kt + 1, dma64_stage<1>(), dma64_stage<0>());
    }
    wait_vmcnt<0>();
    if constexpr (Kind >= KIND_BZ)
        dma_epilogue_bwd<Kind, TM, TN>(p, acc, tl, m0 + wm * WTM, n0 + wn * WTN, lane, trow, gate,
                                       tl.tn * WN + wn);
    else if constexpr (GEN && Kind == KIND_FFN2)
        dma_epilogue_general<TM, TN>(p, acc, tl, m0 + wm * WTM, n0 + wn * WTN, lane, trow, gate);
    else
        dma_epilogue<Kind, TM, TN>(p, acc, tl, m0 + wm * WTM, n0 + wn * WTN, lane, trow, gate);
}

// Persistent form of the expert products: one block per CU walks a run of
// tiles (each XCD owns a contiguous run of the logical tiles; its blocks take
// every (blocks per XCD)-th one, so the tiles in flight on an XCD are
// neighbours that share operand tiles in its L2). The last two K steps of a
// tile issue the DMAs of the next tile's first two steps, so when its K loop
// ends the registers already hold the next tile's first fragments and its
// epilogue runs while the next tile's first loads are in flight. A slot's
// 32-bit offset inside a step's window does not depend on the tile (the
// per-step buffer descriptor carries the tile), except for the first
// forward product's rows gathered through perm: their offsets from the
// start of h are loaded for the next tile while the current one runs, and
// a row past its group loads zeros. Rows past a group, the k
// tail of an operand with k contiguous, and k-rows past the step's window
// read zeros; columns past M / N of a k-major operand read the start of the
// next k-row of the same tensor (zeros past its end), which only reaches
// accumulator rows / columns the epilogue discards.
BASE_DEV int uni32(int v) { return __builtin_amdgcn_readfirstlane(v); }
BASE_DEV int64_t uni64(int64_t v) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// GATHER: the first forward product with its rows gathered through perm
template <int Kind, int WM, int WN, bool GEN = false, bool GATHER = false>
__global__ __launch_bounds__(WM* WN * 64) void gemm_bf16_pers_kernel(GemmParams p, int64_t ntiles) {
    static_assert(Kind != KIND_AFF, "expert products");
    static_assert(!GATHER || Kind == KIND_FFN1, "only the first forward product gathers");
    constexpr bool AT = Kind == KIND_BW;
    constexpr bool BT = Kind == KIND_BV || Kind == KIND_BX || Kind == KIND_BW;
    constexpr bool ROWTOK = Kind != KIND_BW && Kind != KIND_FFN1;
    constexpr bool gather = GATHER;
    constexpr int BM = 256, BN = 256, BK = 64, NT = WM * WN * 64;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int TM = WTM / 32, TN = WTN / 32;
    constexpr int ROWB = BK * 2, CPR = ROWB / 16;
    constexpr int A_BYTES = BM * ROWB;
    constexpr int AI = BM * CPR / NT, BI = BN * CPR / NT;
    static_assert(AI >= 1 && BI >= 1 && TM >= 1 && TN >= 1, "tile shape");

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;

    // the launch covers ntiles logical tiles (ragged groups: the block map's
    // own count)
    const int64_t nt = p.goff ? (int64_t)p.gblk[p.groups] : ntiles;
    const int64_t xcd = blockIdx.x & 7, bper = gridDim.x >> 3;
    const int64_t per = nt >> 3, rem = nt & 7;
    const int64_t t0 = xcd * per + (xcd < rem ? xcd : rem);
    const int64_t t_end = t0 + per + (xcd < rem ? 1 : 0);
    int64_t lid = t0 + (blockIdx.x >> 3);

    struct TS {
        Tile t;
        int64_t kbeg;
        int Kc, nk, ok;
    };
    auto tile_at = [&](int64_t l) -> TS {
        TS s;
        s.t = Tile{0, 0, 0, 0, 0};
        s.kbeg = 0;
        s.Kc = 0;
        s.nk = 0;
        s.ok = l < t_end && locate_tile<BM, BN>(p, l, s.t);
        if (s.ok) {
            s.Kc = (int)p.K;
            if (Kind == KIND_BW) {
                s.kbeg = p.kgoff ? p.kgoff[s.t.g] : s.t.g * p.K;
                s.Kc = p.kgoff ? (int)(p.kgoff[s.t.g + 1] - s.kbeg) : (int)p.K;
            }
            // at least two steps (an empty group runs two zero steps): the
            // last two steps of every tile load the next tile's first two
            s.nk = s.Kc > 0 ? ((s.Kc + 2 * BK - 1) / (2 * BK)) * 2 : 2;
        }
        // uniform by construction; readfirstlane keeps them in scalar
        // registers, so choosing between this tile and the next one inside
        // the K loop is a scalar select, not a branch or a vector select
        s.t.g = uni64(s.t.g);
        s.t.tm = uni64(s.t.tm);
        s.t.tn = uni64(s.t.tn);
        s.t.row0 = uni64(s.t.row0);
        s.t.rows = uni64(s.t.rows);
        s.kbeg = uni64(s.kbeg);
        s.Kc = uni32(s.Kc);
        s.nk = uni32(s.nk);
        s.ok = uni32(s.ok);
        return s;
    };
    TS cur = tile_at(lid);
    if (!cur.ok) return;
    TS nxt = tile_at(lid + bper);

    uint32_t aoff[AI], boff[BI], agn[AI];
    // k offset of a k-contiguous slot: with an even number of slots per wave,
    // slot j's row is 8 (wave AI + j) + lane / 8 and its chunk
    // (lane % 8) ^ (lane / 16) ^ 4 (j % 2), so one register serves all j
    static_assert(AI % 2 == 0 && BI % 2 == 0 && CPR == 8, "slot chunk pattern");
    const int kc0 = ((lane & 7) ^ (lane >> 4)) * 8;
#pragma unroll
    for (int j = 0; j < AI; ++j) {
        const int slot = (wave * AI + j) * 64 + lane;
        if (AT) {
            const int row = slot >> 5, c = (slot & 31) ^ swz_t(row);
            aoff[j] = (uint32_t)(row * p.lda + 8 * c) * 2u;
        } else {
            const int row = slot / CPR, c = (slot % CPR) ^ swz8(row);
            aoff[j] = (uint32_t)(row * p.K + c * 8) * 2u;
        }
    }
#pragma unroll
    for (int j = 0; j < BI; ++j) {
        const int slot = (wave * BI + j) * 64 + lane;
        if (BT) {
            const int row = slot >> 5, c = (slot & 31) ^ swz_t(row);
            boff[j] = (uint32_t)(row * p.ldb + 8 * c) * 2u;
        } else {
            const int row = slot / CPR, c = (slot % CPR) ^ swz8(row);
            boff[j] = (uint32_t)(row * p.K + c * 8) * 2u;
        }
    }
    // gathered rows: byte offsets from the start of h of tile s's slots
    // (kOob past the group)
    auto gather_offs = [&](const TS& s, uint32_t (&o)[AI]) {
#pragma unroll
        for (int j = 0; j < AI; ++j) {
            const int slot = (wave * AI + j) * 64 + lane;
            const int row = slot / CPR, c = (slot % CPR) ^ swz8(row);
            const int64_t m = s.t.tm * BM + row;
            o[j] = kOob;
            if (s.ok && m < s.t.rows)
                o[j] = (uint32_t)((int64_t)p.perm[s.t.row0 + m] * p.K + c * 8) * 2u;
        }
    };
    if (gather) {
        gather_offs(cur, aoff);
        gather_offs(nxt, agn);
    }
    const uint16_t* A = (const uint16_t*)p.A;
    const uint16_t* Bp = (const uint16_t*)p.B;
    const int k32 = (int)p.K, lda32 = (int)p.lda, ldb32 = (int)p.ldb;

    // DMAs of step k0 / BK of tile s into stage st (a tile that does not
    // exist loads zeros)
    auto issue = [&](const TS& s, bool sn, int k0, char* st) {
        const int kv = min(max(s.Kc - k0, 0), BK);
        const int m0 = (int)(s.t.tm * BM), n0 = (int)(s.t.tn * BN);
        const uint16_t* B = Bp + s.t.g * p.b_gstride;
        int an, bn;
        const uint16_t *ab, *bb;
        if (AT) {
            ab = A + (s.kbeg + k0) * p.lda + m0;
            an = max(kv * lda32 - m0, 0);
        } else if (gather) {
            ab = A + k0;  // the whole of h (its size fits 32 bits: checked at launch)
            an = max(p.a_bytes / 2 - k0, 0);
        } else {
            ab = A + (s.t.row0 + m0) * p.K + k0;
            an = max(min((int)s.t.rows - m0, BM) * k32 - k0, 0);
        }
        if (BT) {
            bb = B + (s.kbeg + k0) * p.ldb + n0;
            bn = max(kv * ldb32 - n0, 0);
        } else {
            bb = B + (int64_t)n0 * p.K + k0;
            bn = max(min((int)p.N - n0, BN) * k32 - k0, 0);
        }
        if (!s.ok) an = bn = 0;
        const buf_rsrc_t ra = make_rsrc(ab, (uint32_t)an * 2u), rb = make_rsrc(bb, (uint32_t)bn * 2u);
#pragma unroll
        for (int j = 0; j < AI; ++j) {
            uint32_t v = (gather && sn) ? agn[j] : aoff[j];
            if (!AT && k0 + (kc0 ^ (32 * (j & 1))) >= s.Kc) v = kOob;
            dma16_buf(ra, v, st + (wave * AI + j) * 1024);
        }
#pragma unroll
        for (int j = 0; j < BI; ++j) {
            uint32_t v = boff[j];
            if (!BT && k0 + (kc0 ^ (32 * (j & 1))) >= s.Kc) v = kOob;
            dma16_buf(rb, v, st + A_BYTES + (wave * BI + j) * 1024);
        }
    };

    int32_t trow[TM];
    float gate[TM];
    auto rows_of = [&](const TS& s, int32_t (&tr)[TM], float (&ga)[TM]) {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            tr[i] = 0;
            ga[i] = 0.0f;
            const int64_t m = s.t.tm * BM + wm * WTM + i * 32 + (lane & 31);
            if (ROWTOK && s.ok && m < s.t.rows) {
                tr[i] = p.perm[s.t.row0 + m];
                // epi_gate: a gate of 1 (the layer variants' inner blocks, and
                // the backward of layer-norm blocks, whose upstream is g dy)
                ga[i] = p.epi_gate ? 1.0f : sigmoid_f32(p.s_in[(int64_t)tr[i] * p.E + s.t.g]);
            }
        }
    };
    rows_of(cur, trow, gate);

    int atoff = 0, btoff = 0;
    {
        const int r0 = 8 * (lane >> 5) + ((lane & 15) >> 2);
        const int sw = swz_t(r0);
        const int low = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
        const int byte = r0 * 512 + 8 * (lane & 1);
        if (AT) atoff = byte + (((((wm * WTM) >> 3) ^ sw) | low) << 4);
        if (BT) btoff = A_BYTES + byte + (((((wn * WTN) >> 3) ^ sw) | low) << 4);
    }
    const int sx = swz8(lane & 31);
    const int arow0 = (wm * WTM + (lane & 31)) * ROWB;
    const int brow0 = A_BYTES + (wn * WTN + (lane & 31)) * ROWB;

    f32x16_t acc[TM][TN];
    auto ready = [&]() {
        wait_vmcnt<0>();
        wait_lgkmcnt0();
        __builtin_amdgcn_s_barrier();
    };
    bf16x8_t a0[TM], b0[TN], a1[TM], b1[TN];
    auto load_sub = [&](const char* st, int s, bf16x8_t (&fa_)[TM], bf16x8_t (&fb_)[TN]) {
        const int co = ((2 * s + (lane >> 5)) ^ sx) * 16;
#pragma unroll
        for (int i = 0; i < TM; ++i)
            fa_[i] = AT ? tr_frag(st + (atoff ^ (64 * i)) + 16 * s * 512)
                        : *(const bf16x8_t*)(st + arow0 + co + i * 32 * ROWB);
#pragma unroll
        for (int j = 0; j < TN; ++j)
            fb_[j] = BT ? tr_frag(st + (btoff ^ (64 * j)) + 16 * s * 512)
                        : *(const bf16x8_t*)(st + brow0 + co + j * 32 * ROWB);
    };
    auto mfma_sub = [&](const bf16x8_t (&fa_)[TM], const bf16x8_t (&fb_)[TN]) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb_[j], fa_[i], acc[i][j], 0, 0, 0);
    };
    // step kt of the current tile in stage `cs`; refills `cs` with step
    // kt + 2 of this tile or, in the last two steps, of the next tile
    auto step = [&](int kt, char* cs, char* ns) {
        load_sub(cs, 1, a1, b1);
        __builtin_amdgcn_sched_barrier(0);
        mfma_sub(a0, b0);
        load_sub(cs, 2, a0, b0);
        __builtin_amdgcn_sched_barrier(0);
        mfma_sub(a1, b1);
        load_sub(cs, 3, a1, b1);
        __builtin_amdgcn_sched_barrier(0);
        mfma_sub(a0, b0);
        ready();
        const bool to_next = kt + 2 >= cur.nk;
        issue(to_next ? nxt : cur, to_next, (to_next ? kt + 2 - cur.nk : kt + 2) * BK, cs);
        load_sub(ns, 0, a0, b0);
        __builtin_amdgcn_sched_barrier(0);
        mfma_sub(a1, b1);
    };

    issue(cur, false, 0, dma64_stage<0>());
    issue(cur, false, BK, dma64_stage<1>());
    ready();
    load_sub(dma64_stage<0>(), 0, a0, b0);
    for (;;) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
        for (int kt = 0; kt < cur.nk; kt += 2) {
            step(kt, dma64_stage<0>(), dma64_stage<1>());
            step(kt + 1, dma64_stage<1>(), dma64_stage<0>());
        }
        int32_t trn[TM];
        float gan[TM];
        rows_of(nxt, trn, gan);
        const int64_t mw = cur.t.tm * BM + wm * WTM, nw = cur.t.tn * BN + wn * WTN;
        if constexpr (Kind == KIND_BW)
            dma_epilogue_bw<TM, TN>(p, acc, cur.t, mw, nw, lane);
        else if constexpr (Kind == KIND_BZ)
            dma_epilogue_z<TM, TN>(p, acc, cur.t, mw, nw, lane, gate);
        else if constexpr (Kind >= KIND_BZ)
            dma_epilogue_bwd<Kind, TM, TN>(p, acc, cur.t, mw, nw, lane, trow, gate,
                                           cur.t.tn * WN + wn);
        else if constexpr (GEN && Kind == KIND_FFN2)
            dma_epilogue_general<TM, TN>(p, acc, cur.t, mw, nw, lane, trow, gate);
        else
            dma_epilogue<Kind, TM, TN>(p, acc, cur.t, mw, nw, lane, trow, gate);
        if (!nxt.ok) break;
        cur = nxt;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            trow[i] = trn[i];
            gate[i] = gan[i];
        }
        lid += bper;
        nxt = tile_at(lid + bper);
        if (gather) {
#pragma unroll
            for (int j = 0; j < AI; ++j) aoff[j] = agn[j];
            gather_offs(nxt, agn);
        }
    }
    wait_vmcnt<0>();
}
