// Host-side launchers shared between the kernel files and the C ABI (api.cpp).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace base {

// Sanitizing summary of a score matrix: the order-preserving key of the
// smallest finite score (0xffffffff if none) and the count of NaN/inf.
struct ScoreScan {
    uint32_t min_key;
    uint32_t nonfinite;
};

// Device-side stats mirror of base_auction_stats.
struct AucStatsDev {
    int32_t status;
    int32_t phases;
    int64_t bids[16];
    int64_t rounds[16];
};

// ---- gemm.cpp / gemm.hip
// s = h w^T, fp32 out; also fills *scan (must be initialised by scan_init).
hipError_t launch_affinity(const void* h, const void* w, float* s, int64_t T,
                           int64_t E, int64_t D, int dt, ScoreScan* scan,
                           hipStream_t st);
// Expert groups: equal (goff == nullptr: group e owns rows e*k .. e*k+k-1 of
// the grouped order) or ragged (group e owns rows goff[e] .. goff[e+1]-1,
// rows_total = goff[E]; gblk is E+1 ints of scratch for the launch's block
// map).
// H[r, :] = act(h[perm[r], :] W1_e^T) for every row r of group e (bf16 or fp32 H);
// with perm == nullptr the rows of h are already grouped: act(h[r, :] W1_e^T)
hipError_t launch_ffn1(const void* h, const int32_t* perm, const void* W1,
                       void* H, int64_t E, int64_t k, int64_t D, int64_t F,
                       int dt, int act, const int32_t* goff, int32_t* gblk,
                       int64_t rows_total, hipStream_t st);
// out[perm[r], :] = sigmoid(s[perm[r], e]) * (H W2_e^T)[r, :] + h[perm[r], :]
hipError_t launch_ffn2(const void* H, const int32_t* perm, const void* W2,
                       const float* s, const void* h, void* out, int64_t E,
                       int64_t k, int64_t D, int64_t F, int dt,
                       const int32_t* goff, int32_t* gblk, int64_t rows_total,
                       hipStream_t st);

// Generalised second product (layer variants): with C = H W2_e^T and
// t = perm[r], y = g (R + C) + c2 h[t, :] where
//   g  = sigmoid(s[t, e]) (gate == 0) or 1 (gate == 1),
//   c2 = 1 (keep == 0), 1 - g (keep == 1) or 0 (keep == 2),
//   R  = 0 (res == 0), h[t, :] (res == 1) or xr[r, :] (res == 2, grouped rows);
// y goes to out[t, :], or to the grouped row xo[r, :] when xo != nullptr.
// (Eq. 1 is gate 0, keep 0, res 0, scattered.) xr may equal xo.
struct Ffn2Epi {
    int gate, keep, res;
    const void* xr;
    void* xo;
};
hipError_t launch_ffn2_ex(const void* H, const int32_t* perm, const void* W2,
                          const float* s, const void* h, void* out, int64_t E,
                          int64_t k, int64_t D, int64_t F, int dt,
                          const int32_t* goff, int32_t* gblk, int64_t rows_total,
                          const Ffn2Epi& epi, hipStream_t st);

// ---- layernorm.hip
// Y[r, :] = LN(X[r, :]) * gamma[e] + beta[e] over D, e = assign[perm[r]] the
// row's expert, with X[r, :] = x[perm[r], :] (gather != 0) or x[r, :]
// (grouped rows). gamma / beta: E x D fp32 or nullptr (ones / zeros). The
// statistics are fp32; Y has dtype dt.
hipError_t launch_layernorm(const void* x, int gather, const int32_t* perm,
                            const int32_t* assign, const float* gamma,
                            const float* beta, double eps, void* Y, int64_t T,
                            int64_t E, int64_t D, int dt, hipStream_t st);

// ---- route.hip
hipError_t launch_scan_init(ScoreScan* scan, hipStream_t st);
hipError_t launch_stats_reset(AucStatsDev* st, hipStream_t s);
hipError_t launch_scan_scores(const float* s, int64_t n, ScoreScan* scan,
                              hipStream_t st);
hipError_t launch_greedy(const float* s, int64_t T, int64_t E,
                         const ScoreScan* scan, int32_t* assign,
                         int32_t* counts, hipStream_t st);
size_t perm_ws_bytes(int64_t T, int64_t E);
// Stable grouping of tokens by expert. If want_k > 0 also checks that every
// expert holds exactly want_k tokens and all ids are in range, else sets
// *status = BASE_ERR_UNBALANCED (status may be NULL when want_k == 0).
hipError_t launch_perm(const int32_t* assign, int64_t T, int64_t E,
                       int32_t* perm, int32_t* offsets, int32_t* counts,
                       int64_t want_k, int32_t* status, void* ws,
                       hipStream_t st);

// ---- auction.hip
size_t auction_ws_bytes(int64_t T, int64_t E);
hipError_t launch_auction(const float* s, int64_t T, int64_t E,
                          double eps_start, double eps_end, double eps_factor,
                          int64_t max_bids, const ScoreScan* scan,
                          int32_t* assign, int32_t* perm, int32_t* offsets,
                          double* prices, AucStatsDev* stats, void* ws,
                          hipStream_t st);

}  // namespace base
