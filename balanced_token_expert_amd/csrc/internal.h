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
// H[r, :] = act(h[perm[r], :] W1_e^T) for every row r of group e (bf16 or fp32 H)
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
