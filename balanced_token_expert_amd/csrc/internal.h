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
    int64_t tail[16];
};

// Optional event marks of the auction's parts (base_set_auction_events).
void auction_mark(int i, hipStream_t st);

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

// ---- backward products (gemm.hip). Rows are grouped (row r of group e is
// token perm[r]); group e owns rows goff[e] .. goff[e+1]-1, T = goff[E];
// gblk: E+1 ints of scratch. Gate g_r = sigmoid(s[perm[r], e]).
// gate_one != 0 takes g = 1 (the blocks of a layer-norm expert, whose
// upstream gradient already holds the gate).
// Z = Xg W1_e^T and gU = g act(Z), both T x F.
hipError_t launch_bwd_z(const void* Xg, const void* W1, const int32_t* perm, const float* s,
                        void* Z, void* gU, int64_t T, int64_t E, int64_t D, int64_t F, int dt,
                        int act, const int32_t* goff, int32_t* gblk, int gate_one,
                        hipStream_t st);
// V = dYg W2_e (T x F); dZ = g V act'(Z); part[r * bwd_nparts(F, dt) + j]
// = partial sums over column blocks of V . act(Z)
int64_t bwd_nparts(int64_t F, int dt);
hipError_t launch_bwd_v(const void* dYg, const void* W2, const int32_t* perm, const float* s,
                        const void* Z, void* dZ, float* part, int64_t T, int64_t E, int64_t D,
                        int64_t F, int dt, int act, const int32_t* goff, int32_t* gblk,
                        int gate_one, hipStream_t st);
// dh[perm[r]] = (dZ W1_e)[r] + c dYg[r] + dl[r] w_e, c = 1 (mix 0) or 1 - g;
// with grouped_out != nullptr instead grouped_out[r] = (dZ W1_e)[r]
hipError_t launch_bwd_x(const void* dZ, const void* W1, const int32_t* perm, const float* s,
                        const void* dYg, const void* w, const float* dl, int mix, void* dh,
                        int64_t T, int64_t E, int64_t D, int64_t F, int dt, const int32_t* goff,
                        int32_t* gblk, void* grouped_out, hipStream_t st);
// dW_e = P_e^T Q_e: P rows of length M, Q rows of length N, summed over the
// rows of group e; dW is E x M x N. M % 8 == N % 8 == 0 for bf16.
hipError_t launch_bwd_w(const void* P, const void* Q, int64_t M, int64_t N, int64_t E,
                        const int32_t* goff, void* dW, int dt, hipStream_t st);

// ---- grad.hip
// Xg[r] = h[perm[r]], dYg[r] = dy[perm[r]] (rows of D values of dtype dt)
hipError_t launch_gather2(const void* h, const void* dy, const int32_t* perm, void* Xg,
                          void* dYg, int64_t T, int64_t D, int dt, hipStream_t st);
// dl[r] = g (1 - g) dg with dg = sum of the row's nparts partials, minus
// dYg[r] . Xg[r] for the convex mix; g = sigmoid(s[perm[r], e]), e the
// group of r
hipError_t launch_gate_grad(const float* part, int64_t nparts, const void* Xg, const void* dYg,
                            const int32_t* perm, const int32_t* goff, const float* s, int mix,
                            float* dl, int64_t T, int64_t E, int64_t D, int dt, hipStream_t st);
// dw[e] = sum over the rows r of group e of dl[r] Xg[r]
hipError_t launch_centroid_grad(const float* dl, const void* Xg, const int32_t* goff, void* dw,
                                int64_t E, int64_t D, int dt, hipStream_t st);

// experts of layer-norm blocks (grouped rows; expert of row r = its group):
// dXa = g dYg (fp32) and dXo (dtype dt) = the same, dl = g (1 - g) dg with
// dg = dYg . XN (mix 0) or dYg . (XN - X0) (mix 1)
hipError_t launch_block_gate(const void* X0, const void* XN, const void* dYg, const int32_t* perm,
                             const int32_t* goff, const float* s, int mix, float* dXa, void* dXo,
                             float* dl, int64_t T, int64_t E, int64_t D, int dt, hipStream_t st);
// layer-norm backward of the rows X (gamma: E x D fp32 or null): dXa += dx,
// dXo = dXa (dtype dt), stats[2r] = mean, stats[2r+1] = rstd
hipError_t launch_ln_backward(const void* X, const void* dY, const float* gamma,
                              const int32_t* goff, double eps, float* dXa, void* dXo,
                              float* stats, int64_t T, int64_t E, int64_t D, int dt,
                              hipStream_t st);
// dgamma[e] = sum dY (X - mean) rstd, dbeta[e] = sum dY over group e's rows
// (E x D fp32 each; either may be null)
hipError_t launch_ln_param_grad(const void* X, const void* dY, const float* stats,
                                const int32_t* goff, float* dgamma, float* dbeta, int64_t E,
                                int64_t D, int dt, hipStream_t st);
// dh[perm[r]] = dXa[r] + c dYg[r] + dl[r] w_e, c = 1 (mix 0) or 1 - g
hipError_t launch_finish_dh(const float* dXa, const void* dYg, const float* dl, const void* w,
                            const int32_t* perm, const int32_t* goff, const float* s, int mix,
                            void* dh, int64_t T, int64_t E, int64_t D, int dt, hipStream_t st);

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
// largest expert count the grouping kernels take (their per-block LDS holds
// five E-entry tables)
constexpr int64_t kPermMaxE = 4096;
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
