// Balanced assignment of "BASE Layers" eq. 2 (sec. 3.2.1) by a token-side
// auction with eps-scaling, on gfx950.
//
// Problem: maximise sum_t s[t][a_t] with exactly k = T/E tokens per expert.
// Each expert owns k slots; a token t facing prices pi_e computes its values
// v_e = s[t][e] - pi_e, its best expert b1 (lowest id on ties), the best value
// v1 and the best value over the other experts v2, and bids
// beta = pi_b1 + (v1 - v2) + eps for a slot of b1. pi_e is the expert's floor
// p_e while it has a free slot, else the lowest bid it holds; a bid into a
// full expert evicts that lowest holder (equal bids: the higher token id
// goes), who must bid again. When no token is left unassigned every expert is
// full and p_e := its lowest held bid. Phases run with eps_start,
// eps_start/f, ..., eps_end, keeping prices and clearing the assignment.
// Every held token satisfies s[t][e] - p_e >= max_e' (s[t][e'] - p_e') - eps,
// so the result is within T*eps_end of the optimum (and is the optimum when
// eps_end is below the optimality gap over T). The paper's own listing
// (appendix fig. 9) has experts bidding for tokens; this is the same
// primal-dual idea from the token side, which needs only per-token
// max/second-max reductions and per-expert prices.
//
// GPU structure per phase:
//   bulk rounds (all CUs): every unassigned token bids against the round's
//     prices at once (one wave per token, wave-level max/second-max); then one
//     workgroup per expert keeps the k best of its holders and new bidders
//     (bitonic sort in LDS) and returns the rest to the bidder list.
//   tail (one persistent workgroup): once few tokens are left, each wave
//     follows a displacement chain -- bid, take the expert's lock in LDS,
//     evict its lowest holder, continue with the evicted token. Prices,
//     counts and, per expert, a sorted list of its L lowest holders live in
//     LDS, so a step needs one score-row load (often from an LDS cache) plus
//     LDS work; the list is rebuilt from the expert's slots in global memory
//     only when it runs dry.
// Prices and bids are fp64: exactness needs eps below gap/T, far below fp32
// resolution at prices of order one.
#include <float.h>

#include "common.h"
#include "internal.h"

namespace base {

// multi-CU rounds per phase (at most). Small capacities keep more bidders
// in conflict for longer: at k = 128 (16k tokens, 128 experts) 32 rounds cut
// the solve from 12.0 to 9.3 ms, while at k = 256 and 512 more than 16
// rounds were neutral or slower (measured medians of 10 solves).
constexpr int kBulkRounds = 16;
constexpr int kBulkRoundsSmallK = 32;
constexpr int64_t kSmallK = 128;
constexpr int kTailMax = 64;         // bidders left when the tail takes over
constexpr int kResolveCap = 2048;    // bidders sorted at once per expert
constexpr int kBulkKMax = 2048;      // bulk rounds need k <= this
constexpr int32_t kErrNotConverged = -5;
constexpr int32_t kErrNonfinite = -6;
constexpr int32_t kNoTok = 0x7fffffff;

// lowest-holder list length per expert (LDS budget of the tail; at most 64,
// one entry per lane). A longer list means fewer rebuilds from the slots.
static int low_len(int64_t E) {
    return E <= 64 ? 64 : (E <= 128 ? 32 : (E <= 256 ? 16 : (E <= 512 ? 8 : 4)));
}

struct AucCtl {
    int32_t cur;          // bidder list in use (0/1)
    int32_t bulk_done;    // the tail owns the rest of this phase
    int32_t identity;     // the bidder list is 0..T-1 (round 0)
    int32_t done_blocks;  // resolve blocks finished (last one flips cur)
    int32_t nbid[2];
    int32_t abort;        // a device error is set: skip all work
    int32_t pad;
    unsigned long long bids_total;
    unsigned long long bids_phase;
    long long rounds_phase;
};

struct AucWs {
    AucCtl* ctl;
    double* floor_;    // E   price floors p_e
    double* pi;        // E   prices for the next bulk round
    int32_t* cnt;      // E   holders per expert
    int32_t* nlow;     // E   entries in the lowest-holder list
    int32_t* comp;     // E   1 if the list holds every holder
    double* lowb;      // E*L lowest holders, eviction order: bid
    int32_t* lowt;     // E*L                                 token
    int32_t* lows;     // E*L                                 slot
    int32_t* list0;    // T
    int32_t* list1;    // T
    int32_t* bexp;     // T   bid of token t: expert
    double* bval;      // T   bid of token t: amount
    int32_t* stok;     // E*k slot tokens
    double* sbid;      // E*k slot bids
    int L;
};

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

static AucWs carve(void* ws, int64_t T, int64_t E) {
    char* p = (char*)ws;
    const int L = low_len(E);
    AucWs w;
    w.L = L;
    w.ctl = (AucCtl*)p; p += align256(sizeof(AucCtl));
    w.floor_ = (double*)p; p += align256(E * 8);
    w.pi = (double*)p; p += align256(E * 8);
    w.cnt = (int32_t*)p; p += align256(E * 4);
    w.nlow = (int32_t*)p; p += align256(E * 4);
    w.comp = (int32_t*)p; p += align256(E * 4);
    w.lowb = (double*)p; p += align256(E * L * 8);
    w.lowt = (int32_t*)p; p += align256(E * L * 4);
    w.lows = (int32_t*)p; p += align256(E * L * 4);
    w.list0 = (int32_t*)p; p += align256(T * 4);
    w.list1 = (int32_t*)p; p += align256(T * 4);
    w.bexp = (int32_t*)p; p += align256(T * 4);
    w.bval = (double*)p; p += align256(T * 8);
    w.stok = (int32_t*)p; p += align256(T * 4);
    w.sbid = (double*)p; p += align256(T * 8);
    return w;
}

size_t auction_ws_bytes(int64_t T, int64_t E) {
    const int L = low_len(E);
    return align256(sizeof(AucCtl)) + 2 * align256(E * 8) + 3 * align256(E * 4) +
           align256(E * L * 8) + 2 * align256(E * L * 4) + 4 * align256(T * 4) +
           2 * align256(T * 8) + 256;
}

// ---------------------------------------------------------------- helpers

struct Sani {
    bool fix;
    float repl;
};

BASE_DEV Sani read_sani(const ScoreScan* scan) {
    Sani s;
    s.fix = scan->nonfinite != 0;
    s.repl = scan->min_key == 0xffffffffu ? 0.0f : f32_unkey(scan->min_key);
    return s;
}

template <int NCH>
BASE_DEV void load_row(const float* s, int64_t t, int64_t E, int lane, Sani sn, float (&v)[NCH]) {
    const float* row = s + t * E;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int64_t e = lane + 64 * c;
        float x = (e < E) ? row[e] : 0.0f;
        if (sn.fix && !is_finite_f32(x)) x = sn.repl;
        v[c] = x;
    }
}

// Best expert (lowest id on ties), best value and the best value over the
// other experts, of s[t][e] - pi[e], reduced over the wave in one pass: each
// lane keeps its top two values and the pairs are merged by DPP (row steps,
// then row broadcasts; lane 63 ends with the wave's pair); the best expert is
// then found by ballots. pb returns the price of b1 exactly as used for v1
// (prices in LDS may be raised by other waves meanwhile; the bid must use one
// consistent value).
BASE_DEV void top2_merge(double& m1, double& m2, double o1, double o2) {
    const double hi = fmax(m1, o1), lo = fmin(m1, o1);
    m2 = fmax(lo, fmax(m2, o2));
    m1 = hi;
}
template <int CTRL>
BASE_DEV void top2_step(double& m1, double& m2) {
    top2_merge(m1, m2, dpp_f64<CTRL>(m1), dpp_f64<CTRL>(m2));
}
template <int CTRL, int ROWS>
BASE_DEV void top2_rows(double& m1, double& m2) {
    // rows outside ROWS see their own pair, which merges to itself only if
    // it is not counted twice: keep them unchanged
    const double o1 = dpp_rows_f64<CTRL, ROWS>(m1), o2 = dpp_rows_f64<CTRL, ROWS>(m2);
    double n1 = m1, n2 = m2;
    top2_merge(n1, n2, o1, o2);
    const int row = (int)(__lane_id() >> 4);
    if ((ROWS >> row) & 1) { m1 = n1; m2 = n2; }
}

// core of best_two: the prices of this lane's experts (lane + 64 c) are given
template <int NCH>
BASE_DEV void best_two_pv(const float (&v)[NCH], const double (&pv)[NCH], int64_t E, int lane,
                          int& b1, double& v1, double& v2, double& pb) {
    double val[NCH];
    double m1 = -DBL_MAX, m2 = -DBL_MAX;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int e = lane + 64 * c;
        val[c] = -DBL_MAX;
        if (e < E) {
            val[c] = (double)v[c] - pv[c];
            top2_merge(m1, m2, val[c], -DBL_MAX);
        }
    }
    top2_step<kDppXor1>(m1, m2);
    top2_step<kDppXor2>(m1, m2);
    top2_step<kDppHalfMirror>(m1, m2);
    top2_step<kDppMirror>(m1, m2);
    top2_rows<kDppBcast15, 0xA>(m1, m2);
    top2_rows<kDppBcast31, 0xC>(m1, m2);
    const double vmax = readlane_f64(m1, 63);
    double sec = readlane_f64(m2, 63);
    int bi = -1;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const unsigned long long m = __ballot(lane + 64 * c < E && val[c] == vmax);
        if (bi < 0 && m) bi = 64 * c + __builtin_ctzll(m);
    }
    if (E == 1) sec = vmax;
    double mine = 0.0;
#pragma unroll
    for (int c = 0; c < NCH; ++c)
        if (c == (bi >> 6)) mine = pv[c];
    b1 = bi;
    v1 = vmax;
    v2 = sec;
    pb = readlane_f64(mine, bi & 63);
}

template <int NCH, typename PiT>
BASE_DEV void best_two(const float (&v)[NCH], PiT pi, int64_t E, int lane, int& b1, double& v1,
                       double& v2, double& pb) {
    double pv[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int e = lane + 64 * c;
        pv[c] = (e < E) ? pi[e] : 0.0;
    }
    best_two_pv<NCH>(v, pv, E, lane, b1, v1, v2, pb);
}

// The bid beta = pb + (v1 - v2) + eps. It is at least the next double above
// pb, so a bid always outbids the price it was made against even where eps
// is below the resolution of the prices (then eps is effectively larger).
BASE_DEV double bid_amount(double pb, double v1, double v2, double eps) {
    return fmax(pb + (v1 - v2) + eps, nextafter(pb, DBL_MAX));
}

// a is evicted before b: lower bid, or equal bid and higher token id
BASE_DEV bool evict_first(double ba, int ta, double bb, int tb) {
    return ba < bb || (ba == bb && ta > tb);
}

// ---------------------------------------------------------------- phase control

__global__ void auc_init_kernel(AucWs w, int64_t E, const ScoreScan* scan, int64_t n,
                                AucStatsDev* st, int32_t* assign, int64_t T) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < E) w.floor_[i] = 0.0;
    if (i < T) assign[i] = 0;
    if (i == 0) {
        st->status = (scan->min_key == 0xffffffffu && n > 0) ? kErrNonfinite : 0;
        st->phases = 0;
        for (int q = 0; q < 16; ++q) { st->bids[q] = 0; st->rounds[q] = 0; }
        w.ctl->bids_total = 0;
        w.ctl->abort = st->status != 0;
    }
}

__global__ void auc_phase_start_kernel(AucWs w, int64_t T, int64_t E, const AucStatsDev* st) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < E) {
        w.cnt[i] = 0;
        w.nlow[i] = 0;
        w.comp[i] = 1;
        w.pi[i] = w.floor_[i];
    }
    if (i == 0) {
        AucCtl* c = w.ctl;
        c->cur = 0;
        c->bulk_done = 0;
        c->identity = 1;
        c->done_blocks = 0;
        c->nbid[0] = (int32_t)T;
        c->nbid[1] = 0;
        c->abort = st->status != 0;
        c->bids_phase = 0;
        c->rounds_phase = 0;
    }
}

// ---------------------------------------------------------------- bulk rounds

template <int NCH>
__global__ __launch_bounds__(256) void auc_bulk_bid_kernel(const float* s, int64_t T, int64_t E,
                                                           AucWs w, const ScoreScan* scan,
                                                           int round, double eps) {
    AucCtl* ctl = w.ctl;
    if (ctl->abort || ctl->bulk_done) return;
    const int cur = ctl->cur;
    const int64_t nb = ctl->nbid[cur];
    if (round > 0 && nb <= kTailMax) {
        if (blockIdx.x == 0 && threadIdx.x == 0) ctl->bulk_done = 1;
        return;
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        ctl->nbid[cur ^ 1] = 0;
        ctl->bids_phase += (unsigned long long)nb;  // every listed token bids once
    }
    const bool ident = ctl->identity;
    const int32_t* list = cur ? w.list1 : w.list0;
    const Sani sn = read_sani(scan);
    const int lane = threadIdx.x & 63;
    const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int64_t nw = ((int64_t)gridDim.x * blockDim.x) >> 6;
    // the round's prices do not change during the kernel: keep this lane's
    double pv[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int64_t e = lane + 64 * c;
        pv[c] = (e < E) ? w.pi[e] : 0.0;
    }
    int64_t mine = 0;
    // each wave's tokens, the next token's row loaded while the current bids
    int64_t j = wave;
    float v[NCH], vn[NCH];
    int64_t t = (j < nb) ? (ident ? j : list[j]) : -1;
    if (t >= 0) load_row<NCH>(s, t, E, lane, sn, v);
    while (t >= 0) {
        const int64_t jn = j + nw;
        const int64_t tn = (jn < nb) ? (ident ? jn : list[jn]) : -1;
        if (tn >= 0) load_row<NCH>(s, tn, E, lane, sn, vn);
        int b1;
        double v1, v2, pb;
        best_two_pv<NCH>(v, pv, E, lane, b1, v1, v2, pb);
        if (lane == 0) {
            w.bexp[t] = b1;
            w.bval[t] = bid_amount(pb, v1, v2, eps);
        }
        ++mine;
        j = jn;
        t = tn;
#pragma unroll
        for (int c = 0; c < NCH; ++c) v[c] = vn[c];
    }
    (void)mine;
}

// One block per expert: keep the k best of (current holders + this round's
// bidders for this expert), return the others to the next bidder list, and
// publish the expert's price and its L lowest holders. The holders are kept
// sorted best first (bid descending, then token ascending) in the expert's
// slots across the bulk rounds of a phase, so a round sorts only its new
// bidders and merges by rank: a holder's new position is its old one plus
// the number of bidders better than it, a bidder's is its position among the
// bidders plus the number of holders better than it (binary searches).
// Bidders are gathered kResolveCap at a time; a full buffer is merged before
// the scan goes on.
BASE_DEV bool better(double ba, int ta, double bb, int tb) { return ba > bb || (ba == bb && ta < tb); }

// Sort (bid, token) pairs across the wave, best first (bitonic network over
// the 64 lanes by shuffles).
BASE_DEV void wave_sort_best(double& b, int& t, int lane) {
#pragma unroll
    for (int k2 = 2; k2 <= 64; k2 <<= 1) {
#pragma unroll
        for (int j = k2 >> 1; j > 0; j >>= 1) {
            const double ob = shfl_xor_f64(b, j);
            const int ot = __shfl_xor(t, j, 64);
            const bool take_first = ((lane & j) == 0) == ((lane & k2) == 0);
            const bool swap = take_first ? better(ob, ot, b, t) : better(b, t, ob, ot);
            if (swap) { b = ob; t = ot; }
        }
    }
}

// Sort cb/ct[0, n) best first (n <= 2048, arrays of the next power of two
// at least 64): each wave sorts runs of 64 in registers, then runs are merged
// pairwise by rank (an element's place = its index in its run + the partner
// run's elements ahead of it; ties between runs go to the left run),
// ping-ponging with ob/ot. Called by every thread of the block.
BASE_DEV void block_sort_best(double* cb, int32_t* ct, double* ob, int32_t* ot, int n) {
    const int tid = threadIdx.x, lane = tid & 63;
    int P = 64;
    while (P < n) P <<= 1;
    for (int i = n + tid; i < P; i += blockDim.x) { cb[i] = -DBL_MAX; ct[i] = kNoTok; }
    __syncthreads();
    const int wv = tid >> 6, nwv = blockDim.x >> 6;
    for (int r = wv; r < P / 64; r += nwv) {
        double b = cb[r * 64 + lane];
        int t = ct[r * 64 + lane];
        wave_sort_best(b, t, lane);
        cb[r * 64 + lane] = b;
        ct[r * 64 + lane] = t;
    }
    __syncthreads();
    double* sb = cb;
    int32_t* st = ct;
    double* db = ob;
    int32_t* dt = ot;
    for (int len = 64; len < P; len <<= 1) {
        for (int i = tid; i < P; i += blockDim.x) {
            const int run = i / len, pos = i - run * len;
            const int other = (run ^ 1) * len;
            const double b = sb[i];
            const int t = st[i];
            int lo = 0, hi = len;  // partner elements ahead of this one
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                const double pb = sb[other + mid];
                const int pt = st[other + mid];
                const bool ahead = (run & 1) ? !better(b, t, pb, pt) : better(pb, pt, b, t);
                if (ahead) lo = mid + 1;
                else hi = mid;
            }
            const int at = (run & ~1) * len + pos + lo;
            db[at] = b;
            dt[at] = t;
        }
        __syncthreads();
        double* xb = sb; sb = db; db = xb;
        int32_t* xt = st; st = dt; dt = xt;
    }
    if (sb != cb) {
        for (int i = tid; i < P; i += blockDim.x) { cb[i] = sb[i]; ct[i] = st[i]; }
        __syncthreads();
    }
}

// An expert's lowest holders in eviction order (slots m-1, m-2, ... of its
// best-first slots), its count, list state and price.
BASE_DEV void publish_expert(AucWs& w, int e, int64_t k, int m, const double* hb,
                             const int32_t* ht) {
    const int L = w.L;
    const int nl = min(m, L);
    for (int i = threadIdx.x; i < nl; i += blockDim.x) {
        w.lowb[(int64_t)e * L + i] = hb[m - 1 - i];
        w.lowt[(int64_t)e * L + i] = ht[m - 1 - i];
        w.lows[(int64_t)e * L + i] = m - 1 - i;
    }
    if (threadIdx.x == 0) {
        w.cnt[e] = m;
        w.nlow[e] = nl;
        w.comp[e] = (m <= L) ? 1 : 0;
        w.pi[e] = (m == k) ? hb[k - 1] : w.floor_[e];
    }
}

__global__ __launch_bounds__(256) void auc_bulk_resolve_kernel(int64_t T, int64_t E, int64_t k,
                                                               AucWs w) {
    __shared__ double cb[kResolveCap];   // bidders
    __shared__ int32_t ct[kResolveCap];
    __shared__ double hb[kBulkKMax];     // holders, best first
    __shared__ int32_t ht[kBulkKMax];
    __shared__ double ob[kBulkKMax];     // merged
    __shared__ int32_t ot[kBulkKMax];
    __shared__ int32_t ncand, nhold;
    AucCtl* ctl = w.ctl;
    if (ctl->abort || ctl->bulk_done) return;
    const int cur = ctl->cur;
    const int64_t nb = ctl->nbid[cur];
    const bool ident = ctl->identity;
    const int32_t* list = cur ? w.list1 : w.list0;
    int32_t* outl = cur ? w.list0 : w.list1;
    const int e = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63;
    const int L = w.L;
    int32_t* stok = w.stok + (int64_t)e * k;
    double* sbid = w.sbid + (int64_t)e * k;

    // append the token of each thread with rej set to the next bidder list
    auto reject = [&](bool rej, int tok) {
        const unsigned long long m = __ballot(rej);
        int base = 0;
        if (lane == 0 && m) base = atomicAdd(&ctl->nbid[cur ^ 1], (int)__popcll(m));
        base = __shfl(base, 0, 64);
        if (rej) {
            const unsigned long long below = lane ? (~0ull >> (64 - lane)) : 0ull;
            outl[base + __popcll(m & below)] = tok;
        }
    };
    // merge the n gathered bidders into the holders
    auto merge = [&](int n) {
        block_sort_best(cb, ct, ob, ot, n);
        const int c = nhold;
        // holder i moves to i + (bidders better than it)
        for (int i0 = 0; i0 < c; i0 += blockDim.x) {
            const int i = i0 + tid;
            bool rej = false;
            int tok = 0;
            if (i < c) {
                int lo = 0, hi = n;  // first bidder not better than holder i
                while (lo < hi) {
                    const int mid = (lo + hi) >> 1;
                    if (better(cb[mid], ct[mid], hb[i], ht[i])) lo = mid + 1;
                    else hi = mid;
                }
                const int r = i + lo;
                if (r < k) { ob[r] = hb[i]; ot[r] = ht[i]; }
                else { rej = true; tok = ht[i]; }
            }
            reject(rej, tok);
        }
        // bidder j moves to j + (holders better than it)
        for (int j0 = 0; j0 < n; j0 += blockDim.x) {
            const int j = j0 + tid;
            bool rej = false;
            int tok = 0;
            if (j < n) {
                int lo = 0, hi = c;
                while (lo < hi) {
                    const int mid = (lo + hi) >> 1;
                    if (better(hb[mid], ht[mid], cb[j], ct[j])) lo = mid + 1;
                    else hi = mid;
                }
                const int r = j + lo;
                if (r < k) { ob[r] = cb[j]; ot[r] = ct[j]; }
                else { rej = true; tok = ct[j]; }
            }
            reject(rej, tok);
        }
        __syncthreads();
        const int c2 = (int)min<int64_t>(c + n, k);
        for (int i = tid; i < c2; i += blockDim.x) { hb[i] = ob[i]; ht[i] = ot[i]; }
        if (tid == 0) { nhold = c2; ncand = 0; }
        __syncthreads();
    };

    const int c0 = w.cnt[e];
    for (int i = tid; i < c0; i += blockDim.x) { hb[i] = sbid[i]; ht[i] = stok[i]; }
    // gather this expert's bidders in one pass with 16 loads in flight per
    // thread (the bids were written by other XCDs: every load is a far round
    // trip); tokens first, their bids in a second, parallel sweep. More
    // bidders than the buffer holds (rare) fall back to chunks merged in turn.
    if (tid == 0) { ncand = 0; nhold = c0; }
    __syncthreads();
    auto scan_bidders = [&](auto&& fn) {
        constexpr int U = 16;
        for (int64_t j0 = 0; j0 < nb; j0 += U * (int64_t)blockDim.x) {
            int64_t tt[U];
            int ee[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t j = j0 + (int64_t)u * blockDim.x + tid;
                tt[u] = (j < nb) ? (ident ? j : (int64_t)list[j]) : -1;
            }
#pragma unroll
            for (int u = 0; u < U; ++u) ee[u] = (tt[u] >= 0) ? w.bexp[tt[u]] : -1;
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (ee[u] == e) fn(tt[u]);
        }
    };
    scan_bidders([&](int64_t t) {
        const int pos = atomicAdd(&ncand, 1);
        if (pos < kResolveCap) ct[pos] = (int32_t)t;
    });
    __syncthreads();
    const int nbe = ncand;
    const bool changed = nbe > 0;
    if (nbe > 0 && nbe <= kResolveCap) {
        for (int i = tid; i < nbe; i += blockDim.x) cb[i] = w.bval[ct[i]];
        __syncthreads();
        merge(nbe);
    } else if (nbe > 0) {
        __syncthreads();
        if (tid == 0) ncand = 0;
        __syncthreads();
        for (int64_t j0 = 0; j0 < nb; j0 += blockDim.x) {
            const int64_t j = j0 + tid;
            if (j < nb) {
                const int64_t t = ident ? j : list[j];
                if (w.bexp[t] == e) {
                    const int pos = atomicAdd(&ncand, 1);
                    cb[pos] = w.bval[t];
                    ct[pos] = (int32_t)t;
                }
            }
            __syncthreads();
            const int n = ncand;
            if (n > kResolveCap - (int)blockDim.x) merge(n);
        }
        if (ncand > 0) merge(ncand);
    }
    if (changed) {
        const int m = nhold;
        for (int i = tid; i < m; i += blockDim.x) { sbid[i] = hb[i]; stok[i] = ht[i]; }
        publish_expert(w, e, k, m, hb, ht);
    }
    __syncthreads();
    if (tid == 0) {
        __threadfence();
        const int done = atomicAdd(&ctl->done_blocks, 1);
        if (done == (int)gridDim.x - 1) {
            ctl->done_blocks = 0;
            ctl->identity = 0;
            ctl->cur = cur ^ 1;
            ctl->rounds_phase += 1;
            __threadfence();
        }
    }
}

#include "auction_tail.h"

// ---------------------------------------------------------------- finalize

__global__ void auc_finalize_kernel(AucWs w, int64_t E, int64_t k, int32_t* assign, double* prices) {
    const int e = blockIdx.x;
    const int64_t n = min<int64_t>(w.cnt[e], k);
    for (int64_t i = threadIdx.x; i < n; i += blockDim.x) {
        const int32_t t = w.stok[(int64_t)e * k + i];
        assign[t] = e;
    }
    if (threadIdx.x == 0) prices[e] = w.floor_[e];
}

// ---------------------------------------------------------------- launcher

template <int NCH>
static void launch_tail(const float* s, int64_t T, int64_t E, int64_t k, const AucWs& w,
                        const ScoreScan* scan, double eps, int phase, int64_t max_bids,
                        AucStatsDev* st, size_t lds, hipStream_t stream) {
    hipLaunchKernelGGL(auc_tail_kernel<NCH>, dim3(1), dim3(tail_threads(NCH)), lds, stream, s, T, E,
                       k, w, scan, eps, phase, max_bids, st);
}

template <int NCH>
static hipError_t run_auction(const float* s, int64_t T, int64_t E, double eps_start,
                              double eps_end, double eps_factor, int64_t max_bids,
                              const ScoreScan* scan, int32_t* assign, double* prices,
                              AucStatsDev* st, AucWs w, hipStream_t stream) {
    const int64_t k = T / E;
    const unsigned g1 = (unsigned)(((T > E ? T : E) + 255) / 256);
    hipLaunchKernelGGL(auc_init_kernel, dim3(g1), dim3(256), 0, stream, w, E, scan, T * E, st, assign, T);
    const int rounds = (k > kBulkKMax) ? 0 : (k <= kSmallK ? kBulkRoundsSmallK : kBulkRounds);
    int64_t bid_blocks = (T + 15) / 16;
    if (bid_blocks > 2048) bid_blocks = 2048;
    const size_t tail_lds = tail_lds_bytes(E, w.L, tail_threads(NCH));
    double eps = eps_start;
    for (int phase = 0;; ++phase) {
        hipLaunchKernelGGL(auc_phase_start_kernel, dim3((unsigned)((E + 255) / 256)), dim3(256), 0,
                           stream, w, T, E, st);
        for (int r = 0; r < rounds; ++r) {
            // round 0: every token bids; later rounds: the returned few
            const unsigned nblk = (unsigned)(r == 0 ? bid_blocks : (bid_blocks < 256 ? bid_blocks : 256));
            hipLaunchKernelGGL(auc_bulk_bid_kernel<NCH>, dim3(nblk), dim3(256), 0,
                               stream, s, T, E, w, scan, r, eps);
            hipLaunchKernelGGL(auc_bulk_resolve_kernel, dim3((unsigned)E), dim3(256), 0, stream, T,
                               E, k, w);
        }
        launch_tail<NCH>(s, T, E, k, w, scan, eps, phase, max_bids, st, tail_lds, stream);
        if (eps <= eps_end) break;
        eps = eps / eps_factor;
        if (eps < eps_end) eps = eps_end;
    }
    hipLaunchKernelGGL(auc_finalize_kernel, dim3((unsigned)E), dim3(256), 0, stream, w, E, k, assign,
                       prices);
    return hipGetLastError();
}

hipError_t launch_auction(const float* s, int64_t T, int64_t E, double eps_start, double eps_end,
                          double eps_factor, int64_t max_bids, const ScoreScan* scan,
                          int32_t* assign, int32_t* perm, int32_t* offsets, double* prices,
                          AucStatsDev* stats, void* ws, hipStream_t stream) {
    AucWs w = carve(ws, T, E);
    hipError_t err;
    const int64_t nch = (E + 63) / 64;
    if (nch <= 1) err = run_auction<1>(s, T, E, eps_start, eps_end, eps_factor, max_bids, scan, assign, prices, stats, w, stream);
    else if (nch <= 2) err = run_auction<2>(s, T, E, eps_start, eps_end, eps_factor, max_bids, scan, assign, prices, stats, w, stream);
    else if (nch <= 4) err = run_auction<4>(s, T, E, eps_start, eps_end, eps_factor, max_bids, scan, assign, prices, stats, w, stream);
    else if (nch <= 8) err = run_auction<8>(s, T, E, eps_start, eps_end, eps_factor, max_bids, scan, assign, prices, stats, w, stream);
    else err = run_auction<16>(s, T, E, eps_start, eps_end, eps_factor, max_bids, scan, assign, prices, stats, w, stream);
    if (err != hipSuccess) return err;
    // expert grouping (ascending token id within each expert); the perm
    // workspace follows the auction's
    return launch_perm(assign, T, E, perm, offsets, nullptr, 0, nullptr,
                       (char*)ws + auction_ws_bytes(T, E), stream);
}

}  // namespace base
