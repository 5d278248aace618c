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
//   tail (one persistent workgroup): once few tokens are left, the rest of
//     the phase is finished by shortest augmenting paths on the graph whose
//     nodes are the experts (auction_tail.h): a token's displacement chain
//     becomes one path search, and the prices rise in one step by the
//     amounts the chain would have added bid by bid.
// Prices and bids are fp64: exactness needs eps below gap/T, far below fp32
// resolution at prices of order one.
#include <float.h>

#include "common.h"
#include "internal.h"

namespace base {

// Multi-CU rounds per phase (at most), and the bidders left when the phase
// end takes over. A round costs 10-20 us whatever its size; the phase end
// about 6 us per token it places. Small capacities keep more bidders in
// conflict for longer. Measured (medians of 8 solves, 3 interleaved runs):
// at k = 128 (16k tokens, 128 experts) 48 rounds and a hand-over at 16
// bidders took the solve from 5.65 to 5.07 ms; at k = 512 (64k tokens) 20
// rounds and a hand-over at 24 from 5.42 to 3.83 ms; at k = 256 from 6.83
// to 6.01 ms (skewed scores) and 2.06 to 2.06 ms (64 experts).
constexpr int kBulkRounds = 20;
constexpr int kBulkRoundsSmallK = 48;
constexpr int64_t kSmallK = 128;
constexpr int kTailMax = 24;
constexpr int kTailMaxSmallK = 16;
constexpr int kResolveCap = 2048;    // bidders sorted at once per expert
constexpr int64_t kBinMax = 2048;    // rounds with at most this many bidders file bids by expert
constexpr int kOvfCap = 6144;        // an expert's bidders beyond kResolveCap kept in its bin
static_assert(kBinMax <= kResolveCap, "a round's bin for one expert must fit the resolve buffer");
static_assert(kBinMax <= kOvfCap, "the bins hold either a round's bids or the overflow");
constexpr int kBulkKMax = 2048;      // bulk rounds need k <= this
constexpr int64_t kLateGWs = 8;      // late rounds (auction_late.h): workgroups,
constexpr int64_t kLateCapWs = 256;  // and bids per (workgroup, expert) bin
constexpr int32_t kErrNotConverged = -5;
constexpr int32_t kErrNonfinite = -6;
constexpr int32_t kErrInvariant = -9;

// Checking build (BASE_CHECKS): the auction's kernels verify its invariants
// on the device and report a failure through the status word (never by a
// trap): every expert holds at most k tokens, sorted best first during the
// bulk rounds, and after the solve exactly k distinct ones.
#ifdef BASE_CHECKS
constexpr bool kChecks = true;
#else
constexpr bool kChecks = false;
#endif
BASE_DEV void report_invariant(AucStatsDev* st) {
    __hip_atomic_store(&st->status, kErrInvariant, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
constexpr int32_t kNoTok = 0x7fffffff;

struct AucCtl {
    int32_t cur;          // bidder list in use (0/1)
    int32_t bulk_done;    // the tail owns the rest of this phase
    int32_t identity;     // the bidder list is 0..T-1 (round 0)
    int32_t nbid[2];
    int32_t abort;        // a device error is set: skip all work
    int32_t pairs_done;   // the late-round launch owns the rest of the bulk rounds
    unsigned long long bids_total;
    unsigned long long bids_phase;
    long long rounds_phase;
    unsigned lbar;        // late rounds: barrier arrivals this phase
    int32_t lnb[2];       // late rounds: next bidders summed over workgroups
    int32_t lcw[2][16];   // late rounds: each workgroup's next bidders
};

struct AucWs {
    AucCtl* ctl;
    double* floor_;    // E   price floors p_e
    double* pi;        // E   prices for the next bulk round
    int32_t* cnt;      // E   holders per expert
    int32_t* list0;    // T
    int32_t* list1;    // T
    int32_t* bexp;     // T   bid of token t: expert
    double* bval;      // T   bid of token t: amount
    int32_t* stok;     // E*k slot tokens (slots 0 .. cnt-1 of each expert are held)
    double* sbid;      // E*k slot bids
    int32_t* slot_of;  // T   slot of each held token (tail)
    float* sown;       // E*k tail: each slot's holder's score at the slot's expert (E > 128)
    float* xt;         // E*E*k tail, E <= 128: xt[(a E + b) k + i] = score at b of a's holder i
    double* C;         // E*E tail: cheapest move of a holder of a to b
    int32_t* Ct;       // E*E tail: the holder that makes it
    unsigned long long* stale;  // E*ceil(E/64) tail: C entries whose holder left
    int32_t* bcnt;     // E   bids filed for each expert this round
    int32_t* bin_t;    // E*kOvfCap  the bidders (few-bidder rounds), else the overflow
    double* bin_v;     // E*kBinMax  their bids (few-bidder rounds)
    int32_t* llist;    // kLateG*2*T late rounds: each workgroup's bidder lists
    int32_t* lbin_t;   // kLateG*E*kLateCap  late rounds: bids by (workgroup, expert)
    double* lbin_v;    // kLateG*E*kLateCap
    int32_t* lbc;      // kLateG*E  their counts
};

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
static bool late_ok(int64_t T, int64_t E, int64_t k);  // auction_late.h
// the phase end's expert-major copy of its holders' scores (E <= 128, exactly when
// its C matrix lives in LDS: ssp_c_in_lds in auction_tail.h)
// Workgroups per expert in the phase-end setup: two when E <= 128 (128
// experts would leave half of the 256 CUs idle), each over half of the
// expert's holders, its C and Ct minima in a plane of its own that the
// phase end merges when it copies C into LDS.
__host__ __device__ static inline int64_t ssp_parts(int64_t E) { return E <= 128 ? 2 : 1; }
static int64_t xt_floats(int64_t T, int64_t E) { return E <= 128 ? E * T : 0; }

// the late-round launch's buffers, reserved only when a solve of this size
// uses it
static int64_t late_ws_g(int64_t T, int64_t E) { return (E > 0 && late_ok(T, E, T / E)) ? kLateGWs : 0; }

static AucWs carve(void* ws, int64_t T, int64_t E) {
    char* p = (char*)ws;
    AucWs w;
    w.ctl = (AucCtl*)p; p += align256(sizeof(AucCtl));
    w.floor_ = (double*)p; p += align256(E * 8);
    w.pi = (double*)p; p += align256(E * 8);
    w.cnt = (int32_t*)p; p += align256(E * 4);
    w.list0 = (int32_t*)p; p += align256(T * 4);
    w.list1 = (int32_t*)p; p += align256(T * 4);
    w.bexp = (int32_t*)p; p += align256(T * 4);
    w.bval = (double*)p; p += align256(T * 8);
    w.stok = (int32_t*)p; p += align256(T * 4);
    w.sbid = (double*)p; p += align256(T * 8);
    w.slot_of = (int32_t*)p; p += align256(T * 4);
    w.sown = (float*)p; p += align256(T * 4);
    w.xt = (float*)p; p += align256(xt_floats(T, E) * 4);
    w.C = (double*)p; p += align256(ssp_parts(E) * E * E * 8);
    w.Ct = (int32_t*)p; p += align256(ssp_parts(E) * E * E * 4);
    w.stale = (unsigned long long*)p; p += align256(E * ((E + 63) / 64) * 8);
    w.bcnt = (int32_t*)p; p += align256(E * 4);
    w.bin_t = (int32_t*)p; p += align256(E * kOvfCap * 4);
    w.bin_v = (double*)p; p += align256(E * kBinMax * 8);
    const int64_t lg = late_ws_g(T, E);
    w.llist = (int32_t*)p; p += align256(lg * 2 * T * 4);
    w.lbin_t = (int32_t*)p; p += align256(lg * E * kLateCapWs * 4);
    w.lbin_v = (double*)p; p += align256(lg * E * kLateCapWs * 8);
    w.lbc = (int32_t*)p; p += align256(lg * E * 4);
    return w;
}

size_t auction_ws_bytes(int64_t T, int64_t E) {
    return align256(sizeof(AucCtl)) + 2 * align256(E * 8) + align256(E * 4) +
           6 * align256(T * 4) + 2 * align256(T * 8) + align256(ssp_parts(E) * E * E * 8) +
           align256(xt_floats(T, E) * 4) +
           align256(ssp_parts(E) * E * E * 4) + align256(E * ((E + 63) / 64) * 8) + align256(E * 4) +
           align256(E * kOvfCap * 4) + align256(E * kBinMax * 8) +
           align256(late_ws_g(T, E) * 2 * T * 4) + align256(late_ws_g(T, E) * E * kLateCapWs * 4) +
           align256(late_ws_g(T, E) * E * kLateCapWs * 8) + align256(late_ws_g(T, E) * E * 4) + 256;
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
        for (int q = 0; q < 16; ++q) { st->bids[q] = 0; st->rounds[q] = 0; st->tail[q] = 0; }
        w.ctl->bids_total = 0;
        w.ctl->abort = st->status != 0;
    }
}

__global__ void auc_phase_start_kernel(AucWs w, int64_t T, int64_t E, const AucStatsDev* st) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < E) {
        w.cnt[i] = 0;
        w.bcnt[i] = 0;
        w.pi[i] = w.floor_[i];
    }
    if (i == 0) {
        AucCtl* c = w.ctl;
        c->cur = 0;
        c->bulk_done = 0;
        c->pairs_done = 0;
        c->identity = 1;
        c->nbid[0] = (int32_t)T;
        c->nbid[1] = 0;
        c->abort = st->status != 0;
        c->bids_phase = 0;
        c->rounds_phase = 0;
        c->lbar = 0;
        c->lnb[0] = 0;
        c->lnb[1] = 0;
    }
}

// ---------------------------------------------------------------- bulk rounds

template <int NCH>
__global__ __launch_bounds__(256) void auc_bulk_bid_kernel(const float* s, int64_t T, int64_t E,
                                                           AucWs w, const ScoreScan* scan,
                                                           int round, double eps, int tail_max,
                                                           int late_enter) {
    AucCtl* ctl = w.ctl;
    const int lane = threadIdx.x & 63;
    const int cur = round & 1;  // round r bids from list r % 2
    const bool ident = round == 0;
    const int32_t* list = cur ? w.list1 : w.list0;
    const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int64_t nw = ((int64_t)gridDim.x * blockDim.x) >> 6;
    // One round trip for all the first bid needs but its score row: this
    // lane's prices (fixed for the round), the control word, the score scan
    // and the wave's first list entry. The entry is read before the count is
    // known (the list holds T entries; one past the count is ignored).
    double pv[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int64_t e = lane + 64 * c;
        pv[c] = (e < E) ? w.pi[e] : 0.0;
    }
    const int32_t first = (!ident && wave < T) ? list[wave] : 0;
    const Sani sn = read_sani(scan);
    const int aborted = ctl->abort, done = ctl->bulk_done | ctl->pairs_done;
    const int64_t nb = ctl->nbid[cur];
    if (aborted || done) return;
    if (round > 0 && nb <= tail_max) {
        if (blockIdx.x == 0 && threadIdx.x == 0) ctl->bulk_done = 1;
        return;
    }
    if (round > 0 && nb <= late_enter) {  // few bidders left: the late launch takes over
        if (blockIdx.x == 0 && threadIdx.x == 0) ctl->pairs_done = 1;
        return;
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        ctl->nbid[cur ^ 1] = 0;
        ctl->bids_phase += (unsigned long long)nb;  // every listed token bids once
    }
    const bool binned = nb <= kBinMax;
    int64_t mine = 0;
    // each wave's tokens, the next token's row loaded while the current bids
    int64_t j = wave;
    float v[NCH], vn[NCH];
    int64_t t = (j < nb) ? (ident ? j : (int64_t)first) : -1;
    if (t >= 0) load_row<NCH>(s, t, E, lane, sn, v);
    while (t >= 0) {
        const int64_t jn = j + nw;
        const int64_t tn = (jn < nb) ? (ident ? jn : list[jn]) : -1;
        if (tn >= 0) load_row<NCH>(s, tn, E, lane, sn, vn);
        int b1;
        double v1, v2, pb;
        best_two_pv<NCH>(v, pv, E, lane, b1, v1, v2, pb);
        if (lane == 0) {
            // the bid, and in a round with few bidders a copy filed under its
            // expert (the resolve kernel then reads only its own)
            const double bid = bid_amount(pb, v1, v2, eps);
            w.bexp[t] = b1;
            w.bval[t] = bid;
            if (binned) {
                const int pos = atomicAdd(&w.bcnt[b1], 1);
                w.bin_t[(int64_t)b1 * kOvfCap + pos] = (int32_t)t;
                w.bin_v[(int64_t)b1 * kBinMax + pos] = bid;
            }
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
// publish the expert's price. In a round with at most kBinMax bidders the bid
// kernel files each bid under its expert, so an expert reads only its own
// bidders; in larger rounds (where those atomics would contend) every expert
// scans the round's list. The list a round reads and writes follows from the
// round's parity, so no block waits for the others. The holders are kept
// sorted best first (bid descending, then token ascending) in the expert's
// slots across the bulk rounds of a phase, so a round sorts only its new
// bidders and merges by rank: a holder's new position is its old one plus
// the number of bidders better than it, a bidder's is its position among the
// bidders plus the number of holders better than it (binary searches).
BASE_DEV bool better(double ba, int ta, double bb, int tb) { return ba > bb || (ba == bb && ta < tb); }

// Rank of this lane's (bid, token) pair among those of lanes 0 .. n-1, best
// first: the number of those lanes holding a better pair. The other lanes'
// pairs arrive by readlane (a scalar broadcast, a few cycles each), so the
// count is one short dependent chain; the pairs must be distinct.
BASE_DEV int wave_rank_best(double b, int t, int n = 64) {
    int r = 0;
#pragma unroll 8
    for (int m = 0; m < n; ++m) {
        const double bm = readlane_f64(b, m);
        const int tm = __builtin_amdgcn_readlane(t, m);
        r += better(bm, tm, b, t) ? 1 : 0;
    }
    return r;
}

// Sort cb/ct[0, n) best first (n <= 2048, arrays of the next power of two
// at least 64): each wave ranks runs of 64 in registers and places them,
// padded with distinct worst entries, then runs are merged
// pairwise by rank (an element's place = its index in its run + the partner
// run's elements ahead of it; ties between runs go to the left run),
// ping-ponging with ob/ot. Called by every thread of the block.
BASE_DEV void block_sort_best(double* cb, int32_t* ct, double* ob, int32_t* ot, int n) {
    const int tid = threadIdx.x, lane = tid & 63;
    int P = 64;
    while (P < n) P <<= 1;
    const int wv = tid >> 6, nwv = blockDim.x >> 6;
    for (int r = wv; r < P / 64; r += nwv) {
        const int i = r * 64 + lane;
        const double b = i < n ? cb[i] : -DBL_MAX;
        const int t = i < n ? ct[i] : kNoTok - i;
        const int q = wave_rank_best(b, t);
        cb[r * 64 + q] = b;
        ct[r * 64 + q] = t;
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

// An expert's count and price after a round: the lowest bid it holds once
// full, else its floor.
BASE_DEV void publish_expert(AucWs& w, int e, int64_t k, int m, const double* hb) {
    if (threadIdx.x == 0) {
        w.cnt[e] = m;
        w.pi[e] = (m == k) ? hb[k - 1] : w.floor_[e];
    }
}

constexpr int kResolveThreads = 256;
constexpr int kSpecHold = 2;  // holder slots prefetched per thread (k <= 512)

__global__ __launch_bounds__(kResolveThreads) void auc_bulk_resolve_kernel(int64_t T, int64_t E,
                                                                           int64_t k, AucWs w,
                                                                           int round,
                                                                           AucStatsDev* st) {
    __shared__ double cb[kResolveCap];   // bidders
    __shared__ int32_t ct[kResolveCap];
    __shared__ double hb[kBulkKMax];     // holders, best first
    __shared__ int32_t ht[kBulkKMax];
    __shared__ double ob[kBulkKMax];     // merged
    __shared__ int32_t ot[kBulkKMax];
    __shared__ int32_t rej[kResolveCap];  // a merge's rejected tokens, by rank - k
    __shared__ int32_t frj[kResolveCap];  // bidders rejected before any merge (below)
    __shared__ int32_t ncand, nhold, rbase, nfrj, nsurv, ncut;
    __shared__ double cut_s;
    static_assert(kResolveThreads <= kBinMax && kResolveThreads <= kOvfCap,
                  "one prefetched bin entry per thread");
    AucCtl* ctl = w.ctl;
    const int e = blockIdx.x;
    const int tid = threadIdx.x;
    const int cur = round & 1;
    int32_t* stok = w.stok + (int64_t)e * k;
    double* sbid = w.sbid + (int64_t)e * k;
    // One round trip for the expert's counts, the control word, its holder
    // slots and the first entries of its bin. Slots and bin entries are read
    // before their counts are known (those past the counts are ignored): a
    // dependent round trip costs more than the bytes.
    const bool spec_hold = k <= (int64_t)kSpecHold * kResolveThreads;
    double phb[kSpecHold];
    int32_t pht[kSpecHold];
#pragma unroll
    for (int u = 0; u < kSpecHold; ++u) {
        const int i = tid + u * kResolveThreads;
        phb[u] = 0.0;
        pht[u] = 0;
        if (spec_hold && i < k) { phb[u] = sbid[i]; pht[u] = stok[i]; }
    }
    const int32_t pbt = w.bin_t[(int64_t)e * kOvfCap + tid];
    const double pbv = w.bin_v[(int64_t)e * kBinMax + tid];
    const int c0 = w.cnt[e];
    const int nbin = w.bcnt[e];
    const int aborted = ctl->abort, done = ctl->bulk_done | ctl->pairs_done;
    const int64_t nb = ctl->nbid[cur];
    if (aborted || done) return;
    const bool ident = round == 0;
    const int32_t* list = cur ? w.list1 : w.list0;
    int32_t* outl = cur ? w.list0 : w.list1;

    // the holders into LDS (from the prefetch when it covered them)
    auto load_holders = [&]() {
        if (spec_hold) {
#pragma unroll
            for (int u = 0; u < kSpecHold; ++u) {
                const int i = tid + u * kResolveThreads;
                if (i < c0) { hb[i] = phb[u]; ht[i] = pht[u]; }
            }
        } else {
            for (int i = tid; i < c0; i += kResolveThreads) { hb[i] = sbid[i]; ht[i] = stok[i]; }
        }
    };
    // merge the n gathered bidders into the holders. The bidders are sorted,
    // then every element's new rank is its rank in its own run plus the
    // elements of the other run ahead of it (binary search); those ranked
    // >= k are rejected, staged at rank - k, and leave for the next bidder
    // list at a base reserved by one atomic per merge. The atomic's result
    // stays in a register until the ranks are known, so its round trip
    // overlaps the sort.
    auto merge = [&](int n) {
        const int c = nhold;
        const int nrej = c + n - (int)min<int64_t>(c + n, k);  // <= n, as c <= k
        int my_base = 0;
        if (tid == 0 && nrej > 0) my_base = atomicAdd(&ctl->nbid[cur ^ 1], nrej);
        block_sort_best(cb, ct, ob, ot, n);
        for (int i = tid; i < c; i += kResolveThreads) {
            const double b = hb[i];
            const int t = ht[i];
            int lo = 0, hi = n;  // bidders better than holder i
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (better(cb[mid], ct[mid], b, t)) lo = mid + 1;
                else hi = mid;
            }
            const int r = i + lo;
            if (r < k) { ob[r] = b; ot[r] = t; }
            else rej[r - k] = t;
        }
        for (int j = tid; j < n; j += kResolveThreads) {
            const double b = cb[j];
            const int t = ct[j];
            int lo = 0, hi = c;  // holders better than bidder j
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (better(hb[mid], ht[mid], b, t)) lo = mid + 1;
                else hi = mid;
            }
            const int r = j + lo;
            if (r < k) { ob[r] = b; ot[r] = t; }
            else rej[r - k] = t;
        }
        if (tid == 0) rbase = my_base;
        __syncthreads();
        const int base = rbase;
        for (int q = tid; q < nrej; q += kResolveThreads) outl[base + q] = rej[q];
        const int c2 = (int)min<int64_t>(c + n, k);
        for (int i = tid; i < c2; i += kResolveThreads) { hb[i] = ob[i]; ht[i] = ot[i]; }
        if (tid == 0) { nhold = c2; ncand = 0; }
        __syncthreads();
    };

    // Once e is full, a bidder not better than its worst holder would be
    // ranked >= k by any merge: in rounds with many bidders for e it goes
    // straight back to the bidder list (staged in frj, one atomic per
    // flush) and only the others are sorted. Holders only get better, so
    // the result is the same as merging everyone.
    auto flush_frj = [&]() {  // every thread, with nfrj read after a barrier
        const int n = nfrj;
        if (n > 0) {
            if (tid == 0) rbase = atomicAdd(&ctl->nbid[cur ^ 1], n);
            __syncthreads();
            const int b = rbase;
            for (int q = tid; q < n; q += kResolveThreads) outl[b + q] = frj[q];
            __syncthreads();
            if (tid == 0) nfrj = 0;
            __syncthreads();
        }
    };
    if (tid == 0) { ncand = 0; nhold = c0; nfrj = 0; }
    int nbe;  // this round's bidders for e
    if (nb <= kBinMax) {
        // as the bid kernel filed them (at most kBinMax <= kResolveCap)
        nbe = nbin;
        if (nbe > 0) {
            load_holders();
            if (tid < nbe) { ct[tid] = pbt; cb[tid] = pbv; }
            for (int i = tid + kResolveThreads; i < nbe; i += kResolveThreads) {
                ct[i] = w.bin_t[(int64_t)e * kOvfCap + i];
                cb[i] = w.bin_v[(int64_t)e * kBinMax + i];
            }
            __syncthreads();
            if (tid == 0) w.bcnt[e] = 0;
            merge(nbe);
        }
    } else {
        // gather e's bidders from the round's list in one pass, 16 loads in
        // flight per thread (the bids were written by other XCDs: every load
        // is a far round trip); tokens first, their bids in a second sweep
        load_holders();
        __syncthreads();
        {
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
                    if (ee[u] == e) {
                        const int pos = atomicAdd(&ncand, 1);
                        if (pos < kResolveCap) ct[pos] = (int32_t)tt[u];
                        else if (pos < kResolveCap + kOvfCap)
                            w.bin_t[(int64_t)e * kOvfCap + pos - kResolveCap] = (int32_t)tt[u];
                    }
            }
        }
        __syncthreads();
        nbe = ncand;
        if (nbe > kResolveCap) {
            __threadfence();  // the overflow stores, before other threads load them
            __syncthreads();
        }
        if (nbe > 0 && nbe <= kResolveCap + kOvfCap) {
            // the first kResolveCap from LDS, the rest from the bin, merged
            // kResolveCap at a time
            constexpr int UC = kResolveCap / kResolveThreads;
            for (int c0 = 0; c0 < nbe; c0 += kResolveCap) {
                const int cn = min(kResolveCap, nbe - c0);
                const bool full = nhold == k;
                const double thb = full ? hb[k - 1] : 0.0;
                const int tht = full ? ht[k - 1] : 0;
                int32_t tk[UC];
                double bk[UC];
#pragma unroll
                for (int u = 0; u < UC; ++u) {
                    const int i = tid + u * kResolveThreads;
                    tk[u] = -1;
                    if (i < cn)
                        tk[u] = c0 == 0 ? ct[i]
                                        : __hip_atomic_load(w.bin_t + (int64_t)e * kOvfCap + (c0 - kResolveCap) + i,
                                                            __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
#pragma unroll
                for (int u = 0; u < UC; ++u) bk[u] = tk[u] >= 0 ? w.bval[tk[u]] : 0.0;
                if (tid == 0) { nsurv = 0; ncut = 0; }
                __syncthreads();  // every thread has read ct before the survivors overwrite it
                // A large chunk for an expert not yet full (a crowded expert
                // in a phase's first round): a cut from a sample of its bids.
                // When at least k of the chunk's bids are at or above it, a
                // bid below it is ranked >= k by any merge, so it leaves at
                // once and only the ~k others are sorted.
                double cut = -DBL_MAX;
                if (!full && cn >= 2 * k && cn > 512) {
                    // one sample per thread (cn > 512 >= kResolveThreads)
                    constexpr int nsm = kResolveThreads;
                    ob[tid] = bk[0];
                    __syncthreads();
                    const int want = min(nsm - 1, (int)((int64_t)nsm * k * 5 / (4 * (int64_t)cn)) + 4);
                    int r = 0;  // samples ahead of this one (index breaks ties)
                    for (int j = 0; j < nsm; ++j) {
                        const double o = ob[j];
                        r += (o > bk[0] || (o == bk[0] && j < tid)) ? 1 : 0;
                    }
                    if (r == want) cut_s = bk[0];
                    __syncthreads();
                    const double cv = cut_s;
                    int mc = 0;
#pragma unroll
                    for (int u = 0; u < UC; ++u) mc += (tk[u] >= 0 && bk[u] >= cv) ? 1 : 0;
                    if (mc > 0) atomicAdd(&ncut, mc);
                    __syncthreads();
                    if (ncut >= k) cut = cv;
                }
#pragma unroll
                for (int u = 0; u < UC; ++u) {
                    if (tk[u] < 0) continue;
                    if ((full && !better(bk[u], tk[u], thb, tht)) || bk[u] < cut) {
                        frj[atomicAdd(&nfrj, 1)] = tk[u];
                    } else {
                        const int q = atomicAdd(&nsurv, 1);
                        cb[q] = bk[u];
                        ct[q] = tk[u];
                    }
                }
                __syncthreads();
                const int ns = nsurv;
                flush_frj();
                if (ns > 0) merge(ns);
            }
        } else if (nbe > 0) {
            // more than the buffer and the bin hold (a crowded expert in a
            // phase's first round): gather again, 16 loads in flight per
            // thread, the candidates appended four loads' worth at a time so
            // the buffer may always take another group, merging (which
            // raises the threshold that filters the rest) whenever it may
            // not. Every thread reads the counts between two barriers, so
            // all take the same branch.
            __syncthreads();
            if (tid == 0) ncand = 0;
            __syncthreads();
            constexpr int U = 16, G = 4;
            for (int64_t j0 = 0; j0 < nb; j0 += U * (int64_t)blockDim.x) {
                int32_t tt[U];
                int ee[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int64_t j = j0 + (int64_t)u * blockDim.x + tid;
                    tt[u] = (j < nb) ? (ident ? (int32_t)j : list[j]) : -1;
                }
#pragma unroll
                for (int u = 0; u < U; ++u) ee[u] = (tt[u] >= 0) ? w.bexp[tt[u]] : -1;
                double bv[U];
#pragma unroll
                for (int u = 0; u < U; ++u) bv[u] = (ee[u] == e) ? w.bval[tt[u]] : 0.0;
#pragma unroll
                for (int g0 = 0; g0 < U; g0 += G) {
                    const bool full = nhold == k;
                    const double thb = full ? hb[k - 1] : 0.0;
                    const int tht = full ? ht[k - 1] : 0;
#pragma unroll
                    for (int u = g0; u < g0 + G; ++u)
                        if (ee[u] == e) {
                            if (full && !better(bv[u], tt[u], thb, tht)) {
                                frj[atomicAdd(&nfrj, 1)] = tt[u];
                            } else {
                                const int pos = atomicAdd(&ncand, 1);
                                cb[pos] = bv[u];
                                ct[pos] = tt[u];
                            }
                        }
                    __syncthreads();
                    const int n = ncand;
                    const int nf = nfrj;
                    __syncthreads();
                    if (nf > kResolveCap - G * (int)blockDim.x) flush_frj();
                    if (n > kResolveCap - G * (int)blockDim.x) merge(n);
                }
            }
            const int n = ncand;
            __syncthreads();
            flush_frj();
            if (n > 0) merge(n);
        }
    }
    const bool changed = nbe > 0;
    if (changed) {
        const int m = nhold;
        for (int i = tid; i < m; i += blockDim.x) { sbid[i] = hb[i]; stok[i] = ht[i]; }
        publish_expert(w, e, k, m, hb);
        if constexpr (kChecks) {
            bool bad = (tid == 0) && (m < 0 || m > k);
            for (int i = tid + 1; i < m && i < k; i += blockDim.x)
                bad = bad || better(hb[i], ht[i], hb[i - 1], ht[i - 1]) || ht[i] == ht[i - 1];
            if (bad) report_invariant(st);
        }
    }
    // where the tail finds the bidders if it takes over after this round
    // (no block of this kernel reads these fields)
    if (e == 0 && tid == 0) {
        ctl->cur = cur ^ 1;
        ctl->identity = 0;
        ctl->rounds_phase = round + 1;
    }
}

#include "auction_tail.h"
#include "auction_late.h"
static_assert(kLateG == kLateGWs && kLateCap == kLateCapWs && kLateG == 8,
              "late-round workspace sizes");

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

// Checking build: after the solve every expert holds exactly k tokens and
// no token is held twice (bexp, free by then, counts each token's holders).
__global__ void auc_check_zero_kernel(AucWs w, int64_t T) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t < T) w.bexp[t] = 0;
}
__global__ void auc_check_final_kernel(AucWs w, int64_t T, int64_t k, AucStatsDev* st) {
    const int e = blockIdx.x;
    if (w.ctl->abort) return;  // an error is already reported
    const int n = w.cnt[e];
    bool bad = threadIdx.x == 0 && n != k;
    for (int64_t i = threadIdx.x; i < n && i < k; i += blockDim.x) {
        const int32_t t = w.stok[(int64_t)e * k + i];
        bad = bad || t < 0 || t >= T || atomicAdd(&w.bexp[t], 1) != 0;
    }
    if (bad) report_invariant(st);
}

// ---------------------------------------------------------------- launcher

template <int NCH>
static void launch_tail(const float* s, int64_t T, int64_t E, int64_t k, const AucWs& w,
                        const ScoreScan* scan, double eps, int phase, int64_t max_bids,
                        AucStatsDev* st, hipStream_t stream) {
    auction_mark(4 * phase + 1, stream);
    const int sth = ssp_setup_threads(E);
    hipLaunchKernelGGL(auc_ssp_setup_kernel<NCH>, dim3((unsigned)(E * ssp_parts(E))), dim3(sth),
                       (size_t)(sth / 64) * 12 * E + 4 * kSetupChunk +
                           (E <= 128 ? (size_t)(sth / 64) * 8 * E * 4 : 0), stream, s,
                       E, k, w, scan);
    auction_mark(4 * phase + 2, stream);
    const size_t lds = ssp_lds_bytes(E);
    if (ssp_c_in_lds(E))
        hipLaunchKernelGGL((auc_ssp_kernel<NCH, true>), dim3(1), dim3(kSspThreads), lds, stream, s,
                           T, E, k, w, scan, eps, phase, max_bids, st);
    else
        hipLaunchKernelGGL((auc_ssp_kernel<NCH, false>), dim3(1), dim3(kSspThreads), lds, stream,
                           s, T, E, k, w, scan, eps, phase, max_bids, st);
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
    const int tail_max = k <= kSmallK ? kTailMaxSmallK : kTailMax;
    // the late rounds of a phase in one cooperative launch when the experts'
    // holders fit the workgroups' LDS
    const bool late = rounds > kLatePairs && late_ok(T, E, k);
    const int pair_rounds = late ? kLatePairs : rounds;
    const int late_enter = late ? kLateEnter : 0;
    const size_t late_lds = late ? late_lds_bytes(E, k) : 0;
    int64_t bid_blocks = (T + 15) / 16;
    if (bid_blocks > 2048) bid_blocks = 2048;
    double eps = eps_start;
    for (int phase = 0;; ++phase) {
        auction_mark(4 * phase, stream);
        hipLaunchKernelGGL(auc_phase_start_kernel, dim3((unsigned)((E + 255) / 256)), dim3(256), 0,
                           stream, w, T, E, st);
        for (int r = 0; r < pair_rounds; ++r) {
            // round 0: every token bids; later rounds: the returned few
            const unsigned nblk = (unsigned)(r == 0 ? bid_blocks : (bid_blocks < 256 ? bid_blocks : 256));
            hipLaunchKernelGGL(auc_bulk_bid_kernel<NCH>, dim3(nblk), dim3(256), 0,
                               stream, s, T, E, w, scan, r, eps, tail_max, late_enter);
            hipLaunchKernelGGL(auc_bulk_resolve_kernel, dim3((unsigned)E), dim3(256), 0, stream, T,
                               E, k, w, r, st);
        }
        if (late) {
            const float* sa = s;
            int64_t Ta = T, Ea = E, ka = k;
            AucWs wa = w;
            double epsa = eps;
            int tm = tail_max, mr = rounds;
            AucStatsDev* sta = st;
            void* args[] = {&sa, &Ta, &Ea, &ka, &wa, (void*)&scan, &epsa, &tm, &mr, &sta};
            const hipError_t le = hipLaunchCooperativeKernel((const void*)auc_late_kernel<NCH>,
                                                             dim3(kLateG), dim3(kLateThreads), args,
                                                             (unsigned)late_lds, stream);
            if (le != hipSuccess) return le;
        }
        launch_tail<NCH>(s, T, E, k, w, scan, eps, phase, max_bids, st, stream);
        auction_mark(4 * phase + 3, stream);
        if (eps <= eps_end) break;
        eps = eps / eps_factor;
        if (eps < eps_end) eps = eps_end;
    }
    hipLaunchKernelGGL(auc_finalize_kernel, dim3((unsigned)E), dim3(256), 0, stream, w, E, k, assign,
                       prices);
    if (kChecks) {
        hipLaunchKernelGGL(auc_check_zero_kernel, dim3((unsigned)((T + 255) / 256)), dim3(256), 0,
                           stream, w, T);
        hipLaunchKernelGGL(auc_check_final_kernel, dim3((unsigned)E), dim3(256), 0, stream, w, T, k,
                           st);
    }
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
