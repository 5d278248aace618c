// Late bulk rounds of an eps phase of the auction (included by auction.hip,
// inside namespace base), as one cooperative launch.
//
// After a phase's first rounds most tokens hold a slot, and each further
// round carries a few hundred bids or fewer: two launches per round (bid,
// then resolve) then cost more than the work, since every launch boundary
// and every round trip to memory is on the critical path. Here the rounds
// run inside one launch of kLateG workgroups that meet at a device-wide
// barrier twice per round (an 8-way barrier costs about a microsecond on
// gfx950, a dependent launch about three).
//
// Ownership. Expert e belongs to workgroup e % kLateG, and within it to wave
// (e / kLateG) % 16; its holders stay in that workgroup's LDS for the whole
// launch, sorted best first. Each workgroup keeps its own list of bidders
// (the tokens its experts rejected, and those of its bids that found no room)
// in global memory; no list is shared between workgroups.
//
// Round:
//  bid      every wave takes bidders of its workgroup's list, loads the
//           token's score row and bids against the round's prices exactly as
//           the bulk rounds do; the bid goes to the (workgroup, expert) bin at
//           a place counted in LDS. A bin holds kLateCap bids: a bid that
//           finds it full is not delivered, and its token bids again next
//           round. The bin counts go to global memory.
//  barrier
//  resolve  the owner wave of expert e reads the kLateG bin counts and the
//           bids, 64 at a time: ranks them among themselves (readlane
//           counts), places each by binary search among the holders, shifts
//           the holders past it, and appends those ranked >= k to its
//           workgroup's next list at rank - k; then publishes e's price.
//  barrier  (the workgroups' next-list sizes are summed on the way).
// It stops once at most tail_max bidders remain, or after max_rounds rounds,
// and leaves the state where the bulk rounds would: holders in the expert
// slots, the bidders in the global list named by ctl->cur.
//
// Every wait is bounded: a barrier that does not complete within its spin
// budget sets the abort flag and an error status, and every workgroup leaves.

constexpr int kLateG = 8;
constexpr int kLateWaves = 16;
constexpr int kLateThreads = 64 * kLateWaves;
constexpr int kLateCap = 256;       // bids one workgroup files with one expert per round
constexpr int kLateHold = 8;        // holder slots per lane of the owner wave (k <= 512)
// The bulk rounds (two launches each) hand over to the late launch once at
// most kLateEnter bidders remain; the host launches kLatePairs of them first
// (those after the hand-over return at once). The late launch is used up to
// kLateMaxT tokens: there a solve is mostly launch latency (a 512-token
// solve's rounds went from 0.21 to 0.06 ms). At 16k-64k tokens it measured
// no faster than the two-launch rounds (its rounds with a few hundred
// bidders are bound by each wave's serial bids), so those keep the bulk
// rounds throughout.
constexpr int kLateEnter = 2048;
constexpr int kLatePairs = 2;
constexpr int64_t kLateMaxT = 8192;
constexpr unsigned kLateSpin = 1u << 20;
constexpr size_t kLateLdsMax = 140 * 1024;  // dynamic LDS; 12 KB more are static

__host__ __device__ static inline int64_t late_ne(int64_t E) { return (E + kLateG - 1) / kLateG; }

static size_t late_lds_bytes(int64_t E, int64_t k) {
    const int64_t ne = late_ne(E);
    return (size_t)(ne * k * 8 + ne * 8 + ne * k * 4 + ne * 4 + E * 4 + 16);
}

static bool late_ok(int64_t T, int64_t E, int64_t k) {
    return T <= kLateMaxT && k >= 1 && k <= 64 * kLateHold && late_lds_bytes(E, k) <= kLateLdsMax;
}

// Device-wide barrier of the late launch. Every thread first waits until its
// own memory operations have completed (so its stores have reached this
// XCD's L2); thread 0 then releases at device scope (one write-back of the
// L2 for the whole workgroup), arrives, waits for the target count (kLateG
// arrivals per barrier) and acquires (one invalidate of this CU's caches,
// which the other waves share). False if the wait ran out of budget or
// another workgroup gave up (the launch is then abandoned).
BASE_DEV bool late_sync(AucCtl* ctl, unsigned target, AucStatsDev* st, int* ok_s) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
        __hip_atomic_fetch_add(&ctl->lbar, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        unsigned spins = 0;
        int ok = 1;
        while (__hip_atomic_load(&ctl->lbar, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
            if (__hip_atomic_load(&ctl->abort, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
                ok = 0;
                break;
            }
            if (++spins > kLateSpin) {
                __hip_atomic_store(&ctl->abort, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(&st->status, kErrNotConverged, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
                ok = 0;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // polled relaxed, acquire once
        *ok_s = ok;
    }
    __syncthreads();
    return *ok_s != 0;
}

// One owner wave merges a chunk of n <= 64 bids (lane l < n holds bid bb,
// token bt; the other lanes hold distinct worse-than-any pads) into the c
// holders H/Ht (sorted best first, c <= k <= 64 * kLateHold). A bid's new
// place is its rank among the chunk plus the holders better than it (binary
// search); holder i moves past the bids better than it, which are those
// whose count of better holders is <= i. Places >= k are rejected and go to
// the workgroup's next list at base + place - k. Returns the new count.
BASE_DEV int late_merge_chunk(double* H, int32_t* Ht, int c, int64_t k, double bb, int bt, int n,
                              int32_t* lnext, int32_t* nl_next, int lane) {
    const int qr = wave_rank_best(bb, bt, n);
    int lo = 0;
    if (lane < n) {
        int hi = c;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (better(H[mid], Ht[mid], bb, bt)) lo = mid + 1;
            else hi = mid;
        }
    }
    double hv[kLateHold];
    int hk[kLateHold], sh[kLateHold];
#pragma unroll
    for (int u = 0; u < kLateHold; ++u) {
        const int i = lane + 64 * u;
        hv[u] = i < c ? H[i] : 0.0;
        hk[u] = i < c ? Ht[i] : 0;
        sh[u] = 0;
    }
    for (int l = 0; l < n; ++l) {
        const int lol = __builtin_amdgcn_readlane(lo, l);
#pragma unroll
        for (int u = 0; u < kLateHold; ++u) sh[u] += (lol <= lane + 64 * u) ? 1 : 0;
    }
    const int c2 = (int)min<int64_t>(c + n, k);
    const int nrej = c + n - c2;
    int base = 0;
    if (lane == 0 && nrej > 0) base = atomicAdd(nl_next, nrej);
    base = __builtin_amdgcn_readlane(base, 0);
#pragma unroll
    for (int u = 0; u < kLateHold; ++u) {
        const int i = lane + 64 * u;
        if (i < c) {
            const int r = i + sh[u];
            if (r < k) { H[r] = hv[u]; Ht[r] = hk[u]; }
            else lnext[base + r - k] = hk[u];
        }
    }
    if (lane < n) {
        const int r = qr + lo;
        if (r < k) { H[r] = bb; Ht[r] = bt; }
        else lnext[base + r - k] = bt;
    }
    return c2;
}

template <int NCH>
__global__ __launch_bounds__(kLateThreads) void auc_late_kernel(const float* s, int64_t T,
                                                               int64_t E, int64_t k, AucWs w,
                                                               const ScoreScan* scan, double eps,
                                                               int tail_max, int max_total,
                                                               AucStatsDev* st) {
    extern __shared__ __attribute__((aligned(16))) char sm[];
    const int ne = (int)late_ne(E);
    double* hb = (double*)sm;                          // ne x k holder bids, best first
    double* fl = hb + (int64_t)ne * k;                 // ne price floors
    int32_t* ht = (int32_t*)(fl + ne);                 // ne x k holder tokens
    int32_t* hc = ht + (int64_t)ne * k;                // ne holder counts
    int32_t* lcnt = hc + ne;                           // E bids filed this round, per expert
    __shared__ int32_t nl_cur, nl_next, ok_s, base_s, cw_s[kLateG + 1];
    __shared__ int64_t go_s;
    __shared__ unsigned long long bids_s;

    AucCtl* ctl = w.ctl;
    const int g = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // where the bulk rounds left the bidders (nothing below changes these
    // fields before every workgroup has read them)
    const int cur0 = ctl->cur;
    const int64_t nb0 = ctl->nbid[cur0];
    const bool ident = ctl->identity;
    const int round0 = (int)ctl->rounds_phase;  // bulk rounds already run
    const int max_rounds = max_total - round0;
    if (ctl->abort || ctl->bulk_done || nb0 <= tail_max || max_rounds <= 0) return;
    const int X = cur0 ^ 1;  // the global list the bidders leave in
    if (g == 0 && tid == 0) ctl->nbid[X] = 0;
    const int32_t* gl = cur0 ? w.list1 : w.list0;
    int32_t* gx = X ? w.list1 : w.list0;
    int32_t* myl[2] = {w.llist + (int64_t)(2 * g) * T, w.llist + (int64_t)(2 * g + 1) * T};
    const Sani sn = read_sani(scan);

    // this workgroup's share of the bidders (every kLateG-th), its experts'
    // holders, counts and floors
    const int64_t n0 = nb0 > g ? (nb0 - g + kLateG - 1) / kLateG : 0;
    for (int64_t i = tid; i < n0; i += kLateThreads) {
        const int64_t j = g + (int64_t)kLateG * i;
        myl[0][i] = ident ? (int32_t)j : gl[j];
    }
    for (int q = tid; q < ne; q += kLateThreads) {
        const int64_t e = g + (int64_t)kLateG * q;
        hc[q] = e < E ? w.cnt[e] : 0;
        fl[q] = e < E ? w.floor_[e] : 0.0;
    }
    for (int64_t e = tid; e < E; e += kLateThreads) lcnt[e] = 0;
    if (tid == 0) { nl_cur = (int32_t)n0; nl_next = 0; bids_s = 0; go_s = 0; }
    __syncthreads();
    for (int64_t x = tid; x < (int64_t)ne * k; x += kLateThreads) {
        const int q = (int)(x / k);
        const int64_t i = x - (int64_t)q * k;
        const int64_t e = g + (int64_t)kLateG * q;
        if (e < E && i < hc[q]) { hb[x] = w.sbid[e * k + i]; ht[x] = w.stok[e * k + i]; }
    }
    __syncthreads();

    unsigned target = 0;
    int par = 0, r = 0;
    double pv[NCH];
    while (r < max_rounds) {
        // This round's bidders. In the first round, and while few remain,
        // each workgroup takes its own list; with more, the lists'
        // concatenation is split evenly (rejected tokens land in their
        // expert's workgroup, so contested experts would load one workgroup).
        const bool split = r > 0 && go_s > kLateWaves * kLateG;
        int64_t lo = 0;
        int nl = nl_cur;
        if (split) {
            lo = go_s * g / kLateG;
            nl = (int)(go_s * (g + 1) / kLateG - lo);
        }
        // token of bidder j of this workgroup's share
        auto bidder = [&](int j) -> int {
            if (!split) return myl[par][j];
            const int64_t x = lo + j;
            int src = 0;
#pragma unroll
            for (int gg = 1; gg < kLateG; ++gg)
                if (x >= cw_s[gg]) src = gg;
            return w.llist[(int64_t)(2 * src + par) * T + (x - cw_s[src])];
        };
        int32_t* lnxt = myl[par ^ 1];
        // ---- bid: the round's prices, then each wave's bidders (the next
        // bidder's row loaded while the current one bids)
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int64_t e = lane + 64 * c;
            pv[c] = (e < E) ? w.pi[e] : 0.0;
        }
        {
            // LB bidders per wave at a time, their rows loaded together
            constexpr int LB = NCH <= 2 ? 4 : (NCH <= 4 ? 2 : 1);
            for (int j0 = wave; j0 < nl; j0 += LB * kLateWaves) {
                int tt[LB];
                float v[LB][NCH];
#pragma unroll
                for (int u = 0; u < LB; ++u) {
                    const int j = j0 + u * kLateWaves;
                    tt[u] = j < nl ? bidder(j) : -1;
                }
#pragma unroll
                for (int u = 0; u < LB; ++u)
                    if (tt[u] >= 0) load_row<NCH>(s, tt[u], E, lane, sn, v[u]);
#pragma unroll
                for (int u = 0; u < LB; ++u) {
                    if (tt[u] < 0) continue;
                    int b1;
                    double v1, v2, pb;
                    best_two_pv<NCH>(v[u], pv, E, lane, b1, v1, v2, pb);
                    if (lane == 0) {
                        const double bid = bid_amount(pb, v1, v2, eps);
                        const int pos = atomicAdd(&lcnt[b1], 1);
                        if (pos < kLateCap) {
                            const int64_t at = ((int64_t)g * E + b1) * kLateCap + pos;
                            w.lbin_t[at] = tt[u];
                            w.lbin_v[at] = bid;
                        } else {
                            lnxt[atomicAdd(&nl_next, 1)] = tt[u];  // not delivered: bids again
                        }
                    }
                }
            }
        }
        if (tid == 0) bids_s += (unsigned long long)nl;
        __syncthreads();
        for (int64_t e = tid; e < E; e += kLateThreads) {
            w.lbc[(int64_t)g * E + e] = min(lcnt[e], kLateCap);
            lcnt[e] = 0;
        }
        target += kLateG;
        if (!late_sync(ctl, target, st, &ok_s)) return;
        if (g == 0 && tid == 0) ctl->lnb[(r + 1) & 1] = 0;
        // ---- resolve: one wave per owned expert
        for (int q = wave; q < ne; q += kLateWaves) {
            const int64_t e = g + (int64_t)kLateG * q;
            if (e >= E) continue;
            // the kLateG bin counts, and the first kSpec bids of every bin
            // loaded with them (read before the counts are known: the bins
            // hold kLateCap entries, those past a count are ignored)
            constexpr int kSpec = 64 / kLateG;
            const int sg = lane / kSpec, si = lane % kSpec;
            const int64_t sat = ((int64_t)sg * E + e) * kLateCap + si;
            const int spt = w.lbin_t[sat];
            const double spv = w.lbin_v[sat];
            const int myc = lane < kLateG ? w.lbc[(int64_t)lane * E + e] : 0;
            int pre[kLateG + 1];
            pre[0] = 0;
#pragma unroll
            for (int gg = 0; gg < kLateG; ++gg) pre[gg + 1] = pre[gg] + __builtin_amdgcn_readlane(myc, gg);
            const int ntot = pre[kLateG];
            if (ntot == 0) continue;
            double* H = hb + (int64_t)q * k;
            int32_t* Ht = ht + (int64_t)q * k;
            int c = hc[q];
            bool few = true;  // every bin within the prefetched entries
#pragma unroll
            for (int gg = 0; gg < kLateG; ++gg) few = few && (pre[gg + 1] - pre[gg] <= kSpec);
            if (few) {
                // lane sg*kSpec+si holds entry si of bin sg: compact the live
                // ones into lanes 0 .. ntot-1
                int cnt_sg = 0, pre_sg = 0;
#pragma unroll
                for (int gg = 0; gg < kLateG; ++gg)
                    if (gg == sg) { cnt_sg = pre[gg + 1] - pre[gg]; pre_sg = pre[gg]; }
                const bool live = si < cnt_sg;
                const int dst = pre_sg + si;
                __shared__ double spv_s[kLateWaves][64];
                __shared__ int32_t spt_s[kLateWaves][64];
                if (live) { spv_s[wave][dst] = spv; spt_s[wave][dst] = spt; }
                __builtin_amdgcn_s_waitcnt(0);
                __builtin_amdgcn_wave_barrier();
                const double bb = lane < ntot ? spv_s[wave][lane] : -DBL_MAX;
                const int bt = lane < ntot ? spt_s[wave][lane] : kNoTok - lane;
                c = late_merge_chunk(H, Ht, c, k, bb, bt, ntot, lnxt, &nl_next, lane);
            }
            for (int c0 = 0; !few && c0 < ntot; c0 += 64) {
                const int x = c0 + lane;
                double bb = -DBL_MAX;
                int bt = kNoTok - lane;
                if (x < ntot) {
                    int src = 0, off0 = 0;
#pragma unroll
                    for (int gg = 1; gg < kLateG; ++gg)
                        if (x >= pre[gg]) { src = gg; off0 = pre[gg]; }
                    const int64_t at = ((int64_t)src * E + e) * kLateCap + (x - off0);
                    bt = w.lbin_t[at];
                    bb = w.lbin_v[at];
                }
                c = late_merge_chunk(H, Ht, c, k, bb, bt, min(64, ntot - c0), lnxt, &nl_next, lane);
            }
            if (lane == 0) {
                hc[q] = c;
                w.pi[e] = (c == k) ? H[k - 1] : fl[q];
            }
        }
        __syncthreads();
        if (tid == 0) {
            ctl->lcw[r & 1][g] = nl_next;
            atomicAdd(&ctl->lnb[r & 1], nl_next);
        }
        target += kLateG;
        if (!late_sync(ctl, target, st, &ok_s)) return;
        if (tid == 0) {
            // the total and every workgroup's count, loaded together; their
            // prefix sums place each list in the concatenation
            int cw[kLateG];
#pragma unroll
            for (int gg = 0; gg < kLateG; ++gg) cw[gg] = ctl->lcw[r & 1][gg];
            go_s = __hip_atomic_load(&ctl->lnb[r & 1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            int acc = 0;
#pragma unroll
            for (int gg = 0; gg < kLateG; ++gg) { cw_s[gg] = acc; acc += cw[gg]; }
            cw_s[kLateG] = acc;
            nl_cur = nl_next;
            nl_next = 0;
        }
        __syncthreads();
        par ^= 1;
        ++r;
        if (go_s <= tail_max) break;
    }

    // ---- leave the state as the bulk rounds would: holders in the expert
    // slots, the bidders in global list X
    for (int64_t x = tid; x < (int64_t)ne * k; x += kLateThreads) {
        const int q = (int)(x / k);
        const int64_t i = x - (int64_t)q * k;
        const int64_t e = g + (int64_t)kLateG * q;
        if (e < E && i < hc[q]) { w.sbid[e * k + i] = hb[x]; w.stok[e * k + i] = ht[x]; }
    }
    for (int q = tid; q < ne; q += kLateThreads) {
        const int64_t e = g + (int64_t)kLateG * q;
        if (e < E) w.cnt[e] = hc[q];
    }
    if constexpr (kChecks) {
        for (int64_t x = tid; x < (int64_t)ne * k; x += kLateThreads) {
            const int q = (int)(x / k);
            const int64_t i = x - (int64_t)q * k;
            const bool bad = hc[q] > k ||
                             (i > 0 && i < hc[q] && (better(hb[x], ht[x], hb[x - 1], ht[x - 1]) || ht[x] == ht[x - 1]));
            if (bad) report_invariant(st);
        }
    }
    const int nl = nl_cur;
    if (tid == 0) {
        base_s = nl > 0 ? atomicAdd(&ctl->nbid[X], nl) : 0;
        atomicAdd(&ctl->bids_phase, bids_s);
    }
    __syncthreads();
    const int base = base_s;
    for (int i = tid; i < nl; i += kLateThreads) gx[base + i] = myl[par][i];
    if (g == 0 && tid == 0) {
        ctl->cur = X;
        ctl->identity = 0;
        ctl->rounds_phase = round0 + r;
    }
}
