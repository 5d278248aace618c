// Tail of each eps phase of the auction (included by auction.hip, inside
// namespace base): one persistent workgroup finishes the displacement chains
// left after the bulk rounds.
//
// The end of a phase is a long sequence of dependent steps (a token evicts
// an expert's lowest holder, which bids next, ...). Each wave takes a queued
// bidder and follows its chain: bid against the current prices (b1 / v1 / v2
// by wave-wide DPP reductions), take the expert's lock in LDS, compare with
// its lowest holder, evict it, continue with the evicted token; when the
// chain ends (a free slot was filled) the wave takes the next queued bidder.
// A bid made against prices that rose meanwhile is just compared with the
// expert's current lowest holder: if it no longer beats it, the token bids
// again. Prices, price floors, holder counts and, per expert, a sorted list
// of its L lowest holders (bid, token, slot) with a flag telling whether it
// holds every holder live in LDS, so a step needs no memory round trip
// except the score row. Slot stores go to global memory; a full expert whose
// list runs dry rebuilds it from its k slots, after every store issued to
// that expert has landed (per expert counters: issued under the lock; a wave
// counts its store as landed at its next step, after its memory wait and
// before it takes any lock, so waiting for them cannot deadlock). The slots
// are written and read by this workgroup only, so plain loads (through the
// CU's own L1 and its XCD's L2) see them.
// For E <= 128 each expert's lowest holder -- the next token it will evict --
// has its score row cached in LDS: the wave that makes a token the lowest
// holder loads its row and publishes it at its next step (under the lock,
// if that token is still the lowest holder; the tag is cleared first and set
// last, and a reader checks it before and after reading), so an evicted
// token usually bids from LDS.

__host__ __device__ static inline bool tail_row_cache(int64_t E) { return E <= 128; }
__host__ __device__ constexpr int tail_threads(int nch) { return nch <= 8 ? 1024 : 512; }

static size_t tail_lds_bytes(int64_t E, int L, int threads) {
    size_t b = 8 * (2 * (size_t)E + (size_t)E * L) + 4 * (2 * (size_t)E * L + 6 * (size_t)E);
    b += (size_t)threads * 16;  // rebuild scratch: 64 entries per wave
    if (tail_row_cache(E)) b += 4 * (size_t)E + 4 * (size_t)E * (size_t)E;
    return b;
}

constexpr int kRbBatch = 8;  // slots per lane loaded at once by a rebuild
// bids a wave makes before it adds them to the workgroup's count and checks
// the bid cap (one shared atomic per batch instead of one per bid)
constexpr int kBidBatch = 8;

// Loads of data this workgroup wrote (after the writer's memory wait):
// workgroup scope, i.e. plain loads that may hit the CU's L1.
BASE_DEV double load_wg_f64(const double* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
BASE_DEV int load_wg_i32(const int32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

BASE_DEV void lds_lock(int32_t* p, int lane) {
    if (lane == 0) {
        int expect = 0;
        while (!__hip_atomic_compare_exchange_strong(p, &expect, 1, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_WORKGROUP)) {
            expect = 0;
            __builtin_amdgcn_s_sleep(1);
        }
    }
    asm volatile("" ::: "memory");
}
BASE_DEV bool lds_trylock(int32_t* p, int lane) {
    int ok = 0;
    if (lane == 0) {
        int expect = 0;
        ok = __hip_atomic_compare_exchange_strong(p, &expect, 1, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    asm volatile("" ::: "memory");
    return first_lane_i32(ok) != 0;
}
// release after this wave's LDS writes have completed (its global stores are
// tracked by the store counters instead)
BASE_DEV void lds_unlock(int32_t* p, int lane) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (lane == 0) __hip_atomic_store(p, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
BASE_DEV void lds_count(int32_t* p, int lane) {
    if (lane == 0) __hip_atomic_fetch_add(p, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Sort (bid, token, slot) triples across the wave into eviction order
// (bitonic network over the 64 lanes; entries (DBL_MAX, kNoTok) pad).
BASE_DEV void wave_sort_evict(double& b, int& t, int& s, int lane) {
#pragma unroll
    for (int k2 = 2; k2 <= 64; k2 <<= 1) {
#pragma unroll
        for (int j = k2 >> 1; j > 0; j >>= 1) {
            const double ob = shfl_xor_f64(b, j);
            const int ot = __shfl_xor(t, j, 64), os = __shfl_xor(s, j, 64);
            const bool take_first = ((lane & j) == 0) == ((lane & k2) == 0);
            const bool swap = take_first ? evict_first(ob, ot, b, t) : evict_first(b, t, ob, ot);
            if (swap) { b = ob; t = ot; s = os; }
        }
    }
}

// Rebuild an expert's lowest-holder list from its k slots (k >= 1, a full
// expert): the result is exactly its n lowest holders in eviction order, in
// lanes 0..n-1, n = min(L, k) as a rule. Each lane takes the first of the
// slots it reads (at most S = ceil(k / 64)); the r-th of those 64 lane minima
// bounds the r lowest holders from above, so only the slots at or before it
// -- typically a few more than r -- are gathered (scratch: 64 entries per
// wave in LDS) and sorted. At most r * S slots can qualify, so if more than
// 64 do, the gather is redone with r = 64 / S and the list is that long.
BASE_DEV void wave_rebuild(const double* sbid, const int32_t* stok, int64_t k, int lane, int L,
                           double* xb, int32_t* xt, int32_t* xs, double& lb, int& lt, int& ls,
                           int& n) {
    const bool single = k <= kRbBatch * 64;  // every slot of this lane stays in registers
    double bb[kRbBatch];
    int tt[kRbBatch];
    auto load = [&](int64_t i0) {
#pragma unroll
        for (int u = 0; u < kRbBatch; ++u) {
            const int64_t i = i0 + u * 64 + lane;
            bb[u] = DBL_MAX;
            tt[u] = kNoTok;
            if (i < k) { bb[u] = load_wg_f64(sbid + i); tt[u] = load_wg_i32(stok + i); }
        }
    };
    // pass 1: the first slot of each lane in eviction order, then sorted
    double mb = DBL_MAX;
    int mt = kNoTok, ms = -1;
    for (int64_t i0 = 0; i0 < k; i0 += kRbBatch * 64) {
        load(i0);
#pragma unroll
        for (int u = 0; u < kRbBatch; ++u)
            if (evict_first(bb[u], tt[u], mb, mt)) { mb = bb[u]; mt = tt[u]; ms = (int)(i0 + u * 64 + lane); }
    }
    wave_sort_evict(mb, mt, ms, lane);
    // pass 2: gather every slot at or before the r-th lane minimum
    auto gather = [&](int r) -> int {
        const double tb = readlane_f64(mb, r - 1);
        const int tk = readlane_i32(mt, r - 1);
        int cnt = 0;
        for (int64_t i0 = 0; i0 < k; i0 += kRbBatch * 64) {
            if (!single) load(i0);
#pragma unroll
            for (int u = 0; u < kRbBatch; ++u) {
                const bool in = tt[u] != kNoTok && !evict_first(tb, tk, bb[u], tt[u]);
                const unsigned long long m = __ballot(in);
                if (in) {
                    const unsigned long long below = lane ? (~0ull >> (64 - lane)) : 0ull;
                    const int at = cnt + __popcll(m & below);
                    if (at < 64) { xb[at] = bb[u]; xt[at] = tt[u]; xs[at] = (int)(i0 + u * 64 + lane); }
                }
                cnt += __popcll(m);
            }
        }
        return cnt;
    };
    int r = (int)(k < (int64_t)L ? k : (int64_t)L);
    int cnt = gather(r);
    if (cnt > 64) {
        const int S = (int)((k + 63) / 64);
        r = 64 / S < r ? 64 / S : r;
        if (r < 1) r = 1;
        cnt = gather(r);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    lb = DBL_MAX; lt = kNoTok; ls = -1;
    if (lane < cnt) { lb = xb[lane]; lt = xt[lane]; ls = xs[lane]; }
    wave_sort_evict(lb, lt, ls, lane);
    n = r;
    if (lane >= n) { lb = DBL_MAX; lt = kNoTok; ls = -1; }
}

template <int NCH>
__global__ __launch_bounds__(tail_threads(NCH)) void auc_tail_kernel(const float* s, int64_t T,
                                                                     int64_t E, int64_t k, AucWs w,
                                                                     const ScoreScan* scan,
                                                                     double eps, int phase,
                                                                     int64_t max_bids,
                                                                     AucStatsDev* st) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    constexpr int kThreads = tail_threads(NCH);
    const int L = w.L;
    double* pi = (double*)smem;                  // E
    double* flo = pi + E;                        // E
    double* lowb = flo + E;                      // E*L
    double* rbx_b = lowb + E * L;                // 64 per wave: rebuild scratch
    int32_t* lowt = (int32_t*)(rbx_b + kThreads);  // E*L
    int32_t* lows = lowt + E * L;                // E*L
    int32_t* cnt = lows + E * L;                 // E
    int32_t* nlow = cnt + E;                     // E
    int32_t* comp = nlow + E;                    // E
    int32_t* lock = comp + E;                    // E
    int32_t* st_issued = lock + E;               // E   slot stores issued
    int32_t* st_done = st_issued + E;            // E   slot stores landed
    int32_t* rbx_t = st_done + E;                // 64 per wave
    int32_t* rbx_s = rbx_t + kThreads;           // 64 per wave
    int32_t* rowtag = rbx_s + kThreads;          // E   token whose row is cached (cache on)
    float* rowc = (float*)(rowtag + E);          // E*E cached rows             (cache on)
    __shared__ int32_t next;
    __shared__ int32_t stop;
    __shared__ int32_t max_steps;
    __shared__ unsigned long long nbids;

    AucCtl* ctl = w.ctl;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = first_lane_i32(tid >> 6);
    const bool cache = tail_row_cache(E);
    const bool aborted = ctl->abort;
    const int cur = ctl->cur;
    const int64_t nb = aborted ? 0 : ctl->nbid[cur];
    const bool ident = ctl->identity;
    const int32_t* list = cur ? w.list1 : w.list0;
    for (int64_t e = tid; e < E; e += kThreads) {
        pi[e] = w.pi[e];
        flo[e] = w.floor_[e];
        cnt[e] = w.cnt[e];
        nlow[e] = w.nlow[e];
        comp[e] = w.comp[e];
        lock[e] = 0;
        st_issued[e] = 0;
        st_done[e] = 0;
        if (cache) rowtag[e] = -1;
    }
    for (int64_t i = tid; i < E * L; i += kThreads) {
        lowb[i] = w.lowb[i];
        lowt[i] = w.lowt[i];
        lows[i] = w.lows[i];
    }
    if (tid == 0) {
        next = 0;
        max_steps = 0;
        const unsigned long long before = ctl->bids_total + ctl->bids_phase;
        stop = (max_bids > 0 && before >= (unsigned long long)max_bids && nb > 0) ? 1 : 0;
        nbids = 0;
    }
    __syncthreads();
    const Sani sn = read_sani(scan);
    const unsigned long long cap =
        max_bids > 0 ? (unsigned long long)max_bids - min<unsigned long long>(
                           (unsigned long long)max_bids, ctl->bids_total + ctl->bids_phase)
                     : ~0ull;
    // fill the row cache with every expert's lowest holder (its next victim)
    if (cache) {
        for (int64_t e = wave; e < E; e += kThreads / 64) {
            if (first_lane_i32(nlow[e]) == 0) continue;
            const int h = first_lane_i32(lowt[e * L]);
            float r[NCH];
            load_row<NCH>(s, h, E, lane, sn, r);
#pragma unroll
            for (int c = 0; c < NCH; ++c)
                if (lane + 64 * c < E) rowc[e * E + lane + 64 * c] = r[c];
            if (lane == 0) rowtag[e] = h;
        }
        __syncthreads();
    }
    double* xb = rbx_b + wave * 64;
    int32_t* xt = rbx_t + wave * 64;
    int32_t* xs = rbx_s + wave * 64;
    // this wave's bids not yet in nbids, and whether the cap had been reached
    // at its last check (other waves' stops are seen at this wave's next one)
    int lbids = 0;
    bool halted = first_lane_i32(stop) != 0;
    auto flush_bids = [&]() {
        if (lane == 0 && lbids > 0) {
            const unsigned long long nbd =
                atomicAdd(&nbids, (unsigned long long)lbids) + (unsigned long long)lbids;
            if (nbd >= cap) stop = 1;
        }
        lbids = 0;
        halted = first_lane_i32(stop) != 0;
    };
    auto count_bid = [&]() {
        if (++lbids >= kBidBatch) flush_bids();
    };

    int pending = -1;        // expert with this wave's last slot store not yet counted
    int cpe = -1, cpt = -1;  // row loaded for the cache: expert, token
    float cpv[NCH];
    int steps = 0;
    for (;;) {
        int j = 0;
        if (lane == 0) j = atomicAdd(&next, 1);
        j = first_lane_i32(j);
        if (j >= nb || first_lane_i32(stop)) break;
        int t = ident ? j : first_lane_i32(list[j]);
        int fr = -1;  // expert t was just evicted from
        while (t >= 0) {
            if (halted) break;
            // the row: from the cache when the tag names t before and after
            float v[NCH];
            bool hit = false;
            if (cache && fr >= 0 && first_lane_i32(rowtag[fr]) == t) {
#pragma unroll
                for (int c = 0; c < NCH; ++c) v[c] = (lane + 64 * c < E) ? rowc[fr * E + lane + 64 * c] : 0.0f;
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                hit = first_lane_i32(rowtag[fr]) == t;
            }
            if (!hit) load_row<NCH>(s, t, E, lane, sn, v);
            if (cpe >= 0) {
                // publish the row loaded last step if its token is still the lowest holder
                if (lds_trylock(&lock[cpe], lane)) {
                    if (first_lane_i32(nlow[cpe]) > 0 && first_lane_i32(lowt[(int64_t)cpe * L]) == cpt) {
                        if (lane == 0) rowtag[cpe] = -1;
                        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
                        for (int c = 0; c < NCH; ++c) {
                            float x = cpv[c];
                            if (sn.fix && !is_finite_f32(x)) x = sn.repl;
                            if (lane + 64 * c < E) rowc[cpe * E + lane + 64 * c] = x;
                        }
                        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                        if (lane == 0) rowtag[cpe] = cpt;
                    }
                    lds_unlock(&lock[cpe], lane);
                }
                cpe = -1;
            }
            for (;;) {
                int e;
                double v1, v2, pb;
                best_two<NCH>(v, pi, E, lane, e, v1, v2, pb);
                const double beta = bid_amount(pb, v1, v2, eps);
                // the slot store of the previous step has landed once this
                // returns; it is counted before this wave waits for any lock
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                if (pending >= 0) {
                    lds_count(&st_done[pending], lane);
                    pending = -1;
                }
                lds_lock(&lock[e], lane);
                // ---- under the lock of e
                const int64_t eb = (int64_t)e * L;
                int32_t* stk = w.stok + (int64_t)e * k;
                double* sbd = w.sbid + (int64_t)e * k;
                int c = first_lane_i32(cnt[e]), nl = first_lane_i32(nlow[e]);
                int cp = first_lane_i32(comp[e]);
                double lb = DBL_MAX;
                int lt = kNoTok, ls = -1;
                if (lane < nl) { lb = lowb[eb + lane]; lt = lowt[eb + lane]; ls = lows[eb + lane]; }
                const int head0 = readlane_i32(lt, 0);
                auto rebuild = [&]() {
                    if (lane == 0) {
                        const int want = __hip_atomic_load(&st_issued[e], __ATOMIC_RELAXED,
                                                           __HIP_MEMORY_SCOPE_WORKGROUP);
                        while (__hip_atomic_load(&st_done[e], __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_WORKGROUP) != want)
                            __builtin_amdgcn_s_sleep(1);
                    }
                    asm volatile("" ::: "memory");
                    wave_rebuild(sbd, stk, k, lane, L, xb, xt, xs, lb, lt, ls, nl);
                    cp = (nl >= k) ? 1 : 0;
                };
                if (c >= k && nl == 0) rebuild();
                if (c >= k && !evict_first(readlane_f64(lb, 0), readlane_i32(lt, 0), beta, t)) {
                    // the price rose since the bid: bid again (counted, so the
                    // bid cap also ends a phase that cannot progress)
                    lds_unlock(&lock[e], lane);
                    count_bid();
                    if (halted) { t = -1; break; }
                    continue;
                }
                int slot, victim = -1;
                if (c < k) {
                    slot = c++;
                } else {
                    // pop the lowest holder (lane 0 of the list)
                    victim = readlane_i32(lt, 0);
                    slot = readlane_i32(ls, 0);
                    const double nb_ = dpp_f64<kDppWaveShl1>(lb);
                    const int nt = dpp_i32<kDppWaveShl1>(lt);
                    const int ns = dpp_i32<kDppWaveShl1>(ls);
                    if (lane + 1 < nl) { lb = nb_; lt = nt; ls = ns; }
                    else { lb = DBL_MAX; lt = kNoTok; ls = -1; }
                    --nl;
                }
                if (lane == 0) {
                    stk[slot] = t;
                    sbd[slot] = beta;
                    // no-return LDS add: visible before the unlock's wait ends
                    __hip_atomic_fetch_add(&st_issued[e], 1, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_WORKGROUP);
                }
                pending = e;
                // the new holder enters the list if the list covers it
                const bool before = lane < nl && evict_first(lb, lt, beta, t);
                const int pos = __popcll(__ballot(before));
                if ((nl < L && cp) || pos < nl) {
                    const double pb_ = dpp_f64<kDppWaveShr1>(lb);
                    const int pt_ = dpp_i32<kDppWaveShr1>(lt);
                    const int ps = dpp_i32<kDppWaveShr1>(ls);
                    if (lane == pos) { lb = beta; lt = t; ls = slot; }
                    else if (lane > pos) { lb = pb_; lt = pt_; ls = ps; }
                    if (nl == L) cp = 0;  // the old last entry dropped out
                    else ++nl;
                } else {
                    cp = 0;
                }
                if (c >= k && nl == 0) {
                    // a full expert publishes its lowest bid: count this wave's
                    // own store as landed first, then rebuild
                    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                    lds_count(&st_done[e], lane);
                    pending = -1;
                    rebuild();
                }
                if (lane < nl) { lowb[eb + lane] = lb; lowt[eb + lane] = lt; lows[eb + lane] = ls; }
                const double head_bid = readlane_f64(lb, 0);
                const int head1 = readlane_i32(lt, 0);
                if (lane == 0) {
                    cnt[e] = c;
                    nlow[e] = nl;
                    comp[e] = cp;
                    pi[e] = (c >= k) ? head_bid : flo[e];
                }
                if (cache && nl > 0 && head1 != head0) {
                    // a new lowest holder: load its row for the cache
                    cpe = e;
                    cpt = head1;
                    if (head1 == t) {
#pragma unroll
                        for (int cc = 0; cc < NCH; ++cc) cpv[cc] = v[cc];
                    } else {
                        // raw load (sanitized when published): nothing waits for it here
                        const float* row = s + (int64_t)head1 * E;
#pragma unroll
                        for (int cc = 0; cc < NCH; ++cc)
                            cpv[cc] = (lane + 64 * cc < E) ? row[lane + 64 * cc] : 0.0f;
                    }
                }
                lds_unlock(&lock[e], lane);
                count_bid();
                ++steps;
                t = victim;
                fr = e;
                break;
            }
        }
    }
    flush_bids();
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (pending >= 0) lds_count(&st_done[pending], lane);
    if (lane == 0) atomicMax(&max_steps, steps);
    __syncthreads();
    if (tid == 0) {
        const unsigned long long pb = ctl->bids_phase + nbids;
        ctl->bids_total += pb;
        if (phase < 16) {
            st->bids[phase] = (long long)pb;
            st->rounds[phase] = ctl->rounds_phase + max_steps;
        }
        st->phases = phase + 1;
        if (stop && !aborted) st->status = kErrNotConverged;
    }
    // every expert is full: its price floor becomes its lowest held bid
    for (int64_t e = tid; e < E; e += kThreads) {
        w.floor_[e] = (cnt[e] == k) ? pi[e] : flo[e];
        w.cnt[e] = cnt[e];
    }
}
