// Tail of each eps phase of the auction (included by auction.hip, inside
// namespace base): one persistent workgroup of 16 waves finishes the
// displacement chains left after the bulk rounds.
//
// The end of a phase is a long sequence of dependent steps (bid, evict the
// expert's lowest holder, the evicted token bids, ...), so a step must be
// short: each chain wave holds one token with its E scores spread over the
// 64 lanes, reductions use DPP within rows of 16 plus four readlanes, and
// every per-expert structure lives in LDS:
//   price, holder count, lock, a sorted list of the L lowest holders (bid,
//   token, slot) with a flag telling whether it holds every holder, and two
//   counters of slot stores (issued / landed);
//   for E <= 128, a cache of the score row of each expert's lowest holder --
//   the next token it will evict. A chain wave that evicts that token takes
//   its row from LDS instead of memory; helper waves keep the cache filled.
// A commit -- pop the lowest holder, store the new holder into its slot,
// insert the new bid into the list if the list covers it, set the new price
// -- touches only LDS, plus two fire-and-forget global stores, and releases
// the lock with an LDS-only wait. When a full expert's list runs dry it is
// rebuilt from the expert's k slots in global memory; the rebuild first waits
// until every slot store issued to the expert has landed (a wave counts its
// stores as landed at its next step, after its memory wait) and reads the
// slots past the L1.

constexpr int kHelperWaves = 4;  // row-cache fillers when the cache is on

__host__ __device__ static inline bool tail_row_cache(int64_t E) { return E <= 128; }

static size_t tail_lds_bytes(int64_t E, int L) {
    size_t b = (size_t)E * (8 + 8 + 6 * 4) + (size_t)E * (size_t)L * 16;
    if (tail_row_cache(E)) b += (size_t)E * 4 + (size_t)E * (size_t)E * 4;
    return b;
}

BASE_DEV void lds_lock(int32_t* p) {
    int expect = 0;
    while (!__hip_atomic_compare_exchange_strong(p, &expect, 1, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_WORKGROUP)) {
        expect = 0;
        __builtin_amdgcn_s_sleep(1);
    }
    asm volatile("" ::: "memory");
}
BASE_DEV bool lds_trylock(int32_t* p) {
    int expect = 0;
    const bool ok = __hip_atomic_compare_exchange_strong(p, &expect, 1, __ATOMIC_RELAXED,
                                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    asm volatile("" ::: "memory");
    return ok;
}
// Release after this wave's LDS writes have completed (global stores may
// still be in flight: they are tracked by the store counters instead).
BASE_DEV void lds_unlock(int32_t* p) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __hip_atomic_store(p, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

BASE_DEV double load_l2_f64(const double* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
BASE_DEV int load_l2_i32(const int32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int C>
BASE_DEV void argmin4_step(double& b, int& t, int& s, int& w) {
    const double ob = dpp_f64<C>(b);
    const int ot = dpp_i32<C>(t), os = dpp_i32<C>(s), ow = dpp_i32<C>(w);
    if (evict_first(ob, ot, b, t) || (ob == b && ot == t && ow < w)) { b = ob; t = ot; s = os; w = ow; }
}
// the first entry in eviction order over the wave; result in all lanes
BASE_DEV void wave_argmin4(double& b, int& t, int& s, int& w) {
    argmin4_step<kDppXor1>(b, t, s, w);
    argmin4_step<kDppXor2>(b, t, s, w);
    argmin4_step<kDppHalfMirror>(b, t, s, w);
    argmin4_step<kDppMirror>(b, t, s, w);
    double bb = readlane_f64(b, 0);
    int bt = readlane_i32(t, 0), bs = readlane_i32(s, 0), bw = readlane_i32(w, 0);
#pragma unroll
    for (int r = 16; r < 64; r += 16) {
        const double ob = readlane_f64(b, r);
        const int ot = readlane_i32(t, r), os = readlane_i32(s, r), ow = readlane_i32(w, r);
        if (evict_first(ob, ot, bb, bt) || (ob == bb && ot == bt && ow < bw)) {
            bb = ob; bt = ot; bs = os; bw = ow;
        }
    }
    b = bb; t = bt; s = bs; w = bw;
}

// Rebuild an expert's lowest-holder list from its k slots: each lane keeps
// the 4 lowest of the slots it reads, then the wave merges the lanes' heads.
// The merge stops once a lane's 4 entries are used up, so the result is
// always exactly the n lowest holders (n <= L), in eviction order, in lanes
// 0..n-1. The slot just written (slot_new, or -1) comes from registers.
BASE_DEV void wave_rebuild(const double* sbid, const int32_t* stok, int64_t k, int lane, int L,
                           int slot_new, double b_new, int t_new, double& lb, int& lt, int& ls,
                           int& n) {
    double qb[4];
    int qt[4], qs[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) { qb[j] = DBL_MAX; qt[j] = kNoTok; qs[j] = -1; }
    for (int64_t i = lane; i < k; i += 64) {
        double b = load_l2_f64(sbid + i);
        int t = load_l2_i32(stok + i);
        const int sl = (int)i;
        if (sl == slot_new) { b = b_new; t = t_new; }
        if (!evict_first(b, t, qb[3], qt[3])) continue;
        int p = 3;
#pragma unroll
        for (int j = 3; j > 0; --j) {
            if (p == j && evict_first(b, t, qb[j - 1], qt[j - 1])) {
                qb[j] = qb[j - 1]; qt[j] = qt[j - 1]; qs[j] = qs[j - 1];
                p = j - 1;
            }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (j == p) { qb[j] = b; qt[j] = t; qs[j] = sl; }
    }
    int head = 0;
    n = 0;
    lb = DBL_MAX; lt = kNoTok; ls = -1;
    for (int r = 0; r < L; ++r) {
        double mb = DBL_MAX;
        int mt = kNoTok, ms = -1, mw = lane;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (j == head) { mb = qb[j]; mt = qt[j]; ms = qs[j]; }
        wave_argmin4(mb, mt, ms, mw);
        if (mt == kNoTok) break;  // no holder left
        if (lane == r) { lb = mb; lt = mt; ls = ms; }
        ++n;
        if (lane == mw) ++head;
        if (readlane_i32(head, mw) == 4) break;  // that lane's candidates are used up
    }
}

template <int NCH>
__global__ __launch_bounds__(kTailThreads) void auc_tail_kernel(const float* s, int64_t T, int64_t E,
                                                                int64_t k, AucWs w,
                                                                const ScoreScan* scan, double eps,
                                                                int phase, int64_t max_bids,
                                                                AucStatsDev* st) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int L = w.L;
    const bool cache = tail_row_cache(E);
    double* pi = (double*)smem;                 // E
    double* flo = pi + E;                       // E
    double* lowb = flo + E;                     // E*L
    int32_t* lowt = (int32_t*)(lowb + E * L);   // E*L
    int32_t* lows = lowt + E * L;               // E*L
    int32_t* cnt = lows + E * L;                // E
    int32_t* nlow = cnt + E;                    // E
    int32_t* comp = nlow + E;                   // E
    int32_t* lock = comp + E;                   // E
    int32_t* st_issued = lock + E;              // E
    int32_t* st_done = st_issued + E;           // E
    int32_t* rowtag = st_done + E;              // E      (cache on)
    float* rowc = (float*)(rowtag + E);         // E*E    (cache on)
    __shared__ int32_t next;
    __shared__ int32_t stop;
    __shared__ int32_t workers_left;
    __shared__ unsigned long long nbids;

    AucCtl* ctl = w.ctl;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nwaves = blockDim.x >> 6;
    const int nworkers = cache ? nwaves - kHelperWaves : nwaves;
    const bool aborted = ctl->abort;
    const int cur = ctl->cur;
    const int64_t nb = aborted ? 0 : ctl->nbid[cur];
    const bool ident = ctl->identity;
    const int32_t* list = cur ? w.list1 : w.list0;
    for (int64_t e = tid; e < E; e += blockDim.x) {
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
    for (int64_t i = tid; i < E * L; i += blockDim.x) {
        lowb[i] = w.lowb[i];
        lowt[i] = w.lowt[i];
        lows[i] = w.lows[i];
    }
    if (tid == 0) {
        next = 0;
        workers_left = nworkers;
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

    if (wave >= nworkers) {
        // ---- helper: keep each expert's lowest-holder row in the LDS cache
        const int hid = wave - nworkers;
        while (__hip_atomic_load(&workers_left, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) > 0) {
            bool idle = true;
            for (int64_t e = hid; e < E; e += kHelperWaves) {
                const int h = (nlow[e] > 0) ? lowt[e * L] : -1;
                if (h < 0 || rowtag[e] == h) continue;
                idle = false;
                float r[NCH];
                load_row<NCH>(s, h, E, lane, sn, r);
                int ok = 0;
                if (lane == 0 && lds_trylock(&lock[e])) {
                    ok = (nlow[e] > 0 && lowt[e * L] == h) ? 1 : 2;
                    if (ok == 2) lds_unlock(&lock[e]);
                }
                ok = first_lane_i32(ok);
                if (ok == 1) {
#pragma unroll
                    for (int c = 0; c < NCH; ++c)
                        if (lane + 64 * c < E) rowc[e * E + lane + 64 * c] = r[c];
                    if (lane == 0) {
                        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                        rowtag[e] = h;
                        lds_unlock(&lock[e]);
                    }
                }
            }
            if (idle) __builtin_amdgcn_s_sleep(8);
        }
    } else {
        // ---- chain worker
        int pending = -1;  // expert with this wave's slot stores in flight
        for (;;) {
            int j = 0;
            if (lane == 0) j = atomicAdd(&next, 1);
            j = first_lane_i32(j);
            if (j >= nb) break;
            int64_t t = ident ? j : list[j];
            float v[NCH];
            load_row<NCH>(s, t, E, lane, sn, v);
            while (t >= 0) {
                if (__hip_atomic_load(&stop, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) break;
                // slot stores of the previous step have landed once this wait returns
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                if (pending >= 0) {
                    if (lane == 0)
                        __hip_atomic_fetch_add(&st_done[pending], 1, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_WORKGROUP);
                    pending = -1;
                }
                int b1;
                double v1, v2, pib;
                for (;;) {
                    best_two<NCH>(v, pi, E, lane, b1, v1, v2, pib);
                    int ok = 0;
                    if (lane == 0) {
                        lds_lock(&lock[b1]);
                        ok = (pi[b1] == pib);
                        if (!ok) lds_unlock(&lock[b1]);
                    }
                    ok = first_lane_i32(ok);
                    if (ok) break;
                }
                // ---- commit under lock[b1] (held by lane 0)
                const double beta = pib + (v1 - v2) + eps;
                const int64_t eb = (int64_t)b1 * L;
                int32_t* stk = w.stok + (int64_t)b1 * k;
                double* sbd = w.sbid + (int64_t)b1 * k;
                const int c = cnt[b1];
                int n = nlow[b1];
                int cp = comp[b1];
                double lb = DBL_MAX;
                int lt = kNoTok, ls = -1;
                if (lane < n) { lb = lowb[eb + lane]; lt = lowt[eb + lane]; ls = lows[eb + lane]; }
                if (c >= k && n == 0) {
                    // a full expert keeps a non-empty list; rebuild it if not
                    if (lane == 0) {
                        const int want = st_issued[b1];
                        while (__hip_atomic_load(&st_done[b1], __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_WORKGROUP) != want)
                            __builtin_amdgcn_s_sleep(1);
                    }
                    asm volatile("" ::: "memory");
                    wave_rebuild(sbd, stk, k, lane, L, -1, 0.0, 0, lb, lt, ls, n);
                    cp = (n >= k) ? 1 : 0;
                }
                int slot, victim = -1;
                if (c < k || n == 0) {
                    slot = (int)min<int64_t>(c, k - 1);
                } else {
                    // full: the list head (lane 0) is the lowest holder; pop it
                    victim = readlane_i32(lt, 0);
                    slot = readlane_i32(ls, 0);
                    const double nb_ = dpp_f64<kDppShl1>(lb);
                    const int nt = dpp_i32<kDppShl1>(lt);
                    const int ns = dpp_i32<kDppShl1>(ls);
                    if (lane + 1 < n) { lb = nb_; lt = nt; ls = ns; }
                    else { lb = DBL_MAX; lt = kNoTok; ls = -1; }
                    --n;
                }
                if (lane == 0) {
                    stk[slot] = (int32_t)t;
                    sbd[slot] = beta;
                }
                // the new holder enters the list if the list covers it
                const bool before = lane < n && evict_first(lb, lt, beta, (int)t);
                const int pos = __popcll(__ballot(before));
                bool new_head = false;
                if ((n < L && cp) || pos < n) {
                    const double pb_ = dpp_f64<kDppShr1>(lb);
                    const int pt = dpp_i32<kDppShr1>(lt);
                    const int ps = dpp_i32<kDppShr1>(ls);
                    if (lane == pos) { lb = beta; lt = (int)t; ls = slot; }
                    else if (lane > pos) { lb = pb_; lt = pt; ls = ps; }
                    if (n == L) cp = 0;  // the old last entry dropped out
                    else ++n;
                    new_head = (pos == 0);
                } else {
                    cp = 0;
                }
                const bool full = (c + 1 >= k);
                if (full && n == 0) {
                    if (lane == 0) {
                        const int want = st_issued[b1];
                        while (__hip_atomic_load(&st_done[b1], __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_WORKGROUP) != want)
                            __builtin_amdgcn_s_sleep(1);
                    }
                    asm volatile("" ::: "memory");
                    wave_rebuild(sbd, stk, k, lane, L, slot, beta, (int)t, lb, lt, ls, n);
                    cp = (n >= k) ? 1 : 0;
                    new_head = false;
                }
                if (lane < n) { lowb[eb + lane] = lb; lowt[eb + lane] = lt; lows[eb + lane] = ls; }
                // the evicted token's row: from the cache when it holds it
                bool cached = false;
                if (cache && victim >= 0) {
                    cached = (rowtag[b1] == victim);
                    if (cached) {
#pragma unroll
                        for (int cc = 0; cc < NCH; ++cc)
                            v[cc] = (lane + 64 * cc < E) ? rowc[b1 * E + lane + 64 * cc] : 0.0f;
                    }
                }
                if (cache && new_head) {
                    // this token became the lowest holder: cache its row now
                    float mine[NCH];
#pragma unroll
                    for (int cc = 0; cc < NCH; ++cc) mine[cc] = cached ? 0.0f : v[cc];
                    if (!cached) {
#pragma unroll
                        for (int cc = 0; cc < NCH; ++cc)
                            if (lane + 64 * cc < E) rowc[b1 * E + lane + 64 * cc] = mine[cc];
                        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                        if (lane == 0) rowtag[b1] = (int)t;
                    }
                }
                const double head_bid = readlane_f64(lb, 0);
                if (lane == 0) {
                    nlow[b1] = n;
                    comp[b1] = cp;
                    cnt[b1] = (c < k) ? c + 1 : c;
                    if (full) pi[b1] = head_bid;
                    st_issued[b1] += 1;
                    lds_unlock(&lock[b1]);
                    const unsigned long long nbd = atomicAdd(&nbids, 1ull) + 1;
                    if (nbd >= cap) stop = 1;
                }
                pending = b1;
                if (victim >= 0 && !cached) load_row<NCH>(s, victim, E, lane, sn, v);
                t = victim;
            }
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        if (pending >= 0 && lane == 0)
            __hip_atomic_fetch_add(&st_done[pending], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        if (lane == 0) __hip_atomic_fetch_add(&workers_left, -1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    __syncthreads();
    if (tid == 0) {
        const unsigned long long pb = ctl->bids_phase + nbids;
        ctl->bids_total += pb;
        if (phase < 16) {
            st->bids[phase] = (long long)pb;
            st->rounds[phase] = ctl->rounds_phase;
        }
        st->phases = phase + 1;
        if (stop && !aborted) st->status = kErrNotConverged;
    }
    // every expert is full: its price floor becomes its lowest held bid
    for (int64_t e = tid; e < E; e += blockDim.x) {
        w.floor_[e] = (cnt[e] == k) ? pi[e] : flo[e];
        w.cnt[e] = cnt[e];
    }
}
