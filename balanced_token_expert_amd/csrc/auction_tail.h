// End of each eps phase of the auction (included by auction.hip, inside
// namespace base): the tokens the bulk rounds left unassigned are placed by
// shortest augmenting paths on the graph whose nodes are the experts.
//
// Why: near the end of a phase an unassigned token starts a displacement
// chain -- it evicts a holder, who evicts another, ... -- that ends only at
// an expert with a free slot. Each step raises one price by the evicted
// token's margin, often about eps, so a chain that must lift a group of
// experts by some amount takes about (group size) * amount / eps dependent
// steps: hundreds to thousands at these sizes. A chain is an augmenting path
// of the transportation problem behind eq. 2 ("BASE Layers" sec. 3.2.1); the
// cheapest one, and a price change that keeps every holder
// eps-complementary-slack after it, come from a shortest-path computation
// over the E experts (the successive-shortest-path step of min-cost flow,
// with the auction's prices as node potentials).
//
// Graph. For holders t of expert a, moving t to b costs, in reduced terms,
//   r_t(a,b) = (s[t][a] - p_a) - (s[t][b] - p_b) >= -eps   (eps-CS),
// so arc a->b gets length w(a,b) = C[a][b] - p_a + p_b + eps >= 0 with
// C[a][b] = min over holders t of a of s[t][a] - s[t][b] (and Ct[a][b] that
// holder). D(a) is the length of a shortest path from a to an expert with a
// free slot (0 at those), computed for all experts at once by Bellman-Ford
// rounds over a frontier (the experts whose distance just changed); nx(a) is
// the next expert on it. An unassigned token u
// enters expert e at cost entry(u,e) = max_e' (s[u][e'] - p_e') -
// (s[u][e] - p_e) >= 0; its best augmentation enters at the e1 minimising
// L_u = entry(u,e1) + D(e1) and follows nx to a free slot.
//
// Prices. With L the largest L_u among the paths a batch applies, every
// price drops by max(0, L - D(e)). Each holder's reduced costs stay >= -eps
// (D(a) <= w(a,b) + D(b) for every arc), each applied path's arcs become
// tight -- a moved token is eps-CS at its new expert -- and each entering
// token is exactly CS at e1 (L_u <= entry(u,e) + D(e) for every e). So all
// paths of a batch are valid under one price change, provided they move
// distinct tokens and their free slots suffice: paths through a full expert
// a use its one "out" holder Ct[a][nx(a)], so the applied paths are those,
// in order of L_u, whose full experts no earlier applied path used and whose
// free expert still has a slot. The others wait for the next batch.
//
// Slots. Counts only grow in the tail (a path's inner experts lose one
// holder and gain one), so an expert's free slots are always cnt .. k-1 and
// a moved token takes the slot of the token it displaces.
//
// C is maintained lazily. After each batch, one wave per expert the applied
// paths touched (no two waves share an expert, so no locks) lets every token
// that joined lower the columns it beats; a column whose cheapest holder
// left is only marked stale. A stale C[a][b] can only be too small (the
// minimum over fewer holders), so the distances computed with it still obey
// D(a) <= w(a,b) + D(b) for the true lengths, which is all the price change
// needs; what an applied path needs is exact arcs. So the Bellman-Ford
// rounds never let a row take a stale arc: it is recomputed over its
// expert's holders first, and the row looks again. When the rounds end, every
// arc of the tree a -> nx(a) is exact, and then so is D. C and the stale bits
// live in LDS for E <= 128 (128 KB of fp64), in global memory otherwise.
// Every loop of the kernel is bounded: a batch places at least one token (its
// first path in order of L_u is always applied), and a batch count beyond
// that bound stops the phase with an error status instead of looping.

constexpr int kSspWaves = 16;
constexpr int kJq = 2;  // joiner rows a C update loads at once
constexpr int kSspThreads = 64 * kSspWaves;
constexpr int kSspCand = 64;  // unassigned tokens a batch considers (one per lane of wave 0)

__host__ __device__ static inline bool ssp_c_in_lds(int64_t E) { return E <= 128; }
// row stride of C in LDS: 8 doubles of padding move consecutive rows to
// different LDS banks
__host__ __device__ static inline int64_t ssp_c_stride(int64_t E) { return ssp_c_in_lds(E) ? E + 8 : E; }

static size_t ssp_lds_bytes(int64_t E) {
    const size_t nw = (size_t)((E + 63) / 64);
    size_t b = 0;
    if (ssp_c_in_lds(E)) b += 8 * (size_t)E * ((size_t)ssp_c_stride(E) + nw);  // C, stale bits
    b += 8 * 5 * (size_t)E;               // prices, distances, frontier values (three lists)
    b += 4 * 11 * (size_t)E;              // counts, next, frontier experts (three lists), full
                                          // experts, out token, list head, touched, stale arcs (two)
    b += 4 * 3 * (size_t)(E + kSspCand);  // item joiner / leaver / next
    return b;
}

// Loads of data other waves of this workgroup wrote during the kernel (after
// their memory wait and a barrier): device scope, so the
// load is served by L2, never by a stale line of the CU's L1.
BASE_DEV int ld_fresh_i32(const int32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
BASE_DEV double ld_fresh_f64(const double* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
BASE_DEV unsigned long long ld_fresh_u64(const unsigned long long* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A frontier expert's D + p + eps, rounded up by 2^-50 times the magnitudes
// summed. An arc's length then adds C (rounded up the same way) and -p_a
// (likewise); the margins exceed the rounding error of every sum, so each
// computed path length is at least its exact value, rounding makes no cycle
// negative and the rounds end. The eps-CS the tail keeps is eps plus that
// margin (about 1e-15 relative), far below any eps in use.
BASE_DEV double frontier_value(double d, double pe, double eps) {
    return (d + pe + eps) + 0x1p-50 * (fabs(d) + fabs(pe) + eps);
}

// Wave-wide (value, index) minimum, lowest index among equal values; the
// result is uniform.
BASE_DEV void argmin_merge(double& v, int& i, double ov, int oi) {
    if (ov < v || (ov == v && oi < i)) { v = ov; i = oi; }
}
BASE_DEV void wave_argmin_f64(double& v, int& i) {
    argmin_merge(v, i, dpp_f64<kDppXor1>(v), dpp_i32<kDppXor1>(i));
    argmin_merge(v, i, dpp_f64<kDppXor2>(v), dpp_i32<kDppXor2>(i));
    argmin_merge(v, i, dpp_f64<kDppHalfMirror>(v), dpp_i32<kDppHalfMirror>(i));
    argmin_merge(v, i, dpp_f64<kDppMirror>(v), dpp_i32<kDppMirror>(i));
    double bv = readlane_f64(v, 0);
    int bi = readlane_i32(i, 0);
    argmin_merge(bv, bi, readlane_f64(v, 16), readlane_i32(i, 16));
    argmin_merge(bv, bi, readlane_f64(v, 32), readlane_i32(i, 32));
    argmin_merge(bv, bi, readlane_f64(v, 48), readlane_i32(i, 48));
    v = bv;
    i = bi;
}

BASE_DEV float sani(float x, Sani sn) { return (sn.fix && !is_finite_f32(x)) ? sn.repl : x; }

// C and Ct of every expert from its holders after the bulk rounds, and the
// slot of every holder. One block per expert: the holders' ids are staged in
// LDS (up to kSetupChunk at a time), then each wave takes groups of holders
// whose rows it loads together (32 / NCH rows in flight), lanes over the
// columns; the waves' minima meet in LDS. 16 waves when E <= 256 (their
// minima fit in LDS), else 4.
constexpr int kSetupChunk = 4096;
__host__ __device__ static inline int ssp_setup_threads(int64_t E) { return E <= 256 ? 1024 : 256; }

template <int NCH>
__global__ __launch_bounds__(1024) void auc_ssp_setup_kernel(const float* s, int64_t E, int64_t k,
                                                             AucWs w, const ScoreScan* scan) {
    extern __shared__ __attribute__((aligned(16))) char sm[];
    const int nwv = blockDim.x >> 6;
    double* pv = (double*)sm;                   // waves x E
    int32_t* pt = (int32_t*)(pv + nwv * E);     // waves x E
    int32_t* hl = pt + nwv * E;                 // kSetupChunk holder ids
    float* tl = (float*)(hl + kSetupChunk);     // E <= 128: 8 x E scores per wave (xt staging)
    const bool xtl = ssp_c_in_lds(E);  // the phase end keeps xt exactly when C is in LDS
    const AucCtl* ctl = w.ctl;
    if (ctl->abort || ctl->nbid[ctl->cur] == 0) return;
    const int parts = (int)ssp_parts(E);
    const int a = blockIdx.x / parts, part = blockIdx.x % parts;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const Sani sn = read_sani(scan);
    const int n = w.cnt[a];
    // this workgroup's share of a's holders: slots [p0, p1)
    const int share = (n + parts - 1) / parts;
    const int p0 = min(n, part * share), p1 = min(n, p0 + share);
    constexpr int U = NCH >= 16 ? 2 : 32 / NCH;
    double bv[NCH];
    int bt[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) { bv[c] = DBL_MAX; bt[c] = kNoTok; }
    for (int c0 = p0; c0 < p1; c0 += kSetupChunk) {
        const int cn = min(kSetupChunk, p1 - c0);
        for (int i = threadIdx.x; i < cn; i += blockDim.x) {
            const int h = w.stok[(int64_t)a * k + c0 + i];
            hl[i] = h;
            w.slot_of[h] = c0 + i;
        }
        __syncthreads();
        for (int i0 = wave * U; i0 < cn; i0 += nwv * U) {
            int h[U];
            float v[U][NCH];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                h[u] = i0 + u < cn ? hl[i0 + u] : -1;
                if (h[u] >= 0) load_row<NCH>(s, h[u], E, lane, sn, v[u]);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (h[u] < 0) continue;
                float ra = 0.0f;
#pragma unroll
                for (int c = 0; c < NCH; ++c)
                    if (c == (a >> 6)) ra = v[u][c];
                const float sa32 = __builtin_bit_cast(float, readlane_i32(__builtin_bit_cast(int, ra), a & 63));
                if (!xtl && lane == 0) w.sown[(int64_t)a * k + c0 + i0 + u] = sa32;
                const double sa = (double)sa32;
#pragma unroll
                for (int c = 0; c < NCH; ++c) {
                    const int e = lane + 64 * c;
                    if (e < E) argmin_merge(bv[c], bt[c], sa - (double)v[u][c], h[u]);
                }
            }
            // the group's rows into xt, expert-major: eight rows at a time
            // through the wave's LDS tile, so that each store writes 32-byte
            // runs of consecutive slots (8 columns x 8 slots per instruction)
            if (xtl) {
                float* tw = tl + (int64_t)wave * 8 * E;
#pragma unroll
                for (int h0 = 0; h0 < U; h0 += 8) {
#pragma unroll
                    for (int uu = 0; uu < 8; ++uu) {
                        if (h0 + uu >= U || h[h0 + uu] < 0) continue;
#pragma unroll
                        for (int c = 0; c < NCH; ++c) {
                            const int e = lane + 64 * c;
                            if (e < E) tw[uu * E + e] = v[h0 + uu][c];
                        }
                    }
                    __builtin_amdgcn_s_waitcnt(0);
                    __builtin_amdgcn_wave_barrier();
                    const int j = lane & 7, eo = lane >> 3;
                    const int iu = i0 + h0 + j;
                    if (h0 + j < U && iu < cn)
                        for (int e = eo; e < E; e += 8)
                            w.xt[((int64_t)a * E + e) * k + c0 + iu] = tw[j * E + e];
                    __builtin_amdgcn_s_waitcnt(0);
                    __builtin_amdgcn_wave_barrier();
                }
            }
        }
        __syncthreads();
    }
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int e = lane + 64 * c;
        if (e < E) { pv[wave * E + e] = bv[c]; pt[wave * E + e] = bt[c]; }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        double v = pv[e];
        int t = pt[e];
        for (int q = 1; q < nwv; ++q) argmin_merge(v, t, pv[q * E + e], pt[q * E + e]);
        w.C[(int64_t)part * E * E + (int64_t)a * E + e] = v;
        w.Ct[(int64_t)part * E * E + (int64_t)a * E + e] = t;
    }
}

template <int NCH, bool CL>
__global__ __launch_bounds__(kSspThreads) void auc_ssp_kernel(const float* s, int64_t T, int64_t E,
                                                              int64_t k, AucWs w,
                                                              const ScoreScan* scan, double eps,
                                                              int phase, int64_t max_bids,
                                                              AucStatsDev* st) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int64_t cs = ssp_c_stride(E);
    const int nw = (int)((E + 63) / 64);
    char* sp = smem;
    double* Cl = (double*)sp;                                    // E x cs (CL)
    if (CL) sp += 8 * E * cs;
    unsigned long long* stl = (unsigned long long*)sp;           // E x nw stale bits (CL)
    if (CL) sp += 8 * E * nw;
    double* p = (double*)sp;                                     // E   prices
    double* D = p + E;                                           // E   distance to a free slot
    double* fq = D + E;                                          // 3E  frontier: D + p + eps
    int32_t* cnt = (int32_t*)(fq + 3 * E);                       // E   holders
    int32_t* nx = cnt + E;                                       // E   next expert
    int32_t* fl = nx + E;                                        // 3E  frontier experts
    int32_t* rows = fl + 3 * E;                                  // E   full experts
    int32_t* otok = rows + E;                                    // E   out holder Ct[a][nx(a)]
    int32_t* head = otok + E;                                    // E   item list per expert
    int32_t* ux = head + E;                                      // E   touched experts
    int32_t* sarc = ux + E;                                      // 2E  stale best arcs (two lists)
    int32_t* ij = sarc + 2 * E;                                      // E + kSspCand  item joiner
    int32_t* il = ij + (E + kSspCand);                           //               item leaver
    int32_t* inext = il + (E + kSspCand);                        //               item next
    __shared__ int32_t cand[kSspCand], ce1[kSspCand], cf[kSspCand], clen[kSspCand],
        alist[kSspCand], ring[kSspCand];
    __shared__ double cL[kSspCand];
    __shared__ unsigned long long cmk[kSspCand * NCH], cfl[kSspCand], csf[kSspCand];
    __shared__ int32_t crk[kSspCand];
    __shared__ int32_t nring, nc_s, nacc_s, nux, nitem, stop, nrows, nsarc[2], fn[3];
    __shared__ double Lmax_s;
    __shared__ int64_t ghead;
    __shared__ long long placed, batches;

    AucCtl* ctl = w.ctl;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = first_lane_i32(tid >> 6);
    const bool aborted = ctl->abort;
    const int cur = ctl->cur;
    const int64_t nb = aborted ? 0 : ctl->nbid[cur];
    const bool ident = ctl->identity;
    const int32_t* list = cur ? w.list1 : w.list0;
    const Sani sn = read_sani(scan);
    double* Cg = w.C;
    int32_t* Ct = w.Ct;
    unsigned long long* stg = w.stale;
    auto cget = [&](int a, int e) -> double {
        if constexpr (CL) return Cl[a * cs + e];
        else return ld_fresh_f64(Cg + (int64_t)a * E + e);
    };
    auto cset = [&](int a, int e, double v) {
        if constexpr (CL) Cl[a * cs + e] = v;
        else __hip_atomic_store(Cg + (int64_t)a * E + e, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    auto sget = [&](int a, int c) -> unsigned long long {
        if constexpr (CL) return stl[a * nw + c];
        else return ld_fresh_u64(stg + (int64_t)a * nw + c);
    };
    auto sput = [&](int a, int c, unsigned long long v) {
        if constexpr (CL) stl[a * nw + c] = v;
        else __hip_atomic_store(stg + (int64_t)a * nw + c, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    auto stale = [&](int a, int b) -> bool { return (sget(a, b >> 6) >> (b & 63)) & 1ull; };
    // C[a][b] and Ct[a][b] over a's current holders, and the column's stale
    // bit cleared (one wave; every holder's two scores loaded at once, up to
    // 512 holders per pass)
    auto recompute_col = [&](int a, int b) {
        const int ha = first_lane_i32(cnt[a]);
        double bv = DBL_MAX;
        int bt = kNoTok;
        for (int j0 = 0; j0 < ha; j0 += 8 * 64) {
            int hh[8];
#pragma unroll
            for (int v = 0; v < 8; ++v) {
                const int j = j0 + v * 64 + lane;
                hh[v] = (j < ha) ? ld_fresh_i32(w.stok + (int64_t)a * k + j) : -1;
            }
            // E <= 128: both scores come from the expert-major copy xt,
            // read contiguously with the holder ids; else a holder's score at
            // a is kept beside its slot (sown) and only the one at b is a
            // scattered load
            float sa[8], sb[8];
            if constexpr (CL) {
                const int32_t* xa = (const int32_t*)w.xt + ((int64_t)a * E + a) * k;
                const int32_t* xb = (const int32_t*)w.xt + ((int64_t)a * E + b) * k;
#pragma unroll
                for (int v = 0; v < 8; ++v) {
                    const int j = j0 + v * 64 + lane;
                    sa[v] = (j < ha) ? __int_as_float(ld_fresh_i32(xa + j)) : 0.0f;
                    sb[v] = (j < ha) ? __int_as_float(ld_fresh_i32(xb + j)) : 0.0f;
                }
            } else {
#pragma unroll
                for (int v = 0; v < 8; ++v) {
                    const int j = j0 + v * 64 + lane;
                    sa[v] = (j < ha) ? __int_as_float(ld_fresh_i32((const int32_t*)w.sown + (int64_t)a * k + j)) : 0.0f;
                }
#pragma unroll
                for (int v = 0; v < 8; ++v) {
                    const float* row = s + (int64_t)(hh[v] < 0 ? 0 : hh[v]) * E;
                    sb[v] = hh[v] >= 0 ? sani(row[b], sn) : 0.0f;
                }
            }
#pragma unroll
            for (int v = 0; v < 8; ++v)
                if (hh[v] >= 0) argmin_merge(bv, bt, (double)sa[v] - (double)sb[v], hh[v]);
        }
        wave_argmin_f64(bv, bt);
        if (lane == 0) {
            cset(a, b, bv);
            __hip_atomic_store(Ct + (int64_t)a * E + b, bt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            sput(a, b >> 6, sget(a, b >> 6) & ~(1ull << (b & 63)));
        }
    };

    for (int64_t e = tid; e < E; e += kSspThreads) {
        p[e] = w.pi[e];
        cnt[e] = w.cnt[e];
        head[e] = -1;
    }
    if (nb > 0) {
        if (CL) {
            // the setup's planes merged (one per workgroup of an expert)
            const int parts = (int)ssp_parts(E);
            for (int64_t i = tid; i < E * E; i += kSspThreads) {
                double v = Cg[i];
                int t = Ct[i];
                for (int q = 1; q < parts; ++q) argmin_merge(v, t, Cg[q * E * E + i], Ct[q * E * E + i]);
                Cl[(i / E) * cs + i % E] = v;
                if (parts > 1) Ct[i] = t;
            }
            __builtin_amdgcn_s_waitcnt(0);  // the merged Ct in L2 before the barrier below
        }
        for (int i = tid; i < (int)E * nw; i += kSspThreads) sput(i / nw, i % nw, 0ull);
    }
    const unsigned long long used0 = ctl->bids_total + ctl->bids_phase;
    const long long cap_left =
        max_bids > 0 ? (long long)max_bids - (long long)min<unsigned long long>(used0, (unsigned long long)max_bids)
                     : LLONG_MAX;
    if (tid == 0) {
        nring = 0;
        ghead = 0;
        placed = 0;
        batches = 0;
        stop = (nb > 0 && cap_left <= 0) ? 1 : 0;
    }
    __syncthreads();

    for (;;) {
        // ---- this batch's tokens: those not placed last batch, then the list
        if (tid == 0) {
            int n = 0;
            for (int r = 0; r < nring; ++r) cand[n++] = ring[r];
            nring = 0;
            while (n < kSspCand && ghead < nb) {
                cand[n++] = ident ? (int32_t)ghead : list[ghead];
                ++ghead;
            }
            nc_s = stop ? 0 : n;
            nacc_s = 0;
            nux = 0;
            nitem = 0;
        }
        __syncthreads();
        const int nc = first_lane_i32(nc_s);
        if (nc == 0) break;

        // ---- D and nx: shortest paths to a free slot, with every arc of the
        // tree they form exact
        for (int64_t e = tid; e < E; e += kSspThreads) {
            D[e] = cnt[e] < k ? 0.0 : DBL_MAX;
            nx[e] = -1;
        }
        if (tid == 0) {
            fn[0] = 0;
            fn[1] = 0;
            fn[2] = 0;
            nrows = 0;
            nsarc[0] = 0;
            nsarc[1] = 0;
        }
        __syncthreads();
        for (int64_t e = tid; e < E; e += kSspThreads) {
            if (cnt[e] < k) {
                const int j = atomicAdd(&fn[0], 1);
                fl[j] = (int)e;
                fq[j] = frontier_value(0.0, p[e], eps);
            } else {
                rows[atomicAdd(&nrows, 1)] = (int)e;
            }
        }
        __syncthreads();
        const int nr = first_lane_i32(nrows);
        // Bellman-Ford rounds. Round r relaxes the full experts' arcs into the
        // experts listed in frontier list r % 3 (those whose distance changed
        // in round r - 1; the free experts first) and lists the experts it
        // improves in list (r + 1) % 3; list (r + 2) % 3, read in round r - 1,
        // is emptied for round r + 1. The distance of a full expert is written
        // only by the lanes that own its row, and read by others only through
        // the lists. A row whose best arc is stale does not move: the arc goes
        // on a repair list, all waves recompute the listed arcs over their
        // expert's holders, and those rows look at the same frontier again
        // (a repair only raises C, so the arcs a row passed over stay no
        // better than its distance). Each repair clears a stale bit, so this
        // ends; then every tree arc is exact and so is D.
        //
        // Evaluation of a list of rows against the frontier. Lanes per row: a
        // power of two that covers the frontier, at most 16 and at most what
        // lets all rows run at once.
        auto relax = [&](const int32_t* rl, int n, bool coded, const int32_t* fle, const double* fqe,
                         int nf, int ln, int tl) {
            int sh = 0;
            while (sh < 4 && (1 << sh) < nf && (n << (sh + 1)) <= kSspThreads) ++sh;
            const int G = 1 << sh, gpw = 64 >> sh;
            const int l = lane & (G - 1);
            for (int r0 = wave * gpw; r0 < n; r0 += kSspWaves * gpw) {
                const int r = r0 + (lane >> sh);
                const bool ok = r < n;
                const int a = ok ? (coded ? rl[r] / (int)E : rl[r]) : 0;
                double bv = DBL_MAX;
                int bn = 0x7fffffff;
                if (ok) {
                    const double pa = p[a];
                    const double ra = fma(fabs(pa), 0x1p-50, -pa);
#pragma unroll 2
                    for (int j = l; j < nf; j += G) {
                        const int b = fle[j];
                        const double c = cget(a, b);
                        const double v = (fma(fabs(c), 0x1p-50, c) + fqe[j]) + ra;
                        const bool take = (v < bv) | ((v == bv) & (b < bn));
                        bv = take ? v : bv;
                        bn = take ? b : bn;
                    }
                }
                // the row's minimum, then the lowest expert that reaches it
                double m = bv;
                if (sh >= 1) m = fmin(m, dpp_f64<kDppXor1>(m));
                if (sh >= 2) m = fmin(m, dpp_f64<kDppXor2>(m));
                if (sh >= 3) m = fmin(m, dpp_f64<kDppHalfMirror>(m));
                if (sh >= 4) m = fmin(m, dpp_f64<kDppMirror>(m));
                int ib = bv == m ? bn : 0x7fffffff;
                if (sh >= 1) ib = min(ib, dpp_i32<kDppXor1>(ib));
                if (sh >= 2) ib = min(ib, dpp_i32<kDppXor2>(ib));
                if (sh >= 3) ib = min(ib, dpp_i32<kDppHalfMirror>(ib));
                if (sh >= 4) ib = min(ib, dpp_i32<kDppMirror>(ib));
                if (ok && l == 0 && m < D[a]) {
                    if (stale(a, ib)) {
                        sarc[tl * E + atomicAdd(&nsarc[tl], 1)] = a * (int)E + ib;
                    } else {
                        D[a] = m;
                        nx[a] = ib;
                        const int j = atomicAdd(&fn[ln], 1);
                        fl[ln * E + j] = a;
                        fq[ln * E + j] = frontier_value(m, p[a], eps);
                    }
                }
            }
        };
        bool conv = false;
        int par = 0;  // repair list the current evaluation fills
        for (int it = 0; it <= E + 1; ++it) {
            const int li = it % 3, ln = (it + 1) % 3;
            const int nf = first_lane_i32(fn[li]);
            if (nf == 0) { conv = true; break; }
            if (tid == 0) fn[(it + 2) % 3] = 0;
            const int32_t* fle = fl + li * E;
            const double* fqe = fq + li * E;
            relax(rows, nr, false, fle, fqe, nf, ln, par);
            __syncthreads();
            for (int rep = 0;; ++rep) {
                const int ns = first_lane_i32(nsarc[par]);
                if (ns == 0) break;
                if (rep > E * nw * 64) { it = (int)E + 2; break; }
                if (tid == 0) nsarc[par ^ 1] = 0;
                const int32_t* sl = sarc + par * E;
                for (int i = wave; i < ns; i += kSspWaves) {
                    const int code = first_lane_i32(sl[i]);
                    const int a = code / (int)E;
                    recompute_col(a, code - a * (int)E);
                }
                __syncthreads();
                relax(sl, ns, true, fle, fqe, nf, ln, par ^ 1);
                __syncthreads();
                par ^= 1;
            }
        }
        if (!conv) {
            // rounding made a cycle negative: stop with an error status
            if (tid == 0) stop = 1;
            __syncthreads();
            continue;
        }
        // each full expert's out holder (the token its shortest path moves)
        for (int64_t a = tid; a < E; a += kSspThreads)
            otok[a] = (cnt[a] >= k && nx[a] >= 0) ? ld_fresh_i32(Ct + a * E + nx[a]) : -1;

        // ---- each token's best entry: L_u = min_e entry(u,e) + D(e)
        for (int q = wave; q < nc; q += kSspWaves) {
            const int u = first_lane_i32(cand[q]);
            float v[NCH];
            load_row<NCH>(s, u, E, lane, sn, v);
            double val[NCH], best = -DBL_MAX;
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                const int e = lane + 64 * c;
                val[c] = e < E ? (double)v[c] - p[e] : -DBL_MAX;
                best = fmax(best, val[c]);
            }
            const double pu = wave_max_f64(best);
            double bv = DBL_MAX;
            int be = 0x7fffffff;
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                const int e = lane + 64 * c;
                if (e < E && D[e] < DBL_MAX) {
                    const double cst = (pu - val[c]) + D[e];
                    if (cst < bv) { bv = cst; be = e; }
                }
            }
            wave_argmin_f64(bv, be);
            if (lane == 0) {
                cL[q] = bv;
                ce1[q] = be == 0x7fffffff ? -1 : be;
            }
        }
        __syncthreads();

        // ---- apply, in order of L_u, the paths whose full experts no
        // earlier applied path uses and whose free expert has a slot left.
        // Wave 0 walks each candidate's path; then all waves compare every
        // candidate with a share of the others (rank by L, path overlap,
        // same free expert) into per-candidate bitmasks; then wave 0 takes
        // the candidates in rank order, each a few reads of those masks.
        if (wave == 0) {
            const bool mine = lane < nc;
            unsigned long long msk[NCH];
#pragma unroll
            for (int c = 0; c < NCH; ++c) msk[c] = 0;
            int f = -1, steps = 0;
            if (mine && ce1[lane] >= 0) {
                int a = ce1[lane];
                while (a >= 0 && cnt[a] >= k && steps < E) {
#pragma unroll
                    for (int c = 0; c < NCH; ++c)
                        if (c == (a >> 6)) msk[c] |= 1ull << (a & 63);
                    a = nx[a];
                    ++steps;
                }
                f = (a >= 0 && cnt[a] < k) ? a : -1;
            }
            if (mine) {
                cf[lane] = f;
                clen[lane] = steps;
#pragma unroll
                for (int c = 0; c < NCH; ++c) cmk[lane * NCH + c] = msk[c];
                crk[lane] = 0;
                cfl[lane] = 0;
                csf[lane] = 0;
            }
        }
        __syncthreads();
        {
            const bool mine = lane < nc;
            const double li = mine ? cL[lane] : 0.0;
            const int fi = mine ? cf[lane] : -1;
            unsigned long long mi[NCH];
#pragma unroll
            for (int c = 0; c < NCH; ++c) mi[c] = mine ? cmk[lane * NCH + c] : 0ull;
            unsigned long long conf = 0, same = 0;
            int before = 0;
            for (int j = wave; j < nc; j += kSspWaves) {
                const double lj = cL[j];
                const int fj = cf[j];
                bool cj = false;
#pragma unroll
                for (int c = 0; c < NCH; ++c) cj = cj || (cmk[j * NCH + c] & mi[c]) != 0;
                before += (lj < li || (lj == li && j < lane)) ? 1 : 0;
                if (cj) conf |= 1ull << j;
                if (fj >= 0 && fj == fi) same |= 1ull << j;
            }
            if (mine) {
                if (before) atomicAdd(&crk[lane], before);
                if (conf) atomicOr(&cfl[lane], conf);
                if (same) atomicOr(&csf[lane], same);
            }
        }
        __syncthreads();
        if (wave == 0) {
            const bool mine = lane < nc;
            const int rank = mine ? crk[lane] : lane;
            // lane r receives the lane ranked r (a cross-lane push; lanes past
            // nc push to themselves and are never read)
            const int order_r = __builtin_amdgcn_ds_permute(rank * 4, lane);
            const int fi = mine ? cf[lane] : -1;
            const int capi = fi >= 0 ? (int)(k - cnt[fi]) : 0;
            const unsigned long long conf = mine ? cfl[lane] : 0ull, same = mine ? csf[lane] : 0ull;
            const double lq = mine ? cL[lane] : 0.0;
            const unsigned long long lqb = __builtin_bit_cast(unsigned long long, lq);
            // every candidate's fields pulled into the lane of its rank
            const int capr = __builtin_amdgcn_ds_bpermute(order_r * 4, capi);
            const unsigned cfl_lo = (unsigned)__builtin_amdgcn_ds_bpermute(order_r * 4, (int)(unsigned)conf);
            const unsigned cfl_hi = (unsigned)__builtin_amdgcn_ds_bpermute(order_r * 4, (int)(unsigned)(conf >> 32));
            const unsigned csf_lo = (unsigned)__builtin_amdgcn_ds_bpermute(order_r * 4, (int)(unsigned)same);
            const unsigned csf_hi = (unsigned)__builtin_amdgcn_ds_bpermute(order_r * 4, (int)(unsigned)(same >> 32));
            const unsigned lql = (unsigned)__builtin_amdgcn_ds_bpermute(order_r * 4, (int)(unsigned)lqb);
            const unsigned lqh = (unsigned)__builtin_amdgcn_ds_bpermute(order_r * 4, (int)(unsigned)(lqb >> 32));
            const double lqr = __builtin_bit_cast(double, ((unsigned long long)lqh << 32) | lql);
            int nacc = 0;
            double Lmax = 0.0;
            unsigned long long accm = 0;  // the paths applied, by candidate
            for (int r = 0; r < nc; ++r) {
                const int cap = readlane_i32(capr, r);
                if (cap <= 0) continue;  // no free expert, or one with no slot
                const unsigned long long cr = ((unsigned long long)(unsigned)readlane_i32((int)cfl_hi, r) << 32) |
                                              (unsigned)readlane_i32((int)cfl_lo, r);
                const unsigned long long sr = ((unsigned long long)(unsigned)readlane_i32((int)csf_hi, r) << 32) |
                                              (unsigned)readlane_i32((int)csf_lo, r);
                // a path overlapping an applied one, or a free expert whose
                // slots the applied paths took
                if ((cr & accm) != 0 || __popcll(sr & accm) >= cap) continue;
                const int q = readlane_i32(order_r, r);
                if (lane == 0) alist[nacc] = q;
                accm |= 1ull << q;
                ++nacc;
                Lmax = fmax(Lmax, readlane_f64(lqr, r));
            }
            if (lane == 0) {
                nacc_s = nacc;
                Lmax_s = Lmax;
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            // tokens not placed search again next batch (in candidate order)
            const bool placedq = (accm >> lane) & 1ull;
            const unsigned long long rej = __ballot(mine && !placedq);
            if (mine && !placedq) {
                const unsigned long long below = lane ? (~0ull >> (64 - lane)) : 0ull;
                ring[__popcll(rej & below)] = cand[lane];
            }
            if (lane == 0) nring = __popcll(rej);
        }
        __syncthreads();

        // ---- prices drop by max(0, L - D(e))
        {
            const double Lmax = Lmax_s;
            for (int64_t e = tid; e < E; e += kSspThreads)
                if (D[e] < Lmax) p[e] = p[e] - (Lmax - D[e]);
        }
        // ---- move the tokens of the applied paths; one item per expert on a
        // path. Lane i takes node i of the path (nodes 0 .. m; node m is the
        // free expert), found by following nx from e1.
        const int nacc = first_lane_i32(nacc_s);
        for (int j = wave; j < nacc; j += kSspWaves) {
            const int q = first_lane_i32(alist[j]);
            const int u = first_lane_i32(cand[q]);
            const int m = first_lane_i32(clen[q]);
            const int e1 = first_lane_i32(ce1[q]);
            for (int i0 = 0; i0 <= m; i0 += 64) {
                const int i = i0 + lane;
                int x = e1, prv = -1;
                if (i <= m)
                    for (int h = 0; h < i; ++h) {
                        prv = x;
                        x = nx[x];
                    }
                int jn = 0, lv = -1, slot = 0;
                float sj = 0.0f;  // the joiner's score at x, kept beside its slot
                if (i <= m) {
                    jn = i == 0 ? u : otok[prv];
                    lv = i < m ? otok[x] : -1;
                    if (i < m) slot = ld_fresh_i32(w.slot_of + lv);
                    if (!CL) sj = s[(int64_t)jn * E + x];
                }
                asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
                if (i == m) slot = atomicAdd(&cnt[x], 1);
                if (i <= m) {
                    w.stok[(int64_t)x * k + slot] = jn;
                    if (!CL) w.sown[(int64_t)x * k + slot] = sani(sj, sn);
                    w.slot_of[jn] = slot;
                    const int id = atomicAdd(&nitem, 1);
                    ij[id] = jn;
                    il[id] = lv;
                    const int prev = __hip_atomic_exchange(&head[x], id, __ATOMIC_RELAXED,
                                                           __HIP_MEMORY_SCOPE_WORKGROUP);
                    inext[id] = prev;
                    if (prev < 0) ux[atomicAdd(&nux, 1)] = x;
                }
            }
            asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        }
        __syncthreads();

        // ---- C and Ct after the moves: one wave per touched expert. The
        // tokens that joined lower the columns they beat (those become
        // exact); every other column whose cheapest holder left is marked
        // stale and keeps its old value, which can only underestimate it.
        const int nx_ = first_lane_i32(nux);
        // A wave with several touched experts defers each one's arc
        // recompute (E <= 128, at most 512 holders: one pass of loads) to
        // after the next expert's joiner and leaver work, so the recompute's
        // loads are in flight while that work runs. The deferred arc is in
        // a row no other part of this loop touches.
        int pa = -1, pb = 0;
        int phh[8];
        float psa[8], psb[8];
        auto finish_pending = [&]() {
            double bv = DBL_MAX;
            int bt = kNoTok;
#pragma unroll
            for (int v = 0; v < 8; ++v)
                if (phh[v] >= 0) argmin_merge(bv, bt, (double)psa[v] - (double)psb[v], phh[v]);
            wave_argmin_f64(bv, bt);
            if (lane == 0) {
                cset(pa, pb, bv);
                __hip_atomic_store(Ct + (int64_t)pa * E + pb, bt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                sput(pa, pb >> 6, sget(pa, pb >> 6) & ~(1ull << (pb & 63)));
            }
            pa = -1;
        };
        for (int uu = wave; uu < nx_; uu += kSspWaves) {
            const int x = first_lane_i32(ux[uu]);
            // this expert's items: lane j holds item j's joiner and leaver
            int myj = -1, myl = -1, nit = 0;
            for (int id = first_lane_i32(head[x]); id >= 0 && nit < 64;
                 id = first_lane_i32(inext[id]), ++nit) {
                const int jn = first_lane_i32(ij[id]);
                const int lv = first_lane_i32(il[id]);
                if (lane == nit) { myj = jn; myl = lv; }
            }
            int ct[NCH];
            double cv[NCH];
            bool upd[NCH];
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                const int e = lane + 64 * c;
                ct[c] = e < E ? ld_fresh_i32(Ct + (int64_t)x * E + e) : -1;
                cv[c] = e < E ? cget(x, e) : 0.0;
                upd[c] = false;
            }
            // joiners (their rows four at a time; with E <= 128 each row also
            // goes into xt at the joiner's slot)
            for (int j0 = 0; j0 < nit; j0 += kJq) {
                float r[kJq][NCH];
                int jt[kJq], js[kJq];
#pragma unroll
                for (int q = 0; q < kJq; ++q) {
                    jt[q] = (j0 + q < nit) ? readlane_i32(myj, (j0 + q) & 63) : -1;
                    js[q] = 0;
                    if (jt[q] >= 0) {
                        load_row<NCH>(s, jt[q], E, lane, sn, r[q]);
                        if (CL) js[q] = ld_fresh_i32(w.slot_of + jt[q]);
                    }
                }
                if constexpr (CL) {
#pragma unroll
                    for (int q = 0; q < kJq; ++q) {
                        if (jt[q] < 0) continue;
#pragma unroll
                        for (int c = 0; c < NCH; ++c) {
                            const int e = lane + 64 * c;
                            if (e < E) w.xt[((int64_t)x * E + e) * k + js[q]] = r[q][c];
                        }
                    }
                }
#pragma unroll
                for (int q = 0; q < kJq; ++q) {
                    if (jt[q] < 0) continue;
                    float rx = 0.0f;
#pragma unroll
                    for (int c = 0; c < NCH; ++c)
                        if (c == (x >> 6)) rx = r[q][c];
                    const double sx = (double)readlane_f64((double)rx, x & 63);
#pragma unroll
                    for (int c = 0; c < NCH; ++c) {
                        const int e = lane + 64 * c;
                        const double v = sx - (double)r[q][c];
                        if (e < E && (v < cv[c] || (v == cv[c] && jt[q] < ct[c]))) {
                            cv[c] = v;
                            ct[c] = jt[q];
                            upd[c] = true;
                            cset(x, e, v);
                            __hip_atomic_store(Ct + (int64_t)x * E + e, jt[q], __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
                        }
                    }
                }
            }
            bool bad[NCH];
#pragma unroll
            for (int c = 0; c < NCH; ++c) bad[c] = false;
            for (int j = 0; j < nit; ++j) {
                const int lv = readlane_i32(myl, j & 63);
                if (lv < 0) continue;
#pragma unroll
                for (int c = 0; c < NCH; ++c) bad[c] = bad[c] || ct[c] == lv;
            }
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                const bool in = lane + 64 * c < E;
                const unsigned long long nb_ = __ballot(bad[c] && in), nu = __ballot(upd[c] && in);
                if (c < nw && lane == 0 && (nb_ | nu)) sput(x, c, (sget(x, c) & ~nu) | nb_);
            }
            // the arc this expert's path left by: its mover was that column's
            // cheapest holder, so the column is usually stale now, and the
            // next batch's tree tends to use it again -- recompute it here,
            // in parallel with the other touched experts, rather than in a
            // repair step of the next batch's rounds
            const int xb = first_lane_i32(nx[x]);
            if (CL) __builtin_amdgcn_s_waitcnt(0);  // this wave's xt stores, before it reads them
            if (pa >= 0) finish_pending();
            if (xb >= 0 && stale(x, xb)) {
                const int hx = first_lane_i32(cnt[x]);
                if (CL && hx <= 8 * 64) {
                    const int32_t* xa = (const int32_t*)w.xt + ((int64_t)x * E + x) * k;
                    const int32_t* xc = (const int32_t*)w.xt + ((int64_t)x * E + xb) * k;
#pragma unroll
                    for (int v = 0; v < 8; ++v) {
                        const int j = v * 64 + lane;
                        phh[v] = (j < hx) ? ld_fresh_i32(w.stok + (int64_t)x * k + j) : -1;
                        psa[v] = (j < hx) ? __int_as_float(ld_fresh_i32(xa + j)) : 0.0f;
                        psb[v] = (j < hx) ? __int_as_float(ld_fresh_i32(xc + j)) : 0.0f;
                    }
                    pa = x;
                    pb = xb;
                } else {
                    recompute_col(x, xb);
                }
            }
            if (lane == 0) head[x] = -1;
        }
        if (pa >= 0) finish_pending();
        __syncthreads();
        if constexpr (kChecks) {
            for (int64_t e = tid; e < E; e += kSspThreads)
                if (cnt[e] > k) report_invariant(st);
        }
        if (tid == 0) {
            placed += nacc;
            ++batches;
            // every batch places a token: more batches than tokens means the
            // state is inconsistent; stop with an error instead of looping
            if (placed >= cap_left || batches > nb + 1) stop = 1;
        }
        __syncthreads();
    }

    if (tid == 0) {
        const unsigned long long pb = ctl->bids_phase + (unsigned long long)placed;
        ctl->bids_total += pb;
        if (phase < 16) {
            st->bids[phase] = (long long)pb;
            st->rounds[phase] = ctl->rounds_phase + batches;
            st->tail[phase] = placed;
        }
        st->phases = phase + 1;
        if (stop && !aborted) st->status = kErrNotConverged;
    }
    // the next phase starts from these prices
    for (int64_t e = tid; e < E; e += kSspThreads) {
        w.floor_[e] = p[e];
        w.cnt[e] = cnt[e];
    }
}
