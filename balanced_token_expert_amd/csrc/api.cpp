// C ABI of libbase_layer.so: argument checks, workspace layout and the launch
// sequence of each entry point (see include/base_layer.h for the contract).
#include "../../include/base_layer.h"

#include <hip/hip_runtime.h>
#include <math.h>

#include <mutex>

#include "internal.h"

using namespace base;

namespace {

constexpr int64_t kMaxT = int64_t(1) << 24;  // int32 token ids and offsets
constexpr int64_t kMaxE = 1024;              // auction keeps E prices per lane group
constexpr int kMaxPhases = 64;
constexpr int kMaxSublayers = 64;
constexpr int64_t kMaxBwdWidth = int64_t(1) << 20;  // D, F of base_layer_backward

size_t al(size_t x) { return (x + 255) & ~size_t(255); }

// Workspace layout shared by base_workspace_bytes and the entry points.
struct Layout {
    size_t scan = 0, stats = 0, prices = 0, scores = 0, perm = 0, offsets = 0, hidden = 0,
           auction = 0, permws = 0, assign = 0, gblk = 0, xbuf = 0, ybuf = 0, xg = 0, dyg = 0,
           zbuf = 0, gubuf = 0, dzbuf = 0, part = 0, dl = 0, xs = 0, dxa = 0, dxo = 0, dyn = 0,
           lnst = 0, total = 0;
};

// (op BASE_OP_LAYER_BWD with nsub >= 1: the backward of layer-norm blocks)
Layout layout(int op, int64_t T, int64_t E, int64_t D, int64_t F, int dt, int nsub = 0) {
    Layout L;
    size_t off = 0;
    auto take = [&](size_t& slot, size_t bytes) {
        slot = off;
        off += al(bytes);
    };
    if (op == BASE_OP_AFFINITY) {
        L.total = 0;
        return L;
    }
    take(L.scan, sizeof(ScoreScan));
    take(L.stats, sizeof(AucStatsDev));
    if (op == BASE_OP_LAYER_BWD) {
        const size_t b = dt == BASE_BF16 ? 2 : 4;
        take(L.perm, (size_t)T * 4);
        take(L.offsets, (size_t)(E + 1) * 4);
        take(L.gblk, (size_t)(E + 1) * 4);
        take(L.permws, perm_ws_bytes(T, E));
        // token rows, grouped (with blocks, the first block input holds them)
        if (nsub == 0) take(L.xg, (size_t)T * D * b);
        take(L.dyg, (size_t)T * D * b);   // upstream gradient rows, grouped
        // with blocks, Z and act(Z) (and below the normalised rows) of every
        // block, kept from the forward recompute for the way back
        const size_t nk = nsub >= 1 ? (size_t)nsub : 1;
        take(L.zbuf, nk * T * F * b);     // pre-activations Z
        take(L.gubuf, nk * T * F * b);    // gate * act(Z), or act(Z) of a block
        take(L.dzbuf, (size_t)T * F * b); // dZ
        take(L.part, (size_t)T * bwd_nparts(F, dt == BASE_BF16) * 4);
        take(L.dl, (size_t)T * 4);        // gate-logit gradients
        if (nsub >= 1) {
            take(L.xs, (size_t)(nsub + 1) * T * D * b);  // each block's input, then x_N
            take(L.dxa, (size_t)T * D * 4);   // upstream gradient of a block, fp32
            take(L.dxo, (size_t)T * D * b);   // the same as an operand
            take(L.dyn, (size_t)T * D * b);   // gradient of a block's normalised rows
            take(L.lnst, (size_t)T * 8);      // per-row mean and rstd
            take(L.ybuf, nk * T * D * b);     // normalised rows of each block
        }
        L.total = off;
        return L;
    }
    if (op == BASE_OP_GREEDY) {
        take(L.perm, (size_t)T * 4);
        take(L.offsets, (size_t)(E + 1) * 4);
        take(L.permws, perm_ws_bytes(T, E));
        L.total = off;
        return L;
    }
    take(L.prices, (size_t)E * 8);
    take(L.offsets, (size_t)(E + 1) * 4);
    if (op == BASE_OP_LAYER || op == BASE_OP_LAYER_EX) {
        const size_t b = dt == BASE_BF16 ? 2 : 4;
        take(L.scores, (size_t)T * E * 4);
        take(L.perm, (size_t)T * 4);
        take(L.hidden, (size_t)T * F * b);
        take(L.gblk, (size_t)(E + 1) * 4);
        if (op == BASE_OP_LAYER_EX) {
            take(L.xbuf, (size_t)T * D * b);  // an expert's running block output
            take(L.ybuf, (size_t)T * D * b);  // its layer-norm output
        }
    }
    // the auction's own scratch, followed by the grouping's
    take(L.auction, auction_ws_bytes(T, E) + perm_ws_bytes(T, E));
    L.permws = L.auction + auction_ws_bytes(T, E);
    L.total = off;
    return L;
}

int cfg_phases(const base_auction_cfg& c) {
    if (!(c.eps_end > 0) || !(c.eps_start >= c.eps_end) || !isfinite(c.eps_start) ||
        !(c.eps_factor > 1) || !isfinite(c.eps_factor))
        return -1;
    int n = 1;
    double eps = c.eps_start;
    while (eps > c.eps_end) {
        eps /= c.eps_factor;
        if (eps < c.eps_end) eps = c.eps_end;
        if (++n > kMaxPhases) return -1;
    }
    return n;
}

bool misaligned(const void* p) { return ((uintptr_t)p & 15u) != 0; }

thread_local hipEvent_t g_events[6];
thread_local int g_nevents = 0;

void mark(int i, hipStream_t st) {
    if (i < g_nevents && g_events[i]) (void)hipEventRecord(g_events[i], st);
}

constexpr int kAucEvents = 64;
thread_local hipEvent_t g_auc_events[kAucEvents];
thread_local int g_auc_nevents = 0;

int hip_rc(hipError_t e) { return e == hipSuccess ? BASE_OK : BASE_ERR_HIP; }

}  // namespace

void base::auction_mark(int i, hipStream_t st) {
    if (i < g_auc_nevents && g_auc_events[i]) (void)hipEventRecord(g_auc_events[i], st);
}

// Shared body of base_layer_forward (o == nullptr: eq. 1, plain experts)
// and base_layer_forward_ex.
static int layer_forward(const void* h, const void* w, const void* W1, const void* W2, int64_t T,
                         int64_t E, int64_t D, int64_t F, int dt, int act, int mode,
                         base_auction_cfg cfg, int32_t* assign, float* scores, int32_t* perm,
                         void* out, base_auction_stats* stats, const base_layer_opts* o,
                         void* ws, size_t ws_bytes, base_stream_t stream) {
    if (!h || !w || !W1 || !W2 || !assign || !out) return BASE_ERR_INVALID_ARG;
    if (T <= 0 || E <= 0 || D <= 0 || F <= 0 || E > T) return BASE_ERR_INVALID_ARG;
    if (dt != BASE_F32 && dt != BASE_BF16) return BASE_ERR_INVALID_ARG;
    if (act != BASE_ACT_RELU && act != BASE_ACT_GELU) return BASE_ERR_INVALID_ARG;
    if (mode != BASE_ROUTE_BALANCED && mode != BASE_ROUTE_GREEDY && mode != BASE_ROUTE_GIVEN)
        return BASE_ERR_INVALID_ARG;
    const int mix = o ? o->mix : BASE_MIX_RESIDUAL;
    const int nsub = o ? o->sublayers : 0;
    if (mix != BASE_MIX_RESIDUAL && mix != BASE_MIX_CONVEX) return BASE_ERR_INVALID_ARG;
    if (nsub < 0 || nsub > kMaxSublayers) return BASE_ERR_INVALID_ARG;
    if (nsub > 0 && !(o->ln_eps >= 0) ) return BASE_ERR_INVALID_ARG;
    if (mode == BASE_ROUTE_BALANCED && cfg_phases(cfg) < 0) return BASE_ERR_INVALID_ARG;
    if (mode != BASE_ROUTE_GREEDY && T % E) return BASE_ERR_INDIVISIBLE;
    if (T > kMaxT || E > kMaxE) return BASE_ERR_UNSUPPORTED;
    if (dt == BASE_BF16 && (D % 8 != 0 || F % 8 != 0 || misaligned(h) || misaligned(w) ||
                            misaligned(W1) || misaligned(W2) || misaligned(out)))
        return BASE_ERR_UNSUPPORTED;
    const Layout L = layout(o ? BASE_OP_LAYER_EX : BASE_OP_LAYER, T, E, D, F, dt);
    if (!ws || ws_bytes < L.total) return BASE_ERR_INVALID_ARG;
    hipStream_t st = (hipStream_t)stream;
    char* W = (char*)ws;
    const int64_t k = T / E;
    ScoreScan* scan = (ScoreScan*)(W + L.scan);
    AucStatsDev* sd = stats ? (AucStatsDev*)stats : (AucStatsDev*)(W + L.stats);
    float* s = scores ? scores : (float*)(W + L.scores);
    int32_t* pm = perm ? perm : (int32_t*)(W + L.perm);
    int32_t* offs = (int32_t*)(W + L.offsets);
    double* prices = (double*)(W + L.prices);
    void* H = W + L.hidden;
    int32_t* gblk = (int32_t*)(W + L.gblk);
    // greedy routing gives ragged expert groups (rows offs[e] .. offs[e+1]-1)
    const int32_t* goff = (mode == BASE_ROUTE_GREEDY) ? offs : nullptr;

    mark(0, st);
    hipError_t e = launch_scan_init(scan, st);
    if (e == hipSuccess) e = launch_affinity(h, w, s, T, E, D, dt, scan, st);
    mark(1, st);
    if (e == hipSuccess) {
        if (mode == BASE_ROUTE_BALANCED) {
            e = launch_auction(s, T, E, cfg.eps_start, cfg.eps_end, cfg.eps_factor, cfg.max_bids,
                               scan, assign, pm, offs, prices, sd, W + L.auction, st);
        } else if (mode == BASE_ROUTE_GREEDY) {
            e = launch_stats_reset(sd, st);
            if (e == hipSuccess) e = launch_greedy(s, T, E, scan, assign, nullptr, st);
            if (e == hipSuccess)
                e = launch_perm(assign, T, E, pm, offs, nullptr, 0, nullptr, W + L.permws, st);
        } else {
            e = launch_stats_reset(sd, st);
            if (e == hipSuccess)
                e = launch_perm(assign, T, E, pm, offs, nullptr, k, &sd->status, W + L.permws, st);
        }
    }
    mark(2, st);
    if (nsub == 0) {
        if (e == hipSuccess) e = launch_ffn1(h, pm, W1, H, E, k, D, F, dt, act, goff, gblk, T, st);
        mark(3, st);
        if (e == hipSuccess) {
            if (mix == BASE_MIX_RESIDUAL) {
                e = launch_ffn2(H, pm, W2, s, h, out, E, k, D, F, dt, goff, gblk, T, st);
            } else {
                const Ffn2Epi epi = {0, 1, 0, nullptr, nullptr};  // g C + (1 - g) h
                e = launch_ffn2_ex(H, pm, W2, s, h, out, E, k, D, F, dt, goff, gblk, T, epi, st);
            }
        }
    } else {
        // sec. 4.1 experts: blocks x <- x + W2_n act(W1_n LN_n(x)); block 0
        // reads the token rows through perm, later blocks the grouped running
        // output X (updated in place: each element is read and rewritten by
        // the lane that owns it); the last block mixes into out
        const size_t b = dt == BASE_BF16 ? 2 : 4;
        void* X = W + L.xbuf;
        void* Y = W + L.ybuf;
        for (int n = 0; n < nsub && e == hipSuccess; ++n) {
            const float* ga = o->ln_gamma ? o->ln_gamma + (size_t)n * E * D : nullptr;
            const float* be = o->ln_beta ? o->ln_beta + (size_t)n * E * D : nullptr;
            const char* w1 = (const char*)W1 + (size_t)n * E * F * D * b;
            const char* w2 = (const char*)W2 + (size_t)n * E * D * F * b;
            e = launch_layernorm(n == 0 ? h : X, n == 0, pm, assign, ga, be, o->ln_eps, Y, T, E,
                                 D, dt, st);
            if (e == hipSuccess)
                e = launch_ffn1(Y, nullptr, w1, H, E, k, D, F, dt, act, goff, gblk, T, st);
            if (n == nsub - 1) mark(3, st);
            if (e != hipSuccess) break;
            const int res = n == 0 ? 1 : 2;  // R = x (block 0) or X
            if (n < nsub - 1) {
                const Ffn2Epi epi = {1, 2, res, X, X};  // X = R + C, grouped
                e = launch_ffn2_ex(H, pm, w2, s, h, out, E, k, D, F, dt, goff, gblk, T, epi, st);
            } else {
                const int keep = mix == BASE_MIX_CONVEX ? 1 : 0;
                const Ffn2Epi epi = {0, keep, res, X, nullptr};  // g (R + C) + c2 x
                e = launch_ffn2_ex(H, pm, w2, s, h, out, E, k, D, F, dt, goff, gblk, T, epi, st);
            }
        }
    }
    mark(4, st);
    mark(5, st);
    return hip_rc(e);
}

// Shared body of base_layer_backward (plain experts) and
// base_layer_backward_ex (also experts of layer-norm blocks).
static int layer_backward(const void* h, const void* w, const void* W1, const void* W2, int64_t T,
                          int64_t E, int64_t D, int64_t F, int dt, int act, const int32_t* assign,
                          const float* scores, const void* dy, void* dh, void* dw, void* dW1,
                          void* dW2, float* dgamma, float* dbeta, base_auction_stats* stats,
                          const base_layer_opts* opts, void* ws, size_t ws_bytes,
                          base_stream_t stream) {
    if (!h || !w || !W1 || !W2 || !assign || !scores || !dy || !dh || !dw || !dW1 || !dW2)
        return BASE_ERR_INVALID_ARG;
    if (T <= 0 || E <= 0 || D <= 0 || F <= 0 || E > T) return BASE_ERR_INVALID_ARG;
    if (dt != BASE_F32 && dt != BASE_BF16) return BASE_ERR_INVALID_ARG;
    if (act != BASE_ACT_RELU && act != BASE_ACT_GELU) return BASE_ERR_INVALID_ARG;
    const int mix = opts ? opts->mix : BASE_MIX_RESIDUAL;
    const int nsub = opts ? opts->sublayers : 0;
    if (mix != BASE_MIX_RESIDUAL && mix != BASE_MIX_CONVEX) return BASE_ERR_INVALID_ARG;
    if (nsub < 0 || nsub > kMaxSublayers) return BASE_ERR_INVALID_ARG;
    if (nsub > 0 && !(opts->ln_eps >= 0)) return BASE_ERR_INVALID_ARG;
    if (T > kMaxT || E > kMaxE) return BASE_ERR_UNSUPPORTED;
    // the backward products address a tile's operands with 32-bit offsets
    if (D > kMaxBwdWidth || F > kMaxBwdWidth) return BASE_ERR_UNSUPPORTED;
    if (dt == BASE_BF16 &&
        (D % 8 != 0 || F % 8 != 0 || misaligned(h) || misaligned(w) || misaligned(W1) ||
         misaligned(W2) || misaligned(dy) || misaligned(dh) || misaligned(dW1) || misaligned(dW2)))
        return BASE_ERR_UNSUPPORTED;
    const Layout L = layout(BASE_OP_LAYER_BWD, T, E, D, F, dt, nsub);
    if (!ws || ws_bytes < L.total) return BASE_ERR_INVALID_ARG;
    hipStream_t st = (hipStream_t)stream;
    char* W = (char*)ws;
    AucStatsDev* sd = stats ? (AucStatsDev*)stats : (AucStatsDev*)(W + L.stats);
    int32_t* pm = (int32_t*)(W + L.perm);
    int32_t* offs = (int32_t*)(W + L.offsets);
    int32_t* gblk = (int32_t*)(W + L.gblk);
    void* Xg = W + L.xg;
    void* dYg = W + L.dyg;
    void* Z = W + L.zbuf;
    void* gU = W + L.gubuf;
    void* dZ = W + L.dzbuf;
    float* part = (float*)(W + L.part);
    float* dl = (float*)(W + L.dl);
    const int64_t np = bwd_nparts(F, dt == BASE_BF16);
    const size_t b = dt == BASE_BF16 ? 2 : 4;

    mark(0, st);
    // expert groups of the given assignment (any sizes; ids outside [0, E)
    // are reported through stats->status)
    hipError_t e = launch_stats_reset(sd, st);
    if (e == hipSuccess)
        e = launch_perm(assign, T, E, pm, offs, nullptr, 0, &sd->status, W + L.permws, st);
    if (nsub == 0) {
        if (e == hipSuccess) e = launch_gather2(h, dy, pm, Xg, dYg, T, D, dt, st);
        if (e == hipSuccess)
            e = launch_bwd_z(Xg, W1, pm, scores, Z, gU, T, E, D, F, dt, act, offs, gblk, 0, st);
        mark(1, st);
        if (e == hipSuccess)
            e = launch_bwd_v(dYg, W2, pm, scores, Z, dZ, part, T, E, D, F, dt, act, offs, gblk, 0,
                             st);
        if (e == hipSuccess)
            e = launch_gate_grad(part, np, Xg, dYg, pm, offs, scores, mix, dl, T, E, D, dt, st);
        mark(2, st);
        if (e == hipSuccess) e = launch_bwd_w(dYg, gU, D, F, E, offs, dW2, dt, st);
        mark(3, st);
        if (e == hipSuccess) e = launch_bwd_w(dZ, Xg, F, D, E, offs, dW1, dt, st);
        mark(4, st);
        if (e == hipSuccess)
            e = launch_bwd_x(dZ, W1, pm, scores, dYg, w, dl, mix, dh, T, E, D, F, dt, offs, gblk,
                             nullptr, st);
        if (e == hipSuccess) e = launch_centroid_grad(dl, Xg, offs, dw, E, D, dt, st);
        mark(5, st);
        return hip_rc(e);
    }

    // experts of nsub layer-norm blocks (sec. 4.1): run the blocks forward on
    // the grouped rows, keeping every block's input x_n (x_0 = h's rows), then
    // take the blocks back, last first, on the upstream g dy
    char* xs = W + L.xs;
    auto X = [&](int n) -> void* { return xs + (size_t)n * T * D * b; };
    float* dXa = (float*)(W + L.dxa);
    void* dXo = W + L.dxo;
    void* dYn = W + L.dyn;
    float* lnst = (float*)(W + L.lnst);
    auto Yn = [&](int n) -> void* { return W + L.ybuf + (size_t)n * T * D * b; };
    auto Zn = [&](int n) -> void* { return (char*)Z + (size_t)n * T * F * b; };
    auto Un = [&](int n) -> void* { return (char*)gU + (size_t)n * T * F * b; };
    const int64_t k = T / E;  // unused with ragged groups, which all launches here use
    auto ga = [&](int n) -> const float* {
        return opts->ln_gamma ? opts->ln_gamma + (size_t)n * E * D : nullptr;
    };
    auto be = [&](int n) -> const float* {
        return opts->ln_beta ? opts->ln_beta + (size_t)n * E * D : nullptr;
    };
    auto w1 = [&](int n) { return (const char*)W1 + (size_t)n * E * F * D * b; };
    auto w2 = [&](int n) { return (const char*)W2 + (size_t)n * E * D * F * b; };
    if (e == hipSuccess) e = launch_gather2(h, dy, pm, X(0), dYg, T, D, dt, st);
    for (int n = 0; n < nsub && e == hipSuccess; ++n) {
        e = launch_layernorm(X(n), 0, pm, assign, ga(n), be(n), opts->ln_eps, Yn(n), T, E, D, dt,
                             st);
        if (e == hipSuccess)  // Z_n and act(Z_n) (gate 1)
            e = launch_bwd_z(Yn(n), w1(n), pm, scores, Zn(n), Un(n), T, E, D, F, dt, act, offs,
                             gblk, 1, st);
        const Ffn2Epi epi = {1, 2, 2, X(n), X(n + 1)};  // x_{n+1} = x_n + C, grouped
        if (e == hipSuccess)
            e = launch_ffn2_ex(Un(n), pm, w2(n), scores, h, nullptr, E, k, D, F, dt, offs, gblk,
                               T, epi, st);
    }
    mark(1, st);
    if (e == hipSuccess)
        e = launch_block_gate(X(0), X(nsub), dYg, pm, offs, scores, mix, dXa, dXo, dl, T, E, D, dt,
                              st);
    mark(2, st);
    for (int n = nsub - 1; n >= 0 && e == hipSuccess; --n) {
        // gate 1: the upstream dX already holds g
        e = launch_bwd_v(dXo, w2(n), pm, scores, Zn(n), dZ, part, T, E, D, F, dt, act, offs, gblk,
                         1, st);
        if (e == hipSuccess)
            e = launch_bwd_w(dXo, Un(n), D, F, E, offs, (char*)dW2 + (size_t)n * E * D * F * b,
                             dt, st);
        if (e == hipSuccess)
            e = launch_bwd_w(dZ, Yn(n), F, D, E, offs, (char*)dW1 + (size_t)n * E * F * D * b, dt,
                             st);
        if (e == hipSuccess)
            e = launch_bwd_x(dZ, w1(n), pm, scores, dYg, w, dl, mix, dh, T, E, D, F, dt, offs,
                             gblk, dYn, st);
        if (e == hipSuccess)
            e = launch_ln_backward(X(n), dYn, ga(n), offs, opts->ln_eps, dXa, dXo, lnst, T, E, D,
                                   dt, st);
        if (e == hipSuccess)
            e = launch_ln_param_grad(X(n), dYn, lnst, offs,
                                     dgamma ? dgamma + (size_t)n * E * D : nullptr,
                                     dbeta ? dbeta + (size_t)n * E * D : nullptr, E, D, dt, st);
    }
    mark(3, st);
    mark(4, st);
    if (e == hipSuccess)
        e = launch_finish_dh(dXa, dYg, dl, w, pm, offs, scores, mix, dh, T, E, D, dt, st);
    if (e == hipSuccess) e = launch_centroid_grad(dl, X(0), offs, dw, E, D, dt, st);
    mark(5, st);
    return hip_rc(e);
}

extern "C" {

const char* base_strerror(int code) {
    switch (code) {
        case BASE_OK: return "ok";
        case BASE_ERR_INVALID_ARG: return "invalid argument";
        case BASE_ERR_INDIVISIBLE: return "T is not a multiple of E";
        case BASE_ERR_UNSUPPORTED: return "unsupported: outside the library's size or layout limits";
        case BASE_ERR_HIP: return "HIP launch failed";
        case BASE_ERR_NOT_CONVERGED: return "auction stopped at its bid cap";
        case BASE_ERR_NONFINITE: return "no finite affinity";
        case BASE_ERR_UNBALANCED: return "given assignment is not balanced";
        case BASE_ERR_INVARIANT: return "an auction invariant failed (checking build)";
        default: return "unknown error";
    }
}

int base_set_auction_events(void** events, int n) {
    if (n < 0 || n > kAucEvents) return BASE_ERR_INVALID_ARG;
    if (!events) n = 0;
    for (int i = 0; i < kAucEvents; ++i) g_auc_events[i] = (events && i < n) ? (hipEvent_t)events[i] : nullptr;
    g_auc_nevents = n;
    return BASE_OK;
}

int base_set_phase_events(void** events, int n) {
    if (n < 0 || n > 6) return BASE_ERR_INVALID_ARG;
    if (!events) n = 0;
    for (int i = 0; i < 6; ++i) g_events[i] = (events && i < n) ? (hipEvent_t)events[i] : nullptr;
    g_nevents = n;
    return BASE_OK;
}

size_t base_workspace_bytes(int op, int64_t T, int64_t E, int64_t D, int64_t F, int dtype) {
    if (T <= 0 || E <= 0 || op < 0 || op > BASE_OP_LAYER_BWD) return 0;
    if ((op == BASE_OP_LAYER || op == BASE_OP_LAYER_EX || op == BASE_OP_LAYER_BWD) &&
        (F <= 0 || D <= 0))
        return 0;
    return layout(op, T, E, D, F, dtype).total;
}

int base_affinity(const void* h, const void* w, float* scores, int64_t T, int64_t E, int64_t D,
                  int dt, base_stream_t stream) {
    if (!h || !w || !scores || T <= 0 || E <= 0 || D <= 0) return BASE_ERR_INVALID_ARG;
    if (dt != BASE_F32 && dt != BASE_BF16) return BASE_ERR_INVALID_ARG;
    if (T > kMaxT) return BASE_ERR_UNSUPPORTED;
    if (dt == BASE_BF16 && (D % 8 != 0 || misaligned(h) || misaligned(w)))
        return BASE_ERR_UNSUPPORTED;
    return hip_rc(launch_affinity(h, w, scores, T, E, D, dt, nullptr, (hipStream_t)stream));
}

int base_assign_auction(const float* scores, int64_t T, int64_t E, base_auction_cfg cfg,
                        int32_t* assign, int32_t* perm, int32_t* offsets, double* prices,
                        base_auction_stats* stats, void* ws, size_t ws_bytes,
                        base_stream_t stream) {
    if (!scores || !assign || !perm || !offsets || !prices) return BASE_ERR_INVALID_ARG;
    if (T <= 0 || E <= 0 || E > T) return BASE_ERR_INVALID_ARG;
    if (T % E) return BASE_ERR_INDIVISIBLE;
    if (T > kMaxT || E > kMaxE) return BASE_ERR_UNSUPPORTED;
    if (cfg_phases(cfg) < 0) return BASE_ERR_INVALID_ARG;
    const Layout L = layout(BASE_OP_AUCTION, T, E, 0, 0, 0);
    if (!ws || ws_bytes < L.total) return BASE_ERR_INVALID_ARG;
    hipStream_t st = (hipStream_t)stream;
    char* W = (char*)ws;
    ScoreScan* scan = (ScoreScan*)(W + L.scan);
    AucStatsDev* sd = stats ? (AucStatsDev*)stats : (AucStatsDev*)(W + L.stats);
    hipError_t e = launch_scan_init(scan, st);
    if (e == hipSuccess) e = launch_scan_scores(scores, T * E, scan, st);
    if (e == hipSuccess)
        e = launch_auction(scores, T, E, cfg.eps_start, cfg.eps_end, cfg.eps_factor, cfg.max_bids,
                           scan, assign, perm, offsets, prices, sd, W + L.auction, st);
    return hip_rc(e);
}

int base_route_greedy(const float* scores, int64_t T, int64_t E, int32_t* assign, int32_t* counts,
                      int32_t* perm, int32_t* offsets, void* ws, size_t ws_bytes,
                      base_stream_t stream) {
    if (!scores || !assign || T <= 0 || E <= 0) return BASE_ERR_INVALID_ARG;
    if ((perm == nullptr) != (offsets == nullptr)) return BASE_ERR_INVALID_ARG;
    if (T > kMaxT || E > kMaxT) return BASE_ERR_UNSUPPORTED;
    // counts and the grouping come from the grouping kernels, whose LDS
    // tables hold E entries: refuse before anything is enqueued
    if ((counts || perm) && E > kPermMaxE) return BASE_ERR_UNSUPPORTED;
    const Layout L = layout(BASE_OP_GREEDY, T, E, 0, 0, 0);
    if (!ws || ws_bytes < L.total) return BASE_ERR_INVALID_ARG;
    hipStream_t st = (hipStream_t)stream;
    char* W = (char*)ws;
    ScoreScan* scan = (ScoreScan*)(W + L.scan);
    hipError_t e = launch_scan_init(scan, st);
    if (e == hipSuccess) e = launch_scan_scores(scores, T * E, scan, st);
    if (e == hipSuccess) e = launch_greedy(scores, T, E, scan, assign, counts, st);
    if (e == hipSuccess && (counts || perm)) {
        int32_t* p = perm ? perm : (int32_t*)(W + L.perm);
        int32_t* o = offsets ? offsets : (int32_t*)(W + L.offsets);
        e = launch_perm(assign, T, E, p, o, counts, 0, nullptr, W + L.permws, st);
    }
    return hip_rc(e);
}

// ---- greedy routing without a workspace argument. Its scratch (the score
// scan, the grouping's chunk tables, and the permutation and offsets when
// the caller does not want them) lives in a fixed device array; every GPU
// the library runs on holds its own copy until the process ends. Host code
// never passes the array's name to a kernel: it takes the array's device
// address from hipGetSymbolAddress, once per device, and uses that.
constexpr size_t kNoAllocScratchBytes = size_t(8) << 20;
constexpr int kNoAllocMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kNoAllocMaxDevices] = {};

// The current device's scratch address (looked up on its first use), or
// nullptr if HIP fails.
static void* device_scratch() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kNoAllocMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

int base_route_greedy_noalloc(const float* scores, int64_t T, int64_t E, int32_t* assign,
                              int32_t* counts, int32_t* perm, int32_t* offsets,
                              base_stream_t stream) {
    if (!scores || !assign || T <= 0 || E <= 0) return BASE_ERR_INVALID_ARG;
    if ((perm == nullptr) != (offsets == nullptr)) return BASE_ERR_INVALID_ARG;
    if (T > kMaxT || E > kMaxT) return BASE_ERR_UNSUPPORTED;
    if ((counts || perm) && E > kPermMaxE) return BASE_ERR_UNSUPPORTED;
    const Layout L = layout(BASE_OP_GREEDY, T, E, 0, 0, 0);
    if (L.total > kNoAllocScratchBytes) return BASE_ERR_UNSUPPORTED;
    void* ws = device_scratch();
    if (!ws) return BASE_ERR_HIP;
    return base_route_greedy(scores, T, E, assign, counts, perm, offsets, ws,
                             kNoAllocScratchBytes, stream);
}

int base_layer_forward(const void* h, const void* w, const void* W1, const void* W2, int64_t T,
                       int64_t E, int64_t D, int64_t F, int dt, int act, int mode,
                       base_auction_cfg cfg, int32_t* assign, float* scores, int32_t* perm,
                       void* out, base_auction_stats* stats, void* ws, size_t ws_bytes,
                       base_stream_t stream) {
    return layer_forward(h, w, W1, W2, T, E, D, F, dt, act, mode, cfg, assign, scores, perm, out,
                         stats, nullptr, ws, ws_bytes, stream);
}

int base_layer_forward_ex(const void* h, const void* w, const void* W1, const void* W2,
                          int64_t T, int64_t E, int64_t D, int64_t F, int dt, int act, int mode,
                          base_auction_cfg cfg, int32_t* assign, float* scores, int32_t* perm,
                          void* out, base_auction_stats* stats, const base_layer_opts* opts,
                          void* ws, size_t ws_bytes, base_stream_t stream) {
    const base_layer_opts dflt = {BASE_MIX_RESIDUAL, 0, 1e-5, nullptr, nullptr};
    return layer_forward(h, w, W1, W2, T, E, D, F, dt, act, mode, cfg, assign, scores, perm, out,
                         stats, opts ? opts : &dflt, ws, ws_bytes, stream);
}

int base_layer_backward(const void* h, const void* w, const void* W1, const void* W2, int64_t T,
                        int64_t E, int64_t D, int64_t F, int dt, int act, const int32_t* assign,
                        const float* scores, const void* dy, void* dh, void* dw, void* dW1,
                        void* dW2, base_auction_stats* stats, const base_layer_opts* opts,
                        void* ws, size_t ws_bytes, base_stream_t stream) {
    if (opts && opts->sublayers != 0) return BASE_ERR_UNSUPPORTED;
    return layer_backward(h, w, W1, W2, T, E, D, F, dt, act, assign, scores, dy, dh, dw, dW1, dW2,
                          nullptr, nullptr, stats, opts, ws, ws_bytes, stream);
}

int base_layer_backward_ex(const void* h, const void* w, const void* W1, const void* W2,
                           int64_t T, int64_t E, int64_t D, int64_t F, int dt, int act,
                           const int32_t* assign, const float* scores, const void* dy, void* dh,
                           void* dw, void* dW1, void* dW2, float* dgamma, float* dbeta,
                           base_auction_stats* stats, const base_layer_opts* opts, void* ws,
                           size_t ws_bytes, base_stream_t stream) {
    return layer_backward(h, w, W1, W2, T, E, D, F, dt, act, assign, scores, dy, dh, dw, dW1, dW2,
                          dgamma, dbeta, stats, opts, ws, ws_bytes, stream);
}

size_t base_workspace_bytes_ex(int op, int64_t T, int64_t E, int64_t D, int64_t F, int dtype,
                               int sublayers) {
    if (sublayers < 0 || sublayers > kMaxSublayers) return 0;
    if (op != BASE_OP_LAYER_BWD || sublayers == 0) return base_workspace_bytes(op, T, E, D, F, dtype);
    if (T <= 0 || E <= 0 || F <= 0 || D <= 0) return 0;
    return layout(op, T, E, D, F, dtype, sublayers).total;
}

}  // extern "C"
