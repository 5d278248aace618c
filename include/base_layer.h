/*
 * base_layer.h -- C ABI of the MI355X (gfx950) BASE-layer forward library
 * (libbase_layer.so).
 *
 * The operation is the forward pass of a BASE layer -- Lewis, Bhosale,
 * Dettmers, Goyal, Zettlemoyer, "BASE Layers: Simplifying Training of Large,
 * Sparse Models" (arXiv 2103.16716):
 *   - token-expert affinities s[t][e] = h_t . w_e (sec. 3.1; fig. 2 scores the
 *     tokens against the expert centroids);
 *   - the balanced assignment of eq. 2 (sec. 3.2.1): maximise sum_t s[t][a_t]
 *     subject to every expert receiving exactly k = T/E tokens, solved by an
 *     auction (sec. 3.2.1; the paper's own listing, fig. 9, is prior art --
 *     here tokens bid for expert slots, see base_assign_auction);
 *   - greedy test-time routing, a_t = argmax_e s[t][e] (sec. 3.2.2);
 *   - grouping the tokens by expert (fig. 2's expert sort), running each
 *     expert's position-wise FFN, and the output of eq. 1 (sec. 3.1):
 *       y_t = sigmoid(h_t . w_{a_t}) * f_{a_t}(h_t) + h_t,
 *     returned in the original token order (fig. 2 undoes the sort).
 *
 * Conventions for every entry point:
 *   - Every pointer argument except `stats` results and host structs passed by
 *     value is a DEVICE pointer (HIP global memory) owned by the caller. The
 *     library allocates nothing and keeps no pointer after the enqueued work
 *     completes.
 *   - Work is enqueued asynchronously on `stream` (0 = the null stream); the
 *     call returns without synchronising. Outputs are valid after the stream
 *     reaches the enqueued work.
 *   - Matrices are row-major and dense. Shapes: h T x D, w E x D, scores
 *     T x E (fig. 2's orientation), W1 E x F x D and W2 E x D x F (each
 *     expert's matrices in the [out, in] layout, so the reduction dimension
 *     is contiguous for both products).
 *   - Return value: BASE_OK (0) or a negative BASE_ERR_* code found on the
 *     host before anything is enqueued (nothing is enqueued then), or
 *     BASE_ERR_HIP if a launch failed. Conditions that only the device can
 *     see are written to stats->status (see base_auction_stats).
 *   - Calls that share a workspace must not overlap; use distinct workspaces
 *     (or one stream) for concurrent calls.
 */
#ifndef BASE_LAYER_H_
#define BASE_LAYER_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *base_stream_t; /* a hipStream_t */

typedef enum {
    BASE_OK = 0,
    BASE_ERR_INVALID_ARG = -1,   /* null pointer, size <= 0, E > T, bad enum,
                                    eps schedule not eps_start >= eps_end > 0,
                                    workspace too small */
    BASE_ERR_INDIVISIBLE = -2,   /* T % E != 0 (eq. 2 needs T/E per expert;
                                    the paper leaves this case open) */
    BASE_ERR_UNSUPPORTED = -3,   /* a valid request outside the library's limits */
    BASE_ERR_HIP = -4,           /* a HIP launch or query failed */
    BASE_ERR_NOT_CONVERGED = -5, /* device: the auction hit cfg.max_bids */
    BASE_ERR_NONFINITE = -6,     /* device: no finite affinity at all */
    BASE_ERR_INVARIANT = -9,     /* device, checking build only (libbase_layer_checks.so,
                                    compiled with BASE_CHECKS): an auction invariant
                                    failed (an expert holding more than T/E tokens or
                                    holders out of order, or at the end an expert
                                    without exactly T/E distinct tokens) */
    BASE_ERR_UNBALANCED = -8     /* device: a given assignment is not balanced
                                    or holds an expert id outside [0, E) */
} base_status;

typedef enum { BASE_F32 = 0, BASE_BF16 = 1 } base_dtype;

/* Expert activation: ReLU (the paper's feed-forward blocks, sec. 4.1) or
 * GELU in its exact erf form, x/2 * (1 + erf(x / sqrt 2)). */
typedef enum { BASE_ACT_RELU = 0, BASE_ACT_GELU = 1 } base_act;

/* How base_layer_forward routes tokens: the balanced assignment used in
 * training (sec. 3.2.1), greedy argmax as at test time (sec. 3.2.2), or an
 * assignment the caller gives (must be balanced). */
typedef enum {
    BASE_ROUTE_BALANCED = 0,
    BASE_ROUTE_GREEDY = 1,
    BASE_ROUTE_GIVEN = 2
} base_route;

/* Auction settings. The paper's listing leaves its epsilon undefined; this
 * library takes Bertsekas-style eps-scaling: phases with eps = eps_start,
 * max(eps/eps_factor, eps_end), ..., eps_end (eps_start == eps_end: a single
 * phase). The result is within T * eps_end of the optimum of eq. 2, and is
 * the optimum itself when eps_end < gap / T, gap being the distance from the
 * optimum to the second-best balanced assignment. max_bids <= 0 means no cap;
 * otherwise the auction stops at its first check after that many bids (after
 * every parallel round, and after every batch of augmenting paths of a
 * phase's end) and reports BASE_ERR_NOT_CONVERGED (a safety valve, not part
 * of the method). */
typedef struct {
    double eps_start;
    double eps_end;
    double eps_factor; /* > 1; 10 is the usual choice */
    int64_t max_bids;
} base_auction_cfg;

/* Written by the device (a DEVICE pointer); read it after the stream has
 * reached the call. status is BASE_OK or BASE_ERR_NOT_CONVERGED /
 * BASE_ERR_NONFINITE / BASE_ERR_UNBALANCED. For eps phase p (p < 16):
 * bids[p] counts its bids -- one per token per parallel bidding round (all
 * unassigned tokens bidding at once) plus one per token that the phase's end
 * placed by an augmenting path; tail[p] is that last part alone; rounds[p]
 * is the phase's sequential depth: its parallel rounds plus the batches of
 * augmenting paths of its end. */
typedef struct {
    int32_t status;
    int32_t phases;
    int64_t bids[16];
    int64_t rounds[16];
    int64_t tail[16];
} base_auction_stats;

/* Workspace queries: the bytes of device scratch memory each entry point
 * needs for the given sizes. The caller allocates it (any alignment the HIP
 * allocator gives); its contents need not be initialised and are garbage on
 * return. */
typedef enum {
    BASE_OP_AFFINITY = 0,
    BASE_OP_AUCTION = 1,
    BASE_OP_GREEDY = 2,
    BASE_OP_LAYER = 3,
    BASE_OP_LAYER_EX = 4, /* base_layer_forward_ex: LAYER plus two T x D buffers */
    BASE_OP_LAYER_BWD = 5 /* base_layer_backward */
} base_op;

size_t base_workspace_bytes(int op, int64_t T, int64_t E, int64_t D, int64_t F,
                            int dtype);

/* Text for a base_status code (static storage; never NULL). */
const char *base_strerror(int code);

/*
 * base_affinity -- s[t][e] = sum_d h[t][d] * w[e][d]  (sec. 3.1, fig. 2).
 *   h: T x D, w: E x D, both of dtype dt (bf16 or fp32);
 *   scores: T x E fp32 output. Products and sums in fp32 (bf16 inputs are
 *   widened exactly); the summation order is the kernel's.
 * Errors: BASE_ERR_INVALID_ARG for null pointers or non-positive sizes.
 * No workspace. Non-finite results are stored as computed.
 */
int base_affinity(const void *h, const void *w, float *scores, int64_t T,
                  int64_t E, int64_t D, int dt, base_stream_t stream);

/*
 * base_assign_auction -- balanced assignment of eq. 2 (sec. 3.2.1) by a
 * token-side auction with eps-scaling.
 *   scores: T x E fp32 (read only). NaN and +-inf are read as the smallest
 *     finite score of the matrix, as the released code does before solving;
 *     if no score is finite, stats->status = BASE_ERR_NONFINITE.
 *   assign[T] (out, int32): the expert of each token; every expert gets
 *     exactly k = T/E tokens.
 *   perm[T] (out, int32): token ids grouped by expert, ascending within
 *     each expert: perm[e*k .. e*k+k-1] are expert e's tokens.
 *   offsets[E+1] (out, int32): offsets[e] = e*k.
 *   prices[E] (out, fp64): final expert prices p_e (the lowest bid each
 *     expert holds). They certify the result: with
 *     D(p) = sum_t max_e (s[t][e] - p_e) + k sum_e p_e (>= optimum),
 *     sum_t s[t][a_t] >= D(p) - T * eps_end.
 *   stats (device pointer, may be NULL): see base_auction_stats.
 *   ws / ws_bytes: scratch of base_workspace_bytes(BASE_OP_AUCTION, ...).
 * Errors (host): INVALID_ARG, INDIVISIBLE (T % E), UNSUPPORTED if
 *   T > 2^24 or E > 1024.
 */
int base_assign_auction(const float *scores, int64_t T, int64_t E,
                        base_auction_cfg cfg, int32_t *assign, int32_t *perm,
                        int32_t *offsets, double *prices,
                        base_auction_stats *stats, void *ws, size_t ws_bytes,
                        base_stream_t stream);

/*
 * base_route_greedy -- test-time routing (sec. 3.2.2): a_t = the expert with
 * the highest score, the lowest expert id among equal scores (scores
 * sanitised as in base_assign_auction; if no score is finite every token
 * goes to expert 0 -- this entry point has no status output).
 *   assign[T], counts[E] (tokens per expert), perm[T] (grouped by expert,
 *   ascending token id within a group), offsets[E+1] (prefix sums of
 *   counts). Any of counts/perm/offsets may be NULL to skip it (perm and
 *   offsets go together).
 *   ws: scratch of base_workspace_bytes(BASE_OP_GREEDY, ...).
 * T % E need not be 0.
 * Errors: INVALID_ARG (null scores/assign, sizes <= 0, perm without
 *   offsets, workspace too small); UNSUPPORTED for T or E above 2^24, and
 *   for E above 4096 when counts or perm is asked for (the grouping keeps
 *   per-expert tables in on-chip memory); nothing is enqueued then.
 */
int base_route_greedy(const float *scores, int64_t T, int64_t E,
                      int32_t *assign, int32_t *counts, int32_t *perm,
                      int32_t *offsets, void *ws, size_t ws_bytes,
                      base_stream_t stream);

/*
 * base_layer_forward -- the whole BASE layer forward (fig. 2 without the
 * cross-worker shuffle and all-to-alls: one device holds every expert):
 * affinities, routing, expert grouping, y = sigmoid(s[t][a_t]) * f(h_t) + h_t
 * (eq. 1) with f_e(x) = W2_e act(W1_e x) (no bias), output in token order.
 *   h: T x D, w: E x D, W1: E x F x D, W2: E x D x F, out: T x D, all dtype
 *     dt. For bf16, products accumulate in fp32 and the hidden activation
 *     act(W1 x) is stored as bf16 between the two products; for fp32 all
 *     arithmetic is fp32. The gate uses the fp32 affinity of the chosen
 *     expert.
 *   mode: BASE_ROUTE_BALANCED (the auction of eq. 2, cfg used; every
 *     expert gets k = T/E tokens), BASE_ROUTE_GIVEN (assign is an input; a
 *     token with an id outside [0,E) or an expert without exactly k tokens
 *     sets stats->status = BASE_ERR_UNBALANCED and out is left unspecified)
 *     or BASE_ROUTE_GREEDY (test-time routing, sec. 3.2.2: each token to its
 *     highest-scoring expert, lowest id on ties, as base_route_greedy; the
 *     expert groups are ragged -- any size, including empty -- and T % E
 *     need not be 0; cfg is ignored).
 *   assign[T]: output (BALANCED, GREEDY) or input (GIVEN).
 *   scores: T x E fp32 output, or NULL (then kept in the workspace).
 *   perm: T int32 output of the expert grouping, or NULL.
 *   stats: device pointer or NULL; prices are written to the workspace.
 *   ws: scratch of base_workspace_bytes(BASE_OP_LAYER, T, E, D, F, dt).
 * Errors: as base_assign_auction (INDIVISIBLE for BALANCED and GIVEN).
 */
int base_layer_forward(const void *h, const void *w, const void *W1,
                       const void *W2, int64_t T, int64_t E, int64_t D,
                       int64_t F, int dt, int act, int mode,
                       base_auction_cfg cfg, int32_t *assign, float *scores,
                       int32_t *perm, void *out, base_auction_stats *stats,
                       void *ws, size_t ws_bytes, base_stream_t stream);

/* Layer variants (base_layer_forward_ex). The pages note two places where
 * the released code differs from eq. 1: it mixes with a convex blend,
 * y = g f(x) + (1 - g) x, g = sigmoid(s[t][a_t]) (page "Paper vs code",
 * mixing equation), and its experts are residual internally; sec. 4.1 makes
 * each expert a stack of feed-forward blocks, each with layer norm, a
 * projection to the hidden width, the activation, a projection back and a
 * residual connection:  x <- x + W2_n act(W1_n LN_n(x)),  n = 0 .. N-1. */
typedef enum { BASE_MIX_RESIDUAL = 0, BASE_MIX_CONVEX = 1 } base_mix;

typedef struct {
    int32_t mix;       /* BASE_MIX_RESIDUAL: y = g f(x) + x (eq. 1);
                          BASE_MIX_CONVEX: y = g f(x) + (1 - g) x */
    int32_t sublayers; /* 0: f(x) = W2 act(W1 x) as in base_layer_forward;
                          N in 1..64: f = N blocks of sec. 4.1 (above) */
    double ln_eps;     /* layer-norm epsilon (>= 0; N >= 1 only) */
    const float *ln_gamma; /* DEVICE, N x E x D fp32 layer-norm scales, or
                              NULL for ones */
    const float *ln_beta;  /* DEVICE, N x E x D fp32 layer-norm shifts, or
                              NULL for zeros */
} base_layer_opts;

/*
 * base_layer_forward_ex -- base_layer_forward with the layer variants above
 * (`opts` is a HOST pointer, NULL = residual mix, plain experts).
 *   With sublayers = N >= 1, W1 is N x E x F x D and W2 is N x E x D x F
 *   (block-major), and each block's layer norm uses the population variance
 *   over D, fp32 statistics, fp32 gamma / beta of the token's expert; the
 *   block input and the normalised rows are stored in dtype dt (bf16: the
 *   running block output is rounded to bf16 after each block). The gate is
 *   the fp32 affinity of the chosen expert, as in base_layer_forward.
 *   Everything else (routing modes, outputs, errors) is as base_layer_forward.
 *   Extra error: INVALID_ARG for an unknown mix, sublayers outside [0, 64],
 *   or ln_eps < 0.
 *   ws: scratch of base_workspace_bytes(BASE_OP_LAYER_EX, T, E, D, F, dt).
 */
int base_layer_forward_ex(const void *h, const void *w, const void *W1,
                          const void *W2, int64_t T, int64_t E, int64_t D,
                          int64_t F, int dt, int act, int mode,
                          base_auction_cfg cfg, int32_t *assign, float *scores,
                          int32_t *perm, void *out, base_auction_stats *stats,
                          const base_layer_opts *opts, void *ws,
                          size_t ws_bytes, base_stream_t stream);

/*
 * base_layer_backward -- gradients of the plain-expert layer (sublayers = 0)
 * for an upstream gradient dy of its output, with the assignment held fixed:
 * the affinities that chose the experts carry no gradient and the centroids
 * learn through the sigmoid gate only (BASE Layers sec. 3.1, learning the
 * centroids through the gate; page "Paper vs code", gradient into routing:
 * the released code scores under no_grad). For token t in expert e = a_t,
 * x = h_t, z = W1_e x, u = act(z), c = W2_e u, g = sigmoid(scores[t][e]):
 *   dW2_e = sum_t g dy u^T,  dz = g (W2_e^T dy) * act'(z),  dW1_e = sum_t dz x^T
 *   dg = dy . c (eq. 1) or dy . (c - x) (convex),  dl = g (1 - g) dg
 *   dh_t = W1_e^T dz + dy (eq. 1) or (1 - g) dy (convex) + dl w_e
 *   dw_e = sum_t dl x
 *   h, w, W1, W2, dt, act: as given to the forward call. assign: the T
 *   expert ids it used (DEVICE; any group sizes, e.g. greedy routing).
 *   scores: DEVICE T x E fp32, the affinities the forward gated with (its
 *   `scores` output). dy: DEVICE T x D (dtype dt), original token order.
 *   opts: HOST, NULL or with sublayers == 0 (mix selects eq. 1 or convex;
 *   layer-norm blocks: base_layer_backward_ex).
 *   Outputs (DEVICE, dtype dt, overwritten): dh T x D (original order),
 *   dw E x D, dW1 E x F x D, dW2 E x D x F. An expert with no token gets
 *   zero gradients.
 *   Precision: bf16 products with fp32 accumulation; the saved
 *   pre-activations, gate * act, dz and the grouped rows of h and dy are
 *   stored as bf16 (fp32 for dt = F32); gate sums in fp32.
 *   stats: device pointer or NULL. Device-side error: stats->status =
 *   BASE_ERR_UNBALANCED when an id of assign lies outside [0, E) (the
 *   gradients are then undefined).
 *   Errors: INVALID_ARG as base_layer_forward (null pointer, sizes, dtype,
 *   act, mix, workspace); UNSUPPORTED for sublayers != 0, D or F above
 *   2^20, and the bf16 layout limits of base_layer_forward (plus dy, dh,
 *   dW1, dW2 16-byte aligned). Phase events (base_set_phase_events): [0] start, [1] after
 *   the grouping and Z, [2] after dz and dl, [3] after dW2, [4] after dW1,
 *   [5] at the end.
 *   ws: scratch of base_workspace_bytes(BASE_OP_LAYER_BWD, T, E, D, F, dt).
 */
int base_layer_backward(const void *h, const void *w, const void *W1,
                        const void *W2, int64_t T, int64_t E, int64_t D,
                        int64_t F, int dt, int act, const int32_t *assign,
                        const float *scores, const void *dy, void *dh,
                        void *dw, void *dW1, void *dW2,
                        base_auction_stats *stats, const base_layer_opts *opts,
                        void *ws, size_t ws_bytes, base_stream_t stream);

/*
 * base_layer_backward_ex -- base_layer_backward for the layer variants of
 * base_layer_forward_ex as well: with opts->sublayers = N >= 1 each expert is
 * N blocks of sec. 4.1 (layer norm, projection up, activation, projection
 * back, residual; W1 N x E x F x D, W2 N x E x D x F, gamma / beta from
 * opts), mixed by opts->mix. The chain rule of those blocks (the
 * assignment fixed, the centroids learning through the gate only, as in
 * base_layer_backward): the blocks' upstream is dx_N = g dy, the gate gets
 * dg = dy . x_N (eq. 1) or dy . (x_N - x_0) (convex), and block n, last
 * first, adds the layer-norm backward of W1_n^T dz_n to the residual path,
 * dz_n = (W2_n^T dx_{n+1}) * act'(z_n).
 *   Outputs as base_layer_backward (dW1, dW2 block-major) plus dgamma,
 *   dbeta: DEVICE N x E x D fp32, the gradients of the layer norms' scales
 *   and shifts (taken at ones / zeros when opts gives none), either may be
 *   NULL. Unused when N = 0.
 *   Precision: the blocks' forward is run again and its state kept for the
 *   way back (each block's input, layer-norm output, Z and act(Z), bf16 for
 *   bf16 workloads); the residual path's gradient accumulates in fp32;
 *   layer-norm statistics fp32. The scratch grows by about
 *   N (2 T F + 2 T D) elements.
 *   Errors: as base_layer_backward, plus INVALID_ARG for sublayers outside
 *   [0, 64] or ln_eps < 0.
 *   ws: scratch of base_workspace_bytes_ex(BASE_OP_LAYER_BWD, T, E, D, F,
 *   dt, N). Phase events with N >= 1: [0] start, [1] after the grouping and
 *   the blocks' forward, [2] after the gate, [3] = [4] after the blocks'
 *   backward, [5] at the end.
 */
int base_layer_backward_ex(const void *h, const void *w, const void *W1,
                           const void *W2, int64_t T, int64_t E, int64_t D,
                           int64_t F, int dt, int act, const int32_t *assign,
                           const float *scores, const void *dy, void *dh,
                           void *dw, void *dW1, void *dW2, float *dgamma,
                           float *dbeta, base_auction_stats *stats,
                           const base_layer_opts *opts, void *ws,
                           size_t ws_bytes, base_stream_t stream);

/* base_workspace_bytes for calls whose scratch depends on the number of
 * layer-norm blocks: BASE_OP_LAYER_BWD with sublayers N (0 ..
 * 64); every other op ignores N. Returns 0 for invalid arguments. */
size_t base_workspace_bytes_ex(int op, int64_t T, int64_t E, int64_t D,
                               int64_t F, int dtype, int sublayers);

/*
 * base_route_greedy_noalloc -- base_route_greedy for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). Same arguments and results as
 * base_route_greedy without ws/ws_bytes: its scratch is a static 8 MiB
 * array in device memory that every GPU the library runs on holds until the
 * process ends (the current device's copy is used; `stream` must belong to
 * that device). The call allocates nothing. Every call on one GPU shares
 * that array, so calls on one GPU must not overlap (use one stream, or
 * order them); overlapping calls race.
 * Errors: those of base_route_greedy, plus UNSUPPORTED when the scratch
 * that T and E need exceeds 8 MiB (about T = 1M tokens at E = 128) and
 * HIP when the array's device address cannot be obtained; nothing is
 * enqueued then.
 */
int base_route_greedy_noalloc(const float *scores, int64_t T, int64_t E,
                              int32_t *assign, int32_t *counts, int32_t *perm,
                              int32_t *offsets, base_stream_t stream);

/*
 * base_set_phase_events -- optional tracing. When `events` is non-NULL, every
 * later base_layer_forward(_ex) and base_layer_backward call on this host
 * thread records n (<= 6) HIP
 * events (hipEvent_t, created by the caller) on its stream: [0] before the
 * affinity product, [1] after it, [2] after routing and grouping, [3] after
 * the first expert product (base_layer_forward_ex with blocks: after the
 * last block's first product), [4] at the end, [5] = [4] (the backward
 * call's six points are listed with it). The
 * caller reads durations with hipEventElapsedTime. NULL turns tracing off.
 * Returns BASE_ERR_INVALID_ARG if n is outside [0, 6].
 */
int base_set_phase_events(void **events, int n);

/*
 * base_set_auction_events -- optional tracing of the auction's parts. When
 * `events` is non-NULL, every later auction on this host thread (in
 * base_assign_auction, base_layer_forward(_ex) and base_layer_backward with
 * BALANCED routing) records, for eps phase p while 4p + 3 < n (n <= 64), HIP
 * events (hipEvent_t, created by the caller) on its stream: [4p] before the
 * phase's parallel rounds, [4p+1] after them, [4p+2] after the setup of the
 * phase's end (C and the holders' slots), [4p+3] after its augmenting paths.
 * NULL turns tracing off. Returns BASE_ERR_INVALID_ARG if n is outside
 * [0, 64].
 */
int base_set_auction_events(void **events, int n);

#ifdef __cplusplus
}
#endif

#endif /* BASE_LAYER_H_ */
