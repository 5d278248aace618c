/*
 * CPU oracle for the BASE layer's balanced assignment -- TEST INFRASTRUCTURE.
 *
 * Plain, slow, single-threaded C in fp64. Only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg load this library; the GPU
 * library never links or calls it, and it shares no code with the GPU path.
 *
 * The problem (Lewis et al., "BASE Layers", sec. 3.2.1, eq. 2): given scores
 * s[t][e] (T tokens x E experts, row-major) choose a_t in [0,E) maximising
 * sum_t s[t][a_t] subject to every expert receiving exactly k = T/E tokens.
 *
 *  orc_auction       token-side auction with eps-scaling (Gauss-Seidel: one
 *                    bidder at a time, FIFO queue). The paper solves eq. 2 by
 *                    an auction (sec. 3.2.1, appendix fig. 9, where experts
 *                    bid); here tokens bid for expert slots, per-expert
 *                    capacity k, Bertsekas' eps-scaling between phases.
 *  orc_hungarian     exact: Hungarian method on the T x T matrix in which
 *                    expert e owns the k columns e*k .. e*k+k-1.
 *  orc_cycle_cancel  exact: from any balanced assignment, cancel negative
 *                    cycles of the expert exchange graph (min-cost-flow
 *                    optimality), until none is left.
 *  orc_min_cycle     the minimum cycle cost of that exchange graph: >= 0 iff
 *                    the assignment is optimal, and then equal to the gap
 *                    between the optimum and the second-best balanced
 *                    assignment (0 means several optima tie).
 *
 * Return codes: 0 ok, -1 invalid argument, -2 T % E != 0, -5 bid cap hit,
 * -7 out of memory.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_EINVAL (-1)
#define ORC_EINDIV (-2)
#define ORC_ECAP (-5)
#define ORC_ENOMEM (-7)

/* ------------------------------------------------------------------ auction
 * Each expert e keeps the set of tokens it currently holds, with the bid each
 * paid, in a binary heap whose top is the holder to evict next: the lowest
 * bid, and among equal bids the higher token id. The price a new bidder must
 * beat is pi_e: the floor p_e while e holds fewer than k tokens, else the
 * lowest bid it holds.
 */
typedef struct {
    double bid;
    int32_t tok;
} held_t;

/* a is evicted before b */
static int evict_before(const held_t *a, const held_t *b) {
    if (a->bid != b->bid) return a->bid < b->bid;
    return a->tok > b->tok;
}

static void heap_push(held_t *h, int *n, held_t x) {
    int i = (*n)++;
    h[i] = x;
    while (i > 0) {
        int p = (i - 1) / 2;
        if (!evict_before(&h[i], &h[p])) break;
        held_t tmp = h[i]; h[i] = h[p]; h[p] = tmp;
        i = p;
    }
}

static held_t heap_pop(held_t *h, int *n) {
    held_t top = h[0];
    h[0] = h[--(*n)];
    int i = 0;
    for (;;) {
        int l = 2 * i + 1, r = l + 1, m = i;
        if (l < *n && evict_before(&h[l], &h[m])) m = l;
        if (r < *n && evict_before(&h[r], &h[m])) m = r;
        if (m == i) break;
        held_t tmp = h[i]; h[i] = h[m]; h[m] = tmp;
        i = m;
    }
    return top;
}

/*
 * s: T x E fp64 scores, already free of NaN/inf.
 * eps schedule: eps_start, then max(eps/eps_factor, eps_end), ... , eps_end.
 * Outputs: assign[T], prices[E] (final p_e = lowest bid each expert holds),
 * bids_per_phase[max_phases], *phases. max_bids <= 0 means no cap.
 */
int orc_auction(const double *s, int T, int E, double eps_start, double eps_end,
                double eps_factor, int64_t max_bids, int32_t *assign,
                double *prices, int64_t *bids_per_phase, int max_phases,
                int *phases) {
    if (!s || !assign || !prices || T <= 0 || E <= 0 || E > T) return ORC_EINVAL;
    if (T % E) return ORC_EINDIV;
    if (!(eps_end > 0) || !(eps_start >= eps_end) || !(eps_factor > 1)) return ORC_EINVAL;
    const int k = T / E;
    held_t *heap = (held_t *)malloc(sizeof(held_t) * (size_t)E * (size_t)(k + 1));
    int *cnt = (int *)calloc((size_t)E, sizeof(int));
    double *pi = (double *)malloc(sizeof(double) * (size_t)E);
    int32_t *queue = (int32_t *)malloc(sizeof(int32_t) * (size_t)T);
    if (!heap || !cnt || !pi || !queue) {
        free(heap); free(cnt); free(pi); free(queue);
        return ORC_ENOMEM;
    }
    for (int e = 0; e < E; ++e) prices[e] = 0.0;
    int64_t total = 0;
    int nph = 0;
    int rc = ORC_OK;
    double eps = eps_start;
    for (;;) {
        /* new phase: every expert empty, every token queued in id order */
        for (int e = 0; e < E; ++e) { cnt[e] = 0; pi[e] = prices[e]; }
        for (int t = 0; t < T; ++t) { queue[t] = t; assign[t] = -1; }
        int64_t head = 0, tail = T; /* FIFO over a ring of size T */
        int64_t phase_bids = 0;
        while (head < tail) {
            int t = queue[head % T];
            ++head;
            const double *row = s + (size_t)t * E;
            /* best and second-best value of s[t][e] - pi_e */
            int b1 = 0;
            double v1 = row[0] - pi[0];
            for (int e = 1; e < E; ++e) {
                double v = row[e] - pi[e];
                if (v > v1) { v1 = v; b1 = e; }
            }
            double v2 = v1;
            if (E > 1) {
                v2 = -INFINITY;
                for (int e = 0; e < E; ++e) {
                    if (e == b1) continue;
                    double v = row[e] - pi[e];
                    if (v > v2) v2 = v;
                }
            }
            double beta = pi[b1] + (v1 - v2) + eps;
            held_t *hb = heap + (size_t)b1 * (size_t)(k + 1);
            held_t x = {beta, t};
            heap_push(hb, &cnt[b1], x);
            assign[t] = b1;
            if (cnt[b1] > k) {
                held_t out = heap_pop(hb, &cnt[b1]);
                assign[out.tok] = -1;
                queue[tail % T] = out.tok;
                ++tail;
            }
            pi[b1] = (cnt[b1] == k) ? hb[0].bid : prices[b1];
            ++phase_bids;
            ++total;
            if (max_bids > 0 && total >= max_bids && head < tail) { rc = ORC_ECAP; break; }
        }
        if (nph < max_phases && bids_per_phase) bids_per_phase[nph] = phase_bids;
        ++nph;
        if (rc != ORC_OK) break;
        /* every expert is full: its price becomes the lowest bid it holds */
        for (int e = 0; e < E; ++e) prices[e] = heap[(size_t)e * (size_t)(k + 1)].bid;
        if (eps <= eps_end) break;
        eps = eps / eps_factor;
        if (eps < eps_end) eps = eps_end;
    }
    if (phases) *phases = nph;
    free(heap); free(cnt); free(pi); free(queue);
    return rc;
}

/* ---------------------------------------------------------------- Hungarian
 * Minimise sum cost[i][col(i)] over permutations, cost[i][j] = -s[i][j / k].
 * Shortest augmenting paths with row/column potentials u, v; O(T^3).
 * Rows and columns are 1-based inside, column 0 is the virtual start.
 */
int orc_hungarian(const double *s, int T, int E, int32_t *assign) {
    if (!s || !assign || T <= 0 || E <= 0 || E > T) return ORC_EINVAL;
    if (T % E) return ORC_EINDIV;
    const int n = T, k = T / E;
    double *u = (double *)calloc((size_t)n + 1, sizeof(double));
    double *v = (double *)calloc((size_t)n + 1, sizeof(double));
    double *minv = (double *)malloc(sizeof(double) * ((size_t)n + 1));
    int *match = (int *)calloc((size_t)n + 1, sizeof(int)); /* column -> row */
    int *way = (int *)calloc((size_t)n + 1, sizeof(int));
    char *used = (char *)malloc((size_t)n + 1);
    if (!u || !v || !minv || !match || !way || !used) {
        free(u); free(v); free(minv); free(match); free(way); free(used);
        return ORC_ENOMEM;
    }
    for (int i = 1; i <= n; ++i) {
        match[0] = i;
        int j0 = 0;
        for (int j = 0; j <= n; ++j) { minv[j] = INFINITY; used[j] = 0; }
        do {
            used[j0] = 1;
            int i0 = match[j0], j1 = 0;
            double delta = INFINITY;
            const double *row = s + (size_t)(i0 - 1) * E;
            for (int j = 1; j <= n; ++j) {
                if (used[j]) continue;
                double cur = -row[(j - 1) / k] - u[i0] - v[j];
                if (cur < minv[j]) { minv[j] = cur; way[j] = j0; }
                if (minv[j] < delta) { delta = minv[j]; j1 = j; }
            }
            for (int j = 0; j <= n; ++j) {
                if (used[j]) { u[match[j]] += delta; v[j] -= delta; }
                else minv[j] -= delta;
            }
            j0 = j1;
        } while (match[j0] != 0);
        do {
            int j1 = way[j0];
            match[j0] = match[j1];
            j0 = j1;
        } while (j0);
    }
    for (int j = 1; j <= n; ++j) assign[match[j] - 1] = (j - 1) / k;
    free(u); free(v); free(minv); free(match); free(way); free(used);
    return ORC_OK;
}

/* ------------------------------------------------------ exchange graph
 * For a balanced assignment a, moving one token t from expert x to expert y
 * changes the objective by s[t][y] - s[t][x]. The exchange graph has an edge
 * x -> y of cost c[x][y] = min over t held by x of (s[t][x] - s[t][y]), the
 * cheapest way to push one token out of x into y. A cycle of it moves one
 * token along each edge and keeps every expert's count; its cost is the
 * objective lost. (The residual graph of the transportation problem,
 * contracted over tokens: a cycle there visits each expert once, so uses
 * distinct tokens.)
 */
static void build_exchange(const double *s, int T, int E, const int32_t *a,
                           double *c, int32_t *tok) {
    for (size_t i = 0; i < (size_t)E * E; ++i) { c[i] = INFINITY; tok[i] = -1; }
    for (int t = 0; t < T; ++t) {
        int x = a[t];
        const double *row = s + (size_t)t * E;
        for (int y = 0; y < E; ++y) {
            if (y == x) continue;
            double d = row[x] - row[y];
            size_t i = (size_t)x * E + y;
            if (d < c[i]) { c[i] = d; tok[i] = t; }
        }
    }
}

static int check_balanced(const int32_t *a, int T, int E) {
    int k = T / E;
    int *cnt = (int *)calloc((size_t)E, sizeof(int));
    if (!cnt) return ORC_ENOMEM;
    int ok = 1;
    for (int t = 0; t < T; ++t) {
        if (a[t] < 0 || a[t] >= E) { ok = 0; break; }
        cnt[a[t]]++;
    }
    for (int e = 0; ok && e < E; ++e) if (cnt[e] != k) ok = 0;
    free(cnt);
    return ok ? ORC_OK : ORC_EINVAL;
}

/*
 * Start from a_in (balanced), cancel negative cycles until the exchange graph
 * has none below -tol. Cycles are found with Bellman-Ford from a virtual
 * source. Writes the optimum to a_out; *cancelled = cycles cancelled.
 */
int orc_cycle_cancel(const double *s, int T, int E, const int32_t *a_in,
                     int32_t *a_out, double tol, int max_iter, int *cancelled) {
    if (!s || !a_in || !a_out || T <= 0 || E <= 0 || E > T) return ORC_EINVAL;
    if (T % E) return ORC_EINDIV;
    int rc = check_balanced(a_in, T, E);
    if (rc) return rc;
    memcpy(a_out, a_in, sizeof(int32_t) * (size_t)T);
    if (cancelled) *cancelled = 0;
    if (E == 1) return ORC_OK;
    double *c = (double *)malloc(sizeof(double) * (size_t)E * E);
    int32_t *tok = (int32_t *)malloc(sizeof(int32_t) * (size_t)E * E);
    double *dist = (double *)malloc(sizeof(double) * (size_t)E);
    int *pred = (int *)malloc(sizeof(int) * (size_t)E);
    int *cyc = (int *)malloc(sizeof(int) * (size_t)E);
    char *seen = (char *)malloc((size_t)E);
    int32_t *moved = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
    if (!c || !tok || !dist || !pred || !cyc || !seen || !moved) {
        free(c); free(tok); free(dist); free(pred); free(cyc); free(seen); free(moved);
        return ORC_ENOMEM;
    }
    int iter = 0;
    for (; iter < max_iter; ++iter) {
        build_exchange(s, T, E, a_out, c, tok);
        for (int x = 0; x < E; ++x) { dist[x] = 0.0; pred[x] = -1; }
        int last = -1;
        for (int pass = 0; pass <= E; ++pass) {
            last = -1;
            for (int x = 0; x < E; ++x) {
                for (int y = 0; y < E; ++y) {
                    double w = c[(size_t)x * E + y];
                    if (!(w < INFINITY)) continue;
                    if (dist[x] + w < dist[y] - tol) {
                        dist[y] = dist[x] + w;
                        pred[y] = x;
                        last = y;
                    }
                }
            }
            if (last < 0) break;
        }
        if (last < 0) break; /* no negative cycle: optimal */
        /* walk back E steps to land on the cycle, then collect it */
        int x = last;
        for (int i = 0; i < E && x >= 0; ++i) x = pred[x];
        if (x < 0) break;
        memset(seen, 0, (size_t)E);
        int len = 0, y = x;
        while (y >= 0 && !seen[y]) { seen[y] = 1; cyc[len++] = y; y = pred[y]; }
        if (y != x) break; /* not a closed cycle: numerical corner, stop */
        /* cyc lists the cycle backwards: pred[cyc[i]] = cyc[i+1] */
        double cost = 0.0;
        for (int i = 0; i < len; ++i) {
            int to = cyc[i], from = cyc[(i + 1) % len];
            cost += c[(size_t)from * E + to];
        }
        if (!(cost < -tol)) break;
        for (int i = 0; i < len; ++i) {
            int to = cyc[i], from = cyc[(i + 1) % len];
            moved[i] = tok[(size_t)from * E + to];
        }
        for (int i = 0; i < len; ++i) a_out[moved[i]] = cyc[i];
    }
    if (cancelled) *cancelled = iter;
    free(c); free(tok); free(dist); free(pred); free(cyc); free(seen); free(moved);
    return check_balanced(a_out, T, E);
}

/*
 * Minimum cost over cycles of the exchange graph of a (Floyd-Warshall with
 * the diagonal started at +inf, so dist[x][x] ends as the shortest cycle
 * through x). Writes it to *gap; +inf when E == 1 (no other assignment).
 */
int orc_min_cycle(const double *s, int T, int E, const int32_t *a, double *gap) {
    if (!s || !a || !gap || T <= 0 || E <= 0 || E > T) return ORC_EINVAL;
    if (T % E) return ORC_EINDIV;
    int rc = check_balanced(a, T, E);
    if (rc) return rc;
    if (E == 1) { *gap = INFINITY; return ORC_OK; }
    double *c = (double *)malloc(sizeof(double) * (size_t)E * E);
    int32_t *tok = (int32_t *)malloc(sizeof(int32_t) * (size_t)E * E);
    if (!c || !tok) { free(c); free(tok); return ORC_ENOMEM; }
    build_exchange(s, T, E, a, c, tok);
    for (int m = 0; m < E; ++m)
        for (int x = 0; x < E; ++x) {
            double dxm = c[(size_t)x * E + m];
            if (!(dxm < INFINITY)) continue;
            for (int y = 0; y < E; ++y) {
                double alt = dxm + c[(size_t)m * E + y];
                if (alt < c[(size_t)x * E + y]) c[(size_t)x * E + y] = alt;
            }
        }
    double g = INFINITY;
    for (int x = 0; x < E; ++x) if (c[(size_t)x * E + x] < g) g = c[(size_t)x * E + x];
    *gap = g;
    free(c); free(tok);
    return ORC_OK;
}
