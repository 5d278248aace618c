"""fp64 numpy definitions of the BASE-layer forward -- TEST INFRASTRUCTURE.

Each function writes out the plain definition of one step of the layer as
Lewis et al., "BASE Layers: Simplifying Training of Large, Sparse Models"
describe it. Library primitives used as steps: ``numpy.matmul`` (fp64),
``numpy.argmax``/``argsort``, ``scipy.special.erf``.
"""
from __future__ import annotations

import numpy as np
from scipy.special import erf


def affinity(h: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Token-expert affinities s[t, e] = h_t . w_e (sec. 3.1; fig. 2 scores
    the tokens against the centroids by ``features @ centroids.T``).

    h: T x D, w: E x D, both already the exact fp64 values of the stored
    inputs. Every bf16 x bf16 (and every fp32 x fp32) product is exact in
    fp64, so the only rounding is the fp64 summation.
    """
    h = np.asarray(h, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    return h @ w.T


def sanitize(s: np.ndarray) -> np.ndarray:
    """Replace every NaN/+-inf score with the smallest finite score of the
    matrix, as the released code does before solving (the wikillm page's
    "Paper vs code" list, item on non-finite scores). Raises ValueError when
    no score is finite."""
    s = np.array(s, dtype=np.float64, copy=True)
    fin = np.isfinite(s)
    if fin.all():
        return s
    if not fin.any():
        raise ValueError("no finite score")
    s[~fin] = s[fin].min()
    return s


def greedy_route(s: np.ndarray):
    """Test-time routing (sec. 3.2.2): each token goes to its highest-scoring
    expert; among equal scores the lowest expert index. Returns (a, counts)."""
    s = sanitize(s)
    a = np.argmax(s, axis=1).astype(np.int32)  # first maximum = lowest index
    return a, counts_of(a, s.shape[1])


def counts_of(a: np.ndarray, E: int) -> np.ndarray:
    return np.bincount(np.asarray(a, dtype=np.int64), minlength=E).astype(np.int32)


def canonical_perm(a: np.ndarray, E: int):
    """Tokens grouped by expert (fig. 2's ``sort_by_expert``), ascending token
    id within each group; offsets[e] = first slot of expert e, offsets[E] = T.
    """
    a = np.asarray(a, dtype=np.int64)
    perm = np.argsort(a, kind="stable").astype(np.int32)
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts_of(a, E))
    return perm, offsets


def objective(s: np.ndarray, a: np.ndarray) -> float:
    """Eq. 2's objective: sum_t s[t, a_t]."""
    a = np.asarray(a, dtype=np.int64)
    return float(np.asarray(s, dtype=np.float64)[np.arange(len(a)), a].sum())


def dual_value(s: np.ndarray, p: np.ndarray, k: int) -> float:
    """Dual of eq. 2 as a transportation LP: D(p) = sum_t max_e (s[t,e] - p_e)
    + k * sum_e p_e. By weak duality D(p) >= optimum for every p."""
    s = np.asarray(s, dtype=np.float64)
    p = np.asarray(p, dtype=np.float64)
    return float((s - p[None, :]).max(axis=1).sum() + k * p.sum())


def eps_cs_violation(s: np.ndarray, a: np.ndarray, p: np.ndarray) -> float:
    """max_t [ max_e (s[t,e] - p_e) - (s[t,a_t] - p_{a_t}) ] >= 0. An
    assignment is eps-complementary-slack w.r.t. prices p iff this is <= eps."""
    s = np.asarray(s, dtype=np.float64)
    p = np.asarray(p, dtype=np.float64)
    a = np.asarray(a, dtype=np.int64)
    v = s - p[None, :]
    return float((v.max(axis=1) - v[np.arange(len(a)), a]).max())


def sigmoid(x):
    x = np.asarray(x, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-x))


def gelu(x):
    """GELU in its exact form x * Phi(x) = x/2 * (1 + erf(x / sqrt 2))."""
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + erf(x / np.sqrt(2.0)))


def _act(z, act: str):
    if act == "relu":
        return np.maximum(z, 0.0)
    if act == "gelu":
        return gelu(z)
    raise ValueError(f"unknown activation {act!r}")


def expert_ffn(x: np.ndarray, W1: np.ndarray, W2: np.ndarray, act: str) -> np.ndarray:
    """Position-wise expert f_e(x) = W2 act(W1 x) for each row x: W1 is F x D
    and W2 is D x F (nn.Linear [out, in] layout), no bias, no layer norm, no
    inner residual (the plain two-matrix reading of sec. 4.1's feed-forward
    block)."""
    x = np.asarray(x, dtype=np.float64)
    W1 = np.asarray(W1, dtype=np.float64)
    W2 = np.asarray(W2, dtype=np.float64)
    return _act(x @ W1.T, act) @ W2.T


def layer_forward(h, w, W1, W2, a, act: str, experts=None, s=None):
    """BASE layer output, eq. 1: y_t = sigma(h_t . w_{a_t}) f_{a_t}(h_t) + h_t,
    in the original token order (fig. 2 undoes the expert sort).

    h: T x D, w: E x D, W1: E x F x D (or a callable e -> F x D), W2: E x D x F
    (or callable), a: the assignment (T,). ``experts``: if given, only the
    tokens of these experts are computed and the other rows are NaN. ``s``:
    affinities if already computed (only the chosen entries are used). The
    gate uses the raw affinity of the chosen expert.
    """
    h = np.asarray(h, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    a = np.asarray(a, dtype=np.int64)
    T, D = h.shape
    E = w.shape[0]
    out = np.full((T, D), np.nan)
    todo = range(E) if experts is None else experts
    for e in todo:
        rows = np.nonzero(a == e)[0]
        if rows.size == 0:
            continue
        x = h[rows]
        w1 = W1(e) if callable(W1) else W1[e]
        w2 = W2(e) if callable(W2) else W2[e]
        if s is None:
            g = sigmoid(x @ w[e])
        else:
            g = sigmoid(np.asarray(s, dtype=np.float64)[rows, e])
        out[rows] = g[:, None] * expert_ffn(x, w1, w2, act) + x
    return out


# ---------------------------------------------------------------- layer variants
# The released code mixes with a convex blend, and the paper's experts are
# stacks of feed-forward blocks (sec. 4.1; the "Paper vs code" notes list
# both differences). These definitions serve base_layer_forward_ex.

def layer_norm(x, gamma=None, beta=None, eps: float = 1e-5) -> np.ndarray:
    """Layer norm over the last axis: (x - mean) / sqrt(var + eps) * gamma
    + beta, with the population (biased) variance; gamma = 1 and beta = 0
    when not given. Parity: pinned against torch's layer_norm in fp64 and
    by its invariances (tests/test_oracle_variants.py)."""
    x = np.asarray(x, dtype=np.float64)
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    y = (x - mu) / np.sqrt(var + eps)
    if gamma is not None:
        y = y * np.asarray(gamma, dtype=np.float64)
    if beta is not None:
        y = y + np.asarray(beta, dtype=np.float64)
    return y


def expert_blocks(x, W1s, W2s, act: str, gammas=None, betas=None, ln_eps: float = 1e-5):
    """Sec. 4.1's expert: N feed-forward blocks, each with layer norm, the
    projection up, the activation, the projection back and a residual
    connection: x <- x + W2_n act(W1_n LN_n(x)), n = 0 .. N-1. W1s / W2s /
    gammas / betas are sequences over n (gammas, betas may be None or hold
    None). Parity: pinned against the same block built from torch.nn modules
    in fp64, and by structural cases (zero second projections)."""
    x = np.asarray(x, dtype=np.float64)
    for n in range(len(W1s)):
        g = None if gammas is None else gammas[n]
        b = None if betas is None else betas[n]
        x = x + expert_ffn(layer_norm(x, g, b, ln_eps), W1s[n], W2s[n], act)
    return x


def layer_forward_ex(h, w, W1, W2, a, act: str, mix: str = "residual", sublayers: int = 0,
                     gamma=None, beta=None, ln_eps: float = 1e-5, experts=None, s=None):
    """BASE layer with the variants of the released code and sec. 4.1:

      y_t = g f_{a_t}(h_t) + h_t          (mix "residual", eq. 1)
      y_t = g f_{a_t}(h_t) + (1 - g) h_t  (mix "convex", the released code)

    with g = sigma(h_t . w_{a_t}) (or of ``s``). sublayers = 0: f_e is the
    plain W2 act(W1 x) of ``layer_forward`` (W1, W2 indexed [e] or callables
    e -> matrix); sublayers = N >= 1: f_e = expert_blocks with N blocks (W1,
    W2 indexed [n][e] or callables (n, e) -> matrix; gamma, beta N x E x D or
    None). Rows of experts not in ``experts`` are NaN. Parity: reduces to the
    pinned ``layer_forward`` for residual / 0 sublayers; the convex mix is
    pinned by its gate-to-0 and gate-to-1 limits."""
    h = np.asarray(h, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    a = np.asarray(a, dtype=np.int64)
    T, D = h.shape
    E = w.shape[0]
    out = np.full((T, D), np.nan)
    todo = range(E) if experts is None else experts
    for e in todo:
        rows = np.nonzero(a == e)[0]
        if rows.size == 0:
            continue
        x = h[rows]
        if s is None:
            g = sigmoid(x @ w[e])
        else:
            g = sigmoid(np.asarray(s, dtype=np.float64)[rows, e])
        if sublayers == 0:
            w1 = W1(e) if callable(W1) else W1[e]
            w2 = W2(e) if callable(W2) else W2[e]
            f = expert_ffn(x, w1, w2, act)
        else:
            w1s = [W1(n, e) if callable(W1) else W1[n][e] for n in range(sublayers)]
            w2s = [W2(n, e) if callable(W2) else W2[n][e] for n in range(sublayers)]
            gs = None if gamma is None else [gamma[n][e] for n in range(sublayers)]
            bs = None if beta is None else [beta[n][e] for n in range(sublayers)]
            f = expert_blocks(x, w1s, w2s, act, gs, bs, ln_eps)
        if mix == "residual":
            out[rows] = g[:, None] * f + x
        elif mix == "convex":
            out[rows] = g[:, None] * f + (1.0 - g[:, None]) * x
        else:
            raise ValueError(f"unknown mix {mix!r}")
    return out
