"""fp64 numpy gradients of the BASE layer -- TEST INFRASTRUCTURE.

The layer of eq. 1 (and the released code's convex blend) differentiated by
the chain rule with the assignment held fixed: the affinities that choose the
experts carry no gradient (the released code computes them under no_grad),
and the centroids learn only through the sigmoid gate (BASE Layers sec. 3.1;
the "Paper vs code" notes, item on gradient into routing). For a token t in
expert e with x = h_t, z = W1_e x, u = act(z), c = W2_e u, logit l = x . w_e
and g = sigma(l):

  y = g c + x             (residual, eq. 1)
  y = g c + (1 - g) x     (convex, the released code)

and for an upstream gradient dy of y:

  dc = g dy,  dW2_e += dc u^T,  dz = (W2_e^T dc) * act'(z),  dW1_e += dz x^T
  dg = dy . c  (residual)  or  dy . (c - x)  (convex),  dl = g (1 - g) dg
  dx = W1_e^T dz + dy (residual) or + (1 - g) dy (convex), + dl w_e
  dw_e += dl x

Library primitives used as steps: numpy.matmul (fp64), scipy.special.erf.
Parity: pinned by central finite differences of the pinned forward
(``layer_forward_ex``, with and without layer-norm blocks), by torch.autograd
in fp64 over torch.nn modules (Linear, LayerNorm), and by structural cases
(tests/test_oracle_grad.py).
"""
from __future__ import annotations

import numpy as np
from scipy.special import erf

from .reference import _act, layer_norm, sigmoid


def act_grad(z, act: str) -> np.ndarray:
    """Derivative of the activation: ReLU' = 1 for z > 0 else 0 (0 at the
    kink, as torch takes it); GELU(z) = z Phi(z) gives Phi(z) + z phi(z)."""
    z = np.asarray(z, dtype=np.float64)
    if act == "relu":
        return (z > 0.0).astype(np.float64)
    if act == "gelu":
        phi = np.exp(-0.5 * z * z) / np.sqrt(2.0 * np.pi)
        return 0.5 * (1.0 + erf(z / np.sqrt(2.0))) + z * phi
    raise ValueError(f"unknown activation {act!r}")


def layer_backward(h, w, W1, W2, a, act: str, dy, mix: str = "residual", s=None,
                   experts=None):
    """Gradients of sum(dy * y) for the plain-expert layer (sublayers = 0)
    with respect to h, w, W1 and W2, the assignment a fixed.

    h: T x D, w: E x D, W1: E x F x D (or callable e -> F x D), W2: E x D x F
    (or callable), dy: T x D. ``s``: the affinities the forward gated with
    (only s[t, a_t] is read; the logit's derivative is still h_t . w_e's).
    ``experts``: compute only these experts' tokens and matrices.

    Returns (dh, dw, dW1, dW2): dh T x D and dw E x D with NaN in the rows of
    experts not computed; dW1 / dW2 dicts e -> F x D / D x F.
    """
    h = np.asarray(h, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    a = np.asarray(a, dtype=np.int64)
    T, D = h.shape
    E = w.shape[0]
    if mix not in ("residual", "convex"):
        raise ValueError(f"unknown mix {mix!r}")
    dh = np.full((T, D), np.nan)
    dw = np.full((E, D), np.nan)
    dW1, dW2 = {}, {}
    todo = range(E) if experts is None else experts
    for e in todo:
        w1 = np.asarray(W1(e) if callable(W1) else W1[e], dtype=np.float64)
        w2 = np.asarray(W2(e) if callable(W2) else W2[e], dtype=np.float64)
        rows = np.nonzero(a == e)[0]
        x = h[rows]
        d_y = dy[rows]
        l = x @ w[e] if s is None else np.asarray(s, dtype=np.float64)[rows, e]
        g = sigmoid(l)[:, None]
        z = x @ w1.T
        u = _act(z, act)
        c = u @ w2.T
        dc = g * d_y
        dW2[e] = dc.T @ u
        dz = (dc @ w2) * act_grad(z, act)
        dW1[e] = dz.T @ x
        if mix == "residual":
            dg = (d_y * c).sum(axis=1)
            keep = d_y
        else:
            dg = (d_y * (c - x)).sum(axis=1)
            keep = (1.0 - g) * d_y
        dl = (g[:, 0] * (1.0 - g[:, 0])) * dg
        dh[rows] = dz @ w1 + keep + dl[:, None] * w[e][None, :]
        dw[e] = dl @ x
    return dh, dw, dW1, dW2


def layer_norm_backward(x, gamma, dy, eps: float = 1e-5):
    """Gradients of y = (x - mean) / sqrt(var + eps) * gamma + beta over the
    last axis (population variance) for an upstream dy: returns (dx, dgamma,
    dbeta) with dgamma, dbeta summed over the rows. gamma None means ones.
    With xh the normalised rows and g = dy * gamma:
    dx = rstd (g - mean(g) - xh mean(g xh))."""
    x = np.asarray(x, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    D = x.shape[-1]
    mu = x.mean(axis=-1, keepdims=True)
    rstd = 1.0 / np.sqrt(((x - mu) ** 2).mean(axis=-1, keepdims=True) + eps)
    xh = (x - mu) * rstd
    gm = np.ones(D) if gamma is None else np.asarray(gamma, dtype=np.float64)
    g = dy * gm
    dx = rstd * (g - g.mean(axis=-1, keepdims=True) - xh * (g * xh).mean(axis=-1, keepdims=True))
    return dx, (dy * xh).sum(axis=0), dy.sum(axis=0)


def stored(x, store=None) -> np.ndarray:
    """x as a kernel that computes in fp32 and keeps the result in ``store``
    holds it: None keeps fp64; "f32" rounds to the nearest fp32; "bf16"
    rounds to the nearest fp32 and then to the nearest bfloat16 (8 bits of
    significand, ties to even; overflow goes to infinity)."""
    x = np.asarray(x, dtype=np.float64)
    if store is None:
        return x
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    if store == "f32":
        return x32.astype(np.float64)
    if store != "bf16":
        raise ValueError(f"unknown storage type {store!r}")
    b = x32.view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    return b.astype(np.uint32).view(np.float32).astype(np.float64)


def layer_backward_ex(h, w, W1, W2, a, act: str, dy, mix: str = "residual", sublayers: int = 0,
                      gamma=None, beta=None, ln_eps: float = 1e-5, s=None, experts=None,
                      store=None):
    """Gradients of sum(dy * y) for ``layer_forward_ex`` with the assignment
    fixed. sublayers = 0 is ``layer_backward``. With N >= 1 sec. 4.1 blocks
    per expert (x_{n+1} = x_n + W2_n act(W1_n LN_n(x_n)), f = x_N), the
    upstream of the blocks is dx_N = g dy, dg = dy . x_N (residual) or
    dy . (x_N - x_0) (convex), and each block, last first, adds
    LN_n'(W1_n^T dz_n) to the residual path, dz_n = (W2_n^T dx_{n+1}) act'.

    W1, W2 indexed [n][e] (or callables (n, e)); gamma, beta N x E x D or
    None. Returns (dh, dw, dW1, dW2, dgamma, dbeta): dh, dw as in
    layer_backward; dW1, dW2 dicts (n, e) -> matrix; dgamma, dbeta dicts
    (n, e) -> D-vector, the gradients of each layer norm's scale and shift
    (at gamma = 1, beta = 0 when they are not given).

    ``store`` ("bf16", "f32" or None): the blocks' forward state -- each
    block's input x_n, its layer-norm output and act(z) -- is taken at its
    value after a store in that type (``stored``), the rest in fp64. ReLU's
    derivative is a 0/1 decision on the sign of z; with the state kept in
    bf16, z moves by bf16 rounding and decisions near z = 0 follow the
    precision the state was kept in, so a comparison with a bf16 kernel takes
    them from the same rounded state."""
    if sublayers == 0:
        dh, dw, dW1, dW2 = layer_backward(h, w, W1, W2, a, act, dy, mix=mix, s=s,
                                          experts=experts)
        return dh, dw, dW1, dW2, {}, {}
    h = np.asarray(h, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    a = np.asarray(a, dtype=np.int64)
    T, D = h.shape
    E = w.shape[0]
    if mix not in ("residual", "convex"):
        raise ValueError(f"unknown mix {mix!r}")
    dh = np.full((T, D), np.nan)
    dw = np.full((E, D), np.nan)
    dW1, dW2, dgam, dbet = {}, {}, {}, {}
    todo = range(E) if experts is None else experts
    for e in todo:
        rows = np.nonzero(a == e)[0]
        x0 = h[rows]
        d_y = dy[rows]
        l = x0 @ w[e] if s is None else np.asarray(s, dtype=np.float64)[rows, e]
        g = sigmoid(l)[:, None]
        w1s = [np.asarray(W1(n, e) if callable(W1) else W1[n][e], dtype=np.float64)
               for n in range(sublayers)]
        w2s = [np.asarray(W2(n, e) if callable(W2) else W2[n][e], dtype=np.float64)
               for n in range(sublayers)]
        gs = [None if gamma is None else np.asarray(gamma[n][e], dtype=np.float64)
              for n in range(sublayers)]
        bs = [None if beta is None else np.asarray(beta[n][e], dtype=np.float64)
              for n in range(sublayers)]
        # forward, keeping each block's input
        xs = [stored(x0, store)]
        for n in range(sublayers):
            yn = stored(layer_norm(xs[-1], gs[n], bs[n], ln_eps), store)
            un = stored(_act(yn @ w1s[n].T, act), store)
            xs.append(stored(xs[-1] + un @ w2s[n].T, store))
        xN = xs[-1]
        if mix == "residual":
            dg = (d_y * xN).sum(axis=1)
            keep = d_y
        else:
            dg = (d_y * (xN - x0)).sum(axis=1)
            keep = (1.0 - g) * d_y
        dx = g * d_y
        for n in reversed(range(sublayers)):
            xn = xs[n]
            yn = stored(layer_norm(xn, gs[n], bs[n], ln_eps), store)
            z = yn @ w1s[n].T
            u = stored(_act(z, act), store)
            dW2[(n, e)] = dx.T @ u
            dz = (dx @ w2s[n]) * act_grad(z, act)
            dW1[(n, e)] = dz.T @ yn
            dxn, dgam[(n, e)], dbet[(n, e)] = layer_norm_backward(xn, gs[n], dz @ w1s[n], ln_eps)
            dx = dx + dxn
        dl = (g[:, 0] * (1.0 - g[:, 0])) * dg
        dh[rows] = dx + keep + dl[:, None] * w[e][None, :]
        dw[e] = dl @ x0
    return dh, dw, dW1, dW2, dgam, dbet
