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
(``layer_forward_ex``), by torch.autograd in fp64 over torch.nn modules, and
by structural cases (tests/test_oracle_grad.py).
"""
from __future__ import annotations

import numpy as np
from scipy.special import erf

from .reference import _act, sigmoid


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
