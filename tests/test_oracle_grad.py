"""Pins of the oracle's layer gradients (oracle/grad.py) against things other
than themselves: central finite differences of the pinned forward
(layer_forward_ex), torch.autograd over torch.nn modules in fp64 (an
independent differentiation), and structural cases."""
import numpy as np
import pytest
import torch

import oracle
from oracle.grad import act_grad, layer_backward

RNG = np.random.default_rng(11)


def _inputs(T=12, E=3, D=5, F=7, ragged=False):
    h = RNG.standard_normal((T, D))
    w = RNG.standard_normal((E, D)) * 0.7
    W1 = RNG.standard_normal((E, F, D)) * D ** -0.5
    W2 = RNG.standard_normal((E, D, F)) * F ** -0.5
    if ragged:
        a = RNG.integers(0, E, T)
        a[:E] = np.arange(E)
        a[0] = 0  # keep expert E-1 reachable but the groups uneven
    else:
        a = RNG.permutation(np.repeat(np.arange(E), T // E))
    dy = RNG.standard_normal((T, D))
    return h, w, W1, W2, a, dy


def _loss(h, w, W1, W2, a, act, dy, mix):
    y = oracle.layer_forward_ex(h, w, W1, W2, a, act, mix=mix)
    return float((dy * y).sum())


@pytest.mark.parametrize("mix", ["residual", "convex"])
@pytest.mark.parametrize("act", ["relu", "gelu"])
@pytest.mark.parametrize("ragged", [False, True])
def test_gradients_match_finite_differences(mix, act, ragged):
    h, w, W1, W2, a, dy = _inputs(ragged=ragged)
    dh, dw, dW1, dW2 = layer_backward(h, w, W1, W2, a, act, dy, mix=mix)
    E = w.shape[0]
    num = {"h": np.zeros_like(h), "w": np.zeros_like(w), "W1": np.zeros_like(W1),
           "W2": np.zeros_like(W2)}
    step = 1e-6
    params = {"h": h, "w": w, "W1": W1, "W2": W2}
    for name, arr in params.items():
        for idx in np.ndindex(arr.shape):
            keep = arr[idx]
            arr[idx] = keep + step
            lp = _loss(h, w, W1, W2, a, act, dy, mix)
            arr[idx] = keep - step
            lm = _loss(h, w, W1, W2, a, act, dy, mix)
            arr[idx] = keep
            num[name][idx] = (lp - lm) / (2 * step)
    got = {"h": dh, "w": dw, "W1": np.stack([dW1[e] for e in range(E)]),
           "W2": np.stack([dW2[e] for e in range(E)])}
    for name in params:
        err = np.abs(got[name] - num[name]).max()
        assert err < 1e-7 * max(1.0, np.abs(num[name]).max()), (name, err)


@pytest.mark.parametrize("mix", ["residual", "convex"])
@pytest.mark.parametrize("act", ["relu", "gelu"])
def test_gradients_match_torch_autograd(mix, act):
    """The layer rebuilt from torch.nn.functional pieces in fp64; torch's
    autograd differentiates it independently of the hand-written chain rule."""
    T, E, D, F = 64, 4, 16, 40
    h, w, W1, W2, a, dy = _inputs(T, E, D, F)
    th, tw, tW1, tW2 = (torch.tensor(x, requires_grad=True) for x in (h, w, W1, W2))
    y = torch.zeros(T, D, dtype=torch.float64)
    tact = torch.relu if act == "relu" else torch.nn.functional.gelu
    for e in range(E):
        rows = torch.from_numpy(np.nonzero(a == e)[0])
        x = th[rows]
        g = torch.sigmoid(x @ tw[e])[:, None]
        f = torch.nn.functional.linear(tact(torch.nn.functional.linear(x, tW1[e])), tW2[e])
        y = y.index_put((rows,), g * f + (x if mix == "residual" else (1 - g) * x))
    (y * torch.from_numpy(dy)).sum().backward()
    dh, dw, dW1, dW2 = layer_backward(h, w, W1, W2, a, act, dy, mix=mix)
    assert np.allclose(dh, th.grad.numpy(), rtol=0, atol=1e-12)
    assert np.allclose(dw, tw.grad.numpy(), rtol=0, atol=1e-12)
    assert np.allclose(np.stack([dW1[e] for e in range(E)]), tW1.grad.numpy(), rtol=0, atol=1e-12)
    assert np.allclose(np.stack([dW2[e] for e in range(E)]), tW2.grad.numpy(), rtol=0, atol=1e-12)


def test_act_grad_special_values():
    z = np.array([-3.0, -1e-300, 0.0, 1e-300, 2.0])
    assert np.array_equal(act_grad(z, "relu"), [0.0, 0.0, 0.0, 1.0, 1.0])
    # GELU'(0) = Phi(0) = 1/2; GELU' -> 1 far right, -> 0 far left
    g = act_grad(np.array([0.0, 40.0, -40.0]), "gelu")
    assert g[0] == 0.5 and abs(g[1] - 1.0) < 1e-15 and abs(g[2]) < 1e-15


def test_zero_second_projection():
    """W2 = 0: the expert output and the first matrix's gradient vanish; with
    the residual mix dh = dy exactly and the gate gets nothing; with the
    convex mix the gate still learns from -dy . x."""
    h, w, W1, W2, a, dy = _inputs()
    W2 = np.zeros_like(W2)
    dh, dw, dW1, dW2g = layer_backward(h, w, W1, W2, a, "gelu", dy, mix="residual")
    assert np.array_equal(dh, dy)
    assert not np.any(dw)
    assert all(not np.any(dW1[e]) for e in dW1)
    assert any(np.any(dW2g[e]) for e in dW2g)
    dh, dw, _, _ = layer_backward(h, w, W1, W2, a, "gelu", dy, mix="convex")
    g = oracle.sigmoid((h * w[a]).sum(axis=1))[:, None]
    dl = g[:, 0] * (1 - g[:, 0]) * -(dy * h).sum(axis=1)
    assert np.allclose(dh, (1 - g) * dy + dl[:, None] * w[a], rtol=0, atol=1e-14)


def test_zero_upstream_gradient_and_empty_expert():
    h, w, W1, W2, a, dy = _inputs(T=12, E=4)
    a = np.where(a == 3, 0, a)  # expert 3 gets no token
    dh, dw, dW1, dW2 = layer_backward(h, w, W1, W2, a, "relu", np.zeros_like(dy))
    assert not np.any(dh) and not np.any(dw)
    assert all(not np.any(dW1[e]) and not np.any(dW2[e]) for e in range(4))
    dh, dw, dW1, dW2 = layer_backward(h, w, W1, W2, a, "relu", dy)
    assert not np.any(dw[3]) and not np.any(dW1[3]) and not np.any(dW2[3])


# ---------------------------------------------------------------- sec. 4.1 blocks

def test_layer_norm_backward_matches_torch():
    x = RNG.standard_normal((13, 24)) * 2.0 + 1.0
    g, b = 1.0 + 0.2 * RNG.standard_normal(24), 0.2 * RNG.standard_normal(24)
    dy = RNG.standard_normal((13, 24))
    tx, tg, tb = (torch.tensor(v, requires_grad=True) for v in (x, g, b))
    y = torch.nn.functional.layer_norm(tx, (24,), tg, tb, eps=1e-5)
    (y * torch.from_numpy(dy)).sum().backward()
    dx, dg, db = oracle.layer_norm_backward(x, g, dy, 1e-5)
    assert np.allclose(dx, tx.grad.numpy(), rtol=0, atol=1e-12)
    assert np.allclose(dg, tg.grad.numpy(), rtol=0, atol=1e-12)
    assert np.allclose(db, tb.grad.numpy(), rtol=0, atol=1e-12)


def _block_inputs(T=10, E=2, D=6, F=8, N=2):
    h = RNG.standard_normal((T, D))
    w = RNG.standard_normal((E, D)) * 0.7
    W1 = RNG.standard_normal((N, E, F, D)) * D ** -0.5
    W2 = RNG.standard_normal((N, E, D, F)) * F ** -0.5
    gam = 1.0 + 0.2 * RNG.standard_normal((N, E, D))
    bet = 0.2 * RNG.standard_normal((N, E, D))
    a = RNG.permutation(np.repeat(np.arange(E), T // E))
    dy = RNG.standard_normal((T, D))
    return h, w, W1, W2, gam, bet, a, dy


@pytest.mark.parametrize("mix", ["residual", "convex"])
@pytest.mark.parametrize("act,N", [("relu", 1), ("gelu", 2)])
def test_block_gradients_match_finite_differences(mix, act, N):
    h, w, W1, W2, gam, bet, a, dy = _block_inputs(N=N)
    E = w.shape[0]

    def loss():
        y = oracle.layer_forward_ex(h, w, W1, W2, a, act, mix=mix, sublayers=N, gamma=gam,
                                    beta=bet, ln_eps=1e-5)
        return float((dy * y).sum())

    dh, dw, dW1, dW2, dga, dbe = oracle.layer_backward_ex(h, w, W1, W2, a, act, dy, mix=mix,
                                                          sublayers=N, gamma=gam, beta=bet)
    got = {"h": dh, "w": dw,
           "W1": np.stack([np.stack([dW1[(n, e)] for e in range(E)]) for n in range(N)]),
           "W2": np.stack([np.stack([dW2[(n, e)] for e in range(E)]) for n in range(N)]),
           "gam": np.stack([np.stack([dga[(n, e)] for e in range(E)]) for n in range(N)]),
           "bet": np.stack([np.stack([dbe[(n, e)] for e in range(E)]) for n in range(N)])}
    params = {"h": h, "w": w, "W1": W1, "W2": W2, "gam": gam, "bet": bet}
    step = 1e-6
    for name, arr in params.items():
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            keep = arr[idx]
            arr[idx] = keep + step
            lp = loss()
            arr[idx] = keep - step
            lm = loss()
            arr[idx] = keep
            num[idx] = (lp - lm) / (2 * step)
        err = np.abs(got[name] - num).max()
        assert err < 2e-7 * max(1.0, np.abs(num).max()), (name, err)


@pytest.mark.parametrize("mix", ["residual", "convex"])
def test_block_gradients_match_torch_modules(mix):
    """Two blocks built from torch.nn.LayerNorm / Linear / GELU per expert."""
    T, E, D, F, N = 32, 2, 12, 20, 2
    h, w, W1, W2, gam, bet, a, dy = _block_inputs(T, E, D, F, N)
    th, tw = torch.tensor(h, requires_grad=True), torch.tensor(w, requires_grad=True)
    mods = {}
    for n in range(N):
        for e in range(E):
            ln = torch.nn.LayerNorm(D, eps=1e-5, dtype=torch.float64)
            up = torch.nn.Linear(D, F, bias=False, dtype=torch.float64)
            down = torch.nn.Linear(F, D, bias=False, dtype=torch.float64)
            with torch.no_grad():
                ln.weight.copy_(torch.from_numpy(gam[n, e]))
                ln.bias.copy_(torch.from_numpy(bet[n, e]))
                up.weight.copy_(torch.from_numpy(W1[n, e]))
                down.weight.copy_(torch.from_numpy(W2[n, e]))
            mods[(n, e)] = (ln, up, down)
    y = torch.zeros(T, D, dtype=torch.float64)
    for e in range(E):
        rows = torch.from_numpy(np.nonzero(a == e)[0])
        x0 = th[rows]
        g = torch.sigmoid(x0 @ tw[e])[:, None]
        x = x0
        for n in range(N):
            ln, up, down = mods[(n, e)]
            x = x + down(torch.nn.functional.gelu(up(ln(x))))
        y = y.index_put((rows,), g * x + (x0 if mix == "residual" else (1 - g) * x0))
    (y * torch.from_numpy(dy)).sum().backward()
    dh, dw, dW1, dW2, dga, dbe = oracle.layer_backward_ex(h, w, W1, W2, a, "gelu", dy, mix=mix,
                                                          sublayers=N, gamma=gam, beta=bet)
    assert np.allclose(dh, th.grad.numpy(), rtol=0, atol=1e-11)
    assert np.allclose(dw, tw.grad.numpy(), rtol=0, atol=1e-11)
    for (n, e), (ln, up, down) in mods.items():
        assert np.allclose(dW1[(n, e)], up.weight.grad.numpy(), rtol=0, atol=1e-11)
        assert np.allclose(dW2[(n, e)], down.weight.grad.numpy(), rtol=0, atol=1e-11)
        assert np.allclose(dga[(n, e)], ln.weight.grad.numpy(), rtol=0, atol=1e-11)
        assert np.allclose(dbe[(n, e)], ln.bias.grad.numpy(), rtol=0, atol=1e-11)


def test_stored_matches_torch_casts():
    """``stored`` against torch's own fp32 and bfloat16 conversions: random
    magnitudes over many binades, exact ties of both parities, values just
    off a tie, tiny and huge values (overflow to infinity)."""
    rng = np.random.default_rng(11)
    x = rng.standard_normal(20000) * np.exp2(rng.integers(-60, 60, 20000))
    ties = (np.arange(1, 2001, dtype=np.float64) * 2 + 1) * 2.0 ** -8  # odd multiples of 2^-8
    near = np.concatenate([ties * (1 + 2.0 ** -20), ties * (1 - 2.0 ** -20)])
    special = np.array([0.0, -0.0, 1e-40, -1e-40, 3.4e38, -3.4e38, 65504.0, 1.0 + 2.0 ** -8])
    x = np.concatenate([x, ties, -ties, near, special])
    t = torch.from_numpy(x)
    want_f32 = t.to(torch.float32).to(torch.float64).numpy()
    want_bf16 = t.to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(oracle.stored(x, "f32"), want_f32)
    assert np.array_equal(oracle.stored(x, "bf16"), want_bf16)
    assert oracle.stored(x) is not None and np.array_equal(oracle.stored(x), x)


@pytest.mark.parametrize("mix", ["residual", "convex"])
@pytest.mark.parametrize("act", ["relu", "gelu"])
def test_stored_block_gradients_match_straight_through_torch(mix, act):
    """store="bf16": torch.nn modules with each block's input, layer-norm
    output and activation replaced in the forward by its bfloat16 value
    (torch's cast) while the gradient passes through unchanged -- the
    gradient of the blocks evaluated at the rounded state."""
    T, E, D, F, N = 32, 2, 12, 20, 2
    h, w, W1, W2, gam, bet, a, dy = _block_inputs(T, E, D, F, N)

    def st(x):
        r = x.detach().to(torch.float32).to(torch.bfloat16).to(torch.float64)
        return x + (r - x).detach()

    fn = torch.nn.functional.relu if act == "relu" else torch.nn.functional.gelu
    th, tw = torch.tensor(h, requires_grad=True), torch.tensor(w, requires_grad=True)
    mods = {}
    for n in range(N):
        for e in range(E):
            ln = torch.nn.LayerNorm(D, eps=1e-5, dtype=torch.float64)
            up = torch.nn.Linear(D, F, bias=False, dtype=torch.float64)
            down = torch.nn.Linear(F, D, bias=False, dtype=torch.float64)
            with torch.no_grad():
                ln.weight.copy_(torch.from_numpy(gam[n, e]))
                ln.bias.copy_(torch.from_numpy(bet[n, e]))
                up.weight.copy_(torch.from_numpy(W1[n, e]))
                down.weight.copy_(torch.from_numpy(W2[n, e]))
            mods[(n, e)] = (ln, up, down)
    y = torch.zeros(T, D, dtype=torch.float64)
    for e in range(E):
        rows = torch.from_numpy(np.nonzero(a == e)[0])
        x0 = th[rows]
        g = torch.sigmoid(x0 @ tw[e])[:, None]
        x = st(x0)
        for n in range(N):
            ln, up, down = mods[(n, e)]
            x = st(x + down(st(fn(up(st(ln(x)))))))
        y = y.index_put((rows,), g * x + (x0 if mix == "residual" else (1 - g) * x0))
    (y * torch.from_numpy(dy)).sum().backward()
    dh, dw, dW1, dW2, dga, dbe = oracle.layer_backward_ex(h, w, W1, W2, a, act, dy, mix=mix,
                                                          sublayers=N, gamma=gam, beta=bet,
                                                          store="bf16")
    assert np.allclose(dh, th.grad.numpy(), rtol=0, atol=1e-11)
    assert np.allclose(dw, tw.grad.numpy(), rtol=0, atol=1e-11)
    for (n, e), (ln, up, down) in mods.items():
        assert np.allclose(dW1[(n, e)], up.weight.grad.numpy(), rtol=0, atol=1e-11)
        assert np.allclose(dW2[(n, e)], down.weight.grad.numpy(), rtol=0, atol=1e-11)
        assert np.allclose(dga[(n, e)], ln.weight.grad.numpy(), rtol=0, atol=1e-11)
        assert np.allclose(dbe[(n, e)], ln.bias.grad.numpy(), rtol=0, atol=1e-11)
    # and the rounding does move the result (the pin is not vacuous)
    dh0 = oracle.layer_backward_ex(h, w, W1, W2, a, act, dy, mix=mix, sublayers=N, gamma=gam,
                                   beta=bet)[0]
    assert np.abs(dh0 - dh).max() > 1e-6
