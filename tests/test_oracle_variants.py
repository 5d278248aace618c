"""Pins of the oracle's layer variants (released code's convex mix, sec. 4.1's
multi-block experts with layer norm) against things other than themselves:
torch's fp64 layer norm and nn modules (independent library routines), the
invariances of layer norm, the reduction to the already pinned eq. 1 layer,
the limits of the convex blend, and structural cases."""
import numpy as np
import pytest
import torch

import oracle

RNG = np.random.default_rng(7)


def _rand(*shape, scale=1.0):
    return RNG.standard_normal(shape) * scale


def test_layer_norm_matches_torch():
    x = _rand(37, 48, scale=3.0) + 5.0
    g, b = 1.0 + 0.1 * _rand(48), 0.1 * _rand(48)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(x), (48,), torch.from_numpy(g),
                                         torch.from_numpy(b), eps=1e-5).numpy()
    assert np.allclose(oracle.layer_norm(x, g, b, 1e-5), ref, rtol=0, atol=1e-12)


def test_layer_norm_invariances():
    x = _rand(20, 64)
    y = oracle.layer_norm(x, eps=0.0)
    assert np.allclose(y.mean(axis=1), 0.0, atol=1e-12)
    assert np.allclose((y ** 2).mean(axis=1), 1.0, atol=1e-12)
    # a positive scale and a shift of each row leave it unchanged
    z = oracle.layer_norm(2.5 * x + 7.0, eps=0.0)
    assert np.allclose(z, y, atol=1e-12)
    # gamma and beta act elementwise after the normalisation
    g, b = _rand(64), _rand(64)
    assert np.allclose(oracle.layer_norm(x, g, b, eps=0.0), y * g + b, atol=1e-12)


@pytest.mark.parametrize("act", ["relu", "gelu"])
def test_block_matches_torch_modules(act):
    """One sec. 4.1 block (layer norm, projection up, activation, projection
    back, residual) built from torch.nn modules in fp64."""
    D, F = 24, 96
    x = _rand(30, D)
    ln = torch.nn.LayerNorm(D, eps=1e-5, dtype=torch.float64)
    up = torch.nn.Linear(D, F, bias=False, dtype=torch.float64)
    down = torch.nn.Linear(F, D, bias=False, dtype=torch.float64)
    with torch.no_grad():
        ln.weight.copy_(torch.from_numpy(1.0 + 0.2 * _rand(D)))
        ln.bias.copy_(torch.from_numpy(0.2 * _rand(D)))
        up.weight.copy_(torch.from_numpy(_rand(F, D, scale=D ** -0.5)))
        down.weight.copy_(torch.from_numpy(_rand(D, F, scale=F ** -0.5)))
        tact = torch.nn.ReLU() if act == "relu" else torch.nn.GELU(approximate="none")
        xt = torch.from_numpy(x)
        ref = (xt + down(tact(up(ln(xt))))).numpy()
    got = oracle.expert_blocks(x, [up.weight.detach().numpy()], [down.weight.detach().numpy()], act,
                               [ln.weight.detach().numpy()], [ln.bias.detach().numpy()], 1e-5)
    assert np.allclose(got, ref, rtol=0, atol=1e-12)


def test_blocks_structural():
    D, F = 16, 40
    x = _rand(9, D)
    W1 = [_rand(F, D, scale=0.3) for _ in range(3)]
    W2 = [_rand(D, F, scale=0.3) for _ in range(3)]
    zero = np.zeros((D, F))
    # every second projection zero: the stack is the identity
    assert np.allclose(oracle.expert_blocks(x, W1, [zero] * 3, "relu"), x, atol=0)
    # a zero second projection in the last block leaves the first two
    two = oracle.expert_blocks(x, W1[:2], W2[:2], "gelu")
    assert np.allclose(oracle.expert_blocks(x, W1, W2[:2] + [zero], "gelu"), two, atol=1e-14)
    assert not np.allclose(two, x)


def _layer_inputs(T=24, E=4, D=16, F=32, N=2):
    h = _rand(T, D)
    w = _rand(E, D, scale=D ** -0.5)
    a = RNG.permutation(np.repeat(np.arange(E), T // E))
    W1 = _rand(N, E, F, D, scale=D ** -0.5)
    W2 = _rand(N, E, D, F, scale=F ** -0.5)
    return h, w, a, W1, W2


def test_residual_plain_reduces_to_eq1_layer():
    h, w, a, W1, W2 = _layer_inputs(N=1)
    ref = oracle.layer_forward(h, w, W1[0], W2[0], a, "gelu")
    got = oracle.layer_forward_ex(h, w, W1[0], W2[0], a, "gelu", mix="residual", sublayers=0)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("sub", [0, 1, 2])
def test_convex_mix_limits(sub):
    """Gate -> 1 gives the expert output, gate -> 0 the input (sigma of
    +-60 is 1 and ~1e-26 in fp64)."""
    h, w, a, W1, W2 = _layer_inputs()
    T, E = h.shape[0], w.shape[0]
    W1s = W1[0] if sub == 0 else W1[:sub]
    W2s = W2[0] if sub == 0 else W2[:sub]
    for sval, want_expert in ((60.0, True), (-60.0, False)):
        s = np.full((T, E), sval)
        y = oracle.layer_forward_ex(h, w, W1s, W2s, a, "relu", mix="convex", sublayers=sub, s=s)
        if want_expert:
            for e in range(E):
                rows = a == e
                f = (oracle.expert_ffn(h[rows], W1s[e], W2s[e], "relu") if sub == 0 else
                     oracle.expert_blocks(h[rows], [W1s[n][e] for n in range(sub)],
                                          [W2s[n][e] for n in range(sub)], "relu"))
                assert np.allclose(y[rows], f, atol=1e-12)
        else:
            assert np.allclose(y, h, atol=1e-12)


def test_convex_one_block_is_gated_residual():
    """With one residual block, g (x + F(LN x)) + (1 - g) x = x + g F(LN x):
    the convex blend of a residual block is eq. 1 with layer norm inside."""
    h, w, a, W1, W2 = _layer_inputs(N=1)
    y = oracle.layer_forward_ex(h, w, W1, W2, a, "gelu", mix="convex", sublayers=1)
    for e in range(w.shape[0]):
        rows = a == e
        g = oracle.sigmoid(h[rows] @ w[e])[:, None]
        f = oracle.expert_ffn(oracle.layer_norm(h[rows]), W1[0][e], W2[0][e], "gelu")
        assert np.allclose(y[rows], h[rows] + g * f, atol=1e-12)


@pytest.mark.parametrize("sub", [0, 2])
def test_residual_mix_limits(sub):
    """Residual mix: gate -> 1 gives f(x) + x, gate -> 0 gives x."""
    h, w, a, W1, W2 = _layer_inputs()
    T, E = h.shape[0], w.shape[0]
    W1s = W1[0] if sub == 0 else W1[:sub]
    W2s = W2[0] if sub == 0 else W2[:sub]
    hi = oracle.layer_forward_ex(h, w, W1s, W2s, a, "gelu", mix="residual", sublayers=sub,
                                 s=np.full((T, E), 60.0))
    lo = oracle.layer_forward_ex(h, w, W1s, W2s, a, "gelu", mix="residual", sublayers=sub,
                                 s=np.full((T, E), -60.0))
    assert np.allclose(lo, h, atol=1e-12)
    for e in range(E):
        rows = a == e
        f = (oracle.expert_ffn(h[rows], W1s[e], W2s[e], "gelu") if sub == 0 else
             oracle.expert_blocks(h[rows], [W1s[n][e] for n in range(sub)],
                                  [W2s[n][e] for n in range(sub)], "gelu"))
        assert np.allclose(hi[rows], f + h[rows], atol=1e-12)
