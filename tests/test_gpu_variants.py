"""Parity of base_layer_forward_ex (the released code's convex mix, sec. 4.1's
multi-block experts with layer norm) against the oracle's fp64 layer, given
the routing the GPU chose. Shapes span several 256-row / 256-column tiles
with ragged ends; routing modes balanced, given and greedy (ragged groups).
Tolerances as for the plain layer: 1e-5 (fp32) and 2e-2 (bf16, max-abs
relative), which the bf16 runs meet with the block output rounded to bf16
after every block."""
import numpy as np
import pytest
import torch

import oracle
from balanced_token_expert_amd import api
from balanced_token_expert_amd import workloads as W
from tests.gpu_util import dev_to_f64, f64, rel_err, to_dev

pytestmark = pytest.mark.gpu

CASES = [
    # T, E, D, F, dtype, act, kind, mix, sublayers, ln params
    dict(T=512, E=8, D=64, F=256, dtype="f32", act="relu", kind="iid", mix=1, sub=0, ln=False),
    dict(T=512, E=8, D=64, F=256, dtype="f32", act="relu", kind="iid", mix=1, sub=1, ln=True),
    dict(T=600, E=6, D=72, F=96, dtype="f32", act="gelu", kind="mixture", mix=0, sub=3, ln=True),
    dict(T=1536, E=4, D=320, F=520, dtype="bf16", act="gelu", kind="iid", mix=1, sub=0, ln=False),
    dict(T=1536, E=4, D=320, F=520, dtype="bf16", act="gelu", kind="iid", mix=1, sub=2, ln=True),
    dict(T=1536, E=4, D=320, F=520, dtype="bf16", act="relu", kind="skew", mix=0, sub=2, ln=False),
    dict(T=2048, E=8, D=256, F=512, dtype="bf16", act="gelu", kind="mixture", mix=1, sub=3, ln=True),
    # layer-norm row widths: 2, 4, 8 and 16 register chunks of 8 per lane
    # with ragged chunk tails, and a row too long to keep in registers
    dict(T=512, E=4, D=776, F=64, dtype="bf16", act="relu", kind="iid", mix=1, sub=1, ln=True),
    dict(T=512, E=4, D=1032, F=64, dtype="bf16", act="gelu", kind="iid", mix=0, sub=2, ln=True),
    dict(T=512, E=4, D=2056, F=64, dtype="bf16", act="relu", kind="iid", mix=1, sub=1, ln=False),
    dict(T=256, E=2, D=4104, F=32, dtype="bf16", act="gelu", kind="iid", mix=0, sub=2, ln=True),
    dict(T=256, E=2, D=8200, F=32, dtype="bf16", act="relu", kind="iid", mix=1, sub=1, ln=True),
    # one expert holding every token; one token per expert
    dict(T=300, E=1, D=128, F=96, dtype="bf16", act="gelu", kind="iid", mix=1, sub=2, ln=True),
    dict(T=64, E=64, D=64, F=64, dtype="f32", act="relu", kind="iid", mix=0, sub=1, ln=True),
]
MODES = [api.BASE_ROUTE_BALANCED, api.BASE_ROUTE_GIVEN, api.BASE_ROUTE_GREEDY]


def _setup(c, wid):
    wl = W.custom(c["T"], c["E"], c["D"], c["F"], dtype=c["dtype"], act=c["act"], kind=c["kind"],
                  wid=wid)
    w = W.gen_centroids(wl)
    h = W.gen_tokens(wl, centroids=w)
    n = max(c["sub"], 1)
    if c["sub"] == 0:
        W1 = np.stack([W.gen_w1(wl, e) for e in range(wl.E)])
        W2 = np.stack([W.gen_w2(wl, e) for e in range(wl.E)])
    else:
        W1 = np.stack([np.stack([W.gen_block_w1(wl, b, e) for e in range(wl.E)]) for b in range(n)])
        W2 = np.stack([np.stack([W.gen_block_w2(wl, b, e) for e in range(wl.E)]) for b in range(n)])
    gam = bet = None
    if c["ln"]:
        lnp = [W.gen_ln(wl, b) for b in range(n)]
        gam = np.stack([g for g, _ in lnp])
        bet = np.stack([b for _, b in lnp])
    return wl, h, w, W1, W2, gam, bet


def _ref(wl, c, h, w, W1, W2, gam, bet, a, s32):
    act = wl.act
    mix = "convex" if c["mix"] == api.BASE_MIX_CONVEX else "residual"
    h64, w64 = f64(h, wl.dtype), f64(w, wl.dtype)
    if c["sub"] == 0:
        W1f = lambda e: f64(W1[e], wl.dtype)
        W2f = lambda e: f64(W2[e], wl.dtype)
    else:
        W1f = lambda n, e: f64(W1[n][e], wl.dtype)
        W2f = lambda n, e: f64(W2[n][e], wl.dtype)
    return oracle.layer_forward_ex(h64, w64, W1f, W2f, a, act, mix=mix, sublayers=c["sub"],
                                   gamma=gam, beta=bet, ln_eps=1e-5,
                                   s=s32.astype(np.float64))


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("ci", range(len(CASES)))
def test_layer_variant_parity(ci, mode):
    c = CASES[ci]
    wl, h, w, W1, W2, gam, bet = _setup(c, wid=930 + ci)
    dev = dict(h=to_dev(h, wl.dtype), w=to_dev(w, wl.dtype), W1=to_dev(W1, wl.dtype),
               W2=to_dev(W2, wl.dtype))
    g_d = None if gam is None else torch.from_numpy(gam).cuda()
    b_d = None if bet is None else torch.from_numpy(bet).cuda()
    act = api.BASE_ACT_GELU if wl.act == "gelu" else api.BASE_ACT_RELU
    assign = None
    if mode == api.BASE_ROUTE_GIVEN:
        rng = np.random.default_rng(ci)
        a0 = rng.permutation(np.repeat(np.arange(wl.E), wl.T // wl.E)).astype(np.int32)
        assign = torch.from_numpy(a0).cuda()
    cfg = api.cfg(wl.eps_start, wl.eps_end, wl.eps_factor, max_bids=500 * wl.T)
    r = api.base_layer_forward_ex(dev["h"], dev["w"], dev["W1"], dev["W2"], act, mode, cfg,
                                  mix=c["mix"], sublayers=c["sub"], ln_gamma=g_d, ln_beta=b_d,
                                  ln_eps=1e-5, assign=assign)
    torch.cuda.synchronize()
    assert api.read_stats(r["stats"]).status == 0
    a = r["assign"].cpu().numpy()
    s32 = r["scores"].cpu().numpy()
    counts = np.bincount(a, minlength=wl.E)
    if mode == api.BASE_ROUTE_GREEDY:
        assert (a == oracle.greedy_route(s32.astype(np.float64))[0]).all()
    else:
        assert (counts == wl.T // wl.E).all()
    ref = _ref(wl, c, h, w, W1, W2, gam, bet, a, s32)
    tol = 1e-5 if wl.dtype == "f32" else 2e-2
    err = rel_err(dev_to_f64(r["out"]), ref)
    assert err <= tol, err


def test_layer_ex_default_matches_plain_layer():
    """opts = NULL (residual mix, plain experts) gives base_layer_forward's
    output bit for bit."""
    c = dict(T=1024, E=4, D=256, F=512, dtype="bf16", act="gelu", kind="iid", mix=0, sub=0,
             ln=False)
    wl, h, w, W1, W2, _, _ = _setup(c, wid=950)
    dev = [to_dev(x, wl.dtype) for x in (h, w, W1, W2)]
    a0 = np.random.default_rng(3).permutation(np.repeat(np.arange(wl.E), wl.T // wl.E))
    assign = torch.from_numpy(a0.astype(np.int32)).cuda()
    r0 = api.base_layer_forward(*dev, api.BASE_ACT_GELU, api.BASE_ROUTE_GIVEN, assign=assign)
    r1 = api.base_layer_forward_ex(*dev, api.BASE_ACT_GELU, api.BASE_ROUTE_GIVEN, assign=assign)
    torch.cuda.synchronize()
    assert torch.equal(r0["out"], r1["out"])


def test_blocks_with_zero_second_projections_are_identity():
    """Every block's second projection zero: the expert is the identity, so
    the convex mix returns h exactly and the residual mix g h + h."""
    c = dict(T=1024, E=4, D=256, F=264, dtype="bf16", act="relu", kind="iid", mix=1, sub=2,
             ln=True)
    wl, h, w, W1, W2, gam, bet = _setup(c, wid=951)
    dev = [to_dev(x, wl.dtype) for x in (h, w, W1)]
    z = torch.zeros(W2.shape, dtype=torch.bfloat16, device="cuda")
    g_d, b_d = torch.from_numpy(gam).cuda(), torch.from_numpy(bet).cuda()
    r = api.base_layer_forward_ex(dev[0], dev[1], dev[2], z, api.BASE_ACT_RELU,
                                  api.BASE_ROUTE_BALANCED, mix=api.BASE_MIX_CONVEX, sublayers=2,
                                  ln_gamma=g_d, ln_beta=b_d)
    torch.cuda.synchronize()
    assert api.read_stats(r["stats"]).status == 0
    assert torch.equal(r["out"], dev[0])
