"""Parity of base_layer_backward against the oracle's fp64 gradients
(oracle.layer_backward), with the gate taken from the scores the GPU's
affinity product gave. Shapes span several 256-wide tiles with ragged ends
in every dimension the backward products tile (rows of a group, D, F, and
the k = tokens-per-expert sum of the weight gradients); assignments are
balanced, ragged, or leave an expert empty; both mixes, both activations.
Tolerances: 1e-5 (fp32), 2e-2 (bf16) max-abs relative per gradient.

At the large workload's full size (T = 65536, E = 128, D = 2048, F = 8192,
the configuration the benchmark times), a few experts' gradients are
checked against the oracle computed for those experts only."""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
from balanced_token_expert_amd import api
from balanced_token_expert_amd import workloads as W
from tests.gpu_util import dev_to_f64, f64, rel_err, to_dev

pytestmark = pytest.mark.gpu

CASES = [
    # T, E, D, F, dtype, act, kind, mix, assignment
    dict(T=512, E=8, D=64, F=256, dtype="f32", act="relu", kind="iid", mix=0, asg="balanced"),
    dict(T=600, E=6, D=72, F=96, dtype="f32", act="gelu", kind="mixture", mix=1, asg="ragged"),
    dict(T=1536, E=4, D=320, F=520, dtype="bf16", act="gelu", kind="iid", mix=0, asg="balanced"),
    dict(T=1536, E=4, D=320, F=520, dtype="bf16", act="gelu", kind="iid", mix=1, asg="ragged"),
    dict(T=2048, E=8, D=256, F=512, dtype="bf16", act="relu", kind="mixture", mix=1,
         asg="balanced"),
    dict(T=1000, E=5, D=264, F=200, dtype="bf16", act="gelu", kind="iid", mix=0, asg="empty"),
    dict(T=3000, E=3, D=136, F=784, dtype="bf16", act="relu", kind="skew", mix=0, asg="ragged"),
    # one expert holding every token; one token per expert
    dict(T=700, E=1, D=128, F=200, dtype="bf16", act="gelu", kind="iid", mix=1, asg="balanced"),
    dict(T=256, E=256, D=64, F=96, dtype="f32", act="relu", kind="iid", mix=0, asg="balanced"),
]


def _assignment(T, E, how, seed):
    rng = np.random.default_rng(seed)
    if how == "balanced":
        return rng.permutation(np.repeat(np.arange(E), T // E)).astype(np.int32)
    if how == "empty":  # expert E-1 gets nothing, the rest ragged
        return rng.integers(0, E - 1, T).astype(np.int32)
    # ragged: skewed group sizes, every expert present
    p = np.arange(1, E + 1, dtype=np.float64) ** 2
    a = rng.choice(E, size=T, p=p / p.sum()).astype(np.int32)
    a[:E] = np.arange(E)
    return a


def _run(wl, host, a, mix, dev=None):
    dev = dev or {k: to_dev(v, wl.dtype) for k, v in host.items()}
    act = api.BASE_ACT_GELU if wl.act == "gelu" else api.BASE_ACT_RELU
    s = api.base_affinity(dev["h"], dev["w"])
    assign = torch.from_numpy(a).cuda()
    r = api.base_layer_backward(dev["h"], dev["w"], dev["W1"], dev["W2"], act, assign, s,
                                dev["dy"], mix=mix)
    torch.cuda.synchronize()
    assert api.read_stats(r["stats"]).status == 0
    return r, s.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_backward_parity(ci):
    c = CASES[ci]
    wl = W.custom(c["T"], c["E"], c["D"], c["F"], dtype=c["dtype"], act=c["act"],
                  kind=c["kind"], wid=960 + ci)
    host = W.gen_all(wl)
    host["dy"] = W.gen_dy(wl)
    a = _assignment(wl.T, wl.E, c["asg"], ci)
    r, s = _run(wl, host, a, c["mix"])
    mix = "convex" if c["mix"] else "residual"
    dh, dw, dW1, dW2 = oracle.layer_backward(
        f64(host["h"], wl.dtype), f64(host["w"], wl.dtype), f64(host["W1"], wl.dtype),
        f64(host["W2"], wl.dtype), a, wl.act, f64(host["dy"], wl.dtype), mix=mix, s=s)
    tol = 1e-5 if wl.dtype == "f32" else 2e-2
    got = {"dh": dev_to_f64(r["dh"]), "dw": dev_to_f64(r["dw"]),
           "dW1": dev_to_f64(r["dW1"]), "dW2": dev_to_f64(r["dW2"])}
    ref = {"dh": dh, "dw": dw, "dW1": np.stack([dW1[e] for e in range(wl.E)]),
           "dW2": np.stack([dW2[e] for e in range(wl.E)])}
    errs = {k: rel_err(got[k], ref[k]) for k in got}
    print(ci, {k: f"{v:.2e}" for k, v in errs.items()})
    for k, v in errs.items():
        assert v <= tol, (k, v)
    if c["asg"] == "empty":
        # no token: exactly zero gradients for the expert and its centroid
        assert not got["dW1"][-1].any() and not got["dW2"][-1].any() and not got["dw"][-1].any()


def test_backward_zero_upstream_gradient_is_zero():
    wl = W.custom(1024, 4, 256, 512, dtype="bf16", act="gelu", kind="iid", wid=975)
    host = W.gen_all(wl)
    host["dy"] = np.zeros((wl.T, wl.D), dtype=host["h"].dtype)
    r, _ = _run(wl, host, _assignment(wl.T, wl.E, "balanced", 1), 1)
    for k in ("dh", "dw", "dW1", "dW2"):
        assert not r[k].float().abs().max().item(), k


def test_backward_out_of_range_id_reported():
    wl = W.custom(512, 4, 64, 128, dtype="bf16", act="relu", kind="iid", wid=976)
    host = W.gen_all(wl)
    host["dy"] = W.gen_dy(wl)
    dev = {k: to_dev(v, wl.dtype) for k, v in host.items()}
    a = _assignment(wl.T, wl.E, "balanced", 2)
    a[7] = wl.E  # outside [0, E)
    s = api.base_affinity(dev["h"], dev["w"])
    r = api.base_layer_backward(dev["h"], dev["w"], dev["W1"], dev["W2"], api.BASE_ACT_RELU,
                                torch.from_numpy(a).cuda(), s, dev["dy"])
    torch.cuda.synchronize()
    assert api.read_stats(r["stats"]).status == api.BASE_ERR_UNBALANCED


def test_backward_full_size_sampled_experts():
    """The large workload at full size: every gradient of three experts (and
    their tokens' dh rows, their centroids' dw rows) against the oracle."""
    wl = W.workload(5)
    T, E, D, F = wl.T, wl.E, wl.D, wl.F
    with ThreadPoolExecutor(16) as ex:
        w = W.gen_centroids(wl)
        h = np.concatenate(list(ex.map(
            lambda r0: W.gen_tokens(wl, rows=slice(r0, min(T, r0 + 4096)), centroids=w),
            range(0, T, 4096))))
        dy = np.concatenate(list(ex.map(
            lambda r0: W.gen_dy(wl, rows=slice(r0, min(T, r0 + 4096))), range(0, T, 4096))))
        W1 = list(ex.map(lambda e: W.gen_w1(wl, e), range(E)))
        W2 = list(ex.map(lambda e: W.gen_w2(wl, e), range(E)))
    dev = {"h": to_dev(h, wl.dtype), "w": to_dev(w, wl.dtype), "dy": to_dev(dy, wl.dtype)}
    dev["W1"] = torch.empty((E, F, D), dtype=torch.bfloat16, device="cuda")
    dev["W2"] = torch.empty((E, D, F), dtype=torch.bfloat16, device="cuda")
    for e in range(E):
        dev["W1"][e].copy_(to_dev(W1[e], wl.dtype))
        dev["W2"][e].copy_(to_dev(W2[e], wl.dtype))
    # the balanced assignment of the benchmark's forward
    c = api.cfg(wl.eps_start, wl.eps_end, wl.eps_factor, max_bids=500 * T)
    fwd = api.base_layer_forward(dev["h"], dev["w"], dev["W1"], dev["W2"], api.BASE_ACT_GELU,
                                 api.BASE_ROUTE_BALANCED, c)
    torch.cuda.synchronize()
    assert api.read_stats(fwd["stats"]).status == 0
    r = api.base_layer_backward(dev["h"], dev["w"], dev["W1"], dev["W2"], api.BASE_ACT_GELU,
                                fwd["assign"], fwd["scores"], dev["dy"])
    torch.cuda.synchronize()
    assert api.read_stats(r["stats"]).status == 0
    a = fwd["assign"].cpu().numpy()
    experts = [0, 77, E - 1]
    rows = np.nonzero(np.isin(a, experts))[0]
    s = fwd["scores"].cpu().numpy().astype(np.float64)
    dh, dw, dW1, dW2 = oracle.layer_backward(
        f64(h, wl.dtype), f64(w, wl.dtype), lambda e: f64(W1[e], wl.dtype),
        lambda e: f64(W2[e], wl.dtype), a, wl.act, f64(dy, wl.dtype), s=s, experts=experts)
    assert rel_err(dev_to_f64(r["dh"][torch.from_numpy(rows).cuda()]), dh[rows]) <= 2e-2
    for e in experts:
        assert rel_err(dev_to_f64(r["dw"][e]), dw[e]) <= 2e-2, e
        assert rel_err(dev_to_f64(r["dW1"][e]), dW1[e]) <= 2e-2, e
        assert rel_err(dev_to_f64(r["dW2"][e]), dW2[e]) <= 2e-2, e


# ---------------------------------------------------------------- layer-norm blocks

BLOCK_CASES = [
    # T, E, D, F, dtype, act, kind, mix, blocks, layer-norm params, assignment
    dict(T=600, E=6, D=72, F=96, dtype="f32", act="gelu", kind="mixture", mix=1, sub=2, ln=True,
         asg="balanced"),
    dict(T=1536, E=4, D=320, F=520, dtype="bf16", act="gelu", kind="iid", mix=1, sub=1, ln=True,
         asg="balanced"),
    dict(T=2048, E=8, D=256, F=512, dtype="bf16", act="relu", kind="mixture", mix=0, sub=2,
         ln=True, asg="ragged"),
    dict(T=1000, E=5, D=264, F=200, dtype="bf16", act="gelu", kind="iid", mix=1, sub=3, ln=False,
         asg="empty"),
    # rows of 1032 and 2056 elements: the layer-norm backward holds 4 and 8
    # pieces of 8 per lane
    dict(T=900, E=3, D=1032, F=136, dtype="bf16", act="gelu", kind="iid", mix=0, sub=1, ln=True,
         asg="ragged"),
    dict(T=1024, E=4, D=2056, F=256, dtype="bf16", act="relu", kind="iid", mix=1, sub=1, ln=True,
         asg="balanced"),
    # D not a multiple of 8: the row kernels' one-element form
    dict(T=700, E=5, D=100, F=120, dtype="f32", act="gelu", kind="mixture", mix=1, sub=2, ln=True,
         asg="ragged"),
    # one expert; one token per expert
    dict(T=640, E=1, D=192, F=256, dtype="bf16", act="gelu", kind="iid", mix=0, sub=2, ln=True,
         asg="balanced"),
    dict(T=128, E=128, D=64, F=64, dtype="f32", act="gelu", kind="iid", mix=1, sub=1, ln=True,
         asg="balanced"),
    # three ReLU blocks over 4096 tokens: many z near the kink
    dict(T=4096, E=8, D=256, F=512, dtype="bf16", act="relu", kind="mixture", mix=0, sub=3,
         ln=True, asg="balanced"),
]


@pytest.mark.parametrize("ci", range(len(BLOCK_CASES)))
def test_block_backward_parity(ci):
    c = BLOCK_CASES[ci]
    N = c["sub"]
    wl = W.custom(c["T"], c["E"], c["D"], c["F"], dtype=c["dtype"], act=c["act"],
                  kind=c["kind"], wid=985 + ci)
    E = wl.E
    w = W.gen_centroids(wl)
    h = W.gen_tokens(wl, centroids=w)
    dy = W.gen_dy(wl)
    W1 = np.stack([np.stack([W.gen_block_w1(wl, n, e) for e in range(E)]) for n in range(N)])
    W2 = np.stack([np.stack([W.gen_block_w2(wl, n, e) for e in range(E)]) for n in range(N)])
    gam = bet = None
    if c["ln"]:
        lnp = [W.gen_ln(wl, n) for n in range(N)]
        gam = np.stack([g for g, _ in lnp])
        bet = np.stack([b for _, b in lnp])
    a = _assignment(wl.T, E, c["asg"], 40 + ci)
    dev = {k: to_dev(v, wl.dtype) for k, v in dict(h=h, w=w, W1=W1, W2=W2, dy=dy).items()}
    s = api.base_affinity(dev["h"], dev["w"])
    act = api.BASE_ACT_GELU if wl.act == "gelu" else api.BASE_ACT_RELU
    r = api.base_layer_backward_ex(
        dev["h"], dev["w"], dev["W1"], dev["W2"], act, torch.from_numpy(a).cuda(), s, dev["dy"],
        mix=c["mix"], sublayers=N,
        ln_gamma=None if gam is None else torch.from_numpy(gam).cuda(),
        ln_beta=None if bet is None else torch.from_numpy(bet).cuda())
    torch.cuda.synchronize()
    assert api.read_stats(r["stats"]).status == 0
    s64 = s.cpu().numpy().astype(np.float64)
    stack = lambda d: np.stack([np.stack([d[(n, e)] for e in range(E)]) for n in range(N)])
    args = (f64(h, wl.dtype), f64(w, wl.dtype), lambda n, e: f64(W1[n][e], wl.dtype),
            lambda n, e: f64(W2[n][e], wl.dtype), a, wl.act, f64(dy, wl.dtype))
    kw = dict(mix="convex" if c["mix"] else "residual", sublayers=N, gamma=gam, beta=bet,
              ln_eps=1e-5, s=s64)
    names = ("dh", "dw", "dW1", "dW2", "dgamma", "dbeta")

    def as_ref(res):
        dh, dw, dW1, dW2, dga, dbe = res
        return dict(zip(names, (dh, dw, stack(dW1), stack(dW2), stack(dga), stack(dbe))))

    ref = as_ref(oracle.layer_backward_ex(*args, **kw))   # the plain fp64 oracle
    got = {k: dev_to_f64(r[k]) for k in ref}
    # the oracle with its block state rounded where the kernel stores it
    # (each block's input, layer-norm output and act(z)): printed beside
    # the check, and for ReLU the source of the bar below
    rnd = as_ref(oracle.layer_backward_ex(*args, **kw, store=wl.dtype))
    base = 1e-5 if wl.dtype == "f32" else 2e-2
    tol = {k: base for k in ref}
    if wl.act == "relu":
        # ReLU's derivative is a 0/1 decision on the sign of z; z is computed
        # from the block state the kernel keeps in its dtype, so decisions
        # with z inside that rounding flip. How far that alone moves the exact
        # gradients is what the oracle shows between its unrounded and
        # rounded-state results; the kernel may differ by that, half again,
        # on top of the usual bar.
        tol = {k: base + 1.5 * rel_err(rnd[k], ref[k]) for k in ref}
    errs = {k: rel_err(got[k], ref[k]) for k in ref}
    print(ci, {k: f"{v:.2e}/{tol[k]:.2e}" for k, v in errs.items()},
          "vs rounded-state oracle:", {k: f"{rel_err(got[k], rnd[k]):.2e}" for k in ref})
    for k, v in errs.items():
        assert v <= tol[k], (k, v, tol[k])
    if c["asg"] == "empty":
        assert not got["dW1"][:, -1].any() and not got["dW2"][:, -1].any()
        assert not got["dgamma"][:, -1].any() and not got["dbeta"][:, -1].any()


def test_block_backward_rejects_bad_options():
    wl = W.custom(512, 4, 64, 128, dtype="bf16", act="relu", kind="iid", wid=990)
    host = W.gen_all(wl)
    dev = {k: to_dev(v, wl.dtype) for k, v in host.items()}
    s = api.base_affinity(dev["h"], dev["w"])
    a = torch.from_numpy(_assignment(wl.T, wl.E, "balanced", 3)).cuda()
    dyd = dev["h"].clone()
    W1x = dev["W1"][None].expand(65, *dev["W1"].shape).contiguous()
    W2x = dev["W2"][None].expand(65, *dev["W2"].shape).contiguous()
    with pytest.raises(api.BaseError):  # more blocks than the library takes
        api.base_layer_backward_ex(dev["h"], dev["w"], W1x, W2x, 0, a, s, dyd, sublayers=65,
                                   want_ln_grads=False)
    del W1x, W2x
    # shapes that do not match the block count never reach the library
    with pytest.raises(ValueError):
        api.base_layer_backward_ex(dev["h"], dev["w"], dev["W1"][None], dev["W2"][None], 0, a, s,
                                   dyd, sublayers=2)
    with pytest.raises(TypeError):
        api.base_layer_backward_ex(dev["h"], dev["w"], dev["W1"][None], dev["W2"][None], 0, a, s,
                                   dyd, sublayers=1,
                                   ln_gamma=torch.ones((1, wl.E, wl.D), dtype=torch.bfloat16,
                                                       device="cuda"))
    with pytest.raises(api.BaseError):
        api.base_layer_backward_ex(dev["h"], dev["w"], dev["W1"][None], dev["W2"][None], 0, a, s,
                                   dyd, sublayers=1, ln_eps=-1.0)
    # the plain entry point does not take blocks
    with pytest.raises(api.BaseError):
        opts_call = api.base_layer_backward
        lib = api.load()
        o = api.LayerOpts(0, 1, 1e-5, None, None)
        ws = api.workspace(api.BASE_OP_LAYER_BWD, wl.T, wl.E, wl.D, wl.F, api.BASE_BF16)
        outs = [torch.empty_like(x) for x in (dev["h"], dev["w"], dev["W1"], dev["W2"])]
        rc = lib.base_layer_backward(*(api._ptr(x) for x in (dev["h"], dev["w"], dev["W1"],
                                                              dev["W2"])),
                                     wl.T, wl.E, wl.D, wl.F, api.BASE_BF16, 0, api._ptr(a),
                                     api._ptr(s), api._ptr(dyd), *(api._ptr(x) for x in outs),
                                     None, api.ctypes.byref(o), api._ptr(ws), ws.numel(),
                                     api._stream(None))
        api._check(rc, "base_layer_backward")
        del opts_call


@pytest.mark.parametrize("mix", [0, 1])
def test_backward_ex_without_blocks_matches_plain(mix):
    """sublayers = 0 through base_layer_backward_ex is base_layer_backward,
    bit for bit."""
    wl = W.custom(1536, 4, 320, 520, dtype="bf16", act="gelu", kind="iid", wid=995 + mix)
    host = W.gen_all(wl)
    host["dy"] = W.gen_dy(wl)
    a = _assignment(wl.T, wl.E, "ragged", 7)
    r, _ = _run(wl, host, a, mix)
    dev = {k: to_dev(v, wl.dtype) for k, v in host.items()}
    s = api.base_affinity(dev["h"], dev["w"])
    rx = api.base_layer_backward_ex(dev["h"], dev["w"], dev["W1"], dev["W2"], api.BASE_ACT_GELU,
                                    torch.from_numpy(a).cuda(), s, dev["dy"], mix=mix,
                                    sublayers=0)
    torch.cuda.synchronize()
    assert api.read_stats(rx["stats"]).status == 0
    for k in ("dh", "dw", "dW1", "dW2"):
        assert torch.equal(r[k], rx[k]), k


def test_block_backward_zero_upstream_gradient_is_zero():
    wl = W.custom(1024, 4, 256, 512, dtype="bf16", act="gelu", kind="iid", wid=997)
    N, E = 2, wl.E
    w = W.gen_centroids(wl)
    h = W.gen_tokens(wl, centroids=w)
    W1 = np.stack([np.stack([W.gen_block_w1(wl, n, e) for e in range(E)]) for n in range(N)])
    W2 = np.stack([np.stack([W.gen_block_w2(wl, n, e) for e in range(E)]) for n in range(N)])
    lnp = [W.gen_ln(wl, n) for n in range(N)]
    dev = {k: to_dev(v, wl.dtype) for k, v in dict(h=h, w=w, W1=W1, W2=W2).items()}
    s = api.base_affinity(dev["h"], dev["w"])
    a = torch.from_numpy(_assignment(wl.T, E, "balanced", 8)).cuda()
    r = api.base_layer_backward_ex(
        dev["h"], dev["w"], dev["W1"], dev["W2"], api.BASE_ACT_GELU, a, s,
        torch.zeros_like(dev["h"]), mix=1, sublayers=N,
        ln_gamma=torch.from_numpy(np.stack([g for g, _ in lnp])).cuda(),
        ln_beta=torch.from_numpy(np.stack([b for _, b in lnp])).cuda())
    torch.cuda.synchronize()
    assert api.read_stats(r["stats"]).status == 0
    for k in ("dh", "dw", "dW1", "dW2", "dgamma", "dbeta"):
        assert not r[k].float().abs().max().item(), k
