"""Parity at the five workloads' full sizes, in the launch configuration the
benchmark times (base_layer_forward BALANCED with the workload's eps
schedule; base_assign_auction for the assignment-only workload; greedy
routing of the same scores).

What the oracle cannot recompute at these sizes is checked on samples or by
properties that hold at any size:
  - affinities: sampled rows against the exact fp64 value, within Higham's
    fp32 dot-product bound;
  - the assignment: exact balance, the canonical grouping, and total
    affinity within T * eps_end of the optimum of the same scores -- the
    optimum found by cancelling negative cycles of the expert exchange graph
    from the GPU's assignment (exact at any size); for the solver entry point
    also eps-complementary slackness and the dual certificate of the
    returned prices;
  - greedy routing: bit-exact on the same scores (a full pass, cheap);
  - the layer output: every token of a few experts against the oracle's
    fp64 layer, within 1e-5 (fp32) / 2e-2 (bf16) relative error; and with
    W2 = 0 the output must equal h bit for bit, every row.
The tiny workload is small enough to check everything in full.
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
from balanced_token_expert_amd import api
from balanced_token_expert_amd import workloads as W
from tests.gpu_util import dev_to_f64, f64, higham_bound, rel_err, to_dev

pytestmark = pytest.mark.gpu

CAP_PER_TOKEN = 500  # bid cap (a safety valve): bids per token over all phases


def _gen(wl):
    """Inputs of a workload, generated in parallel (same recipe as everywhere)."""
    w = W.gen_centroids(wl)
    with ThreadPoolExecutor(16) as ex:
        blocks = list(ex.map(lambda c: W.gen_tokens(wl, rows=slice(c, min(wl.T, c + 4096)),
                                                    centroids=w), range(0, wl.T, 4096)))
        host = {"w": w, "h": np.concatenate(blocks)}
        if wl.F is not None:
            host["W1"] = np.stack(list(ex.map(lambda e: W.gen_w1(wl, e), range(wl.E))))
            host["W2"] = np.stack(list(ex.map(lambda e: W.gen_w2(wl, e), range(wl.E))))
    return host


def _cfg(wl):
    return api.cfg(wl.eps_start, wl.eps_end, wl.eps_factor, max_bids=CAP_PER_TOKEN * wl.T)


def _act(wl):
    return api.BASE_ACT_GELU if wl.act == "gelu" else api.BASE_ACT_RELU


def _check_affinity_rows(wl, host, s32, n=256, seed=0):
    rng = np.random.default_rng(seed)
    rows = np.unique(np.concatenate([[0, wl.T - 1], rng.integers(0, wl.T, n)]))
    h64, w64 = f64(host["h"][rows], wl.dtype), f64(host["w"], wl.dtype)
    exact = oracle.affinity(h64, w64)
    bound = higham_bound(h64, w64)
    err = np.abs(s32[rows].astype(np.float64) - exact)
    assert (err <= bound + 1e-30).all(), float((err / (bound + 1e-30)).max())


def _check_assignment(wl, s32, a, perm=None, offsets=None):
    """Balance, grouping and the T*eps_end bound against the exact optimum."""
    T, E, k = wl.T, wl.E, wl.T // wl.E
    s = s32.astype(np.float64)
    assert (np.bincount(a, minlength=E) == k).all(), "unbalanced"
    cperm, coff = oracle.canonical_perm(a, E)
    if perm is not None:
        assert (perm == cperm).all()
    if offsets is not None:
        assert (offsets == coff).all()
    opt_a, _ = oracle.cycle_cancel(s, a)
    assert (np.bincount(opt_a, minlength=E) == k).all()
    assert oracle.min_cycle_gap(s, opt_a) >= -1e-9  # certified optimal
    P, opt = oracle.objective(s, a), oracle.objective(s, opt_a)
    assert P >= opt - T * wl.eps_end - 1e-9 * abs(opt), (P, opt)
    return P, opt


def test_full_tiny_fp32_everything():
    """T=512, E=8, D=64, F=256 fp32 ReLU: affinities, the auction against the
    Hungarian optimum (within T * eps_end), greedy routing and every output
    row."""
    wl = W.workload(1)
    host = _gen(wl)
    dev = {k: to_dev(v, wl.dtype) for k, v in host.items()}
    r = api.base_layer_forward(dev["h"], dev["w"], dev["W1"], dev["W2"], _act(wl),
                               api.BASE_ROUTE_BALANCED, _cfg(wl))
    g = api.base_route_greedy(r["scores"])
    torch.cuda.synchronize()
    assert api.read_stats(r["stats"]).status == 0
    s32 = r["scores"].cpu().numpy()
    _check_affinity_rows(wl, host, s32, n=wl.T)
    a = r["assign"].cpu().numpy()
    _check_assignment(wl, s32, a, r["perm"].cpu().numpy(), None)
    s = s32.astype(np.float64)
    # within T * eps_end of the Hungarian optimum (exactness below the gap is
    # tests/test_gpu_exact.py's, with eps_end set from the gap)
    opt = oracle.objective(s, oracle.hungarian(s))
    assert oracle.objective(s, a) >= opt - wl.T * wl.eps_end - 1e-9 * abs(opt)
    ga, gc = oracle.greedy_route(s)
    assert (g["assign"].cpu().numpy() == ga).all() and (g["counts"].cpu().numpy() == gc).all()
    ref = oracle.layer_forward(f64(host["h"], wl.dtype), f64(host["w"], wl.dtype),
                               f64(host["W1"], wl.dtype), f64(host["W2"], wl.dtype), a, wl.act,
                               s=s)
    assert rel_err(dev_to_f64(r["out"]), ref) <= 1e-5


@pytest.mark.parametrize("wid", [2, 4])
def test_full_assignment(wid):
    """The solver entry point at the mixture (T=16384, E=128) and skew
    (T=32768, E=128) workloads: certificates of the returned prices, the
    bound against the exact optimum, greedy routing of the same scores."""
    wl = W.workload(wid)
    w = W.gen_centroids(wl)
    host = {"w": w, "h": W.gen_tokens(wl, centroids=w)}
    hd, wd = to_dev(host["h"], wl.dtype), to_dev(host["w"], wl.dtype)
    scores = api.base_affinity(hd, wd)
    res = api.base_assign_auction(scores, _cfg(wl))
    g = api.base_route_greedy(scores)
    torch.cuda.synchronize()
    st = api.read_stats(res["stats"])
    assert st.status == 0, st
    s32 = scores.cpu().numpy()
    _check_affinity_rows(wl, host, s32)
    a = res["assign"].cpu().numpy()
    P, opt = _check_assignment(wl, s32, a, res["perm"].cpu().numpy(), res["offsets"].cpu().numpy())
    s = s32.astype(np.float64)
    p = res["prices"].cpu().numpy()
    assert oracle.eps_cs_violation(s, a, p) <= wl.eps_end * (1 + 1e-9) + 1e-12
    assert P >= oracle.dual_value(s, p, wl.T // wl.E) - wl.T * wl.eps_end - 1e-9 * abs(P)
    ga, gc = oracle.greedy_route(s)
    assert (g["assign"].cpu().numpy() == ga).all() and (g["counts"].cpu().numpy() == gc).all()


@pytest.mark.parametrize("wid", [3, 4, 5])
def test_full_layer(wid):
    """The whole layer at T=16384/E=64/D=1536/F=6144, T=32768/E=128/D=1024/
    F=4096 (skew) and T=65536/E=128/D=2048/F=8192, bf16 GELU: the
    assignment's bound, greedy routing, every row of three experts against
    the fp64 oracle, and W2 = 0 giving h exactly."""
    wl = W.workload(wid)
    host = _gen(wl)
    dev = {k: to_dev(v, wl.dtype) for k, v in host.items()}
    r = api.base_layer_forward(dev["h"], dev["w"], dev["W1"], dev["W2"], _act(wl),
                               api.BASE_ROUTE_BALANCED, _cfg(wl))
    g = api.base_route_greedy(r["scores"])
    torch.cuda.synchronize()
    assert api.read_stats(r["stats"]).status == 0
    s32 = r["scores"].cpu().numpy()
    a = r["assign"].cpu().numpy()
    _check_affinity_rows(wl, host, s32)
    _check_assignment(wl, s32, a, r["perm"].cpu().numpy(), None)
    s = s32.astype(np.float64)
    ga, gc = oracle.greedy_route(s)
    assert (g["assign"].cpu().numpy() == ga).all() and (g["counts"].cpu().numpy() == gc).all()
    experts = [0, wl.E // 2, wl.E - 1]
    rows = np.nonzero(np.isin(a, experts))[0]
    h64 = f64(host["h"], wl.dtype)
    ref = oracle.layer_forward(h64, f64(host["w"], wl.dtype),
                               lambda e: f64(host["W1"][e], wl.dtype),
                               lambda e: f64(host["W2"][e], wl.dtype), a, wl.act,
                               experts=experts, s=s)[rows]
    y = dev_to_f64(r["out"])[rows]
    assert rel_err(y, ref) <= 2e-2, rel_err(y, ref)
    # W2 = 0: the output is h, bit for bit, in every row
    z = torch.zeros_like(dev["W2"])
    r0 = api.base_layer_forward(dev["h"], dev["w"], dev["W1"], z, _act(wl),
                                api.BASE_ROUTE_BALANCED, _cfg(wl))
    torch.cuda.synchronize()
    assert api.read_stats(r0["stats"]).status == 0
    assert torch.equal(r0["out"], dev["h"])


@pytest.mark.parametrize("wid", [4, 5])
def test_full_greedy_layer(wid):
    """Greedy-mode layer (ragged expert groups) at the skew workload (about
    80 % of the tokens on one expert) and the large workload: routing
    bit-exact with the oracle's argmax of the same scores, canonical
    grouping, and sampled rows -- up to 256 of the largest group plus every
    row of the smallest non-empty group and of expert E-1 -- against the fp64
    layer."""
    wl = W.workload(wid)
    host = _gen(wl)
    dev = {k: to_dev(v, wl.dtype) for k, v in host.items()}
    r = api.base_layer_forward(dev["h"], dev["w"], dev["W1"], dev["W2"], _act(wl),
                               api.BASE_ROUTE_GREEDY)
    torch.cuda.synchronize()
    assert api.read_stats(r["stats"]).status == 0
    s = r["scores"].cpu().numpy().astype(np.float64)
    a = r["assign"].cpu().numpy()
    ga, gc = oracle.greedy_route(s)
    assert (a == ga).all()
    cperm, _ = oracle.canonical_perm(a, wl.E)
    assert (r["perm"].cpu().numpy() == cperm).all()
    rng = np.random.default_rng(wid)
    big = int(np.argmax(gc))
    nonempty = np.nonzero(gc)[0]
    small = int(nonempty[np.argmin(gc[nonempty])])
    pick = [np.nonzero(a == big)[0]]
    pick[0] = rng.choice(pick[0], size=min(256, pick[0].size), replace=False)
    pick += [np.nonzero(a == small)[0], np.nonzero(a == wl.E - 1)[0]]
    rows = np.unique(np.concatenate(pick))
    sub = np.full(wl.T, -1, dtype=np.int64)  # only the sampled rows keep their expert
    sub[rows] = a[rows]
    ref = oracle.layer_forward(f64(host["h"], wl.dtype), f64(host["w"], wl.dtype),
                               lambda e: f64(host["W1"][e], wl.dtype),
                               lambda e: f64(host["W2"][e], wl.dtype), sub, wl.act,
                               experts=sorted({big, small, wl.E - 1}), s=s)[rows]
    y = dev_to_f64(r["out"])[rows]
    assert rel_err(y, ref) <= 2e-2, rel_err(y, ref)
