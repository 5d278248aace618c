"""Exactness of the balanced assignment (eq. 2 of "BASE Layers", sec. 3.2.1)
on the workloads' own inputs and on closed forms at full size.

An assignment that is eps-complementary-slack is within T * eps of the
optimum; when eps is below gap / T, with gap the distance from the optimum
to the second-best balanced assignment, it IS the optimum. Each test here
computes gap first and then runs the GPU auction with eps_end = gap / (2T),
asserting equality with the unique optimum -- never conditionally: a test
whose gap is not positive fails.

  - the tiny workload (T=512, E=8): optimum by the Hungarian method on the
    GPU's own fp32 scores, gap by the minimum cycle of the expert exchange
    graph;
  - the mixture (T=16384, E=128) and skew (T=32768, E=128) workloads: the
    optimum by cancelling negative cycles from the default-schedule result,
    certified by the minimum cycle, which is also the gap;
  - closed forms at T=16384, E=128 through base_affinity on bf16 inputs
    built so that the fp32 scores are exact: rank one s = x_t y_e (the
    optimum is assortative: tokens sorted by x fill the experts in the order
    of y), two experts (expert 0 takes the k tokens with the largest
    s[t,0] - s[t,1]), and a greedy routing that is already balanced (then
    it is the optimum).
"""
import numpy as np
import pytest
import torch

import oracle
from balanced_token_expert_amd import api
from balanced_token_expert_amd import workloads as W
from tests.gpu_util import to_dev

pytestmark = pytest.mark.gpu

CAP_PER_TOKEN = 2000  # bid cap per token over every phase (a safety valve)


def _solve(scores, eps_end, eps_start=1.0):
    T = scores.shape[0]
    c = api.cfg(max(eps_start, eps_end), eps_end, 10.0, max_bids=CAP_PER_TOKEN * T)
    res = api.base_assign_auction(scores, c)
    torch.cuda.synchronize()
    st = api.read_stats(res["stats"])
    assert st.status == 0, st
    return res, st


def _scores(wid):
    wl = W.workload(wid)
    w = W.gen_centroids(wl)
    h = W.gen_tokens(wl, centroids=w)
    s = api.base_affinity(to_dev(h, wl.dtype), to_dev(w, wl.dtype))
    torch.cuda.synchronize()
    return wl, s


def test_exact_tiny_workload_hungarian():
    wl, scores = _scores(1)
    s = scores.cpu().numpy().astype(np.float64)
    opt = oracle.hungarian(s)
    gap = oracle.min_cycle_gap(s, opt)
    assert gap > 0, gap
    eps = gap / (2 * wl.T)
    res, st = _solve(scores, eps)
    a = res["assign"].cpu().numpy()
    print(f"tiny: gap {gap:.3e} eps_end {eps:.3e} bids {sum(st.bids)} phases {st.phases}")
    assert (a == opt).all()


@pytest.mark.parametrize("wid", [2, 4])
def test_exact_assignment_workloads(wid):
    wl, scores = _scores(wid)
    s = scores.cpu().numpy().astype(np.float64)
    res0, _ = _solve(scores, wl.eps_end, wl.eps_start)
    opt, _ = oracle.cycle_cancel(s, res0["assign"].cpu().numpy())
    gap = oracle.min_cycle_gap(s, opt)
    assert gap > 0, gap
    eps = gap / (2 * wl.T)
    res, st = _solve(scores, eps, wl.eps_start)
    a = res["assign"].cpu().numpy()
    print(f"{wl.name}: gap {gap:.3e} eps_end {eps:.3e} bids/phase {st.bids} "
          f"depth/phase {st.rounds}")
    assert (a == opt).all()
    # the returned grouping is the canonical one of that assignment
    cperm, coff = oracle.canonical_perm(opt, wl.E)
    assert (res["perm"].cpu().numpy() == cperm).all()
    assert (res["offsets"].cpu().numpy() == coff).all()


@pytest.mark.parametrize("E", [128, 16])
def test_exact_late_rounds(E):
    """8192 tokens of the contested mixture recipe: after two bulk rounds
    each phase's remaining rounds run in the cooperative late-round launch
    (holders resident in the workgroups' LDS, two device-wide barriers per
    round). Same bar: with eps_end = gap / (2T) the result is the optimum
    (cycle cancelling from the default-schedule result, certified by the
    minimum cycle)."""
    wl = W.custom(8192, E, 256, None, dtype="bf16", kind="mixture", wid=993 + E)
    w = W.gen_centroids(wl)
    h = W.gen_tokens(wl, centroids=w)
    scores = api.base_affinity(to_dev(h, wl.dtype), to_dev(w, wl.dtype))
    torch.cuda.synchronize()
    s = scores.cpu().numpy().astype(np.float64)
    res0, st0 = _solve(scores, wl.eps_end, wl.eps_start)
    a0 = res0["assign"].cpu().numpy()
    assert (np.bincount(a0, minlength=E) == wl.T // E).all()
    p0 = res0["prices"].cpu().numpy()
    assert oracle.eps_cs_violation(s, a0, p0) <= wl.eps_end * (1 + 1e-9)
    opt, _ = oracle.cycle_cancel(s, a0)
    gap = oracle.min_cycle_gap(s, opt)
    assert gap > 0, gap
    eps = gap / (2 * wl.T)
    res, st = _solve(scores, eps, wl.eps_start)
    a = res["assign"].cpu().numpy()
    print(f"T=8192 E={E}: gap {gap:.3e} eps_end {eps:.3e} bids/phase {st.bids} "
          f"depth/phase {st.rounds}")
    assert (a == opt).all()


def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).cuda()


def test_exact_rank1_closed_form_full_size():
    """h_t = (a_t, b_t, 0...), w_e = (y_e, y_e / 256, 0...): s = y_e x_t with
    x_t = a_t + b_t / 256. a_t, b_t run over the integers 128..255 (every
    pair once: 16384 distinct x with 16 significant bits), y_e = (128 + e)/128
    (8 bits): every product and the sum fit fp32's 24 bits, so the GPU's
    scores are exact. Rearrangement: the unique optimum gives the k tokens
    of smallest x to the expert of smallest y, and so on. The gap is at
    least (min x step)(min y step) = 2^-8 * 2^-7, so eps_end = 2^-31 is below
    gap / T = 2^-29."""
    T, E, D = 16384, 128, 8
    k = T // E
    rng = np.random.default_rng(11)
    pairs = rng.permutation(T)
    a_t = 128 + pairs // 128
    b_t = 128 + pairs % 128
    h = np.zeros((T, D), np.float32)
    h[:, 0], h[:, 1] = a_t, b_t
    ye = (128 + rng.permutation(E)) / 128.0
    w = np.zeros((E, D), np.float32)
    w[:, 0], w[:, 1] = ye, ye / 256.0
    scores = api.base_affinity(_bf16(h), _bf16(w))
    torch.cuda.synchronize()
    x = a_t + b_t / 256.0
    assert (scores.cpu().numpy().astype(np.float64) == np.outer(x, ye)).all()
    expect = np.empty(T, np.int64)
    expect[np.argsort(x)] = np.repeat(np.argsort(ye), k)
    res, st = _solve(scores, 2.0 ** -31)
    print(f"rank-1: bids/phase {st.bids} depth/phase {st.rounds}")
    assert (res["assign"].cpu().numpy() == expect).all()


def test_exact_rank1_crowded_first_round():
    """The rank-1 closed form at T = 4096, E = 8 (k = 512): every token's
    first bid goes to the expert of largest y, 4096 bidders for 512 slots,
    so the resolve takes its chunked path and the sampled cut on a chunk of
    2048 (at least 2k bids) decides which bids leave before the sort.
    a_t in 128..255, b_t in 128..159 (every pair once), y_e = (128 + e)/128:
    exact fp32 products, gap at least 2^-15, eps_end = 2^-31 below gap / T."""
    T, E, D = 4096, 8, 8
    k = T // E
    rng = np.random.default_rng(12)
    pairs = rng.permutation(T)
    a_t = 128 + pairs // 32
    b_t = 128 + pairs % 32
    h = np.zeros((T, D), np.float32)
    h[:, 0], h[:, 1] = a_t, b_t
    ye = (128 + rng.permutation(E)) / 128.0
    w = np.zeros((E, D), np.float32)
    w[:, 0], w[:, 1] = ye, ye / 256.0
    scores = api.base_affinity(_bf16(h), _bf16(w))
    torch.cuda.synchronize()
    x = a_t + b_t / 256.0
    assert (scores.cpu().numpy().astype(np.float64) == np.outer(x, ye)).all()
    expect = np.empty(T, np.int64)
    expect[np.argsort(x)] = np.repeat(np.argsort(ye), k)
    res, st = _solve(scores, 2.0 ** -31)
    assert st.bids[0] >= T  # the first phase's first round: every token bids
    assert (res["assign"].cpu().numpy() == expect).all()


def test_exact_two_experts_closed_form_full_size():
    """E = 2: expert 0 takes the k tokens with the largest s[t,0] - s[t,1]
    (every balanced assignment scores sum_t s[t,1] + sum_{t in expert 0}
    (s[t,0] - s[t,1])). Unique when the k-th and (k+1)-th largest
    differences differ; that difference is the gap."""
    T, E, D = 16384, 2, 64
    k = T // E
    rng = np.random.default_rng(12)
    h = rng.standard_normal((T, D)).astype(np.float32)
    w = (rng.standard_normal((E, D)) / np.sqrt(D)).astype(np.float32)
    scores = api.base_affinity(_bf16(h), _bf16(w))
    torch.cuda.synchronize()
    s = scores.cpu().numpy().astype(np.float64)
    d = s[:, 0] - s[:, 1]
    order = np.argsort(-d, kind="stable")
    gap = d[order[k - 1]] - d[order[k]]
    assert gap > 0, gap
    expect = np.ones(T, np.int64)
    expect[order[:k]] = 0
    res, _ = _solve(scores, gap / (2 * T))
    assert (res["assign"].cpu().numpy() == expect).all()


def test_exact_greedy_already_balanced_full_size():
    """Tokens drawn near their own centroid, exactly k per expert: each
    token's best expert is its own, the greedy routing is balanced and so
    optimal; any other balanced assignment moves a cycle of at least two
    tokens off their best expert, so the gap is at least twice the smallest
    best-minus-second margin."""
    T, E, D = 16384, 128, 64
    k = T // E
    rng = np.random.default_rng(13)
    w = rng.standard_normal((E, D)).astype(np.float32)
    w /= np.linalg.norm(w, axis=1, keepdims=True)
    own = rng.permutation(np.repeat(np.arange(E), k))
    h = (4.0 * w[own] + 0.05 * rng.standard_normal((T, D))).astype(np.float32)
    scores = api.base_affinity(_bf16(h), _bf16(w))
    torch.cuda.synchronize()
    s = scores.cpu().numpy().astype(np.float64)
    srt = np.sort(s, axis=1)
    assert (s.argmax(axis=1) == own).all()
    gap_lb = 2.0 * float((srt[:, -1] - srt[:, -2]).min())
    assert gap_lb > 0
    res, _ = _solve(scores, gap_lb / (2 * T))
    assert (res["assign"].cpu().numpy() == own).all()
