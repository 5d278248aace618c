#!/usr/bin/env python3
"""Benchmark of the BASE-layer forward on one MI355X.

One step = one pass of the whole hot path over one batch: affinities, the
balanced assignment (auction, eps 1.0 -> 1e-4), the expert
grouping, both expert products with the fused gate/residual/scatter
(``base_layer_forward``, BALANCED) plus greedy test-time routing of the same
scores (``base_route_greedy``), on the large workload: T=65536 tokens
(32 x 2048), E=128 experts, D=2048, FFN 2048->8192->2048 GELU, bf16 (about
8.6 GB of expert weights). Inputs are seeded synthetic data, resident in HBM
before timing starts.

Also reported: the auction solve time on the mixture workload (T=16384,
E=128, D=1024, eps 1.0 -> 1e-4), the per-phase kernel times (HIP events
recorded by the library on its stream), the roofline of the dominant kernel,
the CPU oracle timed on a bounded sample of the same work, and, outside the
step, the greedy-mode layer, the layer variants (convex mix, layer-norm
blocks) and the backward pass on the same inputs.

    python bench.py [--gpus 1] [--steps 10] [--warmup 2]
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PHASES = ("affinity", "route", "ffn1", "ffn2")

# HBM bytes per launch of the step's kernels at the large workload, from
# two rocprofv3 counter passes (FETCH_SIZE, WRITE_SIZE; KiB per dispatch,
# mean over the dispatches of the profiled steps) scaled by what the same
# counters read for a 1 GiB copy (--copy-probe): fetched = FETCH_SIZE * 1024
# * FETCH_SCALE, written = WRITE_SIZE * 1024 * WRITE_SCALE. Each figure
# describes the kernel built from the sources whose hash is recorded; after
# any change to those sources it is stale and reported as null.
GEMM_SOURCES = ("balanced_token_expert_amd/csrc/gemm.hip",
                "balanced_token_expert_amd/csrc/gemm_dma.h",
                "balanced_token_expert_amd/csrc/common.h")
AUCTION_SOURCES = ("balanced_token_expert_amd/csrc/auction.hip",
                   "balanced_token_expert_amd/csrc/auction_tail.h",
                   "balanced_token_expert_amd/csrc/auction_late.h",
                   "balanced_token_expert_amd/csrc/common.h")
FETCH_SCALE = 1.99992
WRITE_SCALE = 1.0
MEASURED_TRAFFIC = {
    # kernel: (workload, sources, sources sha256, FETCH_SIZE KiB, WRITE_SIZE KiB), means over
    # the dispatches of the balanced step
    "ffn1": ("large_t64k_e128_d2048", GEMM_SOURCES,
             "8695e9d768e779a6446828c43f56586668b688f505037704cdcad5c56d212b0d", 2513144.5, 1185996.9),
    "ffn2": ("large_t64k_e128_d2048", GEMM_SOURCES,
             "8695e9d768e779a6446828c43f56586668b688f505037704cdcad5c56d212b0d", 2907136.1, 353352.6),
    "auction_tail": ("large_t64k_e128_d2048", AUCTION_SOURCES,
                     "27a2f4c6a6b45d10224f920866823bc1267073d4c7b0e6d0b311ceb0199ba249", 638.0, 881.0),
}


def sources_sha256(files):
    import hashlib
    h = hashlib.sha256()
    for rel in files:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the recorded counters, or None when they
    were taken on another workload or on different kernel sources."""
    rec = MEASURED_TRAFFIC.get(kernel)
    if rec is None or rec[0] != workload or rec[2] != sources_sha256(rec[1]):
        return None
    return rec[3] * 1024 * FETCH_SCALE + rec[4] * 1024 * WRITE_SCALE


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class HipEvents:
    """Raw hipEvent_t handles for the library's phase markers."""

    def __init__(self, n):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                 ctypes.c_void_p, ctypes.c_void_p]
        self.ev = (ctypes.c_void_p * n)()
        for i in range(n):
            h = ctypes.c_void_p()
            rc = self.hip.hipEventCreate(ctypes.byref(h))
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed ({rc})")
            self.ev[i] = h

    def block(self, i):
        """Address of handles [i, i+6) (a hipEvent_t array for the library)."""
        return ctypes.addressof(self.ev) + i * ctypes.sizeof(ctypes.c_void_p)

    def ms(self, a, b):
        out = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(out), self.ev[a], self.ev[b])
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(out.value)


def gen_inputs(wl, threads=16):
    from balanced_token_expert_amd import workloads as W
    t0 = time.time()
    w = W.gen_centroids(wl)
    with ThreadPoolExecutor(threads) as ex:
        blocks = list(ex.map(lambda c: W.gen_tokens(wl, rows=slice(c, min(wl.T, c + 4096)),
                                                    centroids=w), range(0, wl.T, 4096)))
        h = np.concatenate(blocks)
        W1 = W2 = None
        if wl.F is not None:
            W1 = list(ex.map(lambda e: W.gen_w1(wl, e), range(wl.E)))
            W2 = list(ex.map(lambda e: W.gen_w2(wl, e), range(wl.E)))
    log(f"[bench] generated {wl.name} in {time.time() - t0:.1f}s")
    return h, w, W1, W2


def to_dev(x, dtype="bf16"):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def stack_dev(parts, dtype="bf16"):
    import torch
    E = len(parts)
    out = torch.empty((E,) + parts[0].shape,
                      dtype=torch.bfloat16 if dtype == "bf16" else torch.float32, device="cuda")
    for e, p in enumerate(parts):
        out[e].copy_(to_dev(p, dtype))
    return out


def cpu_baseline(wl, h, w, W1, W2, sample_experts=96):
    """The oracle as it stands, on a bounded sample: affinities, CPU auction
    and greedy routing over all T tokens; the fp64 layer forward for the
    tokens of `sample_experts` experts. Scaled to tokens/s of the full step."""
    import oracle
    from balanced_token_expert_amd import workloads as W
    t0 = time.perf_counter()
    s = oracle.affinity(W.as_f64(h, wl.dtype), W.as_f64(w, wl.dtype))
    t_aff = time.perf_counter() - t0
    t0 = time.perf_counter()
    r = oracle.auction(s, wl.eps_start, wl.eps_end, wl.eps_factor)
    t_auc = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.greedy_route(s)
    t_gr = time.perf_counter() - t0
    a = r["assign"]
    ex = list(range(sample_experts))
    n_tok = int(np.isin(a, ex).sum())
    t0 = time.perf_counter()
    oracle.layer_forward(W.as_f64(h, wl.dtype), W.as_f64(w, wl.dtype),
                         lambda e: W.as_f64(W1[e], wl.dtype), lambda e: W.as_f64(W2[e], wl.dtype),
                         a, wl.act, experts=ex, s=s)
    t_ffn = time.perf_counter() - t0
    per_tok = (t_aff + t_auc + t_gr) / wl.T + t_ffn / max(n_tok, 1)
    cores = len(os.sched_getaffinity(0))
    return {"value": round(1.0 / per_tok, 1), "unit": "tokens/s", "cores": cores,
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": (f"{wl.name}: fp64 affinity, CPU auction (1 thread) and greedy over all "
                       f"{wl.T} tokens ({t_aff:.2f}s, {t_auc:.2f}s, {t_gr:.2f}s); fp64 expert "
                       f"FFN + eq. 1 for the {n_tok} tokens of experts 0..{sample_experts - 1} "
                       f"({t_ffn:.2f}s); per-token costs summed"),
            "auction_s": round(t_auc, 3)}


def greedy_layer(hd, wd, W1d, W2d, act, T, E, reps=5):
    """The layer with test-time greedy routing (ragged expert groups) on the
    same inputs: median ms of the whole call and the largest group."""
    import torch
    from balanced_token_expert_amd import api
    bufs = dict(assign=torch.empty(T, dtype=torch.int32, device="cuda"),
                scores=torch.empty((T, E), dtype=torch.float32, device="cuda"),
                perm=torch.empty(T, dtype=torch.int32, device="cuda"),
                out=torch.empty_like(hd), stats=api.new_stats(),
                ws=api.workspace(api.BASE_OP_LAYER, T, E, hd.shape[1], W1d.shape[1],
                                 api.BASE_BF16 if hd.dtype == torch.bfloat16 else api.BASE_F32))
    api.base_layer_forward(hd, wd, W1d, W2d, act, api.BASE_ROUTE_GREEDY, **bufs)
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        api.base_layer_forward(hd, wd, W1d, W2d, act, api.BASE_ROUTE_GREEDY, **bufs)
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    counts = np.bincount(bufs["assign"].cpu().numpy(), minlength=E)
    return {"ms": round(float(np.median(times)), 4), "tokens_per_s": round(T / (np.median(times) * 1e-3), 1),
            "largest_group": int(counts.max()), "empty_experts": int((counts == 0).sum())}


def layer_variants(wl, hd, wd, W1d, W2d, act, c, host=None, reps=5):
    """base_layer_forward_ex on the same inputs and balanced routing: the
    released code's convex mix with plain experts, and experts of one and two
    sec. 4.1 blocks (layer norm, up, activation, down, residual). Block 0
    uses the layer's expert matrices; the second block reuses them (the
    values do not change the work). Median ms of the whole call and of the
    expert part (grouping done -> output written, library phase events)."""
    import torch
    from balanced_token_expert_amd import api
    from balanced_token_expert_amd import workloads as W
    T, E, D, F = wl.T, wl.E, wl.D, wl.F
    dt = api.BASE_BF16 if wl.dtype == "bf16" else api.BASE_F32
    bufs = dict(assign=torch.empty(T, dtype=torch.int32, device="cuda"),
                scores=torch.empty((T, E), dtype=torch.float32, device="cuda"),
                perm=torch.empty(T, dtype=torch.int32, device="cuda"),
                out=torch.empty_like(hd), stats=api.new_stats(),
                ws=api.workspace(api.BASE_OP_LAYER_EX, T, E, D, F, dt))
    lnp = [W.gen_ln(wl, b) for b in range(2)]
    gam = torch.from_numpy(np.stack([g for g, _ in lnp])).cuda()
    bet = torch.from_numpy(np.stack([b for _, b in lnp])).cuda()
    W1x2, W2x2 = torch.stack([W1d, W1d]), torch.stack([W2d, W2d])
    cases = {"convex_plain": dict(mix=api.BASE_MIX_CONVEX, sublayers=0, W1=W1d, W2=W2d),
             "convex_blocks1_ln": dict(mix=api.BASE_MIX_CONVEX, sublayers=1, W1=W1d[None],
                                       W2=W2d[None], ln_gamma=gam[:1], ln_beta=bet[:1]),
             "convex_blocks2_ln": dict(mix=api.BASE_MIX_CONVEX, sublayers=2, W1=W1x2, W2=W2x2,
                                       ln_gamma=gam, ln_beta=bet)}
    ev = HipEvents(6 * reps)
    res = {}
    for name, kw in cases.items():
        kw = dict(kw)
        W1v, W2v = kw.pop("W1"), kw.pop("W2")

        def call():
            api.base_layer_forward_ex(hd, wd, W1v, W2v, act, api.BASE_ROUTE_BALANCED, c, **kw,
                                      **bufs)
        call()
        torch.cuda.synchronize()
        for i in range(reps):
            api.base_set_phase_events(ev.block(6 * i), 6)
            call()
        torch.cuda.synchronize()
        api.base_set_phase_events(None, 0)
        tot = [ev.ms(6 * i, 6 * i + 4) for i in range(reps)]
        exp = [ev.ms(6 * i + 2, 6 * i + 4) for i in range(reps)]
        st = api.read_stats(bufs["stats"])
        xt = 2.0 * 2 * T * D * F * max(kw["sublayers"], 1) / (np.median(exp) * 1e-3) / 1e12
        res[name] = {"ms": round(float(np.median(tot)), 4),
                     "tokens_per_s": round(T / (np.median(tot) * 1e-3), 1),
                     "expert_ms": round(float(np.median(exp)), 4),
                     "expert_tflops": round(xt, 1),
                     "expert_frac_bf16_peak": round(xt / PEAK_BF16_TFLOPS, 4),
                     "status": st.status}
        if host is not None and name == "convex_blocks2_ln":
            import oracle
            a = bufs["assign"].cpu().numpy()
            s = bufs["scores"].cpu().numpy().astype(np.float64)
            n_tok = int(np.isin(a, ORACLE_EXPERTS).sum())
            g2, b2 = gam.cpu().numpy(), bet.cpu().numpy()
            res[name]["cpu_oracle"] = oracle_leg(lambda: oracle.layer_forward_ex(
                host["h64"], host["w64"], lambda n, e: W.as_f64(host["W1"][e], wl.dtype),
                lambda n, e: W.as_f64(host["W2"][e], wl.dtype), a, wl.act, mix="convex",
                sublayers=2, gamma=g2, beta=b2, ln_eps=1e-5, experts=list(ORACLE_EXPERTS),
                s=s), n_tok, "fp64 layer with two layer-norm blocks (convex)")
    del W1x2, W2x2
    return res


def layer_backward(wl, hd, wd, W1d, W2d, act, lay, host=None, reps=5):
    """base_layer_backward on the same inputs, with the assignment and the
    scores of the last balanced forward step and a seeded upstream gradient
    (eq. 1's residual mix). Median ms of the whole call and of its phases
    (library phase events): grouping + Z = X W1^T, dZ and the gate gradient
    (V = dY W2), dW2, dW1, and dX + dh + dw; each product is 2 T D F flops."""
    import torch
    from balanced_token_expert_amd import api
    from balanced_token_expert_amd import workloads as W
    T, E, D, F = wl.T, wl.E, wl.D, wl.F
    dt = api.BASE_BF16 if wl.dtype == "bf16" else api.BASE_F32
    with ThreadPoolExecutor(16) as ex:
        dy = np.concatenate(list(ex.map(lambda r0: W.gen_dy(wl, rows=slice(r0, min(T, r0 + 4096))),
                                        range(0, T, 4096))))
    dyd = to_dev(dy, wl.dtype)
    out = dict(dh=torch.empty_like(hd), dw=torch.empty_like(wd), dW1=torch.empty_like(W1d),
               dW2=torch.empty_like(W2d), stats=api.new_stats(),
               ws=api.workspace(api.BASE_OP_LAYER_BWD, T, E, D, F, dt))

    def call():
        api.base_layer_backward(hd, wd, W1d, W2d, act, lay["assign"], lay["scores"], dyd, **out)
    call()
    torch.cuda.synchronize()
    ev = HipEvents(6 * reps)
    for i in range(reps):
        api.base_set_phase_events(ev.block(6 * i), 6)
        call()
    torch.cuda.synchronize()
    api.base_set_phase_events(None, 0)
    names = ("group_z", "dz_gate", "dW2", "dW1", "dx_dw")
    ph = {n: float(np.median([ev.ms(6 * i + j, 6 * i + j + 1) for i in range(reps)]))
          for j, n in enumerate(names)}
    tot = float(np.median([ev.ms(6 * i, 6 * i + 5) for i in range(reps)]))
    flop = 2.0 * T * D * F
    st = api.read_stats(out["stats"])
    del out
    cpu = None
    if host is not None:
        import oracle
        a = lay["assign"].cpu().numpy()
        s = lay["scores"].cpu().numpy().astype(np.float64)
        n_tok = int(np.isin(a, ORACLE_EXPERTS).sum())
        cpu = oracle_leg(lambda: oracle.layer_backward(
            host["h64"], host["w64"], lambda e: W.as_f64(host["W1"][e], wl.dtype),
            lambda e: W.as_f64(host["W2"][e], wl.dtype), a, wl.act, W.as_f64(dy, wl.dtype),
            s=s, experts=list(ORACLE_EXPERTS)), n_tok, "fp64 gradients of the layer (residual)")
    return {"ms": round(tot, 4), "tokens_per_s": round(T / (tot * 1e-3), 1),
            "tflops": round(5 * flop / (tot * 1e-3) / 1e12, 1),
            "frac_bf16_peak": round(5 * flop / (tot * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "cpu_oracle": cpu,
            "phase_ms": {k: round(v, 4) for k, v in ph.items()},
            "phase_tflops": {k: round(flop / (v * 1e-3) / 1e12, 1) for k, v in ph.items()},
            "mix": "residual", "status": st.status}


def layer_backward_blocks(wl, hd, wd, W1d, W2d, act, lay, host=None, reps=3):
    """base_layer_backward_ex with experts of one and two sec. 4.1 blocks
    (layer norm, up, activation, down, residual; the convex mix), on the
    assignment and scores of the last balanced forward step; the blocks reuse
    the layer's expert matrices and seeded layer-norm parameters. Median ms of
    the whole call and of its phases (library phase events): grouping and the
    blocks' forward recompute (2 products per block, keeping Z and act(Z)),
    the gate, the blocks taken back (4 products per block: dZ, dW2, dW1, dX,
    and the layer-norm backward), and dh + dw; each product is 2 T D F
    flops."""
    import torch
    from balanced_token_expert_amd import api
    from balanced_token_expert_amd import workloads as W
    T, E, D, F = wl.T, wl.E, wl.D, wl.F
    with ThreadPoolExecutor(16) as ex:
        dy = np.concatenate(list(ex.map(lambda r0: W.gen_dy(wl, rows=slice(r0, min(T, r0 + 4096))),
                                        range(0, T, 4096))))
    dyd = to_dev(dy, wl.dtype)
    lnp = [W.gen_ln(wl, b) for b in range(2)]
    gam = torch.from_numpy(np.stack([g for g, _ in lnp])).cuda()
    bet = torch.from_numpy(np.stack([b for _, b in lnp])).cuda()
    flop = 2.0 * T * D * F
    res = {}
    for N in (1, 2):
        W1n = W1d[None].expand(N, *W1d.shape).contiguous()
        W2n = W2d[None].expand(N, *W2d.shape).contiguous()
        out = dict(dh=torch.empty_like(hd), dw=torch.empty_like(wd), dW1=torch.empty_like(W1n),
                   dW2=torch.empty_like(W2n), stats=api.new_stats())

        def call():
            api.base_layer_backward_ex(hd, wd, W1n, W2n, act, lay["assign"], lay["scores"], dyd,
                                       mix=api.BASE_MIX_CONVEX, sublayers=N, ln_gamma=gam[:N],
                                       ln_beta=bet[:N], **out)
        call()
        torch.cuda.synchronize()
        ev = HipEvents(6 * reps)
        for i in range(reps):
            api.base_set_phase_events(ev.block(6 * i), 6)
            call()
        torch.cuda.synchronize()
        api.base_set_phase_events(None, 0)
        med = lambda j0, j1: float(np.median([ev.ms(6 * i + j0, 6 * i + j1) for i in range(reps)]))
        tot = med(0, 5)
        ph = {"group_fwd": med(0, 1), "gate": med(1, 2), "blocks_back": med(2, 3),
              "dh_dw": med(4, 5)}
        st = api.read_stats(out["stats"])
        res[f"convex_blocks{N}_ln"] = {
            "ms": round(tot, 4), "tokens_per_s": round(T / (tot * 1e-3), 1),
            "products": 6 * N, "tflops": round(6 * N * flop / (tot * 1e-3) / 1e12, 1),
            "frac_bf16_peak": round(6 * N * flop / (tot * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "phase_ms": {k: round(v, 4) for k, v in ph.items()},
            "blocks_back_tflops": round(4 * N * flop / (ph["blocks_back"] * 1e-3) / 1e12, 1),
            "status": st.status}
        del out, W1n, W2n
        torch.cuda.empty_cache()
    if host is not None:
        import oracle
        a = lay["assign"].cpu().numpy()
        s = lay["scores"].cpu().numpy().astype(np.float64)
        n_tok = int(np.isin(a, ORACLE_EXPERTS).sum())
        g1, b1 = gam[:1].cpu().numpy(), bet[:1].cpu().numpy()
        res["convex_blocks1_ln"]["cpu_oracle"] = oracle_leg(lambda: oracle.layer_backward_ex(
            host["h64"], host["w64"], lambda n, e: W.as_f64(host["W1"][e], wl.dtype),
            lambda n, e: W.as_f64(host["W2"][e], wl.dtype), a, wl.act, W.as_f64(dy, wl.dtype),
            mix="convex", sublayers=1, gamma=g1, beta=b1, ln_eps=1e-5, s=s,
            experts=list(ORACLE_EXPERTS), store="bf16"), n_tok,
            "fp64 gradients of one layer-norm block (convex)")
    return res


def auction_solve(reps=10):
    """Auction solve ms on the mixture workload (device-resident fp32 scores)."""
    import torch
    from balanced_token_expert_amd import api
    from balanced_token_expert_amd import workloads as W
    import oracle
    wl = W.workload(2)
    h, w, _, _ = gen_inputs(wl)
    hd, wd = to_dev(h), to_dev(w)
    s = api.base_affinity(hd, wd)
    T, E = wl.T, wl.E
    c = api.cfg(wl.eps_start, wl.eps_end, wl.eps_factor, max_bids=100 * T * 5)
    bufs = dict(assign=torch.empty(T, dtype=torch.int32, device="cuda"),
                perm=torch.empty(T, dtype=torch.int32, device="cuda"),
                offsets=torch.empty(E + 1, dtype=torch.int32, device="cuda"),
                prices=torch.empty(E, dtype=torch.float64, device="cuda"),
                stats=api.new_stats(), ws=api.workspace(api.BASE_OP_AUCTION, T, E))
    for _ in range(2):
        api.base_assign_auction(s, c, **bufs)
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        api.base_assign_auction(s, c, **bufs)
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    st = api.read_stats(bufs["stats"])
    s32 = s.cpu().numpy().astype(np.float64)
    asg = bufs["assign"].cpu().numpy()
    p = bufs["prices"].cpu().numpy()
    k = T // E
    gap = oracle.dual_value(s32, p, k) - oracle.objective(s32, asg)
    balanced = bool((np.bincount(asg, minlength=E) == k).all())
    t0 = time.perf_counter()
    oracle.auction(s32, wl.eps_start, wl.eps_end, wl.eps_factor)
    t_cpu = time.perf_counter() - t0
    return {"value": round(float(np.median(times)), 4), "unit": "ms", "workload": wl.name,
            "eps": f"{wl.eps_start}->{wl.eps_end} x1/{wl.eps_factor}", "reps": reps,
            "min_ms": round(float(np.min(times)), 4), "status": st.status,
            "bids_per_phase": st.bids, "rounds_per_phase": st.rounds,
            "balanced": balanced, "dual_gap": gap, "dual_gap_bound": T * wl.eps_end,
            "cpu_oracle_ms": round(1e3 * t_cpu, 2), "cpu_oracle_cores": 1,
            "last_solve": solve_rates(times[-1], st, T, E)}


ORACLE_EXPERTS = tuple(range(8))


def oracle_leg(fn, tokens, what):
    """The oracle as it stands, timed on the host for a bounded sample (the
    tokens of eight experts), as tokens/s: the CPU reference beside a GPU leg."""
    t0 = time.perf_counter()
    fn()
    sec = time.perf_counter() - t0
    return {"value": round(tokens / sec, 1), "unit": "tokens/s",
            "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": f"{what}, the {tokens} tokens of experts {list(ORACLE_EXPERTS)}",
            "seconds": round(sec, 2)}


def solve_rates(ms, st, T, E):
    """Bid rate, time per dependent round and effective bandwidth of one
    solve: a bid reads a score row (4E bytes) and writes an fp64 bid; the
    result is T int32 ids and the permutation."""
    nb, nr = int(sum(st.bids)), int(sum(st.rounds))
    sec = ms * 1e-3
    alg = nb * (4 * E + 8) + 8 * T
    return {"ms": round(ms, 4), "bids": nb, "bids_per_s": round(nb / sec, 1),
            "dependent_rounds": nr, "us_per_dependent_round": round(1e6 * sec / max(nr, 1), 3),
            "algorithmic_bytes": alg, "effective_GBps": round(alg / sec / 1e9, 2)}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def copy_probe(nbytes=1 << 30, reps=4):
    """A plain device copy of known size (1 GiB read + 1 GiB written per
    launch): the reference point that scales the HBM byte counters of a
    profiler run (FETCH_SIZE / WRITE_SIZE) to bytes."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    print(json.dumps({"copy_bytes_each_way": nbytes, "ms": round(ms, 4),
                      "GB/s_read_plus_write": round(2 * nbytes / ms / 1e6, 1)}), flush=True)


def layer_bufs(T, E, D, F, dtype, hd):
    import torch
    from balanced_token_expert_amd import api
    return dict(assign=torch.empty(T, dtype=torch.int32, device="cuda"),
                scores=torch.empty((T, E), dtype=torch.float32, device="cuda"),
                perm=torch.empty(T, dtype=torch.int32, device="cuda"),
                out=torch.empty_like(hd), stats=api.new_stats(),
                ws=api.workspace(api.BASE_OP_LAYER, T, E, D, F,
                                 api.BASE_BF16 if dtype == "bf16" else api.BASE_F32))


def route_parts(aev, base, nph):
    """Bulk rounds, setup of the phase ends and the augmenting-path kernel,
    summed over the eps phases of one call (ms), and the tail launches."""
    bulk = sum(aev.ms(base + 4 * p, base + 4 * p + 1) for p in range(nph))
    setup = sum(aev.ms(base + 4 * p + 1, base + 4 * p + 2) for p in range(nph))
    tail = [aev.ms(base + 4 * p + 2, base + 4 * p + 3) for p in range(nph)]
    return bulk, setup, tail


def phase_rooflines(wl, ph, st, nph):
    """Every phase of the step against the bound that limits it, with the
    algorithmic bytes or flops of one call (per-unit figures: a score row
    and an fp64 bid per auction bid, 4E + 8 bytes; T*D*b + E*D*b + 4TE for
    the affinity; 4TE + 4T + 4E for greedy; 2TDF flops per expert product)."""
    T, E, D, F = wl.T, wl.E, wl.D, wl.F
    b = 2 if wl.dtype == "bf16" else 4
    out = {}
    if "affinity" in ph:
        byt = T * D * b + E * D * b + 4 * T * E
        out["affinity"] = {"bound": "hbm", "algorithmic_bytes": byt,
                           "achieved_GBps": round(byt / (ph["affinity"] * 1e-3) / 1e9, 1),
                           "frac": round(byt / (ph["affinity"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    nb = int(sum(st.bids))
    byt = nb * (4 * E + 8) + 8 * T
    out["route"] = {"bound": "hbm (latency-bound in practice)", "bids": nb,
                    "algorithmic_bytes": byt,
                    "achieved_GBps": round(byt / (ph["route"] * 1e-3) / 1e9, 2),
                    "frac": round(byt / (ph["route"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 5),
                    "bids_per_s": round(nb / (ph["route"] * 1e-3), 1),
                    "dependent_steps": int(sum(st.rounds)),
                    "us_per_dependent_step": round(1e3 * ph["route"] / max(sum(st.rounds), 1), 3)}
    nt = int(sum(st.tail))
    if "auction_tail" in ph and ph["auction_tail"] > 0:
        byt = nt * (4 * E + 8)
        out["auction_tail"] = {"bound": "hbm (latency-bound in practice)", "tokens_placed": nt,
                               "algorithmic_bytes": byt,
                               "achieved_GBps": round(byt / (ph["auction_tail"] * 1e-3) / 1e9, 3),
                               "frac": round(byt / (ph["auction_tail"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 6),
                               "us_per_token_placed": round(1e3 * ph["auction_tail"] / max(nt, 1), 2)}
    if F is not None:
        fl = 2.0 * T * D * F
        for k in ("ffn1", "ffn2"):
            if k in ph:
                out[k] = {"bound": "mfma", "algorithmic_flops": fl,
                          "achieved_TFLOPs": round(fl / (ph[k] * 1e-3) / 1e12, 1),
                          "frac": round(fl / (ph[k] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    if "greedy" in ph:
        byt = 4 * T * E + 4 * T + 4 * E
        out["greedy"] = {"bound": "hbm", "algorithmic_bytes": byt,
                         "achieved_GBps": round(byt / (ph["greedy"] * 1e-3) / 1e9, 1),
                         "frac": round(byt / (ph["greedy"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    return out


def run_step(wid, steps, warmup):
    """The timed step on one workload: base_layer_forward (BALANCED) plus
    greedy routing of the same scores. Returns the step time, the mean time
    of every phase (library events on the call's stream) and the auction's
    counters."""
    import torch
    from balanced_token_expert_amd import api
    from balanced_token_expert_amd import workloads as W
    wl = W.workload(wid)
    T, E, D, F = wl.T, wl.E, wl.D, wl.F
    h, w, W1, W2 = gen_inputs(wl)
    hd, wd = to_dev(h, wl.dtype), to_dev(w, wl.dtype)
    W1d, W2d = stack_dev(W1, wl.dtype), stack_dev(W2, wl.dtype)
    torch.cuda.synchronize()
    act = api.BASE_ACT_GELU if wl.act == "gelu" else api.BASE_ACT_RELU
    c = api.cfg(wl.eps_start, wl.eps_end, wl.eps_factor, max_bids=100 * T * 5)
    nph = n_phases(wl)
    lay = layer_bufs(T, E, D, F, wl.dtype, hd)
    gr = dict(assign=torch.empty(T, dtype=torch.int32, device="cuda"),
              counts=torch.empty(E, dtype=torch.int32, device="cuda"),
              perm=torch.empty(T, dtype=torch.int32, device="cuda"),
              offsets=torch.empty(E + 1, dtype=torch.int32, device="cuda"),
              ws=api.workspace(api.BASE_OP_GREEDY, T, E))
    nsteps = warmup + steps
    ev = HipEvents(6 * nsteps)
    aev = HipEvents(4 * nph * nsteps)
    gr_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(nsteps)]

    def step(i):
        api.base_set_phase_events(ev.block(6 * i), 6)
        api.base_set_auction_events(aev.block(4 * nph * i), 4 * nph)
        api.base_layer_forward(hd, wd, W1d, W2d, act, api.BASE_ROUTE_BALANCED, c, **lay)
        gr_ev[i][0].record()
        api.base_route_greedy(lay["scores"], **gr)
        gr_ev[i][1].record()

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    wall0 = time.perf_counter()
    for i in range(warmup, nsteps):
        step(i)
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    api.base_set_phase_events(None, 0)
    api.base_set_auction_events(None, 0)
    ms_step = t_start.elapsed_time(t_end) / steps
    ph = {p: [] for p in PHASES + ("greedy", "bulk_rounds", "tail_setup", "auction_tail")}
    tails = []
    for i in range(warmup, nsteps):
        b = 6 * i
        for j, p in enumerate(PHASES):
            ph[p].append(ev.ms(b + j, b + j + 1))
        ph["greedy"].append(gr_ev[i][0].elapsed_time(gr_ev[i][1]))
        bulk, setup, tail = route_parts(aev, 4 * nph * i, nph)
        ph["bulk_rounds"].append(bulk)
        ph["tail_setup"].append(setup)
        ph["auction_tail"].append(sum(tail))
        tails.extend(tail)
    avg = {p: float(np.mean(v)) for p, v in ph.items()}
    st = api.read_stats(lay["stats"])
    a = lay["assign"].cpu().numpy()
    balanced = bool((np.bincount(a, minlength=E) == T // E).all())
    gcount = gr["counts"].cpu().numpy()
    out = {"workload": wl.name, "T": T, "E": E, "D": D, "F": F, "dtype": wl.dtype, "act": wl.act,
           "eps": f"{wl.eps_start}->{wl.eps_end} x1/{wl.eps_factor}",
           "steps": steps, "warmup": warmup, "ms_per_step": round(ms_step, 4),
           "tokens_per_s": round(T / (ms_step * 1e-3), 1), "wall_s_timed": round(wall, 3),
           "phase_ms": {p: round(v, 4) for p, v in avg.items()},
           "auction": {"status": st.status, "balanced": balanced, "bids_per_phase": st.bids,
                       "depth_per_phase": st.rounds, "tail_tokens_per_phase": st.tail,
                       "tail_launch_ms_mean": round(float(np.mean(tails)), 4)},
           "greedy_load": {"max_over_mean": round(float(gcount.max() / (T / E)), 3)},
           "rooflines": phase_rooflines(wl, avg, st, nph)}
    extra = dict(wl=wl, h=h, w=w, W1=W1, W2=W2, hd=hd, wd=wd, W1d=W1d, W2d=W2d, act=act, c=c,
                 lay=lay, avg=avg, st=st, tails=tails)
    return out, extra


def run_assign(wid, steps, warmup):
    """The assignment-only workload: affinity, then base_assign_auction
    (with grouping); median solve ms and its parts (library events)."""
    import torch
    from balanced_token_expert_amd import api
    from balanced_token_expert_amd import workloads as W
    wl = W.workload(wid)
    T, E = wl.T, wl.E
    h, w, _, _ = gen_inputs(wl)
    hd, wd = to_dev(h, wl.dtype), to_dev(w, wl.dtype)
    c = api.cfg(wl.eps_start, wl.eps_end, wl.eps_factor, max_bids=100 * T * 5)
    nph = n_phases(wl)
    bufs = dict(assign=torch.empty(T, dtype=torch.int32, device="cuda"),
                perm=torch.empty(T, dtype=torch.int32, device="cuda"),
                offsets=torch.empty(E + 1, dtype=torch.int32, device="cuda"),
                prices=torch.empty(E, dtype=torch.float64, device="cuda"),
                stats=api.new_stats(), ws=api.workspace(api.BASE_OP_AUCTION, T, E))
    scores = torch.empty((T, E), dtype=torch.float32, device="cuda")
    nsteps = warmup + steps
    aev = HipEvents(4 * nph * nsteps)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(nsteps)]
    for i in range(nsteps):
        api.base_set_auction_events(aev.block(4 * nph * i), 4 * nph)
        evs[i][0].record()
        api.base_affinity(hd, wd, scores)
        evs[i][1].record()
        api.base_assign_auction(scores, c, **bufs)
        evs[i][2].record()
        torch.cuda.synchronize()
    api.base_set_auction_events(None, 0)
    aff = [evs[i][0].elapsed_time(evs[i][1]) for i in range(warmup, nsteps)]
    sol = [evs[i][1].elapsed_time(evs[i][2]) for i in range(warmup, nsteps)]
    parts = [route_parts(aev, 4 * nph * i, nph) for i in range(warmup, nsteps)]
    st = api.read_stats(bufs["stats"])
    asg = bufs["assign"].cpu().numpy()
    balanced = bool((np.bincount(asg, minlength=E) == T // E).all())
    avg = {"affinity": float(np.mean(aff)), "route": float(np.median(sol)),
           "bulk_rounds": float(np.mean([p[0] for p in parts])),
           "tail_setup": float(np.mean([p[1] for p in parts])),
           "auction_tail": float(np.mean([sum(p[2]) for p in parts]))}
    return {"workload": wl.name, "T": T, "E": E, "D": wl.D, "dtype": wl.dtype,
            "eps": f"{wl.eps_start}->{wl.eps_end} x1/{wl.eps_factor}", "reps": steps,
            "auction_solve_ms_median": round(float(np.median(sol)), 4),
            "auction_solve_ms_min": round(float(np.min(sol)), 4),
            "tokens_per_s": round(T / (float(np.median(np.add(aff, sol))) * 1e-3), 1),
            "phase_ms": {p: round(v, 4) for p, v in avg.items()},
            "auction": {"status": st.status, "balanced": balanced, "bids_per_phase": st.bids,
                        "depth_per_phase": st.rounds, "tail_tokens_per_phase": st.tail},
            "rooflines": phase_rooflines(wl, avg, st, nph)}


def n_phases(wl):
    n, eps = 1, wl.eps_start
    while eps > wl.eps_end:
        eps = max(eps / wl.eps_factor, wl.eps_end)
        n += 1
    return n


def dominant_roofline(wl, avg, st, tails):
    """Roofline of the kernel with the most time in the step: the auction's
    augmenting-path kernel (one launch per eps phase), an expert product or
    the affinity product (one launch each)."""
    T, E, D, F = wl.T, wl.E, wl.D, wl.F
    per_step = {"auction_tail": avg["auction_tail"], "ffn1": avg["ffn1"], "ffn2": avg["ffn2"],
                "affinity": avg["affinity"]}
    kern = max(per_step, key=per_step.get)
    if kern == "auction_tail":
        nt = int(sum(st.tail))
        launch_ms = float(np.mean(tails))
        per_launch = nt * (4 * E + 8) / max(len(st.tail), 1)
        ach = per_launch / (launch_ms * 1e-3) / 1e9
        traffic = measured_traffic("auction_tail", wl.name)
        return {"kernel": f"auc_ssp_kernel (augmenting paths that end each eps phase; "
                          f"{len(st.tail)} launches per step, {avg['auction_tail']:.3f} ms per step)",
                "bound": "hbm", "achieved": round(ach, 3), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBS, 7),
                "traffic": None if traffic is None else round(traffic),
                "algorithmic_bytes_per_launch": round(per_launch),
                "per_unit": f"{4 * E + 8} bytes per token placed (a score row and an fp64 bid)",
                "tokens_placed_per_step": nt, "avg_launch_ms": round(launch_ms, 4),
                "us_per_token_placed": round(1e3 * avg["auction_tail"] / max(nt, 1), 2)}
    if kern in ("ffn1", "ffn2"):
        fl = 2.0 * T * D * F
        ach = fl / (avg[kern] * 1e-3) / 1e12
        traffic = measured_traffic(kern, wl.name)
        return {"kernel": f"{kern} (expert GEMM {'1' if kern == 'ffn1' else '2'}, "
                          f"{E} experts x [{T // E}x{D if kern == 'ffn1' else F}]"
                          f"x[{D if kern == 'ffn1' else F}x{F if kern == 'ffn1' else D}])",
                "bound": "mfma", "achieved": round(ach, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                "traffic": None if traffic is None else round(traffic),
                "algorithmic_flops": fl, "avg_launch_ms": round(avg[kern], 4)}
    byt = T * D * 2 + E * D * 2 + 4 * T * E
    ach = byt / (avg["affinity"] * 1e-3) / 1e9
    return {"kernel": "affinity product", "bound": "hbm", "achieved": round(ach, 1),
            "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4),
            "traffic": None, "algorithmic_bytes": byt, "avg_launch_ms": round(avg["affinity"], 4)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", type=int, default=5, help=argparse.SUPPRESS)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true", help="only the headline workload")
    ap.add_argument("--no-auction", action="store_true")
    ap.add_argument("--no-variants", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--copy-probe", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--solve-only", type=int, default=0, metavar="REPS",
                    help="only the auction solve on the mixture workload, REPS timed solves "
                         "(for profiling the auction's kernels)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: this implementation runs on one GPU only (every expert resident on one "
              "MI355X, no collectives); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    from balanced_token_expert_amd import api

    if args.copy_probe:
        copy_probe()
        return
    if args.solve_only:
        api.load()
        print(json.dumps({"auction_solve_ms": auction_solve(reps=args.solve_only)}), flush=True)
        return
    api.load()
    torch.cuda.init()
    head, x = run_step(args.workload, args.steps, args.warmup)
    wl, avg, st = x["wl"], x["avg"], x["st"]
    T, E = wl.T, wl.E
    log(f"[bench] {wl.name}: {head['ms_per_step']} ms/step")
    res = {"metric": "BASE layer fwd tokens/s at 1 GPU + auction solve ms (T=16k, E=128)",
           "value": head["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": head["ms_per_step"],
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic (seeded numpy PCG64, shapes of the paper's setting)",
           "config": {"workload": wl.name, "T": T, "E": E, "D": wl.D, "F": wl.F, "act": wl.act,
                      "route": f"balanced auction eps {wl.eps_start}->{wl.eps_end} (factor "
                               f"{wl.eps_factor:g}) + greedy on the "
                               "same scores", "parallelism": "single GPU, all experts resident"},
           "phase_ms": head["phase_ms"], "auction": head["auction"],
           "greedy_load": head["greedy_load"],
           "roofline": dominant_roofline(wl, avg, st, x["tails"]),
           "phase_rooflines": head["rooflines"], "wall_s_timed": head["wall_s_timed"]}
    res["greedy_layer"] = greedy_layer(x["hd"], x["wd"], x["W1d"], x["W2d"], x["act"], T, E)
    host = None
    if not args.no_cpu_baseline:  # the oracle beside each GPU leg, on eight experts' tokens
        from balanced_token_expert_amd import workloads as W
        host = {"h64": W.as_f64(x["h"], wl.dtype), "w64": W.as_f64(x["w"], wl.dtype),
                "W1": x["W1"], "W2": x["W2"]}
    if not args.no_backward:
        res["layer_backward"] = layer_backward(wl, x["hd"], x["wd"], x["W1d"], x["W2d"], x["act"],
                                               x["lay"], host)
        res["layer_backward_blocks"] = layer_backward_blocks(wl, x["hd"], x["wd"], x["W1d"],
                                                             x["W2d"], x["act"], x["lay"], host)
    if not args.no_variants:
        res["layer_variants"] = layer_variants(wl, x["hd"], x["wd"], x["W1d"], x["W2d"], x["act"],
                                               x["c"], host)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, x["h"], x["w"], x["W1"], x["W2"])
    del x, host
    torch.cuda.empty_cache()
    if not args.no_configs:
        cfgs = {}
        for wid in (1, 3, 4):
            if wid == args.workload:
                continue
            o, _ = run_step(wid, 10, 2)
            cfgs[o["workload"]] = o
            log(f"[bench] {o['workload']}: {o['ms_per_step']} ms/step")
            torch.cuda.empty_cache()
        o = run_assign(2, 10, 2)
        cfgs[o["workload"]] = o
        log(f"[bench] {o['workload']}: solve {o['auction_solve_ms_median']} ms")
        cfgs[head["workload"]] = {k: v for k, v in head.items()}
        res["configs"] = cfgs
    if not args.no_auction:
        res["auction_solve_ms"] = auction_solve()
    if cpu is not None:
        res["cpu_baseline"] = cpu
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
