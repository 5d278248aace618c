"""Thin ctypes binding of libbase_layer.so (include/base_layer.h).

Argument marshalling only: torch tensors give device memory and streams,
every step of the computation runs in the library's HIP kernels. The library
is loaded on first use; if it is missing, calls raise (there is no fallback).
Functions carry the C names; outputs not passed in are allocated with torch.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libbase_layer.so")

BASE_OK, BASE_ERR_INVALID_ARG, BASE_ERR_INDIVISIBLE = 0, -1, -2
BASE_ERR_UNSUPPORTED, BASE_ERR_HIP, BASE_ERR_NOT_CONVERGED = -3, -4, -5
BASE_ERR_NONFINITE, BASE_ERR_UNBALANCED, BASE_ERR_INVARIANT = -6, -8, -9
BASE_F32, BASE_BF16 = 0, 1
BASE_ACT_RELU, BASE_ACT_GELU = 0, 1
BASE_ROUTE_BALANCED, BASE_ROUTE_GREEDY, BASE_ROUTE_GIVEN = 0, 1, 2
BASE_OP_AFFINITY, BASE_OP_AUCTION, BASE_OP_GREEDY, BASE_OP_LAYER = 0, 1, 2, 3
BASE_OP_LAYER_EX = 4
BASE_OP_LAYER_BWD = 5
BASE_MIX_RESIDUAL, BASE_MIX_CONVEX = 0, 1
EXPORTED = ("base_workspace_bytes", "base_strerror", "base_affinity",
            "base_assign_auction", "base_route_greedy", "base_layer_forward",
            "base_layer_forward_ex", "base_layer_backward", "base_layer_backward_ex",
            "base_workspace_bytes_ex", "base_set_phase_events", "base_set_auction_events",
            "base_route_greedy_noalloc")
STATS_BYTES = 8 + 16 * 8 * 3


class AuctionCfg(ctypes.Structure):
    _fields_ = [("eps_start", ctypes.c_double), ("eps_end", ctypes.c_double),
                ("eps_factor", ctypes.c_double), ("max_bids", ctypes.c_int64)]


class LayerOpts(ctypes.Structure):
    _fields_ = [("mix", ctypes.c_int32), ("sublayers", ctypes.c_int32),
                ("ln_eps", ctypes.c_double), ("ln_gamma", ctypes.c_void_p),
                ("ln_beta", ctypes.c_void_p)]


class BaseError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where}: {strerror(code)} ({code})")
        self.code = code


_lib = None


def load(path: str = LIB_PATH):
    """Load the shared library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m balanced_token_expert_amd.build`")
    lib = ctypes.CDLL(path)
    P, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.base_workspace_bytes.argtypes = [i32, i64, i64, i64, i64, i32]
    lib.base_workspace_bytes.restype = ctypes.c_size_t
    lib.base_strerror.argtypes = [i32]
    lib.base_strerror.restype = ctypes.c_char_p
    lib.base_affinity.argtypes = [P, P, P, i64, i64, i64, i32, P]
    lib.base_assign_auction.argtypes = [P, i64, i64, AuctionCfg, P, P, P, P, P, P,
                                        ctypes.c_size_t, P]
    lib.base_route_greedy.argtypes = [P, i64, i64, P, P, P, P, P, ctypes.c_size_t, P]
    lib.base_layer_forward.argtypes = [P, P, P, P, i64, i64, i64, i64, i32, i32, i32,
                                       AuctionCfg, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.base_layer_forward_ex.argtypes = [P, P, P, P, i64, i64, i64, i64, i32, i32, i32,
                                          AuctionCfg, P, P, P, P, P, ctypes.POINTER(LayerOpts),
                                          P, ctypes.c_size_t, P]
    lib.base_layer_backward.argtypes = [P, P, P, P, i64, i64, i64, i64, i32, i32, P, P, P, P, P,
                                        P, P, P, ctypes.POINTER(LayerOpts), P, ctypes.c_size_t, P]
    lib.base_layer_backward_ex.argtypes = [P, P, P, P, i64, i64, i64, i64, i32, i32, P, P, P, P,
                                           P, P, P, P, P, P, ctypes.POINTER(LayerOpts), P,
                                           ctypes.c_size_t, P]
    lib.base_workspace_bytes_ex.argtypes = [i32, i64, i64, i64, i64, i32, i32]
    lib.base_workspace_bytes_ex.restype = ctypes.c_size_t
    lib.base_set_phase_events.argtypes = [P, i32]
    lib.base_set_auction_events.argtypes = [P, i32]
    lib.base_route_greedy_noalloc.argtypes = [P, i64, i64, P, P, P, P, P]
    for f in ("base_affinity", "base_assign_auction", "base_route_greedy", "base_layer_forward",
              "base_layer_forward_ex", "base_layer_backward", "base_layer_backward_ex",
              "base_set_phase_events", "base_set_auction_events", "base_route_greedy_noalloc"):
        getattr(lib, f).restype = ctypes.c_int
    _lib = lib
    return lib


def strerror(code: int) -> str:
    return load().base_strerror(int(code)).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BASE_BF16
    if t.dtype == torch.float32:
        return BASE_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _check(rc: int, where: str):
    if rc != BASE_OK:
        raise BaseError(rc, where)


def _dev(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous and on the GPU")


def _expect(t, shape, dtype, name):
    """The library sees plain pointers and trusts the sizes it is given: check
    each tensor's shape and dtype here, before anything is launched."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")


def _score_shapes(scores, assign=None, perm=None, offsets=None):
    """scores T x E fp32; assign, perm T int32; offsets E + 1 int32."""
    if scores.dim() != 2:
        raise ValueError("scores must be T x E")
    T, E = scores.shape
    _expect(scores, (T, E), torch.float32, "scores")
    _expect(assign, (T,), torch.int32, "assign")
    _expect(perm, (T,), torch.int32, "perm")
    _expect(offsets, (E + 1,), torch.int32, "offsets")
    return T, E


def _layer_shapes(h, w, W1, W2, nsub, assign=None, scores=None, io=(), ln=(), lngrad=()):
    """Shapes of a layer call: h T x D, w E x D, W1 [N x] E x F x D, W2
    [N x] E x D x F (N = nsub when nsub >= 1), assign T int32, scores T x E
    fp32; io: tensors shaped and typed like h / w / W1 / W2 (name, tensor,
    like); ln / lngrad: N x E x D fp32 tensors. Returns (T, E, D, F)."""
    if h.dim() != 2 or w.dim() != 2:
        raise ValueError("h and w must be 2-D")
    T, D = h.shape
    E = w.shape[0]
    lead = (nsub,) if nsub >= 1 else ()
    if W1.dim() != len(lead) + 3:
        raise ValueError(f"W1 must be {'N x ' if lead else ''}E x F x D")
    F = W1.shape[-2]
    _expect(w, (E, D), h.dtype, "w")
    _expect(W1, lead + (E, F, D), h.dtype, "W1")
    _expect(W2, lead + (E, D, F), h.dtype, "W2")
    _expect(assign, (T,), torch.int32, "assign")
    _expect(scores, (T, E), torch.float32, "scores")
    like = {"h": h, "w": w, "W1": W1, "W2": W2}
    for name, t, ref in io:
        _expect(t, like[ref].shape, h.dtype, name)
    for name, t in tuple(ln) + tuple(lngrad):
        _expect(t, (nsub, E, D), torch.float32, name)
    return T, E, D, F


def base_workspace_bytes(op: int, T: int, E: int, D: int = 0, F: int = 0,
                         dtype: int = BASE_BF16) -> int:
    return int(load().base_workspace_bytes(op, T, E, D, F, dtype))


def workspace(op, T, E, D=0, F=0, dtype=BASE_BF16, device="cuda"):
    n = base_workspace_bytes(op, T, E, D, F, dtype)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device)


@dataclass
class AuctionStats:
    status: int
    phases: int
    bids: list
    rounds: list
    tail: list


def read_stats(buf: torch.Tensor) -> AuctionStats:
    raw = buf.cpu()
    head = raw[:8].view(torch.int32).tolist()
    tail = raw[8:STATS_BYTES].view(torch.int64).tolist()
    ph = head[1]
    n = min(ph, 16)
    return AuctionStats(head[0], ph, tail[:16][:n], tail[16:32][:n], tail[32:48][:n])


def new_stats(device="cuda") -> torch.Tensor:
    return torch.zeros(STATS_BYTES, dtype=torch.uint8, device=device)


def cfg(eps_start=1.0, eps_end=1e-4, eps_factor=10.0, max_bids=0) -> AuctionCfg:
    return AuctionCfg(float(eps_start), float(eps_end), float(eps_factor), int(max_bids))


def base_affinity(h: torch.Tensor, w: torch.Tensor, scores=None, stream=None):
    _dev(h, w, scores)
    if h.dim() != 2 or w.dim() != 2:
        raise ValueError("h and w must be 2-D")
    T, D = h.shape
    E = w.shape[0]
    _expect(w, (E, D), h.dtype, "w")
    _expect(scores, (T, E), torch.float32, "scores")
    if scores is None:
        scores = torch.empty((T, E), dtype=torch.float32, device=h.device)
    rc = load().base_affinity(_ptr(h), _ptr(w), _ptr(scores), T, E, D, _dt(h), _stream(stream))
    _check(rc, "base_affinity")
    return scores


def base_assign_auction(scores: torch.Tensor, c: AuctionCfg, assign=None, perm=None,
                        offsets=None, prices=None, stats=None, ws=None, stream=None):
    _dev(scores, assign, perm, offsets, prices)
    T, E = _score_shapes(scores, assign=assign, perm=perm, offsets=offsets)
    _expect(prices, (E,), torch.float64, "prices")
    dev = scores.device
    assign = torch.empty(T, dtype=torch.int32, device=dev) if assign is None else assign
    perm = torch.empty(T, dtype=torch.int32, device=dev) if perm is None else perm
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev) if offsets is None else offsets
    prices = torch.empty(E, dtype=torch.float64, device=dev) if prices is None else prices
    stats = new_stats(dev) if stats is None else stats
    ws = workspace(BASE_OP_AUCTION, T, E, device=dev) if ws is None else ws
    rc = load().base_assign_auction(_ptr(scores), T, E, c, _ptr(assign), _ptr(perm),
                                    _ptr(offsets), _ptr(prices), _ptr(stats), _ptr(ws),
                                    ws.numel(), _stream(stream))
    _check(rc, "base_assign_auction")
    return {"assign": assign, "perm": perm, "offsets": offsets, "prices": prices,
            "stats": stats}


def base_route_greedy(scores: torch.Tensor, assign=None, counts=None, perm=None,
                      offsets=None, ws=None, stream=None, with_perm=True):
    _dev(scores, assign, counts, perm, offsets)
    T, E = _score_shapes(scores, assign=assign, perm=perm, offsets=offsets)
    _expect(counts, (E,), torch.int32, "counts")
    dev = scores.device
    assign = torch.empty(T, dtype=torch.int32, device=dev) if assign is None else assign
    counts = torch.empty(E, dtype=torch.int32, device=dev) if counts is None else counts
    if with_perm:
        perm = torch.empty(T, dtype=torch.int32, device=dev) if perm is None else perm
        offsets = torch.empty(E + 1, dtype=torch.int32, device=dev) if offsets is None else offsets
    ws = workspace(BASE_OP_GREEDY, T, E, device=dev) if ws is None else ws
    rc = load().base_route_greedy(_ptr(scores), T, E, _ptr(assign), _ptr(counts), _ptr(perm),
                                  _ptr(offsets), _ptr(ws), ws.numel(), _stream(stream))
    _check(rc, "base_route_greedy")
    return {"assign": assign, "counts": counts, "perm": perm, "offsets": offsets}


def base_route_greedy_noalloc(scores: torch.Tensor, assign: torch.Tensor, counts=None, perm=None,
                              offsets=None, stream=None):
    """base_route_greedy without a workspace (the library's static device
    scratch); the outputs are the caller's buffers: assign[T] int32, and
    optionally counts[E], perm[T] and offsets[E+1] int32."""
    _dev(scores, assign, counts, perm, offsets)
    T, E = _score_shapes(scores, assign=assign, perm=perm, offsets=offsets)
    _expect(counts, (E,), torch.int32, "counts")
    if assign is None:
        raise ValueError("assign is required")
    rc = load().base_route_greedy_noalloc(_ptr(scores), T, E, _ptr(assign), _ptr(counts),
                                          _ptr(perm), _ptr(offsets), _stream(stream))
    _check(rc, "base_route_greedy_noalloc")
    return {"assign": assign, "counts": counts, "perm": perm, "offsets": offsets}


def base_layer_forward(h, w, W1, W2, act: int, mode: int, c: AuctionCfg = None, assign=None,
                       scores=None, perm=None, out=None, stats=None, ws=None, stream=None,
                       want_scores=True):
    _dev(h, w, W1, W2, assign, scores, perm, out)
    T, E, D, F = _layer_shapes(h, w, W1, W2, 0, assign, scores, io=(("out", out, "h"),))
    _expect(perm, (T,), torch.int32, "perm")
    dev = h.device
    dt = _dt(h)
    c = cfg() if c is None else c
    if assign is None:
        if mode == BASE_ROUTE_GIVEN:
            raise ValueError("GIVEN routing needs an assignment")
        assign = torch.empty(T, dtype=torch.int32, device=dev)
    if scores is None and want_scores:
        scores = torch.empty((T, E), dtype=torch.float32, device=dev)
    perm = torch.empty(T, dtype=torch.int32, device=dev) if perm is None else perm
    out = torch.empty_like(h) if out is None else out
    stats = new_stats(dev) if stats is None else stats
    ws = workspace(BASE_OP_LAYER, T, E, D, F, dt, device=dev) if ws is None else ws
    rc = load().base_layer_forward(_ptr(h), _ptr(w), _ptr(W1), _ptr(W2), T, E, D, F, dt, act,
                                   mode, c, _ptr(assign), _ptr(scores), _ptr(perm), _ptr(out),
                                   _ptr(stats), _ptr(ws), ws.numel(), _stream(stream))
    _check(rc, "base_layer_forward")
    return {"out": out, "assign": assign, "scores": scores, "perm": perm, "stats": stats}


def base_layer_forward_ex(h, w, W1, W2, act: int, mode: int, c: AuctionCfg = None, mix: int = 0,
                          sublayers: int = 0, ln_gamma=None, ln_beta=None, ln_eps: float = 1e-5,
                          assign=None, scores=None, perm=None, out=None, stats=None, ws=None,
                          stream=None, want_scores=True):
    """The layer variants: W1 / W2 are E x F x D / E x D x F (sublayers = 0)
    or N x E x F x D / N x E x D x F; ln_gamma / ln_beta N x E x D fp32 or
    None."""
    _dev(h, w, W1, W2, assign, scores, perm, out, ln_gamma, ln_beta)
    T, E, D, F = _layer_shapes(h, w, W1, W2, sublayers, assign, scores,
                               io=(("out", out, "h"),),
                               ln=(("ln_gamma", ln_gamma), ("ln_beta", ln_beta)))
    _expect(perm, (T,), torch.int32, "perm")
    dev = h.device
    dt = _dt(h)
    c = cfg() if c is None else c
    if assign is None:
        if mode == BASE_ROUTE_GIVEN:
            raise ValueError("GIVEN routing needs an assignment")
        assign = torch.empty(T, dtype=torch.int32, device=dev)
    if scores is None and want_scores:
        scores = torch.empty((T, E), dtype=torch.float32, device=dev)
    perm = torch.empty(T, dtype=torch.int32, device=dev) if perm is None else perm
    out = torch.empty_like(h) if out is None else out
    stats = new_stats(dev) if stats is None else stats
    ws = workspace(BASE_OP_LAYER_EX, T, E, D, F, dt, device=dev) if ws is None else ws
    opts = LayerOpts(int(mix), int(sublayers), float(ln_eps),
                     None if ln_gamma is None else ln_gamma.data_ptr(),
                     None if ln_beta is None else ln_beta.data_ptr())
    rc = load().base_layer_forward_ex(_ptr(h), _ptr(w), _ptr(W1), _ptr(W2), T, E, D, F, dt, act,
                                      mode, c, _ptr(assign), _ptr(scores), _ptr(perm), _ptr(out),
                                      _ptr(stats), ctypes.byref(opts), _ptr(ws), ws.numel(),
                                      _stream(stream))
    _check(rc, "base_layer_forward_ex")
    return {"out": out, "assign": assign, "scores": scores, "perm": perm, "stats": stats}


def base_layer_backward(h, w, W1, W2, act: int, assign, scores, dy, mix: int = 0, dh=None,
                        dw=None, dW1=None, dW2=None, stats=None, ws=None, stream=None):
    """Gradients of the plain-expert layer for the upstream gradient dy, the
    assignment fixed; returns dict(dh, dw, dW1, dW2, stats), each gradient
    in the dtype of h."""
    _dev(h, w, W1, W2, assign, scores, dy, dh, dw, dW1, dW2)
    T, E, D, F = _layer_shapes(h, w, W1, W2, 0, assign, scores,
                               io=(("dy", dy, "h"), ("dh", dh, "h"), ("dw", dw, "w"),
                                   ("dW1", dW1, "W1"), ("dW2", dW2, "W2")))
    dev = h.device
    dt = _dt(h)
    dh = torch.empty_like(h) if dh is None else dh
    dw = torch.empty_like(w) if dw is None else dw
    dW1 = torch.empty_like(W1) if dW1 is None else dW1
    dW2 = torch.empty_like(W2) if dW2 is None else dW2
    stats = new_stats(dev) if stats is None else stats
    ws = workspace(BASE_OP_LAYER_BWD, T, E, D, F, dt, device=dev) if ws is None else ws
    opts = LayerOpts(int(mix), 0, 1e-5, None, None)
    rc = load().base_layer_backward(_ptr(h), _ptr(w), _ptr(W1), _ptr(W2), T, E, D, F, dt, act,
                                    _ptr(assign), _ptr(scores), _ptr(dy), _ptr(dh), _ptr(dw),
                                    _ptr(dW1), _ptr(dW2), _ptr(stats), ctypes.byref(opts),
                                    _ptr(ws), ws.numel(), _stream(stream))
    _check(rc, "base_layer_backward")
    return {"dh": dh, "dw": dw, "dW1": dW1, "dW2": dW2, "stats": stats}


def base_workspace_bytes_ex(op: int, T: int, E: int, D: int, F: int, dtype: int,
                            sublayers: int) -> int:
    return int(load().base_workspace_bytes_ex(op, T, E, D, F, dtype, sublayers))


def base_layer_backward_ex(h, w, W1, W2, act: int, assign, scores, dy, mix: int = 0,
                           sublayers: int = 0, ln_gamma=None, ln_beta=None, ln_eps: float = 1e-5,
                           dh=None, dw=None, dW1=None, dW2=None, dgamma=None, dbeta=None,
                           want_ln_grads=True, stats=None, ws=None, stream=None):
    """base_layer_backward for the layer variants: W1 / W2 as for
    base_layer_forward_ex; returns dict(dh, dw, dW1, dW2, dgamma, dbeta,
    stats) (dgamma / dbeta N x E x D fp32 when sublayers >= 1)."""
    _dev(h, w, W1, W2, assign, scores, dy, dh, dw, dW1, dW2, ln_gamma, ln_beta, dgamma, dbeta)
    T, E, D, F = _layer_shapes(h, w, W1, W2, sublayers, assign, scores,
                               io=(("dy", dy, "h"), ("dh", dh, "h"), ("dw", dw, "w"),
                                   ("dW1", dW1, "W1"), ("dW2", dW2, "W2")),
                               ln=(("ln_gamma", ln_gamma), ("ln_beta", ln_beta)),
                               lngrad=(("dgamma", dgamma), ("dbeta", dbeta)))
    dev = h.device
    dt = _dt(h)
    dh = torch.empty_like(h) if dh is None else dh
    dw = torch.empty_like(w) if dw is None else dw
    dW1 = torch.empty_like(W1) if dW1 is None else dW1
    dW2 = torch.empty_like(W2) if dW2 is None else dW2
    if sublayers >= 1 and want_ln_grads:
        shape = (sublayers, E, D)
        dgamma = torch.empty(shape, dtype=torch.float32, device=dev) if dgamma is None else dgamma
        dbeta = torch.empty(shape, dtype=torch.float32, device=dev) if dbeta is None else dbeta
    stats = new_stats(dev) if stats is None else stats
    if ws is None:
        n = base_workspace_bytes_ex(BASE_OP_LAYER_BWD, T, E, D, F, dt, sublayers)
        ws = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
    opts = LayerOpts(int(mix), int(sublayers), float(ln_eps),
                     None if ln_gamma is None else ln_gamma.data_ptr(),
                     None if ln_beta is None else ln_beta.data_ptr())
    rc = load().base_layer_backward_ex(_ptr(h), _ptr(w), _ptr(W1), _ptr(W2), T, E, D, F, dt, act,
                                       _ptr(assign), _ptr(scores), _ptr(dy), _ptr(dh), _ptr(dw),
                                       _ptr(dW1), _ptr(dW2), _ptr(dgamma), _ptr(dbeta),
                                       _ptr(stats), ctypes.byref(opts), _ptr(ws), ws.numel(),
                                       _stream(stream))
    _check(rc, "base_layer_backward_ex")
    return {"dh": dh, "dw": dw, "dW1": dW1, "dW2": dW2, "dgamma": dgamma, "dbeta": dbeta,
            "stats": stats}


def base_set_phase_events(events, n: int):
    """events: a ctypes array of hipEvent_t handles (or None to stop)."""
    _check(load().base_set_phase_events(events, int(n)), "base_set_phase_events")


def base_set_auction_events(events, n: int):
    """events: a ctypes array of hipEvent_t handles, four per eps phase (or
    None to stop)."""
    _check(load().base_set_auction_events(events, int(n)), "base_set_auction_events")
