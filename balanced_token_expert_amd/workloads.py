"""Seeded synthetic inputs for the BASE-layer forward.

This module is shared by the GPU path's tests and benchmark and by the CPU
oracle's tests. It holds only random-number generation and bf16 bit
handling: none of the layer's arithmetic lives here.

Workloads follow the problem statement of BASE layers (Lewis et al.,
"BASE Layers: Simplifying Training of Large, Sparse Models", sec. 3.1 and
3.2.1): T tokens of width D, E expert centroids, an expert FFN D -> F -> D.
The five named workloads below are synthetic stand-ins shaped like the
paper's setting (model width 2048, FFN width 4x, 128 experts, sec. 4.1); no
dataset is used.

Generation: numpy PCG64 seeded with ``SeedSequence([1000*wid + 100*rep +
tensor_id, chunk])`` where ``chunk`` is the expert index for per-expert
tensors and the 2048-row block index for token tensors, so that any expert's
weights or any block of tokens can be regenerated on its own. Samples are
drawn in fp32 and, for bf16 workloads, rounded to bf16 by
round-to-nearest-even. ``N(0, v)`` below names the variance ``v``.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

# tensor ids inside a workload's seed space
TID_H, TID_W, TID_W1, TID_W2, TID_AUX, TID_DY = 0, 1, 2, 3, 4, 5
ROW_CHUNK = 2048  # token rows per generator chunk
BLOCK_CHUNK = 100000  # chunk offset of an expert's feed-forward block
LN_CHUNK = 200000     # chunk offset of the layer-norm parameters (TID_AUX)


@dataclass(frozen=True)
class Workload:
    wid: int            # workload id (1..5), part of every seed
    name: str
    T: int
    E: int
    D: int
    F: Optional[int]    # None: assignment only, no expert FFN
    dtype: str          # "f32" or "bf16"
    act: str            # "relu" or "gelu"
    kind: str           # "iid", "mixture" or "skew"
    eps_start: float
    eps_end: float
    eps_factor: float = 10.0   # eps-scaling: eps_start, eps_start/f, ..., eps_end
    note: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def k(self) -> int:
        return self.T // self.E


WORKLOADS = {
    1: Workload(1, "tiny_fp32_t512_e8", 512, 8, 64, 256, "f32", "relu", "iid",
                1e-4, 1e-4,
                note="h~N(0,1), w~N(0,1/D), W1~N(0,1/D), W2~N(0,1/F); ReLU"),
    2: Workload(2, "mixture_assign_t16k_e128", 16384, 128, 1024, None, "bf16",
                "gelu", "mixture", 1.0, 1e-4,
                note="h from a 16-component Gaussian mixture (means N(0,I), "
                     "std 0.3), w~N(0,1/D); assignment only"),
    3: Workload(3, "layer_t16k_e64_d1536", 16384, 64, 1536, 6144, "bf16",
                "gelu", "iid", 1.0, 1e-4, 100.0,
                note="h~N(0,1), w,W1~N(0,1/D), W2~N(0,1/F); GELU"),
    4: Workload(4, "skew_t32k_e128_d1024", 32768, 128, 1024, 4096, "bf16",
                "gelu", "skew", 1.0, 1e-4, 30.0,
                note="80% of tokens at 3*w0/|w0| + N(0,0.1), rest N(0,1); "
                     "w,W1~N(0,1/D), W2~N(0,1/F); GELU"),
    5: Workload(5, "large_t64k_e128_d2048", 65536, 128, 2048, 8192, "bf16",
                "gelu", "iid", 1.0, 1e-4, 100.0,
                note="h~N(0,1), w,W1~N(0,1/D), W2~N(0,1/F); GELU; "
                     "about 8.6 GB of expert weights"),
}


def workload(wid: int) -> Workload:
    return WORKLOADS[wid]


def custom(T, E, D, F=None, dtype="bf16", act="gelu", kind="iid", wid=900,
           eps_start=1.0, eps_end=1e-4, name=None) -> Workload:
    """A workload of arbitrary shape with the i.i.d./mixture/skew recipes."""
    return Workload(wid, name or f"custom_t{T}_e{E}_d{D}_f{F}", T, E, D, F,
                    dtype, act, kind, eps_start, eps_end)


# ----------------------------------------------------------------- bf16 bits

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round to nearest, ties to even); returns uint16."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))
    out = ((b + rounding) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    u = np.ascontiguousarray(u, dtype=np.uint16)
    return (u.astype(np.uint32) << np.uint32(16)).view(np.float32)


def as_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp64 values of stored inputs (uint16 bf16 bits or fp32)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def _store(x32: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x32) if dtype == "bf16" else x32.astype(np.float32)


def _rng(wl: Workload, rep: int, tid: int, chunk: int) -> np.random.Generator:
    seed = 1000 * wl.wid + 100 * rep + tid
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, chunk])))


def _normal(rng, shape, std) -> np.ndarray:
    return (rng.standard_normal(shape, dtype=np.float32) * np.float32(std))


# ----------------------------------------------------------------- tensors

def gen_centroids(wl: Workload, rep: int = 0) -> np.ndarray:
    """Expert centroids w (E x D), N(0, 1/D)."""
    rng = _rng(wl, rep, TID_W, 0)
    return _store(_normal(rng, (wl.E, wl.D), 1.0 / np.sqrt(wl.D)), wl.dtype)


def gen_w1(wl: Workload, expert: int, rep: int = 0) -> np.ndarray:
    """Expert ``expert``'s first FFN matrix (F x D, [out, in]), N(0, 1/D)."""
    rng = _rng(wl, rep, TID_W1, expert)
    return _store(_normal(rng, (wl.F, wl.D), 1.0 / np.sqrt(wl.D)), wl.dtype)


def gen_w2(wl: Workload, expert: int, rep: int = 0) -> np.ndarray:
    """Expert ``expert``'s second FFN matrix (D x F, [out, in]), N(0, 1/F)."""
    rng = _rng(wl, rep, TID_W2, expert)
    return _store(_normal(rng, (wl.D, wl.F), 1.0 / np.sqrt(wl.F)), wl.dtype)


def gen_block_w1(wl: Workload, block: int, expert: int, rep: int = 0) -> np.ndarray:
    """First matrix of feed-forward block ``block`` of an expert (F x D);
    block 0 is ``gen_w1``."""
    rng = _rng(wl, rep, TID_W1, block * BLOCK_CHUNK + expert)
    return _store(_normal(rng, (wl.F, wl.D), 1.0 / np.sqrt(wl.D)), wl.dtype)


def gen_block_w2(wl: Workload, block: int, expert: int, rep: int = 0) -> np.ndarray:
    """Second matrix of feed-forward block ``block`` of an expert (D x F);
    block 0 is ``gen_w2``."""
    rng = _rng(wl, rep, TID_W2, block * BLOCK_CHUNK + expert)
    return _store(_normal(rng, (wl.D, wl.F), 1.0 / np.sqrt(wl.F)), wl.dtype)


def gen_ln(wl: Workload, block: int, rep: int = 0):
    """Layer-norm scales and shifts of block ``block`` for every expert (two
    E x D fp32 arrays): 1 + 0.1 N(0,1) and 0.1 N(0,1), away from the identity
    initialisation so that both take part."""
    rng = _rng(wl, rep, TID_AUX, LN_CHUNK + block)
    g = (1.0 + 0.1 * rng.standard_normal((wl.E, wl.D))).astype(np.float32)
    b = (0.1 * rng.standard_normal((wl.E, wl.D))).astype(np.float32)
    return g, b


def _skew_rows(wl: Workload, rep: int) -> np.ndarray:
    """Sorted positions of the round(0.8*T) tokens drawn near centroid 0."""
    n = int(round(0.8 * wl.T))
    rng = _rng(wl, rep, TID_AUX, 2)
    return np.sort(rng.permutation(wl.T)[:n])


def _mixture_params(wl: Workload, rep: int):
    rng_mu = _rng(wl, rep, TID_AUX, 0)
    mu = rng_mu.standard_normal((16, wl.D), dtype=np.float32)
    rng_c = _rng(wl, rep, TID_AUX, 1)
    comp = rng_c.integers(0, 16, size=wl.T)
    return mu, comp


def gen_tokens(wl: Workload, rep: int = 0, rows: Optional[slice] = None,
               centroids: Optional[np.ndarray] = None) -> np.ndarray:
    """Token features h (T x D) or a contiguous row range of them."""
    r0 = 0 if rows is None or rows.start is None else rows.start
    r1 = wl.T if rows is None or rows.stop is None else rows.stop
    assert 0 <= r0 <= r1 <= wl.T
    out = np.empty((r1 - r0, wl.D), dtype=np.float32)
    if wl.kind == "mixture":
        mu, comp = _mixture_params(wl, rep)
    if wl.kind == "skew":
        skew = np.zeros(wl.T, dtype=bool)
        skew[_skew_rows(wl, rep)] = True
        w = centroids if centroids is not None else gen_centroids(wl, rep)
        w0 = as_f64(w[0], wl.dtype)
        anchor = (3.0 * w0 / np.linalg.norm(w0)).astype(np.float32)
    c0, c1 = r0 // ROW_CHUNK, (r1 + ROW_CHUNK - 1) // ROW_CHUNK
    for c in range(c0, c1):
        lo, hi = c * ROW_CHUNK, min(wl.T, (c + 1) * ROW_CHUNK)
        z = _rng(wl, rep, TID_H, c).standard_normal((hi - lo, wl.D), dtype=np.float32)
        if wl.kind == "mixture":
            z = mu[comp[lo:hi]] + np.float32(0.3) * z
        elif wl.kind == "skew":
            m = skew[lo:hi]
            z[m] = anchor[None, :] + np.float32(np.sqrt(0.1)) * z[m]
        a, b = max(lo, r0), min(hi, r1)
        out[a - r0:b - r0] = z[a - lo:b - lo]
    return _store(out, wl.dtype)


def gen_dy(wl: Workload, rep: int = 0, rows: Optional[slice] = None) -> np.ndarray:
    """Upstream gradient of the layer output (T x D, or a contiguous row
    range): N(0, 1) entries in the workload's dtype, drawn per row chunk."""
    r0 = 0 if rows is None or rows.start is None else rows.start
    r1 = wl.T if rows is None or rows.stop is None else rows.stop
    assert 0 <= r0 <= r1 <= wl.T
    out = np.empty((r1 - r0, wl.D), dtype=np.float32)
    c0, c1 = r0 // ROW_CHUNK, (r1 + ROW_CHUNK - 1) // ROW_CHUNK
    for c in range(c0, c1):
        lo, hi = c * ROW_CHUNK, min(wl.T, (c + 1) * ROW_CHUNK)
        z = _rng(wl, rep, TID_DY, c).standard_normal((hi - lo, wl.D), dtype=np.float32)
        a, b = max(lo, r0), min(hi, r1)
        out[a - r0:b - r0] = z[a - lo:b - lo]
    return _store(out, wl.dtype)


def gen_all(wl: Workload, rep: int = 0, experts: bool = True) -> dict:
    """All inputs of a workload as host arrays (bf16 as uint16 bits)."""
    w = gen_centroids(wl, rep)
    d = {"w": w, "h": gen_tokens(wl, rep, centroids=w)}
    if experts and wl.F is not None:
        d["W1"] = np.stack([gen_w1(wl, e, rep) for e in range(wl.E)])
        d["W2"] = np.stack([gen_w2(wl, e, rep) for e in range(wl.E)])
    return d
