"""ctypes wrapper over the oracle's C solvers (oracle/solvers.c) -- TEST
INFRASTRUCTURE. Builds ``oracle/liborcsolvers.so`` with gcc on first use if
it is missing or older than its source.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "solvers.c")
_LIB = os.path.join(_HERE, "liborcsolvers.so")
_lib = None

_ERRORS = {-1: "invalid argument", -2: "T is not a multiple of E",
           -5: "bid cap reached before convergence", -7: "out of memory"}


class OracleError(RuntimeError):
    def __init__(self, code, what):
        super().__init__(f"{what}: {_ERRORS.get(code, code)}")
        self.code = code


def build(force: bool = False) -> str:
    """Compile the oracle's C solvers (gcc -O2, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        P = ctypes.c_void_p
        i32, i64, f64 = ctypes.c_int, ctypes.c_int64, ctypes.c_double
        lib.orc_auction.argtypes = [P, i32, i32, f64, f64, f64, i64, P, P, P, i32, P]
        lib.orc_hungarian.argtypes = [P, i32, i32, P]
        lib.orc_cycle_cancel.argtypes = [P, i32, i32, P, P, f64, i32, P]
        lib.orc_min_cycle.argtypes = [P, i32, i32, P, P]
        for f in (lib.orc_auction, lib.orc_hungarian, lib.orc_cycle_cancel, lib.orc_min_cycle):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _scores(s) -> np.ndarray:
    s = np.ascontiguousarray(s, dtype=np.float64)
    if s.ndim != 2:
        raise ValueError("scores must be T x E")
    if not np.isfinite(s).all():
        raise ValueError("scores must be finite (sanitize first)")
    return s


def auction(s, eps_start: float, eps_end: float, eps_factor: float = 10.0,
            max_bids: int = 0):
    """Token-side auction with eps-scaling, Gauss-Seidel order (one bidder at
    a time from a FIFO queue of unassigned tokens). Solves eq. 2 of "BASE
    Layers" (sec. 3.2.1) to within T * eps_end of the optimum.

    Returns dict(assign, prices, bids_per_phase, phases).
    """
    s = _scores(s)
    T, E = s.shape
    a = np.empty(T, dtype=np.int32)
    p = np.empty(E, dtype=np.float64)
    bids = np.zeros(64, dtype=np.int64)
    ph = ctypes.c_int(0)
    rc = _load().orc_auction(_ptr(s), T, E, float(eps_start), float(eps_end),
                             float(eps_factor), int(max_bids), _ptr(a), _ptr(p),
                             _ptr(bids), 64, ctypes.byref(ph))
    if rc:
        raise OracleError(rc, "orc_auction")
    return {"assign": a, "prices": p, "bids_per_phase": bids[:ph.value].copy(),
            "phases": ph.value}


def hungarian(s) -> np.ndarray:
    """Exact optimum of eq. 2 by the Hungarian method on the T x T expanded
    matrix (expert e owns k identical columns). O(T^3): T up to ~2048."""
    s = _scores(s)
    T, E = s.shape
    a = np.empty(T, dtype=np.int32)
    rc = _load().orc_hungarian(_ptr(s), T, E, _ptr(a))
    if rc:
        raise OracleError(rc, "orc_hungarian")
    return a


def cycle_cancel(s, a_start, tol: float = 1e-10, max_iter: int = 1_000_000):
    """Exact optimum of eq. 2 from any balanced start, by cancelling negative
    cycles of the expert exchange graph. Returns (assign, cycles_cancelled)."""
    s = _scores(s)
    T, E = s.shape
    a_in = np.ascontiguousarray(a_start, dtype=np.int32)
    a = np.empty(T, dtype=np.int32)
    n = ctypes.c_int(0)
    rc = _load().orc_cycle_cancel(_ptr(s), T, E, _ptr(a_in), _ptr(a), float(tol),
                                  int(max_iter), ctypes.byref(n))
    if rc:
        raise OracleError(rc, "orc_cycle_cancel")
    return a, n.value


def min_cycle_gap(s, a) -> float:
    """Minimum cycle cost of the exchange graph of the balanced assignment a.
    >= 0 iff a is optimal; then it is the optimum minus the second-best
    balanced objective (0: ties; +inf: E == 1)."""
    s = _scores(s)
    T, E = s.shape
    a = np.ascontiguousarray(a, dtype=np.int32)
    g = ctypes.c_double(0.0)
    rc = _load().orc_min_cycle(_ptr(s), T, E, _ptr(a), ctypes.byref(g))
    if rc:
        raise OracleError(rc, "orc_min_cycle")
    return g.value


def exact_assignment(s, start=None):
    """An optimal balanced assignment: Hungarian for T <= 1024, else cycle
    cancelling from ``start`` (default: a fine CPU auction's result)."""
    s = _scores(s)
    T, E = s.shape
    if T <= 1024 and start is None:
        return hungarian(s)
    if start is None:
        start = auction(s, 1.0, 1e-4)["assign"]
    return cycle_cancel(s, start)[0]
