"""Helpers for the GPU parity tests: move generated inputs to the device and
compute the oracle's reference values on the CPU."""
from __future__ import annotations

import numpy as np
import torch

from balanced_token_expert_amd import workloads as W


def to_dev(x: np.ndarray, dtype: str) -> torch.Tensor:
    """Host array from the generators -> contiguous CUDA tensor (bf16 from
    its uint16 bits, fp32 as is)."""
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.cuda()


def inputs(wl: W.Workload, rep: int = 0, experts: bool = True):
    host = W.gen_all(wl, rep, experts=experts)
    dev = {k: to_dev(v, wl.dtype) for k, v in host.items()}
    return host, dev


def f64(x: np.ndarray, dtype: str) -> np.ndarray:
    return W.as_f64(x, dtype)


def higham_bound(h64: np.ndarray, w64: np.ndarray) -> np.ndarray:
    """gamma_D * sum_d |h_d w_d| for every (t, e): Higham's bound on the error
    of an fp32 dot product of length D (unit roundoff 2^-24)."""
    D = h64.shape[1]
    u = 2.0 ** -24
    gamma = D * u / (1 - D * u)
    return gamma * (np.abs(h64) @ np.abs(w64).T)


def rel_err(y: np.ndarray, ref: np.ndarray) -> float:
    """max |y - ref| / max |ref| over the tensor."""
    return float(np.abs(y - ref).max() / max(np.abs(ref).max(), 1e-300))


def dev_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)

