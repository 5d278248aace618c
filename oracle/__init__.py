"""CPU oracle for the BASE layer -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously-correct fp64 implementations of what the BASE layer
computes (Lewis et al., "BASE Layers: Simplifying Training of Large, Sparse
Models"): affinities, the balanced assignment of eq. 2 (CPU auction plus
exact Hungarian / cycle-cancelling solvers and optimality certificates),
greedy test-time routing (sec. 3.2.2), the expert grouping, the layer
output of eq. 1 with its variants, and the layer's gradients (grad.py).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. It shares no code with the GPU library
``balanced_token_expert_amd`` and imports nothing from it except the seeded
input generators (``balanced_token_expert_amd.workloads``), which hold no
arithmetic of the method.

Parity status of each function is stated in its docstring; every function
here is pinned by a ``-m "not gpu"`` test against closed forms, brute force,
invariants or an independent library routine.
"""
from .reference import (  # noqa: F401
    affinity, sanitize, greedy_route, canonical_perm, layer_forward,
    expert_ffn, gelu, sigmoid, dual_value, eps_cs_violation, objective,
    counts_of, layer_norm, expert_blocks, layer_forward_ex,
)
from .grad import (  # noqa: F401
    act_grad, layer_backward, layer_backward_ex, layer_norm_backward, stored,
)
from .solvers import (  # noqa: F401
    auction, hungarian, cycle_cancel, min_cycle_gap, exact_assignment,
    OracleError,
)
