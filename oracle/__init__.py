"""CPU oracle for the single-GPU MoE layer forward.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package.  The product path (the HIP library and its Python binding) never
imports it, and this package imports nothing from the product path.

Modules
-------
moe_oracle
    Plain numpy float64 implementation of each step of the layer (router
    logits, softmax + top-K selection + renormalised gates, per-expert
    histogram, capacity, exclusive scan, scatter index, SwiGLU expert FFN,
    gate-weighted combine), vectorised only where a library primitive (a
    matmul, a stable sort) is a whole step.
brute
    Pure-Python loops over every (token, expert) pair for tiny inputs, written
    independently of ``moe_oracle``; it pins the oracle.
moe_backward
    numpy float64 backward of the layer (training), pinned by finite
    differences of ``moe_oracle``'s loss.
token_rounding
    tile-aware token rounding of the expert-major metadata (readings TR1-TR4),
    pinned by a hand-worked example and ``brute.round_tokens_brute``.
omni_oracle
    the atomic-expert layer with a Cartesian router (readings O1-O7), pinned
    by ``brute.brute_omni_forward`` and the exactness of the pruned search.

Parity status of each function is listed in the module docstrings; every
function is pinned by at least one ``-m "not gpu"`` test (worked example,
brute force, closed form or invariant).  The published performance figures
of the pages are the only item with "parity unpinned".
"""

from . import moe_oracle, brute, moe_backward, token_rounding, omni_oracle  # noqa: F401
