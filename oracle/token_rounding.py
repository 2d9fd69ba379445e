"""numpy oracle of tile-aware token rounding.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): only the tests, the
smoke check and the bench's CPU-baseline leg use it.  It shares no code with
the HIP library and imports nothing from it.

Page cited: [P5] the SonicMoE article (gitcode.csdn.net), §6.5: the grouped
GEMM runs in row tiles, so an expert whose token count is not a tile multiple
pays for padding; token rounding makes routing aware of the tile size so that
per-expert counts sit closer to tile multiples (the article's summary reports
a 1.16x kernel-time gain in high-sparsity settings).  The page gives no rule;
the reading taken here (TR1-TR4):

* TR1 the tile M is the grouped GEMM's row tile (256 rows on the device).
* TR2 per expert, with c its kept count after the capacity cut: when c >= M
  and c mod M < M/2 (the nearest multiple of M lies below c), the count
  becomes M * floor(c / M); otherwise c stays.  A count whose nearest
  multiple lies above would need assignments added, which the fixed
  K-entries-per-token layout (ids, gates, inv_slot [T, K]) cannot hold; a
  count below one tile stays whole so that no expert is emptied.
* TR3 the dropped assignments are the expert's lowest-gate ones (the gates
  are taken as given, e.g. the device's fp32 gates, so both sides decide on
  the same numbers); among equal gates the larger token id goes first.
* TR4 a dropped assignment is handled like a capacity drop (R6 of the
  forward oracle): inv_slot = -1, the token's other gates are not
  renormalised, and the surviving slots of an expert keep ascending token
  order (R7).

Parity status: pinned by ``tests/test_oracle_rounding.py`` (a hand-worked
example in ``tests/golden/token_rounding_example.json``, the pure-Python twin
``brute.round_tokens_brute`` on random tiny cases with ties, invariants and
planted mistakes).
"""

from __future__ import annotations

import numpy as np


def rounded_count(c: int, M: int) -> int:
    """TR2: the count an expert keeps after rounding."""
    c, M = int(c), int(M)
    if c >= M and (c % M) < M / 2:
        return M * (c // M)
    return c


def round_tokens(meta: dict, ids, gates, M: int = 256) -> dict:
    """Apply TR1-TR4 to expert-major metadata (as ``moe_oracle.permute``
    returns it: counts, offsets, perm_token, inv_slot).  Returns the new
    counts, offsets, perm_token (first offsets[E] valid), inv_slot and the
    number of assignments dropped by the rounding."""
    ids = np.asarray(ids, dtype=np.int64)
    g = np.asarray(gates)
    offsets = np.asarray(meta["offsets"], dtype=np.int64)
    perm = np.asarray(meta["perm_token"], dtype=np.int64)
    inv = np.asarray(meta["inv_slot"], dtype=np.int64)
    T, K = ids.shape
    E = len(offsets) - 1
    new_counts = np.zeros(E, dtype=np.int64)
    segments = []
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        toks = perm[lo:hi]
        c = hi - lo
        r = rounded_count(c, M)
        if r < c:
            k_of = np.argmax(ids[toks] == e, axis=1)          # e's position in each token's list
            ge = g[toks, k_of]
            order = np.lexsort((-toks, ge))                   # gate ascending, then token descending
            drop = np.zeros(c, dtype=bool)
            drop[order[: c - r]] = True
            toks = toks[~drop]                                # survivors keep ascending token order
        new_counts[e] = len(toks)
        segments.append(toks)
    new_offsets = np.zeros(E + 1, dtype=np.int64)
    new_offsets[1:] = np.cumsum(new_counts)
    new_perm = np.full(T * K, -1, dtype=np.int64)
    new_inv = np.full((T, K), -1, dtype=np.int64)
    for e in range(E):
        base = int(new_offsets[e])
        for j, t in enumerate(segments[e]):
            new_perm[base + j] = t
            k = int(np.argmax(ids[t] == e))
            new_inv[t, k] = base + j
    dropped = int(offsets[E] - new_offsets[E])
    assert np.count_nonzero(new_inv >= 0) == int(new_offsets[E])
    assert dropped >= 0 and np.count_nonzero(inv >= 0) == int(offsets[E])
    return {
        "counts": new_counts.astype(np.int32),
        "offsets": new_offsets.astype(np.int32),
        "perm_token": new_perm.astype(np.int32),
        "inv_slot": new_inv.astype(np.int32),
        "dropped": dropped,
    }


def padded_rows(offsets, M: int = 256) -> int:
    """Rows the row tiles cover beyond the kept rows: sum over experts of
    M * ceil(c / M) - c (the padding that [P5] §6.5 is about)."""
    offsets = np.asarray(offsets, dtype=np.int64)
    c = np.diff(offsets)
    return int(np.sum((c + M - 1) // M * M - c))
