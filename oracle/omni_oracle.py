"""numpy float64 oracle of the OmniMoE-style layer: atomic (rank-1) experts
with a Cartesian-product router and expert-centric execution.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): only the tests, the
smoke check and the bench's CPU-baseline leg use it.  It shares no code with
the HIP library and imports nothing from it.

Page cited: [P2] "MoE 的两个上游创新：Routing-Free 与 OmniMoE"
(chatdocs.ruinique.com), part 2:

* §2.1 an atomic expert is two d-vectors, E_i(x) = sigma(x . w_in_i) w_out_i,
  a rank-1 FFN piece; the experts are stacked into two [N, d] tables;
* §2.2 the Cartesian-product router: the id i splits into (i_r, i_c) with
  N = N_r * N_c; p_r = x W_r, p_c = x W_c; the score of (i_r, i_c) is the sum
  of the two LogSoftmax values; the page's pruning first keeps the top
  k0 = min(sqrt(N), K) of each axis and searches the top-K in the k0 x k0
  candidates;
* §2.3 expert-centric scheduling: the L*K (token, expert) tasks are ordered
  by (expert, token) and run expert by expert (each expert's vectors are
  read once for all its tokens; reuse eta = L*K / |E_active|), and the
  outputs are summed back per token.

Readings taken where the page is silent (O1-O7, repeated where used):

* O1 sigma = SiLU; the routing weight g plays the gating role of SwiGLU (an
  atomic expert holds only the two vectors the page names).
* O2 the atomic id is i = i_r * N_c + i_c.
* O3 scores S = ls_r[i_r] + ls_c[i_c], ls = log-softmax of p over its axis.
* O4 selection: the K largest S by (S desc, id asc) (R2 of the forward
  oracle); gates: softmax over the K selected S (renormalised over the
  selection, R1), i.e. g proportional to P_r * P_c.
* O5 pruning: keep the top min(K, N_r) rows and top min(K, N_c) columns,
  then take the top K of their sums.  This returns exactly the ids of O4: if
  (r, c) is in the top K, every row r' ranked above r (larger ls_r, or equal
  with a lower id) gives (r', c) ranked above (r, c), so r is among the top
  K rows, and likewise c.  For the square grid the page assumes
  (N_r = N_c = sqrt(N)) this is its k0 = min(sqrt(N), K); on a non-square
  grid that k0 can cut an axis below min(K, N_axis) and lose pairs (a pin
  shows one), so the per-axis form is the one taken.  The device always
  prunes.
* O6 no capacity: every task is kept; y_t = sum_k g_k E_{id_k}(x_t).
* O7 tasks are ordered by (expert, token): ``moe_oracle.permute`` with
  E = N and C = T gives the metadata (counts, offsets, perm_token, inv_slot).

Decisions on device numbers: given the device's fp32 log-softmax rows, the
scores are added in float32 (as the device does) and the selection is made
on those float32 sums; gates are then taken in float64 from them.

Parity status: pinned by ``tests/test_oracle_omni.py`` (the pure-Python twin
``brute.brute_omni_forward`` on tiny layers, pruned == full search on random
and tied scores, closed forms and invariants, planted mistakes).
"""

from __future__ import annotations

import math

import numpy as np

from . import moe_oracle as mo


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def log_softmax(p) -> np.ndarray:
    """Row-wise log-softmax (O3)."""
    p = _f64(p)
    m = np.max(p, axis=1, keepdims=True)
    return p - m - np.log(np.sum(np.exp(p - m), axis=1, keepdims=True))


def axis_scores(X, W_r, W_c):
    """[P2] §2.2: ls_r = log-softmax(x W_r), ls_c = log-softmax(x W_c)."""
    X = _f64(X)
    return log_softmax(X @ _f64(W_r)), log_softmax(X @ _f64(W_c))


def _grid(lr, lc, float32: bool):
    if float32:
        return np.asarray(lr, np.float32)[:, :, None] + np.asarray(lc, np.float32)[:, None, :]
    return _f64(lr)[:, :, None] + _f64(lc)[:, None, :]


def select_full(lr, lc, K: int, float32: bool = False):
    """O4 over the whole N_r x N_c grid.  Returns (ids [T, K], S [T, K])."""
    S = _grid(lr, lc, float32)
    T, Nr, Nc = S.shape
    flat = S.reshape(T, Nr * Nc)
    ids = np.empty((T, K), dtype=np.int64)
    vals = np.empty((T, K), dtype=flat.dtype)
    cand = np.arange(Nr * Nc)
    for t in range(T):
        order = np.lexsort((cand, -flat[t]))[:K]          # S desc, id asc
        ids[t] = order
        vals[t] = flat[t, order]
    return ids, vals


def _axis_top(v, k):
    """Indices of the k largest entries by (value desc, index asc)."""
    idx = np.arange(len(v))
    return np.lexsort((idx, -v))[:k]


def select_pruned(lr, lc, K: int, k0: int | None = None, float32: bool = False):
    """O5: the top min(k0, N_r) rows and min(k0, N_c) columns, then the top K
    of their sums; k0 = K unless given (k0 = min(sqrt(N), K) is the page's
    choice, the same for a square grid)."""
    lr = np.asarray(lr, np.float32) if float32 else _f64(lr)
    lc = np.asarray(lc, np.float32) if float32 else _f64(lc)
    T, Nr = lr.shape
    Nc = lc.shape[1]
    if k0 is None:
        k0 = K
    ids = np.empty((T, K), dtype=np.int64)
    vals = np.empty((T, K), dtype=lr.dtype)
    for t in range(T):
        rows = _axis_top(lr[t], min(k0, Nr))
        cols = _axis_top(lc[t], min(k0, Nc))
        cand_ids = (rows[:, None] * Nc + cols[None, :]).ravel()
        cand_s = (lr[t][rows][:, None] + lc[t][cols][None, :]).ravel()
        order = np.lexsort((cand_ids, -cand_s))[:K]
        ids[t] = cand_ids[order]
        vals[t] = cand_s[order]
    return ids, vals


def gates_from_scores(S) -> np.ndarray:
    """O4: softmax over the K selected scores."""
    S = _f64(S)
    e = np.exp(S - S[:, :1])
    return e / np.sum(e, axis=1, keepdims=True)


def silu(z):
    return mo.silu(z)


def expert_pass(X, W_in, meta) -> np.ndarray:
    """[P2] §2.3 expert by expert: a[s] = silu(x_t . w_in_e) for every slot s
    of expert e (token t = perm_token[s])."""
    offsets = np.asarray(meta["offsets"], dtype=np.int64)
    perm = np.asarray(meta["perm_token"], dtype=np.int64)
    X = _f64(X)
    N = len(offsets) - 1
    a = np.zeros(int(offsets[N]))
    active = np.flatnonzero(np.diff(offsets) > 0)
    for e in active:
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        a[lo:hi] = silu(X[perm[lo:hi]] @ _f64(W_in[e]))
    return a


def combine(a, gates, ids, inv_slot, W_out) -> np.ndarray:
    """y_t = sum over k of g_tk * a[slot(t, k)] * w_out[id_tk], in k order."""
    g = _f64(gates)
    ids = np.asarray(ids, dtype=np.int64)
    inv = np.asarray(inv_slot, dtype=np.int64)
    T, K = ids.shape
    d = np.asarray(W_out).shape[1]
    Y = np.zeros((T, d))
    for k in range(K):
        Y += (g[:, k] * a[inv[:, k]])[:, None] * _f64(W_out[ids[:, k]])
    return Y


def forward(X, W_r, W_c, W_in, W_out, K: int, scores=None, prune: bool = True) -> dict:
    """The whole layer.  ``scores`` = (ls_r, ls_c) as fp32 device rows, else the
    float64 definition.  Returns every intermediate."""
    X = np.asarray(X)
    T = X.shape[0]
    Nr, Nc = np.asarray(W_r).shape[1], np.asarray(W_c).shape[1]
    if scores is None:
        lr, lc = axis_scores(X, W_r, W_c)
        f32 = False
    else:
        lr, lc = scores
        f32 = True
    ids, S = (select_pruned if prune else select_full)(lr, lc, K, float32=f32)
    g = gates_from_scores(S)
    meta = mo.permute(ids, Nr * Nc, T)
    a = expert_pass(X, W_in, meta)
    Y = combine(a, g, ids, meta["inv_slot"], W_out)
    out = {"ls_r": lr, "ls_c": lc, "ids": ids, "S": S, "gates": g, "a": a, "Y": Y}
    out.update(meta)
    return out


def token_outputs(tokens, X, ids, gates, W_in, W_out) -> np.ndarray:
    """y_t for the listed tokens only, straight from the closed form of
    [P2] §2.1 (for sampled checks at full size)."""
    X = _f64(X)
    g = _f64(gates)
    ids = np.asarray(ids, dtype=np.int64)
    rows = []
    for t in tokens:
        y = np.zeros(X.shape[1])
        for k in range(ids.shape[1]):
            e = int(ids[t, k])
            y += g[t, k] * silu(X[t] @ _f64(W_in[e])) * _f64(W_out[e])
        rows.append(y)
    return np.array(rows)
