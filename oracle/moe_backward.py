"""numpy float64 oracle of the MoE layer backward (training).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): only the tests use
it.  It shares no code, constant or helper with the HIP library and imports
nothing from it; it builds on the forward oracle in ``moe_oracle.py``.

Pages cited: [P5] the SonicMoE article (gitcode.csdn.net), §6.1 (the forward
keeps only X and the pre-SwiGLU activation for the backward), §6.3 (the
dSwiGLU work belongs in a GEMM epilogue) and §6.4 (the backward reordering:
the router-score gradient is taken as dS = <dA', A> with dA' = dO W2^T, where
A is the expert's activation fed to the down projection, instead of
<dO, Y> with Y = A W2 -- the same number without keeping Y).

Notation (per kept slot s of expert e, token t = perm_token[s], k its rank
in the token's list, g = gates[t, k]):

* pre-activations  Hg[s] = X[t] W_gate[e],  Hu[s] = X[t] W_up[e]   (saved)
* activation       A[s]  = silu(Hg[s]) * Hu[s]                     (recomputed)
* expert output    O[s]  = A[s] W_down[e]                          (never kept)
* layer output     Y[t]  = sum over kept k of g[t, k] O[slot(t, k)]

Given dY = dL/dY:

* dA'[s] = dY[t] W_down[e]^T                    ([P5] §6.4)
* dS[s]  = <dA'[s], A[s]>  = dL/dg[t, k]        ([P5] §6.4)
* dA[s]  = g dA'[s]
* dHg[s] = dA[s] * Hu[s] * silu'(Hg[s]),  dHu[s] = dA[s] * silu(Hg[s])   ([P5] §6.3)
  with silu'(z) = sigmoid(z) (1 + z (1 - sigmoid(z)))
* dW_down[e] = sum_s A[s]^T (g dY[t])
* dW_gate[e] = sum_s X[t]^T dHg[s],  dW_up[e] = sum_s X[t]^T dHu[s]
* dX[t] = sum over kept k of (dHg[s] W_gate[e]^T + dHu[s] W_up[e]^T)  +  dl[t] W_r^T

Router (readings R1, R6 of the forward oracle): the gates are the softmax of
the K selected logits, renormalised over those K; the selection itself is
piecewise constant (no gradient through the ids).  A dropped assignment keeps
its gate in the normalisation but contributes nothing to Y, so its dg is 0:

* dg[t, k] = dS[slot(t, k)] if kept, else 0
* dl[t, id_k] = g_k (dg_k - sum_j g_j dg_j) for the K selected; 0 elsewhere
* dW_r = X^T dl;  the bias (an input, not a parameter here) gets no gradient.

Parity status: pinned by ``-m "not gpu"`` tests against central finite
differences of the forward oracle's loss sum(Y * dY) on small float64 layers
(with and without capacity drops), by the identity <dY, O> = <dA', A> and by
the zero row sums of dl (a softmax Jacobian maps onto the sum-zero plane).
``sampled_backward`` and ``backward_by_expert`` are pinned to ``backward`` on
small layers (every expert and token listed).
"""

from __future__ import annotations

import numpy as np

from . import moe_oracle as mo


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def sigmoid(z):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def dsilu(z):
    """d/dz of silu(z) = z sigmoid(z):  sigmoid(z) (1 + z (1 - sigmoid(z)))."""
    s = sigmoid(z)
    return s * (1.0 + z * (1.0 - s))


def forward_train(X, W_r, W_gate, W_up, W_down, K: int, capacity_factor=0.0, bias=None,
                  logits=None) -> dict:
    """The forward of ``moe_oracle.forward`` plus what the backward keeps:
    the per-slot pre-activations Hg, Hu ([P5] §6.1: X and the pre-SwiGLU
    activation are all that is cached)."""
    out = mo.forward(X, W_r, W_gate, W_up, W_down, K, capacity_factor, bias=bias, logits=logits)
    offsets, perm = out["offsets"], out["perm_token"]
    E = len(offsets) - 1
    N = int(offsets[E])
    n = np.asarray(W_gate).shape[2]
    Hg = np.zeros((N, n))
    Hu = np.zeros((N, n))
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            a = _f64(np.asarray(X)[perm[lo:hi]])
            Hg[lo:hi] = a @ _f64(W_gate[e])
            Hu[lo:hi] = a @ _f64(W_up[e])
    out["Hg"], out["Hu"] = Hg, Hu
    return out


def slot_gates(gates, inv_slot, N: int) -> np.ndarray:
    """g per kept slot: gs[inv_slot[t, k]] = gates[t, k]."""
    inv_slot = np.asarray(inv_slot, dtype=np.int64)
    gs = np.zeros(N)
    kept = inv_slot >= 0
    gs[inv_slot[kept]] = _f64(gates)[kept]
    return gs


def expert_backward(dY, fw, X, W_gate, W_up, W_down):
    """Steps of the expert half ([P5] §6.4, §6.3): returns dS[N], dHg, dHu
    [N, n], dA'[N, n], dW_gate, dW_up [E, d, n], dW_down [E, n, d] and the
    per-slot input gradients dXs[N, d] (before the sum over a token's slots)."""
    dY, X = _f64(dY), _f64(X)
    offsets, perm = fw["offsets"], np.asarray(fw["perm_token"], dtype=np.int64)
    E = len(offsets) - 1
    N = int(offsets[E])
    d, n = np.asarray(W_gate).shape[1], np.asarray(W_gate).shape[2]
    gs = slot_gates(fw["gates"], fw["inv_slot"], N)
    Hg, Hu = fw["Hg"], fw["Hu"]
    A = mo.silu(Hg) * Hu
    dAp = np.zeros((N, n))
    dXs = np.zeros((N, d))
    dWg = np.zeros((E, d, n))
    dWu = np.zeros((E, d, n))
    dWd = np.zeros((E, n, d))
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        rows = perm[lo:hi]
        dYe = dY[rows]
        dAp[lo:hi] = dYe @ _f64(W_down[e]).T
        dWd[e] = A[lo:hi].T @ (gs[lo:hi, None] * dYe)
    dS = np.sum(dAp * A, axis=1)
    dA = gs[:, None] * dAp
    dHg = dA * Hu * dsilu(Hg)
    dHu = dA * mo.silu(Hg)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        Xe = X[perm[lo:hi]]
        dWg[e] = Xe.T @ dHg[lo:hi]
        dWu[e] = Xe.T @ dHu[lo:hi]
        dXs[lo:hi] = dHg[lo:hi] @ _f64(W_gate[e]).T + dHu[lo:hi] @ _f64(W_up[e]).T
    return {"dS": dS, "dAp": dAp, "A": A, "dHg": dHg, "dHu": dHu, "dW_gate": dWg, "dW_up": dWu,
            "dW_down": dWd, "dXs": dXs, "gs": gs}


def router_backward(dS, fw, T: int, E: int):
    """dl [T, E] from the slot gradients dS (readings R1, R6)."""
    ids = np.asarray(fw["ids"], dtype=np.int64)
    inv = np.asarray(fw["inv_slot"], dtype=np.int64)
    g = _f64(fw["gates"])
    K = ids.shape[1]
    dg = np.zeros((T, K))
    kept = inv >= 0
    dg[kept] = _f64(dS)[inv[kept]]
    inner = np.sum(g * dg, axis=1, keepdims=True)
    dsel = g * (dg - inner)
    dl = np.zeros((T, E))
    for k in range(K):
        dl[np.arange(T), ids[:, k]] += dsel[:, k]
    return dl, dg


def backward(dY, fw, X, W_r, W_gate, W_up, W_down) -> dict:
    """All gradients of sum(Y * dY) given the forward record ``fw`` (from
    ``forward_train``)."""
    X = _f64(X)
    T, d = X.shape
    E = np.asarray(W_r).shape[1]
    ex = expert_backward(dY, fw, X, W_gate, W_up, W_down)
    dl, dg = router_backward(ex["dS"], fw, T, E)
    inv = np.asarray(fw["inv_slot"], dtype=np.int64)
    dX_ffn = np.zeros((T, d))
    for k in range(inv.shape[1]):
        kept = inv[:, k] >= 0
        dX_ffn[kept] += ex["dXs"][inv[kept, k]]
    dX_router = dl @ _f64(W_r).T
    out = dict(ex)
    out.update({"dl": dl, "dg": dg, "dW_r": X.T @ dl, "dX_ffn": dX_ffn, "dX_router": dX_router,
                "dX": dX_ffn + dX_router})
    return out


def loss(X, W_r, W_gate, W_up, W_down, K, dY, capacity_factor=0.0, bias=None) -> float:
    """sum(Y * dY): the scalar whose gradients ``backward`` returns."""
    Y = mo.forward(X, W_r, W_gate, W_up, W_down, K, capacity_factor, bias=bias)["Y"]
    return float(np.sum(Y * _f64(dY)))


def route_record(X, W_r, K: int, capacity_factor=0.0, bias=None, logits=None) -> dict:
    """Steps 1-5 of the forward oracle only (routing and expert-major
    metadata, no expert FFN): what ``sampled_backward`` needs."""
    X = np.asarray(X)
    T = X.shape[0]
    E = np.asarray(W_r).shape[1]
    r = mo.route(X, W_r, K, bias=bias, logits=logits)
    C = mo.capacity(T, K, E, capacity_factor)
    out = dict(r)
    out.update(mo.permute(r["ids"], E, C))
    out["C"] = C
    return out


def sampled_backward(dY, rec, X, W_r, W_gate, W_up, W_down, experts=(), tokens=()) -> dict:
    """Parts of ``backward``, computed one expert or one token at a time for
    layers too large to do whole: dW_gate[e], dW_up[e], dW_down[e] for the
    listed experts (sums over that expert's slots), and dX[t], dl[t] for the
    listed tokens (from the token's own K assignments).  ``rec`` is a
    ``route_record`` (or ``forward_train``) result.  Same steps as
    ``expert_backward``, ``router_backward`` and ``backward``."""
    X, dY = np.asarray(X), np.asarray(dY)
    offsets = np.asarray(rec["offsets"], dtype=np.int64)
    perm = np.asarray(rec["perm_token"], dtype=np.int64)
    ids = np.asarray(rec["ids"], dtype=np.int64)
    inv = np.asarray(rec["inv_slot"], dtype=np.int64)
    g = _f64(rec["gates"])
    E = len(offsets) - 1
    gs = slot_gates(g, inv, int(offsets[E]))
    out = {"dW_gate": {}, "dW_up": {}, "dW_down": {}, "dX": {}, "dl": {}}
    for e in experts:
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        Xe, dYe = _f64(X[perm[lo:hi]]), _f64(dY[perm[lo:hi]])
        Wg, Wu, Wd = _f64(W_gate[e]), _f64(W_up[e]), _f64(W_down[e])
        Hg, Hu = Xe @ Wg, Xe @ Wu
        A = mo.silu(Hg) * Hu
        ge = gs[lo:hi, None]
        dA = ge * (dYe @ Wd.T)
        out["dW_down"][e] = A.T @ (ge * dYe)
        out["dW_gate"][e] = Xe.T @ (dA * Hu * dsilu(Hg))
        out["dW_up"][e] = Xe.T @ (dA * mo.silu(Hg))
    K = ids.shape[1]
    for t in tokens:
        x, dy = _f64(X[t]), _f64(dY[t])
        dg = np.zeros(K)
        dxs = np.zeros(x.shape[0])
        for k in range(K):
            if inv[t, k] < 0:
                continue
            e = int(ids[t, k])
            Wg, Wu, Wd = _f64(W_gate[e]), _f64(W_up[e]), _f64(W_down[e])
            hg, hu = x @ Wg, x @ Wu
            dap = dy @ Wd.T
            dg[k] = float(dap @ (mo.silu(hg) * hu))
            da = g[t, k] * dap
            dxs += (da * hu * dsilu(hg)) @ Wg.T + (da * mo.silu(hg)) @ Wu.T
        dsel = g[t] * (dg - float(np.sum(g[t] * dg)))
        dl = np.zeros(E)
        dl[ids[t]] += dsel
        out["dl"][t] = dl
        out["dX"][t] = dxs + dl @ _f64(W_r).T
    return out


def backward_by_expert(dY, rec, X, W_r, W_gate, W_up, W_down, visit=None) -> dict:
    """All gradients of ``backward``, computed one expert at a time.

    The same steps as ``expert_backward``, ``router_backward`` and
    ``backward`` ([P5] §6.4, §6.3), arranged so that only one expert's rows
    and weight gradients exist at a time: for each expert e with kept slots
    [lo, hi) the pre-activations are recomputed from its gathered rows,
    dA' = dY W_down^T, dS = <dA', A> and the dSwiGLU terms follow, the
    callback ``visit(e, dW_gate_e, dW_up_e, dW_down_e)`` (if given) sees the
    expert's weight gradients, and each slot's input gradient is added to
    its token's dX row.  Then the router part (dl from dS) and dX, dW_r.
    ``rec`` is a ``route_record`` (or ``forward_train``) result.  Returns
    dX, dW_r, dl, dg and dS[N]; the per-expert weight gradients are only
    handed to ``visit``."""
    X, dY = np.asarray(X), np.asarray(dY)
    offsets = np.asarray(rec["offsets"], dtype=np.int64)
    perm = np.asarray(rec["perm_token"], dtype=np.int64)
    inv = np.asarray(rec["inv_slot"], dtype=np.int64)
    T, d = X.shape
    E = len(offsets) - 1
    N = int(offsets[E])
    gs = slot_gates(rec["gates"], inv, N)
    dS = np.zeros(N)
    dX_ffn = np.zeros((T, d))
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        rows = perm[lo:hi]
        if np.any(np.diff(rows) <= 0):
            raise ValueError("backward_by_expert: tokens of a segment must be strictly increasing")
        Xe, dYe = _f64(X[rows]), _f64(dY[rows])
        Wg, Wu, Wd = _f64(W_gate[e]), _f64(W_up[e]), _f64(W_down[e])
        Hg, Hu = Xe @ Wg, Xe @ Wu
        A = mo.silu(Hg) * Hu
        ge = gs[lo:hi, None]
        dAp = dYe @ Wd.T
        dS[lo:hi] = np.sum(dAp * A, axis=1)
        dA = ge * dAp
        dHg = dA * Hu * dsilu(Hg)
        dHu = dA * mo.silu(Hg)
        if visit is not None:
            visit(e, Xe.T @ dHg, Xe.T @ dHu, A.T @ (ge * dYe))
        dX_ffn[rows] += dHg @ Wg.T + dHu @ Wu.T
    dl, dg = router_backward(dS, rec, T, np.asarray(W_r).shape[1])
    return {"dS": dS, "dl": dl, "dg": dg, "dW_r": _f64(X).T @ dl,
            "dX": dX_ffn + dl @ _f64(W_r).T}
