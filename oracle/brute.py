"""Brute-force twin of the oracle: pure-Python loops over every (token, expert).

TEST INFRASTRUCTURE ONLY.  Written independently of ``moe_oracle`` (no shared
helper, no numpy arithmetic) so that the two agreeing on tiny inputs pins the
oracle.  It follows the same pages and readings R1-R8 listed in
``moe_oracle``'s docstring, but takes a different road to each result:

* selection: a full Python ``sorted`` of all E (score, id) pairs per token;
* gates: the full softmax over E written out with ``math.exp``;
* permutation: enumerate every (token, expert) pair, keep the selected ones,
  sort them lexicographically by (expert, token) ([P2] §2.3), then walk each
  expert's list applying the cap ([P1] §4);
* FFN and output: every selected (token, expert) pair evaluated with scalar
  loops, y_t = sum of gate * expert output ([P5] §1).

Only for tiny shapes (T*E*d*n up to a few million scalar operations).
"""

from __future__ import annotations

import math


def _mat(a):
    """Nested Python lists of floats from any array-like."""
    if hasattr(a, "tolist"):
        a = a.tolist()
    return a


def brute_logits(X, W_r, bias=None):
    X, W = _mat(X), _mat(W_r)
    T, d, E = len(X), len(W), len(W[0])
    b = _mat(bias) if bias is not None else [0.0] * E
    out = []
    for t in range(T):
        row = []
        for e in range(E):
            s = 0.0
            for i in range(d):
                s += float(X[t][i]) * float(W[i][e])
            row.append(s + float(b[e]))
        out.append(row)
    return out


def brute_select(L, K):
    """Top-K per token by a full sort of (-score, id) keys."""
    ids = []
    for row in _mat(L):
        E = len(row)
        ranked = sorted(range(E), key=lambda e: (-float(row[e]), e))
        ids.append(ranked[:K])
    return ids


def brute_gates(L, ids):
    gates = []
    for row, sel in zip(_mat(L), ids):
        m = max(float(v) for v in row)
        ex = [math.exp(float(v) - m) for v in row]
        z = sum(ex)
        p = [v / z for v in ex]
        s = sum(p[e] for e in sel)
        gates.append([p[e] / s for e in sel])
    return gates


def brute_permute(ids, E, C):
    """Metadata by enumerating all (token, expert) pairs."""
    T = len(ids)
    pairs = []
    for t in range(T):
        for e in range(E):
            if e in ids[t]:
                pairs.append((e, t))
    pairs.sort()
    raw = [0] * E
    for e, _ in pairs:
        raw[e] += 1
    kept_pos = {}
    counts = [0] * E
    for e in range(E):
        members = [t for (ee, t) in pairs if ee == e]
        for p, t in enumerate(members):
            if p < C:
                kept_pos[(t, e)] = p
                counts[e] += 1
    offsets = [0]
    for e in range(E):
        offsets.append(offsets[-1] + counts[e])
    perm = [None] * offsets[E]
    inv = []
    for t in range(T):
        row = []
        for e in ids[t]:
            if (t, e) in kept_pos:
                s = offsets[e] + kept_pos[(t, e)]
                perm[s] = t
                row.append(s)
            else:
                row.append(-1)
        inv.append(row)
    return {"raw_counts": raw, "counts": counts, "offsets": offsets,
            "perm_token": perm, "inv_slot": inv}


def brute_expert(x, Wg, Wu, Wd):
    """One expert on one token: h_j = silu(x.Wg[:, j]) * (x.Wu[:, j]); o = h.Wd."""
    d, n = len(Wg), len(Wg[0])
    h = []
    for j in range(n):
        v = 0.0
        u = 0.0
        for i in range(d):
            v += float(x[i]) * float(Wg[i][j])
            u += float(x[i]) * float(Wu[i][j])
        sig = 1.0 / (1.0 + math.exp(-v)) if v > -700.0 else 0.0
        h.append(v * sig * u)
    o = []
    for c in range(len(Wd[0])):
        s = 0.0
        for j in range(n):
            s += h[j] * float(Wd[j][c])
        o.append(s)
    return h, o


def brute_forward(X, W_r, W_gate, W_up, W_down, K, C, bias=None, logits=None):
    """Every intermediate of the layer on tiny inputs, pure Python."""
    X = _mat(X)
    Wg, Wu, Wd = _mat(W_gate), _mat(W_up), _mat(W_down)
    E = len(_mat(W_r)[0])
    L_ref = brute_logits(X, W_r, bias)
    L = L_ref if logits is None else _mat(logits)
    ids = brute_select(L, K)
    gates = brute_gates(L, ids)
    meta = brute_permute(ids, E, C)
    T, d = len(X), len(X[0])
    n = len(Wg[0][0])
    N = meta["offsets"][E]
    H = [[0.0] * n for _ in range(N)]
    O = [[0.0] * d for _ in range(N)]
    Y = []
    for t in range(T):
        y = [0.0] * d
        for k, e in enumerate(ids[t]):
            s = meta["inv_slot"][t][k]
            if s < 0:
                continue
            h, o = brute_expert(X[t], Wg[e], Wu[e], Wd[e])
            H[s], O[s] = h, o
            for c in range(d):
                y[c] += gates[t][k] * o[c]
        Y.append(y)
    out = {"logits": L_ref, "ids": ids, "gates": gates, "H": H, "O": O, "Y": Y}
    out.update(meta)
    return out


def round_tokens_brute(ids, gates, kept_pairs, E, M):
    """Tile-aware token rounding (readings TR1-TR4 of ``token_rounding``) by
    brute force.  ``kept_pairs`` is the set of (token, expert) assignments
    that survived the capacity cut.  Per expert: list its kept (gate, token)
    pairs, sort them by (gate, -token) with ``sorted``, and remove from the
    front until the count is the multiple of M that the rule asks for.
    Returns (counts, surviving pairs sorted by (expert, token))."""
    ids, g = _mat(ids), _mat(gates)
    T, K = len(ids), len(ids[0])
    counts = []
    survivors = []
    for e in range(E):
        mine = []
        for t in range(T):
            for k in range(K):
                if ids[t][k] == e and (t, e) in kept_pairs:
                    mine.append((g[t][k], -t))
        c = len(mine)
        target = c
        while target >= M and target % M != 0 and (c % M) * 2 < M:
            target -= 1
        ranked = sorted(mine)
        keep = ranked[c - target:] if target < c else ranked
        toks = sorted(-mt for _, mt in keep)
        counts.append(len(toks))
        survivors.extend((e, t) for t in toks)
    return counts, survivors


def brute_omni_forward(X, W_r, W_c, W_in, W_out, K):
    """Atomic-expert layer with a Cartesian router ([P2] §2.1-2.2; readings
    O1-O6 of ``omni_oracle``) by brute force: every (row, column) pair of the
    grid is scored and the whole list is sorted; each selected expert is
    evaluated with scalar loops.  Returns (ids, gates, Y) as lists."""
    X, Wr, Wc, Win, Wout = _mat(X), _mat(W_r), _mat(W_c), _mat(W_in), _mat(W_out)
    T, d = len(X), len(X[0])
    Nr, Nc = len(Wr[0]), len(Wc[0])

    def logsm(row):
        m = max(row)
        z = sum(math.exp(v - m) for v in row)
        return [v - m - math.log(z) for v in row]

    ids_all, gates_all, Y = [], [], []
    for t in range(T):
        pr = [sum(X[t][i] * Wr[i][r] for i in range(d)) for r in range(Nr)]
        pc = [sum(X[t][i] * Wc[i][c] for i in range(d)) for c in range(Nc)]
        lr, lc = logsm(pr), logsm(pc)
        pairs = sorted((-(lr[r] + lc[c]), r * Nc + c) for r in range(Nr) for c in range(Nc))
        sel = pairs[:K]
        ids = [i for _, i in sel]
        ex = [math.exp(-s) for s, _ in sel]
        z = sum(ex)
        gates = [v / z for v in ex]
        y = [0.0] * d
        for g, e in zip(gates, ids):
            dot = sum(X[t][i] * Win[e][i] for i in range(d))
            h = dot / (1.0 + math.exp(-dot))
            for i in range(d):
                y[i] += g * h * Wout[e][i]
        ids_all.append(ids)
        gates_all.append(gates)
        Y.append(y)
    return ids_all, gates_all, Y
