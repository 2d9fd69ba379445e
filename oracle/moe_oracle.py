"""numpy float64 oracle of the single-GPU MoE layer forward.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): only the tests, the
smoke check and the bench's CPU-baseline leg use it.  It shares no code,
constant or helper with the HIP library and imports nothing from it.

Pages cited (by title and section):

* [P1] "算子与编译器：MoE 路由与稀疏 Kernel" (charles2530.github.io)
* [P2] "MoE 的两个上游创新：Routing-Free 与 OmniMoE" (chatdocs.ruinique.com)
* [P4] "AI芯片如何支持MoE架构", chapter 4
* [P5] SonicMoE article on gitcode.csdn.net ("一句话结论" ... "12. 总结")

What the layer computes, step by step ([P5] §3 lists the GPU pipeline; [P5] §1
gives y = sum over the selected experts of gate * expert output):

1. router logits  l = X W_r (+ b)                        [P2] §1.1, [P4] §4.2
2. softmax, top-K, renormalised gates                    [P2] §1.1, [P4] §4.3
3. per-expert histogram of the [T, K] ids               [P5] §11, [P1] §3
4. capacity C and drop of overflow in token order        [P1] §4
5. exclusive scan -> offsets; scatter index              [P1] §3, [P5] §11,
   (expert, token) order                                 [P2] §2.3, §3.3
6. gathered rows -> SwiGLU FFN first half -> H          [P5] §3 steps 2-4, §6.2-6.3
7. H -> second projection -> O                          [P5] §3 step 5
8. gate-weighted combine back to token order            [P5] §1, §3 step 6, §6.1

Readings taken where the pages leave a step open (each repeated where used):

* R1 softmax -> top-K -> renormalise over the K selected, for every config.
* R2 ties in the selection go to the lower expert id; -0.0 equals +0.0.
* R3 the K ids of a token are listed by descending logit (rank 0 = argmax).
* R4 C = T when the capacity factor is <= 0, else min(T, ceil(cf*T*K/E)),
  computed exactly from the binary value of cf.
* R5 overflow is dropped in token order: per expert, the C lowest token ids
  are kept, whatever the k-rank of the assignment.
* R6 gates are not renormalised after a drop; a fully dropped token gives 0.
* R7 inside an expert segment the slots hold ascending token ids.
* R8 SwiGLU expert: h = silu(x W_gate) * (x W_up), o = h W_down, with
  silu(z) = z / (1 + exp(-z)); no biases.

Parity status: every public function is pinned by ``-m "not gpu"`` tests
(worked example of [P2] §2.3, the brute force in ``oracle/brute.py``, closed
forms and invariants).  No function here is "parity unpinned".
"""

from __future__ import annotations

import math
from fractions import Fraction

import numpy as np


def _f64(a) -> np.ndarray:
    """Exact promotion to float64 (bf16 and fp32 values are representable)."""
    return np.asarray(a, dtype=np.float64)


def router_logits(X, W_r, bias=None) -> np.ndarray:
    """Router scores l[t, e] = sum_i X[t, i] W_r[i, e] (+ b[e]), in float64.

    [P2] §1.1: a token x goes through Router(x), then softmax, then TopK; the
    router is the dense gating layer of [P4] §4.2 (token-by-expert dot
    products).  The optional per-expert bias b is added after the product.
    """
    X = _f64(X)
    W_r = _f64(W_r)
    if X.ndim != 2 or W_r.ndim != 2 or X.shape[1] != W_r.shape[0]:
        raise ValueError("router_logits: X[T,d] and W_r[d,E] expected")
    logits = X @ W_r
    if bias is not None:
        b = _f64(bias)
        if b.shape != (W_r.shape[1],):
            raise ValueError("router_logits: bias must have shape [E]")
        logits = logits + b[None, :]
    return logits


def topk_select(logits, K: int) -> np.ndarray:
    """ids[t, 0..K-1]: the K experts with the largest score, best first.

    [P2] §1.1 (Router -> Softmax -> TopK) and [P4] §4.3 (K is a run-time
    value).  Softmax is strictly increasing, so ranking probabilities and
    ranking logits pick the same experts; the selection is made on the
    logits themselves (R1).  Order key is (score descending, expert id
    ascending) (R2, R3); adding +0.0 folds -0.0 into +0.0 so both compare
    equal.  A stable sort keeps equal keys in ascending expert id.
    """
    scores = _f64(logits)
    if scores.ndim != 2:
        raise ValueError("topk_select: logits[T,E] expected")
    if not np.all(np.isfinite(scores)):
        raise ValueError("topk_select: non-finite logits are outside the input contract")
    T, E = scores.shape
    if not 1 <= K <= E:
        raise ValueError("topk_select: need 1 <= K <= E")
    key = -(scores + 0.0)
    order = np.argsort(key, axis=1, kind="stable")
    return order[:, :K].astype(np.int32)


def topk_gates(logits, ids) -> np.ndarray:
    """Gates g[t, k] = p[t, ids[t,k]] / sum_j p[t, ids[t,j]], p = softmax(l[t]).

    [P2] §1.1 puts the softmax before the TopK; [P5] §1 weights each selected
    expert by its gate.  The selected probabilities are renormalised to sum
    to 1 (R1).  The max is subtracted before exp for range safety only.
    """
    scores = _f64(logits)
    ids = np.asarray(ids, dtype=np.int64)
    m = scores.max(axis=1, keepdims=True)
    p = np.exp(scores - m)
    p = p / p.sum(axis=1, keepdims=True)
    sel = np.take_along_axis(p, ids, axis=1)
    return sel / sel.sum(axis=1, keepdims=True)


def capacity(T: int, K: int, E: int, capacity_factor) -> int:
    """Per-expert token cap C ([P1] §4: the cap bounds what one expert takes).

    R4: C = T when the factor is <= 0 (no limit), else min(T, ceil(cf*T*K/E))
    with cf taken as the exact binary value of the double.
    """
    if capacity_factor is None:
        return int(T)
    cf = float(capacity_factor)
    if not math.isfinite(cf):
        raise ValueError("capacity: capacity factor must be finite")
    if cf <= 0.0:
        return int(T)
    return int(min(T, math.ceil(Fraction(cf) * T * K / E)))


def permute(ids, E: int, C: int) -> dict:
    """Expert-major metadata from the [T, K] ids ([P5] §11; [P1] §3).

    * raw_counts[e]: assignments to expert e (the histogram);
    * rank(t, k): how many earlier tokens (in token order) chose the same
      expert; the assignment is kept iff rank < C (R5, [P1] §4);
    * counts[e] = min(raw_counts[e], C); offsets = exclusive scan of counts;
    * kept (t, k) goes to slot offsets[e] + rank: slots are ordered by
      (expert, token) as in [P2] §2.3 and §3.3 (R7);
    * perm_token[slot] = t (expert-major slot -> token) and
      inv_slot[t, k] = slot or -1 (token-major entry -> expert-major slot).

    perm_token has T*K entries; those at or beyond offsets[E] are -1 here and
    carry no meaning.
    """
    ids = np.asarray(ids)
    T, K = ids.shape
    id_rows = ids.tolist()
    seen = [0] * E
    rank = [[0] * K for _ in range(T)]
    for t in range(T):
        for k in range(K):
            e = id_rows[t][k]
            rank[t][k] = seen[e]
            seen[e] += 1
    raw = np.array(seen, dtype=np.int64)
    counts = np.minimum(raw, C)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    inv_slot = np.full((T, K), -1, dtype=np.int64)
    perm_token = np.full(T * K, -1, dtype=np.int64)
    for t in range(T):
        for k in range(K):
            r = rank[t][k]
            if r < C:
                s = int(offsets[id_rows[t][k]]) + r
                inv_slot[t, k] = s
                perm_token[s] = t
    return {
        "raw_counts": raw.astype(np.int32),
        "counts": counts.astype(np.int32),
        "offsets": offsets.astype(np.int32),
        "perm_token": perm_token.astype(np.int32),
        "inv_slot": inv_slot.astype(np.int32),
    }


def silu(z):
    """silu(z) = z / (1 + exp(-z)) (the gated unit of SwiGLU, beta = 1)."""
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def expert_ffn(a, W_gate_e, W_up_e, W_down_e):
    """One SwiGLU expert on the rows of ``a`` (R8; [P5] §3 steps 3-5).

    Returns (h, o) with h = silu(a W_gate) * (a W_up) and o = h W_down.
    """
    a = _f64(a)
    v = a @ _f64(W_gate_e)
    u = a @ _f64(W_up_e)
    h = silu(v) * u
    return h, h @ _f64(W_down_e)


def grouped_ffn(X, offsets, perm_token, W_gate, W_up, W_down):
    """Expert-major H[N, n] and O[N, d] over the N = offsets[E] kept slots.

    For expert e, its slots s in [offsets[e], offsets[e+1]) read the token row
    X[perm_token[s]] ([P5] §6.2: rows are read by index, no pre-gathered copy
    is needed for the definition) and run the expert's FFN ([P5] §3).
    """
    X = np.asarray(X)
    offsets = np.asarray(offsets, dtype=np.int64)
    perm_token = np.asarray(perm_token, dtype=np.int64)
    E = len(offsets) - 1
    N = int(offsets[E])
    n = W_gate.shape[2]
    d = W_down.shape[2]
    H = np.zeros((N, n))
    O = np.zeros((N, d))
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        a = _f64(X[perm_token[lo:hi]])
        H[lo:hi], O[lo:hi] = expert_ffn(a, W_gate[e], W_up[e], W_down[e])
    return H, O


def combine(O, gates, inv_slot, d: int | None = None) -> np.ndarray:
    """Y[t] = sum over kept k of gates[t, k] * O[inv_slot[t, k]] ([P5] §1, §6.1).

    Dropped entries (inv_slot = -1) contribute nothing (R6); a token whose K
    entries are all dropped gets a zero row.
    """
    O = _f64(O)
    g = _f64(gates)
    inv_slot = np.asarray(inv_slot, dtype=np.int64)
    T, K = inv_slot.shape
    width = O.shape[1] if d is None else d
    Y = np.zeros((T, width))
    for k in range(K):
        kept = inv_slot[:, k] >= 0
        Y[kept] += g[kept, k, None] * O[inv_slot[kept, k]]
    return Y


def route(X, W_r, K: int, bias=None, logits=None) -> dict:
    """Steps 1-2.  With ``logits`` given (e.g. the device's exported fp32
    scores), selection and gates are computed on those values, so the integer
    decisions are taken on the same numbers as on the device."""
    ref = router_logits(X, W_r, bias)
    use = ref if logits is None else _f64(logits)
    ids = topk_select(use, K)
    return {"logits": ref, "ids": ids, "gates": topk_gates(use, ids)}


def forward(X, W_r, W_gate, W_up, W_down, K: int, capacity_factor=0.0,
            bias=None, logits=None) -> dict:
    """The whole layer (steps 1-8) in float64; returns every intermediate."""
    X = np.asarray(X)
    T = X.shape[0]
    E = np.asarray(W_r).shape[1]
    r = route(X, W_r, K, bias=bias, logits=logits)
    C = capacity(T, K, E, capacity_factor)
    meta = permute(r["ids"], E, C)
    H, O = grouped_ffn(X, meta["offsets"], meta["perm_token"], W_gate, W_up, W_down)
    Y = combine(O, r["gates"], meta["inv_slot"], d=X.shape[1])
    out = dict(r)
    out.update(meta)
    out.update({"C": C, "H": H, "O": O, "Y": Y})
    return out


def token_outputs(tokens, X, ids, gates, inv_slot, W_gate, W_up, W_down) -> np.ndarray:
    """Y rows for the listed tokens only.

    Y[t] depends on x_t, its selected experts, its gates and which of its
    entries survived the capacity cut; the cut itself comes from ``inv_slot``
    (computed over all tokens by ``permute``).  The listed tokens' kept
    entries are grouped by expert so that each expert's weights are promoted
    to float64 once; the sum over k then runs in k order per token.  Used for
    sampled checks at sizes where the full H and O would not fit in memory.
    """
    ids = np.asarray(ids)
    inv_slot = np.asarray(inv_slot)
    g = _f64(gates)
    tokens = [int(t) for t in tokens]
    K = ids.shape[1]
    outs = {}                                   # (row, k) -> expert output
    by_expert = {}
    for i, t in enumerate(tokens):
        for k in range(K):
            if inv_slot[t, k] >= 0:
                by_expert.setdefault(int(ids[t, k]), []).append((i, k))
    for e, entries in by_expert.items():
        a = _f64(X[[tokens[i] for i, _ in entries]])
        _, o = expert_ffn(a, W_gate[e], W_up[e], W_down[e])
        for (i, k), row in zip(entries, o):
            outs[(i, k)] = row
    Y = np.zeros((len(tokens), np.asarray(X).shape[1]))
    for i, t in enumerate(tokens):
        for k in range(K):
            if (i, k) in outs:
                Y[i] += g[t, k] * outs[(i, k)]
    return Y


def slot_outputs(slots, X, offsets, perm_token, W_gate, W_up, W_down):
    """(H[s], O[s]) for the listed expert-major slots, one slot at a time."""
    offsets = np.asarray(offsets, dtype=np.int64)
    hs, os_ = [], []
    for s in slots:
        e = int(np.searchsorted(offsets, s, side="right") - 1)
        t = int(perm_token[s])
        h, o = expert_ffn(_f64(X[t])[None, :], W_gate[e], W_up[e], W_down[e])
        hs.append(h[0])
        os_.append(o[0])
    return np.array(hs), np.array(os_)


def forward_by_expert(X, gates, offsets, perm_token, inv_slot, W_gate, W_up, W_down,
                      visit=None) -> np.ndarray:
    """Steps 6-8 one expert at a time; returns Y [T, d] in float64.

    The same definitions as ``grouped_ffn`` followed by ``combine`` ([P5] §3
    steps 3-6, §1), arranged so that only one expert's H and O rows exist at
    a time: for each expert e with kept slots [lo, hi) the rows
    a = X[perm_token[lo:hi]] go through the expert (``expert_ffn``), the
    callback ``visit(e, lo, hi, h, o)`` (if given) sees that segment of H and
    O, and each row o_s, times the gate of its (token, k) entry, is added to
    its token's row of Y.  Inside a segment the tokens are strictly
    increasing (R7), so every token occurs at most once there; this is
    checked.  Used where the whole H and O would not fit in memory.
    """
    X = np.asarray(X)
    offsets = np.asarray(offsets, dtype=np.int64)
    perm_token = np.asarray(perm_token, dtype=np.int64)
    inv_slot = np.asarray(inv_slot, dtype=np.int64)
    g = _f64(gates)
    T, d = X.shape
    E = len(offsets) - 1
    N = int(offsets[E])
    kept = inv_slot >= 0
    slot_gate = np.zeros(N)
    slot_gate[inv_slot[kept]] = g[kept]
    Y = np.zeros((T, d))
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        toks = perm_token[lo:hi]
        if np.any(np.diff(toks) <= 0):
            raise ValueError("forward_by_expert: tokens of a segment must be strictly increasing")
        h, o = expert_ffn(_f64(X[toks]), W_gate[e], W_up[e], W_down[e])
        if visit is not None:
            visit(e, lo, hi, h, o)
        Y[toks] += slot_gate[lo:hi, None] * o
    return Y


def rel_l2(a, b) -> float:
    """||a - b||_2 / ||b||_2 over all elements (0 when both are zero, inf
    when only b is zero).  The relative-L2 error is the measure the output
    tolerances are stated in; a and b must have the same shape (no
    broadcasting)."""
    a = _f64(a)
    b = _f64(b)
    if a.shape != b.shape:
        raise ValueError(f"rel_l2: shapes differ {a.shape} vs {b.shape}")
    den = float(np.linalg.norm(b))
    num = float(np.linalg.norm(a - b))
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return num / den


def rel_l2_rows(a, b) -> np.ndarray:
    """``rel_l2`` of each row (last axis) of two equal-shape 2-D arrays:
    ||a[i] - b[i]||_2 / ||b[i]||_2, 0 where both rows are zero and inf where
    only b's row is zero."""
    a = _f64(a)
    b = _f64(b)
    if a.shape != b.shape or a.ndim != 2:
        raise ValueError(f"rel_l2_rows: equal 2-D shapes expected, got {a.shape} vs {b.shape}")
    den = np.linalg.norm(b, axis=1)
    num = np.linalg.norm(a - b, axis=1)
    out = np.zeros(a.shape[0])
    nz = den > 0.0
    out[nz] = num[nz] / den[nz]
    out[~nz & (num > 0.0)] = np.inf
    return out
