"""Pins of the atomic-expert / Cartesian-router oracle (oracle/omni_oracle.py):
the pure-Python twin on tiny layers, the exactness of the pruned search,
closed forms of [P2] §2.1-2.2, and planted mistakes these pins must catch."""

import math

import numpy as np
import pytest

from oracle import brute
from oracle import moe_oracle as mo
from oracle import omni_oracle as om


def _layer(T, d, Nr, Nc, seed):
    rng = np.random.default_rng(seed)
    N = Nr * Nc
    return (rng.standard_normal((T, d)), rng.standard_normal((d, Nr)) / np.sqrt(d),
            rng.standard_normal((d, Nc)) / np.sqrt(d), rng.standard_normal((N, d)) / np.sqrt(d),
            rng.standard_normal((N, d)))


@pytest.mark.parametrize("T,d,Nr,Nc,K,seed", [(5, 6, 3, 4, 3, 0), (4, 5, 4, 4, 6, 1),
                                              (3, 4, 2, 5, 10, 2), (6, 3, 3, 3, 1, 3)])
@pytest.mark.parametrize("prune", [False, True])
def test_matches_brute_force(T, d, Nr, Nc, K, seed, prune):
    X, W_r, W_c, W_in, W_out = _layer(T, d, Nr, Nc, seed)
    out = om.forward(X, W_r, W_c, W_in, W_out, K, prune=prune)
    ids, gates, Y = brute.brute_omni_forward(X, W_r, W_c, W_in, W_out, K)
    assert np.array_equal(out["ids"], np.array(ids))
    assert np.allclose(out["gates"], np.array(gates), rtol=1e-12, atol=1e-14)
    assert np.allclose(out["Y"], np.array(Y), rtol=1e-10, atol=1e-12)


def test_pruned_search_equals_full_search_with_ties():
    rng = np.random.default_rng(7)
    for _ in range(60):
        T = 8
        Nr, Nc = int(rng.integers(1, 9)), int(rng.integers(1, 9))
        K = int(rng.integers(1, Nr * Nc + 1))
        lr = rng.integers(-3, 1, size=(T, Nr)).astype(np.float64)   # few values: many ties
        lc = rng.integers(-3, 1, size=(T, Nc)).astype(np.float64)
        for f32 in (False, True):
            a = om.select_full(lr, lc, K, float32=f32)
            b = om.select_pruned(lr, lc, K, float32=f32)
            assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_pages_k0_is_exact_on_square_grids_but_not_always_otherwise():
    rng = np.random.default_rng(8)
    for _ in range(40):
        n, K = int(rng.integers(2, 7)), int(rng.integers(1, 30))
        K = min(K, n * n)
        lr, lc = rng.standard_normal((4, n)), rng.standard_normal((4, n))
        k0 = min(math.isqrt(n * n), K)
        assert np.array_equal(om.select_full(lr, lc, K)[0], om.select_pruned(lr, lc, K, k0=k0)[0])
    # 2 x 8 grid, K = 10: the page's k0 = min(4, 10) = 4 keeps 2 x 4 = 8 < 10 candidates
    lr, lc = rng.standard_normal((1, 2)), rng.standard_normal((1, 8))
    short = om.select_pruned(lr, lc, 8, k0=4)[0]
    assert not np.array_equal(short, om.select_full(lr, lc, 8)[0])


def test_closed_forms():
    X, W_r, W_c, W_in, W_out = _layer(6, 5, 4, 4, 11)
    # a zero column projection: every column ties, so the K picks are the best
    # row's lowest columns, with equal gates
    out = om.forward(X, W_r, np.zeros_like(W_c), W_in, W_out, 3, prune=False)
    best = np.argmax(X @ W_r, axis=1)
    assert np.array_equal(out["ids"], best[:, None] * 4 + np.arange(3)[None, :])
    assert np.allclose(out["gates"], 1.0 / 3.0, rtol=1e-14)
    # gates are proportional to P_r * P_c (the LogSoftmax sum is a product of probabilities)
    out = om.forward(X, W_r, W_c, W_in, W_out, 5)
    Pr, Pc = np.exp(out["ls_r"]), np.exp(out["ls_c"])
    r, c = out["ids"] // 4, out["ids"] % 4
    prod = Pr[np.arange(6)[:, None], r] * Pc[np.arange(6)[:, None], c]
    assert np.allclose(out["gates"], prod / prod.sum(axis=1, keepdims=True), rtol=1e-12)
    # one atomic expert per token: y = silu(x . w_in) w_out
    out = om.forward(X, W_r, W_c, W_in, W_out, 1)
    e = out["ids"][:, 0]
    expect = mo.silu(np.sum(X * W_in[e], axis=1))[:, None] * W_out[e]
    assert np.allclose(out["Y"], expect, rtol=1e-12, atol=1e-14)
    # expert-centric execution = the token-centric closed form
    out = om.forward(X, W_r, W_c, W_in, W_out, 7)
    direct = om.token_outputs(range(6), X, out["ids"], out["gates"], W_in, W_out)
    assert np.allclose(out["Y"], direct, rtol=1e-12, atol=1e-13)


def test_reuse_ratio_of_the_expert_centric_order():
    """[P2] §2.3: eta = L*K / |E_active| tasks per loaded expert."""
    X, W_r, W_c, W_in, W_out = _layer(40, 4, 3, 3, 12)
    out = om.forward(X, W_r, W_c, W_in, W_out, 4)
    active = np.count_nonzero(out["counts"])
    assert int(out["offsets"][-1]) == 40 * 4
    eta = 40 * 4 / active
    assert eta == pytest.approx(np.mean(out["counts"][out["counts"] > 0]))


# ---------------------------------------------------------------- planted mistakes

def _planted(kind, X, W_r, W_c, W_in, W_out, K):
    lr, lc = om.axis_scores(X, W_r, W_c)
    Nc = W_c.shape[1]
    ids, S = om.select_full(lr, lc, K)
    g = om.gates_from_scores(S)
    if kind == "tie_to_higher_id":
        flat = (lr[:, :, None] + lc[:, None, :]).reshape(len(X), -1)
        cand = np.arange(flat.shape[1])
        ids = np.stack([np.lexsort((-cand, -f))[:K] for f in flat])
    elif kind == "gates_not_renormalised":
        g = np.exp(S)
    elif kind == "sigmoid_for_silu":
        pass
    elif kind == "transposed_id":
        r, c = ids // Nc, ids % Nc
        ids = c * W_r.shape[1] + r
    act = (lambda z: 1 / (1 + np.exp(-z))) if kind == "sigmoid_for_silu" else mo.silu
    Y = np.zeros_like(X)
    for t in range(len(X)):
        for k in range(K):
            e = ids[t, k]
            Y[t] += g[t, k] * act(X[t] @ W_in[e]) * W_out[e]
    return ids, g, Y


@pytest.mark.parametrize("kind", ["tie_to_higher_id", "gates_not_renormalised",
                                  "sigmoid_for_silu", "transposed_id"])
def test_planted_mistakes_are_caught(kind):
    caught = False
    for seed, zero_c in ((0, False), (1, True)):
        X, W_r, W_c, W_in, W_out = _layer(5, 6, 3, 4, seed)
        if zero_c:
            W_c = np.zeros_like(W_c)                       # ties for the tie-break mistake
        ids, g, Y = _planted(kind, X, W_r, W_c, W_in, W_out, 3)
        bi, bg, bY = brute.brute_omni_forward(X, W_r, W_c, W_in, W_out, 3)
        same = (np.array_equal(ids, np.array(bi)) and np.allclose(g, np.array(bg), rtol=1e-9)
                and np.allclose(Y, np.array(bY), rtol=1e-8, atol=1e-10))
        caught |= not same
    assert caught, kind
