"""Pins of the token-rounding oracle (oracle/token_rounding.py): a hand-worked
example, the pure-Python twin on random tiny cases with ties and capacity
drops, invariants at a realistic size, the forward identity, and planted
mistakes that these pins must catch."""

import json
import os

import numpy as np
import pytest

from oracle import brute
from oracle import moe_oracle as mo
from oracle import token_rounding as tr

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "token_rounding_example.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def test_golden_before_is_the_uncapped_permutation():
    g = _golden()
    ids = np.array(g["ids"])
    meta = mo.permute(ids, g["E"], C=len(ids))
    for key in ("counts", "offsets", "inv_slot"):
        assert np.array_equal(meta[key], np.array(g["before"][key])), key
    N = g["before"]["offsets"][-1]
    assert np.array_equal(meta["perm_token"][:N], g["before"]["perm_token"])


@pytest.mark.parametrize("case", range(3))
def test_golden_cases(case):
    g = _golden()
    c = g["cases"][case]
    out = tr.round_tokens(g["before"], g["ids"], np.array(g["gates"]), M=c["M"])
    for key in ("counts", "offsets", "inv_slot"):
        assert np.array_equal(out[key], np.array(c[key])), key
    N = c["offsets"][-1]
    assert np.array_equal(out["perm_token"][:N], c["perm_token"])
    assert out["dropped"] == c["dropped"]


def _random_case(rng):
    T = int(rng.integers(1, 40))
    E = int(rng.integers(1, 7))
    K = int(rng.integers(1, E + 1))
    ids = np.stack([rng.permutation(E)[:K] for _ in range(T)])
    gates = rng.integers(1, 5, size=(T, K)) / 8.0          # few values: many ties
    C = int(rng.integers(1, T + 1)) if rng.random() < 0.5 else T
    M = int(rng.choice([1, 2, 3, 4, 5, 8]))
    return T, E, K, ids, gates, C, M


def _brute_compare(T, E, K, ids, gates, C, M, fn=None):
    meta = mo.permute(ids, E, C)
    out = (fn or tr.round_tokens)(meta, ids, gates, M)
    kept = {(int(meta["perm_token"][s]), e) for e in range(E)
            for s in range(int(meta["offsets"][e]), int(meta["offsets"][e + 1]))}
    counts, surv = brute.round_tokens_brute(ids, gates, kept, E, M)
    ok = list(out["counts"]) == counts
    got = [(e, int(out["perm_token"][s])) for e in range(E)
           for s in range(int(out["offsets"][e]), int(out["offsets"][e + 1]))]
    return ok and got == surv


def test_matches_brute_force_on_random_tiny_cases():
    rng = np.random.default_rng(0)
    changed = 0
    for _ in range(300):
        T, E, K, ids, gates, C, M = _random_case(rng)
        assert _brute_compare(T, E, K, ids, gates, C, M), (T, E, K, C, M)
        meta = mo.permute(ids, E, C)
        changed += tr.round_tokens(meta, ids, gates, M)["dropped"] > 0
    assert changed > 30                       # the rule actually fired often


def test_invariants_at_a_realistic_size():
    rng = np.random.default_rng(3)
    T, d, E, K, M = 3000, 16, 8, 2, 256
    X = rng.standard_normal((T, d))
    W_r = rng.standard_normal((d, E)) / 4
    r = mo.route(X, W_r, K)
    meta = mo.permute(r["ids"], E, T)
    out = tr.round_tokens(meta, r["ids"], r["gates"], M)
    c0, c1 = np.diff(meta["offsets"]), np.diff(out["offsets"])
    assert out["dropped"] > 0
    for e in range(E):
        want = c0[e] - c0[e] % M if (c0[e] >= M and c0[e] % M < M / 2) else c0[e]
        assert c1[e] == want
        before = meta["perm_token"][meta["offsets"][e]:meta["offsets"][e + 1]]
        after = out["perm_token"][out["offsets"][e]:out["offsets"][e + 1]]
        assert np.all(np.diff(after) > 0)                     # ascending tokens
        assert set(after) <= set(before)
        gate_of = {int(t): float(r["gates"][t][list(r["ids"][t]).index(e)]) for t in before}
        dropped = set(before) - set(after)
        if dropped:
            assert max(gate_of[t] for t in dropped) <= min(gate_of[t] for t in after)
    inv = out["inv_slot"]
    for t in range(T):
        for k in range(K):
            s = inv[t, k]
            if s >= 0:
                assert out["perm_token"][s] == t
    assert tr.padded_rows(out["offsets"], M) <= tr.padded_rows(meta["offsets"], M)


def test_rounding_removes_exactly_the_dropped_contributions():
    """Y after rounding = Y before minus gate * expert output of each dropped
    assignment (the dropped rows are treated like capacity drops)."""
    rng = np.random.default_rng(5)
    T, d, E, K, n, M = 40, 6, 3, 2, 5, 8
    X = rng.standard_normal((T, d))
    W_r = rng.standard_normal((d, E))
    Wg = rng.standard_normal((E, d, n))
    Wu = rng.standard_normal((E, d, n))
    Wd = rng.standard_normal((E, n, d))
    full = mo.forward(X, W_r, Wg, Wu, Wd, K)
    out = tr.round_tokens(full, full["ids"], full["gates"], M)
    assert out["dropped"] > 0
    _, O = mo.grouped_ffn(X, out["offsets"], out["perm_token"], Wg, Wu, Wd)
    Y = mo.combine(O, full["gates"], out["inv_slot"], d=d)
    expect = full["Y"].copy()
    for t in range(T):
        for k in range(K):
            if full["inv_slot"][t, k] >= 0 and out["inv_slot"][t, k] < 0:
                e = full["ids"][t, k]
                _, o = mo.expert_ffn(X[t][None, :], Wg[e], Wu[e], Wd[e])
                expect[t] -= full["gates"][t, k] * o[0]
    assert np.allclose(Y, expect, rtol=1e-12, atol=1e-12)


def test_counts_below_one_tile_and_large_tiles_are_left_alone():
    rng = np.random.default_rng(9)
    T, E, K = 50, 4, 2
    ids = np.stack([rng.permutation(E)[:K] for _ in range(T)])
    gates = rng.random((T, K))
    meta = mo.permute(ids, E, T)
    out = tr.round_tokens(meta, ids, gates, M=256)
    assert out["dropped"] == 0
    assert np.array_equal(out["inv_slot"], meta["inv_slot"])
    assert tr.rounded_count(300, 256) == 256 and tr.rounded_count(384, 256) == 384
    assert tr.rounded_count(383, 256) == 256 and tr.rounded_count(255, 256) == 255
    assert tr.rounded_count(512, 256) == 512 and tr.rounded_count(639, 256) == 512 and tr.rounded_count(640, 256) == 640


# ---------------------------------------------------------------- planted mistakes

class _NpShim:
    """numpy with a different lexsort, to plant an ordering mistake."""

    def __init__(self, lexsort):
        self._lexsort = lexsort

    def __getattr__(self, name):
        return self._lexsort if name == "lexsort" else getattr(np, name)


def _planted(monkeypatch, kind):
    if kind == "tie_to_smaller_token":
        monkeypatch.setattr(tr, "np", _NpShim(lambda keys: np.lexsort((-keys[0], keys[1]))))
    elif kind == "drop_highest_gates":
        monkeypatch.setattr(tr, "np", _NpShim(lambda keys: np.lexsort((keys[0], -keys[1]))))
    elif kind == "half_remainder_rounds_down":
        monkeypatch.setattr(tr, "rounded_count",
                            lambda c, M: M * (c // M) if c >= M and c % M <= M / 2 else c)
    elif kind == "rounds_below_one_tile":
        monkeypatch.setattr(tr, "rounded_count",
                            lambda c, M: M * (c // M) if (c % M) < M / 2 else c)


@pytest.mark.parametrize("kind", ["tie_to_smaller_token", "drop_highest_gates",
                                  "half_remainder_rounds_down", "rounds_below_one_tile"])
def test_planted_mistakes_are_caught(monkeypatch, kind):
    _planted(monkeypatch, kind)
    g = _golden()
    golden_ok = True
    for c in g["cases"]:
        out = tr.round_tokens(g["before"], g["ids"], np.array(g["gates"]), M=c["M"])
        golden_ok &= np.array_equal(out["inv_slot"], np.array(c["inv_slot"]))
    rng = np.random.default_rng(0)
    brute_ok = all(_brute_compare(*_random_case(rng)) for _ in range(300))
    assert not (golden_ok and brute_ok), kind
