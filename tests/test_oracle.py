"""Pins of the CPU oracle against things other than itself (CPU only).

Each test checks the oracle against one of: the worked example printed on the
OmniMoE page (tests/golden), the independent pure-Python brute force, a
closed form, an invariant, or a special case that reduces to a textbook
computation.  ``test_planted_mistakes`` shows that plausible mistakes planted
in a copy of the oracle fail at least one of these pins.
"""

import json
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import expit

from oracle import brute
from oracle import moe_oracle as mo

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _tiny(T, d, E, n, seed, scale_r=1.0):
    g = torch.Generator().manual_seed(seed)
    X = torch.randn(T, d, generator=g, dtype=torch.float64).numpy()
    W_r = (torch.randn(d, E, generator=g, dtype=torch.float64) * scale_r / math.sqrt(d)).numpy()
    Wg = (torch.randn(E, d, n, generator=g, dtype=torch.float64) / math.sqrt(d)).numpy()
    Wu = (torch.randn(E, d, n, generator=g, dtype=torch.float64) / math.sqrt(d)).numpy()
    Wd = (torch.randn(E, n, d, generator=g, dtype=torch.float64) / math.sqrt(n)).numpy()
    return X, W_r, Wg, Wu, Wd


# ---------------------------------------------------------------- worked example

def _load_example():
    with open(os.path.join(GOLDEN, "worked_example_permute.json")) as f:
        return json.load(f)


@pytest.mark.parametrize("case", ["uncapped", "capped"])
def test_worked_example(case):
    ex = _load_example()
    ids = np.array(ex["ids"], dtype=np.int32)
    exp = ex[case]
    got = mo.permute(ids, ex["E"], exp["C"])
    for key in ("raw_counts", "counts", "offsets", "inv_slot"):
        assert got[key].tolist() == exp[key], key
    N = got["offsets"][-1]
    assert got["perm_token"][:N].tolist() == exp["perm_token"]


def test_worked_example_page_groups_and_eta():
    ex = _load_example()
    ids = np.array(ex["ids"], dtype=np.int32)
    got = mo.permute(ids, ex["E"], 3)
    off = got["offsets"]
    for e, toks in ex["page_groups"].items():
        e = int(e)
        assert got["perm_token"][off[e]:off[e + 1]].tolist() == toks
    active = int(np.count_nonzero(got["counts"]))
    assert ids.size / active == ex["eta"]


def test_worked_example_brute_agrees():
    ex = _load_example()
    for case in ("uncapped", "capped"):
        b = brute.brute_permute(ex["ids"], ex["E"], ex[case]["C"])
        assert b["offsets"] == ex[case]["offsets"]
        assert b["perm_token"] == ex[case]["perm_token"]
        assert b["inv_slot"] == ex[case]["inv_slot"]


# ---------------------------------------------------------------- brute force

SHAPES = [
    # T, d, E, K, n, cf
    (7, 5, 4, 2, 6, 0.0),
    (13, 8, 8, 3, 4, 0.0),
    (16, 6, 5, 5, 3, 0.0),     # K = E
    (20, 4, 6, 1, 5, 0.0),     # K = 1
    (24, 6, 8, 2, 4, 0.75),    # capacity drops
    (30, 5, 3, 2, 4, 0.5),
    (9, 3, 1, 1, 2, 0.0),      # single expert
]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_forward_matches_brute(shape, seed):
    T, d, E, K, n, cf = shape
    X, W_r, Wg, Wu, Wd = _tiny(T, d, E, n, seed, scale_r=3.0)
    bias = np.linspace(0.5, -0.5, E)
    ref = mo.forward(X, W_r, Wg, Wu, Wd, K, cf, bias=bias)
    C = mo.capacity(T, K, E, cf)
    b = brute.brute_forward(X, W_r, Wg, Wu, Wd, K, C, bias=bias)
    np.testing.assert_allclose(ref["logits"], np.array(b["logits"]), rtol=1e-12, atol=1e-12)
    assert ref["ids"].tolist() == b["ids"]
    np.testing.assert_allclose(ref["gates"], np.array(b["gates"]), rtol=1e-12, atol=1e-14)
    for key in ("raw_counts", "counts", "offsets", "inv_slot"):
        assert ref[key].tolist() == b[key], key
    N = int(ref["offsets"][-1])
    assert ref["perm_token"][:N].tolist() == b["perm_token"]
    np.testing.assert_allclose(ref["H"], np.array(b["H"]).reshape(N, n), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(ref["O"], np.array(b["O"]).reshape(N, d), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(ref["Y"], np.array(b["Y"]), rtol=1e-10, atol=1e-12)


def test_routing_on_given_logits_matches_brute():
    """Selection and gates on externally given fp32 scores (the device path)."""
    rng = np.random.default_rng(5)
    L = rng.standard_normal((40, 16)).astype(np.float32).astype(np.float64)
    L[3, :] = 0.25                         # all equal
    L[7, [2, 9]] = L[7].max() + 1.0        # exact tie at the top
    ids = mo.topk_select(L, 4)
    assert ids.tolist() == brute.brute_select(L, 4)
    np.testing.assert_allclose(mo.topk_gates(L, ids), np.array(brute.brute_gates(L, ids.tolist())),
                               rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------------- ties

def test_topk_all_equal_gives_lowest_ids():
    L = np.full((3, 10), -1.5)
    assert mo.topk_select(L, 4).tolist() == [[0, 1, 2, 3]] * 3


def test_topk_signed_zero_is_a_tie():
    L = np.array([[-3.0, -0.0, -2.0, 0.0, -1.0],
                  [-3.0, 0.0, -2.0, -0.0, -1.0]])
    assert mo.topk_select(L, 2).tolist() == [[1, 3], [1, 3]]
    assert brute.brute_select(L, 2) == [[1, 3], [1, 3]]


def test_topk_duplicated_router_columns_tie_to_lower_id():
    X, W_r, *_ = _tiny(12, 6, 6, 2, 3)
    W_r[:, 4] = W_r[:, 1]                  # experts 1 and 4 always tie exactly
    L = mo.router_logits(X, W_r)
    ids = mo.topk_select(L, 6)
    pos = {e: i for i, e in enumerate(ids[0])}
    for row in ids:
        p = {e: i for i, e in enumerate(row)}
        assert p[1] + 1 == p[4]            # adjacent, lower id first
    assert pos


def test_topk_k_equals_e_is_a_descending_sort():
    rng = np.random.default_rng(1)
    L = rng.standard_normal((5, 9))
    ids = mo.topk_select(L, 9)
    for t in range(5):
        assert sorted(ids[t].tolist()) == list(range(9))
        vals = L[t, ids[t]]
        assert np.all(np.diff(vals) <= 0)


def test_topk_rejects_nonfinite():
    with pytest.raises(ValueError):
        mo.topk_select(np.array([[0.0, np.nan]]), 1)


# ---------------------------------------------------------------- gates

def test_gate_closed_forms():
    rng = np.random.default_rng(2)
    L = rng.standard_normal((50, 12)) * 3
    for K in (1, 3, 12):
        ids = mo.topk_select(L, K)
        g = mo.topk_gates(L, ids)
        np.testing.assert_allclose(g.sum(axis=1), 1.0, atol=1e-12)
        if K == 1:
            assert np.all(g == 1.0)
        else:
            sel = np.take_along_axis(L, ids.astype(np.int64), axis=1)
            np.testing.assert_allclose(g[:, 0] / g[:, 1], np.exp(sel[:, 0] - sel[:, 1]), rtol=1e-12)
    eq = np.zeros((2, 6))
    np.testing.assert_allclose(mo.topk_gates(eq, mo.topk_select(eq, 4)), 0.25, rtol=0, atol=0)


def test_silu_matches_library_logistic():
    z = np.linspace(-40, 40, 2001)
    np.testing.assert_allclose(mo.silu(z), z * expit(z), rtol=1e-14, atol=1e-300)
    assert mo.silu(np.array([-1000.0]))[0] == 0.0


# ---------------------------------------------------------------- capacity

def test_capacity_values():
    assert mo.capacity(8192, 4, 64, 1.25) == 640          # skewed workload
    assert mo.capacity(100, 2, 4, 0.0) == 100
    assert mo.capacity(100, 2, 4, -1.0) == 100
    assert mo.capacity(100, 2, 4, 1e-9) == 1
    assert mo.capacity(100, 2, 4, 1e9) == 100
    assert mo.capacity(10, 1, 1, 0.25) == 3                 # 2.5 -> 3
    assert mo.capacity(10, 1, 1, 0.5) == 5                  # exact integer, no round-up
    # the binary value of 0.1 is slightly above 1/10, so cf*T*K/E is slightly above 1
    assert mo.capacity(10, 1, 1, 0.1) == 2
    with pytest.raises(ValueError):
        mo.capacity(10, 1, 1, float("inf"))


# ---------------------------------------------------------------- invariants

@pytest.mark.parametrize("cf", [0.0, 0.6, 1.0, 2.0])
def test_permutation_invariants(cf):
    rng = np.random.default_rng(3)
    T, E, K = 300, 12, 3
    L = rng.standard_normal((T, E)) + np.log(1.0 / (np.arange(E) + 1))[None, :] * 1.5
    ids = mo.topk_select(L, K)
    C = mo.capacity(T, K, E, cf)
    p = mo.permute(ids, E, C)
    raw = np.bincount(ids.ravel(), minlength=E)
    assert p["raw_counts"].tolist() == raw.tolist()
    assert p["counts"].tolist() == np.minimum(raw, C).tolist()
    kept = p["inv_slot"] >= 0
    assert p["counts"].sum() == T * K - (~kept).sum()
    assert p["offsets"][0] == 0
    assert np.array_equal(np.diff(p["offsets"]), p["counts"])
    N = p["offsets"][-1]
    slots = p["inv_slot"][kept]
    assert sorted(slots.tolist()) == list(range(N))                 # each kept pair once
    tt = np.repeat(np.arange(T)[:, None], K, axis=1)
    assert np.array_equal(p["perm_token"][slots], tt[kept])
    for e in range(E):
        seg = p["perm_token"][p["offsets"][e]:p["offsets"][e + 1]]
        assert np.all(np.diff(seg) > 0)                             # ascending tokens
        # kept tokens of e are exactly its C earliest choosers
        choosers = np.nonzero((ids == e).any(axis=1))[0]
        assert seg.tolist() == choosers[:C].tolist()
    ee = ids[kept]
    assert np.all((slots >= p["offsets"][ee]) & (slots < p["offsets"][ee + 1]))


# ---------------------------------------------------------------- special cases

def test_single_expert_is_dense_ffn():
    X, W_r, Wg, Wu, Wd = _tiny(10, 6, 1, 5, 4)
    out = mo.forward(X, W_r, Wg, Wu, Wd, 1)
    v = X @ Wg[0]
    dense = (v * expit(v) * (X @ Wu[0])) @ Wd[0]
    np.testing.assert_allclose(out["Y"], dense, rtol=1e-12, atol=1e-12)


def test_identical_experts_give_ffn_independent_of_routing():
    X, W_r, Wg, Wu, Wd = _tiny(25, 6, 5, 4, 6)
    Wg[:] = Wg[0]
    Wu[:] = Wu[0]
    Wd[:] = Wd[0]
    v = X @ Wg[0]
    dense = (v * expit(v) * (X @ Wu[0])) @ Wd[0]
    for K in (1, 2, 5):
        out = mo.forward(X, W_r, Wg, Wu, Wd, K)
        np.testing.assert_allclose(out["Y"], dense, rtol=1e-11, atol=1e-12)


def test_uniform_router_with_k_equal_e_averages_experts():
    X, W_r, Wg, Wu, Wd = _tiny(9, 5, 4, 3, 7)
    W_r[:] = 0.0
    out = mo.forward(X, W_r, Wg, Wu, Wd, 4)
    np.testing.assert_allclose(out["gates"], 0.25, rtol=0, atol=1e-15)
    avg = np.zeros_like(X)
    for e in range(4):
        v = X @ Wg[e]
        avg += (v * expit(v) * (X @ Wu[e])) @ Wd[e]
    np.testing.assert_allclose(out["Y"], avg / 4, rtol=1e-12, atol=1e-12)


def test_zero_router_weights_give_bias_logits():
    X, W_r, *_ = _tiny(4, 3, 5, 2, 8)
    b = np.array([0.5, -1.0, 2.0, 0.0, 0.25])
    np.testing.assert_array_equal(mo.router_logits(X, np.zeros_like(W_r), b), np.tile(b, (4, 1)))


def test_linearity_in_down_projection():
    X, W_r, Wg, Wu, Wd = _tiny(12, 6, 4, 5, 9)
    a = mo.forward(X, W_r, Wg, Wu, Wd, 2)["Y"]
    b = mo.forward(X, W_r, Wg, Wu, 3.0 * Wd, 2)["Y"]
    np.testing.assert_allclose(b, 3.0 * a, rtol=1e-12, atol=1e-13)


def test_fully_dropped_token_gives_zero_row():
    X, W_r, Wg, Wu, Wd = _tiny(6, 4, 2, 3, 10)
    W_r[:] = 0.0                      # every token picks experts 0 and 1
    out = mo.forward(X, W_r, Wg, Wu, Wd, 2, capacity_factor=0.5)   # C = ceil(0.5*6*2/2) = 3
    assert out["C"] == 3
    assert np.all(out["inv_slot"][3:] == -1)
    assert np.all(out["Y"][3:] == 0.0)
    assert np.any(out["Y"][:3] != 0.0)


def test_sampled_helpers_match_full_forward():
    X, W_r, Wg, Wu, Wd = _tiny(40, 6, 5, 4, 11)
    out = mo.forward(X, W_r, Wg, Wu, Wd, 2, capacity_factor=0.8)
    toks = [0, 5, 17, 39]
    y = mo.token_outputs(toks, X, out["ids"], out["gates"], out["inv_slot"], Wg, Wu, Wd)
    np.testing.assert_allclose(y, out["Y"][toks], rtol=1e-12, atol=1e-14)
    slots = [0, 3, int(out["offsets"][-1]) - 1]
    h, o = mo.slot_outputs(slots, X, out["offsets"], out["perm_token"], Wg, Wu, Wd)
    np.testing.assert_allclose(h, out["H"][slots], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(o, out["O"][slots], rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- planted mistakes

def _pins_pass(m):
    """Run a compact set of the pins above against oracle module ``m``.

    A mutant that raises counts as caught."""
    try:
        return _pins_pass_inner(m)
    except Exception:
        return False


def _pins_pass_inner(m):
    checks = []
    ex = _load_example()
    for case in ("uncapped", "capped"):
        got = m.permute(np.array(ex["ids"], dtype=np.int32), ex["E"], ex[case]["C"])
        checks.append(got["inv_slot"].tolist() == ex[case]["inv_slot"])
    L = np.array([[-3.0, -0.0, -2.0, 0.0, -1.0]])
    checks.append(m.topk_select(L, 2).tolist() == [[1, 3]])
    for shape in SHAPES[:5]:
        T, d, E, K, n, cf = shape
        X, W_r, Wg, Wu, Wd = _tiny(T, d, E, n, 0, scale_r=3.0)
        ref = m.forward(X, W_r, Wg, Wu, Wd, K, cf)
        C = m.capacity(T, K, E, cf)
        b = brute.brute_forward(X, W_r, Wg, Wu, Wd, K, C)
        checks.append(ref["ids"].tolist() == b["ids"])
        checks.append(np.allclose(ref["gates"], np.array(b["gates"]), rtol=1e-10, atol=1e-12))
        checks.append(np.allclose(ref["Y"], np.array(b["Y"]), rtol=1e-8, atol=1e-10))
    checks.append(m.capacity(8192, 4, 64, 1.25) == 640)
    checks.append(m.capacity(10, 1, 1, 0.25) == 3)
    return all(checks)


def test_planted_mistakes(monkeypatch):
    import importlib
    import types

    assert _pins_pass(mo)
    src = open(mo.__file__).read()
    mutants = {
        "tie to higher id": ("order = np.argsort(key, axis=1, kind=\"stable\")",
                             "order = (key.shape[1] - 1 - np.argsort(key[:, ::-1], axis=1, kind=\"stable\"))"),
        "silu sign": ("return z / (1.0 + np.exp(-z))", "return z / (1.0 + np.exp(z))"),
        "no renormalisation": ("return sel / sel.sum(axis=1, keepdims=True)", "return sel"),
        "keep latest tokens": ("if r < C:", "if r >= seen[id_rows[t][k]] - C:"),
        "floor capacity": ("math.ceil(Fraction(cf)", "math.floor(Fraction(cf)"),
        "gate on up branch": ("h = silu(v) * u", "h = silu(u) * v"),
        "inclusive scan": ("offsets[1:] = np.cumsum(counts)", "offsets[:] = np.concatenate([counts, [0]]).cumsum()"),
        "dropped term in combine": ("for k in range(K):\n        kept", "for k in range(K - 1):\n        kept"),
    }
    for name, (old, new) in mutants.items():
        assert old in src, name
        mod = types.ModuleType("oracle_mutant")
        exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
        assert not _pins_pass(mod), "planted mistake not caught: " + name
    importlib.reload(mo)


# ---------------------------------------------------------------- comparison measure

def test_rel_l2_hand_values():
    assert mo.rel_l2([1.0, 1.0], [1.0, 0.0]) == 1.0
    assert mo.rel_l2([6.0, 8.0], [3.0, 4.0]) == 1.0            # |(3,4)| / |(3,4)|
    assert mo.rel_l2([0.0, 0.0], [3.0, 4.0]) == 1.0
    assert mo.rel_l2([1.0, 2.0, 2.0], [1.0, 0.0, 0.0]) == pytest.approx(math.sqrt(8.0), rel=1e-15)
    assert mo.rel_l2([3.0, 4.5], [3.0, 4.0]) == pytest.approx(0.1, rel=1e-15)  # 0.5 / 5
    b = np.array([[1.5, -2.0], [0.25, 7.0]])
    assert mo.rel_l2(b, b) == 0.0
    assert mo.rel_l2(np.zeros(3), np.zeros(3)) == 0.0
    assert mo.rel_l2([0.0, 1e-30], [0.0, 0.0]) == float("inf")
    # not symmetric: the reference is the second argument
    assert mo.rel_l2([2.0], [1.0]) == 1.0 and mo.rel_l2([1.0], [2.0]) == 0.5


def test_rel_l2_rejects_shape_mismatch():
    with pytest.raises(ValueError):
        mo.rel_l2(np.ones((2, 3)), np.ones(3))          # would broadcast silently
    with pytest.raises(ValueError):
        mo.rel_l2(np.ones((4, 1)), np.ones((1, 4)))
    with pytest.raises(ValueError):
        mo.rel_l2_rows(np.ones((2, 3)), np.ones((3, 2)))


def test_rel_l2_rows_hand_values():
    a = np.array([[1.0, 1.0], [6.0, 8.0], [0.0, 0.0], [0.0, 2.0], [3.0, 4.5]])
    b = np.array([[1.0, 0.0], [3.0, 4.0], [0.0, 0.0], [0.0, 0.0], [3.0, 4.0]])
    got = mo.rel_l2_rows(a, b)
    assert got[:4].tolist() == [1.0, 1.0, 0.0, float("inf")]
    assert got[4] == pytest.approx(0.1, rel=1e-15)
    # whole-array value from the rows: squares of the numerators add up
    c = np.array([[3.0, 4.0], [0.0, 5.0]])
    d = np.array([[3.0, 0.0], [0.0, 5.0]])
    assert mo.rel_l2(c, d) == pytest.approx(4.0 / math.sqrt(34.0), rel=1e-15)
    assert mo.rel_l2_rows(c, d).tolist() == [4.0 / 3.0, 0.0]


def test_rel_l2_planted_mistakes():
    import types
    src = open(mo.__file__).read()
    mutants = {
        "denominator from a": ("den = float(np.linalg.norm(b))", "den = float(np.linalg.norm(a))"),
        "squared norms": ("num = float(np.linalg.norm(a - b))", "num = float(np.linalg.norm(a - b)) ** 2"),
        "zero reference passes": ('return 0.0 if num == 0.0 else float("inf")', "return 0.0"),
        "rows: no inf": ("out[~nz & (num > 0.0)] = np.inf", "pass"),
        "rows: denominator from a": ("den = np.linalg.norm(b, axis=1)", "den = np.linalg.norm(a, axis=1)"),
        "no shape check": ("if a.shape != b.shape:\n        raise", "if False:\n        raise"),
    }

    def pins(m):
        try:
            return (m.rel_l2([1.0, 1.0], [1.0, 0.0]) == 1.0
                    and m.rel_l2([1.0], [2.0]) == 0.5
                    and m.rel_l2([3.0, 4.5], [3.0, 4.0]) == pytest.approx(0.1, rel=1e-15)
                    and m.rel_l2([0.0, 1e-30], [0.0, 0.0]) == float("inf")
                    and m.rel_l2_rows(np.array([[0.0, 2.0], [1.0, 1.0]]),
                                      np.array([[0.0, 0.0], [1.0, 0.0]])).tolist() == [float("inf"), 1.0]
                    and m.rel_l2_rows(np.array([[2.0]]), np.array([[1.0]])).tolist() == [1.0]
                    and _raises(lambda: m.rel_l2(np.ones((2, 3)), np.ones(3))))
        except Exception:
            return False

    assert pins(mo)
    for name, (old, new) in mutants.items():
        assert old in src, name
        mod = types.ModuleType("oracle_mutant")
        exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
        assert not pins(mod), "planted mistake not caught: " + name


def _raises(fn):
    try:
        fn()
    except ValueError:
        return True
    return False


@pytest.mark.parametrize("cf,bias", [(0.0, False), (0.6, True)])
def test_forward_by_expert_matches_whole_forward(cf, bias):
    X, W_r, Wg, Wu, Wd = _tiny(60, 8, 7, 6, 12, scale_r=2.0)
    b = np.array([1.5 * math.log(1.0 / (e + 1)) for e in range(7)]) if bias else None
    out = mo.forward(X, W_r, Wg, Wu, Wd, 3, capacity_factor=cf, bias=b)
    seen = []

    def visit(e, lo, hi, h, o):
        seen.append(e)
        np.testing.assert_allclose(h, out["H"][lo:hi], rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(o, out["O"][lo:hi], rtol=1e-13, atol=1e-15)

    Y = mo.forward_by_expert(X, out["gates"], out["offsets"], out["perm_token"], out["inv_slot"],
                             Wg, Wu, Wd, visit=visit)
    assert seen == [e for e in range(7) if out["counts"][e] > 0]
    np.testing.assert_allclose(Y, out["Y"], rtol=1e-12, atol=1e-14)
    # and against the brute force, which shares no step with either
    C = mo.capacity(60, 3, 7, cf)
    bf = brute.brute_forward(X, W_r, Wg, Wu, Wd, 3, C, bias=b)
    np.testing.assert_allclose(Y, np.array(bf["Y"]), rtol=1e-9, atol=1e-11)
    if cf:
        assert np.any(out["inv_slot"] < 0)                # the cap dropped something


def test_forward_by_expert_rejects_unordered_segments():
    X, W_r, Wg, Wu, Wd = _tiny(6, 4, 2, 3, 13)
    ids = np.array([[0], [0], [1], [0], [1], [1]])
    meta = mo.permute(ids, 2, 6)
    perm = meta["perm_token"].copy()
    perm[[0, 1]] = perm[[1, 0]]
    with pytest.raises(ValueError):
        mo.forward_by_expert(X, np.ones((6, 1)), meta["offsets"], perm, meta["inv_slot"], Wg, Wu, Wd)
