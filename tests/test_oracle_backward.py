"""Pins of the backward oracle (oracle/moe_backward.py) against things it does
not compute itself: central finite differences of the forward oracle's loss
sum(Y * dY), the identity <dY, O> = <dA', A> of the SonicMoE article §6.4,
and planted mistakes that those pins must catch."""

import numpy as np
import pytest

from oracle import moe_backward as mb
from oracle import moe_oracle as mo


def _layer(T, d, E, K, n, seed, bias=False):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((T, d))
    W_r = rng.standard_normal((d, E)) / np.sqrt(d)
    W_gate = rng.standard_normal((E, d, n)) / np.sqrt(d)
    W_up = rng.standard_normal((E, d, n)) / np.sqrt(d)
    W_down = rng.standard_normal((E, n, d)) / np.sqrt(n)
    dY = rng.standard_normal((T, d))
    b = np.array([1.5 * np.log(1.0 / (e + 1)) for e in range(E)]) if bias else None
    return X, W_r, W_gate, W_up, W_down, dY, b


CASES = [
    # T, d, E, K, n, capacity factor, bias, seed
    (6, 8, 4, 2, 5, 0.0, False, 1),
    (7, 6, 5, 3, 4, 0.5, True, 2),      # capacity drops (C = 3 of up to 7)
    (5, 4, 3, 3, 3, 0.0, False, 3),     # K = E
]


def _fd_check(T, d, E, K, n, cf, bias, seed, bwd=mb.backward):
    X, W_r, Wg, Wu, Wd, dY, b = _layer(T, d, E, K, n, seed, bias)
    fw = mb.forward_train(X, W_r, Wg, Wu, Wd, K, cf, bias=b)
    g = bwd(dY, fw, X, W_r, Wg, Wu, Wd)
    params = {"X": X, "W_r": W_r, "W_gate": Wg, "W_up": Wu, "W_down": Wd}
    grads = {"X": g["dX"], "W_r": g["dW_r"], "W_gate": g["dW_gate"], "W_up": g["dW_up"],
             "W_down": g["dW_down"]}
    eps = 1e-6
    worst = 0.0
    skipped = 0
    for name, P in params.items():
        G = grads[name]
        assert G.shape == P.shape, name
        for idx in np.ndindex(P.shape):
            vals = []
            same = True
            for sgn in (1.0, -1.0):
                Q = {k: v.copy() for k, v in params.items()}
                Q[name][idx] += sgn * eps
                f = mo.forward(Q["X"], Q["W_r"], Q["W_gate"], Q["W_up"], Q["W_down"], K, cf, bias=b)
                same &= np.array_equal(f["ids"], fw["ids"]) and np.array_equal(f["inv_slot"], fw["inv_slot"])
                vals.append(float(np.sum(f["Y"] * dY)))
            if not same:          # the selection moved: the loss is not differentiable here
                skipped += 1
                continue
            fd = (vals[0] - vals[1]) / (2 * eps)
            err = abs(fd - G[idx]) / (1e-6 + abs(fd))
            worst = max(worst, err)
    return worst, skipped


@pytest.mark.parametrize("T,d,E,K,n,cf,bias,seed", CASES)
def test_backward_matches_central_differences(T, d, E, K, n, cf, bias, seed):
    worst, skipped = _fd_check(T, d, E, K, n, cf, bias, seed)
    assert skipped == 0
    assert worst < 1e-5, worst


def test_capacity_case_really_drops():
    X, W_r, Wg, Wu, Wd, dY, b = _layer(7, 6, 5, 3, 4, 2, True)
    fw = mb.forward_train(X, W_r, Wg, Wu, Wd, 3, 0.5, bias=b)
    assert np.any(fw["inv_slot"] < 0)
    g = mb.backward(dY, fw, X, W_r, Wg, Wu, Wd)
    assert np.all(g["dg"][fw["inv_slot"] < 0] == 0.0)     # dropped: no score gradient


def test_score_gradient_identity_of_the_reordering():
    """dS computed as <dA', A> (the backward's way) equals <dY, O> with O
    from the forward oracle (the way the reordering avoids)."""
    X, W_r, Wg, Wu, Wd, dY, b = _layer(9, 8, 4, 2, 6, 7)
    fw = mb.forward_train(X, W_r, Wg, Wu, Wd, 2, 0.0)
    g = mb.backward(dY, fw, X, W_r, Wg, Wu, Wd)
    perm = fw["perm_token"][: fw["offsets"][-1]]
    direct = np.sum(dY[perm] * fw["O"], axis=1)
    assert np.allclose(g["dS"], direct, rtol=1e-12, atol=1e-12)


def test_saved_preactivations_reproduce_the_forward():
    X, W_r, Wg, Wu, Wd, dY, b = _layer(9, 8, 4, 2, 6, 8)
    fw = mb.forward_train(X, W_r, Wg, Wu, Wd, 2, 0.0)
    assert np.allclose(mo.silu(fw["Hg"]) * fw["Hu"], fw["H"], rtol=1e-13, atol=1e-13)


def test_dsilu_is_the_derivative_of_silu():
    z = np.linspace(-8, 8, 101)
    h = 1e-6
    fd = (mo.silu(z + h) - mo.silu(z - h)) / (2 * h)
    assert np.allclose(mb.dsilu(z), fd, rtol=1e-8, atol=1e-9)


# ---------------------------------------------------------------- planted mistakes

def _planted(kind):
    def bwd(dY, fw, X, W_r, Wg, Wu, Wd):
        if kind == "dsilu_is_sigmoid":
            orig = mb.dsilu
            mb.dsilu = mb.sigmoid
            try:
                return mb.backward(dY, fw, X, W_r, Wg, Wu, Wd)
            finally:
                mb.dsilu = orig
        g = mb.backward(dY, fw, X, W_r, Wg, Wu, Wd)
        if kind == "no_renormalisation_term":
            gates = np.asarray(fw["gates"])
            dl = np.zeros_like(g["dl"])
            for k in range(gates.shape[1]):
                dl[np.arange(len(gates)), fw["ids"][:, k]] += gates[:, k] * g["dg"][:, k]
            g["dW_r"] = np.asarray(X).T @ dl
            g["dX"] = g["dX_ffn"] + dl @ np.asarray(W_r).T
        elif kind == "gate_left_out_of_dA":
            fw2 = dict(fw)
            fw2["gates"] = np.ones_like(np.asarray(fw["gates"]))
            g2 = mb.expert_backward(dY, fw2, X, Wg, Wu, Wd)
            g["dW_gate"], g["dW_up"] = g2["dW_gate"], g2["dW_up"]
        elif kind == "dW_down_without_gate":
            fw2 = dict(fw)
            fw2["gates"] = np.ones_like(np.asarray(fw["gates"]))
            g["dW_down"] = mb.expert_backward(dY, fw2, X, Wg, Wu, Wd)["dW_down"]
        elif kind == "router_dX_dropped":
            g["dX"] = g["dX_ffn"]
        return g
    return bwd


@pytest.mark.parametrize("kind", ["dsilu_is_sigmoid", "no_renormalisation_term",
                                  "gate_left_out_of_dA", "dW_down_without_gate",
                                  "router_dX_dropped"])
def test_planted_mistakes_are_caught(kind):
    worst, _ = _fd_check(6, 8, 4, 2, 5, 0.0, False, 1, bwd=_planted(kind))
    assert worst > 1e-3, kind


def test_router_gradient_rows_sum_to_zero():
    """dl[t] = J_t dg with J the softmax-over-the-K Jacobian, whose columns sum
    to zero; so every row of dl, and of dW_r = X^T dl, sums to zero."""
    X, W_r, Wg, Wu, Wd, dY, b = _layer(11, 8, 6, 3, 4, 9, bias=True)
    fw = mb.forward_train(X, W_r, Wg, Wu, Wd, 3, 0.5, bias=b)
    g = mb.backward(dY, fw, X, W_r, Wg, Wu, Wd)
    assert np.max(np.abs(g["dl"].sum(axis=1))) < 1e-13
    assert np.max(np.abs(g["dW_r"].sum(axis=1))) < 1e-12
    assert np.max(np.abs(g["dl"])) > 1e-3


@pytest.mark.parametrize("cf,bias", [(0.0, False), (0.5, True)])
def test_sampled_backward_matches_whole(cf, bias):
    T, d, E, K, n = 13, 8, 5, 2, 6
    X, W_r, Wg, Wu, Wd, dY, b = _layer(T, d, E, K, n, 11, bias)
    fw = mb.forward_train(X, W_r, Wg, Wu, Wd, K, cf, bias=b)
    whole = mb.backward(dY, fw, X, W_r, Wg, Wu, Wd)
    rec = mb.route_record(X, W_r, K, cf, bias=b)
    for key in ("ids", "inv_slot", "offsets", "perm_token"):
        assert np.array_equal(rec[key], fw[key])
    part = mb.sampled_backward(dY, rec, X, W_r, Wg, Wu, Wd, experts=range(E), tokens=range(T))
    for e in range(E):
        for name in ("dW_gate", "dW_up", "dW_down"):
            assert np.allclose(part[name][e], whole[name][e], rtol=1e-12, atol=1e-12)
    for t in range(T):
        assert np.allclose(part["dX"][t], whole["dX"][t], rtol=1e-12, atol=1e-12)
        assert np.allclose(part["dl"][t], whole["dl"][t], rtol=1e-12, atol=1e-12)


def _by_expert_as_whole(dY, fw, X, W_r, Wg, Wu, Wd):
    """backward_by_expert with the visited weight gradients gathered back
    into [E, ...] arrays (experts with no kept row stay zero)."""
    E = Wg.shape[0]
    out = {"dW_gate": np.zeros(Wg.shape), "dW_up": np.zeros(Wu.shape), "dW_down": np.zeros(Wd.shape)}
    seen = []

    def visit(e, dwg, dwu, dwd):
        seen.append(e)
        out["dW_gate"][e], out["dW_up"][e], out["dW_down"][e] = dwg, dwu, dwd

    r = mb.backward_by_expert(dY, fw, X, W_r, Wg, Wu, Wd, visit=visit)
    assert seen == [e for e in range(E) if fw["offsets"][e + 1] > fw["offsets"][e]]
    out.update(r)
    return out


@pytest.mark.parametrize("cf,bias", [(0.0, False), (0.5, True)])
def test_backward_by_expert_matches_whole(cf, bias):
    T, d, E, K, n = 17, 8, 6, 3, 5
    X, W_r, Wg, Wu, Wd, dY, b = _layer(T, d, E, K, n, 21, bias)
    fw = mb.forward_train(X, W_r, Wg, Wu, Wd, K, cf, bias=b)
    whole = mb.backward(dY, fw, X, W_r, Wg, Wu, Wd)
    rec = mb.route_record(X, W_r, K, cf, bias=b)
    part = _by_expert_as_whole(dY, rec, X, W_r, Wg, Wu, Wd)
    for name in ("dX", "dW_r", "dW_gate", "dW_up", "dW_down", "dl", "dS"):
        assert np.allclose(part[name], whole[name], rtol=1e-12, atol=1e-12), name


@pytest.mark.parametrize("T,d,E,K,n,cf,bias,seed", CASES[1:2])
def test_backward_by_expert_matches_central_differences(T, d, E, K, n, cf, bias, seed):
    worst, skipped = _fd_check(T, d, E, K, n, cf, bias, seed, bwd=_by_expert_as_whole)
    assert skipped == 0
    assert worst < 1e-5
