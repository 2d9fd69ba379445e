"""GPU parity of the atomic-expert layer (moe_omni_route / moe_omni_permute /
moe_omni_forward through the C ABI) with the oracle (oracle/omni_oracle.py).

The oracle takes its routing decision on the device's exported fp32
log-softmax rows (adding them in float32 as the device does), so ids must
match bit for bit; the rows themselves are checked against the float64
definition, gates within 2e-6, the permutation bit for bit, Y within the bf16
tolerance (every row at full size)."""

import numpy as np
import pytest
import torch

import moe_inputs as mi
import top_routing_grouped_amd as moe
from gpu_common import TOL, f32np, intnp
from oracle import moe_oracle as mo
from oracle import omni_oracle as om

pytestmark = pytest.mark.gpu
SCORE_TOL = 1e-5
GATE_ATOL = 2e-6


def _run(inp, K):
    dev = {k: inp[k].cuda() for k in ("X", "W_r", "W_c", "W_in", "W_out")}
    ids, gates, ls_r, ls_c = moe.omni_route(dev["X"], dev["W_r"], dev["W_c"], K)
    desc = moe.make_omni_desc(dev["X"].shape[0], dev["X"].shape[1], dev["W_r"].shape[1],
                              dev["W_c"].shape[1], K)
    meta = moe.omni_permute(desc, ids)
    Y = moe.omni_forward(dev["X"], dev["W_r"], dev["W_c"], dev["W_in"], dev["W_out"], K)
    torch.cuda.synchronize()
    return dev, ids, gates, ls_r, ls_c, meta, Y


def _check_route_and_permutation(inp, K, ids, gates, ls_r, ls_c, meta):
    a = {k: f32np(inp[k]) for k in ("X", "W_r", "W_c")}
    ref_r, ref_c = om.axis_scores(a["X"], a["W_r"], a["W_c"])
    lr, lc = f32np(ls_r), f32np(ls_c)
    assert mo.rel_l2(lr, ref_r) <= SCORE_TOL and mo.rel_l2(lc, ref_c) <= SCORE_TOL
    rid, S = om.select_pruned(lr, lc, K, float32=True)
    assert np.array_equal(intnp(ids), rid)
    assert np.max(np.abs(f32np(gates) - om.gates_from_scores(S))) <= GATE_ATOL
    N = inp["W_r"].shape[1] * inp["W_c"].shape[1]
    T = inp["X"].shape[0]
    pm = mo.permute(rid, N, T)
    for key in ("counts", "offsets", "inv_slot"):
        assert np.array_equal(intnp(meta[key]), pm[key].astype(np.int64)), key
    assert np.array_equal(intnp(meta["perm_token"])[: T * K], pm["perm_token"].astype(np.int64))
    return lr, lc, rid


SHAPES = [
    # T, d, Nr, Nc, K
    (300, 128, 16, 16, 8),
    (257, 64, 4, 9, 5),          # non-square grid
    (100, 128, 1, 32, 3),        # one row
    (50, 64, 8, 8, 64),          # K = N: every expert
    (64, 256, 256, 256, 64),     # largest axes and K
    (3, 64, 5, 5, 7),            # K above each axis' length
    (200, 128, 16, 64, 12),      # both axes in one router launch, the first padded to 64
    (130, 192, 136, 8, 9),       # both axes in one router launch, the second padded to 256
    (96, 1536, 12, 8, 16),       # d in (1024, 2048]: expert and combine kernels with 4 chunks per lane
    (48, 4096, 4, 16, 8),        # d = 4096, the largest: 8 chunks per lane
]


@pytest.mark.parametrize("T,d,Nr,Nc,K", SHAPES)
def test_small_layer_parity(T, d, Nr, Nc, K):
    print(f"atomic-expert layer T={T} d={d} Nr={Nr} Nc={Nc} K={K}", flush=True)
    inp = mi.draw_omni(T, d, Nr, Nc, K, seed=T)
    dev, ids, gates, ls_r, ls_c, meta, Y = _run(inp, K)
    lr, lc, _ = _check_route_and_permutation(inp, K, ids, gates, ls_r, ls_c, meta)
    a = {k: f32np(inp[k]) for k in ("X", "W_r", "W_c", "W_in", "W_out")}
    ref = om.forward(a["X"], a["W_r"], a["W_c"], a["W_in"], a["W_out"], K, scores=(lr, lc))
    assert mo.rel_l2(f32np(Y), ref["Y"]) <= TOL["bf16"]


def test_tied_columns_take_the_best_rows_lowest_columns():
    T, d, Nr, Nc, K = 40, 64, 8, 16, 6
    inp = mi.draw_omni(T, d, Nr, Nc, K, seed=3)
    inp["W_c"] = torch.zeros_like(inp["W_c"])
    dev, ids, gates, ls_r, ls_c, meta, Y = _run(inp, K)
    lr, lc, rid = _check_route_and_permutation(inp, K, ids, gates, ls_r, ls_c, meta)
    best = np.argmax(lr, axis=1)
    assert np.array_equal(rid, best[:, None] * Nc + np.arange(K)[None, :])
    assert np.allclose(f32np(gates), 1.0 / K, atol=GATE_ATOL)


def test_hot_experts_are_ranked_by_token_mask():
    """Every token's strongest row and column are row 3 and column 7, so the
    atomic expert (3, 7) is chosen by all T tokens and its row and column
    neighbours by many: segments far longer than 64 entries, ranked through
    the token mask.  Routing, permutation and Y against the oracle."""
    T, d, Nr, Nc, K = 3000, 128, 16, 16, 8
    inp = mi.draw_omni(T, d, Nr, Nc, K, seed=13)
    X = inp["X"].float()
    X[:, 0] = 4.0
    inp["X"] = X.to(torch.bfloat16)
    for key, col in (("W_r", 3), ("W_c", 7)):
        W = inp[key].float()
        W[0, col] = 2.0
        inp[key] = W.to(torch.bfloat16)
    dev, ids, gates, ls_r, ls_c, meta, Y = _run(inp, K)
    lr, lc, rid = _check_route_and_permutation(inp, K, ids, gates, ls_r, ls_c, meta)
    counts = intnp(meta["counts"])
    assert counts[3 * Nc + 7] == T
    assert int((counts > 64).sum()) >= 3
    a = {k: f32np(inp[k]) for k in ("X", "W_r", "W_c", "W_in", "W_out")}
    ref = om.forward(a["X"], a["W_r"], a["W_c"], a["W_in"], a["W_out"], K, scores=(lr, lc))
    Yg = f32np(Y)
    assert mo.rel_l2(Yg, ref["Y"]) <= TOL["bf16"]
    assert float(mo.rel_l2_rows(Yg, ref["Y"]).max()) <= TOL["bf16"]


def test_repeat_runs_are_bitwise_identical():
    inp = mi.draw_omni(500, 128, 32, 32, 16, seed=4)
    dev, *_, Y1 = _run(inp, 16)
    Y2 = moe.omni_forward(dev["X"], dev["W_r"], dev["W_c"], dev["W_in"], dev["W_out"], 16)
    torch.cuda.synchronize()
    assert torch.equal(Y1, Y2)


def test_workload_full_size_atomic_experts():
    """The 65536-expert workload at full size: routing and the permutation
    bit-exact, and every row of Y against the whole oracle forward (as a
    whole and row by row)."""
    inp = mi.make_omni_inputs("omni_bf16")
    w = inp["workload"]
    print(f"atomic-expert workload: T={w.T} d={w.d} Nr={w.Nr} Nc={w.Nc} K={w.K}", flush=True)
    dev, ids, gates, ls_r, ls_c, meta, Y = _run(inp, w.K)
    lr, lc, rid = _check_route_and_permutation(inp, w.K, ids, gates, ls_r, ls_c, meta)
    a = {k: f32np(inp[k]) for k in ("X", "W_r", "W_c", "W_in", "W_out")}
    ref = om.forward(a["X"], a["W_r"], a["W_c"], a["W_in"], a["W_out"], w.K, scores=(lr, lc))
    assert np.array_equal(ref["ids"], rid)
    Yg = f32np(Y)
    assert mo.rel_l2(Yg, ref["Y"]) <= TOL["bf16"]
    rows = mo.rel_l2_rows(Yg, ref["Y"])
    assert float(rows.max()) <= TOL["bf16"], (int(np.argmax(rows)), float(rows.max()))
    print(f"atomic-expert workload: Y rel-L2 {mo.rel_l2(Yg, ref['Y']):.3e}, worst row "
          f"{float(rows.max()):.3e}", flush=True)
