"""GPU parity of the training path (moe_forward_train + moe_backward, through
the C ABI) with the backward oracle (oracle/moe_backward.py).

Small layers are compared whole; the named workloads at full size on every
expert's weight gradients and every row of dX (``backward_by_expert``), plus
dW_r and its zero row sums.
Both sides take the routing decision on the device's exported fp32 logits
(the saved state holds them), so ids, drops and slots must match exactly;
gradients must be within GRAD_TOL relative L2 of the float64 oracle."""

import numpy as np
import pytest
import torch

import moe_inputs as mi
import top_routing_grouped_amd as moe
from gpu_common import LOGIT_TOL, TOL, device_inputs, f32np, intnp
from oracle import moe_backward as mb
from oracle import moe_oracle as mo

pytestmark = pytest.mark.gpu

# bf16 operands; intermediates (pre-activations, dH, g*A, per-slot dX, dl)
# rounded to bf16 (relative error 2^-9 each); every sum in fp32.
GRAD_TOL = 2e-2
GATE_ATOL = 2e-6


def _train(inp, dY, K, cf):
    dev = device_inputs(inp)
    dYd = dY.cuda()
    Y, saved, desc = moe.forward_train(dev["X"], dev["W_r"], dev["W_gate"], dev["W_up"],
                                       dev["W_down"], K, cf, bias=dev["bias"])
    grads = moe.backward(desc, saved, dev["X"], dev["W_r"], dev["W_gate"], dev["W_up"],
                         dev["W_down"], dYd)
    torch.cuda.synchronize()
    return dev, Y, saved, desc, grads


def _np(inp, dY):
    out = {k: (None if inp.get(k) is None else f32np(inp[k]))
           for k in ("X", "W_r", "W_gate", "W_up", "W_down", "bias")}
    out["dY"] = f32np(dY)
    return out


def _check_saved_routing(sv, rec, N):
    """Saved routing state against the oracle's (decisions on the same logits)."""
    assert np.array_equal(intnp(sv["ids"]), rec["ids"])
    assert np.max(np.abs(f32np(sv["gates"]) - rec["gates"])) <= GATE_ATOL
    assert np.array_equal(intnp(sv["inv_slot"]), rec["inv_slot"])
    assert np.array_equal(intnp(sv["offsets"]), rec["offsets"])
    assert np.array_equal(intnp(sv["counts"]), rec["counts"])
    assert np.array_equal(intnp(sv["perm_token"])[:N], rec["perm_token"][:N])


SMALL = [
    # T, d, E, K, n, capacity factor, Zipf bias, some token loses every assignment
    (300, 128, 4, 2, 192, 0.0, False, False),    # ragged row tiles; n below one column tile
    (517, 256, 8, 3, 320, 0.6, True, False),     # capacity drops; n spans a ragged second tile
    (64, 128, 5, 5, 64, 0.0, False, False),      # K = E; E not a multiple of 8
    (1000, 512, 16, 4, 256, 1.0, False, False),
    (3, 64, 2, 1, 64, 0.0, False, False),        # fewer tokens than one row block
    (40, 64, 256, 256, 64, 0.0, False, False),   # K = E = 256: the token kernel's largest K
    (400, 128, 16, 2, 128, 0.25, True, True),    # heavy drops: tokens with no kept slot
]


@pytest.mark.parametrize("T,d,E,K,n,cf,bias,full_drop", SMALL)
def test_small_training_layer_parity(T, d, E, K, n, cf, bias, full_drop):
    print(f"backward parity T={T} d={d} E={E} K={K} n={n} cf={cf} bias={bias}", flush=True)
    inp = mi.draw(T, d, E, n, torch.bfloat16, seed=T, bias="zipf" if bias else None)
    dY = mi.draw_grad_output(T, d, torch.bfloat16, seed=T)
    dev, Y, saved, desc, grads = _train(inp, dY, K, cf)
    # the training forward's Y is the inference forward's (tiled GEMMs), bit for bit
    Y_inf = moe.forward(dev["X"], dev["W_r"], dev["W_gate"], dev["W_up"], dev["W_down"], K, cf,
                        bias=dev["bias"], flags=moe.MOE_FLAG_GEMM_TILED)
    torch.cuda.synchronize()
    assert torch.equal(Y, Y_inf)
    a = _np(inp, dY)
    sv = moe.saved_view(desc, saved)
    L_gpu = f32np(sv["logits"]).astype(np.float64)
    assert mo.rel_l2(L_gpu, mo.router_logits(a["X"], a["W_r"], a["bias"])) <= LOGIT_TOL
    fw = mb.forward_train(a["X"], a["W_r"], a["W_gate"], a["W_up"], a["W_down"], K, cf,
                          bias=a["bias"], logits=L_gpu)
    N = int(fw["offsets"][-1])
    _check_saved_routing(sv, fw, N)
    if full_drop:
        assert bool((fw["inv_slot"] < 0).all(axis=1).any())
    pre = f32np(sv["preact"])[:N]
    assert mo.rel_l2(pre[:, :n], fw["Hg"]) <= TOL["bf16"]
    assert mo.rel_l2(pre[:, n:], fw["Hu"]) <= TOL["bf16"]
    assert mo.rel_l2(f32np(Y), fw["Y"]) <= TOL["bf16"]
    ref = mb.backward(a["dY"], fw, a["X"], a["W_r"], a["W_gate"], a["W_up"], a["W_down"])
    for name in ("dX", "dW_r", "dW_gate", "dW_up", "dW_down"):
        err = mo.rel_l2(f32np(grads[name]), ref[name])
        assert err <= GRAD_TOL, (name, err)


def test_backward_repeats_bitwise():
    inp = mi.draw(700, 256, 8, 192, torch.bfloat16, seed=5)
    dY = mi.draw_grad_output(700, 256, torch.bfloat16, seed=5)
    dev, _, saved, desc, g1 = _train(inp, dY, 2, 0.0)
    dYd = dY.cuda()
    g2 = moe.backward(desc, saved, dev["X"], dev["W_r"], dev["W_gate"], dev["W_up"],
                      dev["W_down"], dYd)
    torch.cuda.synchronize()
    for name in g1:
        assert torch.equal(g1[name], g2[name]), name


def test_threshold_selection_in_training():
    """MOE_FLAG_TOPK_THRESHOLD in moe_forward_train: Y, the saved state and
    every gradient bit-equal to the default flags' (the backward accepts the
    same desc)."""
    T, d, E, K, n = 700, 256, 16, 4, 128
    print(f"case threshold training T={T} d={d} E={E} K={K} n={n}", flush=True)
    inp = mi.draw(T, d, E, n, torch.bfloat16, seed=19, bias="zipf")
    dev = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
    dY = mi.draw_grad_output(T, d, torch.bfloat16, seed=20).cuda()
    outs = []
    for flags in (0, moe.MOE_FLAG_TOPK_THRESHOLD):
        Y, saved, desc = moe.forward_train(dev["X"], dev["W_r"], dev["W_gate"], dev["W_up"],
                                           dev["W_down"], K, 1.0, bias=dev["bias"], flags=flags)
        g = moe.backward(desc, saved, dev["X"], dev["W_r"], dev["W_gate"], dev["W_up"],
                         dev["W_down"], dY)
        outs.append((Y, saved, g))
    torch.cuda.synchronize()
    (Y0, s0, g0), (Y1, s1, g1) = outs
    assert torch.equal(Y1, Y0)
    v0, v1 = moe.saved_view(desc, s0), moe.saved_view(desc, s1)
    N = int(v0["offsets"][E].item())
    for key in ("logits", "ids", "gates", "inv_slot", "counts", "offsets"):
        assert torch.equal(v1[key], v0[key]), key
    assert torch.equal(v1["perm_token"][:N], v0["perm_token"][:N])
    assert torch.equal(v1["preact"][:N], v0["preact"][:N])
    for key in g0:
        assert torch.equal(g1[key], g0[key]), key


def test_backward_of_an_empty_batch_zeroes_the_weight_gradients():
    d, E, K, n = 128, 8, 2, 128
    desc = moe.make_desc(0, d, E, K, n, "bf16")
    dW = {"dW_r": torch.ones((d, E), device="cuda"),
          "dW_gate": torch.ones((E, d, n), device="cuda"),
          "dW_up": torch.ones((E, d, n), device="cuda"),
          "dW_down": torch.ones((E, n, d), device="cuda")}
    moe.moe_backward(desc, None, None, None, None, None, None, None, None, dW["dW_r"],
                     dW["dW_gate"], dW["dW_up"], dW["dW_down"], None)
    torch.cuda.synchronize()
    for name, t in dW.items():
        assert int(torch.count_nonzero(t)) == 0, name


# ---------------------------------------------------------------- full workloads

FULL = ["qwen3_bf16", "skewed_cap_bf16", "granular_bf16", "mixtral_bf16", "granular_decode_bf16"]


@pytest.mark.parametrize("name", FULL)
def test_workload_full_size_training(name):
    """Full-size training step: the saved routing state bit-exact; the
    weight gradients of every expert (each expert's dW_gate, dW_up and
    dW_down within GRAD_TOL), dX as a whole and row by row, and dW_r, all
    against the oracle run one expert at a time (``backward_by_expert``)."""
    inp = mi.make_inputs(name)
    w = inp["workload"]
    print(f"training workload {name}: T={w.T} d={w.d} E={w.E} K={w.K} n={w.n}", flush=True)
    dY = mi.draw_grad_output(w.T, w.d, torch.bfloat16, seed=0)
    dev, Y, saved, desc, grads = _train(inp, dY, w.K, w.capacity_factor)
    Y_inf = moe.forward(dev["X"], dev["W_r"], dev["W_gate"], dev["W_up"], dev["W_down"], w.K,
                        w.capacity_factor, bias=dev["bias"], flags=moe.MOE_FLAG_GEMM_TILED)
    torch.cuda.synchronize()
    assert torch.equal(Y, Y_inf)
    sv = moe.saved_view(desc, saved)
    L_gpu = f32np(sv["logits"]).astype(np.float64)
    a = _np(inp, dY)
    rec = mb.route_record(a["X"], a["W_r"], w.K, w.capacity_factor, bias=a["bias"], logits=L_gpu)
    N = int(rec["offsets"][-1])
    _check_saved_routing(sv, rec, N)
    g_cpu = {k: v.detach().cpu() for k, v in grads.items()}
    counts = rec["counts"]
    visited = []
    worst = {"dW_gate": 0.0, "dW_up": 0.0, "dW_down": 0.0}

    def visit(e, dwg, dwu, dwd):
        visited.append(e)
        for nm, want in (("dW_gate", dwg), ("dW_up", dwu), ("dW_down", dwd)):
            err = mo.rel_l2(g_cpu[nm][e].numpy(), want)
            assert err <= GRAD_TOL, (nm, e, err)
            worst[nm] = max(worst[nm], err)

    ref = mb.backward_by_expert(a["dY"], rec, a["X"], a["W_r"], a["W_gate"], a["W_up"],
                                a["W_down"], visit=visit)
    assert visited == [e for e in range(w.E) if counts[e] > 0]
    # experts that kept no row have exactly zero weight gradients
    for e in np.flatnonzero(counts == 0):
        for nm in ("dW_gate", "dW_up", "dW_down"):
            assert int(torch.count_nonzero(g_cpu[nm][int(e)])) == 0
    dX = g_cpu["dX"].to(torch.float64).numpy()
    assert mo.rel_l2(dX, ref["dX"]) <= GRAD_TOL
    rows = mo.rel_l2_rows(dX, ref["dX"])
    assert float(rows.max()) <= GRAD_TOL, (int(np.argmax(rows)), float(rows.max()))
    assert mo.rel_l2(g_cpu["dW_r"].numpy(), ref["dW_r"]) <= GRAD_TOL
    # dl rows sum to zero, so do the rows of dW_r (up to dl's bf16 rounding)
    dWr = grads["dW_r"].double()
    assert float(dWr.sum(dim=1).norm()) <= GRAD_TOL * float(dWr.norm())
    assert float(dWr.norm()) > 0
    print(f"training workload {name}: worst per-expert {worst}, dX rel-L2 "
          f"{mo.rel_l2(dX, ref['dX']):.3e} (worst row {float(rows.max()):.3e}), dW_r "
          f"{mo.rel_l2(g_cpu['dW_r'].numpy(), ref['dW_r']):.3e}", flush=True)
