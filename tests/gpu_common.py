"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
compare it with the oracle at the tolerances the layer is judged by."""

import numpy as np
import torch

import top_routing_grouped_amd as moe
from oracle import moe_oracle as mo

# Output tolerance (relative L2): fp32 inputs vs bf16 inputs with fp32 accumulation.
TOL = {"fp32": 1e-5, "bf16": 2e-2}
LOGIT_TOL = 1e-5      # both dtypes: bf16 x bf16 products are exact in fp32
GATE_ATOL = 2e-6


def f32np(t):
    return t.detach().to("cpu", torch.float32).numpy()


def intnp(t):
    return t.detach().cpu().numpy().astype(np.int64)


def device_inputs(inp):
    out = {}
    for k in ("X", "W_r", "W_gate", "W_up", "W_down", "bias"):
        v = inp.get(k)
        out[k] = None if v is None else v.cuda().contiguous()
    return out


# grouped-GEMM kernel choice for a test: the library's own choice, or forced
GEMM_PATHS = {"auto": 0, "tiled": moe.MOE_FLAG_GEMM_TILED, "skinny": moe.MOE_FLAG_GEMM_SKINNY}


def run_stepwise(dev, K, cf, gemm_flags=0):
    """route -> permute -> grouped_ffn -> combine through the C ABI."""
    X, W_gate = dev["X"], dev["W_gate"]
    T, d = X.shape
    E, _, n = W_gate.shape
    dtype = "bf16" if X.dtype == torch.bfloat16 else "fp32"
    desc = moe.make_desc(T, d, E, K, n, dtype, cf)
    ids, gates, logits = moe.route(X, dev["W_r"], K, bias=dev["bias"], want_logits=True, n=n)
    meta = moe.permute(desc, ids)
    ffn_desc = moe.make_desc(T, d, E, K, n, dtype, cf, flags=gemm_flags)
    H, O = moe.grouped_ffn(ffn_desc, X, meta["offsets"], meta["perm_token"], W_gate, dev["W_up"],
                           dev["W_down"])
    Y = moe.combine(desc, O, gates, meta["inv_slot"])
    res = {"desc": desc, "ids": ids, "gates": gates, "logits": logits, "H": H, "O": O, "Y": Y}
    res.update(meta)
    return res


def check_routing(res, inp, K):
    """Logits within tolerance of the fp64 definition; ids and gates from the
    device's own fp32 logits (same decision inputs on both sides)."""
    L_gpu = f32np(res["logits"]).astype(np.float64)
    L_ref = mo.router_logits(f32np(inp["X"]), f32np(inp["W_r"]),
                             None if inp.get("bias") is None else f32np(inp["bias"]))
    assert mo.rel_l2(L_gpu, L_ref) <= LOGIT_TOL
    ids_ref = mo.topk_select(L_gpu, K)
    ids_gpu = intnp(res["ids"])
    assert np.array_equal(ids_gpu, ids_ref), "top-K ids differ"
    g_ref = mo.topk_gates(L_gpu, ids_ref)
    g_gpu = f32np(res["gates"]).astype(np.float64)
    assert np.max(np.abs(g_gpu - g_ref)) <= GATE_ATOL
    return L_gpu, ids_ref, g_ref


def check_permutation(res, ids, E, C):
    ref = mo.permute(ids, E, C)
    for key in ("raw_counts", "counts", "offsets", "inv_slot"):
        assert np.array_equal(intnp(res[key]), ref[key].astype(np.int64)), key
    N = int(ref["offsets"][-1])
    assert np.array_equal(intnp(res["perm_token"])[:N], ref["perm_token"][:N].astype(np.int64))
    return ref


TILE_ROWS = 256      # row tile of the tiled grouped GEMMs (rows of one expert segment)


def check_outputs_streamed(inp, ref, gates, H, O, Y, tol, label=""):
    """Every kept row of H and O and every row of Y against the oracle.

    The oracle runs expert by expert (``forward_by_expert``), so that the
    float64 H and O of only one expert exist at a time.  Each expert segment
    of H and O must meet ``tol`` as a whole, per row tile of TILE_ROWS rows
    (the grouped GEMM's tile, counted from the segment start) and row by
    row; Y must meet it as a whole and row by row (a fully dropped token's
    row is exactly zero on both sides).  Returns the worst values seen."""
    X32 = f32np(inp["X"])
    Wg, Wu, Wd = (f32np(inp[k]) for k in ("W_gate", "W_up", "W_down"))
    Hc, Oc = H.detach().cpu(), O.detach().cpu()
    worst = {"H": 0.0, "O": 0.0, "H_row": 0.0, "O_row": 0.0, "segments": 0, "tiles": 0}

    def visit(e, lo, hi, h, o):
        for name, want in (("H", h), ("O", o)):
            got = Hc[lo:hi] if name == "H" else Oc[lo:hi]
            got = got.to(torch.float64).numpy()
            err = mo.rel_l2(got, want)
            assert err <= tol, f"{label} {name} expert {e} rows [{lo},{hi}): rel-L2 {err:.3e}"
            for r0 in range(0, hi - lo, TILE_ROWS):
                r1 = min(hi - lo, r0 + TILE_ROWS)
                et = mo.rel_l2(got[r0:r1], want[r0:r1])
                assert et <= tol, f"{label} {name} expert {e} tile rows [{lo + r0},{lo + r1}): {et:.3e}"
                worst["tiles"] += name == "H"
            rows = mo.rel_l2_rows(got, want)
            i = int(np.argmax(rows))
            assert rows[i] <= tol, f"{label} {name} expert {e} slot {lo + i}: rel-L2 {rows[i]:.3e}"
            worst[name] = max(worst[name], err)
            worst[name + "_row"] = max(worst[name + "_row"], float(rows[i]))
        worst["segments"] += 1

    Y_ref = mo.forward_by_expert(X32, gates, ref["offsets"], ref["perm_token"], ref["inv_slot"],
                                 Wg, Wu, Wd, visit=visit)
    Y_gpu = Y.detach().cpu().to(torch.float64).numpy()
    err = mo.rel_l2(Y_gpu, Y_ref)
    assert err <= tol, f"{label} Y rel-L2 {err:.3e}"
    rows = mo.rel_l2_rows(Y_gpu, Y_ref)
    i = int(np.argmax(rows))
    assert rows[i] <= tol, f"{label} Y token {i}: rel-L2 {rows[i]:.3e}"
    dropped = np.all(np.asarray(ref["inv_slot"]) < 0, axis=1)
    assert np.all(Y_gpu[dropped] == 0.0)
    worst["Y"], worst["Y_row"] = err, float(rows[i])
    assert worst["segments"] == int(np.count_nonzero(np.asarray(ref["counts"])))
    return worst
