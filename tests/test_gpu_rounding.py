"""GPU parity of tile-aware token rounding (moe_round_tokens, and moe_forward
with MOE_FLAG_TOKEN_ROUNDING) with the oracle (oracle/token_rounding.py).

The rounding decides on the router's fp32 gates, so the oracle is given the
device's gates (the same decision inputs on both sides); the metadata after
rounding must match bit for bit; H, O and Y within the bf16 / fp32 tolerance
of the float64 oracle evaluated on the rounded metadata, per expert segment,
per row tile and per row (at full size too)."""

import numpy as np
import pytest
import torch

import moe_inputs as mi
import top_routing_grouped_amd as moe
from gpu_common import TOL, check_outputs_streamed, device_inputs, f32np, intnp, run_stepwise
from oracle import moe_oracle as mo
from oracle import token_rounding as tr

pytestmark = pytest.mark.gpu
M = 256          # the tiled GEMM's row tile


def _round_on_device(res, T, d, E, K, n, dtype, cf):
    desc = moe.make_desc(T, d, E, K, n, dtype, cf)
    meta = {k: res[k].clone() for k in ("counts", "offsets", "perm_token", "inv_slot")}
    moe.round_tokens(desc, res["ids"], res["gates"], meta)
    torch.cuda.synchronize()
    return meta


def _check_rounded(meta_dev, res, E, C):
    """Device rounding vs the oracle applied to the oracle's own permutation
    of the device ids, with the device's gates."""
    ids = intnp(res["ids"])
    before = mo.permute(ids, E, C)
    ref = tr.round_tokens(before, ids, f32np(res["gates"]), M)
    for key in ("counts", "offsets", "inv_slot"):
        assert np.array_equal(intnp(meta_dev[key]), ref[key].astype(np.int64)), key
    N = int(ref["offsets"][-1])
    assert np.array_equal(intnp(meta_dev["perm_token"])[:N], ref["perm_token"][:N].astype(np.int64))
    return before, ref


CASES = [
    # T, d, E, K, n, dtype, capacity factor, Zipf bias, whether rows are dropped
    (2100, 128, 4, 2, 128, "bf16", 0.0, False, True),   # ~1050 rows per expert: both branches of the rule
    (3001, 128, 8, 3, 256, "bf16", 0.0, True, True),    # skewed loads
    (2500, 128, 6, 2, 128, "fp32", 1.2, False, True),   # after a capacity cut
    (700, 64, 3, 1, 64, "bf16", 0.0, False, False),     # every expert below one tile: unchanged
    (100, 64, 8, 2, 64, "bf16", 0.0, False, False),
    (1500, 64, 64, 16, 64, "bf16", 0.0, True, True),    # K = 16 under a skewed router
    (1200, 64, 32, 32, 64, "bf16", 0.0, False, False),  # K = E: every expert already holds every token
]


@pytest.mark.parametrize("T,d,E,K,n,dtype,cf,bias,fires", CASES)
def test_rounding_matches_oracle(T, d, E, K, n, dtype, cf, bias, fires):
    print(f"rounding T={T} d={d} E={E} K={K} n={n} {dtype} cf={cf} bias={bias}", flush=True)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    inp = mi.draw(T, d, E, n, tdt, seed=T, bias="zipf" if bias else None)
    dev = device_inputs(inp)
    res = run_stepwise(dev, K, cf)
    C = mo.capacity(T, K, E, cf)
    meta = _round_on_device(res, T, d, E, K, n, dtype, cf)
    before, ref = _check_rounded(meta, res, E, C)
    assert (int(before["offsets"][-1]) > int(ref["offsets"][-1])) == fires
    # the layer on the rounded metadata: fused flag == step-wise chain, and the oracle
    flags = moe.MOE_FLAG_TOKEN_ROUNDING
    Y_fused = moe.forward(dev["X"], dev["W_r"], dev["W_gate"], dev["W_up"], dev["W_down"], K, cf,
                          bias=dev["bias"], flags=flags)
    desc = moe.make_desc(T, d, E, K, n, dtype, cf)
    H, O = moe.grouped_ffn(desc, dev["X"], meta["offsets"], meta["perm_token"], dev["W_gate"],
                           dev["W_up"], dev["W_down"])
    Y_step = moe.combine(desc, O, res["gates"], meta["inv_slot"])
    torch.cuda.synchronize()
    assert torch.equal(Y_fused, Y_step)
    check_outputs_streamed(inp, ref, f32np(res["gates"]), H, O, Y_fused, TOL[dtype])


@pytest.mark.parametrize("T,d,E,K,n,cf,bias", [(3001, 128, 8, 3, 256, 0.0, True),
                                               (1500, 128, 40, 4, 128, 1.0, True)])
def test_rounding_composes_with_the_other_flags(T, d, E, K, n, cf, bias):
    """Flags combined: the threshold selection gives the default selection's
    outputs bit for bit, so with token rounding on as well Y must not change,
    with the default GEMM launch and with the kernel forced to the tiled one."""
    print(f"flags composed T={T} d={d} E={E} K={K} n={n} cf={cf}", flush=True)
    inp = mi.draw(T, d, E, n, torch.bfloat16, seed=T + 1, bias="zipf" if bias else None)
    dev = device_inputs(inp)
    R, TH, TI = moe.MOE_FLAG_TOKEN_ROUNDING, moe.MOE_FLAG_TOPK_THRESHOLD, moe.MOE_FLAG_GEMM_TILED
    out = {}
    for flags in (R, R | TH, R | TI, R | TH | TI):
        out[flags] = moe.forward(dev["X"], dev["W_r"], dev["W_gate"], dev["W_up"], dev["W_down"], K,
                                 cf, bias=dev["bias"], flags=flags)
    torch.cuda.synchronize()
    assert torch.equal(out[R | TH], out[R])
    assert torch.equal(out[R | TH | TI], out[R | TI])


def test_all_ties_drop_the_largest_tokens():
    """A zero router gives every token the same K experts and equal gates:
    each expert keeps its lowest token ids."""
    T, d, E, K, n = 300, 64, 4, 2, 64
    inp = mi.draw(T, d, E, n, torch.bfloat16, seed=1)
    inp["W_r"] = torch.zeros_like(inp["W_r"])
    dev = device_inputs(inp)
    res = run_stepwise(dev, K, 0.0)
    meta = _round_on_device(res, T, d, E, K, n, "bf16", 0.0)
    _check_rounded(meta, res, E, T)
    off = intnp(meta["offsets"])
    perm = intnp(meta["perm_token"])
    for e in range(K):
        assert off[e + 1] - off[e] == 256
        assert np.array_equal(perm[off[e]:off[e + 1]], np.arange(256))
    assert np.all(intnp(meta["inv_slot"])[256:] == -1)


def test_hot_expert_beyond_the_lds_cache():
    """One expert with more rows than the selection kernel keeps in LDS
    (15360): the gates are re-read from memory in every pass."""
    T, d, E, K, n = 20000, 64, 4, 1, 64
    inp = mi.draw(T, d, E, n, torch.bfloat16, seed=2)
    inp["bias"] = torch.tensor([8.0, 0.0, 0.0, 0.0])
    dev = device_inputs(inp)
    res = run_stepwise(dev, K, 0.0)
    counts = intnp(res["counts"])
    assert counts[0] > 15360 and counts[0] % 256 < 128
    meta = _round_on_device(res, T, d, E, K, n, "bf16", 0.0)
    _check_rounded(meta, res, E, T)


@pytest.mark.parametrize("name", ["qwen3_bf16", "granular_bf16", "skewed_cap_bf16"])
def test_workload_full_size_rounding(name):
    """Full-size workloads: the rounded metadata bit-exact; the grouped FFN
    and the combine on it compared with the oracle on every kept row of H
    and O and every row of Y (per expert segment, per row tile, per row);
    the fused flag equal to the step-wise chain."""
    inp = mi.make_inputs(name)
    w = inp["workload"]
    print(f"rounding workload {name}: T={w.T} d={w.d} E={w.E} K={w.K} n={w.n}", flush=True)
    dev = device_inputs(inp)
    res = run_stepwise(dev, w.K, w.capacity_factor)
    C = mo.capacity(w.T, w.K, w.E, w.capacity_factor)
    meta = _round_on_device(res, w.T, w.d, w.E, w.K, w.n, w.dtype, w.capacity_factor)
    before, ref = _check_rounded(meta, res, w.E, C)
    print(f"  dropped {int(before['offsets'][-1]) - int(ref['offsets'][-1])} of "
          f"{int(before['offsets'][-1])}; padded rows {tr.padded_rows(before['offsets'])} -> "
          f"{tr.padded_rows(ref['offsets'])}", flush=True)
    Y = moe.forward(dev["X"], dev["W_r"], dev["W_gate"], dev["W_up"], dev["W_down"], w.K,
                    w.capacity_factor, bias=dev["bias"], flags=moe.MOE_FLAG_TOKEN_ROUNDING)
    desc = moe.make_desc(w.T, w.d, w.E, w.K, w.n, w.dtype, w.capacity_factor)
    H, O = moe.grouped_ffn(desc, dev["X"], meta["offsets"], meta["perm_token"], dev["W_gate"],
                           dev["W_up"], dev["W_down"])
    Y_step = moe.combine(desc, O, res["gates"], meta["inv_slot"])
    torch.cuda.synchronize()
    assert torch.equal(Y, Y_step)
    worst = check_outputs_streamed(inp, ref, f32np(res["gates"]), H, O, Y, TOL[w.dtype],
                                   label=name + " rounded")
    print(f"  {worst}", flush=True)
