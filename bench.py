"""Benchmark of the MoE layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = one pass of the whole hot path over one batch (route -> permute
-> grouped GEMM up -> grouped GEMM down -> combine) on synthetic seeded
inputs already resident in HBM.  The timed region runs K steps through the
C ABI's step-wise entry points with HIP events between the stages on the
stream the kernels run on (the same kernels moe_forward launches); the fused
moe_forward is timed as well.  Prints one JSON line.

Extra modes (used for profiler runs):
    --calib-copy BYTES   only run a plain device-to-device copy of BYTES
                         (the reference kernel for scaling HBM counters).
    --no-cpu-baseline    skip the oracle timing on the host cores.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 MFMA (256 CU x 4096 flop/clk x 2.4 GHz)
PEAK_FP32_TFLOPS = 157.3
PEAK_HBM_GBPS = 8000.0        # MI355X HBM3E
METRIC = "MoE-layer fwd tokens/s; grouped-GEMM MFMA util; permute/combine HBM GB/s"
DEFAULT_WORKLOAD = "qwen3_bf16"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=0,
                    help="tokens for the oracle timing (0 = pick automatically)")
    ap.add_argument("--calib-copy", type=int, default=0)
    return ap.parse_args()


def calib_copy(nbytes: int) -> None:
    import torch
    n = nbytes // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calib_copy_bytes": n * 4, "read_bytes": n * 4, "write_bytes": n * 4}))


def cpu_baseline(inp, w, sample_tokens: int):
    """Time the oracle (as it stands) on the first `sample_tokens` tokens."""
    import numpy as np
    from oracle import moe_oracle as mo
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"] or [1])
    except Exception:  # noqa: BLE001 - informational only
        threads = len(os.sched_getaffinity(0))
    Ts = min(w.T, sample_tokens)
    X = inp["X"][:Ts].float().numpy()
    W_r = inp["W_r"].float().numpy()
    Wg, Wu, Wd = (inp[k].float().numpy() for k in ("W_gate", "W_up", "W_down"))
    bias = None if inp["bias"] is None else inp["bias"].numpy()
    t0 = time.perf_counter()
    out = mo.forward(X, W_r, Wg, Wu, Wd, w.K, w.capacity_factor, bias=bias)
    dt = time.perf_counter() - t0
    assert np.all(np.isfinite(out["Y"]))
    return {"value": Ts / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"oracle forward (numpy fp64) on the first {Ts} of {w.T} tokens of "
                      f"{w.name}, all {w.E} experts' weights; {dt:.2f} s wall",
            "seconds": dt, "host_cpus": len(os.sched_getaffinity(0))}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the layer would shard as described in DESIGN.md, but no multi-GPU path exists)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if args.calib_copy:
        calib_copy(args.calib_copy)
        return

    import moe_inputs as mi
    import top_routing_grouped_amd as moe

    torch.cuda.set_device(0)
    inp = mi.make_inputs(args.workload)
    w = inp["workload"]
    dev = {k: (None if inp[k] is None else inp[k].cuda())
           for k in ("X", "W_r", "W_gate", "W_up", "W_down", "bias")}
    T, d, E, K, n = w.T, w.d, w.E, w.K, w.n
    s = 2 if w.dtype == "bf16" else 4
    desc = moe.make_desc(T, d, E, K, n, w.dtype, w.capacity_factor)
    desc_ready = moe.make_desc(T, d, E, K, n, w.dtype, w.capacity_factor,
                               flags=moe.MOE_FLAG_TILE_TABLE_READY)
    rows = moe.moe_max_rows(desc)
    i32 = dict(dtype=torch.int32, device="cuda")
    ids = torch.empty((T, K), **i32)
    gates = torch.empty((T, K), dtype=torch.float32, device="cuda")
    counts = torch.empty(E, **i32)
    offsets = torch.empty(E + 1, **i32)
    perm = torch.empty(T * K, **i32)
    inv = torch.empty((T, K), **i32)
    H = torch.empty((rows, n), dtype=dev["X"].dtype, device="cuda")
    O = torch.empty((rows, d), dtype=dev["X"].dtype, device="cuda")
    Y = torch.empty((T, d), dtype=dev["X"].dtype, device="cuda")
    ws_p = moe.workspace(desc, moe.MOE_WS_PERMUTE)
    ws_f = moe.workspace(desc, moe.MOE_WS_GROUPED_FFN)
    ws_fwd = moe.workspace(desc, moe.MOE_WS_FORWARD)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev: ev[0].record(stream)
        moe.moe_route(desc, dev["X"], dev["W_r"], dev["bias"], None, ids, gates)
        if ev: ev[1].record(stream)
        moe.moe_permute(desc, ids, counts, offsets, None, perm, inv, ws_p)
        if ev: ev[2].record(stream)
        moe.moe_grouped_gemm_up(desc, dev["X"], offsets, perm, dev["W_gate"], dev["W_up"], H, ws_f)
        if ev: ev[3].record(stream)
        moe.moe_grouped_gemm_down(desc_ready, H, offsets, dev["W_down"], O, ws_f)
        if ev: ev[4].record(stream)
        moe.moe_combine(desc, O, gates, inv, Y)
        if ev: ev[5].record(stream)

    for _ in range(args.warmup):
        step()
        moe.moe_forward(desc, dev["X"], dev["W_r"], dev["bias"], dev["W_gate"], dev["W_up"],
                        dev["W_down"], Y, ws_fwd)
    torch.cuda.synchronize()
    N = int(offsets[E].item())            # kept (token, expert) rows: fixed by the inputs
    active = int((counts > 0).sum().item())

    # ---- timed region: K steps, events between stages
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    stage_ms = [0.0] * 5
    total_ms = 0.0
    for ev in evs:
        for j in range(5):
            stage_ms[j] += ev[j].elapsed_time(ev[j + 1])
        total_ms += ev[0].elapsed_time(ev[5])
    stage_ms = [x / args.steps for x in stage_ms]
    ms_per_step = total_ms / args.steps

    # ---- fused entry point, same work
    f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    f0.record(stream)
    for _ in range(args.steps):
        moe.moe_forward(desc, dev["X"], dev["W_r"], dev["bias"], dev["W_gate"], dev["W_up"],
                        dev["W_down"], Y, ws_fwd)
    f1.record(stream)
    torch.cuda.synchronize()
    fused_ms = f0.elapsed_time(f1) / args.steps

    # ---- algorithmic work (no padding, no pre-gather, active experts only)
    t_route, t_perm, t_up, t_down, t_comb = (x * 1e-3 for x in stage_ms)
    route_bytes = T * d * s + d * E * s + T * K * 8
    perm_bytes = T * K * 4 + N * 4 + T * K * 4 + 2 * E * 4
    comb_bytes = N * d * s + T * K * 8 + T * d * s
    up_flops = 4.0 * N * d * n
    down_flops = 2.0 * N * n * d
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS
    up_tflops = up_flops / t_up / 1e12
    mfma_util = (up_flops + down_flops) / (t_up + t_down) / 1e12 / peak
    value = T / (ms_per_step * 1e-3)

    rec = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic: seeded torch.randn, weights N(0, 1/fan_in), see moe_inputs.py",
        "config": {"workload": w.name, "T": T, "d": d, "E": E, "K": K, "n": n,
                   "capacity_factor": w.capacity_factor, "kept_rows": N, "active_experts": active,
                   "G": d / n, "rho": K / E, "eta": N / max(1, active)},
        "fused_forward_ms": fused_ms,
        "fused_tokens_per_s": T / (fused_ms * 1e-3),
        "wall_s_timed_region": wall,
        "stage_us": {"route": stage_ms[0] * 1e3, "permute": stage_ms[1] * 1e3,
                     "gemm_up": stage_ms[2] * 1e3, "gemm_down": stage_ms[3] * 1e3,
                     "combine": stage_ms[4] * 1e3},
        "grouped_gemm_mfma_util": mfma_util,
        "gemm_up_tflops": up_tflops,
        "gemm_down_tflops": down_flops / t_down / 1e12,
        "route_GBps": route_bytes / t_route / 1e9,
        "permute_GBps": perm_bytes / t_perm / 1e9,
        "combine_GBps": comb_bytes / t_comb / 1e9,
        "roofline": {"bound": "mfma", "achieved": up_tflops, "peak": peak, "unit": "TFLOP/s",
                     "frac": up_tflops / peak, "traffic": None,
                     "kernel": "grouped_gemm_bf16<up> (gather + SwiGLU)",
                     "per_unit": "4*d*n flops per kept (token, expert) row",
                     "units_per_launch": N},
    }
    if not args.no_cpu_baseline:
        sample = args.cpu_sample_tokens or min(T, 16384)
        rec["cpu_baseline"] = cpu_baseline(inp, w, sample)
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
