"""Benchmark of the MoE layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = one pass of the whole hot path over one batch: moe_forward (route
-> permute -> grouped GEMM up -> grouped GEMM down -> combine) on seeded
synthetic inputs already resident in HBM.  Before every timed step a 1 GiB
scratch buffer is rewritten so that neither L2 nor the 256 MB MALL holds the
inputs (cold cache); each step is bracketed by HIP events on the stream the
kernels run on, and `value` = T / median step time.  Each step is followed
by the same work through the step-wise entry points with events between the
stages (moe_route_permute, up GEMM, down GEMM, combine: the kernels
moe_forward runs; per-stage medians), and by the router alone plus the
standalone permutation (moe_route_ws, moe_permute), each after its own cache
flush; then the up GEMM alone is timed
for the roofline, and everything is repeated without the flush (warm,
labelled as such).  For bf16 workloads the training step (moe_forward_train
then moe_backward on a seeded dY) is timed the same way and reported under
"training"; moe_forward with tile-aware token rounding is timed the same way
under "token_rounding" (with the rows it drops and the row tiles it saves);
the atomic-expert layer (moe_omni_forward on its 4096-token, 65536-expert
workload) is timed the same way under "atomic_experts".  Prints one JSON
line.

Extra modes (used for profiler runs):
    --calib-copy BYTES   only run a plain device-to-device copy of BYTES
                         (the reference kernel for scaling HBM counters).
    --pmc-summary FETCH_DIR WRITE_DIR CALIB_FETCH_DIR CALIB_WRITE_DIR
                         turn four rocprofv3 --pmc runs into the traffic
                         summary under profiles/ (no GPU needed).
    --no-cpu-baseline    skip the oracle timing on the host cores.
    --warm               skip the cache flush (profiling runs).
    --forward-only       skip the training and token-rounding steps (counter runs
                         of the forward GEMMs: the training forward's up GEMM
                         also writes the pre-activations, the rounded forward's
                         GEMMs see fewer rows); --no-train is the same switch.
    --pmc-kernel NAME    kernel-name substring that --pmc-summary averages
                         (default: the tiled up GEMM).
    --gather-study MODE  only time the up GEMM on the workload's routing, K cold
                         launches: MODE "gathered" reads token rows of X through
                         perm_token (the product path), "pregathered" reads a
                         contiguous copy X[perm_token] built beforehand with
                         torch (a measurement baseline, never a product path),
                         "both" interleaves the two.  Prints one JSON line.
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 MFMA (256 CU x 4096 flop/clk x 2.4 GHz)
PEAK_FP32_TFLOPS = 157.3
PEAK_HBM_GBPS = 8000.0        # MI355X HBM3E
METRIC = "MoE-layer fwd tokens/s; grouped-GEMM MFMA util; permute/combine HBM GB/s"
DEFAULT_WORKLOAD = "qwen3_bf16"
FLUSH_BYTES = 1 << 30
GEMM_SOURCES = ("top_routing_grouped_amd/csrc/gemm.hip", "top_routing_grouped_amd/csrc/gemm_stream.hpp",
                "top_routing_grouped_amd/csrc/moe_internal.hpp")
TRAFFIC_FILE = "profiles/gemm_up_traffic_{workload}.json"
UP_KERNEL = "grouped_gemm_bf16<true"


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
    ap.add_argument("--pmc-summary", nargs=4, default=None)
    ap.add_argument("--warm", action="store_true")
    ap.add_argument("--forward-only", "--no-train", dest="forward_only", action="store_true")
    ap.add_argument("--pmc-kernel", default=None)
    ap.add_argument("--gather-study", choices=["gathered", "pregathered", "both"], default=None)
    return ap.parse_args()


def gemm_source_hash() -> str:
    h = hashlib.sha256()
    for rel in GEMM_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


# ---------------------------------------------------------------- counters
def _pmc_per_dispatch(directory: str, counter: str, name_has: str | None):
    """{dispatch: (kernel name, summed counter value)} from rocprofv3 CSVs."""
    out = {}
    for path in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                if name_has and name_has not in r["Kernel_Name"]:
                    continue
                key = (path, r["Dispatch_Id"])
                name, v = out.get(key, (r["Kernel_Name"], 0.0))
                out[key] = (name, v + float(r["Counter_Value"]))
    return out


def pmc_summary(fetch_dir, write_dir, calib_fetch_dir, calib_write_dir, workload, kernel=None):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the up GEMM (or the
    kernel named by `kernel`), scaled by what the same counters read for a
    plain copy of known size."""
    kname = kernel or UP_KERNEL
    cf = _pmc_per_dispatch(calib_fetch_dir, "FETCH_SIZE", None)
    cw = _pmc_per_dispatch(calib_write_dir, "WRITE_SIZE", None)
    # the calibration run copies FLUSH_BYTES (--calib-copy 1073741824): the
    # copy is the dispatch that fetches the most and writes the most
    copy_fetch = max(v for _, v in cf.values()) * 1024.0
    copy_write = max(v for _, v in cw.values()) * 1024.0
    f_scale = FLUSH_BYTES / copy_fetch
    w_scale = FLUSH_BYTES / copy_write
    fu = [v for _, v in _pmc_per_dispatch(fetch_dir, "FETCH_SIZE", kname).values()]
    wu = [v for _, v in _pmc_per_dispatch(write_dir, "WRITE_SIZE", kname).values()]
    fetch = statistics.mean(fu) * 1024.0 * f_scale
    write = statistics.mean(wu) * 1024.0 * w_scale
    rec = {"workload": workload, "kernel": kname, "dispatches": [len(fu), len(wu)],
           "fetch_bytes_per_launch": fetch, "write_bytes_per_launch": write,
           "traffic_bytes_per_launch": fetch + write,
           "fetch_scale": f_scale, "write_scale": w_scale,
           "raw_fetch_kib_mean": statistics.mean(fu), "raw_write_kib_mean": statistics.mean(wu),
           "gemm_source_sha256": gemm_source_hash()}
    out = os.path.join(ROOT, TRAFFIC_FILE.format(workload=workload))
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


def load_traffic(workload: str):
    path = os.path.join(ROOT, TRAFFIC_FILE.format(workload=workload))
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("gemm_source_sha256") != gemm_source_hash():
        return None                       # kernel changed since the counters were taken
    return rec["traffic_bytes_per_launch"]


# ---------------------------------------------------------------- helpers
def calib_copy(nbytes: int) -> None:
    import torch
    n = nbytes // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calib_copy_bytes": n * 4, "read_bytes": n * 4, "write_bytes": n * 4}))


def sha256_tensor(t) -> str:
    import torch
    v = t.detach().contiguous()
    if v.dtype == torch.bfloat16:
        v = v.view(torch.int16)
    return hashlib.sha256(v.numpy().tobytes()).hexdigest()


def blas_info():
    try:
        from threadpoolctl import threadpool_info
        infos = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if infos:
            return infos[0].get("internal_api", "blas"), max(i.get("num_threads", 1) for i in infos)
    except Exception:  # noqa: BLE001 - informational only
        pass
    return "unknown", len(os.sched_getaffinity(0))


def cpu_baseline(inp, w, sample_tokens: int):
    """Time the oracle (as it stands) per stage on the first `sample_tokens`
    tokens of the workload, all experts' weights."""
    import numpy as np
    from oracle import moe_oracle as mo
    vendor, threads = blas_info()
    Ts = min(w.T, sample_tokens)
    X = inp["X"][:Ts].float().numpy()
    W_r = inp["W_r"].float().numpy()
    Wg, Wu, Wd = (inp[k].float().numpy() for k in ("W_gate", "W_up", "W_down"))
    bias = None if inp["bias"] is None else inp["bias"].numpy()
    t = [time.perf_counter()]
    r = mo.route(X, W_r, w.K, bias=bias)
    t.append(time.perf_counter())
    meta = mo.permute(r["ids"], w.E, mo.capacity(Ts, w.K, w.E, w.capacity_factor))
    t.append(time.perf_counter())
    H, O = mo.grouped_ffn(X, meta["offsets"], meta["perm_token"], Wg, Wu, Wd)
    t.append(time.perf_counter())
    Y = mo.combine(O, r["gates"], meta["inv_slot"], d=X.shape[1])
    t.append(time.perf_counter())
    dt = t[-1] - t[0]
    assert np.all(np.isfinite(Y))
    return {"value": Ts / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"oracle forward (numpy fp64, BLAS {vendor}) on the first {Ts} of {w.T} "
                      f"tokens of {w.name}, all {w.E} experts' weights; {dt:.2f} s wall",
            "seconds": dt,
            "stage_seconds": {"route": t[1] - t[0], "permute": t[2] - t[1],
                              "grouped_ffn": t[3] - t[2], "combine": t[4] - t[3]},
            "blas": vendor, "host_cpus": len(os.sched_getaffinity(0))}


def pct(xs, q):
    s = sorted(xs)
    i = min(len(s) - 1, max(0, int(round(q * (len(s) - 1)))))
    return s[i]


def gather_study(args, moe, dev, desc, desc_ready, offsets, perm, H, ws_f, flush, ev, stream, w,
                 N):
    """The up GEMM on the workload's routing with the token rows gathered
    through perm_token (the product path) and, as a baseline, on a
    contiguous pre-gathered copy X[perm_token[:N]] with the identity
    permutation: same kernel, same tile table, same weights and flops; only
    where the A rows come from differs."""
    import torch
    Xg = dev["X"].index_select(0, perm[:N].long()).contiguous()
    ident = torch.arange(max(1, perm.numel()), dtype=torch.int32, device="cuda")
    modes = ["gathered", "pregathered"] if args.gather_study == "both" else [args.gather_study]
    src = {"gathered": (dev["X"], perm), "pregathered": (Xg, ident)}
    # build the tile table once from the offsets (the launches below reuse it)
    moe.moe_grouped_gemm_up(desc, dev["X"], offsets, perm, dev["W_gate"], dev["W_up"], H, ws_f)
    for i in range(args.warmup):
        for m in modes:
            flush(i)
            moe.moe_grouped_gemm_up(desc_ready, src[m][0], offsets, src[m][1], dev["W_gate"],
                                    dev["W_up"], H, ws_f)
    times = {m: [] for m in modes}
    torch.cuda.synchronize()
    for i in range(args.steps):
        for m in modes:
            flush(i)
            a, b = ev(), ev()
            a.record(stream)
            moe.moe_grouped_gemm_up(desc_ready, src[m][0], offsets, src[m][1], dev["W_gate"],
                                    dev["W_up"], H, ws_f)
            b.record(stream)
            torch.cuda.synchronize()
            times[m].append(a.elapsed_time(b) * 1e3)
    flops = 4.0 * N * w.d * w.n
    out = {"gather_study": w.name, "kept_rows": N,
           "a_rows_bytes": {"gathered_X": w.T * w.d * 2, "pregathered_copy": N * w.d * 2}}
    for m in modes:
        out[m] = {"us_mean": statistics.mean(times[m]), "us_median": statistics.median(times[m]),
                  "tflops": flops / (statistics.mean(times[m]) * 1e-6) / 1e12}
    print(json.dumps(out))


# ---------------------------------------------------------------- main
def main():
    args = parse()
    if args.pmc_summary:
        pmc_summary(*args.pmc_summary, args.workload, args.pmc_kernel)
        return
    if args.gpus != 1:
        print(f"bench.py: the layer runs on one GPU only; --gpus {args.gpus} is not supported "
              "(there is no multi-GPU path)", file=sys.stderr)
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
    hashes = {k: sha256_tensor(inp[k]) for k in ("X", "W_r", "W_gate", "W_up", "W_down", "bias")
              if inp[k] is not None}
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
    ws_r = moe.workspace(desc, moe.MOE_WS_ROUTE)
    ws_rp = moe.workspace(desc, moe.MOE_WS_ROUTE_PERMUTE)
    ws_p = moe.workspace(desc, moe.MOE_WS_PERMUTE)
    ws_f = moe.workspace(desc, moe.MOE_WS_GROUPED_FFN)
    ws_fwd = moe.workspace(desc, moe.MOE_WS_FORWARD)
    scratch = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def fused():
        moe.moe_forward(desc, dev["X"], dev["W_r"], dev["bias"], dev["W_gate"], dev["W_up"],
                        dev["W_down"], Y, ws_fwd)

    def stepwise(ev):
        # the stages moe_forward runs: route + fused permutation, up, down, combine
        ev[0].record(stream)
        moe.moe_route_permute(desc, dev["X"], dev["W_r"], dev["bias"], None, ids, gates, counts,
                              offsets, None, perm, inv, ws_rp)
        ev[1].record(stream)
        moe.moe_grouped_gemm_up(desc, dev["X"], offsets, perm, dev["W_gate"], dev["W_up"], H, ws_f)
        ev[2].record(stream)
        moe.moe_grouped_gemm_down(desc_ready, H, offsets, dev["W_down"], O, ws_f)
        ev[3].record(stream)
        moe.moe_combine(desc, O, gates, inv, Y)
        ev[4].record(stream)

    def route_parts(ev):
        # the router alone (moe_route_ws) and the standalone three-launch
        # permutation from its ids (moe_permute)
        ev[0].record(stream)
        moe.moe_route_ws(desc, dev["X"], dev["W_r"], dev["bias"], None, ids, gates, ws_r)
        ev[1].record(stream)
        moe.moe_permute(desc, ids, counts, offsets, None, perm, inv, ws_p)
        ev[2].record(stream)

    def flush(i):
        scratch.fill_(float(i))

    def ev():
        return torch.cuda.Event(enable_timing=True)

    for i in range(args.warmup):
        stepwise([ev() for _ in range(5)])
        route_parts([ev() for _ in range(3)])
        fused()
    torch.cuda.synchronize()
    N = int(offsets[E].item())            # kept (token, expert) rows: fixed by the inputs
    active = int((counts > 0).sum().item())

    def run(cold: bool):
        """K steps of moe_forward, each followed by the same work through the
        step-wise entry points (interleaved, so both see the same clocks and
        temperatures); with `cold`, the cache flush precedes each of them."""
        fev = [(ev(), ev()) for _ in range(args.steps)]
        sev = [[ev() for _ in range(5)] for _ in range(args.steps)]
        rev = [[ev() for _ in range(3)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        for i in range(args.steps):
            if cold:
                flush(3 * i)
            fev[i][0].record(stream)
            fused()
            fev[i][1].record(stream)
            if cold:
                flush(3 * i + 1)
            stepwise(sev[i])
            if cold:
                flush(3 * i + 2)
            route_parts(rev[i])
        torch.cuda.synchronize()
        return ([a.elapsed_time(b) for a, b in fev],
                [[e[j].elapsed_time(e[j + 1]) for j in range(4)] +
                 [r[0].elapsed_time(r[1]), r[1].elapsed_time(r[2])] for e, r in zip(sev, rev)])

    def run_up_kernel(cold: bool):
        """The up-projection GEMM alone (its tile table already built by the
        step-wise calls above from the same offsets), for the roofline."""
        evs = [(ev(), ev()) for _ in range(args.steps)]
        torch.cuda.synchronize()
        for i in range(args.steps):
            if cold:
                flush(i)
            evs[i][0].record(stream)
            moe.moe_grouped_gemm_up(desc_ready, dev["X"], offsets, perm, dev["W_gate"], dev["W_up"],
                                    H, ws_f)
            evs[i][1].record(stream)
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in evs]

    if args.gather_study:
        gather_study(args, moe, dev, desc, desc_ready, offsets, perm, H, ws_f, flush, ev, stream,
                     w, N)
        return

    train = w.dtype == "bf16" and not args.forward_only
    if train:
        dY = mi.draw_grad_output(T, d, torch.bfloat16, seed=0).cuda()
        Y_t = torch.empty_like(Y)
        saved = moe.workspace(desc, moe.MOE_WS_SAVED)
        ws_b = moe.workspace(desc, moe.MOE_WS_BACKWARD)
        g = {"dX": torch.empty((T, d), dtype=torch.bfloat16, device="cuda"),
             "dW_r": torch.empty((d, E), dtype=torch.float32, device="cuda"),
             "dW_gate": torch.empty((E, d, n), dtype=torch.float32, device="cuda"),
             "dW_up": torch.empty((E, d, n), dtype=torch.float32, device="cuda"),
             "dW_down": torch.empty((E, n, d), dtype=torch.float32, device="cuda")}

    def train_step(evs):
        evs[0].record(stream)
        moe.moe_forward_train(desc, dev["X"], dev["W_r"], dev["bias"], dev["W_gate"], dev["W_up"],
                              dev["W_down"], Y_t, saved, ws_fwd)
        evs[1].record(stream)
        moe.moe_backward(desc, dev["X"], dev["W_r"], dev["W_gate"], dev["W_up"], dev["W_down"], dY,
                         saved, g["dX"], g["dW_r"], g["dW_gate"], g["dW_up"], g["dW_down"], ws_b)
        evs[2].record(stream)

    def run_train(cold: bool):
        """K training steps (forward that keeps the backward's state, then the
        backward), each after a cache flush when `cold`."""
        evs = [[ev() for _ in range(3)] for _ in range(args.steps)]
        for i in range(args.warmup):
            train_step([ev() for _ in range(3)])
        torch.cuda.synchronize()
        for i in range(args.steps):
            if cold:
                flush(i)
            train_step(evs[i])
        torch.cuda.synchronize()
        return ([e[0].elapsed_time(e[1]) for e in evs], [e[1].elapsed_time(e[2]) for e in evs])

    desc_round = moe.make_desc(T, d, E, K, n, w.dtype, w.capacity_factor,
                               flags=moe.MOE_FLAG_TOKEN_ROUNDING)
    ws_round = moe.workspace(desc, moe.MOE_WS_ROUND)

    def run_rounded(cold: bool):
        """K steps of moe_forward with tile-aware token rounding, and the
        metadata it produces (counts before and after the rounding)."""
        for i in range(args.warmup):
            moe.moe_forward(desc_round, dev["X"], dev["W_r"], dev["bias"], dev["W_gate"],
                            dev["W_up"], dev["W_down"], Y, ws_fwd)
        evs = [(ev(), ev()) for _ in range(args.steps)]
        torch.cuda.synchronize()
        for i in range(args.steps):
            if cold:
                flush(i)
            evs[i][0].record(stream)
            moe.moe_forward(desc_round, dev["X"], dev["W_r"], dev["bias"], dev["W_gate"],
                            dev["W_up"], dev["W_down"], Y, ws_fwd)
            evs[i][1].record(stream)
        moe.moe_route_ws(desc, dev["X"], dev["W_r"], dev["bias"], None, ids, gates, ws_r)
        moe.moe_permute(desc, ids, counts, offsets, None, perm, inv, ws_p)
        before = counts.clone()
        moe.moe_round_tokens(desc, ids, gates, counts, offsets, perm, inv, ws_round)
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in evs], before.cpu(), counts.clone().cpu()

    def run_omni(cold: bool):
        """The atomic-expert layer (omni_bf16: T=4096, d=1024, N=256x256,
        K=64): K cold steps of moe_omni_forward, plus its active experts."""
        oi = mi.make_omni_inputs("omni_bf16")
        ow = oi["workload"]
        od = {k: oi[k].cuda() for k in ("X", "W_r", "W_c", "W_in", "W_out")}
        odesc = moe.make_omni_desc(ow.T, ow.d, ow.Nr, ow.Nc, ow.K)
        ows = torch.empty(moe.moe_omni_workspace_size(odesc, moe.MOE_OMNI_WS_FORWARD),
                          dtype=torch.uint8, device="cuda")
        oY = torch.empty_like(od["X"])
        step = lambda: moe.moe_omni_forward(odesc, od["X"], od["W_r"], od["W_c"], od["W_in"],
                                            od["W_out"], oY, ows)
        for _ in range(args.warmup):
            step()
        evs = [(ev(), ev()) for _ in range(args.steps)]
        torch.cuda.synchronize()
        for i in range(args.steps):
            if cold:
                flush(i)
            evs[i][0].record(stream)
            step()
            evs[i][1].record(stream)
        oids, _, _, _ = moe.omni_route(od["X"], od["W_r"], od["W_c"], ow.K)
        ometa = moe.omni_permute(odesc, oids)
        torch.cuda.synchronize()
        act = int((ometa["counts"] > 0).sum().item())
        return ow, [a.elapsed_time(b) for a, b in evs], act

    cold = not args.warm
    # ---- timed region: K steps (moe_forward timed; step-wise diagnostics interleaved)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    fused_ms, stage_ms = run(cold)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    up_kernel_ms = run_up_kernel(cold)
    warm_fused_ms, warm_stage_ms = run(False)
    train_ms = run_train(cold) if train else None
    rounded = None if args.forward_only else run_rounded(cold)
    omni = None if args.forward_only else run_omni(cold)

    med = statistics.median(fused_ms)
    names = ["route_permute", "gemm_up", "gemm_down", "combine", "route", "permute"]
    stage_med = {nm: statistics.median(x[j] for x in stage_ms) for j, nm in enumerate(names)}
    warm_stage_med = {nm: statistics.median(x[j] for x in warm_stage_ms) for j, nm in enumerate(names)}

    # ---- algorithmic work (no padding, no pre-gather, active experts only)
    t_rp, t_up, t_down, t_comb, t_route, t_perm = (stage_med[k] * 1e-3 for k in names)
    route_bytes = T * d * s + d * E * s + T * K * 8
    perm_bytes = T * K * 4 + N * 4 + T * K * 4 + 2 * E * 4
    comb_bytes = N * d * s + T * K * 8 + T * d * s
    up_flops = 4.0 * N * d * n
    down_flops = 2.0 * N * n * d
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS
    t_up_mean = statistics.mean(up_kernel_ms) * 1e-3
    up_tflops = up_flops / t_up_mean / 1e12
    mfma_util = (up_flops + down_flops) / (t_up + t_down) / 1e12 / peak
    traffic = load_traffic(w.name) if w.dtype == "bf16" else None
    # Batches averaging at most 64 rows per expert run the weight-streaming
    # GEMMs (the library's own choice): HBM-bound on the active experts' weights.
    skinny = w.dtype == "bf16" and T * K <= 64 * E
    if skinny:
        up_bytes = active * 2 * d * n * s + N * d * s + N * n * s
        roofline = {"bound": "hbm", "achieved": up_bytes / t_up_mean / 1e9, "peak": PEAK_HBM_GBPS,
                    "unit": "GB/s", "frac": up_bytes / t_up_mean / 1e9 / PEAK_HBM_GBPS,
                    "traffic": traffic,
                    "kernel": "skinny_gemm_bf16<up> (weight-streaming, gather + SwiGLU)",
                    "per_unit": "2*d*n*s weight bytes per active expert (+ d*s in and n*s out "
                                "per kept row)",
                    "units_per_launch": active}
    else:
        roofline = {"bound": "mfma", "achieved": up_tflops, "peak": peak, "unit": "TFLOP/s",
                    "frac": up_tflops / peak, "traffic": traffic,
                    "kernel": "grouped_gemm_bf16<up> (gather + SwiGLU)",
                    "per_unit": "4*d*n flops per kept (token, expert) row",
                    "units_per_launch": N}
    roofline["timing"] = ("mean over K cold launches of the up GEMM alone (events on its "
                          "stream; tile table prebuilt)")
    roofline["launch_us"] = {"mean": statistics.mean(up_kernel_ms) * 1e3,
                             "median": statistics.median(up_kernel_ms) * 1e3}

    rec = {
        "metric": METRIC,
        "value": T / (med * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": med,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic: seeded torch.randn, weights N(0, 1/fan_in), see moe_inputs.py",
        "config": {"workload": w.name, "T": T, "d": d, "E": E, "K": K, "n": n,
                   "capacity_factor": w.capacity_factor, "kept_rows": N, "active_experts": active,
                   "G": d / n, "rho": K / E, "eta": N / max(1, active),
                   "cache": "cold (1 GiB rewritten before every timed step)" if cold else "warm"},
        "step_ms": {"median": med, "mean": statistics.mean(fused_ms), "p10": pct(fused_ms, 0.1),
                    "p90": pct(fused_ms, 0.9)},
        "warm": {"value": T / (statistics.median(warm_fused_ms) * 1e-3),
                 "ms_per_step": statistics.median(warm_fused_ms),
                 "stage_us": {k: v * 1e3 for k, v in warm_stage_med.items()}},
        "wall_s_timed_region": wall,
        "stage_us": {k: v * 1e3 for k, v in stage_med.items()},
        "stepwise_ms_per_step": sum(stage_med[k] for k in names[:4]),
        "grouped_gemm_mfma_util": mfma_util,
        "gemm_up_tflops": up_tflops,
        "gemm_down_tflops": down_flops / t_down / 1e12,
        "route_GBps": route_bytes / t_route / 1e9,
        "permute_GBps": perm_bytes / t_perm / 1e9,
        "route_permute_GBps": (route_bytes + perm_bytes) / t_rp / 1e9,
        "combine_GBps": comb_bytes / t_comb / 1e9,
        "hbm_frac": {"route": route_bytes / t_route / 1e9 / PEAK_HBM_GBPS,
                     "route_permute": (route_bytes + perm_bytes) / t_rp / 1e9 / PEAK_HBM_GBPS,
                     "combine": comb_bytes / t_comb / 1e9 / PEAK_HBM_GBPS},
        "roofline": roofline,
        "gemm_path": "weight-streaming" if skinny else "tiled",
        "input_sha256": hashes,
    }
    if train:
        f_ms, b_ms = statistics.median(train_ms[0]), statistics.median(train_ms[1])
        bwd_flops = 12.0 * N * d * n + 2.0 * T * d * E
        rec["training"] = {
            "what": "moe_forward_train then moe_backward (dX, dW_r, dW_gate, dW_up, dW_down); "
                    "cold cache before each step",
            "fwd_train_ms": f_ms,
            "bwd_ms": b_ms,
            "tokens_per_s": T / ((f_ms + b_ms) * 1e-3),
            "bwd_flops": bwd_flops,
            "bwd_tflops": bwd_flops / (b_ms * 1e-3) / 1e12,
            "bwd_mfma_frac": bwd_flops / (b_ms * 1e-3) / 1e12 / peak,
            "bwd_flops_per_unit": "12*d*n per kept row (dA', per-slot dX, dW_down, dW_gate, "
                                  "dW_up) + 2*d*E per token (dW_r)",
            "bwd_ms_p10_p90": [pct(train_ms[1], 0.1), pct(train_ms[1], 0.9)],
        }
    tiles = lambda c: int(((c + 255) // 256).sum())
    pad = lambda c: int(((c + 255) // 256 * 256 - c).sum())
    if rounded is not None:
        round_ms, round_before, round_after = rounded
        r_med = statistics.median(round_ms)
        rec["token_rounding"] = {
            "what": "moe_forward with MOE_FLAG_TOKEN_ROUNDING (an expert whose last 256-row tile "
                    "would be under half full drops its lowest-gate rows to whole tiles); cold",
            "ms_per_step": r_med,
            "tokens_per_s": T / (r_med * 1e-3),
            "speedup_vs_value": med / r_med,
            "kept_rows": [int(round_before.sum()), int(round_after.sum())],
            "dropped_frac": 1.0 - float(round_after.sum()) / max(1, int(round_before.sum())),
            "row_tiles": [tiles(round_before), tiles(round_after)],
            "padded_rows": [pad(round_before), pad(round_after)],
        }
    if omni is not None:
        ow, o_ms, act = omni
        o_med = statistics.median(o_ms)
        # algorithmic bytes: X and Y once, both router projections, and the two
        # vectors of every active expert once (the expert-centric order reads
        # them once for all their tokens)
        o_bytes = (2 * ow.T * ow.d * 2 + ow.d * (ow.Nr + ow.Nc) * 2 + act * 2 * ow.d * 2)
        rec["atomic_experts"] = {
            "what": "moe_omni_forward: Cartesian router, (expert, token) permutation, "
                    "expert-centric rank-1 experts, combine; cold",
            "workload": {"name": ow.name, "T": ow.T, "d": ow.d, "Nr": ow.Nr, "Nc": ow.Nc,
                         "K": ow.K, "active_experts": act, "eta": ow.T * ow.K / max(1, act)},
            "ms_per_step": o_med,
            "tokens_per_s": ow.T / (o_med * 1e-3),
            "algorithmic_GBps": o_bytes / (o_med * 1e-3) / 1e9,
            "hbm_frac": o_bytes / (o_med * 1e-3) / 1e9 / PEAK_HBM_GBPS,
        }
    if not args.no_cpu_baseline:
        sample = args.cpu_sample_tokens or min(T, 16384)
        rec["cpu_baseline"] = cpu_baseline(inp, w, sample)
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
