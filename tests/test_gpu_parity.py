"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Integer results (ids, counts, offsets, permutation) must match bit for bit,
with the oracle routing on the device's own fp32 logits; floating outputs
must meet the relative-L2 tolerance (1e-5 fp32, 2e-2 bf16) per expert
segment, per 256-row tile and per row for H and O, and as a whole and per
row for Y; gates within 2e-6.  Small shapes are chosen to span several tiles
with ragged tails (token tiles of 64 and 256, row tiles of 256, column tiles
of 128/256, partial last column tiles, more column tiles than one column
block); the full workloads run at their real sizes in the bench's launch
configuration and are compared the same way, row by row.
"""

import json
import os

import numpy as np
import pytest
import torch

import moe_inputs as mi
import top_routing_grouped_amd as moe
from oracle import moe_oracle as mo
from gpu_common import (GEMM_PATHS, TOL, check_outputs_streamed, check_permutation, check_routing,
                        device_inputs, f32np, intnp, run_stepwise)

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _full_check(inp, K, cf, dtype, gemm_flags=0):
    dev = device_inputs(inp)
    res = run_stepwise(dev, K, cf, gemm_flags)
    torch.cuda.synchronize()
    T, E = inp["X"].shape[0], inp["W_r"].shape[1]
    L_gpu, ids, gates = check_routing(res, inp, K)
    C = mo.capacity(T, K, E, cf)
    ref = check_permutation(res, ids, E, C)
    check_outputs_streamed(inp, ref, gates, res["H"], res["O"], res["Y"], TOL[dtype])
    # the fused entry point gives the same bits as the step-wise chain
    Y_fused = moe.forward(dev["X"], dev["W_r"], dev["W_gate"], dev["W_up"], dev["W_down"], K, cf,
                          bias=dev["bias"], flags=gemm_flags)
    torch.cuda.synchronize()
    assert torch.equal(Y_fused, res["Y"])
    return res, ref


SMALL = [
    # T,    d,   E,  K,   n,  dtype, cf,   bias
    (1000, 320, 4, 2, 192, "bf16", 0.0, None),       # partial last column tile in both GEMMs
    (777, 256, 16, 4, 256, "bf16", 1.0, "zipf"),     # capacity drops under a skewed router
    (513, 128, 3, 3, 128, "bf16", 0.0, None),        # K = E, E not a multiple of 8
    (130, 128, 256, 8, 128, "bf16", 0.0, None),      # E = 256
    (200, 192, 1, 1, 64, "bf16", 0.0, None),         # single expert
    (300, 128, 64, 6, 256, "bf16", 0.3, "zipf"),     # heavy drops, fully dropped tokens
    (70, 64, 40, 20, 64, "bf16", 0.0, None),         # K above 16
    (60, 64, 64, 64, 64, "bf16", 0.0, None),         # K = E = 64: every token in every expert
    (40, 64, 256, 256, 64, "bf16", 0.0, None),       # K = E = 256: the largest K and E
    (120, 64, 200, 130, 64, "bf16", 0.5, "zipf"),    # K above 128 under a capacity cap
    (1, 128, 8, 2, 128, "bf16", 0.0, None),          # one token
    (600, 1024, 4, 2, 1152, "bf16", 0.0, None),      # column blocks: up 9 tiles (8 + 1), down 4 (3 + 1)
    (256, 128, 8, 2, 256, "fp32", 0.0, None),        # the tiny fp32 layer's shape, other seed
    (100, 64, 5, 3, 64, "fp32", 0.5, "zipf"),
]


@pytest.mark.parametrize("T,d,E,K,n,dtype,cf,bias", SMALL)
def test_small_layer_parity(T, d, E, K, n, dtype, cf, bias):
    print(f"case T={T} d={d} E={E} K={K} n={n} {dtype} cf={cf} bias={bias}", flush=True)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    inp = mi.draw(T, d, E, n, tdt, seed=7, bias=bias)
    _full_check(inp, K, cf, dtype)


# Both grouped-GEMM kernels on every bf16 shape above, whichever the library
# would pick: the weight-streaming one (passes of 64 rows, 128-column blocks,
# partial last block in the down projection) and the 256x256-tiled one.
@pytest.mark.parametrize("path", ["tiled", "skinny"])
@pytest.mark.parametrize("T,d,E,K,n,dtype,cf,bias", [c for c in SMALL if c[5] == "bf16"])
def test_small_layer_parity_each_gemm_path(T, d, E, K, n, dtype, cf, bias, path):
    print(f"case T={T} d={d} E={E} K={K} n={n} {dtype} cf={cf} bias={bias} path={path}",
          flush=True)
    inp = mi.draw(T, d, E, n, torch.bfloat16, seed=11, bias=bias)
    _full_check(inp, K, cf, dtype, GEMM_PATHS[path])


@pytest.mark.parametrize("T,d,E,K", [(64, 4096, 256, 8), (100, 512, 64, 6), (700, 1024, 16, 2),
                                     (3, 256, 128, 8),
                                     (37, 512, 160, 7)])   # 16-token finishing blocks, ragged, padded E
def test_route_with_and_without_k_split(T, d, E, K):
    """moe_route_ws splits the k range over workgroups for small batches;
    moe_route never does.  Both: logits within tolerance of fp64, ids and
    gates exactly those of the device's own logits."""
    print(f"case route split T={T} d={d} E={E} K={K}", flush=True)
    inp = mi.draw(T, d, E, 64, torch.bfloat16, seed=3, bias="zipf")
    dev = device_inputs(inp)
    desc = moe.make_desc(T, d, E, K, 64, "bf16")
    assert moe.moe_workspace_size(desc, moe.MOE_WS_ROUTE) > 0      # these shapes split
    for split in (True, False):
        ids, gates, logits = moe.route(dev["X"], dev["W_r"], K, bias=dev["bias"], want_logits=True,
                                       split=split)
        torch.cuda.synchronize()
        check_routing({"ids": ids, "gates": gates, "logits": logits}, inp, K)


ROUTE_PERMUTE = [
    # T, d, E, K, dtype, cf, bias
    (3000, 512, 128, 6, "bf16", 0.0, None),      # split-k router: 16-token count blocks, 3 workgroups
    (1500, 256, 256, 8, "bf16", 1.0, "zipf"),    # E = 256, capacity drops, 2 workgroups
    (1024, 128, 8, 2, "bf16", 0.0, None),        # exactly one workgroup
    (1025, 128, 8, 2, "bf16", 0.0, None),        # a second workgroup with one token
    (5000, 256, 5, 3, "bf16", 0.5, "zipf"),      # E % 8 != 0 (register-staged router), drops
    (9000, 256, 64, 4, "bf16", 1.25, "zipf"),    # 64-token count blocks (no k split), 9 workgroups
    (200, 64, 40, 20, "bf16", 0.0, None),        # K above 16
    (2100, 128, 8, 2, "fp32", 0.7, None),        # fp32 router
]


@pytest.mark.parametrize("T,d,E,K,dtype,cf,bias", ROUTE_PERMUTE)
def test_route_permute_equals_route_then_permute(T, d, E, K, dtype, cf, bias):
    """moe_route_permute (router counting per block + one fused permutation
    launch) gives exactly the outputs of moe_route_ws then moe_permute, and
    the permutation is the oracle's on the device's logits."""
    print(f"route_permute T={T} d={d} E={E} K={K} {dtype} cf={cf} bias={bias}", flush=True)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    inp = mi.draw(T, d, E, 64, tdt, seed=41, bias=bias)
    dev = device_inputs(inp)
    desc = moe.make_desc(T, d, E, K, 64, dtype, cf)
    fused = moe.route_permute(dev["X"], dev["W_r"], K, desc, bias=dev["bias"], want_logits=True)
    ids, gates, logits = moe.route(dev["X"], dev["W_r"], K, bias=dev["bias"], want_logits=True, n=64)
    meta = moe.permute(desc, ids)
    torch.cuda.synchronize()
    assert torch.equal(fused["logits"], logits)
    assert torch.equal(fused["ids"], ids) and torch.equal(fused["gates"], gates)
    for key in ("counts", "offsets", "raw_counts", "inv_slot"):
        assert torch.equal(fused[key], meta[key]), key
    N = int(meta["offsets"][E].item())
    assert torch.equal(fused["perm_token"][:N], meta["perm_token"][:N])
    res = {"ids": ids, "gates": gates, "logits": logits}
    res.update(fused)
    _, ids_ref, _ = check_routing(res, inp, K)
    check_permutation(res, ids_ref, E, mo.capacity(T, K, E, cf))


def test_gemm_paths_agree_on_skewed_decode():
    """Decode-sized batch with one expert taking most rows (several 64-row
    passes in the weight-streaming kernel): both kernels against the oracle
    and against each other."""
    print("case decode skew T=160 d=256 E=64 K=2 n=192", flush=True)
    inp = mi.draw(160, 256, 64, 192, torch.bfloat16, seed=5, bias="zipf")
    res_t, ref = _full_check(inp, 2, 0.0, "bf16", GEMM_PATHS["tiled"])
    res_s, _ = _full_check(inp, 2, 0.0, "bf16", GEMM_PATHS["skinny"])
    assert int(np.max(ref["counts"])) > 128          # more than two passes for that expert
    N = int(ref["offsets"][-1])
    assert mo.rel_l2(f32np(res_s["O"])[:N], f32np(res_t["O"])[:N]) <= TOL["bf16"]


# Expert sizes set by hand around the bound up to which a tiled launch hands an
# expert to a weight-streaming block (64 rows): empty, 1, 2, 33, 63, 64 (all
# streamed), 65 (one partial tile), 256, 257, 300, 512 (one and more tiles).
STREAM_COUNTS = [64, 65, 0, 1, 63, 300, 256, 257, 33, 512, 2, 64]


@pytest.mark.parametrize("d,n", [(256, 320), (512, 192)])
def test_tiled_launch_streams_small_experts(d, n):
    """moe_grouped_ffn with default flags on hand-made metadata: every expert
    segment of H and O against the oracle; experts above 64 rows bit-equal to
    the tiles-only launch (MOE_FLAG_GEMM_TILED), experts of at most 64 rows
    bit-equal to the weight-streaming launch (MOE_FLAG_GEMM_SKINNY: the same
    per-element MFMA sums, on 4 instead of 8 waves)."""
    T, K, E = 700, 3, len(STREAM_COUNTS)
    print(f"case streamed experts T={T} d={d} E={E} K={K} n={n}", flush=True)
    inp = mi.draw(T, d, E, n, torch.bfloat16, seed=23)
    rng = np.random.default_rng(23)
    offsets = np.concatenate([[0], np.cumsum(STREAM_COUNTS)]).astype(np.int32)
    perm = np.concatenate([np.sort(rng.choice(T, size=c, replace=False)) for c in STREAM_COUNTS])
    assert offsets[-1] <= T * K and T * K > 64 * E      # tiled launch by default
    dev = device_inputs(inp)
    off_d = torch.from_numpy(offsets).cuda()
    perm_d = torch.from_numpy(perm.astype(np.int32)).cuda()
    outs = {}
    for path in ("auto", "tiled", "skinny"):
        desc = moe.make_desc(T, d, E, K, n, "bf16", 0.0, flags=GEMM_PATHS[path])
        outs[path] = moe.grouped_ffn(desc, dev["X"], off_d, perm_d, dev["W_gate"], dev["W_up"],
                                     dev["W_down"])
    torch.cuda.synchronize()
    X32 = f32np(inp["X"])
    Wg, Wu, Wd = (f32np(inp[k]) for k in ("W_gate", "W_up", "W_down"))
    H, O = (t.cpu() for t in outs["auto"])
    for e, c in enumerate(STREAM_COUNTS):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if c == 0:
            continue
        h, o = mo.expert_ffn(X32[perm[lo:hi]], Wg[e], Wu[e], Wd[e])
        for name, got, want in (("H", H[lo:hi], h), ("O", O[lo:hi], o)):
            rows = mo.rel_l2_rows(got.to(torch.float64).numpy(), want)
            assert rows.max() <= TOL["bf16"], f"{name} expert {e} ({c} rows): {rows.max():.3e}"
        other = "skinny" if c <= 64 else "tiled"
        for i, name in enumerate(("H", "O")):
            ref_rows = outs[other][i][lo:hi].cpu()
            got = (H, O)[i][lo:hi]
            assert torch.equal(got, ref_rows), f"{name} expert {e} ({c} rows) differs from {other}"


def test_zero_router_gives_lowest_ids_and_uniform_gates():
    inp = mi.draw(300, 128, 16, 128, torch.bfloat16, seed=1)
    inp["W_r"] = torch.zeros_like(inp["W_r"])
    res, _ = _full_check(inp, 5, 0.0, "bf16")
    assert np.all(intnp(res["ids"]) == np.arange(5)[None, :])
    assert np.all(f32np(res["gates"]) == np.float32(0.2))


def test_duplicated_router_columns_tie_to_lower_id():
    inp = mi.draw(400, 256, 12, 128, torch.bfloat16, seed=2)
    inp["W_r"][:, 9] = inp["W_r"][:, 2]
    res, _ = _full_check(inp, 12, 0.0, "bf16")
    L = f32np(res["logits"])
    assert np.array_equal(L[:, 2], L[:, 9])
    ids = intnp(res["ids"])
    pos2 = np.argmax(ids == 2, axis=1)
    pos9 = np.argmax(ids == 9, axis=1)
    assert np.all(pos2 + 1 == pos9)


def test_quantised_logits_with_many_exact_ties():
    g = torch.Generator().manual_seed(3)
    T, d, E, n = 600, 128, 32, 128
    inp = mi.draw(T, d, E, n, torch.bfloat16, seed=3)
    inp["X"] = torch.randint(-1, 2, (T, d), generator=g).to(torch.bfloat16)
    inp["W_r"] = (torch.randint(-1, 2, (d, E), generator=g).float() / 8).to(torch.bfloat16)
    res, _ = _full_check(inp, 4, 0.0, "bf16")
    L = f32np(res["logits"])
    ties = sum(len(np.unique(row)) < E for row in L)
    assert ties > T // 2


def _router_case(kind, T, d, E, seed, dtype=torch.bfloat16):
    """Router inputs with or without exact ties among the logits."""
    inp = mi.draw(T, d, E, 64, dtype, seed=seed, bias="zipf" if kind == "zipf" else None)
    g = torch.Generator().manual_seed(seed)
    if kind == "zero":
        inp["W_r"] = torch.zeros_like(inp["W_r"])
    elif kind == "dup":
        inp["W_r"][:, E - 1] = inp["W_r"][:, 0]
        inp["W_r"][:, E // 2] = inp["W_r"][:, 1]
    elif kind == "quant":
        inp["X"] = torch.randint(-1, 2, (T, d), generator=g).to(dtype)
        inp["W_r"] = (torch.randint(-1, 2, (d, E), generator=g).float() / 8).to(dtype)
    return inp


THRESHOLD_CASES = [
    # kind, T, d, E, K, dtype
    ("plain", 700, 512, 128, 8, "bf16"),
    ("zipf", 1000, 256, 256, 8, "bf16"),
    ("plain", 300, 128, 3, 3, "bf16"),       # K = E, E not a multiple of 8 (register-staged router)
    ("plain", 200, 64, 40, 20, "bf16"),      # K above 16
    ("plain", 130, 128, 64, 64, "bf16"),     # K = E = 64: every expert of every token
    ("zero", 300, 128, 16, 5, "bf16"),       # every logit tied
    ("dup", 400, 256, 12, 12, "bf16"),       # duplicated columns
    ("quant", 600, 128, 32, 4, "bf16"),      # many exact ties, ties cut at the threshold
    ("quant", 500, 128, 256, 8, "bf16"),
    ("plain", 64, 4096, 256, 8, "bf16"),     # decode size: k-split router + selection kernel
    ("plain", 256, 128, 8, 2, "fp32"),
    ("quant", 300, 64, 40, 7, "fp32"),
]


@pytest.mark.parametrize("kind,T,d,E,K,dtype", THRESHOLD_CASES)
def test_threshold_selection_matches_default(kind, T, d, E, K, dtype):
    """MOE_FLAG_TOPK_THRESHOLD: ids, their order and gates bit-equal to the
    default selection's (both router paths), and ids equal to the oracle's
    on the device's logits."""
    print(f"case threshold {kind} T={T} d={d} E={E} K={K} {dtype}", flush=True)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    inp = _router_case(kind, T, d, E, seed=31, dtype=tdt)
    dev = device_inputs(inp)
    for split in (True, False):
        base = moe.route(dev["X"], dev["W_r"], K, bias=dev["bias"], want_logits=True, split=split)
        thr = moe.route(dev["X"], dev["W_r"], K, bias=dev["bias"], want_logits=True, split=split,
                        flags=moe.MOE_FLAG_TOPK_THRESHOLD)
        torch.cuda.synchronize()
        assert torch.equal(thr[2], base[2]), "logits differ"
        assert torch.equal(thr[0], base[0]), f"ids differ (split={split})"
        assert torch.equal(thr[1], base[1]), f"gates differ (split={split})"
        check_routing({"ids": thr[0], "gates": thr[1], "logits": thr[2]}, inp, K)


@pytest.mark.parametrize("kind,T,d,E,K,cf", [("zipf", 3000, 512, 128, 6, 1.0), ("quant", 2000, 128, 64, 4, 0.0),
                                             ("plain", 200, 64, 40, 20, 0.0)])
def test_threshold_selection_in_fused_paths(kind, T, d, E, K, cf):
    """moe_route_permute and moe_forward with MOE_FLAG_TOPK_THRESHOLD give
    exactly the default flags' outputs."""
    print(f"case threshold fused {kind} T={T} d={d} E={E} K={K} cf={cf}", flush=True)
    inp = _router_case(kind, T, d, E, seed=37)
    n = 128
    inp.update({k: v for k, v in mi.draw(T, d, E, n, torch.bfloat16, seed=38).items()
                if k in ("W_gate", "W_up", "W_down")})
    dev = device_inputs(inp)
    outs = []
    for flags in (0, moe.MOE_FLAG_TOPK_THRESHOLD):
        desc = moe.make_desc(T, d, E, K, n, "bf16", cf, flags=flags)
        rp = moe.route_permute(dev["X"], dev["W_r"], K, desc, bias=dev["bias"], want_logits=True)
        Y = moe.forward(dev["X"], dev["W_r"], dev["W_gate"], dev["W_up"], dev["W_down"], K, cf,
                        bias=dev["bias"], flags=flags)
        outs.append((rp, Y))
    torch.cuda.synchronize()
    (rp0, Y0), (rp1, Y1) = outs
    N = int(rp0["offsets"][E].item())
    for key in ("ids", "gates", "logits", "counts", "offsets", "raw_counts", "inv_slot"):
        assert torch.equal(rp1[key], rp0[key]), key
    assert torch.equal(rp1["perm_token"][:N], rp0["perm_token"][:N])
    assert torch.equal(Y1, Y0)


def test_capacity_one_keeps_each_experts_first_token():
    inp = mi.draw(257, 128, 8, 128, torch.bfloat16, seed=4)
    cf = 1e-6                                    # C = 1
    assert mo.capacity(257, 2, 8, cf) == 1
    _, ref = _full_check(inp, 2, cf, "bf16")
    assert np.all(ref["counts"] <= 1)


@pytest.mark.parametrize("case,cf", [("uncapped", 0.0), ("capped", 1.0)])
def test_worked_example_on_device(case, cf):
    with open(os.path.join(GOLDEN, "worked_example_permute.json")) as f:
        ex = json.load(f)
    want = ex[case]
    desc = moe.make_desc(3, 64, ex["E"], 3, 64, "bf16", cf)
    assert moe.moe_capacity(desc) == want["C"]
    ids = torch.tensor(ex["ids"], dtype=torch.int32, device="cuda")
    got = moe.permute(desc, ids)
    torch.cuda.synchronize()
    for key in ("raw_counts", "counts", "offsets", "inv_slot"):
        assert intnp(got[key]).tolist() == want[key], key
    N = want["offsets"][-1]
    assert intnp(got["perm_token"])[:N].tolist() == want["perm_token"]


def test_repeat_runs_are_bitwise_identical():
    inp = mi.draw(2000, 256, 32, 256, torch.bfloat16, seed=5)
    dev = device_inputs(inp)
    ys = [moe.forward(dev["X"], dev["W_r"], dev["W_gate"], dev["W_up"], dev["W_down"], 4, 1.0)
          for _ in range(3)]
    torch.cuda.synchronize()
    assert torch.equal(ys[0], ys[1]) and torch.equal(ys[0], ys[2])


def test_zero_tokens_is_a_no_op():
    X = torch.empty((0, 128), dtype=torch.bfloat16, device="cuda")
    W_r = torch.zeros((128, 8), dtype=torch.bfloat16, device="cuda")
    Wg = torch.zeros((8, 128, 128), dtype=torch.bfloat16, device="cuda")
    Y = moe.forward(X, W_r, Wg, Wg, Wg.transpose(1, 2).contiguous(), 2)
    torch.cuda.synchronize()
    assert Y.shape == (0, 128)


def _bench_chain(inp, K, cf):
    """The entry-point sequence bench.py times: route and permute with their
    workspaces, the up GEMM building the tile table, the down GEMM and a
    second up GEMM on that table (MOE_FLAG_TILE_TABLE_READY), the combine,
    and moe_forward on the same inputs."""
    dev = device_inputs(inp)
    X = dev["X"]
    T, d = X.shape
    E, _, n = dev["W_gate"].shape
    dtype = "bf16" if X.dtype == torch.bfloat16 else "fp32"
    desc = moe.make_desc(T, d, E, K, n, dtype, cf)
    ready = moe.make_desc(T, d, E, K, n, dtype, cf, flags=moe.MOE_FLAG_TILE_TABLE_READY)
    rows = moe.moe_max_rows(desc)
    i32 = dict(dtype=torch.int32, device="cuda")
    ids, inv = torch.empty((T, K), **i32), torch.empty((T, K), **i32)
    gates = torch.empty((T, K), dtype=torch.float32, device="cuda")
    counts, offsets, perm = torch.empty(E, **i32), torch.empty(E + 1, **i32), torch.empty(T * K, **i32)
    H = [torch.empty((rows, n), dtype=X.dtype, device="cuda") for _ in range(2)]
    O = [torch.empty((rows, d), dtype=X.dtype, device="cuda") for _ in range(2)]
    Y = [torch.empty((T, d), dtype=X.dtype, device="cuda") for _ in range(2)]
    ws_f = moe.workspace(desc, moe.MOE_WS_GROUPED_FFN)
    moe.moe_route_ws(desc, X, dev["W_r"], dev["bias"], None, ids, gates, moe.workspace(desc, moe.MOE_WS_ROUTE))
    moe.moe_permute(desc, ids, counts, offsets, None, perm, inv, moe.workspace(desc, moe.MOE_WS_PERMUTE))
    moe.moe_grouped_gemm_up(desc, X, offsets, perm, dev["W_gate"], dev["W_up"], H[0], ws_f)
    moe.moe_grouped_gemm_down(ready, H[0], offsets, dev["W_down"], O[0], ws_f)
    moe.moe_grouped_gemm_up(ready, X, offsets, perm, dev["W_gate"], dev["W_up"], H[1], ws_f)
    moe.moe_grouped_gemm_down(desc, H[1], offsets, dev["W_down"], O[1], moe.workspace(desc, moe.MOE_WS_GROUPED_FFN))
    moe.moe_combine(desc, O[0], gates, inv, Y[0])
    moe.moe_forward(desc, X, dev["W_r"], dev["bias"], dev["W_gate"], dev["W_up"], dev["W_down"], Y[1],
                    moe.workspace(desc, moe.MOE_WS_FORWARD))
    torch.cuda.synchronize()
    N = int(offsets[E].item())
    return N, H, O, Y


@pytest.mark.parametrize("case", ["small", "qwen3_bf16"])
def test_prebuilt_tile_table_as_timed(case):
    """GEMMs launched on a tile table built by an earlier call (the bench's
    configuration) give the bits of a freshly built table, and the chain the
    bench times gives the bits of moe_forward."""
    if case == "small":
        inp, K, cf = mi.draw(3001, 256, 16, 384, torch.bfloat16, seed=11), 4, 0.0
    else:
        inp = mi.make_inputs(case)
        w = inp["workload"]
        K, cf = w.K, w.capacity_factor
    print(f"prebuilt tile table: {case}", flush=True)
    N, H, O, Y = _bench_chain(inp, K, cf)
    assert N > 0
    assert torch.equal(H[0][:N], H[1][:N])
    assert torch.equal(O[0][:N], O[1][:N])
    assert torch.equal(Y[0], Y[1])


# ---------------------------------------------------------------- full workloads

def _full_size_check(name):
    """A named workload at full size, in the launch configuration the bench
    times: routing and the permutation bit-exact; every kept row of H and O
    and every row of Y against the oracle (per expert segment, per row tile
    and per row); the fused forward equal to the step-wise chain."""
    inp = mi.make_inputs(name)
    w = inp["workload"]
    print(f"workload {name}: T={w.T} d={w.d} E={w.E} K={w.K} n={w.n}", flush=True)
    dev = device_inputs(inp)
    res = run_stepwise(dev, w.K, w.capacity_factor)
    Y_fused = moe.forward(dev["X"], dev["W_r"], dev["W_gate"], dev["W_up"], dev["W_down"], w.K,
                          w.capacity_factor, bias=dev["bias"])
    torch.cuda.synchronize()
    assert torch.equal(Y_fused, res["Y"])
    L_gpu, ids, gates = check_routing(res, inp, w.K)
    C = mo.capacity(w.T, w.K, w.E, w.capacity_factor)
    ref = check_permutation(res, ids, w.E, C)
    fused = moe.route_permute(dev["X"], dev["W_r"], w.K, res["desc"], bias=dev["bias"])
    torch.cuda.synchronize()
    for key in ("ids", "gates", "counts", "offsets", "raw_counts", "inv_slot"):
        assert torch.equal(fused[key], res[key]), key
    N = int(ref["offsets"][-1])
    assert torch.equal(fused["perm_token"][:N], res["perm_token"][:N])
    worst = check_outputs_streamed(inp, ref, gates, res["H"], res["O"], res["Y"], TOL[w.dtype],
                                   label=name)
    print(f"workload {name}: {worst}", flush=True)
    return res, ref


@pytest.mark.parametrize("name", ["tiny_fp32", "qwen3_bf16", "skewed_cap_bf16", "mixtral_bf16",
                                  "granular_bf16", "granular_decode_bf16"])
def test_workload_full_size(name):
    res, ref = _full_size_check(name)
    if name == "skewed_cap_bf16":
        assert int(ref["offsets"][-1]) < 8192 * 4          # the cap drops assignments
        assert int(np.max(ref["counts"])) == 640
