"""Guard bands around every buffer a call writes (GPU, through the C ABI).

Each output, intermediate and workspace is carved from a larger allocation
whose margins (GUARD bytes before and after) and whose own bytes start as a
sentinel pattern.  After the calls:

* the margins still hold the sentinel (no write before or past a buffer);
* defined outputs hold no sentinel element (every element was written);
* rows a kernel must not touch still hold it: H and O rows at or beyond the
  kept-row count offsets[E] (the grouped GEMMs write kept rows only) and
  perm_token entries at or beyond offsets[E].

The values themselves are checked against the oracle elsewhere; this file
checks the extents of the writes, for the step-wise chain, the fused forward,
token rounding, the training forward and backward, and the atomic-expert
layer."""

import numpy as np
import pytest
import torch

import moe_inputs as mi
import top_routing_grouped_amd as moe
from gpu_common import device_inputs

pytestmark = pytest.mark.gpu

GUARD = 4096                    # bytes on each side (keeps the buffer 256-byte aligned)
SENT = 0xA5                     # sentinel byte


class Guarded:
    """A device buffer of ``shape``/``dtype`` inside a sentinel-filled allocation."""

    def __init__(self, shape, dtype, name):
        self.name = name
        item = torch.empty((), dtype=dtype).element_size()
        count = int(np.prod(shape)) if len(shape) else 1
        self.nbytes = count * item
        self.raw = torch.full((GUARD + self.nbytes + GUARD,), SENT, dtype=torch.uint8,
                              device="cuda")
        self.t = self.raw[GUARD:GUARD + self.nbytes].view(dtype).view(shape)
        assert self.t.data_ptr() % 256 == 0

    def margins_intact(self):
        lo = self.raw[:GUARD]
        hi = self.raw[GUARD + self.nbytes:]
        assert bool(torch.all(lo == SENT)), f"{self.name}: write before the buffer"
        assert bool(torch.all(hi == SENT)), f"{self.name}: write past the end of the buffer"

    def all_written(self, part=None):
        part = self.t if part is None else part
        flat = part.reshape(-1, 1) if part.dim() <= 1 else part.reshape(part.shape[0], -1)
        item = flat.element_size()
        # element by element: an element whose every byte is the sentinel was not written
        b = flat.contiguous().view(torch.uint8).view(-1, item)
        untouched = torch.all(b == SENT, dim=1)
        assert not bool(torch.any(untouched)), f"{self.name}: {int(untouched.sum())} elements not written"

    def untouched(self, part):
        if part.numel() == 0:
            return
        b = part.contiguous().view(torch.uint8)
        assert bool(torch.all(b == SENT)), f"{self.name}: bytes written that must stay untouched"


def _ws(desc, entry, name):
    return Guarded((max(16, moe.moe_workspace_size(desc, entry)),), torch.uint8, name)


CHAIN = [
    # T, d, E, K, n, dtype, cf, bias, gemm flags
    (777, 256, 16, 4, 256, "bf16", 1.0, "zipf", moe.MOE_FLAG_GEMM_TILED),
    (777, 256, 16, 4, 256, "bf16", 1.0, "zipf", moe.MOE_FLAG_GEMM_SKINNY),
    (600, 1024, 4, 2, 1152, "bf16", 0.0, None, 0),
    (64, 512, 64, 6, 128, "bf16", 0.0, None, 0),          # split-k router, one permute block
    (100, 64, 5, 3, 64, "fp32", 0.5, "zipf", 0),
    (300, 128, 64, 6, 256, "bf16", 0.3, "zipf", 0),        # fully dropped tokens
]


@pytest.mark.parametrize("T,d,E,K,n,dtype,cf,bias,flags", CHAIN)
def test_stepwise_chain_and_forward_write_only_their_buffers(T, d, E, K, n, dtype, cf, bias, flags):
    print(f"guards T={T} d={d} E={E} K={K} n={n} {dtype} cf={cf} flags={flags}", flush=True)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    inp = mi.draw(T, d, E, n, tdt, seed=19, bias=bias)
    dev = device_inputs(inp)
    desc = moe.make_desc(T, d, E, K, n, dtype, cf, flags=flags)
    plain = moe.make_desc(T, d, E, K, n, dtype, cf)
    rows = moe.moe_max_rows(desc)
    g = {
        "ids": Guarded((T, K), torch.int32, "ids"),
        "gates": Guarded((T, K), torch.float32, "gates"),
        "logits": Guarded((T, E), torch.float32, "logits"),
        "ws_route": _ws(plain, moe.MOE_WS_ROUTE, "route workspace"),
        "counts": Guarded((E,), torch.int32, "counts"),
        "offsets": Guarded((E + 1,), torch.int32, "offsets"),
        "raw": Guarded((E,), torch.int32, "raw_counts"),
        "perm": Guarded((T * K,), torch.int32, "perm_token"),
        "inv": Guarded((T, K), torch.int32, "inv_slot"),
        "ws_perm": _ws(plain, moe.MOE_WS_PERMUTE, "permute workspace"),
        "H": Guarded((rows, n), tdt, "H"),
        "O": Guarded((rows, d), tdt, "O"),
        "ws_ffn": _ws(desc, moe.MOE_WS_GROUPED_FFN, "grouped-FFN workspace"),
        "Y": Guarded((T, d), tdt, "Y"),
        "Yf": Guarded((T, d), tdt, "Y (fused)"),
        "ws_fwd": _ws(desc, moe.MOE_WS_FORWARD, "forward workspace"),
    }
    t = {k: v.t for k, v in g.items()}
    moe.moe_route_ws(plain, dev["X"], dev["W_r"], dev["bias"], t["logits"], t["ids"], t["gates"],
                     t["ws_route"])
    moe.moe_permute(plain, t["ids"], t["counts"], t["offsets"], t["raw"], t["perm"], t["inv"],
                    t["ws_perm"])
    moe.moe_grouped_gemm_up(desc, dev["X"], t["offsets"], t["perm"], dev["W_gate"], dev["W_up"],
                            t["H"], t["ws_ffn"])
    moe.moe_grouped_gemm_down(desc, t["H"], t["offsets"], dev["W_down"], t["O"], t["ws_ffn"])
    moe.moe_combine(plain, t["O"], t["gates"], t["inv"], t["Y"])
    moe.moe_forward(desc, dev["X"], dev["W_r"], dev["bias"], dev["W_gate"], dev["W_up"],
                    dev["W_down"], t["Yf"], t["ws_fwd"])
    torch.cuda.synchronize()
    for v in g.values():
        v.margins_intact()
    N = int(t["offsets"][E].item())
    for k in ("ids", "gates", "logits", "counts", "offsets", "raw", "inv", "Y", "Yf"):
        g[k].all_written()
    g["perm"].all_written(t["perm"][:N])
    g["perm"].untouched(t["perm"][N:])
    g["H"].all_written(t["H"][:N])
    g["H"].untouched(t["H"][N:])
    g["O"].all_written(t["O"][:N])
    g["O"].untouched(t["O"][N:])
    assert torch.equal(t["Y"], t["Yf"])


def test_qwen3_shaped_forward_writes_only_its_buffers():
    inp = mi.make_inputs("qwen3_bf16")
    w = inp["workload"]
    print("guards qwen3_bf16 full size", flush=True)
    dev = device_inputs(inp)
    desc = moe.make_desc(w.T, w.d, w.E, w.K, w.n, "bf16", w.capacity_factor)
    rows = moe.moe_max_rows(desc)
    g = {
        "ids": Guarded((w.T, w.K), torch.int32, "ids"),
        "gates": Guarded((w.T, w.K), torch.float32, "gates"),
        "counts": Guarded((w.E,), torch.int32, "counts"),
        "offsets": Guarded((w.E + 1,), torch.int32, "offsets"),
        "perm": Guarded((w.T * w.K,), torch.int32, "perm_token"),
        "inv": Guarded((w.T, w.K), torch.int32, "inv_slot"),
        "ws_perm": _ws(desc, moe.MOE_WS_PERMUTE, "permute workspace"),
        "H": Guarded((rows, w.n), torch.bfloat16, "H"),
        "O": Guarded((rows, w.d), torch.bfloat16, "O"),
        "ws_ffn": _ws(desc, moe.MOE_WS_GROUPED_FFN, "grouped-FFN workspace"),
        "Y": Guarded((w.T, w.d), torch.bfloat16, "Y"),
        "ws_fwd": _ws(desc, moe.MOE_WS_FORWARD, "forward workspace"),
        "Yf": Guarded((w.T, w.d), torch.bfloat16, "Y (fused)"),
    }
    t = {k: v.t for k, v in g.items()}
    moe.moe_route(desc, dev["X"], dev["W_r"], None, None, t["ids"], t["gates"])
    moe.moe_permute(desc, t["ids"], t["counts"], t["offsets"], None, t["perm"], t["inv"], t["ws_perm"])
    moe.moe_grouped_ffn(desc, dev["X"], t["offsets"], t["perm"], dev["W_gate"], dev["W_up"],
                        dev["W_down"], t["H"], t["O"], t["ws_ffn"])
    moe.moe_combine(desc, t["O"], t["gates"], t["inv"], t["Y"])
    moe.moe_forward(desc, dev["X"], dev["W_r"], None, dev["W_gate"], dev["W_up"], dev["W_down"],
                    t["Yf"], t["ws_fwd"])
    torch.cuda.synchronize()
    for v in g.values():
        v.margins_intact()
    N = int(t["offsets"][w.E].item())
    assert N == w.T * w.K
    for k in ("ids", "gates", "counts", "offsets", "inv", "perm", "H", "O", "Y", "Yf"):
        g[k].all_written(t[k][:N] if k in ("perm", "H", "O") else None)
    assert torch.equal(t["Y"], t["Yf"])


def test_token_rounding_writes_only_its_buffers():
    T, d, E, K, n = 2100, 128, 8, 2, 128       # about 525 rows per expert: most round down to 512
    inp = mi.draw(T, d, E, n, torch.bfloat16, seed=23)
    dev = device_inputs(inp)
    desc = moe.make_desc(T, d, E, K, n, "bf16")
    ids, gates, _ = moe.route(dev["X"], dev["W_r"], K, n=n)
    g = {
        "counts": Guarded((E,), torch.int32, "counts"),
        "offsets": Guarded((E + 1,), torch.int32, "offsets"),
        "perm": Guarded((T * K,), torch.int32, "perm_token"),
        "inv": Guarded((T, K), torch.int32, "inv_slot"),
        "ws_perm": _ws(desc, moe.MOE_WS_PERMUTE, "permute workspace"),
        "ws_round": _ws(desc, moe.MOE_WS_ROUND, "rounding workspace"),
    }
    t = {k: v.t for k, v in g.items()}
    moe.moe_permute(desc, ids, t["counts"], t["offsets"], None, t["perm"], t["inv"], t["ws_perm"])
    torch.cuda.synchronize()
    N0 = int(t["offsets"][E].item())
    moe.moe_round_tokens(desc, ids, gates, t["counts"], t["offsets"], t["perm"], t["inv"],
                         t["ws_round"])
    torch.cuda.synchronize()
    for v in g.values():
        v.margins_intact()
    N = int(t["offsets"][E].item())
    assert N < N0                            # this shape does drop rows to whole tiles
    g["perm"].all_written(t["perm"][:N])
    g["perm"].untouched(t["perm"][N0:])


def test_training_step_writes_only_its_buffers():
    T, d, E, K, n = 517, 256, 8, 3, 320
    inp = mi.draw(T, d, E, n, torch.bfloat16, seed=29, bias="zipf")
    dev = device_inputs(inp)
    dY = mi.draw_grad_output(T, d, torch.bfloat16, seed=29).cuda()
    desc = moe.make_desc(T, d, E, K, n, "bf16", 0.6)
    g = {
        "Y": Guarded((T, d), torch.bfloat16, "Y"),
        "saved": _ws(desc, moe.MOE_WS_SAVED, "saved state"),
        "ws_fwd": _ws(desc, moe.MOE_WS_FORWARD, "forward workspace"),
        "ws_bwd": _ws(desc, moe.MOE_WS_BACKWARD, "backward workspace"),
        "dX": Guarded((T, d), torch.bfloat16, "dX"),
        "dW_r": Guarded((d, E), torch.float32, "dW_r"),
        "dW_gate": Guarded((E, d, n), torch.float32, "dW_gate"),
        "dW_up": Guarded((E, d, n), torch.float32, "dW_up"),
        "dW_down": Guarded((E, n, d), torch.float32, "dW_down"),
    }
    t = {k: v.t for k, v in g.items()}
    moe.moe_forward_train(desc, dev["X"], dev["W_r"], dev["bias"], dev["W_gate"], dev["W_up"],
                          dev["W_down"], t["Y"], t["saved"], t["ws_fwd"])
    moe.moe_backward(desc, dev["X"], dev["W_r"], dev["W_gate"], dev["W_up"], dev["W_down"], dY,
                     t["saved"], t["dX"], t["dW_r"], t["dW_gate"], t["dW_up"], t["dW_down"],
                     t["ws_bwd"])
    torch.cuda.synchronize()
    for v in g.values():
        v.margins_intact()
    for k in ("Y", "dX", "dW_r", "dW_gate", "dW_up", "dW_down"):
        g[k].all_written()


def test_atomic_expert_layer_writes_only_its_buffers():
    w = mi.OMNI_WORKLOADS["omni_small_bf16"]
    inp = mi.make_omni_inputs(w.name)
    dev = {k: v.cuda() for k, v in inp.items() if k != "workload"}
    desc = moe.make_omni_desc(w.T, w.d, w.Nr, w.Nc, w.K)
    N = w.Nr * w.Nc
    g = {
        "ids": Guarded((w.T, w.K), torch.int32, "ids"),
        "gates": Guarded((w.T, w.K), torch.float32, "gates"),
        "ls_r": Guarded((w.T, w.Nr), torch.float32, "ls_r"),
        "ls_c": Guarded((w.T, w.Nc), torch.float32, "ls_c"),
        "ws_route": Guarded((max(16, moe.moe_omni_workspace_size(desc, moe.MOE_OMNI_WS_ROUTE)),),
                            torch.uint8, "route workspace"),
        "counts": Guarded((N,), torch.int32, "counts"),
        "offsets": Guarded((N + 1,), torch.int32, "offsets"),
        "perm": Guarded((w.T * w.K,), torch.int32, "perm_token"),
        "inv": Guarded((w.T, w.K), torch.int32, "inv_slot"),
        "ws_perm": Guarded((max(16, moe.moe_omni_workspace_size(desc, moe.MOE_OMNI_WS_PERMUTE)),),
                           torch.uint8, "permute workspace"),
        "Y": Guarded((w.T, w.d), torch.bfloat16, "Y"),
        "ws_fwd": Guarded((max(16, moe.moe_omni_workspace_size(desc, moe.MOE_OMNI_WS_FORWARD)),),
                          torch.uint8, "forward workspace"),
    }
    t = {k: v.t for k, v in g.items()}
    moe.moe_omni_route(desc, dev["X"], dev["W_r"], dev["W_c"], t["ls_r"], t["ls_c"], t["ids"],
                       t["gates"], t["ws_route"])
    moe.moe_omni_permute(desc, t["ids"], t["counts"], t["offsets"], t["perm"], t["inv"], t["ws_perm"])
    moe.moe_omni_forward(desc, dev["X"], dev["W_r"], dev["W_c"], dev["W_in"], dev["W_out"], t["Y"],
                         t["ws_fwd"])
    torch.cuda.synchronize()
    for v in g.values():
        v.margins_intact()
    for k in ("ids", "gates", "ls_r", "ls_c", "counts", "offsets", "perm", "inv", "Y"):
        g[k].all_written()
