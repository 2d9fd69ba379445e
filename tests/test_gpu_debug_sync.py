"""MOE_DEBUG_SYNC=1: every launch step synchronises the entry point's stream
and reports a failed kernel as MOE_ERR_HIP naming the step.  The mode only
adds synchronisation, so every output must be bit-equal to a run without it,
and a stream under graph capture is left unsynchronised, so capture still
works with the variable set."""

import pytest
import torch

import moe_inputs as mi
import top_routing_grouped_amd as moe

pytestmark = pytest.mark.gpu


def _layer_outputs(dev, K, cf):
    Y = moe.forward(dev["X"], dev["W_r"], dev["W_gate"], dev["W_up"], dev["W_down"], K, cf,
                    bias=dev["bias"])
    Yt, saved, desc = moe.forward_train(dev["X"], dev["W_r"], dev["W_gate"], dev["W_up"],
                                        dev["W_down"], K, cf, bias=dev["bias"])
    dY = torch.randn(Y.shape, generator=torch.Generator().manual_seed(3)).to(Y.dtype).cuda()
    grads = moe.backward(desc, saved, dev["X"], dev["W_r"], dev["W_gate"], dev["W_up"],
                         dev["W_down"], dY)
    torch.cuda.synchronize()
    return {"Y": Y, "Y_train": Yt, **grads}


def test_debug_sync_gives_the_same_bits(monkeypatch):
    T, d, E, K, n, cf = 600, 256, 16, 4, 192, 1.0
    print(f"case debug sync T={T} d={d} E={E} K={K} n={n} cf={cf}", flush=True)
    inp = mi.draw(T, d, E, n, torch.bfloat16, seed=61, bias="zipf")
    dev = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
    oinp = mi.draw_omni(200, 128, 16, 16, 8, seed=62)
    odev = {k: oinp[k].cuda() for k in ("X", "W_r", "W_c", "W_in", "W_out")}
    runs = []
    for value in (None, "1"):
        if value is None:
            monkeypatch.delenv("MOE_DEBUG_SYNC", raising=False)
        else:
            monkeypatch.setenv("MOE_DEBUG_SYNC", value)
        out = _layer_outputs(dev, K, cf)
        out["Y_omni"] = moe.omni_forward(odev["X"], odev["W_r"], odev["W_c"], odev["W_in"],
                                         odev["W_out"], 8)
        torch.cuda.synchronize()
        runs.append(out)
    for name in runs[0]:
        assert torch.equal(runs[0][name], runs[1][name]), name


def test_debug_sync_leaves_graph_capture_working(monkeypatch):
    T, d, E, K, n = 128, 512, 32, 4, 256
    print(f"case debug sync graph T={T} d={d} E={E} K={K} n={n}", flush=True)
    monkeypatch.setenv("MOE_DEBUG_SYNC", "1")
    inp = mi.draw(T, d, E, n, torch.bfloat16, seed=63)
    dev = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
    desc = moe.make_desc(T, d, E, K, n, "bf16", 0.0)
    ws = moe.workspace(desc, moe.MOE_WS_FORWARD)
    Y = torch.empty_like(dev["X"])
    args = (desc, dev["X"], dev["W_r"], dev["bias"], dev["W_gate"], dev["W_up"], dev["W_down"],
            Y, ws)
    moe.moe_forward(*args)
    torch.cuda.synchronize()
    want = Y.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        moe.moe_forward(*args)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.moe_forward(*args)
    for i in range(3):
        Y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(Y, want), f"replay {i}"
