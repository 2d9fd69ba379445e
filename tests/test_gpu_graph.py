"""The fused entry points under HIP graph capture.

A serving loop records one step into a graph and replays it; the library
launches only kernels on the caller's stream (no memsets, no allocations
inside the call), so `moe_forward` and `moe_omni_forward` can be captured.
Each graph is replayed several times, with eager calls of the same entry
point and other device work in between, and every replay must give the
eager result bit for bit.
"""

import pytest
import torch

import moe_inputs as mi
import top_routing_grouped_amd as moe

pytestmark = pytest.mark.gpu

GRAPH_CASES = [
    # T, d, E, K, n, cf, bias
    (64, 1024, 64, 8, 256, 0.0, None),        # decode-sized: split-k router, weight-streaming GEMMs
    (700, 512, 32, 4, 320, 1.0, "zipf"),      # tiled GEMMs with streamed small experts, capacity drops
]


@pytest.mark.parametrize("T,d,E,K,n,cf,bias", GRAPH_CASES)
def test_forward_replays_from_a_graph(T, d, E, K, n, cf, bias):
    print(f"case graph forward T={T} d={d} E={E} K={K} n={n} cf={cf} bias={bias}", flush=True)
    inp = mi.draw(T, d, E, n, torch.bfloat16, seed=51, bias=bias)
    dev = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
    desc = moe.make_desc(T, d, E, K, n, "bf16", cf)
    ws = moe.workspace(desc, moe.MOE_WS_FORWARD)
    X = dev["X"].clone()
    Y = torch.empty_like(X)
    args = (desc, X, dev["W_r"], dev["bias"], dev["W_gate"], dev["W_up"], dev["W_down"], Y, ws)
    moe.moe_forward(*args)
    torch.cuda.synchronize()
    want = Y.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                  # warm the stream before capture
        moe.moe_forward(*args)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.moe_forward(*args)
    for i in range(4):
        Y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(Y, want), f"replay {i}"
        # eager work in between: the same call on other inputs, then restore
        X2 = torch.randn_like(X)
        Y2 = moe.forward(X2, dev["W_r"], dev["W_gate"], dev["W_up"], dev["W_down"], K, cf,
                         bias=dev["bias"])
        torch.cuda.synchronize()
        assert torch.isfinite(Y2.float()).all()


def test_atomic_expert_forward_replays_from_a_graph():
    T, d, Nr, Nc, K = 300, 128, 16, 16, 8
    print(f"case graph omni T={T} d={d} Nr={Nr} Nc={Nc} K={K}", flush=True)
    inp = mi.draw_omni(T, d, Nr, Nc, K, seed=53)
    dev = {k: v.cuda() for k, v in inp.items()}
    desc = moe.make_omni_desc(T, d, Nr, Nc, K)
    ws = moe._omni_ws(desc, moe.MOE_OMNI_WS_FORWARD, dev["X"].device)
    Y = torch.empty_like(dev["X"])
    args = (desc, dev["X"], dev["W_r"], dev["W_c"], dev["W_in"], dev["W_out"], Y, ws)
    moe.moe_omni_forward(*args)
    torch.cuda.synchronize()
    want = Y.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.moe_omni_forward(*args)
    for i in range(4):
        Y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(Y, want), f"replay {i}"
        moe.moe_omni_forward(*args)            # eager call between replays
        torch.cuda.synchronize()
        assert torch.equal(Y, want)


def test_explicit_stream_argument():
    """The binding's stream argument takes a torch stream object or its raw
    handle; either runs the layer on that stream with the same bits as torch's
    current stream."""
    T, d, E, K, n = 300, 256, 16, 4, 128
    print(f"case explicit stream T={T} d={d} E={E} K={K} n={n}", flush=True)
    inp = mi.draw(T, d, E, n, torch.bfloat16, seed=53)
    dev = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
    desc = moe.make_desc(T, d, E, K, n, "bf16", 0.0)
    ws = moe.workspace(desc, moe.MOE_WS_FORWARD)
    Y = torch.empty_like(dev["X"])
    args = (desc, dev["X"], dev["W_r"], dev["bias"], dev["W_gate"], dev["W_up"], dev["W_down"], Y, ws)
    moe.moe_forward(*args)
    torch.cuda.synchronize()
    want = Y.clone()
    s = torch.cuda.Stream()
    for handle in (s, s.cuda_stream):
        Y.fill_(float("nan"))
        s.wait_stream(torch.cuda.current_stream())
        moe.moe_forward(*args, stream=handle)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        assert torch.equal(Y, want), type(handle).__name__
