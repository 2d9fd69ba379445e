"""The seeded input generator: determinism, shapes and the stated recipe."""
import math

import torch

import moe_inputs as mi


def test_draw_is_deterministic_and_shaped():
    a = mi.draw(16, 32, 4, 8, torch.bfloat16, seed=3)
    b = mi.draw(16, 32, 4, 8, torch.bfloat16, seed=3)
    for k in ("X", "W_r", "W_gate", "W_up", "W_down"):
        assert torch.equal(a[k], b[k])
        assert a[k].dtype == torch.bfloat16
    assert a["X"].shape == (16, 32) and a["W_r"].shape == (32, 4)
    assert a["W_gate"].shape == (4, 32, 8) and a["W_down"].shape == (4, 8, 32)
    c = mi.draw(16, 32, 4, 8, torch.bfloat16, seed=4)
    assert not torch.equal(a["X"], c["X"])


def test_draw_order_and_scale():
    g = torch.Generator().manual_seed(0)
    X = torch.randn(8, 64, generator=g)
    W_r = torch.randn(64, 4, generator=g) / math.sqrt(64)
    got = mi.draw(8, 64, 4, 16, torch.float32, seed=0)
    assert torch.equal(got["X"], X)
    assert torch.allclose(got["W_r"], W_r, rtol=0, atol=0)


def test_zipf_bias():
    b = mi.zipf_bias(64)
    assert b.dtype == torch.float32
    assert b[0].item() == 0.0
    assert abs(b[1].item() - 1.5 * math.log(0.5)) < 1e-6
    assert torch.all(b[1:] < b[:-1])


def test_workload_table():
    w = mi.WORKLOADS["qwen3_bf16"]
    assert (w.T, w.d, w.E, w.K, w.n) == (16384, 2048, 128, 8, 768)
    assert mi.WORKLOADS["skewed_cap_bf16"].capacity_factor == 1.25
    assert mi.WORKLOADS["granular_decode_bf16"].parent == "granular_bf16"
    assert mi.WORKLOADS["tiny_fp32"].dtype == "fp32"
