"""The allocation-free permutation (moe_permute_noalloc, scratch in a static
device array) against moe_permute (caller's workspace), through the C ABI:
the same bits on two calls in a row, the second with a smaller input, so the
second call runs on scratch the first one left behind."""

import numpy as np
import pytest
import torch

import moe_inputs as mi
import top_routing_grouped_amd as moe
from gpu_common import device_inputs, intnp

pytestmark = pytest.mark.gpu


def _route(T, d, E, K, seed, bias):
    inp = mi.draw(T, d, E, 64, torch.bfloat16, seed=seed, bias=bias)
    dev = device_inputs(inp)
    ids, gates, _ = moe.route(dev["X"], dev["W_r"], K, bias=dev["bias"], n=64)
    return ids


def _outputs(T, K, E):
    i32 = dict(dtype=torch.int32, device="cuda")
    return {"counts": torch.full((E,), -7, **i32), "offsets": torch.full((E + 1,), -7, **i32),
            "raw": torch.full((E,), -7, **i32), "perm": torch.full((T * K,), -7, **i32),
            "inv": torch.full((T, K), -7, **i32)}


def _compare(T, d, E, K, cf, seed, bias, with_raw):
    print(f"no-alloc permute T={T} E={E} K={K} cf={cf} raw={with_raw}", flush=True)
    ids = _route(T, d, E, K, seed, bias)
    desc = moe.make_desc(T, d, E, K, 64, "bf16", cf)
    a, b = _outputs(T, K, E), _outputs(T, K, E)
    moe.moe_permute(desc, ids, a["counts"], a["offsets"], a["raw"] if with_raw else None, a["perm"],
                    a["inv"], moe.workspace(desc, moe.MOE_WS_PERMUTE))
    moe.moe_permute_noalloc(desc, ids, b["counts"], b["offsets"], b["raw"] if with_raw else None,
                            b["perm"], b["inv"])
    torch.cuda.synchronize()
    for k in a:
        assert torch.equal(a[k], b[k]), k
    N = int(intnp(a["offsets"])[E])
    assert N > 0 and bool(torch.all(b["perm"][:N] >= 0))
    return N


def test_noalloc_permute_matches_workspace_permute_on_two_calls():
    # first call: several token blocks, capacity drops under a skewed router
    n1 = _compare(5000, 256, 64, 6, 1.0, 31, "zipf", True)
    assert n1 < 5000 * 6
    # second call, smaller: fewer blocks and experts, on the scratch the first left behind
    _compare(1200, 128, 16, 2, 0.0, 32, None, False)


def test_noalloc_permute_one_block_and_full_size():
    # one token block (the single-workgroup path), then the Qwen3-shaped batch
    _compare(200, 128, 32, 4, 0.0, 33, None, False)
    _compare(16384, 2048, 128, 8, 0.0, 34, None, True)
    _compare(300, 128, 8, 2, 1.0, 35, None, True)
