"""The C-ABI library on the host: it loads, exports every symbol that
include/moe.h declares, and its host-only logic (validation, capacity,
workspace sizes, argument errors) behaves as documented.  No compute call is
made: every device entry point below fails validation (or is a T = 0 no-op)
before anything is enqueued, so these run without a GPU."""

import ctypes
import os
import re

import pytest

import top_routing_grouped_amd as moe
from oracle import moe_oracle as mo

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "moe.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:moe_status|const char\*)\s+(moe_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_symbol():
    names = _declared()
    assert len(names) == 25
    lib = moe.lib()
    for name in names:
        assert hasattr(lib, name), name


def test_status_strings():
    lib = moe.lib()
    assert lib.moe_status_str(0) == b"MOE_OK"
    assert lib.moe_status_str(-4) == b"MOE_ERR_WORKSPACE"
    assert lib.moe_status_str(-6) == b"MOE_ERR_HOST"
    assert lib.moe_status_str(7) == b"unknown moe_status"


def test_validate_cases():
    ok = moe.make_desc(16, 128, 8, 2, 256, "bf16")
    assert moe.moe_validate(ok) == moe.MOE_OK
    bad = [
        (moe.make_desc(16, 128, 8, 9, 256), moe.MOE_ERR_INVALID_ARG),          # K > E
        (moe.make_desc(16, 128, 8, 0, 256), moe.MOE_ERR_INVALID_ARG),          # K = 0
        (moe.make_desc(-1, 128, 8, 2, 256), moe.MOE_ERR_INVALID_ARG),          # T < 0
        (moe.make_desc(16, 128, 0, 1, 256), moe.MOE_ERR_INVALID_ARG),          # E = 0
        (moe.make_desc(16, 128, 300, 2, 256), moe.MOE_ERR_UNSUPPORTED),        # E > 256
        (moe.make_desc(16, 100, 8, 2, 256), moe.MOE_ERR_UNSUPPORTED),          # d % 64
        (moe.make_desc(16, 128, 8, 2, 96), moe.MOE_ERR_UNSUPPORTED),           # n % 64
        (moe.make_desc(16, 128, 8, 2, 256, flags=6), moe.MOE_ERR_INVALID_ARG),  # both GEMM paths
        (moe.make_desc(16, 128, 8, 2, 256, flags=32), moe.MOE_ERR_INVALID_ARG),  # undefined bit
        (moe.make_desc(16, 128, 8, 2, 256, capacity_factor=float("nan")), moe.MOE_ERR_INVALID_ARG),
        (moe.make_desc(16, 128, 8, 2, 256, capacity_factor=float("inf")), moe.MOE_ERR_INVALID_ARG),
        (moe.make_desc(2 ** 30, 128, 8, 2, 256), moe.MOE_ERR_UNSUPPORTED),     # T*K >= 2^31
        (moe.make_desc(2 ** 28, 128, 8, 8, 256), moe.MOE_ERR_UNSUPPORTED),     # T*K == 2^31 exactly
        # T*K would wrap a 64-bit product to 0 (2^62 * 8 = 2^65)
        (moe.make_desc(2 ** 62, 128, 8, 8, 256), moe.MOE_ERR_UNSUPPORTED),
        (moe.make_desc(2 ** 63 - 1, 128, 256, 256, 256), moe.MOE_ERR_UNSUPPORTED),
        # grouped-GEMM grids beyond 32-bit tile numbering
        (moe.make_desc(2 ** 20, 2 ** 30, 8, 1, 64), moe.MOE_ERR_UNSUPPORTED),
        (moe.make_desc(2 ** 20, 64, 8, 1, 2 ** 29), moe.MOE_ERR_UNSUPPORTED),
    ]
    for desc, want in bad:
        assert moe.moe_validate(desc) == want
    # the largest T*K accepted: 2^31 - 1
    assert moe.moe_validate(moe.make_desc(2 ** 31 - 1, 128, 8, 1, 256)) == moe.MOE_OK
    for f in (1, 2, 4, 5, 8, 10, 16, 26):                     # defined bits are valid
        assert moe.moe_validate(moe.make_desc(16, 128, 8, 2, 256, flags=f)) == moe.MOE_OK
    d = moe.make_desc(16, 128, 8, 2, 256)
    d.dtype = 7
    assert moe.moe_validate(d) == moe.MOE_ERR_INVALID_ARG


@pytest.mark.parametrize("T,K,E,cf", [
    (8192, 4, 64, 1.25), (100, 2, 4, 0.0), (100, 2, 4, -1.0), (100, 2, 4, 1e-9),
    (100, 2, 4, 1e9), (10, 1, 1, 0.25), (10, 1, 1, 0.5), (10, 1, 1, 0.1), (0, 2, 4, 1.0),
    (16384, 8, 128, 1.0), (12345, 3, 7, 0.3), (777, 5, 200, 2.5), (1, 1, 1, 1e-300),
    (1000, 8, 256, 3.0 / 7.0), (4096, 2, 8, 1e300),
])
def test_capacity_matches_oracle(T, K, E, cf):
    desc = moe.make_desc(T, 128, E, K, 128, "bf16", cf)
    assert moe.moe_capacity(desc) == mo.capacity(T, K, E, cf)
    C = mo.capacity(T, K, E, cf)
    assert moe.moe_max_rows(desc) == min(T * K, E * C)


def test_workspace_sizes_grow_with_problem():
    small = moe.make_desc(64, 128, 8, 2, 128)
    big = moe.make_desc(16384, 2048, 128, 8, 768)
    for entry in (moe.MOE_WS_PERMUTE, moe.MOE_WS_GROUPED_FFN, moe.MOE_WS_FORWARD):
        a = moe.moe_workspace_size(small, entry)
        b = moe.moe_workspace_size(big, entry)
        assert 0 < a < b
    # forward workspace holds H and O for every kept row
    rows = moe.moe_max_rows(big)
    assert moe.moe_workspace_size(big, moe.MOE_WS_FORWARD) >= rows * (768 + 2048) * 2
    with pytest.raises(moe.MoeError):
        moe.moe_workspace_size(small, 9)


def _raw(name):
    return getattr(moe.lib(), name)


def test_device_entry_points_reject_bad_arguments_without_enqueueing():
    lib = moe.lib()
    desc = moe.make_desc(64, 128, 8, 2, 128)
    p = ctypes.byref(desc)
    A = ctypes.c_void_p(1 << 20)          # aligned fake pointers: never dereferenced
    U = ctypes.c_void_p((1 << 20) + 4)    # misaligned
    # null required pointer
    assert lib.moe_route(p, None, A, None, None, A, A, None) == moe.MOE_ERR_INVALID_ARG
    assert b"X is NULL" in lib.moe_last_error()
    # misaligned pointer
    assert lib.moe_route(p, U, A, None, None, A, A, None) == moe.MOE_ERR_ALIGNMENT
    assert lib.moe_combine(p, A, A, A, U, None) == moe.MOE_ERR_ALIGNMENT
    # missing / short workspace
    assert lib.moe_permute(p, A, A, A, None, A, A, None, 0, None) == moe.MOE_ERR_WORKSPACE
    assert lib.moe_forward(p, A, A, None, A, A, A, A, A, 16, None) == moe.MOE_ERR_WORKSPACE
    assert lib.moe_grouped_ffn(p, A, A, A, A, A, A, A, A, A, 0, None) == moe.MOE_ERR_WORKSPACE
    # invalid description
    bad = moe.make_desc(64, 128, 8, 9, 128)
    assert lib.moe_forward(ctypes.byref(bad), A, A, None, A, A, A, A, A, 1 << 30, None) == \
        moe.MOE_ERR_INVALID_ARG
    # T = 0 is a successful no-op (no launch)
    zero = moe.make_desc(0, 128, 8, 2, 128)
    ws = moe.moe_workspace_size(zero, moe.MOE_WS_FORWARD)
    assert lib.moe_forward(ctypes.byref(zero), A, A, None, A, A, A, A, A, ws + 256, None) == moe.MOE_OK
    assert lib.moe_route(ctypes.byref(zero), A, A, None, None, A, A, None) == moe.MOE_OK


def test_route_workspace_only_for_small_batches():
    # a decode-sized batch splits the router's k range (partials in the workspace)
    small = moe.make_desc(64, 4096, 256, 8, 512)
    assert moe.moe_workspace_size(small, moe.MOE_WS_ROUTE) >= 64 * 256 * 4 * 2
    # a batch that fills the GPU with 64-token blocks needs none
    big = moe.make_desc(16384, 2048, 128, 8, 768)
    assert moe.moe_workspace_size(big, moe.MOE_WS_ROUTE) == 0
    # fp32 and E not a multiple of 8 never split
    assert moe.moe_workspace_size(moe.make_desc(64, 4096, 256, 8, 512, "fp32"), moe.MOE_WS_ROUTE) == 0
    assert moe.moe_workspace_size(moe.make_desc(64, 4096, 250, 8, 512), moe.MOE_WS_ROUTE) == 0
    # the forward workspace holds the partials too
    assert moe.moe_workspace_size(small, moe.MOE_WS_FORWARD) > moe.moe_workspace_size(small, moe.MOE_WS_ROUTE)
    lib = moe.lib()
    A = ctypes.c_void_p(1 << 20)
    assert lib.moe_route_ws(ctypes.byref(small), A, A, None, None, A, A, None, 0, None) == \
        moe.MOE_ERR_WORKSPACE
    assert lib.moe_route_ws(ctypes.byref(moe.make_desc(0, 4096, 256, 8, 512)), A, A, None, None, A, A,
                            None, 0, None) == moe.MOE_OK


def test_gemm_path_flags_are_checked_per_entry_point():
    lib = moe.lib()
    A = ctypes.c_void_p(1 << 20)
    T0 = lambda flags: moe.make_desc(0, 128, 8, 2, 128, flags=flags)   # T = 0: checks only
    both = moe.MOE_FLAG_GEMM_TILED | moe.MOE_FLAG_GEMM_SKINNY
    for f in (moe.MOE_FLAG_GEMM_TILED, moe.MOE_FLAG_GEMM_SKINNY,
              moe.MOE_FLAG_GEMM_SKINNY | moe.MOE_FLAG_TILE_TABLE_READY):
        assert lib.moe_grouped_ffn(ctypes.byref(T0(f)), A, A, A, A, A, A, A, A, A, 1 << 20, None) == moe.MOE_OK
    assert lib.moe_grouped_ffn(ctypes.byref(T0(both)), A, A, A, A, A, A, A, A, A, 1 << 20, None) == \
        moe.MOE_ERR_INVALID_ARG
    assert b"exclusive" in lib.moe_last_error()
    ws = moe.moe_workspace_size(T0(0), moe.MOE_WS_FORWARD) + 256
    assert lib.moe_forward(ctypes.byref(T0(moe.MOE_FLAG_GEMM_SKINNY)), A, A, None, A, A, A, A, A, ws,
                           None) == moe.MOE_OK
    # the tile-table bit belongs to the grouped entry points only; route takes
    # only the selection bit, which the grouped GEMMs and the permutation refuse
    assert lib.moe_forward(ctypes.byref(T0(moe.MOE_FLAG_TILE_TABLE_READY)), A, A, None, A, A, A, A,
                           A, ws, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_route(ctypes.byref(T0(moe.MOE_FLAG_GEMM_TILED)), A, A, None, None, A, A, None) == \
        moe.MOE_ERR_INVALID_ARG
    thr = moe.MOE_FLAG_TOPK_THRESHOLD
    assert lib.moe_route(ctypes.byref(T0(thr)), A, A, None, None, A, A, None) == moe.MOE_OK
    assert lib.moe_forward(ctypes.byref(T0(thr | moe.MOE_FLAG_GEMM_TILED)), A, A, None, A, A, A, A,
                           A, ws, None) == moe.MOE_OK
    assert lib.moe_grouped_ffn(ctypes.byref(T0(thr)), A, A, A, A, A, A, A, A, A, 1 << 20, None) == \
        moe.MOE_ERR_INVALID_ARG
    assert lib.moe_permute(ctypes.byref(T0(thr)), A, A, A, A, A, A, None, 0, None) == \
        moe.MOE_ERR_INVALID_ARG


def test_saved_layout_fields():
    desc = moe.make_desc(16384, 2048, 128, 8, 768)
    L = moe.moe_saved_layout_of(desc)
    T, K, E, n = 16384, 8, 128, 768
    rows = moe.moe_max_rows(desc)
    order = [("logits", T * E * 4), ("topk_ids", T * K * 4), ("topk_gates", T * K * 4),
             ("inv_slot", T * K * 4), ("perm_token", T * K * 4), ("counts", E * 4),
             ("offsets", (E + 1) * 4), ("preact", rows * 2 * n * 2)]
    end = 0
    for name, size in order:
        off = getattr(L, name)
        assert off % 256 == 0 and off >= end, name
        end = off + size
    assert L.bytes >= end
    assert moe.moe_workspace_size(desc, moe.MOE_WS_SAVED) == L.bytes
    assert moe.moe_workspace_size(desc, moe.MOE_WS_BACKWARD) > rows * (2 * n + n + 2048) * 2


def test_training_entry_points_check_arguments():
    lib = moe.lib()
    A = ctypes.c_void_p(1 << 20)
    desc = moe.make_desc(64, 128, 8, 2, 128)
    p = ctypes.byref(desc)
    big = 1 << 30
    # bf16 only, tiled GEMMs only
    f32 = moe.make_desc(64, 128, 8, 2, 128, "fp32")
    assert lib.moe_forward_train(ctypes.byref(f32), A, A, None, A, A, A, A, A, big, A, big, None) == \
        moe.MOE_ERR_UNSUPPORTED
    assert lib.moe_backward(ctypes.byref(f32), A, A, A, A, A, A, A, big, A, A, A, A, A, A, big,
                            None) == moe.MOE_ERR_UNSUPPORTED
    sk = moe.make_desc(64, 128, 8, 2, 128, flags=moe.MOE_FLAG_GEMM_SKINNY)
    assert lib.moe_forward_train(ctypes.byref(sk), A, A, None, A, A, A, A, A, big, A, big, None) == \
        moe.MOE_ERR_INVALID_ARG
    # short saved state / workspace
    assert lib.moe_forward_train(p, A, A, None, A, A, A, A, A, 16, A, big, None) == moe.MOE_ERR_WORKSPACE
    assert b"MOE_WS_SAVED" in lib.moe_last_error()
    assert lib.moe_forward_train(p, A, A, None, A, A, A, A, A, big, A, 16, None) == moe.MOE_ERR_WORKSPACE
    assert lib.moe_backward(p, A, A, A, A, A, A, A, 16, A, A, A, A, A, A, big, None) == \
        moe.MOE_ERR_WORKSPACE
    assert lib.moe_backward(p, A, A, A, A, A, A, A, big, A, A, A, A, A, A, 16, None) == \
        moe.MOE_ERR_WORKSPACE
    assert b"MOE_WS_BACKWARD" in lib.moe_last_error()
    # null gradient outputs are rejected before anything else
    assert lib.moe_backward(p, A, A, A, A, A, A, A, big, A, None, A, A, A, A, big, None) == \
        moe.MOE_ERR_INVALID_ARG
    assert b"dW_r is NULL" in lib.moe_last_error()
    # the training forward of an empty batch is a no-op
    zero = moe.make_desc(0, 128, 8, 2, 128)
    assert lib.moe_forward_train(ctypes.byref(zero), A, A, None, A, A, A, A, A, big, A, big, None) == \
        moe.MOE_OK


def test_missing_library_fails_loudly(monkeypatch):
    monkeypatch.setattr(moe, "_lib", None)
    monkeypatch.setattr(moe, "LIB_PATH", "/nonexistent/libmoe_mi355x.so")
    with pytest.raises(RuntimeError, match="no non-HIP fallback"):
        moe.lib()


def test_token_rounding_arguments():
    lib = moe.lib()
    A = ctypes.c_void_p(1 << 20)
    desc = moe.make_desc(64, 128, 8, 2, 128)
    p = ctypes.byref(desc)
    need = moe.moe_workspace_size(desc, moe.MOE_WS_ROUND)
    assert need >= 3 * moe.moe_max_rows(desc) * 4
    assert lib.moe_round_tokens(p, A, A, A, A, A, A, A, need - 1, None) == moe.MOE_ERR_WORKSPACE
    assert b"MOE_WS_ROUND" in lib.moe_last_error()
    assert lib.moe_round_tokens(p, A, None, A, A, A, A, A, need, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_round_tokens(ctypes.byref(moe.make_desc(0, 128, 8, 2, 128)), A, A, A, A, A, A,
                                A, 0, None) == moe.MOE_OK
    # the rounding flag belongs to moe_forward, not to the grouped or training calls
    rd = lambda f: moe.make_desc(0, 128, 8, 2, 128, flags=f)
    big = 1 << 30
    assert lib.moe_forward(ctypes.byref(rd(8)), A, A, None, A, A, A, A, A, big, None) == moe.MOE_OK
    assert lib.moe_grouped_ffn(ctypes.byref(rd(8)), A, A, A, A, A, A, A, A, A, big, None) == \
        moe.MOE_ERR_INVALID_ARG
    assert lib.moe_forward_train(ctypes.byref(rd(8)), A, A, None, A, A, A, A, A, big, A, big,
                                 None) == moe.MOE_ERR_INVALID_ARG


def test_atomic_expert_descriptor_checks():
    ok = moe.make_omni_desc(4096, 1024, 256, 256, 64)
    assert moe.moe_omni_validate(ok) == moe.MOE_OK
    bad = [
        (moe.make_omni_desc(16, 1024, 257, 4, 4), moe.MOE_ERR_UNSUPPORTED),   # axis above 256
        (moe.make_omni_desc(16, 1024, 16, 16, 65), moe.MOE_ERR_UNSUPPORTED),  # K above 64
        (moe.make_omni_desc(16, 1024, 2, 2, 5), moe.MOE_ERR_INVALID_ARG),     # K > N
        (moe.make_omni_desc(16, 1024, 0, 2, 1), moe.MOE_ERR_INVALID_ARG),
        (moe.make_omni_desc(16, 96, 4, 4, 2), moe.MOE_ERR_UNSUPPORTED),       # d % 64
        (moe.make_omni_desc(16, 8192, 4, 4, 2), moe.MOE_ERR_UNSUPPORTED),     # d above 4096
        (moe.make_omni_desc(16, 1024, 4, 4, 2, "fp32"), moe.MOE_ERR_UNSUPPORTED),
        (moe.make_omni_desc(16, 1024, 4, 4, 2, flags=1), moe.MOE_ERR_INVALID_ARG),
        (moe.make_omni_desc(-1, 1024, 4, 4, 2), moe.MOE_ERR_INVALID_ARG),
        (moe.make_omni_desc(2 ** 25, 1024, 256, 256, 64), moe.MOE_ERR_UNSUPPORTED),  # T*K = 2^31
        (moe.make_omni_desc(2 ** 62, 1024, 256, 256, 8), moe.MOE_ERR_UNSUPPORTED),   # would wrap
    ]
    for desc, want in bad:
        assert moe.moe_omni_validate(desc) == want
    fw = moe.moe_omni_workspace_size(ok, moe.MOE_OMNI_WS_FORWARD)
    assert fw > moe.moe_omni_workspace_size(ok, moe.MOE_OMNI_WS_ROUTE)
    assert fw > moe.moe_omni_workspace_size(ok, moe.MOE_OMNI_WS_PERMUTE)
    lib = moe.lib()
    A = ctypes.c_void_p(1 << 20)
    p = ctypes.byref(ok)
    assert lib.moe_omni_forward(p, A, A, A, A, A, A, A, 16, None) == moe.MOE_ERR_WORKSPACE
    assert lib.moe_omni_route(p, A, A, None, None, None, A, A, A, 1 << 30, None) == \
        moe.MOE_ERR_INVALID_ARG
    zero = moe.make_omni_desc(0, 1024, 4, 4, 2)
    assert lib.moe_omni_forward(ctypes.byref(zero), A, A, A, A, A, A, A, 0, None) == moe.MOE_OK


def test_allocation_free_permutation_rejects_problems_beyond_its_scratch():
    """moe_permute_noalloc keeps its scratch in a static device array of
    MOE_NOALLOC_SCRATCH_BYTES: a problem whose permutation needs more gets
    MOE_ERR_WORKSPACE before anything is enqueued (so no GPU is needed)."""
    lib = moe.lib()
    A = ctypes.c_void_p(1 << 20)          # aligned fake pointers: never dereferenced
    fits = moe.make_desc(131072, 128, 256, 8, 128)
    assert moe.moe_workspace_size(fits, moe.MOE_WS_PERMUTE) <= moe.MOE_NOALLOC_SCRATCH_BYTES
    big = moe.make_desc(262144, 128, 256, 8, 128)
    assert moe.moe_workspace_size(big, moe.MOE_WS_PERMUTE) > moe.MOE_NOALLOC_SCRATCH_BYTES
    assert lib.moe_permute_noalloc(ctypes.byref(big), A, A, A, None, A, A, None) == \
        moe.MOE_ERR_WORKSPACE
    assert b"MOE_NOALLOC_SCRATCH_BYTES" in lib.moe_last_error()
    also_big = moe.make_desc(262144 * 2, 128, 128, 2, 128)
    assert lib.moe_permute_noalloc(ctypes.byref(also_big), A, A, A, None, A, A, None) == \
        moe.MOE_ERR_WORKSPACE
    # argument errors come first, as for moe_permute
    small = moe.make_desc(64, 128, 8, 2, 128)
    assert lib.moe_permute_noalloc(ctypes.byref(small), None, A, A, None, A, A, None) == \
        moe.MOE_ERR_INVALID_ARG
    U = ctypes.c_void_p((1 << 20) + 4)
    assert lib.moe_permute_noalloc(ctypes.byref(small), A, A, A, U, A, A, None) == \
        moe.MOE_ERR_ALIGNMENT
    # T = 0 is a no-op
    zero = moe.make_desc(0, 128, 8, 2, 128)
    assert lib.moe_permute_noalloc(ctypes.byref(zero), None, None, None, None, None, None, None) == \
        moe.MOE_OK


def test_route_permute_workspace_and_argument_checks():
    lib = moe.lib()
    A = ctypes.c_void_p(1 << 20)
    for T, E in ((64, 8), (16384, 128), (3000, 128), (32768, 256)):
        desc = moe.make_desc(T, 256, E, 4, 128)
        need = moe.moe_workspace_size(desc, moe.MOE_WS_ROUTE_PERMUTE)
        assert need >= moe.moe_workspace_size(desc, moe.MOE_WS_ROUTE)
        assert need % 256 == 0
    desc = moe.make_desc(64, 128, 8, 2, 128)
    p = ctypes.byref(desc)
    # missing workspace, then a null required pointer, then T = 0 as a no-op
    assert lib.moe_route_permute(p, A, A, None, None, A, A, A, A, None, A, A, A, 16, None) == \
        moe.MOE_ERR_WORKSPACE
    assert lib.moe_route_permute(p, A, A, None, None, None, A, A, A, None, A, A, A, 1 << 20, None) == \
        moe.MOE_ERR_INVALID_ARG
    zero = moe.make_desc(0, 128, 8, 2, 128)
    assert lib.moe_route_permute(ctypes.byref(zero), None, None, None, None, None, None, None, None,
                                 None, None, None, None, 0, None) == moe.MOE_OK


def test_binding_checks_shapes_and_dtypes_before_any_device_pointer():
    # CPU tensors: every refusal below happens before a device pointer is taken
    import torch
    bf = torch.bfloat16
    T, d, E, K, n = 32, 128, 8, 2, 256
    X = torch.zeros(T, d, dtype=bf)
    W_r = torch.zeros(d, E, dtype=bf)
    Wg = torch.zeros(E, d, n, dtype=bf)
    Wu = torch.zeros(E, d, n, dtype=bf)
    Wd = torch.zeros(E, n, d, dtype=bf)
    with pytest.raises(ValueError, match="bfloat16 or float32"):
        moe.forward(X.half(), W_r, Wg, Wu, Wd, K)
    with pytest.raises(ValueError, match="W_r"):                 # weights of another dtype
        moe.forward(X.float(), W_r, Wg.float(), Wu.float(), Wd.float(), K)
    with pytest.raises(ValueError, match="W_down"):              # W_down given as [E, d, n]
        moe.forward(X, W_r, Wg, Wu, Wd.transpose(1, 2).contiguous().view(E, d, n), K)
    with pytest.raises(ValueError, match="bias"):
        moe.forward(X, W_r, Wg, Wu, Wd, K, bias=torch.zeros(E, dtype=bf))
    with pytest.raises(ValueError, match="W_up"):
        moe.forward_train(X, W_r, Wg, Wu[:, :, :128].contiguous(), Wd, K)
    with pytest.raises(ValueError, match="W_r"):
        moe.route(X, torch.zeros(d + 64, E, dtype=bf), K)
    desc = moe.make_desc(T, d, E, K, n, "bf16")
    with pytest.raises(ValueError, match="differs from desc.K"):
        moe.route_permute(X, W_r, K + 1, desc)
    rows = moe.moe_max_rows(desc)
    with pytest.raises(ValueError, match="O: expected at least"):
        moe.combine(desc, torch.zeros(rows - 1, d, dtype=bf), torch.zeros(T, K),
                    torch.zeros(T, K, dtype=torch.int32))
    with pytest.raises(ValueError, match="gates"):
        moe.combine(desc, torch.zeros(rows, d, dtype=bf), torch.zeros(T, K, dtype=bf),
                    torch.zeros(T, K, dtype=torch.int32))
    with pytest.raises(ValueError, match="W_gate"):
        moe.grouped_ffn(desc, X, None, None, Wg.float(), Wu, Wd)
    with pytest.raises(ValueError, match="dY"):
        moe.backward(desc, None, X, W_r, Wg, Wu, Wd, torch.zeros(T, d))
    # consistent CPU tensors pass the checks and reach the device-pointer check
    with pytest.raises(ValueError, match="device tensor"):
        moe.forward(X, W_r, Wg, Wu, Wd, K)


def test_atomic_expert_binding_checks_shapes_and_dtypes():
    import torch
    bf = torch.bfloat16
    T, d, Nr, Nc, K = 16, 128, 8, 8, 4
    X = torch.zeros(T, d, dtype=bf)
    W_r, W_c = torch.zeros(d, Nr, dtype=bf), torch.zeros(d, Nc, dtype=bf)
    W_in, W_out = torch.zeros(Nr * Nc, d, dtype=bf), torch.zeros(Nr * Nc, d, dtype=bf)
    with pytest.raises(ValueError, match="X"):
        moe.omni_forward(X.float(), W_r, W_c, W_in, W_out, K)
    with pytest.raises(ValueError, match="W_c"):
        moe.omni_route(X, W_r, torch.zeros(d + 64, Nc, dtype=bf), K)
    with pytest.raises(ValueError, match="W_out"):
        moe.omni_forward(X, W_r, W_c, W_in, W_out[:-1].contiguous(), K)
    desc = moe.make_omni_desc(T, d, Nr, Nc, K)
    with pytest.raises(ValueError, match="ids"):
        moe.omni_permute(desc, torch.zeros(T, K + 1, dtype=torch.int32))
    with pytest.raises(ValueError, match="device tensor"):      # consistent: reaches the pointers
        moe.omni_forward(X, W_r, W_c, W_in, W_out, K)
