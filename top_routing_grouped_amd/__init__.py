"""MI355X (gfx950) MoE layer (forward and backward): Python binding over the C ABI of include/moe.h.

Argument marshalling only.  Every step of the layer runs in the HIP kernels of
``libmoe_mi355x.so``; PyTorch supplies device memory and the stream.  If the
library has not been built, every call raises (there is no fallback path).

Low-level functions carry the C names (``moe_route``, ``moe_permute``,
``moe_permute_noalloc``, ``moe_route_permute``, ``moe_grouped_gemm_up``, ``moe_grouped_gemm_down``, ``moe_grouped_ffn``,
``moe_round_tokens``, ``moe_combine``, ``moe_forward``, ``moe_forward_train``,
``moe_backward`` and the host-only queries) and take torch tensors.
``route``, ``permute``, ``round_tokens``, ``grouped_ffn``, ``combine``,
``forward``, ``forward_train`` and ``backward`` allocate the outputs with
torch and call them.
"""

from __future__ import annotations

import ctypes
import os

LIB_NAME = "libmoe_mi355x.so"
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), LIB_NAME)

MOE_OK = 0
MOE_ERR_INVALID_ARG = -1
MOE_ERR_UNSUPPORTED = -2
MOE_ERR_ALIGNMENT = -3
MOE_ERR_WORKSPACE = -4
MOE_ERR_HIP = -5
MOE_ERR_HOST = -6
MOE_F32 = 0
MOE_BF16 = 1
MOE_WS_PERMUTE = 0
MOE_WS_GROUPED_FFN = 1
MOE_WS_FORWARD = 2
MOE_WS_ROUTE = 3
MOE_WS_SAVED = 4
MOE_WS_BACKWARD = 5
MOE_WS_ROUND = 6
MOE_WS_ROUTE_PERMUTE = 7
MOE_FLAG_TILE_TABLE_READY = 1
MOE_FLAG_GEMM_TILED = 2
MOE_FLAG_GEMM_SKINNY = 4
MOE_FLAG_TOKEN_ROUNDING = 8
MOE_FLAG_TOPK_THRESHOLD = 16
MOE_NOALLOC_SCRATCH_BYTES = 2 << 20


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: status {status} ({detail})")
        self.status = status


class MoeDesc(ctypes.Structure):
    """Mirror of ``moe_desc`` (same field order, natural alignment)."""

    _fields_ = [
        ("T", ctypes.c_int64),
        ("d", ctypes.c_int32),
        ("E", ctypes.c_int32),
        ("K", ctypes.c_int32),
        ("n", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("capacity_factor", ctypes.c_double),
        ("flags", ctypes.c_uint32),
    ]


def make_desc(T, d, E, K, n, dtype="bf16", capacity_factor=0.0, flags=0) -> MoeDesc:
    code = {"bf16": MOE_BF16, "fp32": MOE_F32, MOE_BF16: MOE_BF16, MOE_F32: MOE_F32}[dtype]
    return MoeDesc(int(T), int(d), int(E), int(K), int(n), code, float(capacity_factor), int(flags))


class MoeOmniDesc(ctypes.Structure):
    """Mirror of ``moe_omni_desc``."""

    _fields_ = [
        ("T", ctypes.c_int64),
        ("d", ctypes.c_int32),
        ("Nr", ctypes.c_int32),
        ("Nc", ctypes.c_int32),
        ("K", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("flags", ctypes.c_uint32),
    ]


MOE_OMNI_WS_ROUTE = 0
MOE_OMNI_WS_PERMUTE = 1
MOE_OMNI_WS_FORWARD = 2


def make_omni_desc(T, d, Nr, Nc, K, dtype="bf16", flags=0) -> MoeOmniDesc:
    code = {"bf16": MOE_BF16, "fp32": MOE_F32, MOE_BF16: MOE_BF16, MOE_F32: MOE_F32}[dtype]
    return MoeOmniDesc(int(T), int(d), int(Nr), int(Nc), int(K), code, int(flags))


class MoeSavedLayout(ctypes.Structure):
    """Mirror of ``moe_saved_layout``: byte offsets of the saved state's fields."""

    _fields_ = [(name, ctypes.c_size_t) for name in
                ("logits", "topk_ids", "topk_gates", "inv_slot", "perm_token", "counts",
                 "offsets", "preact", "bytes")]


_lib = None
_VP = ctypes.c_void_p
_DP = ctypes.POINTER(MoeDesc)
_SIGNATURES = {
    "moe_validate": [_DP],
    "moe_capacity": [_DP, ctypes.POINTER(ctypes.c_int64)],
    "moe_max_rows": [_DP, ctypes.POINTER(ctypes.c_int64)],
    "moe_workspace_size": [_DP, ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)],
    "moe_route": [_DP, _VP, _VP, _VP, _VP, _VP, _VP, _VP],
    "moe_route_ws": [_DP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_size_t, _VP],
    "moe_permute": [_DP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_size_t, _VP],
    "moe_grouped_gemm_up": [_DP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_size_t, _VP],
    "moe_grouped_gemm_down": [_DP, _VP, _VP, _VP, _VP, _VP, ctypes.c_size_t, _VP],
    "moe_grouped_ffn": [_DP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_size_t, _VP],
    "moe_combine": [_DP, _VP, _VP, _VP, _VP, _VP],
    "moe_forward": [_DP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_size_t, _VP],
    "moe_saved_layout_of": [_DP, ctypes.POINTER(MoeSavedLayout)],
    "moe_round_tokens": [_DP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_size_t, _VP],
    "moe_permute_noalloc": [_DP, _VP, _VP, _VP, _VP, _VP, _VP, _VP],
    "moe_route_permute": [_DP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                          ctypes.c_size_t, _VP],
    "moe_omni_validate": [ctypes.c_void_p],
    "moe_omni_workspace_size": [ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)],
    "moe_omni_route": [ctypes.c_void_p, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_size_t,
                       _VP],
    "moe_omni_permute": [ctypes.c_void_p, _VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_size_t, _VP],
    "moe_omni_forward": [ctypes.c_void_p, _VP, _VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_size_t, _VP],
    "moe_forward_train": [_DP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_size_t, _VP,
                          ctypes.c_size_t, _VP],
    "moe_backward": [_DP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_size_t, _VP, _VP, _VP, _VP,
                     _VP, _VP, ctypes.c_size_t, _VP],
}


def lib() -> ctypes.CDLL:
    """The loaded HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m top_routing_grouped_amd.build` "
                "(there is no non-HIP fallback)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int32
        handle.moe_status_str.argtypes = [ctypes.c_int32]
        handle.moe_status_str.restype = ctypes.c_char_p
        handle.moe_last_error.argtypes = []
        handle.moe_last_error.restype = ctypes.c_char_p
        _lib = handle
    return _lib


def _check(status: int, where: str) -> None:
    if status != MOE_OK:
        L = lib()
        detail = (L.moe_last_error() or b"").decode() or L.moe_status_str(status).decode()
        raise MoeError(status, where, detail)


def _p(t):
    """Device pointer of a tensor (None -> NULL)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    """The hipStream_t to enqueue on: a torch stream object (its handle), a raw
    handle as an int, or None for torch's current stream."""
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    handle = getattr(stream, "cuda_stream", stream)
    return ctypes.c_void_p(int(handle))


# ---------------------------------------------------------------- host-only queries

def moe_validate(desc: MoeDesc) -> int:
    return lib().moe_validate(ctypes.byref(desc))


def moe_capacity(desc: MoeDesc) -> int:
    out = ctypes.c_int64(0)
    _check(lib().moe_capacity(ctypes.byref(desc), ctypes.byref(out)), "moe_capacity")
    return out.value


def moe_max_rows(desc: MoeDesc) -> int:
    out = ctypes.c_int64(0)
    _check(lib().moe_max_rows(ctypes.byref(desc), ctypes.byref(out)), "moe_max_rows")
    return out.value


def moe_workspace_size(desc: MoeDesc, entry: int) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().moe_workspace_size(ctypes.byref(desc), int(entry), ctypes.byref(out)),
           "moe_workspace_size")
    return out.value


def moe_saved_layout_of(desc: MoeDesc) -> MoeSavedLayout:
    out = MoeSavedLayout()
    _check(lib().moe_saved_layout_of(ctypes.byref(desc), ctypes.byref(out)), "moe_saved_layout_of")
    return out


# ---------------------------------------------------------------- device entry points

def moe_route(desc, X, W_r, bias, logits, ids, gates, stream=None):
    _check(lib().moe_route(ctypes.byref(desc), _p(X), _p(W_r), _p(bias), _p(logits), _p(ids),
                           _p(gates), _stream(stream)), "moe_route")


def moe_route_ws(desc, X, W_r, bias, logits, ids, gates, ws, stream=None):
    _check(lib().moe_route_ws(ctypes.byref(desc), _p(X), _p(W_r), _p(bias), _p(logits), _p(ids),
                              _p(gates), _p(ws), ws.numel() * ws.element_size(),
                              _stream(stream)), "moe_route_ws")


def moe_permute(desc, ids, counts, offsets, raw_counts, perm_token, inv_slot, ws, stream=None):
    _check(lib().moe_permute(ctypes.byref(desc), _p(ids), _p(counts), _p(offsets), _p(raw_counts),
                             _p(perm_token), _p(inv_slot), _p(ws), ws.numel() * ws.element_size(),
                             _stream(stream)), "moe_permute")


def moe_route_permute(desc, X, W_r, bias, logits, ids, gates, counts, offsets, raw_counts,
                      perm_token, inv_slot, ws, stream=None):
    _check(lib().moe_route_permute(ctypes.byref(desc), _p(X), _p(W_r), _p(bias), _p(logits),
                                   _p(ids), _p(gates), _p(counts), _p(offsets), _p(raw_counts),
                                   _p(perm_token), _p(inv_slot), _p(ws), _nbytes(ws),
                                   _stream(stream)), "moe_route_permute")


def moe_permute_noalloc(desc, ids, counts, offsets, raw_counts, perm_token, inv_slot, stream=None):
    _check(lib().moe_permute_noalloc(ctypes.byref(desc), _p(ids), _p(counts), _p(offsets),
                                     _p(raw_counts), _p(perm_token), _p(inv_slot),
                                     _stream(stream)), "moe_permute_noalloc")


def moe_round_tokens(desc, ids, gates, counts, offsets, perm_token, inv_slot, ws, stream=None):
    _check(lib().moe_round_tokens(ctypes.byref(desc), _p(ids), _p(gates), _p(counts), _p(offsets),
                                  _p(perm_token), _p(inv_slot), _p(ws), _nbytes(ws),
                                  _stream(stream)), "moe_round_tokens")


def moe_grouped_gemm_up(desc, X, offsets, perm_token, W_gate, W_up, H, ws, stream=None):
    _check(lib().moe_grouped_gemm_up(ctypes.byref(desc), _p(X), _p(offsets), _p(perm_token),
                                     _p(W_gate), _p(W_up), _p(H), _p(ws),
                                     ws.numel() * ws.element_size(), _stream(stream)),
           "moe_grouped_gemm_up")


def moe_grouped_gemm_down(desc, H, offsets, W_down, O, ws, stream=None):
    _check(lib().moe_grouped_gemm_down(ctypes.byref(desc), _p(H), _p(offsets), _p(W_down), _p(O),
                                       _p(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "moe_grouped_gemm_down")


def moe_grouped_ffn(desc, X, offsets, perm_token, W_gate, W_up, W_down, H, O, ws, stream=None):
    _check(lib().moe_grouped_ffn(ctypes.byref(desc), _p(X), _p(offsets), _p(perm_token),
                                 _p(W_gate), _p(W_up), _p(W_down), _p(H), _p(O), _p(ws),
                                 ws.numel() * ws.element_size(), _stream(stream)),
           "moe_grouped_ffn")


def moe_combine(desc, O, gates, inv_slot, Y, stream=None):
    _check(lib().moe_combine(ctypes.byref(desc), _p(O), _p(gates), _p(inv_slot), _p(Y),
                             _stream(stream)), "moe_combine")


def moe_forward(desc, X, W_r, bias, W_gate, W_up, W_down, Y, ws, stream=None):
    _check(lib().moe_forward(ctypes.byref(desc), _p(X), _p(W_r), _p(bias), _p(W_gate), _p(W_up),
                             _p(W_down), _p(Y), _p(ws), ws.numel() * ws.element_size(),
                             _stream(stream)), "moe_forward")


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def moe_forward_train(desc, X, W_r, bias, W_gate, W_up, W_down, Y, saved, ws, stream=None):
    _check(lib().moe_forward_train(ctypes.byref(desc), _p(X), _p(W_r), _p(bias), _p(W_gate),
                                   _p(W_up), _p(W_down), _p(Y), _p(saved), _nbytes(saved), _p(ws),
                                   _nbytes(ws), _stream(stream)), "moe_forward_train")


def moe_backward(desc, X, W_r, W_gate, W_up, W_down, dY, saved, dX, dW_r, dW_gate, dW_up, dW_down,
                 ws, stream=None):
    _check(lib().moe_backward(ctypes.byref(desc), _p(X), _p(W_r), _p(W_gate), _p(W_up),
                              _p(W_down), _p(dY), _p(saved), _nbytes(saved), _p(dX), _p(dW_r),
                              _p(dW_gate), _p(dW_up), _p(dW_down), _p(ws), _nbytes(ws),
                              _stream(stream)), "moe_backward")


# ---------------------------------------------------------------- allocating helpers

def _dtype_name(t):
    """The layer dtype of a tensor: bf16 or fp32 (anything else is refused,
    since the kernels would read it with the wrong element size)."""
    import torch
    if t.dtype == torch.bfloat16:
        return "bf16"
    if t.dtype == torch.float32:
        return "fp32"
    raise ValueError(f"expected a bfloat16 or float32 tensor, got {t.dtype}")


def _expect(name, t, shape, dtype):
    """Shape and dtype of a tensor handed to the library, checked before any
    pointer is taken: a mismatch would let a kernel read past a buffer."""
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name}: expected shape {tuple(shape)} and {dtype}, "
                         f"got {tuple(t.shape)} and {t.dtype}")


def _layer_dtype(desc):
    import torch
    return torch.bfloat16 if desc.dtype == MOE_BF16 else torch.float32


def _check_router(desc, X, W_r, bias):
    import torch
    dt = _layer_dtype(desc)
    _expect("X", X, (desc.T, desc.d), dt)
    _expect("W_r", W_r, (desc.d, desc.E), dt)
    if bias is not None:
        _expect("bias", bias, (desc.E,), torch.float32)


def _check_experts(desc, W_gate, W_up, W_down):
    dt = _layer_dtype(desc)
    _expect("W_gate", W_gate, (desc.E, desc.d, desc.n), dt)
    _expect("W_up", W_up, (desc.E, desc.d, desc.n), dt)
    _expect("W_down", W_down, (desc.E, desc.n, desc.d), dt)


def _desc_for(X, W_gate, K, capacity_factor):
    T, d = X.shape
    E, _, n = W_gate.shape
    return make_desc(T, d, E, K, n, _dtype_name(X), capacity_factor)


def workspace(desc: MoeDesc, entry: int, device="cuda"):
    import torch
    nbytes = max(16, moe_workspace_size(desc, entry))
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def route(X, W_r, K, bias=None, want_logits=False, n=64, split=True, flags=0):
    """Steps 1-2.  Returns (ids [T,K] int32, gates [T,K] fp32, logits [T,E] fp32 or None).
    split=True goes through moe_route_ws (k split for small batches, as
    moe_forward does); split=False through moe_route.  flags may carry
    MOE_FLAG_TOPK_THRESHOLD (the threshold selection)."""
    import torch
    T, d = X.shape
    E = W_r.shape[1]
    desc = make_desc(T, d, E, K, n, _dtype_name(X), flags=flags)
    _check_router(desc, X, W_r, bias)
    ids = torch.empty((T, K), dtype=torch.int32, device=X.device)
    gates = torch.empty((T, K), dtype=torch.float32, device=X.device)
    logits = torch.empty((T, E), dtype=torch.float32, device=X.device) if want_logits else None
    if split:
        moe_route_ws(desc, X, W_r, bias, logits, ids, gates, workspace(desc, MOE_WS_ROUTE, X.device))
    else:
        moe_route(desc, X, W_r, bias, logits, ids, gates)
    return ids, gates, logits


def route_permute(X, W_r, K, desc: MoeDesc, bias=None, want_logits=False):
    """Steps 1-5 through moe_route_permute.  Returns dict(ids, gates, logits or
    None, counts, offsets, raw_counts, perm_token, inv_slot)."""
    import torch
    if K != desc.K:
        raise ValueError(f"K = {K} differs from desc.K = {desc.K}")
    _check_router(desc, X, W_r, bias)
    dev = X.device
    T, E = desc.T, desc.E
    out = {
        "ids": torch.empty((T, K), dtype=torch.int32, device=dev),
        "gates": torch.empty((T, K), dtype=torch.float32, device=dev),
        "logits": torch.empty((T, E), dtype=torch.float32, device=dev) if want_logits else None,
        "counts": torch.empty(E, dtype=torch.int32, device=dev),
        "offsets": torch.empty(E + 1, dtype=torch.int32, device=dev),
        "raw_counts": torch.empty(E, dtype=torch.int32, device=dev),
        "perm_token": torch.full((max(1, T * K),), -1, dtype=torch.int32, device=dev),
        "inv_slot": torch.empty((T, K), dtype=torch.int32, device=dev),
    }
    moe_route_permute(desc, X, W_r, bias, out["logits"], out["ids"], out["gates"], out["counts"],
                      out["offsets"], out["raw_counts"], out["perm_token"], out["inv_slot"],
                      workspace(desc, MOE_WS_ROUTE_PERMUTE, dev))
    return out


def permute(desc: MoeDesc, ids):
    """Steps 3-5.  Returns dict(counts, offsets, raw_counts, perm_token, inv_slot)."""
    import torch
    dev = ids.device
    T, K, E = desc.T, desc.K, desc.E
    out = {
        "counts": torch.empty(E, dtype=torch.int32, device=dev),
        "offsets": torch.empty(E + 1, dtype=torch.int32, device=dev),
        "raw_counts": torch.empty(E, dtype=torch.int32, device=dev),
        "perm_token": torch.full((max(1, T * K),), -1, dtype=torch.int32, device=dev),
        "inv_slot": torch.empty((T, K), dtype=torch.int32, device=dev),
    }
    ws = workspace(desc, MOE_WS_PERMUTE, dev)
    moe_permute(desc, ids, out["counts"], out["offsets"], out["raw_counts"], out["perm_token"],
                out["inv_slot"], ws)
    return out


def round_tokens(desc: MoeDesc, ids, gates, meta):
    """Step 5b: tile-aware token rounding of ``permute``'s metadata, in place
    (counts, offsets, perm_token, inv_slot).  Returns meta."""
    ws = workspace(desc, MOE_WS_ROUND, ids.device)
    moe_round_tokens(desc, ids, gates, meta["counts"], meta["offsets"], meta["perm_token"],
                     meta["inv_slot"], ws)
    return meta


def grouped_ffn(desc: MoeDesc, X, offsets, perm_token, W_gate, W_up, W_down):
    """Steps 6-7.  Returns (H [rows_max, n], O [rows_max, d]); rows >= offsets[E] are unspecified."""
    import torch
    _expect("X", X, (desc.T, desc.d), _layer_dtype(desc))
    _check_experts(desc, W_gate, W_up, W_down)
    rows = max(1, moe_max_rows(desc))
    H = torch.empty((rows, desc.n), dtype=X.dtype, device=X.device)
    O = torch.empty((rows, desc.d), dtype=X.dtype, device=X.device)
    ws = workspace(desc, MOE_WS_GROUPED_FFN, X.device)
    moe_grouped_ffn(desc, X, offsets, perm_token, W_gate, W_up, W_down, H, O, ws)
    return H, O


def combine(desc: MoeDesc, O, gates, inv_slot):
    """Step 8.  Returns Y [T, d]."""
    import torch
    if O.dim() != 2 or O.shape[1] != desc.d or O.shape[0] < moe_max_rows(desc) \
            or O.dtype != _layer_dtype(desc):
        raise ValueError(f"O: expected at least {moe_max_rows(desc)} rows of {desc.d} "
                         f"{_layer_dtype(desc)}, got {tuple(O.shape)} {O.dtype}")
    _expect("gates", gates, (desc.T, desc.K), torch.float32)
    _expect("inv_slot", inv_slot, (desc.T, desc.K), torch.int32)
    Y = torch.empty((desc.T, desc.d), dtype=O.dtype, device=O.device)
    moe_combine(desc, O, gates, inv_slot, Y)
    return Y


def forward(X, W_r, W_gate, W_up, W_down, K, capacity_factor=0.0, bias=None, ws=None, flags=0):
    """Steps 1-8 in one library call.  Returns Y [T, d].  `flags` may pick the
    grouped-GEMM kernels (MOE_FLAG_GEMM_TILED / MOE_FLAG_GEMM_SKINNY)."""
    import torch
    desc = _desc_for(X, W_gate, K, capacity_factor)
    desc.flags = int(flags)
    _check_router(desc, X, W_r, bias)
    _check_experts(desc, W_gate, W_up, W_down)
    if ws is None:
        ws = workspace(desc, MOE_WS_FORWARD, X.device)
    Y = torch.empty_like(X)
    moe_forward(desc, X, W_r, bias, W_gate, W_up, W_down, Y, ws)
    return Y


def forward_train(X, W_r, W_gate, W_up, W_down, K, capacity_factor=0.0, bias=None, ws=None,
                  flags=0):
    """Training forward (bf16).  Returns (Y [T, d], saved, desc); pass saved and
    desc unchanged to ``backward``.  `flags` may carry MOE_FLAG_GEMM_TILED and
    MOE_FLAG_TOPK_THRESHOLD."""
    import torch
    desc = _desc_for(X, W_gate, K, capacity_factor)
    desc.flags = int(flags)
    _check_router(desc, X, W_r, bias)
    _check_experts(desc, W_gate, W_up, W_down)
    if ws is None:
        ws = workspace(desc, MOE_WS_FORWARD, X.device)
    saved = workspace(desc, MOE_WS_SAVED, X.device)
    Y = torch.empty_like(X)
    moe_forward_train(desc, X, W_r, bias, W_gate, W_up, W_down, Y, saved, ws)
    return Y, saved, desc


def saved_view(desc: MoeDesc, saved):
    """Typed views of the saved state's fields (no copies)."""
    import torch
    L = moe_saved_layout_of(desc)
    T, K, E, n = desc.T, desc.K, desc.E, desc.n
    rows = moe_max_rows(desc)

    def field(off, count, dtype, shape):
        item = torch.empty((), dtype=dtype).element_size()
        return saved[off: off + count * item].view(dtype).view(shape)

    return {
        "logits": field(L.logits, T * E, torch.float32, (T, E)),
        "ids": field(L.topk_ids, T * K, torch.int32, (T, K)),
        "gates": field(L.topk_gates, T * K, torch.float32, (T, K)),
        "inv_slot": field(L.inv_slot, T * K, torch.int32, (T, K)),
        "perm_token": field(L.perm_token, T * K, torch.int32, (T * K,)),
        "counts": field(L.counts, E, torch.int32, (E,)),
        "offsets": field(L.offsets, E + 1, torch.int32, (E + 1,)),
        "preact": field(L.preact, rows * 2 * n, torch.bfloat16, (rows, 2 * n)),
    }


def backward(desc: MoeDesc, saved, X, W_r, W_gate, W_up, W_down, dY, ws=None):
    """Gradients of sum(Y * dY) after ``forward_train``.  Returns dict(dX bf16,
    dW_r, dW_gate, dW_up, dW_down fp32)."""
    import torch
    dev = X.device
    T, d, E, n = desc.T, desc.d, desc.E, desc.n
    _check_router(desc, X, W_r, None)
    _check_experts(desc, W_gate, W_up, W_down)
    _expect("dY", dY, (T, d), _layer_dtype(desc))
    if ws is None:
        ws = workspace(desc, MOE_WS_BACKWARD, dev)
    out = {
        "dX": torch.empty((T, d), dtype=X.dtype, device=dev),
        "dW_r": torch.empty((d, E), dtype=torch.float32, device=dev),
        "dW_gate": torch.empty((E, d, n), dtype=torch.float32, device=dev),
        "dW_up": torch.empty((E, d, n), dtype=torch.float32, device=dev),
        "dW_down": torch.empty((E, n, d), dtype=torch.float32, device=dev),
    }
    moe_backward(desc, X, W_r, W_gate, W_up, W_down, dY, saved, out["dX"], out["dW_r"],
                 out["dW_gate"], out["dW_up"], out["dW_down"], ws)
    return out


# ---------------------------------------------------------------- atomic experts

def moe_omni_validate(desc: MoeOmniDesc) -> int:
    return lib().moe_omni_validate(ctypes.byref(desc))


def moe_omni_workspace_size(desc: MoeOmniDesc, entry: int) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().moe_omni_workspace_size(ctypes.byref(desc), int(entry), ctypes.byref(out)),
           "moe_omni_workspace_size")
    return out.value


def moe_omni_route(desc, X, W_r, W_c, ls_r, ls_c, ids, gates, ws, stream=None):
    _check(lib().moe_omni_route(ctypes.byref(desc), _p(X), _p(W_r), _p(W_c), _p(ls_r), _p(ls_c),
                                _p(ids), _p(gates), _p(ws), _nbytes(ws), _stream(stream)),
           "moe_omni_route")


def moe_omni_permute(desc, ids, counts, offsets, perm_token, inv_slot, ws, stream=None):
    _check(lib().moe_omni_permute(ctypes.byref(desc), _p(ids), _p(counts), _p(offsets),
                                  _p(perm_token), _p(inv_slot), _p(ws), _nbytes(ws),
                                  _stream(stream)), "moe_omni_permute")


def moe_omni_forward(desc, X, W_r, W_c, W_in, W_out, Y, ws, stream=None):
    _check(lib().moe_omni_forward(ctypes.byref(desc), _p(X), _p(W_r), _p(W_c), _p(W_in),
                                  _p(W_out), _p(Y), _p(ws), _nbytes(ws), _stream(stream)),
           "moe_omni_forward")


def _omni_desc_for(X, W_r, W_c, K, W_in=None, W_out=None):
    """The layer's description, with every tensor's shape and dtype checked
    (bf16: X[T,d], W_r[d,Nr], W_c[d,Nc], W_in/W_out[Nr*Nc, d])."""
    import torch
    T, d = X.shape
    Nr, Nc = W_r.shape[1], W_c.shape[1]
    bf = torch.bfloat16
    _expect("X", X, (T, d), bf)
    _expect("W_r", W_r, (d, Nr), bf)
    _expect("W_c", W_c, (d, Nc), bf)
    if W_in is not None or W_out is not None:
        _expect("W_in", W_in, (Nr * Nc, d), bf)
        _expect("W_out", W_out, (Nr * Nc, d), bf)
    return make_omni_desc(T, d, Nr, Nc, K)


def _omni_ws(desc, entry, device):
    import torch
    return torch.empty(max(16, moe_omni_workspace_size(desc, entry)), dtype=torch.uint8,
                       device=device)


def omni_route(X, W_r, W_c, K):
    """Atomic-expert router.  Returns (ids [T,K], gates [T,K], ls_r [T,Nr], ls_c [T,Nc])."""
    import torch
    desc = _omni_desc_for(X, W_r, W_c, K)
    T, dev = X.shape[0], X.device
    ids = torch.empty((T, K), dtype=torch.int32, device=dev)
    gates = torch.empty((T, K), dtype=torch.float32, device=dev)
    ls_r = torch.empty((T, W_r.shape[1]), dtype=torch.float32, device=dev)
    ls_c = torch.empty((T, W_c.shape[1]), dtype=torch.float32, device=dev)
    moe_omni_route(desc, X, W_r, W_c, ls_r, ls_c, ids, gates, _omni_ws(desc, MOE_OMNI_WS_ROUTE, dev))
    return ids, gates, ls_r, ls_c


def omni_permute(desc: MoeOmniDesc, ids):
    """(expert, token) order over the N experts: dict(counts, offsets, perm_token, inv_slot)."""
    import torch
    _expect("ids", ids, (desc.T, desc.K), torch.int32)
    dev = ids.device
    N = desc.Nr * desc.Nc
    out = {
        "counts": torch.empty(N, dtype=torch.int32, device=dev),
        "offsets": torch.empty(N + 1, dtype=torch.int32, device=dev),
        "perm_token": torch.empty(max(1, desc.T * desc.K), dtype=torch.int32, device=dev),
        "inv_slot": torch.empty((desc.T, desc.K), dtype=torch.int32, device=dev),
    }
    moe_omni_permute(desc, ids, out["counts"], out["offsets"], out["perm_token"], out["inv_slot"],
                     _omni_ws(desc, MOE_OMNI_WS_PERMUTE, dev))
    return out


def omni_forward(X, W_r, W_c, W_in, W_out, K, ws=None):
    """The atomic-expert layer in one library call.  Returns Y [T, d]."""
    import torch
    desc = _omni_desc_for(X, W_r, W_c, K, W_in, W_out)
    if ws is None:
        ws = _omni_ws(desc, MOE_OMNI_WS_FORWARD, X.device)
    Y = torch.empty_like(X)
    moe_omni_forward(desc, X, W_r, W_c, W_in, W_out, Y, ws)
    return Y
