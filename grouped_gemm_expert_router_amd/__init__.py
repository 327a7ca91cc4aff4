"""Python binding of libmoe.so, the MI355X dropless MoE layer (see include/moe.h).

Argument marshalling only: every step of the layer runs in the library's HIP kernels.  PyTorch
provides device memory and the current HIP stream.  Importing this package does not need a GPU;
calling an entry point without the built library raises (there is no fallback path).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe.so")

MOE_BF16, MOE_FP8_E4M3, MOE_MXFP8 = 0, 1, 2
MOE_WS_ROUTE, MOE_WS_FORWARD, MOE_WS_BACKWARD, MOE_WS_ROUTER = 0, 1, 2, 3
MOE_OK, MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_DTYPE, MOE_ERR_WORKSPACE, MOE_ERR_HIP, MOE_ERR_ALIGN = 0, -1, -2, -3, -4, -5, -6

ENTRY_POINTS = ("moe_workspace_bytes", "moe_saved_bytes", "moe_route", "moe_route_noalloc", "moe_plan",
                "moe_forward", "moe_forward_fused", "moe_backward", "moe_router_logits", "moe_router_backward",
                "moe_permute", "moe_combine", "moe_mxfp8_quantize", "moe_mxfp8_quantize_weights", "moe_set_stage_hook",
                "moe_status_string")


class MoeDims(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("d", ctypes.c_int64), ("f", ctypes.c_int64), ("E", ctypes.c_int64),
                ("k", ctypes.c_int64), ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32)]

    def __repr__(self):
        return f"MoeDims(T={self.T}, d={self.d}, f={self.f}, E={self.E}, k={self.k}, dtype={self.dtype})"


# void hook(const char* stage, int begin, void* stream, void* user)
STAGE_HOOK = ctypes.CFUNCTYPE(None, ctypes.c_char_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p)


class MoEError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} failed with status {status}: {text}")
        self.status = status


_lib = None


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libmoe.so (built in-tree by grouped_gemm_expert_router_amd.build)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m grouped_gemm_expert_router_amd.build`")
    lib = ctypes.CDLL(p)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    dp = ctypes.POINTER(MoeDims)
    lib.moe_workspace_bytes.argtypes = [dp, i32, ctypes.POINTER(sz)]
    lib.moe_saved_bytes.argtypes = [dp, ctypes.POINTER(sz)]
    lib.moe_route.argtypes = [dp] + [vp] * 8 + [sz, vp]
    lib.moe_route_noalloc.argtypes = [dp] + [vp] * 7 + [vp]
    lib.moe_plan.argtypes = [dp] + [vp] * 6 + [sz, vp]
    lib.moe_forward.argtypes = [dp] + [vp] * 13 + [sz, vp]
    lib.moe_forward_fused.argtypes = [dp] + [vp] * 10 + [sz, vp]
    lib.moe_backward.argtypes = [dp] + [vp] * 19 + [sz, vp]
    lib.moe_router_logits.argtypes = [dp, vp, vp, vp, vp]
    lib.moe_router_backward.argtypes = [dp] + [vp] * 6 + [sz, vp]
    lib.moe_permute.argtypes = [dp, vp, vp, vp, vp]
    lib.moe_combine.argtypes = [dp, vp, vp, vp, vp]
    lib.moe_mxfp8_quantize.argtypes = [vp, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, i32, vp, vp, vp]
    lib.moe_mxfp8_quantize_weights.argtypes = [vp, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64] + [vp] * 5
    lib.moe_set_stage_hook.argtypes = [STAGE_HOOK, vp]
    lib.moe_status_string.argtypes = [i32]
    lib.moe_status_string.restype = ctypes.c_char_p
    for name in ENTRY_POINTS[:-1]:
        getattr(lib, name).restype = i32
    if path is None:
        _lib = lib
    return lib


def dims(T: int, d: int, f: int, E: int, k: int, dtype: int = MOE_BF16) -> MoeDims:
    return MoeDims(T, d, f, E, k, dtype, 0)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn: str, rc: int) -> None:
    if rc != MOE_OK:
        raise MoEError(fn, rc, load_library().moe_status_string(rc).decode())


def status_string(status: int) -> str:
    return load_library().moe_status_string(status).decode()


def moe_workspace_bytes(dm: MoeDims, which: int) -> int:
    out = ctypes.c_size_t(0)
    _check("moe_workspace_bytes", load_library().moe_workspace_bytes(ctypes.byref(dm), which, ctypes.byref(out)))
    return out.value


def moe_saved_bytes(dm: MoeDims) -> int:
    out = ctypes.c_size_t(0)
    _check("moe_saved_bytes", load_library().moe_saved_bytes(ctypes.byref(dm), ctypes.byref(out)))
    return out.value


def moe_route(dm, logits, topk_ids, topk_w, counts, offsets, perm, inv_perm, ws, ws_bytes=None, stream=None):
    nb = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check("moe_route", load_library().moe_route(
        ctypes.byref(dm), _ptr(logits), _ptr(topk_ids), _ptr(topk_w), _ptr(counts), _ptr(offsets), _ptr(perm),
        _ptr(inv_perm), _ptr(ws), nb, _stream(stream)))


def moe_route_noalloc(dm, logits, topk_ids, topk_w, counts, offsets, perm, inv_perm, stream=None):
    _check("moe_route_noalloc", load_library().moe_route_noalloc(
        ctypes.byref(dm), _ptr(logits), _ptr(topk_ids), _ptr(topk_w), _ptr(counts), _ptr(offsets), _ptr(perm),
        _ptr(inv_perm), _stream(stream)))


def moe_plan(dm, topk_ids, counts, offsets, perm, inv_perm, ws, ws_bytes=None, stream=None):
    nb = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check("moe_plan", load_library().moe_plan(
        ctypes.byref(dm), _ptr(topk_ids), _ptr(counts), _ptr(offsets), _ptr(perm), _ptr(inv_perm), _ptr(ws), nb,
        _stream(stream)))


def moe_forward(dm, x, x_scale, W1, W1_scale, W2, W2_scale, topk_w, offsets, perm, inv_perm, y, saved, ws,
                ws_bytes=None, stream=None):
    nb = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check("moe_forward", load_library().moe_forward(
        ctypes.byref(dm), _ptr(x), _ptr(x_scale), _ptr(W1), _ptr(W1_scale), _ptr(W2), _ptr(W2_scale), _ptr(topk_w),
        _ptr(offsets), _ptr(perm), _ptr(inv_perm), _ptr(y), _ptr(saved), _ptr(ws), nb, _stream(stream)))


def moe_forward_fused(dm, x, W1, W2, topk_w, offsets, perm, inv_perm, y, saved, ws, ws_bytes=None, stream=None):
    nb = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check("moe_forward_fused", load_library().moe_forward_fused(
        ctypes.byref(dm), _ptr(x), _ptr(W1), _ptr(W2), _ptr(topk_w), _ptr(offsets), _ptr(perm), _ptr(inv_perm),
        _ptr(y), _ptr(saved), _ptr(ws), nb, _stream(stream)))


def moe_backward(dm, dy, x, x_scale, W1, W1_scale, W2, W2_scale, topk_ids, topk_w, offsets, perm, inv_perm, saved,
                 dx, dW1, dW2, d_topk_w, d_logits, ws, ws_bytes=None, stream=None):
    nb = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check("moe_backward", load_library().moe_backward(
        ctypes.byref(dm), _ptr(dy), _ptr(x), _ptr(x_scale), _ptr(W1), _ptr(W1_scale), _ptr(W2), _ptr(W2_scale),
        _ptr(topk_ids), _ptr(topk_w), _ptr(offsets), _ptr(perm), _ptr(inv_perm), _ptr(saved), _ptr(dx), _ptr(dW1),
        _ptr(dW2), _ptr(d_topk_w), _ptr(d_logits), _ptr(ws), nb, _stream(stream)))


def moe_router_logits(dm, x, Wg, logits, stream=None):
    _check("moe_router_logits", load_library().moe_router_logits(ctypes.byref(dm), _ptr(x), _ptr(Wg), _ptr(logits),
                                                                 _stream(stream)))


def moe_router_backward(dm, x, Wg, d_logits, dx, dWg, ws, ws_bytes=None, stream=None):
    nb = (ws.numel() * ws.element_size() if ws is not None else 0) if ws_bytes is None else ws_bytes
    _check("moe_router_backward", load_library().moe_router_backward(
        ctypes.byref(dm), _ptr(x), _ptr(Wg), _ptr(d_logits), _ptr(dx), _ptr(dWg), _ptr(ws), nb, _stream(stream)))


def moe_permute(dm, x, inv_perm, xp, stream=None):
    _check("moe_permute", load_library().moe_permute(ctypes.byref(dm), _ptr(x), _ptr(inv_perm), _ptr(xp),
                                                     _stream(stream)))


def moe_combine(dm, op, inv_perm, y, stream=None):
    _check("moe_combine", load_library().moe_combine(ctypes.byref(dm), _ptr(op), _ptr(inv_perm), _ptr(y),
                                                     _stream(stream)))


def moe_mxfp8_quantize(src, batch, rows, cols, block_axis, codes, exps, stream=None):
    _check("moe_mxfp8_quantize", load_library().moe_mxfp8_quantize(_ptr(src), batch, rows, cols, block_axis,
                                                                   _ptr(codes), _ptr(exps), _stream(stream)))


def moe_mxfp8_quantize_weights(src, batch, rows, cols, col_codes, col_exps, row_codes, row_words, stream=None):
    _check("moe_mxfp8_quantize_weights",
           load_library().moe_mxfp8_quantize_weights(_ptr(src), batch, rows, cols, _ptr(col_codes), _ptr(col_exps),
                                                     _ptr(row_codes), _ptr(row_words), _stream(stream)))


_hook_ref = None


def moe_set_stage_hook(fn) -> None:
    """Install fn(stage: str, begin: bool, stream_ptr: int) as the library's profiling hook
    (None removes it).  The ctypes callback object is kept alive here."""
    global _hook_ref
    if fn is None:
        _hook_ref = None
        _check("moe_set_stage_hook", load_library().moe_set_stage_hook(STAGE_HOOK(), None))
        return

    def tramp(stage, begin, stream, user):
        fn(stage.decode(), bool(begin), stream or 0)

    _hook_ref = STAGE_HOOK(tramp)
    _check("moe_set_stage_hook", load_library().moe_set_stage_hook(_hook_ref, None))


# ------------------------------------------------------------------ buffer helpers (torch)
def alloc_layer_buffers(dm: MoeDims, device="cuda", backward: bool = True) -> dict:
    """Device buffers for one route/plan -> forward (-> backward) round, sized by the library."""
    import torch
    T, d, f, E, k = dm.T, dm.d, dm.f, dm.E, dm.k
    A = T * k
    i32 = dict(dtype=torch.int32, device=device)
    b = {
        "topk_ids": torch.empty((T, k), **i32),
        "topk_w": torch.empty((T, k), dtype=torch.float32, device=device),
        "counts": torch.empty((E,), **i32),
        "offsets": torch.empty((E + 1,), **i32),
        "perm": torch.empty((max(A, 1),), **i32),
        "inv_perm": torch.empty((max(A, 1),), **i32),
        "ws_route": torch.empty((max(moe_workspace_bytes(dm, MOE_WS_ROUTE), 256),), dtype=torch.uint8, device=device),
        "y": torch.empty((T, d), dtype=torch.bfloat16, device=device),
        "saved": torch.empty((max(moe_saved_bytes(dm), 256),), dtype=torch.uint8, device=device),
        "ws_fwd": torch.empty((max(moe_workspace_bytes(dm, MOE_WS_FORWARD), 256),), dtype=torch.uint8, device=device),
    }
    if backward:
        b.update({
            "dx": torch.empty((T, d), dtype=torch.bfloat16, device=device),
            "dW1": torch.empty((E, d, 2 * f), dtype=torch.bfloat16, device=device),
            "dW2": torch.empty((E, f, d), dtype=torch.bfloat16, device=device),
            "d_topk_w": torch.empty((T, k), dtype=torch.float32, device=device),
            "d_logits": torch.empty((T, E), dtype=torch.float32, device=device),
            "ws_bwd": torch.empty((max(moe_workspace_bytes(dm, MOE_WS_BACKWARD), 256),), dtype=torch.uint8,
                                  device=device),
        })
    return b


__all__ = ["MoeDims", "MoEError", "dims", "load_library", "status_string", "moe_workspace_bytes", "moe_saved_bytes",
           "moe_route", "moe_route_noalloc", "moe_plan", "moe_forward", "moe_forward_fused", "moe_backward",
           "moe_router_logits",
           "moe_router_backward", "moe_permute", "moe_combine",
           "moe_mxfp8_quantize", "moe_mxfp8_quantize_weights", "moe_set_stage_hook", "alloc_layer_buffers",
           "ENTRY_POINTS", "MOE_BF16",
           "MOE_FP8_E4M3", "MOE_MXFP8", "MOE_WS_ROUTE", "MOE_WS_FORWARD",
           "MOE_WS_BACKWARD", "MOE_WS_ROUTER", "MOE_OK", "MOE_ERR_NULL", "MOE_ERR_SHAPE", "MOE_ERR_DTYPE", "MOE_ERR_WORKSPACE",
           "MOE_ERR_HIP", "MOE_ERR_ALIGN"]
