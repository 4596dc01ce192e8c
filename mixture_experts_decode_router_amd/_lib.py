"""ctypes binding of libmoe_mi355x.so (include/moe.h), argument marshalling only.

Every function here has the name of the C entry point it calls and does no
arithmetic of the block: it turns torch device tensors (or raw integer device
pointers) and streams into the C arguments, calls the library, and raises
MoEError on a non-OK status.  If the library is not built, `lib()` raises: the
block has no other implementation to fall back to.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, Structure, c_char_p, c_int32, c_size_t, c_void_p

import numpy as np

LIB_NAME = "libmoe_mi355x.so"
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), LIB_NAME)

MOE_OK = 0
MOE_ERR_INVALID_ARG = 1
MOE_ERR_UNSUPPORTED = 2
MOE_ERR_WORKSPACE = 3
MOE_ERR_NOT_CAPTURABLE = 4
MOE_ERR_CAPTURE_VIOLATION = 5
MOE_ERR_HIP = 6

MOE_W_BF16 = 0
MOE_W_NF4_B64 = 1
MOE_W_BF16_TILED = 2
MOE_W_NF4_B64_TILED = 3
MOE_OUT_F32 = 0
MOE_OUT_BF16 = 1
MOE_TOPK_RENORM = 0
MOE_TOPK_SOFTMAX = 1

# every entry point include/moe.h declares
EXPORTS = (
    "moe_status_str", "moe_last_error", "moe_config_check", "moe_workspace_size",
    "moe_route", "moe_permute", "moe_forward", "moe_forward_timed", "moe_pack_weights",
    "moe_workspace_views",
    "moe_read_counts", "moe_graph_capture", "moe_graph_replay", "moe_graph_bucket_for",
    "moe_graph_destroy", "moe_forward_prenorm", "moe_graph_capture_prenorm",
    "moe_backward", "moe_forward_noalloc", "moe_probe_read", "moe_probe_mfma", "moe_probe_gather",
)


class moe_config(Structure):
    _fields_ = [("hidden", c_int32), ("inter", c_int32), ("n_experts", c_int32),
                ("top_k", c_int32), ("t_max", c_int32), ("wfmt", c_int32),
                ("out_dtype", c_int32), ("topk_weights", c_int32), ("train", c_int32)]


class moe_lora(Structure):
    _fields_ = [("a_gate_up", c_void_p), ("b_gate_up", c_void_p), ("a_down", c_void_p), ("b_down", c_void_p),
                ("scale", ctypes.c_float), ("rank", c_int32)]


class moe_weights(Structure):
    _fields_ = [("w_router", c_void_p), ("router_bias", c_void_p), ("w_gate_up", c_void_p),
                ("w_down", c_void_p), ("q_gate_up", c_void_p), ("s_gate_up", c_void_p),
                ("q_down", c_void_p), ("s_down", c_void_p), ("codebook", c_void_p),
                ("lora", c_void_p)]   # host pointer to a moe_lora, or None


class moe_lora_grads(Structure):
    _fields_ = [("d_a_gate_up", c_void_p), ("d_b_gate_up", c_void_p), ("d_a_down", c_void_p),
                ("d_b_down", c_void_p)]


class moe_weight_grads(Structure):
    _fields_ = [("d_w_gate_up", c_void_p), ("d_w_down", c_void_p)]


class moe_prenorm(Structure):
    _fields_ = [("residual", c_void_p), ("delta", c_void_p), ("gamma", c_void_p), ("eps", ctypes.c_float),
                ("residual_out", c_void_p), ("x_out", c_void_p)]


class moe_views(Structure):
    _fields_ = [("topk_ids", c_void_p), ("topk_w", c_void_p), ("counts", c_void_p),
                ("offsets", c_void_p), ("perm", c_void_p), ("pos", c_void_p)]


class MoEError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load the HIP library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is not built; build it with "
            "`python -m mixture_experts_decode_router_amd.build` (hipcc, gfx950)")
    L = ctypes.CDLL(LIB_PATH)
    S = c_int32  # moe_status
    sig = {
        "moe_status_str": (c_char_p, [c_int32]),
        "moe_last_error": (c_char_p, []),
        "moe_config_check": (S, [POINTER(moe_config)]),
        "moe_workspace_size": (c_size_t, [POINTER(moe_config)]),
        "moe_route": (S, [POINTER(moe_config), POINTER(moe_weights), c_void_p, c_int32,
                          c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
        "moe_permute": (S, [POINTER(moe_config), c_void_p, c_int32, c_void_p, c_void_p,
                            c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
        "moe_forward": (S, [POINTER(moe_config), POINTER(moe_weights), c_void_p, c_int32,
                            c_void_p, c_void_p, c_size_t, c_void_p]),
        "moe_forward_noalloc": (S, [POINTER(moe_config), POINTER(moe_weights), c_void_p, c_int32,
                                    c_void_p, c_void_p]),
        "moe_probe_read": (S, [c_void_p, c_size_t, c_void_p, c_int32, c_void_p]),
        "moe_probe_mfma": (S, [c_void_p, c_int32, c_int32, c_int32, c_void_p]),
        "moe_probe_gather": (S, [c_void_p, c_size_t, c_int32, c_int32, c_int32, c_void_p, c_int32, c_void_p]),
        "moe_forward_timed": (S, [POINTER(moe_config), POINTER(moe_weights), c_void_p, c_int32,
                                  c_void_p, c_void_p, c_size_t, c_void_p, POINTER(c_void_p)]),
        "moe_pack_weights": (S, [POINTER(moe_config), POINTER(moe_weights), POINTER(moe_weights), c_void_p]),
        "moe_workspace_views": (S, [POINTER(moe_config), c_void_p, c_size_t, POINTER(moe_views)]),
        "moe_read_counts": (S, [POINTER(moe_config), c_void_p, c_size_t, c_void_p, c_void_p]),
        "moe_graph_capture": (S, [POINTER(moe_config), POINTER(moe_weights), c_void_p, c_int32,
                                  c_void_p, c_void_p, c_void_p, c_size_t, c_void_p,
                                  POINTER(c_void_p)]),
        "moe_graph_replay": (S, [c_void_p, c_int32, c_void_p]),
        "moe_graph_bucket_for": (c_int32, [c_void_p, c_int32]),
        "moe_graph_destroy": (None, [c_void_p]),
        "moe_backward": (S, [POINTER(moe_config), POINTER(moe_weights), c_void_p, c_int32, c_void_p, c_void_p,
                             c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
        "moe_forward_prenorm": (S, [POINTER(moe_config), POINTER(moe_weights), POINTER(moe_prenorm), c_int32,
                                    c_void_p, c_void_p, c_size_t, c_void_p]),
        "moe_graph_capture_prenorm": (S, [POINTER(moe_config), POINTER(moe_weights), c_void_p, c_int32,
                                          POINTER(moe_prenorm), c_void_p, c_void_p, c_size_t, c_void_p,
                                          POINTER(c_void_p)]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


def _check(status: int) -> None:
    if status != MOE_OK:
        L = lib()
        raise MoEError(status, f"{L.moe_status_str(status).decode()}: {L.moe_last_error().decode()}")


def ptr(t) -> int | None:
    """Device pointer of a torch tensor (or pass an int / None through)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    return t.data_ptr()


def stream_handle(stream) -> int | None:
    """hipStream_t of a torch stream (None -> torch's current stream)."""
    if isinstance(stream, int):
        return stream
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def moe_status_str(status: int) -> str:
    return lib().moe_status_str(status).decode()


def moe_last_error() -> str:
    return lib().moe_last_error().decode()


def moe_config_check(cfg: moe_config) -> int:
    return lib().moe_config_check(ctypes.byref(cfg))


def moe_workspace_size(cfg: moe_config) -> int:
    return lib().moe_workspace_size(ctypes.byref(cfg))


def moe_route(cfg, w, x, T, topk_ids, topk_w, logits, workspace, ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().moe_route(ctypes.byref(cfg), ctypes.byref(w), ptr(x), T, ptr(topk_ids),
                           ptr(topk_w), ptr(logits), ptr(workspace), ws_bytes, stream_handle(stream)))


def moe_permute(cfg, topk_ids, T, counts, offsets, perm, pos, workspace, ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().moe_permute(ctypes.byref(cfg), ptr(topk_ids), T, ptr(counts), ptr(offsets),
                             ptr(perm), ptr(pos), ptr(workspace), ws_bytes, stream_handle(stream)))


def moe_forward(cfg, w, x, T, out, workspace, ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().moe_forward(ctypes.byref(cfg), ctypes.byref(w), ptr(x), T, ptr(out),
                             ptr(workspace), ws_bytes, stream_handle(stream)))


def moe_forward_noalloc(cfg, w, x, T, out, stream=None):
    _check(lib().moe_forward_noalloc(ctypes.byref(cfg), ctypes.byref(w), ptr(x), T, ptr(out),
                                     stream_handle(stream)))


def moe_probe_read(src, nbytes, sink, n_wg, stream=None):
    _check(lib().moe_probe_read(ptr(src), nbytes, ptr(sink), n_wg, stream_handle(stream)))


def moe_probe_mfma(sink, n_wg, iters, shape, stream=None):
    _check(lib().moe_probe_mfma(ptr(sink), n_wg, iters, shape, stream_handle(stream)))


def moe_probe_gather(src, nbytes, row_bytes, order, iters, sink, n_wg, stream=None):
    _check(lib().moe_probe_gather(ptr(src), nbytes, row_bytes, order, iters, ptr(sink), n_wg, stream_handle(stream)))


def make_prenorm(residual, delta, gamma, eps, residual_out, x_out) -> moe_prenorm:
    return moe_prenorm(ptr(residual), ptr(delta), ptr(gamma), float(eps), ptr(residual_out), ptr(x_out))


def moe_forward_prenorm(cfg, w, pn, T, out, workspace, ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().moe_forward_prenorm(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(pn), T, ptr(out),
                                     ptr(workspace), ws_bytes, stream_handle(stream)))


def make_lora_grads(d_a_gate_up, d_b_gate_up, d_a_down, d_b_down) -> moe_lora_grads:
    return moe_lora_grads(ptr(d_a_gate_up), ptr(d_b_gate_up), ptr(d_a_down), ptr(d_b_down))


def moe_backward(cfg, w, x, T, d_out, d_x, d_topk_w, workspace, ws_bytes=None, stream=None, d_lora=None,
                 d_weights=None):
    """d_lora: a moe_lora_grads (make_lora_grads) when w carries adapters, else
    None; d_weights: a moe_weight_grads for the expert-weight gradients, or None."""
    if ws_bytes is None:
        ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().moe_backward(ctypes.byref(cfg), ctypes.byref(w), ptr(x), T, ptr(d_out), ptr(d_x), ptr(d_topk_w),
                              None if d_lora is None else ctypes.byref(d_lora),
                              None if d_weights is None else ctypes.byref(d_weights),
                              ptr(workspace), ws_bytes, stream_handle(stream)))


def moe_forward_timed(cfg, w, x, T, out, workspace, ws_bytes, stream, events):
    """`events`: six raw hipEvent_t handles (ints), see hip_events()."""
    arr = (c_void_p * 6)(*events)
    _check(lib().moe_forward_timed(ctypes.byref(cfg), ctypes.byref(w), ptr(x), T, ptr(out),
                                   ptr(workspace), ws_bytes, stream_handle(stream), arr))


def moe_pack_weights(cfg, src, dst, stream=None):
    _check(lib().moe_pack_weights(ctypes.byref(cfg), ctypes.byref(src), ctypes.byref(dst),
                                  stream_handle(stream)))


def moe_workspace_views(cfg, workspace, ws_bytes=None) -> moe_views:
    if ws_bytes is None:
        ws_bytes = workspace.numel() * workspace.element_size()
    v = moe_views()
    _check(lib().moe_workspace_views(ctypes.byref(cfg), ptr(workspace), ws_bytes, ctypes.byref(v)))
    return v


def moe_read_counts(cfg, workspace, ws_bytes=None, stream=None) -> np.ndarray:
    if ws_bytes is None:
        ws_bytes = workspace.numel() * workspace.element_size()
    out = np.zeros(cfg.n_experts, dtype=np.int32)
    _check(lib().moe_read_counts(ctypes.byref(cfg), ptr(workspace), ws_bytes,
                                 out.ctypes.data_as(c_void_p), stream_handle(stream)))
    return out


def moe_graph_capture(cfg, w, buckets, x_static, out_static, workspace, ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = workspace.numel() * workspace.element_size()
    b = (c_int32 * len(buckets))(*buckets)
    g = c_void_p()
    _check(lib().moe_graph_capture(ctypes.byref(cfg), ctypes.byref(w), b, len(buckets), ptr(x_static),
                                   ptr(out_static), ptr(workspace), ws_bytes, stream_handle(stream),
                                   ctypes.byref(g)))
    return g.value


def moe_graph_capture_prenorm(cfg, w, buckets, pn_static, out_static, workspace, ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = workspace.numel() * workspace.element_size()
    b = (c_int32 * len(buckets))(*buckets)
    g = c_void_p()
    _check(lib().moe_graph_capture_prenorm(ctypes.byref(cfg), ctypes.byref(w), b, len(buckets),
                                           ctypes.byref(pn_static), ptr(out_static), ptr(workspace), ws_bytes,
                                           stream_handle(stream), ctypes.byref(g)))
    return g.value


def moe_graph_replay(graph, T, stream=None):
    _check(lib().moe_graph_replay(graph, T, stream_handle(stream)))


def moe_graph_bucket_for(graph, T) -> int:
    return lib().moe_graph_bucket_for(graph, T)


def moe_graph_destroy(graph) -> None:
    lib().moe_graph_destroy(graph)


# ---------------------------------------------------------------- HIP events
_hip = None


def _hiprt():
    global _hip
    if _hip is None:
        h = ctypes.CDLL("libamdhip64.so")
        h.hipEventCreate.argtypes = [POINTER(c_void_p)]
        h.hipEventCreateWithFlags.argtypes = [POINTER(c_void_p), ctypes.c_uint]
        h.hipEventDestroy.argtypes = [c_void_p]
        h.hipEventSynchronize.argtypes = [c_void_p]
        h.hipEventElapsedTime.argtypes = [POINTER(ctypes.c_float), c_void_p, c_void_p]
        h.hipEventRecord.argtypes = [c_void_p, c_void_p]
        _hip = h
    return _hip


HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000
HIP_EVENT_RELEASE_TO_DEVICE = 0x40000000


def hip_events(n: int, flags: int = 0) -> list[int]:
    """n raw hipEvent_t handles (caller destroys them with hip_events_destroy).
    flags: hipEventCreateWithFlags flags, e.g. HIP_EVENT_RELEASE_TO_DEVICE for
    timing events whose record should not write back caches to the system."""
    h = _hiprt()
    out = []
    for _ in range(n):
        e = c_void_p()
        if h.hipEventCreateWithFlags(ctypes.byref(e), ctypes.c_uint(flags)) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        out.append(e.value)
    return out


def hip_event_record(ev: int, stream=None) -> None:
    if _hiprt().hipEventRecord(ev, stream_handle(stream)) != 0:
        raise RuntimeError("hipEventRecord failed")


def hip_event_elapsed_ms(a: int, b: int) -> float:
    h = _hiprt()
    if h.hipEventSynchronize(b) != 0:
        raise RuntimeError("hipEventSynchronize failed")
    ms = ctypes.c_float()
    if h.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
        raise RuntimeError("hipEventElapsedTime failed")
    return ms.value


def hip_events_destroy(evs) -> None:
    h = _hiprt()
    for e in evs:
        h.hipEventDestroy(e)
