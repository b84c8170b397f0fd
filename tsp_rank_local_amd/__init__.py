"""Python binding of libtsp.so, the rank-local TSP layer forward for MI355X.

Argument marshalling only: every step of the layer runs in the library's HIP
kernels. Functions carry the C names and take torch tensors (device memory)
or raw integer pointers; they enqueue on the current torch stream unless a
stream is given, and raise TspError on a non-OK status.

The library must have been built (python -m tsp_rank_local_amd.build); there
is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

__all__ = [
    "TspError", "TspShape", "TspLayerWeights", "lib", "make_shape", "workspace_size",
    "tsp_zigzag_index_host", "tsp_zigzag_index", "tsp_zigzag_attn", "tsp_zigzag_attn_ex", "tsp_mlp_ring",
    "tsp_mlp_ring_bwd", "tsp_zigzag_attn_bwd", "tsp_zigzag_attn_bwd_noalloc", "tsp_zigzag_attn_lse",
    "tsp_zigzag_attn_bwd_lse", "tsp_zigzag_attn_bwd_ex", "tsp_layer_fwd", "tsp_layer_bwd", "tsp_mlp_ring_z",
    "tsp_mlp_ring_bwd_z", "tsp_layer_fwd_save", "tsp_layer_bwd_ex", "profile_enable",
    "profile_reset", "profile_read", "TspLayerGrads",
    "TSP_F32", "TSP_BF16", "TSP_ATTN_Q_LOG2_SCALED", "TSP_PHASE_KV", "TSP_PHASE_REST", "TSP_PHASE_ALL",
    "TSP_WS_MLP", "TSP_WS_LAYER", "TSP_WS_MLP_BWD", "TSP_WS_ATTN_BWD", "TSP_WS_LAYER_BWD", "TSP_BWD_ATTN", "TSP_BWD_QKV",
    "TSP_BWD_ALL", "TSP_ATTN_BWD_PLAIN_PDS", "TSP_MLP_GELU", "TSP_MLP_SWIGLU", "MLP_KINDS",
    "KERNEL_CLASSES", "EXPORTED_SYMBOLS",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtsp.so")

TSP_OK, TSP_ERR_INVALID_ARG, TSP_ERR_UNSUPPORTED, TSP_ERR_WORKSPACE, TSP_ERR_HIP = range(5)
TSP_F32, TSP_BF16 = 0, 1
TSP_PHASE_KV, TSP_PHASE_REST, TSP_PHASE_ALL = 1, 2, 3
TSP_WS_MLP, TSP_WS_LAYER, TSP_WS_MLP_BWD, TSP_WS_ATTN_BWD, TSP_WS_LAYER_BWD = 0, 1, 2, 3, 4
TSP_BWD_ATTN, TSP_BWD_QKV, TSP_BWD_ALL = 1, 2, 3
TSP_ATTN_Q_LOG2_SCALED = 1
TSP_ATTN_BWD_PLAIN_PDS = 1
TSP_MLP_GELU, TSP_MLP_SWIGLU = 0, 1
MLP_KINDS = {"gelu": TSP_MLP_GELU, "swiglu": TSP_MLP_SWIGLU}
TSP_MAX_D = 64
KERNEL_CLASSES = {"rmsnorm": 0, "qkv": 1, "attention": 2, "outproj": 3, "mlp_up": 4, "mlp_down": 5, "zigzag": 6,
                  "lead": 7, "bwd_gemm": 8, "transpose": 9,
                  "attn_bwd": 10, "rows_bwd": 11}

EXPORTED_SYMBOLS = [
    "tsp_status_string", "tsp_last_error", "tsp_abi_version", "tsp_workspace_size",
    "tsp_zigzag_index_host", "tsp_zigzag_index", "tsp_zigzag_attn", "tsp_zigzag_attn_ex", "tsp_mlp_ring",
    "tsp_mlp_ring_bwd", "tsp_zigzag_attn_bwd", "tsp_zigzag_attn_bwd_noalloc", "tsp_zigzag_attn_lse",
    "tsp_zigzag_attn_bwd_lse", "tsp_zigzag_attn_bwd_ex", "tsp_layer_fwd", "tsp_layer_bwd", "tsp_mlp_ring_z",
    "tsp_mlp_ring_bwd_z", "tsp_layer_fwd_save", "tsp_layer_bwd_ex", "tsp_profile_enable",
    "tsp_profile_reset", "tsp_profile_read",
]


class TspError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[{status}] {message}")
        self.status = status


class TspShape(ctypes.Structure):
    _fields_ = [("S", ctypes.c_int64), ("D", ctypes.c_int32), ("r", ctypes.c_int32), ("h", ctypes.c_int32),
                ("H", ctypes.c_int32), ("Dh", ctypes.c_int32), ("F", ctypes.c_int32), ("eps", ctypes.c_float),
                ("scale", ctypes.c_float), ("dtype", ctypes.c_int32), ("rope_base", ctypes.c_float),
                ("Hkv", ctypes.c_int32), ("mlp", ctypes.c_int32)]


class TspLayerWeights(ctypes.Structure):
    _fields_ = [("g_attn", ctypes.c_void_p), ("g_mlp", ctypes.c_void_p),
                ("wqkv", ctypes.POINTER(ctypes.c_void_p)), ("wo", ctypes.POINTER(ctypes.c_void_p)),
                ("w1", ctypes.POINTER(ctypes.c_void_p)), ("w2", ctypes.POINTER(ctypes.c_void_p))]


class TspLayerGrads(ctypes.Structure):
    _fields_ = [("g_attn", ctypes.c_void_p), ("g_mlp", ctypes.c_void_p),
                ("wqkv", ctypes.POINTER(ctypes.c_void_p)), ("wo", ctypes.POINTER(ctypes.c_void_p)),
                ("w1", ctypes.POINTER(ctypes.c_void_p)), ("w2", ctypes.POINTER(ctypes.c_void_p))]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libtsp.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m tsp_rank_local_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, sz, i32, i64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int64
    shp = ctypes.POINTER(TspShape)
    L.tsp_status_string.restype = ctypes.c_char_p
    L.tsp_status_string.argtypes = [ctypes.c_int]
    L.tsp_last_error.restype = ctypes.c_char_p
    L.tsp_last_error.argtypes = []
    L.tsp_abi_version.restype = ctypes.c_int
    L.tsp_workspace_size.argtypes = [shp, ctypes.c_int, ctypes.POINTER(sz)]
    L.tsp_zigzag_index_host.argtypes = [i64, i32, i32, ctypes.POINTER(i32)]
    L.tsp_zigzag_index.argtypes = [i64, i32, i32, vp, vp]
    L.tsp_zigzag_attn.argtypes = [shp, vp, vp, vp, vp, i32, vp]
    L.tsp_zigzag_attn_ex.argtypes = [shp, vp, vp, vp, vp, i32, ctypes.c_uint32, vp]
    L.tsp_mlp_ring.argtypes = [shp, vp, ctypes.POINTER(vp), ctypes.POINTER(vp), vp, vp, vp, sz, vp]
    L.tsp_mlp_ring_bwd.argtypes = [shp, vp, ctypes.POINTER(vp), ctypes.POINTER(vp), vp, vp, vp, ctypes.POINTER(vp),
                                   ctypes.POINTER(vp), vp, sz, vp]
    L.tsp_zigzag_attn_bwd.argtypes = [shp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.tsp_zigzag_attn_bwd_noalloc.argtypes = [shp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.tsp_zigzag_attn_lse.argtypes = [shp, vp, vp, vp, vp, vp, vp]
    L.tsp_mlp_ring_z.argtypes = [shp, vp, ctypes.POINTER(vp), ctypes.POINTER(vp), vp, vp, vp, vp, sz, vp]
    L.tsp_mlp_ring_bwd_z.argtypes = [shp, vp, vp, ctypes.POINTER(vp), ctypes.POINTER(vp), vp, vp, vp,
                                     ctypes.POINTER(vp), ctypes.POINTER(vp), vp, sz, vp]
    L.tsp_zigzag_attn_bwd_lse.argtypes = [shp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.tsp_zigzag_attn_bwd_ex.argtypes = [shp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_uint32, vp, sz, vp]
    L.tsp_layer_fwd.argtypes = [shp, ctypes.POINTER(TspLayerWeights), vp, vp, vp, vp, ctypes.c_uint, vp, sz, vp]
    L.tsp_layer_bwd.argtypes = [shp, ctypes.POINTER(TspLayerWeights), vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                ctypes.POINTER(TspLayerGrads), ctypes.c_uint, vp, sz, vp]
    L.tsp_layer_fwd_save.argtypes = [shp, ctypes.POINTER(TspLayerWeights), vp, vp, vp, vp, vp, vp, vp, ctypes.c_uint,
                                     vp, sz, vp]
    L.tsp_layer_bwd_ex.argtypes = [shp, ctypes.POINTER(TspLayerWeights), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                   vp, ctypes.POINTER(TspLayerGrads), ctypes.c_uint, vp, sz, vp]
    L.tsp_profile_enable.argtypes = [ctypes.c_int]
    L.tsp_profile_enable.restype = None
    L.tsp_profile_reset.argtypes = []
    L.tsp_profile_reset.restype = None
    L.tsp_profile_read.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i64)]
    for name in ("tsp_workspace_size", "tsp_zigzag_index_host", "tsp_zigzag_index", "tsp_zigzag_attn",
                 "tsp_zigzag_attn_ex", "tsp_mlp_ring", "tsp_mlp_ring_bwd", "tsp_zigzag_attn_bwd",
                 "tsp_zigzag_attn_bwd_noalloc", "tsp_layer_fwd", "tsp_layer_bwd",
                 "tsp_zigzag_attn_lse", "tsp_zigzag_attn_bwd_lse", "tsp_zigzag_attn_bwd_ex", "tsp_mlp_ring_z",
                 "tsp_mlp_ring_bwd_z", "tsp_layer_fwd_save", "tsp_layer_bwd_ex",
                 "tsp_profile_read"):
        getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def _check(status: int) -> None:
    if status != TSP_OK:
        L = lib()
        raise TspError(status, f"{L.tsp_status_string(status).decode()}: {L.tsp_last_error().decode()}")


def _ptr(t) -> int | None:
    """Device address of a torch tensor, an int, or None."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _ptr_array(ts):
    arr = (ctypes.c_void_p * len(ts))()
    for i, t in enumerate(ts):
        arr[i] = _ptr(t)
    return arr


def _stream(stream) -> int | None:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def make_shape(S, D, r, h, H, Dh, F, eps=1e-5, scale=None, dtype="bf16", rope_base=0.0, Hkv=0,
               mlp="gelu") -> TspShape:
    """A tsp_shape; dtype 'bf16' or 'f32'; scale defaults to 1/sqrt(Dh);
    rope_base 0 means no rotary embedding; Hkv 0 means Hkv = H (multi-head);
    mlp 'gelu' or 'swiglu' (or a TSP_MLP_* value)."""
    if scale is None:
        scale = 1.0 / float(np.sqrt(Dh))
    dt = {"bf16": TSP_BF16, "f32": TSP_F32}[dtype] if isinstance(dtype, str) else int(dtype)
    return TspShape(int(S), int(D), int(r), int(h), int(H), int(Dh), int(F), float(eps), float(scale), dt,
                    float(rope_base), int(Hkv), MLP_KINDS[mlp] if isinstance(mlp, str) else int(mlp))


def workspace_size(shape: TspShape, which: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().tsp_workspace_size(ctypes.byref(shape), int(which), ctypes.byref(n)))
    return int(n.value)


def tsp_zigzag_index_host(S: int, D: int, r: int) -> np.ndarray:
    n = int(S) // int(D) if D > 0 else 0
    out = np.zeros(max(n, 1), dtype=np.int32)
    _check(lib().tsp_zigzag_index_host(int(S), int(D), int(r), out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))))
    return out[:n]


def tsp_zigzag_index(S: int, D: int, r: int, pos, stream=None) -> None:
    _check(lib().tsp_zigzag_index(int(S), int(D), int(r), _ptr(pos), _stream(stream)))


def tsp_zigzag_attn(shape: TspShape, q, k, v, o, o_dtype=TSP_F32, stream=None) -> None:
    _check(lib().tsp_zigzag_attn(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(o), int(o_dtype),
                                 _stream(stream)))


def tsp_zigzag_attn_ex(shape: TspShape, q, k, v, o, o_dtype=TSP_F32, flags=0, stream=None) -> None:
    _check(lib().tsp_zigzag_attn_ex(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(o), int(o_dtype),
                                    int(flags), _stream(stream)))


def tsp_mlp_ring(shape: TspShape, x, w1, w2, residual, y, ws, ws_bytes=None, stream=None) -> None:
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    a1, a2 = _ptr_array(w1), _ptr_array(w2)
    _check(lib().tsp_mlp_ring(ctypes.byref(shape), _ptr(x), a1, a2, _ptr(residual), _ptr(y), _ptr(ws),
                              int(ws_bytes), _stream(stream)))


def tsp_zigzag_attn_bwd(shape: TspShape, q, k, v, dout, dq, dk, dv, ws, ws_bytes=None, stream=None) -> None:
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    _check(lib().tsp_zigzag_attn_bwd(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(dq),
                                     _ptr(dk), _ptr(dv), _ptr(ws), int(ws_bytes), _stream(stream)))


def tsp_zigzag_attn_bwd_noalloc(shape: TspShape, q, k, v, dout, dq, dk, dv, stream=None) -> None:
    _check(lib().tsp_zigzag_attn_bwd_noalloc(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(dq),
                                             _ptr(dk), _ptr(dv), _stream(stream)))


def tsp_mlp_ring_z(shape: TspShape, x, w1, w2, residual, y, z, ws, ws_bytes=None, stream=None) -> None:
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    _check(lib().tsp_mlp_ring_z(ctypes.byref(shape), _ptr(x), _ptr_array(w1), _ptr_array(w2), _ptr(residual), _ptr(y),
                                _ptr(z), _ptr(ws), int(ws_bytes), _stream(stream)))


def tsp_mlp_ring_bwd_z(shape: TspShape, x, z, w1, w2, dy, dx_residual, dx, dw1, dw2, ws, ws_bytes=None,
                       stream=None) -> None:
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    _check(lib().tsp_mlp_ring_bwd_z(ctypes.byref(shape), _ptr(x), _ptr(z), _ptr_array(w1), _ptr_array(w2), _ptr(dy),
                                    _ptr(dx_residual), _ptr(dx), _ptr_array(dw1), _ptr_array(dw2), _ptr(ws),
                                    int(ws_bytes), _stream(stream)))


def tsp_zigzag_attn_lse(shape: TspShape, q, k, v, o, lse, stream=None) -> None:
    _check(lib().tsp_zigzag_attn_lse(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                     _stream(stream)))


def tsp_zigzag_attn_bwd_lse(shape: TspShape, q, k, v, o, lse, dout, dq, dk, dv, ws, ws_bytes=None,
                            stream=None) -> None:
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    _check(lib().tsp_zigzag_attn_bwd_lse(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                         _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws), int(ws_bytes),
                                         _stream(stream)))


def tsp_zigzag_attn_bwd_ex(shape: TspShape, q, k, v, o, lse, dout, dq, dk, dv, flags, ws, ws_bytes=None,
                           stream=None) -> None:
    """o and lse: both None, or the forward's fp32 output and log-sum-exp."""
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    _check(lib().tsp_zigzag_attn_bwd_ex(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                        _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), int(flags), _ptr(ws),
                                        int(ws_bytes), _stream(stream)))


def tsp_mlp_ring_bwd(shape: TspShape, x, w1, w2, dy, dx_residual, dx, dw1, dw2, ws, ws_bytes=None,
                     stream=None) -> None:
    """dw1, dw2: lists of D fp32 device tensors, indexed by shard."""
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    a1, a2, g1, g2 = _ptr_array(w1), _ptr_array(w2), _ptr_array(dw1), _ptr_array(dw2)
    _check(lib().tsp_mlp_ring_bwd(ctypes.byref(shape), _ptr(x), a1, a2, _ptr(dy), _ptr(dx_residual), _ptr(dx), g1,
                                  g2, _ptr(ws), int(ws_bytes), _stream(stream)))


def tsp_layer_fwd(shape: TspShape, w: dict, x, k_full, v_full, y, phases, ws, ws_bytes=None, stream=None) -> None:
    """w: dict with g_attn, g_mlp and lists wqkv, wo, w1, w2 of D device tensors."""
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    arrs = {k: _ptr_array(w[k]) for k in ("wqkv", "wo", "w1", "w2")}
    cw = TspLayerWeights(_ptr(w["g_attn"]), _ptr(w["g_mlp"]), arrs["wqkv"], arrs["wo"], arrs["w1"], arrs["w2"])
    _check(lib().tsp_layer_fwd(ctypes.byref(shape), ctypes.byref(cw), _ptr(x), _ptr(k_full), _ptr(v_full), _ptr(y),
                               int(phases), _ptr(ws), int(ws_bytes), _stream(stream)))


def tsp_layer_fwd_save(shape: TspShape, w: dict, x, k_full, v_full, y, o_save, lse_save, phases, ws, ws_bytes=None,
                       stream=None, z_save=None) -> None:
    """tsp_layer_fwd that also keeps the attention output o_save [N][H][Dh]
    and the rows' natural log-sum-exp lse_save [H][N] (fp32), and optionally
    the MLP pre-activation z_save [N][F] (bf16), for tsp_layer_bwd_ex."""
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    cw, keep_w = _weights(w)
    _check(lib().tsp_layer_fwd_save(ctypes.byref(shape), ctypes.byref(cw), _ptr(x), _ptr(k_full), _ptr(v_full),
                                    _ptr(y), _ptr(o_save), _ptr(lse_save), _ptr(z_save), int(phases), _ptr(ws),
                                    int(ws_bytes), _stream(stream)))
    del keep_w


def _weights(w: dict) -> tuple:
    """A TspLayerWeights for a dict of g_attn, g_mlp and shard lists, plus the
    pointer arrays it refers to (kept alive by the caller)."""
    arrs = {k: _ptr_array(w[k]) for k in ("wqkv", "wo", "w1", "w2")}
    return TspLayerWeights(_ptr(w["g_attn"]), _ptr(w["g_mlp"]), arrs["wqkv"], arrs["wo"], arrs["w1"], arrs["w2"]), arrs


def tsp_layer_bwd(shape: TspShape, w: dict, x, k_full, v_full, dy, dk_full, dv_full, dk_loc, dv_loc, dx,
                  grads: dict, phases, ws, ws_bytes=None, stream=None) -> None:
    """w: as for tsp_layer_fwd; grads: dict with fp32 g_attn, g_mlp and lists
    wqkv, wo, w1, w2 of D fp32 device tensors (entries a phase does not
    write may be None)."""
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    cw, keep_w = _weights(w)
    garr = {k: (_ptr_array(grads[k]) if grads.get(k) is not None else None) for k in ("wqkv", "wo", "w1", "w2")}
    cg = TspLayerGrads(_ptr(grads.get("g_attn")), _ptr(grads.get("g_mlp")), garr["wqkv"], garr["wo"], garr["w1"],
                       garr["w2"])
    _check(lib().tsp_layer_bwd(ctypes.byref(shape), ctypes.byref(cw), _ptr(x), _ptr(k_full), _ptr(v_full), _ptr(dy),
                               _ptr(dk_full), _ptr(dv_full), _ptr(dk_loc), _ptr(dv_loc), _ptr(dx), ctypes.byref(cg),
                               int(phases), _ptr(ws), int(ws_bytes), _stream(stream)))
    del keep_w


def tsp_layer_bwd_ex(shape: TspShape, w: dict, x, k_full, v_full, dy, o_saved, lse_saved, dk_full, dv_full, dk_loc,
                     dv_loc, dx, grads: dict, phases, ws, ws_bytes=None, stream=None, z_saved=None) -> None:
    """tsp_layer_bwd with the saved attention output and statistics (and
    optionally Z) of tsp_layer_fwd_save (all None: the same as tsp_layer_bwd)."""
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    cw, keep_w = _weights(w)
    garr = {k: (_ptr_array(grads[k]) if grads.get(k) is not None else None) for k in ("wqkv", "wo", "w1", "w2")}
    cg = TspLayerGrads(_ptr(grads.get("g_attn")), _ptr(grads.get("g_mlp")), garr["wqkv"], garr["wo"], garr["w1"],
                       garr["w2"])
    _check(lib().tsp_layer_bwd_ex(ctypes.byref(shape), ctypes.byref(cw), _ptr(x), _ptr(k_full), _ptr(v_full),
                                  _ptr(dy), _ptr(o_saved), _ptr(lse_saved), _ptr(z_saved), _ptr(dk_full),
                                  _ptr(dv_full), _ptr(dk_loc), _ptr(dv_loc), _ptr(dx), ctypes.byref(cg), int(phases),
                                  _ptr(ws), int(ws_bytes), _stream(stream)))
    del keep_w


def profile_enable(on: bool = True) -> None:
    lib().tsp_profile_enable(1 if on else 0)


def profile_reset() -> None:
    lib().tsp_profile_reset()


def profile_read(kernel: str):
    """(total milliseconds, launches) for a kernel class since the last reset."""
    ms = ctypes.c_double(0.0)
    n = ctypes.c_int64(0)
    _check(lib().tsp_profile_read(KERNEL_CLASSES[kernel], ctypes.byref(ms), ctypes.byref(n)))
    return float(ms.value), int(n.value)


def to_device(a: np.ndarray, dtype: str, device="cuda"):
    """Upload a host array: 'bf16' takes uint16 bf16 bit patterns, 'f32' float32."""
    import torch
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(device)
