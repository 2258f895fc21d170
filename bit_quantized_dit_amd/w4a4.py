"""ctypes binding of libw4a4.so (argument marshalling only).

Every function carries the name of the C entry point it wraps (see include/w4a4.h for
the operations and their citations).  Torch tensors serve only as device buffers and
their current HIP stream; every step of the computation runs in the library's
kernels.  If the library is not built, every call raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libw4a4.so")

W4A4_X_F32 = 0
W4A4_X_BF16 = 1
W4A4_WS_1X32 = 0
W4A4_WS_32X32_TILE = 1
W4A4_WS_128X1_STRIPE = 2
STATUS = {0: "W4A4_OK", 1: "W4A4_ERR_INVALID", 2: "W4A4_ERR_SHAPE", 3: "W4A4_ERR_ALIGN",
          4: "W4A4_ERR_DEVICE", 5: "W4A4_ERR_NONFINITE", 6: "W4A4_ERR_SCRATCH"}
NOALLOC_SCRATCH_BYTES = 128 << 20    # W4A4_NOALLOC_SCRATCH_BYTES

EXPORTS = ("w4a4_status_string", "w4a4_column_absmax", "w4a4_calibrate_scales", "w4a4_packed_size",
           "w4a4_pack_weights", "w4a4_workspace_layout", "w4a4_workspace_size",
           "w4a4_quantize_activations", "w4a4_gemm_prequantized", "w4a4_linear",
           "w4a4_gemm_prequantized_gelu_bf16", "w4a4_linear_gelu_bf16", "w4a4_gelu_tanh_bf16",
           "w4a4_search_scratch_size", "w4a4_search_alpha_k", "w4a4_packed_dyn_size", "w4a4_pack_weights_dyn",
           "w4a4_workspace_dyn_layout", "w4a4_workspace_dyn_size", "w4a4_linear_dyn",
           "w4a4_ffn_workspace_layout", "w4a4_ffn_workspace_size", "w4a4_ffn_up_quantize", "w4a4_ffn_forward",
           "w4a4_linear_noalloc")


class W4A4Packed(ctypes.Structure):
    _fields_ = [("d_in", ctypes.c_int64), ("d_out", ctypes.c_int64), ("k", ctypes.c_int32),
                ("layout", ctypes.c_int32), ("k_j", ctypes.c_int64), ("k_pad", ctypes.c_int64),
                ("k_ld", ctypes.c_int64), ("colmap", ctypes.c_void_p), ("s", ctypes.c_void_p),
                ("O", ctypes.c_void_p), ("J", ctypes.c_void_p), ("B_q", ctypes.c_void_p),
                ("B_s", ctypes.c_void_p), ("B_s_rows", ctypes.c_void_p), ("W_O", ctypes.c_void_p),
                ("B_q_tiles", ctypes.c_void_p)]


class W4A4WsLayout(ctypes.Structure):
    _fields_ = [("a_q", ctypes.c_size_t), ("a_s", ctypes.c_size_t), ("x_o", ctypes.c_size_t),
                ("partial", ctypes.c_size_t), ("total", ctypes.c_size_t)]


class W4A4PackedDyn(ctypes.Structure):
    _fields_ = [("base", W4A4Packed), ("k", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("W_t", ctypes.c_void_p)]


class W4A4WsDynLayout(ctypes.Structure):
    _fields_ = [("base", W4A4WsLayout), ("colmax", ctypes.c_size_t), ("O", ctypes.c_size_t),
                ("colmap", ctypes.c_size_t), ("W_O", ctypes.c_size_t), ("total", ctypes.c_size_t)]


class W4A4FfnWsLayout(ctypes.Structure):
    _fields_ = [("up", W4A4WsLayout), ("down", W4A4WsLayout), ("up_base", ctypes.c_size_t),
                ("down_base", ctypes.c_size_t), ("rinv", ctypes.c_size_t), ("total", ctypes.c_size_t)]


class W4A4Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)} ({status_string(status)})")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libw4a4.so; raise if it has not been built (no fallback path exists)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m bit_quantized_dit_amd.build` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        i64, i32, vp, sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t
        ci, f32 = ctypes.c_int, ctypes.c_float
        P = ctypes.POINTER
        sig = {
            "w4a4_status_string": (ctypes.c_char_p, [ci]),
            "w4a4_column_absmax": (ci, [vp, ci, i64, i64, vp, vp]),
            "w4a4_calibrate_scales": (ci, [vp, ci, i64, i64, vp, i64, f32, i32, vp, vp, vp, vp, vp]),
            "w4a4_packed_size": (ci, [i64, i64, i32, ci, P(sz)]),
            "w4a4_pack_weights": (ci, [vp, i64, i64, vp, vp, i32, ci, vp, sz, P(W4A4Packed), vp]),
            "w4a4_workspace_layout": (ci, [i64, P(W4A4Packed), P(W4A4WsLayout)]),
            "w4a4_workspace_size": (ci, [i64, P(W4A4Packed), P(sz)]),
            "w4a4_quantize_activations": (ci, [vp, ci, i64, P(W4A4Packed), vp, sz, vp]),
            "w4a4_gemm_prequantized": (ci, [vp, sz, i64, P(W4A4Packed), vp, vp]),
            "w4a4_linear": (ci, [vp, ci, i64, P(W4A4Packed), vp, vp, sz, vp]),
            "w4a4_gemm_prequantized_gelu_bf16": (ci, [vp, sz, i64, P(W4A4Packed), vp, vp]),
            "w4a4_linear_gelu_bf16": (ci, [vp, ci, i64, P(W4A4Packed), vp, vp, sz, vp]),
            "w4a4_gelu_tanh_bf16": (ci, [vp, i64, vp, vp]),
            "w4a4_search_scratch_size": (ci, [i64, i64, i64, vp, ci, ci, P(sz)]),
            "w4a4_search_alpha_k": (ci, [vp, ci, i64, i64, vp, i64, vp, ci, vp, ci, ci, vp, sz, vp, vp, vp]),
            "w4a4_packed_dyn_size": (ci, [i64, i64, i32, ci, P(sz)]),
            "w4a4_pack_weights_dyn": (ci, [vp, i64, i64, vp, i32, ci, vp, sz, P(W4A4PackedDyn), vp]),
            "w4a4_workspace_dyn_layout": (ci, [i64, P(W4A4PackedDyn), P(W4A4WsDynLayout)]),
            "w4a4_workspace_dyn_size": (ci, [i64, P(W4A4PackedDyn), P(sz)]),
            "w4a4_linear_dyn": (ci, [vp, ci, i64, P(W4A4PackedDyn), vp, vp, sz, vp]),
            "w4a4_ffn_workspace_layout": (ci, [i64, P(W4A4Packed), P(W4A4Packed), P(W4A4FfnWsLayout)]),
            "w4a4_ffn_workspace_size": (ci, [i64, P(W4A4Packed), P(W4A4Packed), P(sz)]),
            "w4a4_ffn_up_quantize": (ci, [vp, ci, i64, P(W4A4Packed), P(W4A4Packed), vp, sz, vp]),
            "w4a4_ffn_forward": (ci, [vp, ci, i64, P(W4A4Packed), P(W4A4Packed), vp, vp, sz, vp]),
            "w4a4_linear_noalloc": (ci, [vp, ci, i64, P(W4A4Packed), vp, vp]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def status_string(status: int) -> str:
    try:
        return lib().w4a4_status_string(int(status)).decode()
    except RuntimeError:
        return STATUS.get(status, "?")


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise W4A4Error(fn, status)


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _x_dtype(X: torch.Tensor) -> int:
    if X.dtype == torch.float32:
        return W4A4_X_F32
    if X.dtype == torch.bfloat16:
        return W4A4_X_BF16
    raise TypeError(f"activations must be float32 or bfloat16, got {X.dtype}")


def _dev(t: torch.Tensor, name: str) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


# Shape, dtype and device checks on the host side of the binding: a tensor that does
# not match what the library will read or write would otherwise become an
# out-of-bounds access inside a kernel.  Sizes of the workspace are checked by the
# library itself (status W4A4_ERR_SHAPE).
def _acts(X: torch.Tensor, d_in: int, name: str = "X") -> int:
    _dev(X, name)
    _x_dtype(X)
    if X.dim() != 2 or X.shape[1] != d_in:
        raise ValueError(f"{name} must be [T, {d_in}], got {tuple(X.shape)}")
    return X.shape[0]


def _out(Y: torch.Tensor, T: int, d_out: int, dtype: torch.dtype, name: str, like: torch.Tensor | None = None):
    _dev(Y, name)
    if Y.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {Y.dtype}")
    if tuple(Y.shape) != (T, d_out):
        raise ValueError(f"{name} must be [{T}, {d_out}], got {tuple(Y.shape)}")
    if like is not None and Y.device != like.device:
        raise ValueError(f"{name} is on {Y.device}, expected {like.device}")


def _wsbuf(ws: torch.Tensor, like: torch.Tensor, name: str = "ws") -> None:
    _dev(ws, name)
    if ws.dtype != torch.uint8:
        raise TypeError(f"{name} must be a uint8 buffer, got {ws.dtype}")
    if ws.device != like.device:
        raise ValueError(f"{name} is on {ws.device}, expected {like.device}")


@dataclass
class PackedLayer:
    """A packed layer: the device blob (kept alive here) and its descriptor."""
    blob: torch.Tensor
    desc: W4A4Packed

    @property
    def d_in(self) -> int: return self.desc.d_in
    @property
    def d_out(self) -> int: return self.desc.d_out
    @property
    def k(self) -> int: return self.desc.k
    @property
    def k_pad(self) -> int: return self.desc.k_pad
    @property
    def k_ld(self) -> int: return self.desc.k_ld
    @property
    def layout(self) -> int: return self.desc.layout

    def views(self) -> dict:
        """Device views of the packed arrays inside the blob."""
        base = self.blob.data_ptr()
        d = self.desc

        def view(ptr, nbytes, dtype, shape):
            off = ptr - base
            return self.blob[off:off + nbytes].view(dtype).view(*shape)
        if d.layout == W4A4_WS_1X32:
            bs_shape = (d.d_out, d.k_pad // 32)
        elif d.layout == W4A4_WS_128X1_STRIPE:
            bs_shape = (d.d_out, d.k_pad // 128)
        else:
            bs_shape = (d.k_pad // 32, (d.d_out + 31) // 32)
        out = {"colmap": view(d.colmap, d.d_in * 4, torch.int32, (d.d_in,)),
               "s": view(d.s, d.d_in * 4, torch.float32, (d.d_in,))}
        if d.k_pad:
            out["B_q"] = view(d.B_q, d.d_out * d.k_pad // 2, torch.uint8, (d.d_out, d.k_pad // 2))
            out["B_s"] = view(d.B_s, bs_shape[0] * bs_shape[1], torch.uint8, bs_shape)
            out["J"] = view(d.J, d.k_j * 4, torch.int32, (d.k_j,))
            # step-major [k_pad/128][d_out][4] (raw) and the same codes as [d_out][k_pad/32]
            raw = view(d.B_s_rows, d.d_out * d.k_pad // 32, torch.uint8, (d.k_pad // 128, d.d_out, 4))
            out["B_s_rows_raw"] = raw
            out["B_s_rows"] = raw.permute(1, 0, 2).reshape(d.d_out, d.k_pad // 32)
            rows16 = (d.d_out + 15) // 16 * 16
            tiles = view(d.B_q_tiles, rows16 * d.k_pad // 2, torch.uint8, (rows16 * d.k_pad // 2,))
            out["B_q_tiles_raw"] = tiles
            out["B_q_from_tiles"] = untile_codes(tiles, rows16, d.k_pad)[:d.d_out]
        if d.k:
            out["W_O"] = view(d.W_O, d.d_out * d.k_ld * 2, torch.bfloat16, (d.d_out, d.k_ld))
            out["O"] = view(d.O, d.k * 4, torch.int32, (d.k,))
        return out


# --------------------------------------------------------------------------- calls

def w4a4_column_absmax(X: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    _dev(X, "X")
    _x_dtype(X)
    if X.dim() != 2:
        raise ValueError(f"X must be 2-D, got {tuple(X.shape)}")
    rows, cols = X.shape
    if out is None:
        out = torch.empty(cols, dtype=torch.int32, device=X.device)
    _dev(out, "out")
    if out.dtype not in (torch.int32, torch.uint32) or out.numel() != cols or out.device != X.device:
        raise ValueError(f"out must be a 32-bit integer tensor of {cols} elements on {X.device}")
    _check("w4a4_column_absmax", lib().w4a4_column_absmax(_ptr(X), _x_dtype(X), rows, cols, _ptr(out),
                                                           _stream(stream)))
    return out


def w4a4_calibrate_scales(X_cal: torch.Tensor, W: torch.Tensor, alpha: float, k: int, stream=None):
    """Returns (s, O, act_scale, weight_scale) as host numpy arrays."""
    _dev(X_cal, "X_cal")
    _dev(W, "W")
    if W.dtype != torch.float32:
        raise TypeError("W must be float32")
    T_cal, d_in = X_cal.shape
    d_out = W.shape[0]
    if W.shape[1] != d_in:
        raise ValueError("W must be [d_out, d_in]")
    s = np.zeros(d_in, np.float32)
    O = np.zeros(max(k, 1), np.int32)
    a = np.zeros(d_in, np.float32)
    w = np.zeros(d_in, np.float32)
    vp = lambda arr: arr.ctypes.data_as(ctypes.c_void_p)
    st = lib().w4a4_calibrate_scales(_ptr(X_cal), _x_dtype(X_cal), T_cal, d_in, _ptr(W), d_out,
                                     float(alpha), int(k), vp(s), vp(O), vp(a), vp(w), _stream(stream))
    _check("w4a4_calibrate_scales", st)
    return s, O[:k].copy(), a, w


class PackedLayerDyn:
    """A layer packed for per-call outlier selection: the device blob (kept alive
    here) and its descriptor."""

    def __init__(self, blob: torch.Tensor, desc: W4A4PackedDyn):
        self.blob, self.desc = blob, desc

    @property
    def k(self) -> int: return self.desc.k
    @property
    def d_in(self) -> int: return self.desc.base.d_in
    @property
    def d_out(self) -> int: return self.desc.base.d_out
    @property
    def k_pad(self) -> int: return self.desc.base.k_pad


def w4a4_pack_weights_dyn(W: torch.Tensor, s: np.ndarray, k: int, layout: int, stream=None) -> PackedLayerDyn:
    _dev(W, "W")
    if W.dtype != torch.float32:
        raise TypeError("W must be float32")
    d_out, d_in = W.shape
    s = np.ascontiguousarray(s, dtype=np.float32)
    n = ctypes.c_size_t(0)
    _check("w4a4_packed_dyn_size", lib().w4a4_packed_dyn_size(d_in, d_out, int(k), int(layout), ctypes.byref(n)))
    blob = torch.zeros(max(n.value, 256), dtype=torch.uint8, device=W.device)
    desc = W4A4PackedDyn()
    st = lib().w4a4_pack_weights_dyn(_ptr(W), d_in, d_out, s.ctypes.data_as(ctypes.c_void_p), int(k), int(layout),
                                     _ptr(blob), blob.numel(), ctypes.byref(desc), _stream(stream))
    _check("w4a4_pack_weights_dyn", st)
    return PackedLayerDyn(blob, desc)


def w4a4_workspace_dyn_layout(T: int, packed: PackedLayerDyn) -> W4A4WsDynLayout:
    out = W4A4WsDynLayout()
    _check("w4a4_workspace_dyn_layout",
           lib().w4a4_workspace_dyn_layout(T, ctypes.byref(packed.desc), ctypes.byref(out)))
    return out


def alloc_workspace_dyn(T: int, packed: PackedLayerDyn, device="cuda") -> torch.Tensor:
    return torch.empty(max(w4a4_workspace_dyn_layout(T, packed).total, 256), dtype=torch.uint8, device=device)


def workspace_dyn_views(ws: torch.Tensor, T: int, packed: PackedLayerDyn) -> dict:
    """Device tensors of one call's per-call state inside ws: O [k], the column map
    [d_in], W_O [d_out, k_ld], and the quantized activations as workspace_views gives
    them (over K_pad = roundup(d_in, 128))."""
    L = w4a4_workspace_dyn_layout(T, packed)
    k, d_in, d_out = packed.k, packed.d_in, packed.d_out
    k_ld = (k + 31) // 32 * 32
    kp = packed.k_pad
    raw = ws[L.base.a_s:L.base.a_s + T * kp // 32].view(kp // 128, T, 4)
    rows16 = (T + 15) // 16 * 16
    aq_raw = ws[L.base.a_q:L.base.a_q + rows16 * kp // 2]
    return {"O": ws[L.O:L.O + 4 * k].view(torch.int32),
            "colmap": ws[L.colmap:L.colmap + 4 * d_in].view(torch.int32),
            "W_O": ws[L.W_O:L.W_O + 2 * d_out * k_ld].view(torch.bfloat16).view(d_out, k_ld),
            "A_q": untile_codes(aq_raw, rows16, kp)[:T],
            "A_s": raw.permute(1, 0, 2).reshape(T, kp // 32),
            "X_O": ws[L.base.x_o:L.base.x_o + T * k_ld * 2].view(torch.bfloat16).view(T, k_ld)}


def w4a4_linear_dyn(X: torch.Tensor, packed: PackedLayerDyn, Y: torch.Tensor, ws: torch.Tensor,
                    stream=None) -> None:
    T = _acts(X, packed.d_in)
    _out(Y, T, packed.d_out, torch.float32, "Y", X)
    _wsbuf(ws, X)
    st = lib().w4a4_linear_dyn(_ptr(X), _x_dtype(X), T, ctypes.byref(packed.desc), _ptr(Y), _ptr(ws),
                               ws.numel(), _stream(stream))
    _check("w4a4_linear_dyn", st)


def w4a4_search_scratch_size(T_cal: int, d_in: int, d_out: int, ks, layout: int) -> int:
    ks_a = np.ascontiguousarray(np.asarray(ks, dtype=np.int32))
    n = ctypes.c_size_t(0)
    _check("w4a4_search_scratch_size",
           lib().w4a4_search_scratch_size(T_cal, d_in, d_out, ks_a.ctypes.data_as(ctypes.c_void_p), ks_a.size,
                                          layout, ctypes.byref(n)))
    return n.value


def w4a4_search_alpha_k(X_cal: torch.Tensor, W: torch.Tensor, alphas, ks, layout: int, stream=None):
    """Layer-wise alpha / k search on calibration tokens.  Returns (errors [n_alpha, n_k]
    as a host float64 array, (a, b) indices of the smallest error); the scratch buffer
    is allocated here with torch."""
    _dev(X_cal, "X_cal")
    _dev(W, "W")
    if W.dtype != torch.float32:
        raise TypeError("W must be float32")
    T_cal, d_in = X_cal.shape
    d_out = W.shape[0]
    if W.shape[1] != d_in:
        raise ValueError("W must be [d_out, d_in]")
    al = np.ascontiguousarray(np.asarray(alphas, dtype=np.float32))
    ka = np.ascontiguousarray(np.asarray(ks, dtype=np.int32))
    nbytes = w4a4_search_scratch_size(T_cal, d_in, d_out, ka, layout)
    scratch = torch.empty(nbytes, dtype=torch.uint8, device=X_cal.device)
    err = np.zeros(al.size * ka.size, np.float64)
    best = np.zeros(2, np.int32)
    vp = lambda arr: arr.ctypes.data_as(ctypes.c_void_p)
    st = lib().w4a4_search_alpha_k(_ptr(X_cal), _x_dtype(X_cal), T_cal, d_in, _ptr(W), d_out, vp(al), al.size,
                                   vp(ka), ka.size, layout, _ptr(scratch), nbytes, vp(err), vp(best),
                                   _stream(stream))
    _check("w4a4_search_alpha_k", st)
    return err.reshape(al.size, ka.size), (int(best[0]), int(best[1]))


def w4a4_packed_size(d_in: int, d_out: int, k: int, layout: int) -> int:
    n = ctypes.c_size_t(0)
    _check("w4a4_packed_size", lib().w4a4_packed_size(d_in, d_out, k, layout, ctypes.byref(n)))
    return n.value


def w4a4_pack_weights(W: torch.Tensor, s: np.ndarray, O: np.ndarray, layout: int,
                      stream=None) -> PackedLayer:
    _dev(W, "W")
    if W.dtype != torch.float32:
        raise TypeError("W must be float32")
    d_out, d_in = W.shape
    s = np.ascontiguousarray(s, dtype=np.float32)
    O = np.ascontiguousarray(O, dtype=np.int32)
    k = int(O.size)
    nbytes = w4a4_packed_size(d_in, d_out, k, layout)
    blob = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=W.device)
    desc = W4A4Packed()
    Optr = O.ctypes.data_as(ctypes.c_void_p) if k else None
    st = lib().w4a4_pack_weights(_ptr(W), d_in, d_out, s.ctypes.data_as(ctypes.c_void_p), Optr, k,
                                 int(layout), _ptr(blob), blob.numel(), ctypes.byref(desc),
                                 _stream(stream))
    _check("w4a4_pack_weights", st)
    return PackedLayer(blob, desc)


def w4a4_workspace_layout(T: int, packed: PackedLayer) -> W4A4WsLayout:
    out = W4A4WsLayout()
    _check("w4a4_workspace_layout",
           lib().w4a4_workspace_layout(T, ctypes.byref(packed.desc), ctypes.byref(out)))
    return out


def w4a4_workspace_size(T: int, packed: PackedLayer) -> int:
    n = ctypes.c_size_t(0)
    _check("w4a4_workspace_size", lib().w4a4_workspace_size(T, ctypes.byref(packed.desc), ctypes.byref(n)))
    return n.value


def untile_codes(raw: torch.Tensor, rows: int, k_pad: int) -> torch.Tensor:
    """[rows, k_pad/2] row-major copy of codes stored in the tiled order (1 KiB per
    16-row block and 128-code step; row r of a block at r*64, its 16-byte chunk c at
    chunk position c ^ (r // 4)).  rows is a multiple of 16."""
    nkb = k_pad // 128
    t = raw.view(rows // 16, nkb, 16, 4, 16)
    r = torch.arange(16, device=raw.device).view(16, 1)
    phys = torch.arange(4, device=raw.device).view(1, 4) ^ (r // 4)     # [16, 4]: chunk c -> position
    t = t[:, :, r, phys, :]                                              # [blocks, nkb, 16, 4, 16]
    return t.permute(0, 2, 1, 3, 4).reshape(rows, k_pad // 2)


def alloc_workspace(T: int, packed: PackedLayer, device="cuda") -> torch.Tensor:
    return torch.empty(max(w4a4_workspace_size(T, packed), 256), dtype=torch.uint8, device=device)


def workspace_views(ws: torch.Tensor, T: int, packed: PackedLayer) -> dict:
    """Device tensors of the quantized activations inside ws: A_q_raw (the tiled
    array), A_q (the same codes as a [T, k_pad/2] copy), X_O [T, k_ld], A_s_raw (the
    step-major [k_pad/128, T, 4] array) and A_s (the same codes as a [T, k_pad/32]
    copy)."""
    L = w4a4_workspace_layout(T, packed)
    kp, kl = packed.k_pad, packed.k_ld
    raw = ws[L.a_s:L.a_s + T * kp // 32].view(kp // 128, T, 4)
    rows16 = (T + 15) // 16 * 16
    aq_raw = ws[L.a_q:L.a_q + rows16 * kp // 2]
    return {"A_q_raw": aq_raw,
            "A_q": untile_codes(aq_raw, rows16, kp)[:T],
            "A_s_raw": raw,
            "A_s": raw.permute(1, 0, 2).reshape(T, kp // 32),
            "X_O": ws[L.x_o:L.x_o + T * kl * 2].view(torch.bfloat16).view(T, kl)}


def w4a4_quantize_activations(X: torch.Tensor, packed: PackedLayer, ws: torch.Tensor, stream=None) -> None:
    T = _acts(X, packed.d_in)
    _wsbuf(ws, X)
    st = lib().w4a4_quantize_activations(_ptr(X), _x_dtype(X), T, ctypes.byref(packed.desc), _ptr(ws),
                                         ws.numel(), _stream(stream))
    _check("w4a4_quantize_activations", st)


def w4a4_gemm_prequantized(ws: torch.Tensor, T: int, packed: PackedLayer, Y: torch.Tensor,
                           stream=None) -> None:
    _out(Y, T, packed.d_out, torch.float32, "Y")
    _wsbuf(ws, Y)
    st = lib().w4a4_gemm_prequantized(_ptr(ws), ws.numel(), T, ctypes.byref(packed.desc), _ptr(Y),
                                      _stream(stream))
    _check("w4a4_gemm_prequantized", st)


def w4a4_linear(X: torch.Tensor, packed: PackedLayer, Y: torch.Tensor, ws: torch.Tensor,
                stream=None) -> None:
    T = _acts(X, packed.d_in)
    _out(Y, T, packed.d_out, torch.float32, "Y", X)
    _wsbuf(ws, X)
    st = lib().w4a4_linear(_ptr(X), _x_dtype(X), T, ctypes.byref(packed.desc), _ptr(Y), _ptr(ws),
                           ws.numel(), _stream(stream))
    _check("w4a4_linear", st)


def w4a4_linear_noalloc(X: torch.Tensor, packed: PackedLayer, Y: torch.Tensor, stream=None) -> None:
    """w4a4_linear with the workspace in the library's fixed device scratch (for callers
    that cannot allocate); raises W4A4Error with W4A4_ERR_SCRATCH when T tokens need
    more than NOALLOC_SCRATCH_BYTES."""
    T = _acts(X, packed.d_in)
    _out(Y, T, packed.d_out, torch.float32, "Y", X)
    st = lib().w4a4_linear_noalloc(_ptr(X), _x_dtype(X), T, ctypes.byref(packed.desc), _ptr(Y), _stream(stream))
    _check("w4a4_linear_noalloc", st)


def w4a4_gemm_prequantized_gelu_bf16(ws: torch.Tensor, T: int, packed: PackedLayer, H: torch.Tensor,
                                     stream=None) -> None:
    _out(H, T, packed.d_out, torch.bfloat16, "H")
    _wsbuf(ws, H)
    st = lib().w4a4_gemm_prequantized_gelu_bf16(_ptr(ws), ws.numel(), T, ctypes.byref(packed.desc), _ptr(H),
                                                _stream(stream))
    _check("w4a4_gemm_prequantized_gelu_bf16", st)


def w4a4_linear_gelu_bf16(X: torch.Tensor, packed: PackedLayer, H: torch.Tensor, ws: torch.Tensor,
                          stream=None) -> None:
    T = _acts(X, packed.d_in)
    _out(H, T, packed.d_out, torch.bfloat16, "H", X)
    _wsbuf(ws, X)
    st = lib().w4a4_linear_gelu_bf16(_ptr(X), _x_dtype(X), T, ctypes.byref(packed.desc), _ptr(H), _ptr(ws),
                                      ws.numel(), _stream(stream))
    _check("w4a4_linear_gelu_bf16", st)


def w4a4_gelu_tanh_bf16(Y: torch.Tensor, H: torch.Tensor, stream=None) -> None:
    _dev(Y, "Y")
    _dev(H, "H")
    if Y.dtype != torch.float32 or H.dtype != torch.bfloat16:
        raise TypeError(f"Y must be float32 and H bfloat16, got {Y.dtype} and {H.dtype}")
    if Y.shape != H.shape or Y.device != H.device:
        raise ValueError(f"H must match Y's shape and device: {tuple(H.shape)} vs {tuple(Y.shape)}")
    st = lib().w4a4_gelu_tanh_bf16(_ptr(Y), Y.numel(), _ptr(H), _stream(stream))
    _check("w4a4_gelu_tanh_bf16", st)


def ffn_permutation(O_down: np.ndarray, d_ff: int) -> np.ndarray:
    """Row order of W_up for the fused FFN block: the down layer's J columns
    (ascending), then its O columns (ascending)."""
    O = np.sort(np.asarray(O_down, dtype=np.int64))
    J = np.setdiff1d(np.arange(d_ff), O)
    return np.concatenate([J, O]).astype(np.int64)


def w4a4_ffn_workspace_layout(T: int, up: PackedLayer, down: PackedLayer) -> W4A4FfnWsLayout:
    out = W4A4FfnWsLayout()
    _check("w4a4_ffn_workspace_layout",
           lib().w4a4_ffn_workspace_layout(T, ctypes.byref(up.desc), ctypes.byref(down.desc), ctypes.byref(out)))
    return out


def alloc_workspace_ffn(T: int, up: PackedLayer, down: PackedLayer, device="cuda") -> torch.Tensor:
    return torch.empty(max(w4a4_ffn_workspace_layout(T, up, down).total, 256), dtype=torch.uint8, device=device)


def ffn_workspace_views(ws: torch.Tensor, T: int, up: PackedLayer, down: PackedLayer) -> dict:
    """The down layer's quantized activations inside an FFN workspace, as
    workspace_views gives them for a workspace of the down layer alone."""
    L = w4a4_ffn_workspace_layout(T, up, down)
    return workspace_views(ws[L.down_base:L.down_base + L.down.total], T, down)


def w4a4_ffn_up_quantize(X: torch.Tensor, up: PackedLayer, down: PackedLayer, ws: torch.Tensor, stream=None) -> None:
    T = _acts(X, up.d_in)
    _wsbuf(ws, X)
    st = lib().w4a4_ffn_up_quantize(_ptr(X), _x_dtype(X), T, ctypes.byref(up.desc), ctypes.byref(down.desc),
                                    _ptr(ws), ws.numel(), _stream(stream))
    _check("w4a4_ffn_up_quantize", st)


def w4a4_ffn_forward(X: torch.Tensor, up: PackedLayer, down: PackedLayer, Y: torch.Tensor, ws: torch.Tensor,
                     stream=None) -> None:
    T = _acts(X, up.d_in)
    _out(Y, T, down.d_out, torch.float32, "Y", X)
    _wsbuf(ws, X)
    st = lib().w4a4_ffn_forward(_ptr(X), _x_dtype(X), T, ctypes.byref(up.desc), ctypes.byref(down.desc), _ptr(Y),
                                _ptr(ws), ws.numel(), _stream(stream))
    _check("w4a4_ffn_forward", st)
