"""Python face of the CPU oracle (``w4a4_oracle.c``) for the W4A4 dual-branch linear.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py``; never by the library.  It shares no code with the
HIP path.  Every function here marshals numpy arrays into the C oracle; the arithmetic
lives in ``w4a4_oracle.c`` (see its header for the citations and the readings taken).

Pages cited: [R] = "W4A4 Quantization for Inference on Wan2.2-I2V-A14B (ICME 2026
Challenge)" (xllm-io paper-review blog page), sections 3.2-3.5.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "w4a4_oracle.c")
_LIB = os.path.join(_HERE, "libw4a4_oracle.so")

LAYOUT_1X32 = 0
LAYOUT_TILE32 = 1
LAYOUT_STRIPE128 = 2

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no FMA contraction, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=gnu99", "-ffp-contract=off", "-fno-fast-math",
               "-fopenmp", "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        _lib = ctypes.CDLL(_LIB)
        i64, i32, vp, f32 = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_float
        L = _lib
        L.orc_bf16_value.restype = ctypes.c_double
        L.orc_bf16_value.argtypes = [ctypes.c_uint16]
        L.orc_bf16_round_double.restype = ctypes.c_uint16
        L.orc_bf16_round_double.argtypes = [ctypes.c_double]
        L.orc_bf16_round_f32.restype = ctypes.c_uint16
        L.orc_bf16_round_f32.argtypes = [f32]
        L.orc_e8m0_code.restype = ctypes.c_uint8
        L.orc_e8m0_code.argtypes = [f32]
        L.orc_e2m1_code.restype = ctypes.c_uint8
        L.orc_e2m1_code.argtypes = [ctypes.c_double]
        L.orc_e2m1_value.restype = ctypes.c_double
        L.orc_e2m1_value.argtypes = [ctypes.c_uint8]
        L.orc_e8m0_codes.restype = None
        L.orc_e8m0_codes.argtypes = [vp, i64, vp]
        L.orc_e2m1_codes.restype = None
        L.orc_e2m1_codes.argtypes = [vp, i64, vp]
        L.orc_bf16_round_f32_many.restype = None
        L.orc_bf16_round_f32_many.argtypes = [vp, i64, vp]
        L.orc_quant_group.restype = None
        L.orc_quant_group.argtypes = [vp, i64, vp, vp]
        L.orc_col_absmax.restype = ctypes.c_int
        L.orc_col_absmax.argtypes = [vp, ctypes.c_int, i64, i64, vp]
        L.orc_smoothing.restype = None
        L.orc_smoothing.argtypes = [vp, vp, i64, f32, vp]
        L.orc_scores.restype = None
        L.orc_scores.argtypes = [vp, vp, i64, vp]
        L.orc_select_outliers.restype = None
        L.orc_select_outliers.argtypes = [vp, i64, i32, vp, vp]
        L.orc_weight_scale_bytes.restype = i64
        L.orc_weight_scale_bytes.argtypes = [i64, i64, ctypes.c_int]
        L.orc_pack_weights.restype = None
        L.orc_pack_weights.argtypes = [vp, i64, i64, vp, vp, i64, vp, i32, ctypes.c_int, i64,
                                       vp, vp, vp]
        L.orc_act_prep.restype = None
        L.orc_act_prep.argtypes = [vp, ctypes.c_int, i64, i64, vp, vp, i64, vp, i32, i64,
                                   vp, vp, vp]
        L.orc_output_element.restype = ctypes.c_double
        L.orc_output_pairs.restype = None
        L.orc_output_pairs.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i32, ctypes.c_int,
                                       vp, vp, i64, vp]
        L.orc_output_full.restype = None
        L.orc_output_full.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, ctypes.c_int, vp]
        L.orc_gelu_bf16.restype = None
        L.orc_gelu_bf16.argtypes = [vp, i64, vp]
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p) if a.size else ctypes.c_void_p(0)


def _x_arg(X: np.ndarray):
    """Activations are fp32 arrays or bf16 bit patterns held in uint16 arrays."""
    X = np.ascontiguousarray(X)
    if X.dtype == np.uint16:
        return X, 1
    if X.dtype == np.float32:
        return X, 0
    raise TypeError(f"oracle activations must be float32 or bf16 bits (uint16), got {X.dtype}")


def k_pad_of(K_J: int) -> int:
    """J-compacted K rounded up to a multiple of 128."""
    return ((K_J + 127) // 128) * 128


# ----------------------------------------------------------------- scalars

def bf16_round(x: np.ndarray) -> np.ndarray:
    L = _load()
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32).ravel())
    out = np.zeros(x.size, dtype=np.uint16)
    L.orc_bf16_round_f32_many(_p(x), x.size, _p(out))
    return out


def e8m0_codes(amax: np.ndarray) -> np.ndarray:
    L = _load()
    a = np.ascontiguousarray(np.asarray(amax, dtype=np.float32).ravel())
    out = np.zeros(a.size, dtype=np.uint8)
    L.orc_e8m0_codes(_p(a), a.size, _p(out))
    return out


def e2m1_codes(v: np.ndarray) -> np.ndarray:
    L = _load()
    a = np.ascontiguousarray(np.asarray(v, dtype=np.float64).ravel())
    out = np.zeros(a.size, dtype=np.uint8)
    L.orc_e2m1_codes(_p(a), a.size, _p(out))
    return out


def bf16_value(h) -> np.ndarray:
    L = _load()
    return np.array([L.orc_bf16_value(int(v)) for v in np.asarray(h).ravel()], dtype=np.float64)


def e8m0_code(amax: float) -> int:
    return int(_load().orc_e8m0_code(float(np.float32(amax))))


def e2m1_code(v: float) -> int:
    return int(_load().orc_e2m1_code(float(v)))


def e2m1_value(code: int) -> float:
    return float(_load().orc_e2m1_value(int(code)))


def quant_group(vals) -> tuple[np.ndarray, int]:
    """Quantize one scale group of fp32 values: (codes[n], e8m0 code)."""
    L = _load()
    v = np.ascontiguousarray(np.asarray(vals, dtype=np.float32).ravel())
    codes = np.zeros(v.size, dtype=np.uint8)
    sc = np.zeros(1, dtype=np.uint8)
    L.orc_quant_group(_p(v), v.size, _p(codes), _p(sc))
    return codes, int(sc[0])


# ----------------------------------------------------------------- calibration

def col_absmax(X: np.ndarray) -> np.ndarray:
    L = _load()
    X, is_bf16 = _x_arg(X)
    rows, cols = X.shape
    out = np.zeros(cols, dtype=np.float32)
    bad = L.orc_col_absmax(_p(X), is_bf16, rows, cols, _p(out))
    if bad:
        raise ValueError("non-finite calibration data")
    return out


def smoothing(act_scale: np.ndarray, weight_scale: np.ndarray, alpha: float) -> np.ndarray:
    L = _load()
    a = np.ascontiguousarray(act_scale, dtype=np.float32)
    w = np.ascontiguousarray(weight_scale, dtype=np.float32)
    s = np.zeros(a.size, dtype=np.float32)
    L.orc_smoothing(_p(a), _p(w), a.size, float(alpha), _p(s))
    return s


def scores(act_scale: np.ndarray, s: np.ndarray) -> np.ndarray:
    L = _load()
    a = np.ascontiguousarray(act_scale, dtype=np.float32)
    s = np.ascontiguousarray(s, dtype=np.float32)
    out = np.zeros(a.size, dtype=np.float32)
    L.orc_scores(_p(a), _p(s), a.size, _p(out))
    return out


def select_outliers(score: np.ndarray, k: int) -> tuple[np.ndarray, np.ndarray]:
    L = _load()
    sc = np.ascontiguousarray(score, dtype=np.float32)
    d_in = sc.size
    O = np.zeros(k, dtype=np.int32)
    J = np.zeros(d_in - k, dtype=np.int32)
    L.orc_select_outliers(_p(sc), d_in, int(k), _p(O), _p(J))
    return O, J


def calibrate(X_cal: np.ndarray, W: np.ndarray, alpha: float, k: int):
    """Steps of [R] sec. 3.2-3.3 on calibration data: returns (s, O, J, act_scale,
    weight_scale, score).  W is fp32 [d_out, d_in]."""
    act = col_absmax(X_cal)
    wsc = col_absmax(np.ascontiguousarray(W, dtype=np.float32))
    s = smoothing(act, wsc, alpha)
    sc = scores(act, s)
    O, J = select_outliers(sc, k)
    return s, O, J, act, wsc, sc


# ----------------------------------------------------------------- packing

def weight_scale_shape(d_out: int, K_pad: int, layout: int) -> tuple[int, int]:
    if layout == LAYOUT_1X32:
        return (d_out, K_pad // 32)
    if layout == LAYOUT_STRIPE128:
        return (d_out, K_pad // 128)
    return (K_pad // 32, (d_out + 31) // 32)


def pack_weights(W: np.ndarray, s: np.ndarray, O: np.ndarray, J: np.ndarray, layout: int):
    L = _load()
    W = np.ascontiguousarray(W, dtype=np.float32)
    d_out, d_in = W.shape
    s = np.ascontiguousarray(s, dtype=np.float32)
    O = np.ascontiguousarray(O, dtype=np.int32)
    J = np.ascontiguousarray(J, dtype=np.int32)
    K_J = J.size
    K_pad = k_pad_of(K_J)
    k = O.size
    Bq = np.zeros((d_out, K_pad // 2), dtype=np.uint8)
    Bs = np.zeros(weight_scale_shape(d_out, K_pad, layout), dtype=np.uint8)
    WO = np.zeros((d_out, k), dtype=np.uint16)
    L.orc_pack_weights(_p(W), d_in, d_out, _p(s), _p(J), K_J, _p(O), k, layout, K_pad,
                       _p(Bq), _p(Bs), _p(WO))
    return {"Bq": Bq, "Bs": Bs, "WO": WO, "K_pad": K_pad, "layout": layout,
            "d_in": d_in, "d_out": d_out, "k": k}


def act_prep(X: np.ndarray, s: np.ndarray, O: np.ndarray, J: np.ndarray):
    L = _load()
    X, is_bf16 = _x_arg(X)
    T, d_in = X.shape
    s = np.ascontiguousarray(s, dtype=np.float32)
    O = np.ascontiguousarray(O, dtype=np.int32)
    J = np.ascontiguousarray(J, dtype=np.int32)
    K_J = J.size
    K_pad = k_pad_of(K_J)
    k = O.size
    Aq = np.zeros((T, K_pad // 2), dtype=np.uint8)
    As = np.zeros((T, K_pad // 32), dtype=np.uint8)
    XO = np.zeros((T, k), dtype=np.uint16)
    L.orc_act_prep(_p(X), is_bf16, T, d_in, _p(s), _p(J), K_J, _p(O), k, K_pad,
                   _p(Aq), _p(As), _p(XO))
    return Aq, As, XO


def output_pairs(Aq, As, XO, packed, ts, ns) -> np.ndarray:
    L = _load()
    ts = np.ascontiguousarray(ts, dtype=np.int64)
    ns = np.ascontiguousarray(ns, dtype=np.int64)
    Y = np.zeros(ts.size, dtype=np.float64)
    L.orc_output_pairs(_p(np.ascontiguousarray(Aq)), _p(np.ascontiguousarray(As)),
                       _p(np.ascontiguousarray(XO)), _p(packed["Bq"]), _p(packed["Bs"]),
                       _p(packed["WO"]), packed["d_out"], packed["K_pad"], packed["k"],
                       packed["layout"], _p(ts), _p(ns), ts.size, _p(Y))
    return Y


def output_full(Aq, As, XO, packed) -> np.ndarray:
    L = _load()
    T = Aq.shape[0]
    Y = np.zeros((T, packed["d_out"]), dtype=np.float64)
    L.orc_output_full(_p(np.ascontiguousarray(Aq)), _p(np.ascontiguousarray(As)),
                      _p(np.ascontiguousarray(XO)), _p(packed["Bq"]), _p(packed["Bs"]),
                      _p(packed["WO"]), T, packed["d_out"], packed["K_pad"], packed["k"],
                      packed["layout"], _p(Y))
    return Y


def linear(X, s, O, J, packed) -> np.ndarray:
    """Whole per-call path in the oracle: act-prep then the dual-branch output."""
    Aq, As, XO = act_prep(X, s, O, J)
    return output_full(Aq, As, XO, packed)


def x_values(X: np.ndarray) -> np.ndarray:
    """Activation values in fp64: fp32 as is, bf16 bit patterns widened exactly."""
    if X.dtype == np.uint16:
        return (X.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return X.astype(np.float64)


def select_outliers_dynamic(X: np.ndarray, s: np.ndarray, k: int) -> np.ndarray:
    """Per-call outlier columns (the online selection that [R] sec. 3.3 and sec. 4
    attribute to MixQ): score_j = fl32(max_t |x_tj| / s_j) on the call's own tokens,
    ordered by the binary32 bit pattern of |score| (numeric for finite values and +Inf,
    a NaN above +Inf), larger first, ties to the smaller column; the top k, ascending."""
    # max_t |x_tj| as the largest |x| bit pattern (the numeric maximum, or a NaN)
    xb = (X.astype(np.uint32) << 16) if X.dtype == np.uint16 else np.ascontiguousarray(X, np.float32).view(np.uint32)
    act = (xb & np.uint32(0x7FFFFFFF)).max(axis=0).astype(np.uint32).view(np.float32)
    with np.errstate(invalid="ignore"):
        sc = act / np.asarray(s, dtype=np.float32)
    bits = (sc.view(np.uint32) & np.uint32(0x7FFFFFFF)).astype(np.int64)
    order = np.lexsort((np.arange(bits.size), -bits))
    return np.sort(order[:k]).astype(np.int32)


def linear_dynamic(X: np.ndarray, W: np.ndarray, s: np.ndarray, k: int, layout: int):
    """The layer with per-call outliers: O from select_outliers_dynamic; the MXFP4
    branch keeps every column at its own K position (J = 0..d_in-1, the weights packed
    once with no outlier column) with the O columns of X set to zero, and the BF16
    branch is bf16 X_O . bf16 W_O.  Returns (Y, O, A_q, A_s, X_O, W_O)."""
    d_in = X.shape[1]
    O = select_outliers_dynamic(X, s, k)
    J_all = np.arange(d_in, dtype=np.int32)
    Xz = np.array(X, copy=True)
    Xz[:, O] = 0
    Aq, As, _ = act_prep(Xz, s, np.zeros(0, np.int32), J_all)
    Jc = np.setdiff1d(J_all, O).astype(np.int32)
    _, _, XO = act_prep(X, s, O, Jc)
    pk = pack_weights(W, s, np.zeros(0, np.int32), J_all, layout)
    pk["WO"] = pack_weights(W, s, O, Jc, layout)["WO"]
    pk["k"] = int(O.size)
    return output_full(Aq, As, XO, pk), O, Aq, As, XO, pk["WO"]


def search_alpha_k(X_cal: np.ndarray, W: np.ndarray, alphas, ks, layout: int):
    """Layer-wise alpha and k ([R] sec. 3.2: alpha in [0.5, 0.7] for the FFN up
    projection; sec. 4 lists per-layer alpha and k; sec. 6 names tuning them per layer
    as the next step).  The pages give no selection rule; the one taken is the smallest
    output error on the calibration tokens: for every (alpha, k), calibrate, pack, run
    the layer on X_cal and score it by ||Y_q - X_cal W^T||_F / ||X_cal W^T||_F, the
    reference product in fp64.  Returns (errors [n_alpha, n_k], (a, b) of the smallest
    error, the first in row-major order on ties)."""
    Yref = x_values(X_cal) @ np.asarray(W, dtype=np.float64).T
    nref = np.linalg.norm(Yref)
    errs = np.empty((len(alphas), len(ks)), dtype=np.float64)
    for a, alpha in enumerate(alphas):
        for b, k in enumerate(ks):
            s, O, J, _, _, _ = calibrate(X_cal, W, float(alpha), int(k))
            pk = pack_weights(W, s, O, J, layout)
            errs[a, b] = np.linalg.norm(linear(X_cal, s, O, J, pk) - Yref) / nref
    a, b = np.unravel_index(int(np.argmin(errs)), errs.shape)
    return errs, (int(a), int(b))


def gelu_bf16(Y: np.ndarray) -> np.ndarray:
    L = _load()
    Y = np.ascontiguousarray(Y, dtype=np.float32)
    H = np.zeros(Y.shape, dtype=np.uint16)
    L.orc_gelu_bf16(_p(Y), Y.size, _p(H))
    return H
