"""Second, independently written formulation of the MXFP4 quantizer (numpy).

TEST INFRASTRUCTURE ONLY.  It exists to pin the C oracle: the oracle decides E2M1
codes with a closed-form threshold table and the E8M0 exponent with ``frexp`` in
double; this module decides codes by a nearest-grid search with even-code ties and
the exponent from the binary32 bit fields.  A mistake in either shows up as a
disagreement between the two.  It also offers a plain dequantizer so that the
degenerate cases can be checked against ``numpy.matmul``.

Format: MXFP4 (named in "W4A4 Quantization for Inference on Wan2.2-I2V-A14B (ICME
2026 Challenge)", sections 1-2) as the OCP MX formats define it: E2M1 elements with
one E8M0 power-of-two scale per 32 elements.
"""
from __future__ import annotations

import numpy as np

GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


def floor_log2_from_bits(a: np.ndarray) -> np.ndarray:
    """floor(log2 a) for positive finite binary32 values, read from the bit fields."""
    u = np.asarray(a, dtype=np.float32).view(np.uint32).astype(np.int64)
    e = (u >> 23) & 0xFF
    m = u & 0x7FFFFF
    out = e - 127
    sub = e == 0
    if np.any(sub):
        # subnormal: value = m * 2^-149, floor(log2) = -149 + bit_length(m) - 1
        ms = m[sub]
        bl = np.floor(np.log2(np.maximum(ms, 1).astype(np.float64))).astype(np.int64)
        # guard the float log2 near powers of two with exact integer checks
        bl = np.where((1 << (bl + 1)) <= ms, bl + 1, bl)
        bl = np.where((1 << bl) > ms, bl - 1, bl)
        out[sub] = -149 + bl
    return out


def e8m0(amax: np.ndarray) -> np.ndarray:
    """Scale code per group maximum: 2^(code-127) with code-127 = floor(log2 amax)-2."""
    a = np.asarray(amax, dtype=np.float32)
    code = np.zeros(a.shape, dtype=np.int64)
    fin = np.isfinite(a)
    pos = fin & (a > 0)
    code[~fin] = 0xFF
    if np.any(pos):
        E = floor_log2_from_bits(a[pos]) - 2
        code[pos] = np.maximum(E, -127) + 127
    return code.astype(np.uint8)


def e2m1_nearest(v: np.ndarray) -> np.ndarray:
    """Nearest E2M1 grid point (by search), ties to the even code, saturating."""
    v = np.asarray(v, dtype=np.float64)
    m = np.abs(v)
    d = np.abs(m[..., None] - GRID)                     # distance to every grid point
    best = d.min(axis=-1, keepdims=True)
    cand = d == best                                     # one or two candidates
    idx = np.arange(8)
    # prefer even index among ties: give odd indices a penalty
    pick = np.where(cand, (idx % 2) * 8 + idx, 1000).argmin(axis=-1)
    pick = np.where(m > 6.0, 7, pick)
    sign = np.signbit(v).astype(np.int64) * 8
    return (sign + pick).astype(np.uint8)


def dequant_code(code: np.ndarray) -> np.ndarray:
    c = np.asarray(code).astype(np.int64)
    val = GRID[c & 7]
    return np.where(c & 8, -val, val)


def quant_group(vals: np.ndarray) -> tuple[np.ndarray, int]:
    v = np.asarray(vals, dtype=np.float32).ravel()
    if not np.all(np.isfinite(v)):
        return np.zeros(v.size, dtype=np.uint8), 0xFF
    amax = np.float32(np.max(np.abs(v))) if v.size else np.float32(0)
    sc = int(e8m0(np.array([amax]))[0])
    E = sc - 127
    scaled = v.astype(np.float64) * (2.0 ** (-E))
    return e2m1_nearest(scaled), sc


def quant_rows_1x32(V: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Quantize a [R, K] fp32 matrix (K a multiple of 32) with one scale per 32 along
    K.  Returns (codes [R, K] uint8, scales [R, K/32] uint8)."""
    V = np.asarray(V, dtype=np.float32)
    R, K = V.shape
    Vb = V.reshape(R, K // 32, 32)
    fin = np.all(np.isfinite(Vb), axis=-1)
    amax = np.max(np.abs(np.where(np.isfinite(Vb), Vb, 0)), axis=-1).astype(np.float32)
    sc = e8m0(amax).astype(np.int64)
    sc = np.where(fin, sc, 0xFF)
    E = np.where(sc == 0xFF, 0, sc - 127)
    with np.errstate(invalid="ignore", over="ignore"):
        scaled = Vb.astype(np.float64) * np.exp2(-E.astype(np.float64))[..., None]
    codes = e2m1_nearest(np.where(np.isfinite(scaled), scaled, 0.0))
    codes = np.where(fin[..., None], codes, 0).astype(np.uint8)
    return codes.reshape(R, K), sc.astype(np.uint8)


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] & 0xF) | ((c[..., 1::2] & 0xF) << 4)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def dequant_1x32(Q: np.ndarray, S: np.ndarray) -> np.ndarray:
    """[R, K/2] packed codes + [R, K/32] scales -> fp64 [R, K]."""
    codes = unpack_nibbles(Q)
    R, K = codes.shape
    vals = dequant_code(codes).reshape(R, K // 32, 32)
    s = np.where(S == 0xFF, np.nan, np.exp2(S.astype(np.float64) - 127.0))
    return (vals * s[..., None]).reshape(R, K)


def dequant_weights(Bq: np.ndarray, Bs: np.ndarray, layout: int, d_out: int) -> np.ndarray:
    """Weights in any of the three scale layouts -> fp64 [d_out, K_pad]."""
    codes = unpack_nibbles(Bq)
    K = codes.shape[1]
    vals = dequant_code(codes)
    kk = np.arange(K)
    nn = np.arange(d_out)
    if layout == 0:
        sc = Bs[:, kk // 32]
    elif layout == 2:
        sc = Bs[:, kk // 128]
    else:
        sc = Bs[(kk // 32)[None, :], (nn // 32)[:, None]]
    s = np.where(sc == 0xFF, np.nan, np.exp2(sc.astype(np.float64) - 127.0))
    return vals * s


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 round-to-nearest-even by the usual bias-and-truncate on the bits."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    return np.where(nan, ((u >> 16) | 0x40).astype(np.uint16), r)


def bf16_to_f64(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
