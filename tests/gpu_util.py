"""Shared helpers of the GPU parity tests: device transfer and the output tolerance."""
from __future__ import annotations

import numpy as np
import torch

from bit_quantized_dit_amd import w4a4 as B

# Output tolerance of the fp32 GEMM against the oracle's fp64 sum of the same codes:
# max |dY| <= 1e-3 * max |Y_ref| and ||dY||_F / ||Y_ref||_F <= 1e-5.
Y_MAX_REL = 1e-3
Y_FRO_REL = 1e-5


def to_dev(X: np.ndarray) -> torch.Tensor:
    """numpy fp32, or bf16 bit patterns in uint16, -> device tensor of that dtype."""
    if X.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(X).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(X, dtype=np.float32)).cuda()


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def u8(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().cpu().numpy().view(np.uint8)


def assert_y_close(Y: np.ndarray, Yref: np.ndarray, what: str = "Y") -> dict:
    Y = np.asarray(Y, dtype=np.float64)
    Yref = np.asarray(Yref, dtype=np.float64)
    nan_ref = np.isnan(Yref)
    assert np.array_equal(np.isnan(Y), nan_ref), f"{what}: NaN pattern differs"
    inf_ref = np.isinf(Yref)
    assert np.array_equal(Y[inf_ref], Yref[inf_ref]) and not np.isinf(Y[~inf_ref]).any(), \
        f"{what}: infinities differ"
    fin = ~nan_ref & ~inf_ref
    d = np.abs(Y[fin] - Yref[fin])
    scale = np.abs(Yref[fin]).max() if fin.any() else 0.0
    max_rel = float(d.max() / scale) if d.size and scale > 0 else float(d.max() if d.size else 0.0)
    nrm = np.linalg.norm(Yref[fin])
    fro = float(np.linalg.norm(Y[fin] - Yref[fin]) / nrm) if nrm > 0 else float(np.linalg.norm(Y[fin]))
    assert max_rel <= Y_MAX_REL, f"{what}: max|dY|/max|Y| = {max_rel:.3e}"
    assert fro <= Y_FRO_REL, f"{what}: relative Frobenius error {fro:.3e}"
    return {"max_rel": max_rel, "fro_rel": fro}


def full_y_reference(mini, Aq, As, XO, pk, chunk: int = 1024) -> np.ndarray:
    """The layer's whole output in fp64 from the oracle's act-prep results and packed
    weights, as independently dequantized operands through numpy's matmul (the form
    the CPU pins prove equal to the oracle's own output sum in every weight layout),
    in token chunks so that a large layer stays within memory."""
    Wd = mini.dequant_weights(pk["Bq"], pk["Bs"], pk["layout"], pk["d_out"]).T.copy()
    WO = mini.bf16_to_f64(pk["WO"]).T.copy() if pk["k"] else None
    T = Aq.shape[0]
    Y = np.empty((T, pk["d_out"]), dtype=np.float64)
    for t0 in range(0, T, chunk):
        t1 = min(T, t0 + chunk)
        Y[t0:t1] = mini.dequant_1x32(Aq[t0:t1], As[t0:t1]) @ Wd
        if WO is not None:
            Y[t0:t1] += mini.bf16_to_f64(XO[t0:t1]) @ WO
    return Y


def _banner(msg):
    print(f"[gpu-test] {msg}", flush=True)


def _layer(orc, X, Xc, W, alpha, k, layout):
    """Calibrate + pack + linear on the GPU; the oracle redoes each step on the same
    inputs.  Returns a dict of both sides' results."""
    Xd, Xcd, Wd = to_dev(X), to_dev(Xc), to_dev(W)
    s, O, act, wsc = B.w4a4_calibrate_scales(Xcd, Wd, alpha, k)
    s_o, O_o, J_o, act_o, wsc_o, _ = orc.calibrate(Xc, W, alpha, k)
    assert np.array_equal(act, act_o) and np.array_equal(wsc, wsc_o)
    ulp = np.abs(s.view(np.int32).astype(np.int64) - s_o.view(np.int32).astype(np.int64))
    assert ulp.max() <= 1, "s differs from the oracle by more than 1 ulp"
    assert np.array_equal(O, O_o)
    J = np.setdiff1d(np.arange(W.shape[1]), O).astype(np.int32)
    packed = B.w4a4_pack_weights(Wd, s, O, layout)
    T = X.shape[0]
    ws = B.alloc_workspace(T, packed)
    Y = torch.empty(T, W.shape[0], dtype=torch.float32, device="cuda")
    B.w4a4_linear(Xd, packed, Y, ws)
    torch.cuda.synchronize()
    # downstream steps use the library's s on both sides
    pk_o = orc.pack_weights(W, s, O, J, layout)
    return {"s": s, "O": O, "J": J, "packed": packed, "ws": ws, "Y": Y, "pk_o": pk_o, "T": T}


def _check_packed(r):
    v = r["packed"].views()
    pk = r["pk_o"]
    k = r["O"].size
    assert np.array_equal(v["s"].cpu().numpy(), r["s"])
    cm = v["colmap"].cpu().numpy()
    assert np.array_equal(cm[r["J"]], np.arange(r["J"].size))
    assert np.array_equal(cm[r["O"]], -(np.arange(k) + 1))
    if r["packed"].k_pad:
        assert np.array_equal(u8(v["B_q"]), pk["Bq"]), "B_q differs"
        # the GEMM's tiled copy holds the same codes, and zeros past d_out
        assert np.array_equal(u8(v["B_q_from_tiles"]), pk["Bq"]), "B_q_tiles differs"
        rows16 = (pk["d_out"] + 15) // 16 * 16
        if rows16 > pk["d_out"]:
            from bit_quantized_dit_amd.w4a4 import untile_codes
            full = untile_codes(v["B_q_tiles_raw"], rows16, pk["K_pad"])
            assert not bool(full[pk["d_out"]:].any()), "B_q_tiles padding rows not zero"
        assert np.array_equal(u8(v["B_s"]), pk["Bs"]), "B_s differs"
        # the GEMM's step-major per-row copy holds the group code of every (row, 32-block)
        d_out, K_pad, lay = pk["d_out"], pk["K_pad"], pk["layout"]
        kb = np.arange(K_pad // 32)
        nn = np.arange(d_out)
        if lay == 0:
            want = pk["Bs"]
        elif lay == 2:
            want = pk["Bs"][:, kb // 4]
        else:
            want = pk["Bs"][kb[None, :], (nn // 32)[:, None]]
        assert np.array_equal(u8(v["B_s_rows"]), want), "B_s_rows differs"
    if k:
        wo = bf16_bits(v["W_O"])
        assert np.array_equal(wo[:, :k], pk["WO"]), "W_O differs"
        assert np.all(wo[:, k:] == 0)


def _check_act(orc, r, X, rows=None):
    v = B.workspace_views(r["ws"], r["T"], r["packed"])
    Xs = X if rows is None else X[rows]
    Aq_o, As_o, XO_o = orc.act_prep(Xs, r["s"], r["O"], r["J"])
    sel = slice(None) if rows is None else torch.as_tensor(rows, device="cuda")
    Aq, As = u8(v["A_q"][sel]), u8(v["A_s"][sel])
    assert np.array_equal(As, As_o), "A_s differs"
    assert np.array_equal(Aq, Aq_o), "A_q differs"
    k = r["O"].size
    if k:
        xo = bf16_bits(v["X_O"][sel])
        assert np.array_equal(xo[:, :k], XO_o), "X_O differs"
        assert np.all(xo[:, k:] == 0)
    return Aq_o, As_o, XO_o


def check_act_all_rows(orc, views, X, s, O, J, chunk=8192, what="act-prep", y_gpu=None, pk=None, mini=None):
    """Every token row of the GPU's activation codes, scales and X_O equal the
    oracle's act-prep of the same rows ([R] sec. 3.2 and 3.3), bit for bit.  X is a
    host array (fp32, or bf16 bit patterns in uint16) or a device bf16 tensor (the
    GPU's own H, fed to the oracle as it is).  The comparison runs in chunks of rows
    so that the host never holds more than one chunk of codes.

    With y_gpu (the GPU's output, device tensor [T, d_out]), pk (the oracle's packed
    weights) and mini, every output is also compared with the GEMM tolerance: each
    chunk's reference is the dequantize-then-matmul form of the output sum over the
    oracle's codes of that chunk, and the maximum and Frobenius statistics are taken
    over all chunks.  Returns those statistics (or None)."""
    T = views["A_s"].shape[0]
    k = O.size
    aq_all, as_all, xo_all = views["A_q"], views["A_s"], views["X_O"]
    if y_gpu is not None:
        Wd = mini.dequant_weights(pk["Bq"], pk["Bs"], pk["layout"], pk["d_out"]).T.copy()
        WO = mini.bf16_to_f64(pk["WO"]).T.copy() if pk["k"] else None
        dmax = rmax = d2 = r2 = 0.0
    for t0 in range(0, T, chunk):
        t1 = min(T, t0 + chunk)
        Xc = X[t0:t1]
        if isinstance(Xc, torch.Tensor):
            Xc = bf16_bits(Xc)
        Aq_o, As_o, XO_o = orc.act_prep(Xc, s, O, J)
        assert np.array_equal(u8(as_all[t0:t1]), As_o), f"{what}: A_s differs in rows {t0}..{t1 - 1}"
        aq = u8(aq_all[t0:t1])
        if not np.array_equal(aq, Aq_o):
            r, c = np.argwhere(aq != Aq_o)[0]
            raise AssertionError(f"{what}: A_q differs first at row {t0 + r}, byte {c}: "
                                 f"{aq[r, c]:#04x} vs {Aq_o[r, c]:#04x}")
        if k:
            xo = bf16_bits(xo_all[t0:t1])
            assert np.array_equal(xo[:, :k], XO_o), f"{what}: X_O differs in rows {t0}..{t1 - 1}"
            assert not xo[:, k:].any(), f"{what}: X_O padding columns not zero"
        if y_gpu is not None:
            Yr = mini.dequant_1x32(Aq_o, As_o) @ Wd
            if WO is not None:
                Yr += mini.bf16_to_f64(XO_o) @ WO
            Yg = y_gpu[t0:t1].cpu().numpy().astype(np.float64)
            assert np.array_equal(np.isnan(Yg), np.isnan(Yr)), f"Y: NaN pattern differs in rows {t0}..{t1 - 1}"
            inf = np.isinf(Yr)
            assert np.array_equal(Yg[inf], Yr[inf]) and not np.isinf(Yg[~inf]).any(), \
                f"Y: infinities differ in rows {t0}..{t1 - 1}"
            fin = np.isfinite(Yr)
            d = Yg[fin] - Yr[fin]
            if d.size:
                dmax = max(dmax, float(np.abs(d).max()))
                rmax = max(rmax, float(np.abs(Yr[fin]).max()))
                d2 += float(np.dot(d, d))
                r2 += float(np.dot(Yr[fin], Yr[fin]))
    if y_gpu is None:
        return None
    st = {"max_rel": dmax / rmax if rmax > 0 else dmax, "fro_rel": (d2 ** 0.5) / (r2 ** 0.5) if r2 > 0 else d2 ** 0.5}
    assert st["max_rel"] <= Y_MAX_REL, f"Y (all outputs): max|dY|/max|Y| = {st['max_rel']:.3e}"
    assert st["fro_rel"] <= Y_FRO_REL, f"Y (all outputs): relative Frobenius error {st['fro_rel']:.3e}"
    return st


def _check_y_full(orc, r, X):
    Aq_o, As_o, XO_o = _check_act(orc, r, X)
    Yref = orc.output_full(Aq_o, As_o, XO_o, r["pk_o"])
    return assert_y_close(r["Y"].cpu().numpy(), Yref)


