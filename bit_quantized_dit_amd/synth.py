"""Seeded synthetic inputs for the W4A4 dual-branch linear (shared by tests and bench).

This module only draws random numbers with the shapes and tail statistics of the
workloads; it holds none of the method's arithmetic.  The pages measure on Wan2.2
FFN activations from OpenS2V-5M prompts, which are not available; these draws stand
in for them with the statistics the review page reports ("W4A4 Quantization for
Inference on Wan2.2-I2V-A14B (ICME 2026 Challenge)", sec. 3.1: activation column
maxima above 6 with a visible tail beyond 1.5, weight column maxima below 0.6).

Arrays are numpy: fp32 as float32, bf16 as its bit pattern in uint16 (rounded to
nearest even by torch's CPU conversion).  Seeds: base 1000*c for workload c, with
sub-streams +1 heavy-column indices, +2 run activations, +3 calibration activations,
+4 up weights, +5 down weights, +6 heavy-column targets.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch


@dataclass
class LayerSpec:
    name: str
    T: int
    d_in: int
    d_out: int
    k: int
    alpha: float
    layout: int              # 0 = 1x32, 1 = 32x32 tiles, 2 = 128x1 stripes
    x_dtype: str             # "f32" or "bf16"
    recipe: str              # "normal_rescaled" | "normal_t3" | "gelu_x8"
    n_heavy: int
    w_sigma: float
    w_clip: float | None
    T_cal: int
    seed: int
    extra: dict = field(default_factory=dict)


# The five workloads: a tiny W4A4 linear, the Wan-like FFN up projection at 4096 tokens,
# the FFN down projection, the full 720x1280x61 token count (57600 tokens), and the full
# FFN block at that token count.
WORKLOADS = {
    1: LayerSpec("tiny_256x512x1024_k16", 256, 512, 1024, 16, 0.5, 0, "f32", "normal_rescaled",
                 16, 0.02, 0.6, 256, 1000),
    2: LayerSpec("ffn_up_T4096_5120x13824_k64", 4096, 5120, 13824, 64, 0.6, 0, "bf16",
                 "normal_t3", 64, 0.02, None, 1024, 2000),
    3: LayerSpec("ffn_down_T4096_13824x5120_k64", 4096, 13824, 5120, 64, 0.5, 2, "bf16",
                 "gelu_x8", 64, 0.01, None, 1024, 3000),
    4: LayerSpec("ffn_up_T57600_5120x13824_k128", 57600, 5120, 13824, 128, 0.7, 0, "bf16",
                 "normal_t3", 128, 0.02, None, 1024, 4000),
}
# Full FFN block at 57600 tokens: up as workload 4 but with 32x32 weight tiles, then
# GELU-tanh, then the down projection 13824->5120 (k=64, alpha 0.5, 128x1 stripes).
# The block's input activations and up weights are workload 4's draws (same seed).
FFN_BLOCK = {
    "up": LayerSpec("ffn_block_up_T57600_5120x13824_k128", 57600, 5120, 13824, 128, 0.7, 1,
                    "bf16", "normal_t3", 128, 0.02, None, 1024, 4000),
    "down": LayerSpec("ffn_block_down_T57600_13824x5120_k64", 57600, 13824, 5120, 64, 0.5, 2,
                      "bf16", "from_up", 0, 0.01, None, 1024, 4000),
}


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def heavy_columns(spec: LayerSpec, d_in: int | None = None, n_heavy: int | None = None) -> np.ndarray:
    d_in = spec.d_in if d_in is None else d_in
    n = spec.n_heavy if n_heavy is None else n_heavy
    return np.sort(_rng(spec.seed + 1).choice(d_in, size=min(n, d_in), replace=False)).astype(np.int64)


def _activations(spec: LayerSpec, T: int, d_in: int, cols: np.ndarray, stream: int) -> np.ndarray:
    """fp32 activations following the workload's recipe."""
    g = _rng(spec.seed + stream)
    if spec.recipe == "normal_rescaled":
        X = g.standard_normal((T, d_in), dtype=np.float32) * np.float32(0.3)
        targets = _rng(spec.seed + 6).uniform(6.0, 12.0, size=cols.size).astype(np.float32)
        for c, tgt in zip(cols, targets):
            m = np.max(np.abs(X[:, c]))
            if m > 0:
                X[:, c] *= np.float32(tgt / m)
        return X
    if spec.recipe == "normal_t3":
        X = g.standard_normal((T, d_in), dtype=np.float32) * np.float32(0.3)
        if cols.size:
            tails = np.clip(g.standard_t(3.0, size=(T, cols.size)) * 2.0, -12.0, 12.0)
            X[:, cols] = tails.astype(np.float32)
        return X
    if spec.recipe == "gelu_x8":
        pre = torch.from_numpy(g.standard_normal((T, d_in), dtype=np.float32))
        X = torch.nn.functional.gelu(pre, approximate="tanh").numpy()
        if cols.size:
            X[:, cols] *= np.float32(8.0)
        return X
    raise ValueError(spec.recipe)


def weights(spec: LayerSpec, d_in: int | None = None, d_out: int | None = None,
            stream: int = 4) -> np.ndarray:
    d_in = spec.d_in if d_in is None else d_in
    d_out = spec.d_out if d_out is None else d_out
    W = _rng(spec.seed + stream).standard_normal((d_out, d_in), dtype=np.float32)
    W *= np.float32(spec.w_sigma)
    if spec.w_clip is not None:
        np.clip(W, -spec.w_clip, spec.w_clip, out=W)
    return W


def layer_inputs(spec: LayerSpec, T: int | None = None, d_in: int | None = None,
                 d_out: int | None = None, k: int | None = None, T_cal: int | None = None):
    """Run activations, calibration activations and fp32 weights for one layer.

    Sizes may be overridden (tests use smaller shapes with the same recipe); the
    number of heavy columns follows k when k is overridden."""
    T = spec.T if T is None else T
    d_in = spec.d_in if d_in is None else d_in
    d_out = spec.d_out if d_out is None else d_out
    k = spec.k if k is None else k
    T_cal = spec.T_cal if T_cal is None else T_cal
    n_heavy = spec.n_heavy if (k == spec.k) else min(max(k, 1), d_in)
    cols = heavy_columns(spec, d_in, n_heavy)
    X = _activations(spec, T, d_in, cols, 2)
    Xc = _activations(spec, T_cal, d_in, cols, 3)
    W = weights(spec, d_in, d_out, 4)
    if spec.x_dtype == "bf16":
        X, Xc = to_bf16_bits(X), to_bf16_bits(Xc)
    return {"X": X, "X_cal": Xc, "W": W, "alpha": spec.alpha, "k": k, "layout": spec.layout,
            "heavy": cols, "T": T, "d_in": d_in, "d_out": d_out}


def down_calibration(up_cal_bits: np.ndarray, W_up: np.ndarray) -> np.ndarray:
    """Calibration activations for the FFN down projection: the unquantized fp32 up
    projection of the calibration tokens, rounded to bf16, through torch's GELU-tanh,
    rounded to bf16 again (bf16 bits)."""
    Xc = torch.from_numpy(bf16_bits_to_f32(up_cal_bits))
    Yc = Xc @ torch.from_numpy(W_up).t()
    Yc = Yc.to(torch.bfloat16).float()
    H = torch.nn.functional.gelu(Yc, approximate="tanh").to(torch.bfloat16)
    return H.view(torch.int16).numpy().view(np.uint16)
