"""GPU parity of every step of the path against the CPU oracle, through the C ABI.

Codes, scales, the column map, s and O must be bit-exact; Y must meet the output
tolerance (tests/gpu_util.py).  Shapes span several 256x256 output tiles with ragged
tails in T, d_out, K_J and k, both activation dtypes and all three weight layouts,
plus the degenerate cases k = 0, k = d_in and special values.
"""
import numpy as np
import pytest
import torch

from bit_quantized_dit_amd import synth
from bit_quantized_dit_amd import w4a4 as B
from tests.gpu_util import (_banner, _check_act, _check_packed, _check_y_full, _layer,
                            assert_y_close, bf16_bits, to_dev, u8)

pytestmark = pytest.mark.gpu


SMALL = [
    # T, d_in, d_out, k, layout, dtype
    (300, 704, 200, 13, 0, "bf16"),
    (300, 700, 200, 13, 0, "f32"),      # d_in % 8 != 0: scalar load path
    (257, 1000, 333, 40, 1, "bf16"),    # 32x32 tiles, ragged last tile
    (129, 1536, 130, 64, 2, "f32"),     # 128x1 stripes
    (64, 5120, 256, 128, 0, "bf16"),    # K_J = 4992: odd number of 128-steps
    (1, 512, 64, 16, 2, "bf16"),
    (77, 333, 96, 5, 0, "f32"),         # odd d_in: the generic act-prep kernel
    (45, 333, 70, 7, 1, "bf16"),        # odd d_in, bf16 rows at odd element offsets
    (40, 20000, 64, 16, 0, "bf16"),     # d_in beyond the fast act-prep paths (16384)
    # split K (fewer tiles than CUs): each tile runs as several K ranges whose partial
    # sums a second launch adds up
    (70, 4608, 300, 512, 0, "bf16"),    # 3 ranges of 16 steps: the last is all BF16 steps
    (600, 6400, 520, 24, 2, "f32"),     # 9 ragged tiles x 3 ranges
    (64, 7168, 256, 128, 0, "bf16"),    # the last range mixes FP4 and BF16 steps
    (1, 8192, 100, 16, 1, "bf16"),      # one token, ragged outputs, 32x32 tiles, 4 ranges
]


@pytest.mark.parametrize("T,d_in,d_out,k,layout,dt", SMALL)
def test_layer_parity(orc, T, d_in, d_out, k, layout, dt):
    _banner(f"layer T={T} d_in={d_in} d_out={d_out} k={k} layout={layout} {dt}")
    spec = synth.WORKLOADS[2 if dt == "bf16" else 1]
    inp = synth.layer_inputs(spec, T=T, d_in=d_in, d_out=d_out, k=k, T_cal=97)
    r = _layer(orc, inp["X"], inp["X_cal"], inp["W"], spec.alpha, k, layout)
    _check_packed(r)
    _check_y_full(orc, r, inp["X"])


@pytest.mark.parametrize("layout", [0, 1, 2])
def test_k0_naive_w4a4(orc, layout):
    """k = 0 and s = 1: the plain MXFP4 GEMM (no outlier branch, no smoothing)."""
    _banner(f"naive layout={layout}")
    rng = np.random.default_rng(20 + layout)
    T, d_in, d_out = 200, 384, 160
    X = (rng.standard_normal((T, d_in)) * 0.5).astype(np.float32)
    W = (rng.standard_normal((d_out, d_in)) * 0.05).astype(np.float32)
    s = np.ones(d_in, np.float32)
    O = np.zeros(0, np.int32)
    J = np.arange(d_in, dtype=np.int32)
    packed = B.w4a4_pack_weights(to_dev(W), s, O, layout)
    ws = B.alloc_workspace(T, packed)
    Y = torch.empty(T, d_out, device="cuda")
    B.w4a4_linear(to_dev(X), packed, Y, ws)
    torch.cuda.synchronize()
    r = {"s": s, "O": O, "J": J, "packed": packed, "ws": ws, "Y": Y,
         "pk_o": orc.pack_weights(W, s, O, J, layout), "T": T}
    _check_packed(r)
    _check_y_full(orc, r, X)


def test_k_equals_din_pure_bf16(orc):
    """k = d_in: J is empty, only the BF16 branch runs."""
    _banner("k = d_in")
    rng = np.random.default_rng(30)
    T, d_in, d_out = 150, 96, 140
    X = to_bits = synth.to_bf16_bits((rng.standard_normal((T, d_in))).astype(np.float32))
    W = (rng.standard_normal((d_out, d_in)) * 0.1).astype(np.float32)
    s = np.ones(d_in, np.float32)
    O = np.arange(d_in, dtype=np.int32)
    J = np.zeros(0, np.int32)
    packed = B.w4a4_pack_weights(to_dev(W), s, O, 0)
    assert packed.k_pad == 0
    ws = B.alloc_workspace(T, packed)
    Y = torch.empty(T, d_out, device="cuda")
    B.w4a4_linear(to_dev(to_bits), packed, Y, ws)
    torch.cuda.synchronize()
    r = {"s": s, "O": O, "J": J, "packed": packed, "ws": ws, "Y": Y,
         "pk_o": orc.pack_weights(W, s, O, J, 0), "T": T}
    _check_packed(r)
    _check_y_full(orc, r, X)


def test_special_values(orc):
    """NaN/Inf rows give 0xFF blocks and NaN outputs; subnormals, -0, exact E2M1 ties
    after division, and huge/tiny rows quantize bit-exactly."""
    _banner("special values")
    rng = np.random.default_rng(40)
    T, d_in, d_out = 64, 256, 96
    X = (rng.standard_normal((T, d_in)) * 0.3).astype(np.float32)
    X[1, 5] = np.nan
    X[2, 200] = np.inf
    X[3, :] = np.float32(2.0 ** -140)           # subnormal-only row
    X[4, :] = -0.0
    X[5, ::3] = np.float32(2.0 ** -127)
    X[6, :] *= np.float32(1e30)
    X[7, :] = np.array([0x1], np.uint32).view(np.float32)[0]
    X[8, :] = np.float32(3.0) * np.float32(2.5)  # divides to the tie 2.5 when s = 3
    X[8, 0] = np.float32(21.0)
    X[9, 3] = np.array([0xFFA5A5A5], np.uint32).view(np.float32)[0]   # NaN with payload, outlier column
    X[10, 77] = -np.inf                                                # -Inf, outlier column
    s = np.full(d_in, 3.0, np.float32)
    s[::7] = np.float32(0.37)
    W = (rng.standard_normal((d_out, d_in)) * 0.05).astype(np.float32)
    O = np.array([3, 77], np.int32)
    J = np.setdiff1d(np.arange(d_in), O).astype(np.int32)
    packed = B.w4a4_pack_weights(to_dev(W), s, O, 0)
    ws = B.alloc_workspace(T, packed)
    Y = torch.empty(T, d_out, device="cuda")
    B.w4a4_linear(to_dev(X), packed, Y, ws)
    torch.cuda.synchronize()
    r = {"s": s, "O": O, "J": J, "packed": packed, "ws": ws, "Y": Y,
         "pk_o": orc.pack_weights(W, s, O, J, 0), "T": T}
    Aq_o, As_o, XO_o = _check_act(orc, r, X)
    assert (As_o == 0xFF).any()
    Yref = orc.output_full(Aq_o, As_o, XO_o, r["pk_o"])
    assert_y_close(Y.cpu().numpy(), Yref)


def test_division_exhaustive_sample(orc):
    """IEEE binary32 division on the GPU: 2^22 fp32 patterns spread over all exponents
    (both signs) divided by assorted s, quantized in single-element-dominated blocks,
    compared bit-exactly with the oracle."""
    _banner("division sweep")
    rng = np.random.default_rng(50)
    pats = (np.arange(1 << 22, dtype=np.uint64) * 1021) % (1 << 32)
    X = pats.astype(np.uint32).view(np.float32).reshape(-1, 256)
    X = np.where(np.isfinite(X), X, np.float32(1.0)).astype(np.float32)
    s = rng.uniform(0.01, 100, 256).astype(np.float32)
    s[:8] = np.array([3.0, 1.0, 0.5, 7.0, 0x3FFD37D0, 1e-5, 1e5, 1.1], np.float32)
    s[4] = np.array([0x3FFD37D0], np.uint32).view(np.float32)[0]
    O = np.zeros(0, np.int32)
    J = np.arange(256, dtype=np.int32)
    W = np.ones((32, 256), np.float32) * 0.01
    packed = B.w4a4_pack_weights(to_dev(W), s, O, 0)
    T = X.shape[0]
    ws = B.alloc_workspace(T, packed)
    B.w4a4_quantize_activations(to_dev(X), packed, ws)
    torch.cuda.synchronize()
    r = {"s": s, "O": O, "J": J, "packed": packed, "ws": ws, "T": T}
    _check_act(orc, r, X)


def test_e2m1_threshold_neighbourhoods(orc):
    """Every binary32 pattern within 4096 ulps of each E2M1 rounding threshold
    {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5} * 2^E and of the saturation region
    {6, 8 - ulp} * 2^E, both signs, for block exponents E = -127 (the subnormal
    scale), -126, -20, 0, 60 and 125: each 32-block holds one element that pins E
    (1.5 * 2^(E+2)) and 31 swept values, with s = 1 so the codes are the quantizer
    alone.  Codes and scales must match the oracle bit for bit."""
    _banner("E2M1 threshold neighbourhoods")
    thr = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 7.999999], np.float64)
    vals = []
    for E in (-127, -126, -20, 0, 60, 125):
        for t in thr:
            c = (np.float64(t) * np.float64(2.0) ** E)
            if c < np.finfo(np.float32).tiny / 2 ** 23 or c > np.finfo(np.float32).max:
                continue
            centre = np.array([c], np.float32).view(np.int32)[0]
            pats = (centre + np.arange(-4096, 4097, dtype=np.int64)).clip(1, 0x7F7FFFFF).astype(np.uint32)
            v = pats.view(np.float32)
            pin = np.float32(1.5 * 2.0 ** (E + 2))           # floor(log2) = E + 2 pins E
            v = v[np.abs(v.astype(np.float64)) < 2.0 ** (E + 3)]   # in-group: |v| < 2^(E+3)
            v = v[:(v.size // 31) * 31].reshape(-1, 31)
            blocks = np.concatenate([np.full((v.shape[0], 1), pin, np.float32), v], axis=1)
            neg = -blocks
            vals.append(blocks)
            vals.append(neg)
    X = np.concatenate(vals).reshape(-1)
    d_in = 1024
    X = np.concatenate([X, np.zeros((-X.size) % d_in, np.float32)]).reshape(-1, d_in)
    s = np.ones(d_in, np.float32)
    O = np.zeros(0, np.int32)
    J = np.arange(d_in, dtype=np.int32)
    W = np.ones((32, d_in), np.float32) * 0.01
    packed = B.w4a4_pack_weights(to_dev(W), s, O, 0)
    T = X.shape[0]
    ws = B.alloc_workspace(T, packed)
    B.w4a4_quantize_activations(to_dev(X), packed, ws)
    torch.cuda.synchronize()
    r = {"s": s, "O": O, "J": J, "packed": packed, "ws": ws, "T": T}
    _check_act(orc, r, X)
    _banner(f"  {X.size} elements in {T} rows")


@pytest.mark.parametrize("T,d_in,d_out,k,layout,dt", [(300, 700, 203, 13, 0, "f32"), (520, 1000, 512, 40, 2, "bf16"),
                                                     (200, 8192, 300, 20, 0, "bf16")])   # split K
def test_fused_gelu_matches_unfused(orc, T, d_in, d_out, k, layout, dt):
    """w4a4_linear_gelu_bf16 writes exactly w4a4_gelu_tanh_bf16(w4a4_linear(X)), on a
    ragged tile grid and (203 outputs) the unvectorised store path."""
    _banner(f"fused GELU T={T} d_in={d_in} d_out={d_out}")
    spec = synth.WORKLOADS[1]
    inp = synth.layer_inputs(spec, T=T, d_in=d_in, d_out=d_out, k=k, T_cal=128)
    X = inp["X"] if dt == "f32" else synth.to_bf16_bits(inp["X"])
    Xd, Xcd, Wd = to_dev(X), to_dev(inp["X_cal"]), to_dev(inp["W"])
    s, O, _, _ = B.w4a4_calibrate_scales(Xcd, Wd, spec.alpha, k)
    packed = B.w4a4_pack_weights(Wd, s, O, layout)
    ws = B.alloc_workspace(T, packed)
    Y = torch.empty(T, d_out, dtype=torch.float32, device="cuda")
    B.w4a4_linear(Xd, packed, Y, ws)
    H = torch.empty(T, d_out, dtype=torch.bfloat16, device="cuda")
    B.w4a4_gelu_tanh_bf16(Y, H)
    Hf = torch.full((T, d_out), float("nan"), dtype=torch.bfloat16, device="cuda")
    B.w4a4_linear_gelu_bf16(Xd, packed, Hf, ws)
    torch.cuda.synchronize()
    assert bool(torch.equal(Hf.view(torch.int16), H.view(torch.int16)))


@pytest.mark.parametrize("rows,cols,dt,offset", [
    (333, 1111, "f32", 0),      # odd column count: super-rows of 4 rows
    (333, 1111, "bf16", 0),     # super-rows of 8 rows, 5 rows past the last one
    (1001, 5120, "bf16", 0),    # one row per super-row
    (77, 6, "f32", 0),          # two rows per super-row, a single workgroup column
    (5, 3, "bf16", 0),          # fewer rows than one super-row: all element by element
    (4096, 704, "bf16", 0),
    (333, 1111, "f32", 1),      # X not 16-byte aligned: the scalar kernel
])
def test_column_absmax_bits(orc, rows, cols, dt, offset):
    """Column max |x| as bit patterns, exact against the oracle; a NaN shows as a
    pattern at or above +Inf's."""
    rng = np.random.default_rng(60 + rows + cols)
    X = (rng.standard_normal((rows, cols)) * rng.uniform(0, 5, cols)).astype(np.float32)
    X[rows // 2, cols - 1] = -7.5e3
    Xin = synth.to_bf16_bits(X) if dt == "bf16" else X
    want = orc.col_absmax(Xin).view(np.uint32)
    Xd = to_dev(Xin)
    if offset:
        flat = torch.empty(rows * cols + offset, dtype=Xd.dtype, device="cuda")
        flat[offset:] = Xd.reshape(-1)
        Xd = flat[offset:].view(rows, cols)
    out = B.w4a4_column_absmax(Xd)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint32), want)
    if dt == "f32" and not offset:
        X[rows - 1, 0] = np.nan
        out = B.w4a4_column_absmax(to_dev(X))
        assert out.cpu().numpy().view(np.uint32)[0] >= 0x7F800000


DYN = [
    # T, d_in, d_out, k, layout, dtype, special values
    (300, 704, 200, 13, 0, "bf16", False),
    (129, 1536, 130, 64, 2, "f32", False),
    (257, 1000, 333, 40, 1, "bf16", True),
    (64, 512, 96, 0, 0, "bf16", False),
    (40, 256, 64, 256, 0, "f32", False),      # k = d_in: every column in the BF16 branch
    (700, 16384, 64, 100, 0, "bf16", False),  # the largest d_in of the per-call path
    (96, 5120, 80, 128, 0, "bf16", "ties"),   # few distinct scores: ties decide the choice
    (33, 2, 40, 1, 1, "f32", "ties"),         # the smallest d_in
    (1, 512, 64, 8, 2, "bf16", False),        # a single token
]


@pytest.mark.parametrize("T,d_in,d_out,k,layout,dt,special", DYN)
def test_dynamic_outliers_match_oracle(orc, T, d_in, d_out, k, layout, dt, special):
    """Per-call outlier selection: O and the column map exact, the un-compacted codes and
    scales, X_O and the gathered W_O bit-exact, Y within the output tolerance."""
    _banner(f"dynamic outliers T={T} d_in={d_in} d_out={d_out} k={k} layout={layout} {dt}")
    rng = np.random.default_rng(1000 + d_in + k)
    X = (rng.standard_normal((T, d_in)) * 0.3).astype(np.float32)
    heavy = rng.choice(d_in, size=min(d_in, 2 * k + 3), replace=False)
    X[:, heavy] *= rng.uniform(4, 20, heavy.size).astype(np.float32)
    s = rng.uniform(0.5, 2.0, d_in).astype(np.float32)
    if special == "ties":
        X = rng.choice(np.array([0.0, 0.5, 1.0, 2.0, -3.0], np.float32), size=(T, d_in))
        X[:, heavy[: k // 2]] *= 4
        s = np.ones(d_in, np.float32)
    elif special:
        X[3, heavy[0]] = np.nan
        X[5, heavy[1]] = -np.inf
        X[7, 11] = 3e38
    if dt == "bf16":
        X = synth.to_bf16_bits(X)
    W = (rng.standard_normal((d_out, d_in)) * 0.02).astype(np.float32)
    pk = B.w4a4_pack_weights_dyn(to_dev(W), s, k, layout)
    ws = B.alloc_workspace_dyn(T, pk)
    Y = torch.empty(T, d_out, dtype=torch.float32, device="cuda")
    B.w4a4_linear_dyn(to_dev(X), pk, Y, ws)
    torch.cuda.synchronize()
    Yo, O, Aq, As, XO, WO = orc.linear_dynamic(X, W, s, k, layout)
    v = B.workspace_dyn_views(ws, T, pk)
    assert np.array_equal(v["O"].cpu().numpy(), O), "O differs"
    cm = np.arange(d_in, dtype=np.int32)
    cm[O] = -(np.arange(O.size) + 1)
    assert np.array_equal(v["colmap"].cpu().numpy(), cm), "column map differs"
    assert np.array_equal(u8(v["A_s"]), As), "A_s differs"
    assert np.array_equal(u8(v["A_q"]), Aq), "A_q differs"
    if k:
        xo, wo = bf16_bits(v["X_O"]), bf16_bits(v["W_O"])
        assert np.array_equal(xo[:, :k], XO) and not xo[:, k:].any(), "X_O differs"
        assert np.array_equal(wo[:, :k], WO) and not wo[:, k:].any(), "W_O differs"
    st = assert_y_close(Y.cpu().numpy(), Yo)
    _banner(f"  {st}")


FFN_FUSED = [
    # T, d_model, d_ff, k_up, k_down, layout_up, layout_down, dtype, NaN token
    (300, 256, 704, 8, 13, 0, 2, "bf16", False),   # k_j = 691: one 32-block holds J and O features
    (129, 512, 1024, 0, 64, 1, 0, "f32", True),    # k_j = 960: two zero pad blocks up to k_pad = 1024
    (64, 256, 512, 16, 0, 0, 0, "bf16", False),    # no down-layer outliers
    (257, 384, 640, 4, 128, 2, 1, "bf16", False),  # k_j = 512 = k_pad: no pad
    (70, 256, 700, 6, 12, 0, 0, "bf16", False),    # d_ff = 700: the block at 672 holds J, O and
                                                   # columns past d_ff
    (100, 6144, 512, 8, 16, 0, 2, "bf16", False),  # the up GEMM split along K (3 ranges)
    (64, 256, 8192, 4, 16, 0, 0, "bf16", False),   # the down GEMM split along K (4 ranges)
]


@pytest.mark.parametrize("T,d_model,d_ff,k_up,k_down,lu,ld,dt,nan", FFN_FUSED)
def test_ffn_fused_quantization_matches_unfused(orc, T, d_model, d_ff, k_up, k_down, lu, ld, dt, nan):
    """The FFN block with the down layer's act-prep in the up GEMM's epilogue: the down
    layer's A_q, A_s and X_O bit-identical to act-prep of the unfused H (GELU fused
    into the up GEMM, columns put back in H's order) and to the oracle's act-prep of
    that H; the down output bit-identical to the down GEMM over the unfused codes."""
    _banner(f"fused FFN T={T} {d_model}->{d_ff}->{d_model} k_up={k_up} k_down={k_down} {dt}")
    rng = np.random.default_rng(500 + d_ff + k_down)
    X = (rng.standard_normal((T, d_model)) * 0.5).astype(np.float32)
    X[:, rng.choice(d_model, 5, replace=False)] *= 8
    if nan:
        X[7, 3] = np.nan
    Xc = (rng.standard_normal((96, d_model)) * 0.5).astype(np.float32)
    W_up = (rng.standard_normal((d_ff, d_model)) * 0.05).astype(np.float32)
    W_dn = (rng.standard_normal((d_model, d_ff)) * 0.05).astype(np.float32)
    s_up, O_up, _, _ = B.w4a4_calibrate_scales(to_dev(Xc), to_dev(W_up), 0.6, k_up)
    s_dn = rng.uniform(0.5, 2.0, d_ff).astype(np.float32)
    O_dn = np.sort(rng.choice(d_ff, k_down, replace=False)).astype(np.int32)
    P = B.ffn_permutation(O_dn, d_ff)
    up = B.w4a4_pack_weights(to_dev(W_up[P]), s_up, O_up, lu)
    down = B.w4a4_pack_weights(to_dev(W_dn), s_dn, O_dn, ld)
    Xd = to_dev(synth.to_bf16_bits(X) if dt == "bf16" else X)
    ws = B.alloc_workspace_ffn(T, up, down)
    ws.fill_(0xA5)        # whatever the fused path leaves unwritten shows up
    Y = torch.empty(T, d_model, dtype=torch.float32, device="cuda")
    B.w4a4_ffn_forward(Xd, up, down, Y, ws)
    fz = B.ffn_workspace_views(ws, T, up, down)
    # unfused: H in the permuted order, put back in H's column order, then act-prep
    wsu = B.alloc_workspace(T, up)
    Hp = torch.empty(T, d_ff, dtype=torch.bfloat16, device="cuda")
    B.w4a4_linear_gelu_bf16(Xd, up, Hp, wsu)
    H = torch.empty_like(Hp)
    H[:, torch.as_tensor(P, device="cuda")] = Hp
    wsd = B.alloc_workspace(T, down)
    B.w4a4_quantize_activations(H, down, wsd)
    rf = B.workspace_views(wsd, T, down)
    Y2 = torch.empty_like(Y)
    B.w4a4_gemm_prequantized(wsd, T, down, Y2)
    torch.cuda.synchronize()
    assert np.array_equal(u8(fz["A_s"]), u8(rf["A_s"])), "A_s differs"
    assert np.array_equal(u8(fz["A_q"]), u8(rf["A_q"])), "A_q differs"
    assert np.array_equal(bf16_bits(fz["X_O"]), bf16_bits(rf["X_O"])), "X_O differs"
    assert bool(torch.equal(Y.view(torch.int32), Y2.view(torch.int32))), "down output differs"
    J_dn = np.setdiff1d(np.arange(d_ff), O_dn).astype(np.int32)
    Aq_o, As_o, XO_o = orc.act_prep(bf16_bits(H), s_dn, O_dn, J_dn)
    assert np.array_equal(u8(fz["A_s"]), As_o) and np.array_equal(u8(fz["A_q"]), Aq_o)
    assert np.array_equal(bf16_bits(fz["X_O"])[:, :k_down], XO_o) and not bf16_bits(fz["X_O"])[:, k_down:].any()
    _banner(f"  codes, scales, X_O and Y identical (NaN rows: {int(np.isnan(Y.cpu().numpy()).any(axis=1).sum())})")


@pytest.mark.parametrize("dt,layout", [("f32", 0), ("bf16", 0), ("bf16", 1), ("f32", 2)])
def test_search_alpha_k_matches_oracle(orc, dt, layout):
    """The layer-wise alpha / k search: every candidate's error against the oracle's
    (its calibration, pack and output, and an fp64 reference product), the same choice
    unless the oracle's best two are within the tolerance of each other, and two runs
    bitwise equal."""
    spec = synth.WORKLOADS[1]
    inp = synth.layer_inputs(spec)
    Xc, W = inp["X_cal"], inp["W"]
    if dt == "bf16":
        Xc = synth.to_bf16_bits(Xc)
    alphas, ks = [0.5, 0.6, 0.7], [0, 16, 32]
    _banner(f"alpha/k search {dt} layout={layout} T_cal={Xc.shape[0]} d_in={Xc.shape[1]} d_out={W.shape[0]}")
    eg, bg = B.w4a4_search_alpha_k(to_dev(Xc), to_dev(W), alphas, ks, layout)
    eg2, bg2 = B.w4a4_search_alpha_k(to_dev(Xc), to_dev(W), alphas, ks, layout)
    eo, bo = orc.search_alpha_k(Xc, W, alphas, ks, layout)
    _banner(f"  gpu {np.array2string(eg, precision=5)} best {bg}; oracle best {bo}")
    assert np.array_equal(eg, eg2) and bg == bg2
    # Tolerance from the two error sources.  E = ||Yq - Yr|| / ||Yr|| on both sides;
    # the GPU's Yq' = Yq + a with ||a|| <= 1e-5 ||Yq|| (the GEMM's relative Frobenius
    # bar, checked on every parity layer) and ||Yq|| <= (1 + E) ||Yr||; its reference
    # Yr' = Yr + b is a sequential fp32 FMA chain over K = d_in terms, so elementwise
    # |b| <= gamma_K (|X| |W|^T) with gamma_K = K u / (1 - K u), u = 2^-24 (the standard
    # bound for recursive summation of products).  Then
    # |E' - E| <= (||a|| + (1 + E) ||b||) / (||Yr|| - ||b||).
    xv = orc.x_values(Xc)
    Yr = xv @ np.asarray(W, np.float64).T
    K = xv.shape[1]
    u = 2.0 ** -24
    gamma = K * u / (1 - K * u)
    nb = gamma * np.linalg.norm(np.abs(xv) @ np.abs(np.asarray(W, np.float64)).T)
    nr = np.linalg.norm(Yr)
    tol = (1e-5 * (1 + eo) * nr + (1 + eo) * nb) / (nr - nb)
    _banner(f"  max |E_gpu - E_oracle| {np.abs(eg - eo).max():.3e}, bound {tol.min():.3e} .. {tol.max():.3e}")
    assert np.all(np.abs(eg - eo) <= tol)
    if bg != bo:
        assert eo[bg] - eo[bo] <= tol[bg] + tol[bo]


def test_calibration_rejects_nonfinite():
    X = np.ones((16, 64), np.float32)
    X[3, 3] = np.inf
    W = np.ones((32, 64), np.float32)
    with pytest.raises(B.W4A4Error) as e:
        B.w4a4_calibrate_scales(to_dev(X), to_dev(W), 0.5, 4)
    assert e.value.status == 5


def test_determinism_and_prequantized_split(orc):
    """Two runs are bitwise equal; act-prep + GEMM as separate calls equals w4a4_linear."""
    spec = synth.WORKLOADS[2]
    inp = synth.layer_inputs(spec, T=512, d_in=1024, d_out=384, k=32, T_cal=128)
    r = _layer(orc, inp["X"], inp["X_cal"], inp["W"], spec.alpha, 32, 0)
    Xd = to_dev(inp["X"])
    Y2 = torch.empty_like(r["Y"])
    ws2 = torch.empty_like(r["ws"])
    B.w4a4_quantize_activations(Xd, r["packed"], ws2)
    B.w4a4_gemm_prequantized(ws2, r["T"], r["packed"], Y2)
    torch.cuda.synchronize()
    assert torch.equal(r["Y"].view(torch.int32), Y2.view(torch.int32))
    Y3 = torch.empty_like(r["Y"])
    B.w4a4_linear(Xd, r["packed"], Y3, ws2)
    torch.cuda.synchronize()
    assert torch.equal(r["Y"].view(torch.int32), Y3.view(torch.int32))


SPLIT = [
    # T, d_in, d_out, k, layout: shapes whose GEMM the plan splits along K
    (64, 7168, 256, 128, 0),     # 1 tile x 3 ranges; the last mixes FP4 and BF16 steps
    (70, 4608, 300, 512, 0),     # the last range is BF16 steps only
    (600, 6400, 520, 24, 2),     # 9 ragged tiles x 3 ranges
    (40, 20000, 64, 16, 0),      # 9 ranges
]


@pytest.mark.parametrize("T,d_in,d_out,k,layout", SPLIT)
def test_split_k_is_planned_and_deterministic(T, d_in, d_out, k, layout):
    """These shapes take the split-K path (a partial-sum region in the workspace), and
    their results are bitwise reproducible: the partial sums are added in a fixed order
    (the oracle comparison of the same shapes is in test_layer_parity)."""
    _banner(f"split K T={T} d_in={d_in} d_out={d_out} k={k}")
    spec = synth.WORKLOADS[2]
    inp = synth.layer_inputs(spec, T=T, d_in=d_in, d_out=d_out, k=k, T_cal=64)
    X, Xc, W = to_dev(inp["X"]), to_dev(inp["X_cal"]), to_dev(inp["W"])
    s, O, _, _ = B.w4a4_calibrate_scales(Xc, W, spec.alpha, k)
    packed = B.w4a4_pack_weights(W, s, O, layout)
    L = B.w4a4_workspace_layout(T, packed)
    assert L.total - L.partial >= 256 * 256 * 4 * 3, "the plan does not split this shape"
    ws = B.alloc_workspace(T, packed)
    ws.fill_(0x7F)                      # stale partial sums must not leak into Y
    Y1 = torch.empty(T, d_out, device="cuda")
    B.w4a4_linear(X, packed, Y1, ws)
    Y2 = torch.full((T, d_out), float("nan"), device="cuda")
    B.w4a4_linear(X, packed, Y2, ws)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(Y1).all())
    assert bool(torch.equal(Y1.view(torch.int32), Y2.view(torch.int32)))


def test_half_tiles_match_whole_tiles():
    """A layer with at most 128 output tiles runs as 256 x 128 half tiles; each output
    keeps its K order and MFMA sequence, so the rows equal bit for bit those that a
    larger call (140 whole tiles) computes for the same tokens (act-prep is per token)."""
    _banner("half tiles against whole tiles: 256 of 17920 tokens, 1024 -> 512")
    spec = synth.WORKLOADS[2]
    inp = synth.layer_inputs(spec, T=17920, d_in=1024, d_out=512, k=32, T_cal=64)
    X, Xc, W = to_dev(inp["X"]), to_dev(inp["X_cal"]), to_dev(inp["W"])
    s, O, _, _ = B.w4a4_calibrate_scales(Xc, W, spec.alpha, 32)
    packed = B.w4a4_pack_weights(W, s, O, 0)
    Y = torch.empty(17920, 512, device="cuda")
    B.w4a4_linear(X, packed, Y, B.alloc_workspace(17920, packed))
    Xs = X[:256].contiguous()
    Ys = torch.full((256, 512), float("nan"), device="cuda")
    B.w4a4_linear(Xs, packed, Ys, B.alloc_workspace(256, packed))
    torch.cuda.synchronize()
    assert bool(torch.equal(Ys.view(torch.int32), Y[:256].view(torch.int32)))


def test_error_paths_on_device():
    W = torch.zeros(64, 128, device="cuda")
    packed = B.w4a4_pack_weights(W, np.ones(128, np.float32), np.array([1, 2], np.int32), 0)
    X = torch.zeros(10, 128, device="cuda")
    Y = torch.empty(10, 64, device="cuda")
    ws = B.alloc_workspace(10, packed)
    with pytest.raises(B.W4A4Error) as e:
        B.w4a4_linear(X, packed, Y, ws[:100])
    assert e.value.status == 2
    with pytest.raises(B.W4A4Error) as e:
        B.w4a4_pack_weights(W, np.ones(128, np.float32), np.array([2, 1], np.int32), 0)
    assert e.value.status == 1
    with pytest.raises(B.W4A4Error) as e:
        B.w4a4_pack_weights(W, -np.ones(128, np.float32), np.array([1], np.int32), 0)
    assert e.value.status == 1
    big = torch.empty(10 * 128 + 4, device="cuda")
    with pytest.raises(B.W4A4Error) as e:
        B.w4a4_linear(big[1:1281].view(10, 128), packed, Y, ws)
    assert e.value.status == 3
    # the binding refuses tensors that do not match what the kernels read or write,
    # before anything reaches the library
    with pytest.raises(ValueError):
        B.w4a4_linear(torch.zeros(10, 127, device="cuda"), packed, Y, ws)
    with pytest.raises(ValueError):
        B.w4a4_linear(X, packed, torch.empty(10, 63, device="cuda"), ws)
    with pytest.raises(TypeError):
        B.w4a4_linear(X, packed, torch.empty(10, 64, device="cuda", dtype=torch.bfloat16), ws)
    with pytest.raises(TypeError):
        B.w4a4_linear(X, packed, Y, ws.view(torch.int32))
    with pytest.raises(ValueError):
        B.w4a4_gemm_prequantized(ws, 11, packed, Y)
    with pytest.raises(TypeError):
        B.w4a4_linear_gelu_bf16(X, packed, Y, ws)
    with pytest.raises(ValueError):
        B.w4a4_gelu_tanh_bf16(Y, torch.empty(10, 32, device="cuda", dtype=torch.bfloat16))
    with pytest.raises(TypeError):
        B.w4a4_gelu_tanh_bf16(Y.to(torch.bfloat16), torch.empty(10, 64, device="cuda", dtype=torch.bfloat16))


def test_gelu_kernel(orc, mini):
    """GPU GELU-tanh in fp32 vs the oracle's double-precision formula: at most one bf16
    ulp apart wherever |GELU| >= 2^-120, and the mismatch count is small.  The kernel
    evaluates x / (1 + exp(-2z)) in binary32, whose exp overflows once the exact result
    is below |x| 2^-128 (< 2^-124 here): such results come out as a signed zero, so
    below 2^-120 only smallness and the sign are checked."""
    rng = np.random.default_rng(70)
    Yh = np.concatenate([rng.standard_normal(1 << 20) * 3, np.linspace(-12, 12, 4097),
                         np.linspace(-10.5, -5, 4097)]).astype(np.float32)
    H = torch.empty(Yh.size, dtype=torch.bfloat16, device="cuda")
    B.w4a4_gelu_tanh_bf16(to_dev(Yh), H)
    torch.cuda.synchronize()
    got = bf16_bits(H)
    ref = orc.gelu_bf16(Yh)
    a = mini.bf16_to_f64(got)
    b = mini.bf16_to_f64(ref)
    big = np.abs(b) >= 2.0 ** -120
    ulp = np.abs(b[big]) * 2.0 ** -7
    assert np.all(np.abs(a[big] - b[big]) <= ulp)
    assert np.all(np.abs(a[~big]) < 2.0 ** -120)
    assert np.all(np.signbit(a) == np.signbit(b))
    mism = int(np.sum(got[big] != ref[big]))
    _banner(f"gelu mismatches: {mism} of {int(big.sum())}")
    assert mism <= big.sum() // 1000
