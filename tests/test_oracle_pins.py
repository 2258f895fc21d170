"""Pins of the CPU oracle against what the pages and the mathematics fix (CPU only).

Each test names the fact it pins.  Pages: [R] = "W4A4 Quantization for Inference on
Wan2.2-I2V-A14B (ICME 2026 Challenge)" (xllm-io review), sec. 3.2-3.5; MXFP4 as the
OCP MX formats define it (E2M1 elements, E8M0 scale per 32).
"""
import json
import os

import numpy as np
import pytest
import torch

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _num(v):
    if isinstance(v, str):
        return float(v)   # "-0"
    return float(v)


# ------------------------------------------------------------- worked example

@pytest.fixture(scope="module")
def worked():
    with open(os.path.join(GOLD, "worked_2x32.json")) as f:
        return json.load(f)


def _worked_inputs(w, with_outlier):
    X = np.array([[_num(v) for v in row] for row in w["x_rows"]], dtype=np.float32)
    W = np.stack([np.ones(32, np.float32), np.tile(np.array([1, -1], np.float32), 16)])
    if with_outlier:
        X = np.concatenate([X, np.array(w["outlier"]["x_O"], np.float32)[:, None]], axis=1)
        W = np.concatenate([W, np.array(w["outlier"]["w_O"], np.float32)[:, None]], axis=1)
    d_in = X.shape[1]
    s = np.ones(d_in, np.float32)
    O = np.array([32] if with_outlier else [], np.int32)
    J = np.arange(32, dtype=np.int32)
    return X, W, s, O, J


def test_worked_example_activation_codes(orc, worked):
    """Hand-worked 2x32 rows: scale codes, nibbles, packed bytes (low nibble = even K)."""
    X, W, s, O, J = _worked_inputs(worked, False)
    Aq, As, XO = orc.act_prep(X, s, O, J)
    assert As.shape == (2, 4)  # K_pad = 128: one real block + 3 zero pad blocks
    assert list(As[:, 0]) == worked["x_scale_codes"]
    assert np.all(As[:, 1:] == 0)
    for r in range(2):
        pref = worked["x_bytes_prefix"][r]
        assert list(Aq[r, :len(pref)]) == pref
        codes = np.empty(32, np.uint8)
        codes[0::2] = Aq[r, :16] & 0xF
        codes[1::2] = Aq[r, :16] >> 4
        assert list(codes) == worked["x_codes"][r]
        deq = [orc.e2m1_value(c) * 2.0 ** (worked["x_scale_codes"][r] - 127) for c in codes]
        want = [_num(v) for v in worked["x_dequant"][r]]
        assert deq == want
        assert [np.signbit(v) for v in deq] == [np.signbit(v) for v in want]


def test_worked_example_weights_and_output(orc, worked):
    """Weight codes/scales of the worked example and Y = [[20,14],[44,12]]; with one
    outlier column ([R] sec. 3.3 dual branch) Y = [[25,16.5],[42.5,11.25]]."""
    for with_outlier, key in ((False, None), (True, "outlier")):
        X, W, s, O, J = _worked_inputs(worked, with_outlier)
        pk = orc.pack_weights(W, s, O, J, orc.LAYOUT_1X32)
        assert list(pk["Bs"][:, 0]) == worked["w_scale_codes"]
        assert np.all(pk["Bq"][0, :16] == worked["w_bytes"][0])
        assert np.all(pk["Bq"][1, :16] == worked["w_bytes"][1])
        Y = orc.linear(X, s, O, J, pk)
        want = worked["outlier"]["Y_k1"] if with_outlier else worked["Y_k0"]
        assert Y.tolist() == want


def test_edge_blocks(orc, worked):
    """Clipping block [7.9, 0...] -> code 7 under scale 0x7F; subnormal-only blocks
    clamp E at -127 (scale 0x00); 2^-127 scales to exactly 1 -> code 2."""
    for e in worked["edge_blocks"]:
        blk = np.zeros(32, np.float32)
        if "block_head" in e:
            blk[0] = e["block_head"][0]
        elif "block_head_bits" in e:
            blk[0] = np.array([e["block_head_bits"][0]], np.uint32).view(np.float32)[0]
        else:
            blk[0] = np.float32(2.0 ** e["block_head_pow2"][0])
        codes, sc = orc.quant_group(blk)
        assert sc == e["scale_code"]
        assert codes[0] == e["codes_head"][0]
        assert np.all(codes[1:] == 0)


def test_division_is_correctly_rounded(orc, worked):
    """x / s is one IEEE binary32 division.  With s = 0x3FFD37D0 (1.97826576...) and
    x = fl(2.5 s) the quotient is exactly 2.5, an E2M1 tie that goes to the even code 4
    (2.0); the reciprocal-multiply x * fl(1/s) gives 2.5000002 and would give code 5.
    Also fl(1/3) = 0x3EAAAAAB."""
    assert (np.float32(1.0) / np.float32(3.0)).view(np.uint32) == worked["one_third_f32_bits"]
    s1 = np.array([0x3FFD37D0], np.uint32).view(np.float32)[0]
    x1 = np.float32(2.5) * s1
    assert float(x1) / float(s1) == 2.5                       # exact quotient
    assert x1 * (np.float32(1.0) / s1) > np.float32(2.5)      # the wrong method differs
    X = np.zeros((1, 32), np.float32)
    X[0, 0] = 21.0    # 21/3 = 7 -> E = 0
    X[0, 1] = x1
    s = np.full(32, 3.0, np.float32)
    s[1] = s1
    Aq, As, _ = orc.act_prep(X, s, np.zeros(0, np.int32), np.arange(32, dtype=np.int32))
    assert As[0, 0] == 127
    assert (Aq[0, 0] & 0xF) == 7 and (Aq[0, 0] >> 4) == 4


# ------------------------------------------------- exhaustive-style format checks

def _fp32_classes(rng):
    """Bit patterns covering every sign and exponent with boundary and random mantissas."""
    mants = np.array([0, 1, 2, 3, 0x3FFFFF, 0x400000, 0x400001, 0x7FFFFE, 0x7FFFFF] +
                     list(rng.integers(0, 1 << 23, size=247)), dtype=np.uint32)
    exps = np.arange(256, dtype=np.uint32)
    pats = (exps[:, None] << 23) | mants[None, :]
    pats = pats.ravel()
    pats = np.concatenate([pats, pats | np.uint32(0x80000000)])
    return pats.view(np.float32)


def test_e8m0_matches_bitfield_formulation(orc, mini):
    """Oracle's frexp-based exponent == mini's bit-field exponent on every exponent
    class, all subnormal leading-bit positions, 0, Inf and NaN."""
    rng = np.random.default_rng(1)
    vals = np.abs(_fp32_classes(rng))
    sub = (np.uint32(1) << np.arange(23, dtype=np.uint32)).view(np.float32)
    vals = np.concatenate([vals, sub, np.array([0.0, np.inf, np.nan], np.float32)])
    a = orc.e8m0_codes(vals)
    b = mini.e8m0(vals)
    assert np.array_equal(a, b)
    # closed-form spot checks: 1.0 -> E=-2; 6.0 -> E=0; 8.0 -> E=1; FLT_MAX -> 125+127
    assert orc.e8m0_code(1.0) == 125 and orc.e8m0_code(6.0) == 127
    assert orc.e8m0_code(8.0) == 128 and orc.e8m0_code(np.finfo(np.float32).max) == 252


def test_e2m1_matches_nearest_search(orc, mini):
    """Threshold table == nearest-grid search with even ties: every midpoint and its
    binary32 neighbours, the grid points, +-0, the saturation range, random values."""
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float32)
    pts = np.concatenate([mids, grid, np.array([6.5, 7.0, 7.99, 1e30], np.float32)])
    near = np.concatenate([pts, np.nextafter(pts, np.float32(np.inf)),
                           np.nextafter(pts, np.float32(-np.inf))])
    rng = np.random.default_rng(2)
    v = np.concatenate([near, rng.uniform(0, 8, 200000).astype(np.float32),
                        np.array([0.0, 2.0 ** -149, 1e-30], np.float32)])
    v = np.concatenate([v, -v]).astype(np.float64)
    assert np.array_equal(orc.e2m1_codes(v), mini.e2m1_nearest(v))
    # -0 keeps its sign
    assert orc.e2m1_code(-0.0) == 8 and orc.e2m1_code(0.0) == 0


def test_block_quantizer_matches_second_formulation(orc, mini):
    """Whole 32-blocks through the oracle's act-prep (s = 1, so x/s = x exactly) vs
    mini's vectorized quantizer, over blocks mixing all fp32 classes: subnormals,
    scaled midpoints at E in {-127,-20,-2,0,2,125}, NaN/Inf blocks, zero blocks."""
    rng = np.random.default_rng(3)
    cls = _fp32_classes(rng)
    rows = []
    # random mixes of arbitrary classes (includes NaN/Inf -> 0xFF blocks)
    rows.append(rng.choice(cls, size=(400, 32)))
    # finite-only mixes
    fin = cls[np.isfinite(cls)]
    rows.append(rng.choice(fin, size=(400, 32)))
    # midpoint structure: block max = 6 * 2^E (or 7.9 * 2^E), others at midpoints*2^E
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float64)
    for E in (-127, -20, -2, 0, 2, 125):
        for head in (6.0, 7.9, 4.0):
            blk = np.zeros((50, 32), np.float64)
            blk[:, 0] = head * 2.0 ** E
            m = rng.choice(mids, size=(50, 31)) * 2.0 ** E
            m = m.astype(np.float32)
            nb = rng.integers(-1, 2, size=m.shape)
            m = np.where(nb < 0, np.nextafter(m, np.float32(0)),
                         np.where(nb > 0, np.nextafter(m, np.float32(np.inf)), m))
            sgn = rng.choice([-1.0, 1.0], size=m.shape).astype(np.float32)
            blk[:, 1:] = m * sgn
            rows.append(blk.astype(np.float32))
    rows.append(np.zeros((4, 32), np.float32))
    rows.append(-np.zeros((4, 32), np.float32))
    X = np.concatenate(rows).astype(np.float32)
    s = np.ones(32, np.float32)
    Aq, As, _ = orc.act_prep(X, s, np.zeros(0, np.int32), np.arange(32, dtype=np.int32))
    codes, sc = mini.quant_rows_1x32(X)
    assert np.array_equal(As[:, 0], sc[:, 0])
    assert np.array_equal(Aq[:, :16], mini.pack_nibbles(codes))
    assert np.any(As[:, 0] == 0xFF) and np.any(As[:, 0] == 0) and np.any(As[:, 0] == 252)


def test_bf16_rounding_matches_bit_trick(orc, mini):
    """Oracle's neighbour-comparison bf16 rounding == the bias-and-truncate trick,
    on all exponent classes, exact ties, overflow to Inf, subnormals."""
    rng = np.random.default_rng(4)
    x = _fp32_classes(rng)
    ties = ((rng.integers(0, 1 << 15, 5000).astype(np.uint32) << 16) | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, np.array([np.finfo(np.float32).max, 3.3961e38], np.float32)])
    fin = np.isfinite(x)
    a = orc.bf16_round(x[fin])
    b = mini.bf16_bits(x[fin])
    assert np.array_equal(a, b)
    n = orc.bf16_round(np.array([np.nan], np.float32))[0]
    assert (n & 0x7F80) == 0x7F80 and (n & 0x7F) != 0


# -------------------------------------------------------------- calibration

def test_col_absmax_and_scores(orc):
    """act_scale_j = max_t |x_tj| ([R] sec. 3.2/3.3); score identity: the max of the
    per-element quotients equals the quotient of the max (division is monotone)."""
    rng = np.random.default_rng(5)
    X = (rng.standard_normal((300, 77)) * rng.uniform(0.01, 10, 77)).astype(np.float32)
    act = orc.col_absmax(X)
    assert np.array_equal(act, np.abs(X).max(axis=0))
    s = rng.uniform(0.1, 10, 77).astype(np.float32)
    sc = orc.scores(act, s)
    per_elem = (np.abs(X) / s[None, :]).astype(np.float32).max(axis=0)
    assert np.array_equal(sc, per_elem)


def test_smoothing_closed_forms(orc):
    """s_j = a^alpha / w^(1-alpha) ([R] sec. 3.2): alpha=1 gives s=a exactly, alpha=0
    gives s=1/w, powers of two are exact, and at alpha=0.5 the smoothed activation max
    a/s and the folded weight max w*s meet at sqrt(a*w)."""
    rng = np.random.default_rng(6)
    a = rng.uniform(0.01, 30, 500).astype(np.float32)
    w = rng.uniform(0.001, 0.6, 500).astype(np.float32)
    assert np.array_equal(orc.smoothing(a, w, 1.0), a)
    assert np.array_equal(orc.smoothing(a, w, 0.0), (1.0 / w.astype(np.float64)).astype(np.float32))
    pa = np.float32(2.0) ** rng.integers(-2, 10, 50).astype(np.float32)   # pa^2 above the 1e-5 floor
    pw = np.float32(2.0) ** (2 * rng.integers(-8, 0, 50)).astype(np.float32)
    s2 = orc.smoothing(pa * pa, pw, 0.5)            # sqrt(pa^2 / pw) = pa / sqrt(pw)
    assert np.array_equal(s2, pa / np.sqrt(pw))
    s = orc.smoothing(a, w, 0.5).astype(np.float64)
    g = np.sqrt(a.astype(np.float64) * w)
    assert np.allclose(a / s, g, rtol=3e-7) and np.allclose(w * s, g, rtol=3e-7)
    # floors: zero maxima are floored at 1e-5 (no division by zero)
    z = orc.smoothing(np.zeros(3, np.float32), np.zeros(3, np.float32), 0.7)
    assert np.all(np.isfinite(z)) and np.all(z > 0)


def test_select_outliers_against_sort(orc):
    """Top-k by score, ties to the smaller index, O and J ascending ([R] sec. 3.3):
    the oracle's repeated arg-max agrees with a full sort, including heavy ties."""
    rng = np.random.default_rng(7)
    for trial in range(30):
        d = int(rng.integers(1, 60))
        k = int(rng.integers(0, d + 1))
        sc = rng.integers(0, 5, d).astype(np.float32)  # many ties
        O, J = orc.select_outliers(sc, k)
        order = sorted(range(d), key=lambda j: (-float(sc[j]), j))
        assert list(O) == sorted(order[:k])
        assert list(J) == sorted(order[k:])


# -------------------------------------------------------------- fold identity

def _exact_layer(rng, T, d_in, d_out, k):
    """A layer whose smoothed activations and folded weights sit exactly on the MXFP4
    grid (each 32-block holds a 6*2^e head), with power-of-two s, so that quantization
    is lossless and the oracle must reproduce X W^T exactly."""
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float64)
    s = (2.0 ** rng.integers(-3, 4, d_in)).astype(np.float32)
    perm = rng.permutation(d_in)
    O = np.sort(perm[:k]).astype(np.int32)
    J = np.sort(perm[k:]).astype(np.int32)
    K_J = J.size
    K_pad = ((K_J + 127) // 128) * 128

    def grid_rows(R, per_block_exp):
        V = rng.choice(grid, size=(R, K_pad)) * rng.choice([-1.0, 1.0], size=(R, K_pad))
        for b in range(K_pad // 32):
            V[:, b * 32] = 6.0
        e = per_block_exp(R)
        V = V * np.repeat(2.0 ** e, 32, axis=1)
        return V[:, :K_J]

    Xt = grid_rows(T, lambda R: rng.integers(-4, 3, (R, K_pad // 32)).astype(np.float64))
    Wt = grid_rows(d_out, lambda R: rng.integers(-9, -4, (R, K_pad // 32)).astype(np.float64))
    X = np.zeros((T, d_in), np.float64)
    W = np.zeros((d_out, d_in), np.float64)
    X[:, J] = Xt * s[J]            # x = x~ * s  => x / s = x~ exactly
    W[:, J] = Wt / s[J]            # w = w' / s  => s * w = w' exactly
    X[:, O] = rng.integers(-64, 64, (T, k)) / 8.0     # bf16-exact outlier values
    W[:, O] = rng.integers(-64, 64, (d_out, k)) / 256.0
    return X.astype(np.float32), W.astype(np.float32), s, O, J


def test_fold_identity_exact(orc):
    """(X / s)(s * W) = X W ([R] sec. 3.2) through the oracle's divide, fold, split and
    dual-branch sum: on grid-exact data the oracle output equals fp64 X W^T exactly.
    A dropped branch, a multiply in place of the divide, a wrong J/O index or a
    transposed operand all break equality."""
    rng = np.random.default_rng(8)
    for (T, d_in, d_out, k, layout) in ((5, 200, 40, 7, 0), (3, 300, 33, 0, 0), (4, 129, 20, 1, 0)):
        X, W, s, O, J = _exact_layer(rng, T, d_in, d_out, k)
        pk = orc.pack_weights(W, s, O, J, layout)
        Y = orc.linear(X, s, O, J, pk)
        ref = X.astype(np.float64) @ W.astype(np.float64).T
        assert np.array_equal(Y, ref)


def test_fold_identity_fp64_general(orc, mini):
    """The fold on general data ([R] sec. 3.2 and 3.3), on the tiny workload recipe
    with the oracle's own calibration (general s, k = 8):
    * the premise: (X / s)(s * W) = X W in fp64 within 1e-13 relative;
    * the oracle's act-prep codes equal mini's quantizer applied to fl32(X_J / s_J)
      (numpy's IEEE binary32 divide, gathered by J and zero padded), and its weight
      codes equal mini's quantizer applied to fl32(s_J * W_J);
    * the oracle's output equals the fp64 product of mini's dequantized operands plus
      the bf16 product of the raw outlier columns, within 1e-12 relative;
    * smoothing + split beats naive W4A4 against X W ([R] sec. 5 direction)."""
    from bit_quantized_dit_amd import synth
    spec = synth.WORKLOADS[1]
    inp = synth.layer_inputs(spec, T=64, d_in=256, d_out=96, k=8, T_cal=64)
    X, W = inp["X"], inp["W"]
    s, O, J, *_ = orc.calibrate(inp["X_cal"], W, spec.alpha, 8)
    assert O.size == 8 and not np.all(s == 1)
    ref = X.astype(np.float64) @ W.astype(np.float64).T
    s64 = s.astype(np.float64)
    folded = (X.astype(np.float64) / s64) @ (W.astype(np.float64) * s64).T
    assert np.abs(folded - ref).max() <= 1e-13 * np.abs(ref).max()

    pk = orc.pack_weights(W, s, O, J, 0)
    Aq, As, XO = orc.act_prep(X, s, O, J)
    K_pad = pk["K_pad"]
    Xs = np.zeros((X.shape[0], K_pad), np.float32)
    Xs[:, :J.size] = X[:, J] / s[J][None, :]
    Ws = np.zeros((W.shape[0], K_pad), np.float32)
    Ws[:, :J.size] = s[J][None, :] * W[:, J]
    ca, sa = mini.quant_rows_1x32(Xs)
    cb, sb = mini.quant_rows_1x32(Ws)
    assert np.array_equal(Aq, mini.pack_nibbles(ca)) and np.array_equal(As, sa)
    assert np.array_equal(pk["Bq"], mini.pack_nibbles(cb)) and np.array_equal(pk["Bs"], sb)
    Y = orc.output_full(Aq, As, XO, pk)
    want = (mini.dequant_1x32(mini.pack_nibbles(ca), sa) @ mini.dequant_1x32(mini.pack_nibbles(cb), sb).T +
            mini.bf16_to_f64(mini.bf16_bits(X[:, O])) @ mini.bf16_to_f64(mini.bf16_bits(W[:, O])).T)
    assert np.allclose(Y, want, rtol=1e-12, atol=1e-12 * np.abs(want).max())

    one = np.ones(256, np.float32)
    Yn = orc.linear(X, one, np.zeros(0, np.int32), np.arange(256, dtype=np.int32),
                    orc.pack_weights(W, one, np.zeros(0, np.int32), np.arange(256, dtype=np.int32), 0))
    e_ours = np.linalg.norm(Y - ref) / np.linalg.norm(ref)
    e_naive = np.linalg.norm(Yn - ref) / np.linalg.norm(ref)
    assert e_ours < e_naive
    assert e_ours < 0.2


# -------------------------------------------------------------- degenerate cases

def test_k0_is_dequantize_then_matmul(orc, mini):
    """k = 0, s = 1: the dual branch reduces to plain MXFP4: Y == dequant(A) dequant(B)^T
    with mini's independent codes and numpy matmul."""
    rng = np.random.default_rng(9)
    T, d_in, d_out = 37, 320, 70
    X = (rng.standard_normal((T, d_in)) * 0.5).astype(np.float32)
    W = (rng.standard_normal((d_out, d_in)) * 0.05).astype(np.float32)
    s = np.ones(d_in, np.float32)
    O = np.zeros(0, np.int32)
    J = np.arange(d_in, dtype=np.int32)
    pk = orc.pack_weights(W, s, O, J, 0)
    Aq, As, XO = orc.act_prep(X, s, O, J)
    K_pad = pk["K_pad"]
    Xp = np.zeros((T, K_pad), np.float32)
    Xp[:, :d_in] = X
    Wp = np.zeros((d_out, K_pad), np.float32)
    Wp[:, :d_in] = W
    ca, sa = mini.quant_rows_1x32(Xp)
    cb, sb = mini.quant_rows_1x32(Wp)
    assert np.array_equal(Aq, mini.pack_nibbles(ca)) and np.array_equal(As, sa)
    assert np.array_equal(pk["Bq"], mini.pack_nibbles(cb)) and np.array_equal(pk["Bs"], sb)
    ref = mini.dequant_1x32(Aq, As) @ mini.dequant_1x32(pk["Bq"], pk["Bs"]).T
    Y = orc.output_full(Aq, As, XO, pk)
    assert np.allclose(Y, ref, rtol=1e-12, atol=1e-12)


def test_k_equals_din_is_bf16_matmul(orc, mini):
    """k = d_in: J is empty, the W4A4 branch vanishes, and Y is the bf16 x bf16 product
    accumulated exactly: numpy matmul of the bf16-rounded operands."""
    rng = np.random.default_rng(10)
    T, d_in, d_out = 19, 48, 33
    X = rng.standard_normal((T, d_in)).astype(np.float32)
    W = (rng.standard_normal((d_out, d_in)) * 0.1).astype(np.float32)
    s = rng.uniform(0.5, 2, d_in).astype(np.float32)
    O = np.arange(d_in, dtype=np.int32)
    J = np.zeros(0, np.int32)
    pk = orc.pack_weights(W, s, O, J, 0)
    assert pk["K_pad"] == 0
    Y = orc.linear(X, s, O, J, pk)
    ref = mini.bf16_to_f64(mini.bf16_bits(X)) @ mini.bf16_to_f64(mini.bf16_bits(W)).T
    assert np.allclose(Y, ref, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------- alpha / k search

def test_search_k_equals_din_is_the_bf16_error(orc, mini):
    """With k = d_in every column is an outlier, so each candidate's output is the bf16
    product whatever alpha is: the search's error must equal the closed form
    ||bf16(X) bf16(W)^T - X W^T||_F / ||X W^T||_F for every alpha, and the first
    candidate wins the tie."""
    rng = np.random.default_rng(21)
    T, d_in, d_out = 40, 64, 24
    X = rng.standard_normal((T, d_in)).astype(np.float32)
    W = (rng.standard_normal((d_out, d_in)) * 0.05).astype(np.float32)
    errs, best = orc.search_alpha_k(X, W, [0.3, 0.5, 0.9], [d_in], 0)
    ref = X.astype(np.float64) @ W.astype(np.float64).T
    q = mini.bf16_to_f64(mini.bf16_bits(X)) @ mini.bf16_to_f64(mini.bf16_bits(W)).T
    want = np.linalg.norm(q - ref) / np.linalg.norm(ref)
    assert np.allclose(errs, want, rtol=1e-12, atol=0)
    assert best == (0, 0)


def test_search_prefers_splitting_heavy_columns(orc):
    """Columns whose magnitude dwarfs the rest inflate their blocks' scales ([R] sec.
    3.1, 3.3); keeping them in the BF16 branch must lower the output error, and the
    search must pick the k that covers them."""
    rng = np.random.default_rng(22)
    T, d_in, d_out = 64, 128, 32
    X = (rng.standard_normal((T, d_in)) * 0.3).astype(np.float32)
    heavy = np.array([5, 40, 77, 120])
    X[:, heavy] *= 40.0
    W = (rng.standard_normal((d_out, d_in)) * 0.02).astype(np.float32)
    errs, best = orc.search_alpha_k(X, W, [0.5], [0, heavy.size], 0)
    assert errs[0, 1] < 0.5 * errs[0, 0]
    assert best == (0, 1)


# --------------------------------------------------------- per-call outliers

def test_dynamic_selection_order_matches_calibration(orc):
    """For finite scores the bit-pattern order of the per-call selection is the numeric
    order of the calibration's top-k (larger first, ties to the smaller column)."""
    rng = np.random.default_rng(31)
    X = rng.standard_normal((50, 96)).astype(np.float32)
    X[:, [3, 50]] *= 30.0
    X[:, 70] = X[:, 3]                      # a tie with column 3
    s = rng.uniform(0.5, 2.0, 96).astype(np.float32)
    s[70] = s[3]
    for k in (0, 1, 2, 3, 17, 96):
        O, _ = orc.select_outliers(orc.scores(orc.col_absmax(X), s), k)
        assert np.array_equal(orc.select_outliers_dynamic(X, s, k), O)
    Xn = X.copy()
    Xn[0, 10] = np.nan
    Xn[0, 11] = np.inf
    assert list(orc.select_outliers_dynamic(Xn, s, 2)) == [10, 11]   # NaN ranks above +Inf


def test_dynamic_k_equals_din_is_bf16_matmul(orc, mini):
    """k = d_in: every column goes to the BF16 branch and the MXFP4 operand is all zero."""
    rng = np.random.default_rng(32)
    T, d_in, d_out = 21, 64, 17
    X = rng.standard_normal((T, d_in)).astype(np.float32)
    W = (rng.standard_normal((d_out, d_in)) * 0.1).astype(np.float32)
    s = rng.uniform(0.5, 2, d_in).astype(np.float32)
    Y, O, Aq, As, XO, WO = orc.linear_dynamic(X, W, s, d_in, 0)
    assert np.array_equal(O, np.arange(d_in)) and not Aq.any() and not As.any()
    ref = mini.bf16_to_f64(mini.bf16_bits(X)) @ mini.bf16_to_f64(mini.bf16_bits(W)).T
    assert np.allclose(Y, ref, rtol=1e-12, atol=1e-12)


def test_dynamic_chosen_columns_leave_the_fp4_branch(orc, mini):
    """When only k columns of X are nonzero they are the ones chosen, the MXFP4 branch
    sees zeros everywhere (all codes and scales 0), and Y is exactly their bf16
    product; with k = 0 the layer is the static one with no outlier column."""
    rng = np.random.default_rng(33)
    T, d_in, d_out = 30, 256, 40
    cols = np.array([7, 100, 201])
    X = np.zeros((T, d_in), np.float32)
    X[:, cols] = rng.standard_normal((T, cols.size)).astype(np.float32)
    W = (rng.standard_normal((d_out, d_in)) * 0.1).astype(np.float32)
    s = np.ones(d_in, np.float32)
    Y, O, Aq, As, XO, WO = orc.linear_dynamic(X, W, s, cols.size, 1)
    assert np.array_equal(O, cols) and not Aq.any() and not As.any()
    ref = mini.bf16_to_f64(mini.bf16_bits(X[:, cols])) @ mini.bf16_to_f64(mini.bf16_bits(W[:, cols])).T
    assert np.allclose(Y, ref, rtol=1e-12, atol=1e-12)
    X2 = rng.standard_normal((T, d_in)).astype(np.float32)
    Y0 = orc.linear_dynamic(X2, W, s, 0, 0)[0]
    J = np.arange(d_in, dtype=np.int32)
    assert np.array_equal(Y0, orc.linear(X2, s, np.zeros(0, np.int32), J,
                                         orc.pack_weights(W, s, np.zeros(0, np.int32), J, 0)))


# -------------------------------------------------------------- layouts

@pytest.mark.parametrize("layout", [1, 2])
def test_tile_and_stripe_groups(orc, mini, layout):
    """32x32 tiles and 128x1 K-major stripes ([R] sec. 3.4): every group's scale is the
    E8M0 of the group maximum (mini recomputes the maxima by reshaping) and every code
    is the nearest-even E2M1 of w'/2^E; a ragged last tile (d_out % 32 != 0) is the
    intersection of the tile with the matrix."""
    rng = np.random.default_rng(11 + layout)
    d_in, d_out = 300, 45
    W = (rng.standard_normal((d_out, d_in)) * 0.02).astype(np.float32)
    W[3, 17] = 0.55
    s = rng.uniform(0.5, 4, d_in).astype(np.float32)
    O = np.array([2, 50, 299], np.int32)
    J = np.setdiff1d(np.arange(d_in), O).astype(np.int32)
    pk = orc.pack_weights(W, s, O, J, layout)
    K_pad = pk["K_pad"]
    Wf = np.zeros((d_out, K_pad), np.float32)
    Wf[:, :J.size] = s[J][None, :] * W[:, J]
    A = np.abs(Wf)
    if layout == 2:
        gmax = A.reshape(d_out, K_pad // 128, 128).max(-1)
        assert np.array_equal(pk["Bs"], mini.e8m0(gmax))
        E = np.repeat(pk["Bs"].astype(np.int64) - 127, 128, axis=1)
    else:
        nt = (d_out + 31) // 32
        Ap = np.zeros((nt * 32, K_pad), np.float32)
        Ap[:d_out] = A
        gmax = Ap.reshape(nt, 32, K_pad // 32, 32).max(axis=(1, 3)).T
        assert np.array_equal(pk["Bs"], mini.e8m0(gmax))
        E = np.repeat(pk["Bs"].T.astype(np.int64) - 127, 32, axis=1)
        E = np.repeat(E, 32, axis=0)[:d_out]
    codes = mini.e2m1_nearest(Wf.astype(np.float64) * np.exp2(-E.astype(np.float64)))
    assert np.array_equal(pk["Bq"], mini.pack_nibbles(codes))
    assert np.array_equal(pk["WO"], mini.bf16_bits(W[:, O]))


# -------------------------------------------------------------- invariants

def test_invariants_power_of_two_sign_permutation(orc):
    """X*2^m moves every activation scale by +m with identical nibbles; -X flips bit 3
    of every nibble (zeros included); permuting tokens permutes output rows."""
    rng = np.random.default_rng(12)
    T, d_in = 40, 200
    X = (rng.standard_normal((T, d_in)) * 0.7).astype(np.float32)
    s = rng.uniform(0.5, 3, d_in).astype(np.float32)
    O = np.array([5, 9], np.int32)
    J = np.setdiff1d(np.arange(d_in), O).astype(np.int32)
    Aq, As, XO = orc.act_prep(X, s, O, J)
    Aq2, As2, _ = orc.act_prep(X * np.float32(8.0), s, O, J)
    real = np.arange(As.shape[1]) * 32 < J.size
    assert np.array_equal(Aq2, Aq)
    assert np.array_equal(As2[:, real].astype(int), As[:, real].astype(int) + 3)
    Aq3, As3, _ = orc.act_prep(-X, s, O, J)
    assert np.array_equal(As3, As)
    K_J = J.size
    n_real = K_J // 2
    assert np.array_equal(Aq3[:, :n_real], Aq[:, :n_real] ^ 0x88)
    W = (rng.standard_normal((24, d_in)) * 0.05).astype(np.float32)
    pk = orc.pack_weights(W, s, O, J, 0)
    perm = rng.permutation(T)
    Y = orc.linear(X, s, O, J, pk)
    Yp = orc.linear(np.ascontiguousarray(X[perm]), s, O, J, pk)
    assert np.array_equal(Yp, Y[perm])


def test_output_pairs_match_full(orc):
    rng = np.random.default_rng(13)
    X = rng.standard_normal((10, 100)).astype(np.float32)
    W = (rng.standard_normal((20, 100)) * 0.1).astype(np.float32)
    s = np.ones(100, np.float32)
    O = np.array([1, 2, 3], np.int32)
    J = np.setdiff1d(np.arange(100), O).astype(np.int32)
    pk = orc.pack_weights(W, s, O, J, 2)
    Aq, As, XO = orc.act_prep(X, s, O, J)
    Y = orc.output_full(Aq, As, XO, pk)
    ts = rng.integers(0, 10, 50)
    ns = rng.integers(0, 20, 50)
    assert np.array_equal(orc.output_pairs(Aq, As, XO, pk, ts, ns), Y[ts, ns])


@pytest.mark.parametrize("layout", [0, 1, 2])
@pytest.mark.parametrize("k", [0, 5])
def test_output_any_layout_is_dequantize_then_matmul(orc, mini, layout, k):
    """The oracle's output sum ([R] sec. 3.3 dual branch; sec. 3.4 weight scale groups)
    in every weight layout equals numpy's fp64 matmul of independently dequantized
    operands: mini's 1x32 dequantizer for the activations, mini's layout-aware
    dequantizer (group scale looked up per (n, p)) for the weights, plus the bf16
    product of the outlier columns.  d_out = 45 leaves a ragged last 32x32 tile and
    d_in - k is not a multiple of 128, so the K padding is crossed; k = 0 with s = 1 is
    the pure MXFP4 case."""
    rng = np.random.default_rng(40 + 3 * layout + k)
    T, d_in, d_out = 23, 300, 45
    X = (rng.standard_normal((T, d_in)) * 0.5).astype(np.float32)
    X[:, 17] *= 20.0
    W = (rng.standard_normal((d_out, d_in)) * 0.03).astype(np.float32)
    W[5:9, 100:140] *= 8.0        # uneven magnitudes across tiles and stripes
    if k == 0:
        s = np.ones(d_in, np.float32)
        O = np.zeros(0, np.int32)
        J = np.arange(d_in, dtype=np.int32)
    else:
        s, O, J, *_ = orc.calibrate(X, W, 0.6, k)
    pk = orc.pack_weights(W, s, O, J, layout)
    Aq, As, XO = orc.act_prep(X, s, O, J)
    Y = orc.output_full(Aq, As, XO, pk)
    want = mini.dequant_1x32(Aq, As) @ mini.dequant_weights(pk["Bq"], pk["Bs"], layout, d_out).T
    if k:
        want = want + mini.bf16_to_f64(XO) @ mini.bf16_to_f64(pk["WO"]).T
    assert np.allclose(Y, want, rtol=1e-12, atol=1e-12 * np.abs(want).max())
    # the scales differ across groups, so a wrong group lookup cannot pass unnoticed
    assert len(np.unique(pk["Bs"])) >= 3


def test_col_absmax_bf16(orc, mini):
    """act_scale_j on bf16 activations ([R] sec. 3.2): the oracle widens each bf16 bit
    pattern exactly, so the column maxima equal numpy's maxima of the widened values,
    including signed zeros, subnormal bf16 values and columns whose maximum is negative
    before |.|; a NaN or Inf anywhere is refused."""
    rng = np.random.default_rng(41)
    V = (rng.standard_normal((150, 67)) * rng.uniform(1e-3, 20, 67)).astype(np.float32)
    V[:, 3] = -np.abs(V[:, 3])
    V[:, 4] = 0.0
    V[::2, 4] = -0.0
    V[:, 5] = np.float32(2.0 ** -130) * rng.integers(1, 16, 150)   # bf16 subnormals
    Xb = mini.bf16_bits(V)
    act = orc.col_absmax(Xb)
    want = np.abs(mini.bf16_to_f64(Xb)).max(axis=0).astype(np.float32)
    assert np.array_equal(act.view(np.uint32), want.view(np.uint32))
    assert act[5] > 0 and act[5] < 2.0 ** -126
    for bad in (0x7FC0, 0xFF80):
        Xn = Xb.copy()
        Xn[7, 9] = bad
        with pytest.raises(ValueError):
            orc.col_absmax(Xn)


def test_e8m0_every_positive_pattern(orc, mini):
    """The E8M0 rule on every one of the 2^31 non-negative binary32 patterns (zero,
    every subnormal, every normal, +Inf and every positive NaN): the oracle's frexp
    formulation equals mini's bit-field formulation."""
    from concurrent.futures import ThreadPoolExecutor
    chunk = 1 << 24

    def run(c):
        a = np.arange(c * chunk, (c + 1) * chunk, dtype=np.uint32).view(np.float32)
        x, y = orc.e8m0_codes(a), mini.e8m0(a)
        return int(np.count_nonzero(x != y))

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        bad = sum(ex.map(run, range((1 << 31) // chunk)))
    assert bad == 0


def test_gelu_every_bf16_input(orc):
    """GELU-tanh between the FFN projections ([R] sec. 3.1 and 3.5): H depends only on
    bf16(Y), so all 65536 bf16 inputs cover it.  For every finite input the oracle's H
    is a nearest bf16 value to 0.5 x (1 + tanh(z)), z = sqrt(2/pi)(x + 0.044715 x^3),
    evaluated in 60-digit decimal arithmetic (tanh from its exponential definition), the
    far negative tail included; where the exact value lies within 1e-12 (relative) of a
    rounding boundary either neighbour is accepted.  +Inf gives +Inf, and NaN and -Inf
    give the quiet NaN with the input's sign."""
    from decimal import Decimal, getcontext
    # 240 digits: for |2z| <= 400 the sum 1 + tanh(z) loses at most 174 of them
    getcontext().prec = 240
    pats = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    x32 = (pats.astype(np.uint32) << 16).view(np.float32)
    H = orc.gelu_bf16(x32)
    c = (Decimal(2) / Decimal("3.14159265358979323846264338327950288419716939937510")).sqrt()

    def dval(p):   # exact value of a finite bf16 pattern
        return Decimal(float((np.uint32(p) << 16).view(np.float32)))

    def gelu(x):
        z = c * (x + Decimal("0.044715") * x * x * x)
        # beyond |2z| = 400 the factor 0.5 (1 + tanh z) is within 2 e^-400 of 0 or 1;
        # with |x| < 2^128 the result then rounds to a signed zero or to x itself
        if 2 * z < -400:
            return Decimal(0) * x.copy_sign(Decimal(-1))
        if 2 * z > 400:
            return x
        e = (2 * z).exp()
        return Decimal("0.5") * x * (1 + (e - 1) / (e + 1))

    bad = []
    for p in range(1 << 16):
        mag = p & 0x7FFF
        if mag >= 0x7F80:
            continue
        g = gelu(dval(p))
        h = int(H[p])
        if (h & 0x7FFF) >= 0x7F80:
            bad.append(p)
            continue
        hv = dval(h)
        # neighbours of h in value order (sign-magnitude patterns)
        neigh = []
        for dm in (-1, 1):
            m2 = (h & 0x7FFF) + dm
            if m2 < 0:
                neigh.append(dval(0x0001 | ((h & 0x8000) ^ 0x8000)))
            elif m2 < 0x7F80:
                neigh.append(dval((h & 0x8000) | m2))
        dh = abs(hv - g)
        for nv in neigh:
            dn = abs(nv - g)
            if dn < dh and (dh - dn) > Decimal("1e-12") * abs(g):
                bad.append(p)
                break
    assert bad == [], [hex(b) for b in bad[:10]]
    assert H[0x7F80] == 0x7F80                      # +Inf
    assert H[0xFF80] == 0xFFC0                      # -Inf -> NaN with the sign of x
    assert H[0x7FC0] == 0x7FC0 and H[0xFFC1] == 0xFFC0
    # spot values: the tail reaches bf16 subnormals, and the zero signs follow x
    assert H[0x0000] == 0x0000 and H[0x8000] == 0x8000
    assert 0x8000 < int(H[int(mini_bits(-10.25))]) < 0x8080


def mini_bits(v):
    return int((np.array([v], np.float32).view(np.uint32)[0] >> 16))


def test_gelu_against_library(orc, mini):
    """GELU-tanh between the FFN up and down projections: the oracle's double-precision
    formula rounded once to bf16 agrees with torch's float64 tanh-GELU rounded to bf16
    (the bf16 input rounding is applied first on both sides)."""
    rng = np.random.default_rng(14)
    Y = np.concatenate([rng.standard_normal(20000) * 3, np.linspace(-10, 10, 2001)]).astype(np.float32)
    H = orc.gelu_bf16(Y)
    xb = torch.from_numpy(Y).to(torch.bfloat16).double()
    ref = torch.nn.functional.gelu(xb, approximate="tanh")
    refb = ref.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    # Away from the far negative tail both round the same real number once to bf16.
    # In the tail (true value below ~1e-6 in magnitude) torch's 1 + tanh cancels, so
    # only smallness is compared there (the decimal pin above covers the tail).
    r = ref.numpy()
    big = np.abs(r) > 1e-6
    assert np.mean(H[big] == refb[big]) > 0.9995
    d = np.abs(mini.bf16_to_f64(H[big]) - r[big])
    assert np.all(d <= np.abs(r[big]) * 2.0 ** -8)
    assert np.all(np.abs(mini.bf16_to_f64(H[~big])) <= 2e-6)
