"""GPU parity at the five workloads' full sizes, in the launch configuration the
benchmark times (w4a4_linear on the whole token batch).

Activation codes, scales and X_O are compared bit for bit with the oracle's act-prep on
every token row of every workload (in chunks at 57600 tokens).  Outputs are compared
with the GEMM tolerance on every output: at the tiny workload against the oracle's
output sum, elsewhere (4096 and 57600 tokens, both FFN-block layers) against the
dequantize-then-matmul form of that sum, which the CPU pins prove equal to the oracle's,
computed in token chunks from the oracle's own codes.  The FFN block is checked stage
by stage: up-projection, GELU (oracle applied to the GPU's Y_up), down act-prep (oracle
applied to the GPU's H, every row) and down output; the fully fused block's down codes
are checked against the oracle's act-prep of the H that the unfused chain produces
through the same layer, every row.
"""
import numpy as np
import pytest
import torch

from bit_quantized_dit_amd import synth
from bit_quantized_dit_amd import w4a4 as B
from tests.gpu_util import (_banner, _check_act, _check_packed, _check_y_full, _layer,
                            assert_y_close, bf16_bits, check_act_all_rows, full_y_reference, to_dev, u8)

pytestmark = pytest.mark.gpu


def _sample_pairs(rng, T, N, n_pairs=4096, full_rows=(0,)):
    ts = rng.integers(0, T, n_pairs)
    ns = rng.integers(0, N, n_pairs)
    for t in full_rows:
        ts = np.concatenate([ts, np.full(N, t)])
        ns = np.concatenate([ns, np.arange(N)])
    return ts, ns


def _check_sampled(orc, r, X, rng, n_rows=256):
    T = r["T"]
    rows = np.unique(np.concatenate([[0, T - 1], rng.integers(0, T, n_rows)]))
    Aq_o, As_o, XO_o = _check_act(orc, r, X, rows)
    N = r["pk_o"]["d_out"]
    # outputs at sampled (row, feature) pairs; full rows for the first and last token
    loc = np.arange(rows.size)
    ts_l, ns = _sample_pairs(rng, rows.size, N, 4096, full_rows=(0, rows.size - 1))
    Yref = orc.output_pairs(Aq_o, As_o, XO_o, r["pk_o"], ts_l, ns)
    Ysel = r["Y"][torch.as_tensor(rows[ts_l], device="cuda"), torch.as_tensor(ns, device="cuda")]
    return assert_y_close(Ysel.cpu().numpy(), Yref), loc


def test_workload1_tiny_full(orc):
    spec = synth.WORKLOADS[1]
    _banner(f"workload {spec.name}")
    inp = synth.layer_inputs(spec)
    r = _layer(orc, inp["X"], inp["X_cal"], inp["W"], spec.alpha, spec.k, spec.layout)
    _check_packed(r)
    st = _check_y_full(orc, r, inp["X"])
    _banner(f"  {st}")


@pytest.mark.parametrize("wid", [2, 3])
def test_workload_4096_tokens(orc, mini, wid):
    spec = synth.WORKLOADS[wid]
    _banner(f"workload {spec.name}")
    inp = synth.layer_inputs(spec)
    r = _layer(orc, inp["X"], inp["X_cal"], inp["W"], spec.alpha, spec.k, spec.layout)
    _check_packed(r)
    # the oracle redoes act-prep for every token here (a few seconds)
    Aq_o, As_o, XO_o = _check_act(orc, r, inp["X"])
    rng = np.random.default_rng(wid)
    ts, ns = _sample_pairs(rng, r["T"], spec.d_out, 8192, full_rows=(0, r["T"] - 1))
    Yref = orc.output_pairs(Aq_o, As_o, XO_o, r["pk_o"], ts, ns)
    Ysel = r["Y"][torch.as_tensor(ts, device="cuda"), torch.as_tensor(ns, device="cuda")]
    st = assert_y_close(Ysel.cpu().numpy(), Yref)
    # and every output: the oracle's act-prep results and packed weights through the
    # dequantize-then-matmul form of the output sum
    Yfull = full_y_reference(mini, Aq_o, As_o, XO_o, r["pk_o"])
    st_full = assert_y_close(r["Y"].cpu().numpy(), Yfull, what="Y (all outputs)")
    _banner(f"  all {Yfull.size} outputs: {st_full}")
    # the heavy columns drawn by the generator are the ones calibration selects
    overlap = np.intersect1d(r["O"], inp["heavy"]).size
    _banner(f"  {st}; heavy columns selected as O: {overlap}/{spec.k}")


def test_workload4_57600_tokens(orc, mini):
    spec = synth.WORKLOADS[4]
    _banner(f"workload {spec.name}")
    inp = synth.layer_inputs(spec)
    heavy_max = synth.bf16_bits_to_f32(inp["X"][:, inp["heavy"]]).__abs__().max(axis=0)
    assert np.all(heavy_max > 6.0)     # every heavy column reaches max |x| > 6
    r = _layer(orc, inp["X"], inp["X_cal"], inp["W"], spec.alpha, spec.k, spec.layout)
    _check_packed(r)
    st_all = check_act_all_rows(orc, B.workspace_views(r["ws"], r["T"], r["packed"]), inp["X"], r["s"], r["O"],
                                r["J"], y_gpu=r["Y"], pk=r["pk_o"], mini=mini)
    _banner(f"  act-prep: all {r['T']} rows bit-exact; all {r['T'] * spec.d_out} outputs: {st_all}")
    st, _ = _check_sampled(orc, r, inp["X"], np.random.default_rng(4))
    _banner(f"  {st}")


def test_workload5_ffn_block(orc, mini):
    up, down = synth.FFN_BLOCK["up"], synth.FFN_BLOCK["down"]
    _banner("workload ffn_block_T57600")
    inp = synth.layer_inputs(up)
    r_up = _layer(orc, inp["X"], inp["X_cal"], inp["W"], up.alpha, up.k, up.layout)
    _check_packed(r_up)
    st_all = check_act_all_rows(orc, B.workspace_views(r_up["ws"], r_up["T"], r_up["packed"]), inp["X"],
                                r_up["s"], r_up["O"], r_up["J"], what="up act-prep", y_gpu=r_up["Y"],
                                pk=r_up["pk_o"], mini=mini)
    _banner(f"  up act-prep: all {r_up['T']} rows bit-exact; all {r_up['T'] * up.d_out} outputs "
            f"(32x32-tile weight scales): {st_all}")
    rng = np.random.default_rng(5)
    st_up, _ = _check_sampled(orc, r_up, inp["X"], rng)
    _banner(f"  up: {st_up}")
    T = r_up["T"]
    # GELU stage: oracle GELU of the GPU's Y_up on sampled rows, <= 1 bf16 ulp
    H = torch.empty(T, up.d_out, dtype=torch.bfloat16, device="cuda")
    B.w4a4_gelu_tanh_bf16(r_up["Y"], H)
    torch.cuda.synchronize()
    rows = np.unique(rng.integers(0, T, 64))
    trow = torch.as_tensor(rows, device="cuda")
    Hg = bf16_bits(H[trow])
    Ho = orc.gelu_bf16(r_up["Y"][trow].cpu().numpy()).reshape(Hg.shape)
    a, b = mini.bf16_to_f64(Hg), mini.bf16_to_f64(Ho)
    big = np.abs(b) >= 2.0 ** -120     # below, the kernel's binary32 exp overflows to a signed zero
    assert np.all(np.abs(a[big] - b[big]) <= np.abs(b[big]) * 2.0 ** -7)
    mism = int(np.sum(Hg[big] != Ho[big]))
    _banner(f"  gelu: {mism} of {int(big.sum())} sampled elements differ by one bf16 ulp")
    assert mism <= big.sum() // 1000
    assert np.all(np.abs(a[~big]) < 2.0 ** -120)
    # the fused up projection (GELU in the GEMM epilogue) gives the same H bit for bit
    H_fused = torch.empty_like(H)
    B.w4a4_gemm_prequantized_gelu_bf16(r_up["ws"], T, r_up["packed"], H_fused)
    torch.cuda.synchronize()
    assert bool(torch.equal(H_fused.view(torch.int16), H.view(torch.int16))), "fused GELU output differs"
    _banner("  fused up+GELU: H identical to GELU(Y_up)")
    del H_fused
    # down layer: calibrated on the bf16 GELU of the unquantized up projection of the
    # calibration tokens; run on the GPU's H
    del r_up["ws"]
    Wd = synth.weights(down, stream=5)
    Xc_down = synth.down_calibration(inp["X_cal"], inp["W"])
    Wdd, Xcd = to_dev(Wd), to_dev(Xc_down)
    s, O, _, _ = B.w4a4_calibrate_scales(Xcd, Wdd, down.alpha, down.k)
    s_o, O_o, *_ = orc.calibrate(Xc_down, Wd, down.alpha, down.k)
    assert np.abs(s.view(np.int32).astype(np.int64) - s_o.view(np.int32)).max() <= 1
    assert np.array_equal(O, O_o)
    J = np.setdiff1d(np.arange(down.d_in), O).astype(np.int32)
    packed = B.w4a4_pack_weights(Wdd, s, O, down.layout)
    del r_up["Y"]
    ws = B.alloc_workspace(T, packed)
    Y = torch.empty(T, down.d_out, dtype=torch.float32, device="cuda")
    B.w4a4_linear(H, packed, Y, ws)
    torch.cuda.synchronize()
    r = {"s": s, "O": O, "J": J, "packed": packed, "ws": ws, "Y": Y, "T": T,
         "pk_o": orc.pack_weights(Wd, s, O, J, down.layout)}
    _check_packed(r)
    st_all = check_act_all_rows(orc, B.workspace_views(ws, T, packed), H, s, O, J, what="down act-prep",
                                y_gpu=Y, pk=r["pk_o"], mini=mini)
    _banner(f"  down act-prep of the GPU's H: all {T} rows bit-exact (codes, scales, X_O); "
            f"all {T * down.d_out} outputs (128x1 stripes): {st_all}")
    drows = np.unique(np.concatenate([[0, T - 1], rng.integers(0, T, 128)]))
    Hs = bf16_bits(H[torch.as_tensor(drows, device="cuda")])
    Aq_o, As_o, XO_o = orc.act_prep(Hs, s, O, J)
    ts_l, ns = _sample_pairs(rng, drows.size, down.d_out, 4096, full_rows=(0,))
    Yref = orc.output_pairs(Aq_o, As_o, XO_o, r["pk_o"], ts_l, ns)
    Ysel = Y[torch.as_tensor(drows[ts_l], device="cuda"), torch.as_tensor(ns, device="cuda")]
    st = assert_y_close(Ysel.cpu().numpy(), Yref)
    _banner(f"  down: {st}")
    # the fully fused block: the down layer's act-prep in the up GEMM's epilogue, the
    # up layer packed from its rows in the down layer's J-then-O order.  With this
    # block's 32x32-tile weight scales the row order regroups the shared scales, so the
    # reference is the unfused chain through the same permuted up layer (GELU fused,
    # H put back in column order, act-prep, down GEMM).
    del H, ws, Y, r
    P = B.ffn_permutation(O, down.d_in)
    Xd = to_dev(inp["X"])
    up_p = B.w4a4_pack_weights(to_dev(inp["W"][P]), r_up["s"], r_up["O"], up.layout)
    wsu = B.alloc_workspace(T, up_p)
    Hp = torch.empty(T, down.d_in, dtype=torch.bfloat16, device="cuda")
    B.w4a4_linear_gelu_bf16(Xd, up_p, Hp, wsu)
    del wsu
    Hq = torch.empty_like(Hp)
    Hq[:, torch.as_tensor(P, device="cuda")] = Hp
    del Hp
    wsd = B.alloc_workspace(T, packed)
    B.w4a4_quantize_activations(Hq, packed, wsd)
    Y2 = torch.empty(T, down.d_out, dtype=torch.float32, device="cuda")
    B.w4a4_gemm_prequantized(wsd, T, packed, Y2)
    wsf = B.alloc_workspace_ffn(T, up_p, packed)
    Yf = torch.empty_like(Y2)
    B.w4a4_ffn_forward(Xd, up_p, packed, Yf, wsf)
    torch.cuda.synchronize()
    fz, rf = B.ffn_workspace_views(wsf, T, up_p, packed), B.workspace_views(wsd, T, packed)
    # the fused epilogue's codes against the oracle's act-prep of the same H, every row
    check_act_all_rows(orc, fz, Hq, s, O, J, what="fused down act-prep")
    del Hq
    assert bool(torch.equal(fz["A_s"], rf["A_s"])), "fused A_s differs"
    assert bool(torch.equal(fz["A_q"], rf["A_q"])), "fused A_q differs"
    assert bool(torch.equal(fz["X_O"].view(torch.int16), rf["X_O"].view(torch.int16))), "fused X_O differs"
    assert bool(torch.equal(Yf.view(torch.int32), Y2.view(torch.int32))), "fused Y differs"
    _banner("  fully fused block: down codes, scales, X_O and Y identical to the unfused chain")


def test_dynamic_outliers_57600_tokens(orc):
    """Per-call outlier selection at the full-resolution workload's shape (the launch the
    benchmark times): O and the column map exact, sampled token rows of the codes and
    X_O bit-exact, sampled outputs within the tolerance."""
    spec = synth.WORKLOADS[4]
    _banner(f"per-call outliers {spec.name}")
    inp = synth.layer_inputs(spec)
    X, W = inp["X"], inp["W"]
    s, _, _, _ = B.w4a4_calibrate_scales(to_dev(inp["X_cal"]), to_dev(W), spec.alpha, spec.k)
    pk = B.w4a4_pack_weights_dyn(to_dev(W), s, spec.k, spec.layout)
    T = spec.T
    ws = B.alloc_workspace_dyn(T, pk)
    Y = torch.empty(T, W.shape[0], dtype=torch.float32, device="cuda")
    B.w4a4_linear_dyn(to_dev(X), pk, Y, ws)
    torch.cuda.synchronize()
    v = B.workspace_dyn_views(ws, T, pk)
    O = orc.select_outliers_dynamic(X, s, spec.k)
    assert np.array_equal(v["O"].cpu().numpy(), O), "O differs"
    d_in = X.shape[1]
    cm = np.arange(d_in, dtype=np.int32)
    cm[O] = -(np.arange(O.size) + 1)
    assert np.array_equal(v["colmap"].cpu().numpy(), cm), "column map differs"
    rng = np.random.default_rng(41)
    rows = np.unique(np.concatenate([[0, T - 1], rng.integers(0, T, 192)]))
    Xz = X[rows].copy()
    Xz[:, O] = 0
    J_all = np.arange(d_in, dtype=np.int32)
    Aq_o, As_o, _ = orc.act_prep(Xz, s, np.zeros(0, np.int32), J_all)
    Jc = np.setdiff1d(J_all, O).astype(np.int32)
    _, _, XO_o = orc.act_prep(X[rows], s, O, Jc)
    sel = torch.as_tensor(rows, device="cuda")
    assert np.array_equal(u8(v["A_s"][sel]), As_o), "A_s differs"
    assert np.array_equal(u8(v["A_q"][sel]), Aq_o), "A_q differs"
    assert np.array_equal(bf16_bits(v["X_O"][sel])[:, :spec.k], XO_o), "X_O differs"
    pk_o = orc.pack_weights(W, s, np.zeros(0, np.int32), J_all, spec.layout)
    pk_o["WO"] = orc.pack_weights(W, s, O, Jc, spec.layout)["WO"]
    pk_o["k"] = spec.k
    N = W.shape[0]
    ts_l, ns = _sample_pairs(rng, rows.size, N, 4096, full_rows=(0, rows.size - 1))
    Yref = orc.output_pairs(Aq_o, As_o, XO_o, pk_o, ts_l, ns)
    Ysel = Y[torch.as_tensor(rows[ts_l], device="cuda"), torch.as_tensor(ns, device="cuda")]
    st = assert_y_close(Ysel.cpu().numpy(), Yref)
    _banner(f"  {st}")


@pytest.mark.parametrize("T,d_in,d_out,k,layout", [(2600, 640, 7001, 24, 0), (2600, 640, 6912, 24, 1),
                                                    (600, 100, 40000, 4, 0), (600, 60, 39999, 0, 0)])
def test_many_tiles_per_workgroup_with_ragged_edges(orc, T, d_in, d_out, k, layout):
    """More output tiles than the persistent grid has workgroups, so workgroups run
    several tiles in a row, full and ragged ones (token tail, feature tail, and an
    output width that is not a multiple of 4): every output row and column at a tile
    edge is checked, plus random samples.  The last two cases have fewer K steps than
    the ring has slots (one FP4 step and one or no BF16 step), so the ring pads each
    tile with null steps and the prefetch of the next tile starts within the current
    tile's first steps."""
    spec = synth.WORKLOADS[2]
    _banner(f"many tiles T={T} d_in={d_in} d_out={d_out} k={k} layout={layout}")
    inp = synth.layer_inputs(spec, T=T, d_in=d_in, d_out=d_out, k=k, T_cal=256)
    r = _layer(orc, inp["X"], inp["X_cal"], inp["W"], spec.alpha, k, layout)
    _check_packed(r)
    rng = np.random.default_rng(11)
    Aq_o, As_o, XO_o = orc.act_prep(inp["X"], r["s"], r["O"], r["J"])
    edge_t = np.array(sorted({0, 255, 256, 511, 512, T - 257, T - 256, T - 2, T - 1}))
    edge_n = np.array(sorted({0, 255, 256, d_out - 257, d_out - 256, d_out - 4, d_out - 2, d_out - 1}))
    ts = [np.repeat(edge_t, d_out), np.tile(np.arange(T), edge_n.size), rng.integers(0, T, 8192)]
    ns = [np.tile(np.arange(d_out), edge_t.size), np.repeat(edge_n, T), rng.integers(0, d_out, 8192)]
    ts, ns = np.concatenate(ts), np.concatenate(ns)
    Yref = orc.output_pairs(Aq_o, As_o, XO_o, r["pk_o"], ts, ns)
    Ysel = r["Y"][torch.as_tensor(ts, device="cuda"), torch.as_tensor(ns, device="cuda")]
    st = assert_y_close(Ysel.cpu().numpy(), Yref)
    _banner(f"  {st} over {ts.size} outputs")
