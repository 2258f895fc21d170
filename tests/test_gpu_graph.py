"""The per-call entry points under HIP graph capture.  They allocate nothing and clear
memory with kernels (no memset nodes), so w4a4_linear, w4a4_linear_dyn and
w4a4_ffn_forward can be captured on a stream and replayed.  Each graph is replayed
several times with eager library work in between (on other buffers), and every
replay's output is compared bit for bit with the eager call's; the eager output was
itself checked against the oracle by the parity tests on the same kinds of inputs."""
import numpy as np
import pytest
import torch

from bit_quantized_dit_amd import synth
from bit_quantized_dit_amd import w4a4 as B
from tests.gpu_util import _banner, to_dev

pytestmark = pytest.mark.gpu

REPLAYS = 4


def _capture_and_check(call, Y, Y_eager, between):
    """Capture call(stream) into a graph, then replay it REPLAYS times; before each
    replay Y is filled with NaN, after it Y must equal Y_eager bit for bit."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        call(s)
    torch.cuda.synchronize()
    for i in range(REPLAYS):
        Y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert bool(torch.equal(Y.view(torch.int32), Y_eager.view(torch.int32))), f"replay {i} differs"
        between()
        torch.cuda.synchronize()
    _banner(f"  {REPLAYS} replays bit-identical to the eager call")


def _small_layer(T=300, d_in=704, d_out=320, k=13):
    spec = synth.WORKLOADS[2]
    inp = synth.layer_inputs(spec, T=T, d_in=d_in, d_out=d_out, k=k, T_cal=96)
    X, Xc, W = to_dev(inp["X"]), to_dev(inp["X_cal"]), to_dev(inp["W"])
    s, O, _, _ = B.w4a4_calibrate_scales(Xc, W, spec.alpha, k)
    return X, W, s, O


@pytest.mark.parametrize("layout,T,d_in,d_out,k", [(0, 300, 704, 320, 13), (1, 300, 704, 320, 13),
                                                   (0, 200, 8192, 600, 20)])   # split K: two launches
def test_linear_graph_replays(layout, T, d_in, d_out, k):
    _banner(f"graph capture: w4a4_linear T={T} {d_in}->{d_out} k={k} layout {layout}")
    X, W, s, O = _small_layer(T, d_in, d_out, k)
    packed = B.w4a4_pack_weights(W, s, O, layout)
    T, N = X.shape[0], W.shape[0]
    ws, ws2 = B.alloc_workspace(T, packed), B.alloc_workspace(T, packed)
    Y, Y_eager, Y_other = (torch.empty(T, N, device="cuda") for _ in range(3))
    B.w4a4_linear(X, packed, Y_eager, ws)
    torch.cuda.synchronize()
    _capture_and_check(lambda st: B.w4a4_linear(X, packed, Y, ws, st), Y, Y_eager,
                       lambda: B.w4a4_linear(X, packed, Y_other, ws2))


def test_linear_dyn_graph_replays():
    _banner("graph capture: w4a4_linear_dyn T=300 704->320 k=13")
    X, W, s, _ = _small_layer()
    pk = B.w4a4_pack_weights_dyn(W, s, 13, 0)
    T, N = X.shape[0], W.shape[0]
    ws = B.alloc_workspace_dyn(T, pk)
    Y, Y_eager = torch.empty(T, N, device="cuda"), torch.empty(T, N, device="cuda")
    B.w4a4_linear_dyn(X, pk, Y_eager, ws)
    torch.cuda.synchronize()
    _capture_and_check(lambda st: B.w4a4_linear_dyn(X, pk, Y, ws, st), Y, Y_eager,
                       lambda: B.w4a4_column_absmax(X))


def test_ffn_forward_graph_replays():
    T, d_model, d_ff = 257, 384, 640
    _banner(f"graph capture: w4a4_ffn_forward T={T} {d_model}->{d_ff}->{d_model}")
    rng = np.random.default_rng(77)
    X = to_dev(synth.to_bf16_bits((rng.standard_normal((T, d_model)) * 0.5).astype(np.float32)))
    Xc = (rng.standard_normal((96, d_model)) * 0.5).astype(np.float32)
    W_up = (rng.standard_normal((d_ff, d_model)) * 0.05).astype(np.float32)
    W_dn = (rng.standard_normal((d_model, d_ff)) * 0.05).astype(np.float32)
    s_up, O_up, _, _ = B.w4a4_calibrate_scales(to_dev(Xc), to_dev(W_up), 0.6, 4)
    s_dn = rng.uniform(0.5, 2.0, d_ff).astype(np.float32)
    O_dn = np.sort(rng.choice(d_ff, 40, replace=False)).astype(np.int32)
    up = B.w4a4_pack_weights(to_dev(W_up[B.ffn_permutation(O_dn, d_ff)]), s_up, O_up, 1)
    down = B.w4a4_pack_weights(to_dev(W_dn), s_dn, O_dn, 2)
    ws, ws2 = B.alloc_workspace_ffn(T, up, down), B.alloc_workspace_ffn(T, up, down)
    Y, Y_eager, Y_other = (torch.empty(T, d_model, device="cuda") for _ in range(3))
    B.w4a4_ffn_forward(X, up, down, Y_eager, ws)
    torch.cuda.synchronize()
    _capture_and_check(lambda st: B.w4a4_ffn_forward(X, up, down, Y, ws, st), Y, Y_eager,
                       lambda: B.w4a4_ffn_forward(X, up, down, Y_other, ws2))
