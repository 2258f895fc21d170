"""Two layers on two streams at once, each with its own workspace: the library keeps
no global state and its kernels never wait on one another's workgroups, so concurrent
calls give exactly the results of sequential ones.  One layer's GEMM is split along K
(two launches and a partial-sum region), the other's runs whole tiles."""
import numpy as np
import pytest
import torch

from bit_quantized_dit_amd import synth
from bit_quantized_dit_amd import w4a4 as B
from tests.gpu_util import _banner, to_dev

pytestmark = pytest.mark.gpu


def _layer(T, d_in, d_out, k, layout):
    spec = synth.WORKLOADS[2]
    inp = synth.layer_inputs(spec, T=T, d_in=d_in, d_out=d_out, k=k, T_cal=64)
    X, Xc, W = to_dev(inp["X"]), to_dev(inp["X_cal"]), to_dev(inp["W"])
    s, O, _, _ = B.w4a4_calibrate_scales(Xc, W, spec.alpha, k)
    packed = B.w4a4_pack_weights(W, s, O, layout)
    return X, packed, B.alloc_workspace(T, packed), torch.empty(T, d_out, device="cuda")


def test_two_streams_match_sequential():
    _banner("two layers on two streams: 600x6400->520 (split K) and 1000x2048->1536 (whole)")
    a = _layer(600, 6400, 520, 24, 2)
    b = _layer(1000, 2048, 1536, 32, 0)
    ya, yb = torch.empty_like(a[3]), torch.empty_like(b[3])
    B.w4a4_linear(a[0], a[1], ya, a[2])
    B.w4a4_linear(b[0], b[1], yb, b[2])
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    for rep in range(5):
        a[3].fill_(float("nan"))
        b[3].fill_(float("nan"))
        torch.cuda.synchronize()
        for _ in range(3):       # several calls in flight on each stream
            B.w4a4_linear(a[0], a[1], a[3], a[2], sa)
            B.w4a4_linear(b[0], b[1], b[3], b[2], sb)
        torch.cuda.synchronize()
        assert bool(torch.equal(a[3].view(torch.int32), ya.view(torch.int32))), f"stream A, repetition {rep}"
        assert bool(torch.equal(b[3].view(torch.int32), yb.view(torch.int32))), f"stream B, repetition {rep}"
    _banner("  5 repetitions bit-identical to the sequential calls")
