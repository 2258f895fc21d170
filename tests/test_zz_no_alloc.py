"""w4a4_linear_noalloc (for callers that cannot allocate device memory) against
w4a4_linear: two calls in a row on the same fixed scratch, the second with fewer
tokens, each bit-identical to w4a4_linear with a caller workspace and within the
output tolerance of the oracle; a split-K shape uses the scratch's partial-sum
region; a call that needs more than the scratch holds is refused on the host."""
import numpy as np
import pytest
import torch

from bit_quantized_dit_amd import synth
from bit_quantized_dit_amd import w4a4 as B
from tests.gpu_util import _banner, assert_y_close, to_dev

pytestmark = pytest.mark.gpu


def _packed(T, d_in, d_out, k, layout, seed):
    spec = synth.WORKLOADS[2]
    inp = synth.layer_inputs(spec, T=T, d_in=d_in, d_out=d_out, k=k, T_cal=128)
    W = to_dev(inp["W"])
    s, O, _, _ = B.w4a4_calibrate_scales(to_dev(inp["X_cal"]), W, spec.alpha, k)
    return inp, s, O, B.w4a4_pack_weights(W, s, O, layout)


@pytest.mark.parametrize("T1,T2,d_in,d_out,k,layout", [(3000, 700, 5120, 1536, 64, 0),
                                                       (600, 130, 6400, 520, 24, 2)])
def test_noalloc_matches_linear(orc, T1, T2, d_in, d_out, k, layout):
    _banner(f"no-alloc linear: T={T1} then T={T2}, {d_in}->{d_out}, k={k}, layout {layout}")
    inp, s, O, packed = _packed(T1, d_in, d_out, k, layout, 0)
    J = np.setdiff1d(np.arange(d_in), O).astype(np.int32)
    pk_o = orc.pack_weights(inp["W"], s, O, J, layout)
    assert B.w4a4_workspace_size(T1, packed) <= B.NOALLOC_SCRATCH_BYTES
    rng = np.random.default_rng(T1)
    for T in (T1, T2):
        X = to_dev(inp["X"][:T])
        Yn = torch.full((T, d_out), float("nan"), device="cuda")
        B.w4a4_linear_noalloc(X, packed, Yn)
        Y = torch.empty(T, d_out, device="cuda")
        B.w4a4_linear(X, packed, Y, B.alloc_workspace(T, packed))
        torch.cuda.synchronize()
        assert bool(torch.equal(Yn.view(torch.int32), Y.view(torch.int32))), f"T={T}: differs from w4a4_linear"
        rows = np.unique(np.concatenate([[0, T - 1], rng.integers(0, T, 24)]))
        Aq, As, XO = orc.act_prep(inp["X"][rows], s, O, J)
        Yref = orc.output_full(Aq, As, XO, pk_o)
        st = assert_y_close(Yn[torch.as_tensor(rows, device="cuda")].cpu().numpy(), Yref)
        _banner(f"  T={T}: bit-identical to w4a4_linear; sampled rows vs oracle {st}")


def test_noalloc_refuses_oversized_calls():
    inp, s, O, packed = _packed(64, 4096, 256, 16, 0, 1)
    T = B.NOALLOC_SCRATCH_BYTES // 2048 + 1           # > 2048 workspace bytes per token at d_in 4096
    assert B.w4a4_workspace_size(T, packed) > B.NOALLOC_SCRATCH_BYTES
    X = torch.zeros(T, 4096, dtype=torch.bfloat16, device="cuda")
    Y = torch.empty(T, 256, device="cuda")
    with pytest.raises(B.W4A4Error) as e:
        B.w4a4_linear_noalloc(X, packed, Y)
    assert e.value.status == 6
