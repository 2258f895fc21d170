"""The C-ABI library loads and exports every entry point the header declares; host-side
validation and size queries behave as documented.  No call here reaches the GPU."""
import ctypes
import os
import re

import numpy as np
import pytest

from bit_quantized_dit_amd import w4a4 as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    with open(os.path.join(ROOT, "include", "w4a4.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(w4a4_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(B.LIB_PATH):
        from bit_quantized_dit_amd import build
        build.build_library()
    return B.lib()


def test_every_declared_symbol_is_exported(L):
    names = _declared()
    assert len(names) >= 11
    assert set(names) == set(B.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    assert L.w4a4_status_string(0) == b"ok"
    assert b"invalid" in L.w4a4_status_string(1)
    assert L.w4a4_status_string(99) == b"unknown status"


def test_packed_size_layouts(L):
    # d_in 512, k 16 -> K_J 496, K_pad 512; d_out 1024
    s1 = B.w4a4_packed_size(512, 1024, 16, B.W4A4_WS_1X32)
    s2 = B.w4a4_packed_size(512, 1024, 16, B.W4A4_WS_128X1_STRIPE)
    s3 = B.w4a4_packed_size(512, 1024, 16, B.W4A4_WS_32X32_TILE)
    payload = 1024 * 256
    assert s1 >= payload + 1024 * 16 + 1024 * 32 * 2
    # every layout carries the step-major per-row copy; tiles and stripes have fewer
    # canonical scale bytes than 1x32
    assert s2 < s1 and s3 < s1 and s1 - s2 < 1024 * 16 and s1 - s3 < 1024 * 16
    for s in (s1, s2, s3):
        assert s % 256 == 0


@pytest.mark.parametrize("args,code", [
    ((512, 1024, 16, 7), 1),        # bad layout
    ((512, 1024, 513, 0), 1),       # k > d_in
    ((512, 1024, -1, 0), 1),        # k < 0
    ((0, 1024, 0, 0), 1),           # empty d_in
    ((40000, 1024, 0, 0), 2),       # d_in beyond the supported maximum
])
def test_packed_size_rejects(L, args, code):
    n = ctypes.c_size_t(0)
    assert L.w4a4_packed_size(*args, ctypes.byref(n)) == code


def _fake_desc(d_in=512, d_out=1024, k=16, layout=0):
    d = B.W4A4Packed()
    d.d_in, d.d_out, d.k, d.layout = d_in, d_out, k, layout
    d.k_j = d_in - k
    d.k_pad = (d.k_j + 127) // 128 * 128
    d.k_ld = (k + 31) // 32 * 32
    fake = 0x100000  # never dereferenced: only host-side logic runs below
    d.colmap = d.s = d.O = d.J = d.B_q = d.B_s = d.B_s_rows = d.W_O = d.B_q_tiles = fake
    return d


def test_workspace_layout_is_host_logic(L):
    d = _fake_desc()
    out = B.W4A4WsLayout()
    assert L.w4a4_workspace_layout(1000, ctypes.byref(d), ctypes.byref(out)) == 0
    assert out.a_q == 0 and out.a_s >= 1000 * 256 and out.x_o >= out.a_s + 1000 * 16
    assert out.total >= out.x_o + 1000 * 32 * 2 and out.total % 256 == 0
    # A_q is tiled in 16-token blocks: a ragged T reserves the whole last block
    assert L.w4a4_workspace_layout(1001, ctypes.byref(d), ctypes.byref(out)) == 0
    assert out.a_s >= 1008 * 256
    n = ctypes.c_size_t(0)
    assert L.w4a4_workspace_size(0, ctypes.byref(d), ctypes.byref(n)) == 0 and n.value == 0


def test_split_plan_is_host_logic(L):
    """The GEMM's split-K plan, seen through the workspace's partial-sum region (host
    logic).  Tiles are 256 x 256; the tiles that fill whole rounds of 256 workgroups run
    whole, the rest are cut into s = min(256 // tail, 16, K steps // 16) ranges of K when
    s >= 3, each range taking a 256 KiB block of fp32 partial sums."""
    out = B.W4A4WsLayout()
    blk = 256 * 256 * 4

    def partial(T, d_in, d_out, k):
        d = _fake_desc(d_in, d_out, k)
        assert L.w4a4_workspace_layout(T, ctypes.byref(d), ctypes.byref(out)) == 0
        assert out.partial >= out.x_o and out.total % 256 == 0
        return out.total - out.partial

    # 4096 tokens, 13824 -> 5120: 16 x 20 = 320 tiles, 64 in the last round, 110 K steps
    assert partial(4096, 13824, 5120, 64) == 64 * 4 * blk
    # 57600 tokens, 5120 -> 13824: 225 x 54 tiles, a tail of 118 would give 2 ranges: whole
    assert partial(57600, 5120, 13824, 128) == 0
    # 4096 tokens, 5120 -> 13824: 864 tiles, a tail of 96: 2 ranges, whole
    assert partial(4096, 5120, 13824, 64) == 0
    # 7200 tokens, 13824 -> 5120: 29 x 20 = 580 tiles, a tail of 68: 3 ranges
    assert partial(7200, 13824, 5120, 64) == 68 * 3 * blk
    # 256 tokens, 5120 -> 13824: 54 tiles, but 43 K steps allow only 2 ranges: whole
    assert partial(256, 5120, 13824, 128) == 0
    # 256 tokens, 13824 -> 5120: 20 tiles, 110 K steps: 6 ranges (12 tiles' worth allowed)
    assert partial(256, 13824, 5120, 64) == 20 * 6 * blk
    # one tile, 20000 inputs (158 K steps): 9 ranges
    assert partial(40, 20000, 64, 16) == 9 * blk
    # one tile, 32768 inputs half of them outliers (128 FP4 + 512 BF16 steps): the
    # 16-range cap
    assert partial(16, 32768, 64, 16384) == 16 * blk
    # short K (5 steps): never split; a round of exactly 256 tiles: nothing left over
    assert partial(1000, 512, 1024, 16) == 0
    assert partial(256 * 16, 5120, 256 * 16, 64) == 0


def test_split_plan_invariants(L):
    """Over random shapes: the partial-sum region is whole 256 KiB blocks, one per K
    range of a tail tile; ranges hold at least 16 K steps; at most 255 tail tiles x 16
    ranges; every split puts at least 3 ranges on each tail tile and no more items in
    the last round than there are workgroup slots (256)."""
    rng = np.random.default_rng(7)
    out = B.W4A4WsLayout()
    blk = 256 * 256 * 4
    for _ in range(400):
        T = int(rng.integers(1, 70000))
        d_in = int(rng.integers(2, 32769))
        d_out = int(rng.integers(1, 20000))
        k = int(rng.integers(0, min(d_in, 512) + 1))
        d = _fake_desc(d_in, d_out, k)
        assert L.w4a4_workspace_layout(T, ctypes.byref(d), ctypes.byref(out)) == 0
        nbytes = out.total - out.partial
        # the region is padded to 256 bytes; blocks are 256 KiB, so it is exact
        assert nbytes % blk == 0
        blocks = nbytes // blk
        tiles = -(-T // 256) * -(-d_out // 256)
        tail = tiles if tiles < 256 else tiles % 256
        nsteps = d.k_pad // 128 + d.k_ld // 32
        if blocks:
            assert tail > 0 and blocks % tail == 0
            s = blocks // tail
            assert 3 <= s <= 16 and nsteps // s >= 16 and tail * s <= 256
        else:
            assert tail == 0 or min(256 // tail, 16, nsteps // 16) < 3


def test_dynamic_sizes_are_host_logic(L):
    """Per-call outlier selection: blob and workspace sizes, and the shape rules (d_in
    even and at most 16384 so one workgroup sorts every column's score)."""
    n = ctypes.c_size_t(0)
    assert L.w4a4_packed_dyn_size(512, 1024, 16, 0, ctypes.byref(n)) == 0
    # the k = 0 blob plus a bf16 copy of W
    assert n.value >= B.w4a4_packed_size(512, 1024, 0, 0) + 1024 * 512 * 2 and n.value % 256 == 0
    assert L.w4a4_packed_dyn_size(511, 1024, 16, 0, ctypes.byref(n)) == 2         # odd d_in
    assert L.w4a4_packed_dyn_size(16386, 1024, 16, 0, ctypes.byref(n)) == 2       # d_in > 16384
    assert L.w4a4_packed_dyn_size(512, 1024, 513, 0, ctypes.byref(n)) == 1        # k > d_in
    assert L.w4a4_packed_dyn_size(16384, 64, 16384, 2, ctypes.byref(n)) == 0      # the largest
    d = B.W4A4PackedDyn()
    d.base = _fake_desc(k=0)
    d.k = 40
    d.W_t = 0x100000
    out = B.W4A4WsDynLayout()
    assert L.w4a4_workspace_dyn_layout(1000, ctypes.byref(d), ctypes.byref(out)) == 0
    base = B.W4A4WsLayout()
    assert L.w4a4_workspace_layout(1000, ctypes.byref(_fake_desc(k=40)), ctypes.byref(base)) == 0
    # codes over K_pad = roundup(d_in, 128), X_O over k_ld = roundup(k, 32)
    assert out.base.a_s >= 1008 * 256 and out.base.x_o >= out.base.a_s + 1000 * 16
    assert out.base.total >= out.base.x_o + 1000 * 64 * 2
    assert out.colmax >= out.base.total and out.O >= out.colmax + 512 * 4
    assert out.colmap >= out.O + 40 * 4 and out.W_O >= out.colmap + 512 * 4
    assert out.total >= out.W_O + 1024 * 64 * 2 and out.total % 256 == 0
    d.base = _fake_desc(k=16)          # the base blob must hold no static outliers
    assert L.w4a4_workspace_dyn_layout(1000, ctypes.byref(d), ctypes.byref(out)) == 1
    d.base = _fake_desc(k=0)
    d.W_t = 0
    assert L.w4a4_workspace_dyn_layout(1000, ctypes.byref(d), ctypes.byref(out)) == 1
    # the per-call entry point validates before it touches the device
    d.W_t = 0x100000
    assert L.w4a4_linear_dyn(ctypes.c_void_p(256), 0, 1000, ctypes.byref(d), ctypes.c_void_p(256),
                             ctypes.c_void_p(256), 10, None) == 2                  # workspace too small
    assert L.w4a4_linear_dyn(ctypes.c_void_p(256), 3, 1000, ctypes.byref(d), ctypes.c_void_p(256),
                             ctypes.c_void_p(256), 1 << 40, None) == 1             # bad dtype


def test_ffn_workspace_is_host_logic(L):
    """The fused FFN block's workspace: the up layer's, then the down layer's, then the
    down layer's reciprocals; mismatched layers and bad arguments fail before any launch."""
    up = _fake_desc(d_in=256, d_out=704, k=8)
    dn = _fake_desc(d_in=704, d_out=256, k=13)
    out = B.W4A4FfnWsLayout()
    assert L.w4a4_ffn_workspace_layout(300, ctypes.byref(up), ctypes.byref(dn), ctypes.byref(out)) == 0
    wu, wd = B.W4A4WsLayout(), B.W4A4WsLayout()
    assert L.w4a4_workspace_layout(300, ctypes.byref(up), ctypes.byref(wu)) == 0
    assert L.w4a4_workspace_layout(300, ctypes.byref(dn), ctypes.byref(wd)) == 0
    assert (out.up.a_q, out.up.a_s, out.up.x_o, out.up.total) == (wu.a_q, wu.a_s, wu.x_o, wu.total)
    assert (out.down.a_q, out.down.a_s, out.down.x_o, out.down.total) == (wd.a_q, wd.a_s, wd.x_o, wd.total)
    assert out.up_base == 0 and out.down_base >= wu.total and out.rinv >= out.down_base + wd.total
    assert out.total >= out.rinv + 8 * (704 - 13) and out.total % 256 == 0 and out.down_base % 256 == 0
    n = ctypes.c_size_t(0)
    assert L.w4a4_ffn_workspace_size(300, ctypes.byref(up), ctypes.byref(dn), ctypes.byref(n)) == 0
    assert n.value == out.total
    bad = _fake_desc(d_in=640, d_out=256, k=13)     # up.d_out != down.d_in
    assert L.w4a4_ffn_workspace_size(300, ctypes.byref(up), ctypes.byref(bad), ctypes.byref(n)) == 2
    assert L.w4a4_ffn_workspace_size(-1, ctypes.byref(up), ctypes.byref(dn), ctypes.byref(n)) == 1
    p16 = ctypes.c_void_p(256)
    assert L.w4a4_ffn_forward(p16, 0, 300, ctypes.byref(up), ctypes.byref(dn), p16, p16, 10, None) == 2
    assert L.w4a4_ffn_forward(p16, 9, 300, ctypes.byref(up), ctypes.byref(dn), p16, p16, 1 << 40, None) == 1
    assert L.w4a4_ffn_up_quantize(ctypes.c_void_p(258), 0, 300, ctypes.byref(up), ctypes.byref(dn), p16,
                                  1 << 40, None) == 3
    # T = 0 is a no-op that touches nothing
    assert L.w4a4_ffn_forward(p16, 0, 0, ctypes.byref(up), ctypes.byref(dn), p16, p16, 1 << 40, None) == 0


def test_ffn_permutation_puts_outliers_last():
    P = B.ffn_permutation(np.array([40, 3, 17]), 48)
    assert list(P[-3:]) == [3, 17, 40] and sorted(P) == list(range(48))
    assert np.all(np.diff(P[:-3]) > 0)


def test_search_scratch_size_is_host_logic(L):
    ks = np.array([0, 16, 64], np.int32)
    vp = ks.ctypes.data_as(ctypes.c_void_p)
    n = ctypes.c_size_t(0)
    assert L.w4a4_search_scratch_size(256, 512, 1024, vp, 3, 0, ctypes.byref(n)) == 0
    # two fp32 outputs of T_cal x d_out plus the largest candidate's blob, 256-B granules
    blob = max(B.w4a4_packed_size(512, 1024, int(k), 0) for k in ks)
    assert n.value >= 2 * 256 * 1024 * 4 + blob and n.value % 256 == 0
    bad = np.array([0, 600], np.int32)
    assert L.w4a4_search_scratch_size(256, 512, 1024, bad.ctypes.data_as(ctypes.c_void_p), 2, 0,
                                      ctypes.byref(n)) == 1                      # k > d_in
    assert L.w4a4_search_scratch_size(256, 512, 1024, vp, 0, 0, ctypes.byref(n)) == 1   # no candidates
    assert L.w4a4_search_scratch_size(256, 512, 1024, vp, 3, 7, ctypes.byref(n)) == 1   # bad layout
    assert L.w4a4_search_scratch_size(65535 * 64 + 1, 512, 1024, vp, 3, 0, ctypes.byref(n)) == 2
    # the search itself validates before it touches the device
    al = np.array([0.5, 1.5], np.float32)
    err = np.zeros(6, np.float64)
    best = np.zeros(2, np.int32)
    p = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    assert L.w4a4_search_alpha_k(ctypes.c_void_p(256), 0, 256, 512, ctypes.c_void_p(256), 1024, p(al), 2, vp, 3,
                                 0, ctypes.c_void_p(256), 1 << 30, p(err), p(best), None) == 1   # alpha > 1
    assert L.w4a4_search_alpha_k(ctypes.c_void_p(256), 0, 256, 512, ctypes.c_void_p(256), 1024, p(al), 1, vp, 3,
                                 0, ctypes.c_void_p(256), 1024, p(err), p(best), None) == 2      # scratch too small
    assert L.w4a4_search_alpha_k(ctypes.c_void_p(256), 0, 256, 512, ctypes.c_void_p(260), 1024, p(al), 1, vp, 3,
                                 0, ctypes.c_void_p(256), 1 << 30, p(err), p(best), None) == 3   # misaligned W


def test_per_call_entry_points_validate_before_any_launch(L):
    d = _fake_desc()
    n = ctypes.c_size_t(0)
    # T < 0
    assert L.w4a4_linear(ctypes.c_void_p(16), 0, -1, ctypes.byref(d), ctypes.c_void_p(16),
                         ctypes.c_void_p(16), 1 << 30, None) == 1
    # bad dtype
    assert L.w4a4_quantize_activations(ctypes.c_void_p(16), 5, 4, ctypes.byref(d), ctypes.c_void_p(16),
                                       1 << 30, None) == 1
    # workspace too small
    assert L.w4a4_quantize_activations(ctypes.c_void_p(256), 0, 4, ctypes.byref(d), ctypes.c_void_p(256),
                                       10, None) == 2
    # misaligned pointers
    assert L.w4a4_gemm_prequantized(ctypes.c_void_p(258), 1 << 30, 4, ctypes.byref(d), ctypes.c_void_p(256),
                                    None) == 3
    # T == 0 is a no-op
    assert L.w4a4_linear(None, 0, 0, ctypes.byref(d), None, None, 0, None) == 0
    # inconsistent descriptor
    bad = _fake_desc()
    bad.k_pad = 128
    assert L.w4a4_linear(ctypes.c_void_p(256), 0, 4, ctypes.byref(bad), ctypes.c_void_p(256),
                         ctypes.c_void_p(256), 1 << 30, None) == 1
    # calibration argument checks (alpha outside [0,1], k > d_in)
    assert L.w4a4_calibrate_scales(ctypes.c_void_p(256), 0, 8, 64, ctypes.c_void_p(256), 32,
                                   ctypes.c_float(1.5), 4, ctypes.c_void_p(256), ctypes.c_void_p(256),
                                   None, None, None) == 1
    assert L.w4a4_calibrate_scales(ctypes.c_void_p(256), 0, 8, 64, ctypes.c_void_p(256), 32,
                                   ctypes.c_float(0.5), 65, ctypes.c_void_p(256), ctypes.c_void_p(256),
                                   None, None, None) == 1
    assert L.w4a4_gelu_tanh_bf16(ctypes.c_void_p(258), 8, ctypes.c_void_p(256), None) == 3
    # the fused up projection + GELU entry points validate the same way
    assert L.w4a4_linear_gelu_bf16(ctypes.c_void_p(16), 0, -1, ctypes.byref(d), ctypes.c_void_p(16),
                                   ctypes.c_void_p(16), 1 << 30, None) == 1
    assert L.w4a4_linear_gelu_bf16(ctypes.c_void_p(256), 0, 4, ctypes.byref(d), None,
                                   ctypes.c_void_p(256), 1 << 30, None) == 1
    assert L.w4a4_linear_gelu_bf16(None, 0, 0, ctypes.byref(d), None, None, 0, None) == 0
    assert L.w4a4_gemm_prequantized_gelu_bf16(ctypes.c_void_p(256), 10, 4, ctypes.byref(d),
                                              ctypes.c_void_p(256), None) == 2
    assert L.w4a4_gemm_prequantized_gelu_bf16(ctypes.c_void_p(256), 1 << 30, 4, ctypes.byref(d),
                                              ctypes.c_void_p(264), None) == 3
    assert L.w4a4_gemm_prequantized_gelu_bf16(ctypes.c_void_p(256), 1 << 30, 4, ctypes.byref(bad),
                                              ctypes.c_void_p(256), None) == 1


def test_untile_codes_inverts_the_documented_tiled_order():
    """The binding's de-tiling (used to compare the tiled A_q / B_q copies with the
    oracle's row-major codes) inverts the order the header documents."""
    import torch
    rng = np.random.default_rng(5)
    rows, k_pad = 48, 384
    canon = rng.integers(0, 256, size=(rows, k_pad // 2), dtype=np.uint8)
    nkb = k_pad // 128
    tiled = np.zeros(rows * k_pad // 2, dtype=np.uint8)
    for t in range(rows):
        for byte in range(k_pad // 2):
            p = 2 * byte
            c = (p % 128) // 32
            off = ((t // 16) * nkb + p // 128) * 1024 + (t % 16) * 64 + (c ^ ((t % 16) // 4)) * 16 + ((p % 128) // 2) % 16
            tiled[off] = canon[t, byte]
    got = B.untile_codes(torch.from_numpy(tiled), rows, k_pad).numpy()
    assert np.array_equal(got, canon)
