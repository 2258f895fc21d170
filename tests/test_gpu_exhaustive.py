"""Exhaustive check of the GPU's MXFP4 activation encoding (E8M0 scale per 32-block,
E2M1 codes; the format named in "W4A4 Quantization for Inference on Wan2.2-I2V-A14B
(ICME 2026 Challenge)", sec. 1-2) against the oracle's act-prep, with s = 1 so that the
division is exact and the encoder alone decides the codes.

Every binary32 bit pattern goes through w4a4_quantize_activations at least once:

* natural scales: a block holds one sign and one mantissa at 32 consecutive exponent
  fields (0-31, 32-63, ..., 192-223, 223-254), so its scale comes from its top element
  and the others sit 1, 2, ..., 31 binades below it, crossing every E2M1 threshold,
  the flush to zero and the subnormal range; the 2^24 NaN and Inf patterns fill blocks
  of their own (scale 0xFF, zero nibbles);
* fixed scales E in {-127, -20, -2, 0, 2, 125}: one element of each block is
  +-4 * 2^E, which fixes E, and the other 31 run through every pattern whose value
  scaled by 2^-E lies in [2^-4, 8) (for E = -127 every subnormal), so every rounding
  decision of the E2M1 grid is taken at each of these scales, the subnormal scale
  2^-127 included.

The same patterns also run through the bf16 activation path (all 65536 bf16 patterns in
the same two arrangements).  Codes and scales must be bit-exact; the test stops at the
first mismatch and names it.
"""
import numpy as np
import pytest
import torch

from bit_quantized_dit_amd import w4a4 as B
from tests.gpu_util import _banner, u8

pytestmark = pytest.mark.gpu

D_IN = 4096                  # 128 blocks per token row, the fast act-prep path
ROWS = 16384                 # rows per chunk: 2^26 patterns
GROUP_START = np.array([0, 32, 64, 96, 128, 160, 192, 223], np.uint32)
FIXED_E = (-127, -20, -2, 0, 2, 125)


def natural_chunk(c: int) -> np.ndarray:
    """Chunk c (2^26 patterns, 2^21 blocks) of the natural-scale arrangement: block b
    has mantissa b % 2^23, exponent group (b / 2^23) % 8 and sign b / 2^26, and its
    element i the exponent field GROUP_START[group] + i.  A chunk covers a quarter of
    the mantissas of one group and sign."""
    mant = ((c & 3) << 21) + np.arange(1 << 21, dtype=np.uint32)
    g, sign = (c >> 2) & 7, c >> 5
    ex = GROUP_START[g] + np.arange(32, dtype=np.uint32)
    return ((np.uint32(sign) << 31) | (ex[None, :] << 23) | mant[:, None]).ravel()


def special_patterns() -> np.ndarray:
    """All 2^24 NaN and Inf patterns, 32 consecutive ones per block."""
    m = np.arange(1 << 23, dtype=np.uint32)
    return np.concatenate([0x7F800000 | m, 0xFF800000 | m])


def fixed_e_patterns(E: int, mbits: int = 23) -> np.ndarray:
    """Blocks of one pin +-4 * 2^E and 31 patterns of the window: every sign and
    mantissa (mbits wide: 23 for binary32, 7 for bf16 patterns) at exponent fields
    max(0, E + 123) .. E + 129 (|x| 2^-E in [2^-4, 8)), whose values never raise the
    block's scale above E.  The pin's position cycles through the block."""
    top = 8 + mbits
    lo, hi = max(0, E + 127 - 4), E + 127 + 2
    ex = np.arange(lo, hi + 1, dtype=np.uint32)
    m = np.arange(1 << mbits, dtype=np.uint32)
    body = ((ex[:, None] << mbits) | m[None, :]).ravel()
    body = np.concatenate([body, body | np.uint32(1 << top)])
    nblk = (body.size + 30) // 31
    body = np.concatenate([body, np.zeros(nblk * 31 - body.size, np.uint32)]).reshape(nblk, 31)
    # 4 * 2^E: exponent field E + 129, zero mantissa (for E = -127: 2^-125, field 2)
    pins = np.full(nblk, np.uint32(E + 129) << mbits, np.uint32)
    pins[1::2] |= np.uint32(1 << top)
    pos = np.arange(nblk) % 32
    cols = np.arange(32)[None, :]
    src = np.minimum(cols - (cols > pos[:, None]), 30)   # body index of the non-pin slots
    out = body[np.arange(nblk)[:, None], src]
    out[np.arange(nblk), pos] = pins
    return out.ravel()


@pytest.fixture(scope="module")
def layer():
    """d_in = 4096, no outlier column, s = 1 (x / s = x exactly)."""
    W = torch.zeros(32, D_IN, device="cuda")
    return B.w4a4_pack_weights(W, np.ones(D_IN, np.float32), np.zeros(0, np.int32), 0)


def _run(orc, layer, pats: np.ndarray, dtype: str, what: str) -> None:
    """Quantize pats (a multiple of D_IN elements, one token row per D_IN) on the GPU
    and in the oracle; compare codes and scales bit for bit."""
    if dtype == "bf16":
        xh = pats.astype(np.uint16).reshape(-1, D_IN)
        Xd = torch.from_numpy(xh.view(np.int16)).cuda().view(torch.bfloat16)
    else:
        xh = pats.view(np.float32).reshape(-1, D_IN)
        Xd = torch.from_numpy(xh).cuda()
    T = xh.shape[0]
    ws = B.alloc_workspace(T, layer)
    B.w4a4_quantize_activations(Xd, layer, ws)
    v = B.workspace_views(ws, T, layer)
    Aq, As = u8(v["A_q"]), u8(v["A_s"])
    J = np.arange(D_IN, dtype=np.int32)
    Aq_o, As_o, _ = orc.act_prep(xh, np.ones(D_IN, np.float32), np.zeros(0, np.int32), J)
    if not np.array_equal(As, As_o):
        r, b = np.argwhere(As != As_o)[0]
        raise AssertionError(f"{what}: scale of row {r} block {b} is {As[r, b]:#04x}, oracle {As_o[r, b]:#04x}; "
                             f"block {[hex(int(p)) for p in xh[r, 32 * b:32 * b + 32].view(np.uint32 if dtype == 'f32' else np.uint16)]}")
    if not np.array_equal(Aq, Aq_o):
        r, c = np.argwhere(Aq != Aq_o)[0]
        p = xh[r, 2 * c:2 * c + 2]
        raise AssertionError(f"{what}: code byte {c} of row {r} is {Aq[r, c]:#04x}, oracle {Aq_o[r, c]:#04x}; "
                             f"elements {p}, block scale {As[r, c // 16]:#04x}")


def test_every_fp32_pattern_natural_scales(orc, layer):
    n = (1 << 32) >> 26
    for c in range(n):
        _run(orc, layer, natural_chunk(c), "f32", f"natural chunk {c}")
        if c % 8 == 7:
            _banner(f"exhaustive fp32: {(c + 1) << 26} of 2^32 patterns bit-exact")
    _run(orc, layer, special_patterns(), "f32", "NaN/Inf patterns")
    _banner("exhaustive fp32: all NaN/Inf patterns bit-exact (scale 0xFF, zero nibbles)")


def test_every_fp32_pattern_fixed_scales(orc, layer):
    for E in FIXED_E:
        p = fixed_e_patterns(E)
        p = np.concatenate([p, np.zeros((-p.size) % D_IN, np.uint32)])
        for c0 in range(0, p.size, ROWS * D_IN):
            _run(orc, layer, p[c0:c0 + ROWS * D_IN], "f32", f"fixed E = {E}, offset {c0}")
        _banner(f"exhaustive fp32 at E = {E}: {p.size} elements bit-exact")


def test_every_bf16_pattern(orc, layer):
    """The bf16 activation path over all 65536 patterns, natural and fixed scales."""
    h = np.arange(1 << 16, dtype=np.uint32)
    blocks = []
    m = np.arange(128, dtype=np.uint32)
    for g in GROUP_START:
        for sg in (0, 1):
            e = g + np.arange(32, dtype=np.uint32)
            blocks.append(((np.uint32(sg) << 15) | (e[None, :] << 7) | m[:, None]).ravel())
    blocks.append(h[((h >> 7) & 0xFF) == 0xFF])
    for E in FIXED_E:
        blocks.append(fixed_e_patterns(E, mbits=7))
    p = np.concatenate(blocks).astype(np.uint32)
    assert np.all(np.isin(h, p))
    p = np.concatenate([p, np.zeros((-p.size) % D_IN, np.uint32)])
    _run(orc, layer, p, "bf16", "bf16 patterns")
    _banner(f"exhaustive bf16: {p.size} elements bit-exact")
