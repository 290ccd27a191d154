"""Stochastic rounding at its edges, through the C ABI, bit for bit against the
CPU oracle.

* An element whose random offset is exactly 0 (the generator's 24 drawn bits
  all zero) and whose scaled value is a negative binary32 subnormal: its code
  is floor(y) = -1, not 0 -- the rounding step floors the sum of the scaled
  value and the offset, and the sum is the subnormal itself.  The same
  element with -0 gives 0.  Plain, error-feedback, EF21, weight-difference and
  Hadamard-smoothed compresses.
* Index ranges that cross a multiple of 2^32 inside one tile of the kernels
  (offsets 2^32 - 3B): the generator's input is the 64-bit global index, whose
  high half changes there.

Positions with a zero offset are found by searching the oracle's own
generator over consecutive indices (about one in 2^24).
"""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import assert_same, codes_np, f32_np, f32_to_gpu, say, scales_np
from weight_communication_compression_amd import lowbit as L

pytestmark = pytest.mark.gpu

SEED = 20240611
BITS = [2, 4, 8]
TINY = np.float32(-2.0 ** -140)      # a negative subnormal input


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    L.lib()
    O.lib()
    yield
    torch.cuda.synchronize()


@pytest.fixture(scope="module")
def zero_offset_indices():
    """Global indices (>= 4096) whose stochastic-rounding offset is 0."""
    hits, i0, chunk = [], 4096, 1 << 24
    while len(hits) < 2 and i0 < (1 << 31):
        u = O.sr_uniform(SEED, i0, chunk)
        hits += [i0 + int(k) for k in np.nonzero(u == 0.0)[0]]
        i0 += chunk
    assert hits, "no zero offset found"
    return hits


def _placed(hit, B, nblocks=6):
    """index_offset (a multiple of B) and the position of `hit` in the
    buffer: in its second block."""
    k = hit % B + B
    return hit - k, k, nblocks * B


def _background(n, seed):
    return np.random.default_rng(seed).standard_normal(n).astype(np.float32)


def _code_at(words, k, bits):
    per = 32 // bits
    return (int(words[k // per]) >> ((k % per) * bits)) & ((1 << bits) - 1)


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("B", [64, 256])
@pytest.mark.parametrize("val", ["subnormal", "negzero"])
def test_plain_zero_offset(zero_offset_indices, bits, B, val):
    hit = zero_offset_indices[0]
    off, k, n = _placed(hit, B)
    x = _background(n, bits * 7 + B)
    x[k] = TINY if val == "subnormal" else np.float32(-0.0)
    say(f"sr zero offset plain bits={bits} B={B} {val} k={k} off={off}")
    c, s = L.quantize_pack(f32_to_gpu(x), bits, B, True, SEED, off)
    torch.cuda.synchronize()
    wc, ws = O.quantize_pack(x, bits, B, True, SEED, off)
    assert O.sr_uniform(SEED, off + k, 1)[0] == 0.0
    half = 1 << (bits - 1)
    assert _code_at(wc, k, bits) == (half - 1 if val == "subnormal" else half)
    assert_same(scales_np(s), ws, "scales")
    assert_same(codes_np(c), wc, "codes")


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("B", [64, 256])
def test_ef_and_ef21_zero_offset(zero_offset_indices, bits, B):
    hit = zero_offset_indices[0]
    off, k, n = _placed(hit, B)
    g = _background(n, 3 + bits)
    g[k] = TINY
    e0 = np.zeros(n, np.float32)
    say(f"sr zero offset ef bits={bits} B={B} k={k}")
    ge, gr = f32_to_gpu(g), f32_to_gpu(e0)
    c, s = L.ef_compress(ge, gr, bits, B, True, SEED, off)
    gh = f32_to_gpu(e0)
    c21, s21 = L.ef21_compress(ge, gh, bits, B, True, SEED, off)
    torch.cuda.synchronize()
    wc, ws, we = O.ef_compress(g, e0, bits, B, True, SEED, off)
    assert _code_at(wc, k, bits) == (1 << (bits - 1)) - 1
    assert_same(scales_np(s), ws, "ef scales")
    assert_same(codes_np(c), wc, "ef codes")
    assert_same(f32_np(gr), we, "ef residual")
    wc21, ws21, wh = O.ef21_compress(g, e0, bits, B, True, SEED, off)
    assert_same(scales_np(s21), ws21, "ef21 scales")
    assert_same(codes_np(c21), wc21, "ef21 codes")
    assert_same(f32_np(gh), wh, "ef21 state")


@pytest.mark.parametrize("bits", [4, 8])
def test_wdiff_zero_offset(zero_offset_indices, bits):
    B = 64
    hit = zero_offset_indices[0]
    off, k, n = _placed(hit, B)
    w_old = _background(n, 11)
    w_new = (w_old + _background(n, 12)).astype(np.float32)
    w_new[k] = np.float32(0.0)
    w_old[k] = np.float32(-TINY)        # difference: the negative subnormal
    say(f"sr zero offset wdiff bits={bits} k={k}")
    c, s = L.wdiff_compress(f32_to_gpu(w_new), f32_to_gpu(w_old), bits, B, True, SEED, off)
    torch.cuda.synchronize()
    wc, ws = O.wdiff_compress(w_new, w_old, bits, B, True, SEED, off)
    assert _code_at(wc, k, bits) == (1 << (bits - 1)) - 1
    assert_same(scales_np(s), ws, "scales")
    assert_same(codes_np(c), wc, "codes")


def _hadamard_tiny_at(k, B, n, seed):
    """Input whose block holding position k transforms (before the forward
    scale 2^-h, h = floor(log2(B) / 2)) to -2^(h-149) at every position of
    k's class mod 2, and to about +-2 at the others (so the block scale is
    large): after the scale, -2^-149.  Other blocks random."""
    h = (B.bit_length() - 1) // 2
    x = _background(n, seed)
    b0 = (k // B) * B
    x[b0:b0 + B] = 0.0
    a = np.float32(2.0 ** -126)
    bsub = np.float32(2.0 ** -126 * (1 + 2.0 ** (h - 23)))
    if k % 2 == 0:      # x0 + x1 tiny, x2 + x3 = 0, x2 - x3 = 2
        x[b0:b0 + 4] = [a, -bsub, 1.0, -1.0]
    else:               # x0 - x1 tiny, x2 - x3 = 0, x2 + x3 = 2
        x[b0:b0 + 4] = [a, bsub, 1.0, 1.0]
    return x


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("B", [64, 128, 256])
def test_hadamard_zero_offset(zero_offset_indices, bits, B):
    hit = zero_offset_indices[0]
    off, k, n = _placed(hit, B)
    x = _hadamard_tiny_at(k, B, n, 5 + bits)
    t = O.hadamard_blocks(x, B)
    assert t[k] == np.float32(-2.0 ** -149)
    say(f"sr zero offset hadamard bits={bits} B={B} k={k}")
    c, s = L.hadamard_quantize_pack(f32_to_gpu(x), bits, B, True, SEED, off)
    torch.cuda.synchronize()
    wc, ws = O.hadamard_quantize_pack(x, bits, B, True, SEED, off)
    assert _code_at(wc, k, bits) == (1 << (bits - 1)) - 1
    assert_same(scales_np(s), ws, "scales")
    assert_same(codes_np(c), wc, "codes")


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("B", [32, 64, 128, 256, 1024])
def test_high_index_half_changes_inside_a_tile(bits, B):
    n = B * 40 + 5
    off = (1 << 32) - 3 * B
    x = _background(n, bits + B)
    e0 = np.random.default_rng(B).standard_normal(n).astype(np.float32) * np.float32(0.1)
    say(f"2^32 inside a tile bits={bits} B={B}")
    gx = f32_to_gpu(x)
    c, s = L.quantize_pack(gx, bits, B, True, SEED, off)
    gr = f32_to_gpu(e0)
    ce, se = L.ef_compress(gx, gr, bits, B, True, SEED, off)
    ch, sh = L.hadamard_quantize_pack(gx, bits, B, True, SEED, off)
    torch.cuda.synchronize()
    wc, ws = O.quantize_pack(x, bits, B, True, SEED, off)
    assert_same(scales_np(s), ws, "plain scales")
    assert_same(codes_np(c), wc, "plain codes")
    wce, wse, we = O.ef_compress(x, e0, bits, B, True, SEED, off)
    assert_same(scales_np(se), wse, "ef scales")
    assert_same(codes_np(ce), wce, "ef codes")
    assert_same(f32_np(gr), we, "ef residual")
    wch, wsh = O.hadamard_quantize_pack(x, bits, B, True, SEED, off)
    assert_same(scales_np(sh), wsh, "hadamard scales")
    assert_same(codes_np(ch), wch, "hadamard codes")
