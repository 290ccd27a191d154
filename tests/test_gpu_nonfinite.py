"""Every entry point on inputs that hold infinities and NaNs, through the C ABI.

What such a call returns for the blocks that hold a non-finite value is left
unspecified by the interface; what is checked here is that each call
completes, and that every block with only finite inputs still matches the CPU
oracle bit for bit (blocks are independent, so a non-finite value must not
reach past its own block).
"""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import assert_same, codes_np, f32_np, f32_to_gpu, bf16_np, bf16_to_gpu, say, scales_np
from weight_communication_compression_amd import lowbit as L

pytestmark = pytest.mark.gpu

BITS = [1, 2, 4, 8]
B = 128
NB = 16
BAD = (1, 6)               # blocks that receive a non-finite value


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    L.lib()
    O.lib()
    yield
    torch.cuda.synchronize()


def _poison_f32(x):
    x = x.copy()
    x[BAD[0] * B + 5] = np.inf
    x[BAD[1] * B + 17] = np.nan
    x[BAD[1] * B + 18] = -np.inf
    return x


def _good_blocks(n):
    return [k for k in range(O.num_blocks(n, B)) if k not in BAD]


def _words(k, bits, n):
    per = 32 // bits
    return slice(k * B // per, min((k + 1) * B // per, O.num_words(n, bits)))


def _elems(k, n):
    return slice(k * B, min((k + 1) * B, n))


def _compare_blocks(n, bits, c, s, wc, ws, what):
    for k in _good_blocks(n):
        assert_same(c[_words(k, bits, n)], wc[_words(k, bits, n)], f"{what} codes block {k}")
        assert s[k] == ws[k], f"{what} scale block {k}: {s[k]:#06x} != {ws[k]:#06x}"


def _compare_elems(n, got, want, what):
    for k in _good_blocks(n):
        assert_same(got[_elems(k, n)], want[_elems(k, n)], f"{what} block {k}")


@pytest.mark.parametrize("bits", BITS)
def test_ef_compress_nonfinite(bits):
    n = NB * B + 37
    rng = np.random.default_rng(bits)
    g = _poison_f32(rng.standard_normal(n).astype(np.float32))
    e = (rng.standard_normal(n) * 1e-2).astype(np.float32)
    e[BAD[1] * B + 40] = np.inf                           # a residual that went bad too
    eg = f32_to_gpu(e)
    say(f"nonfinite ef_compress bits={bits} n={n}")
    c, s = L.ef_compress(f32_to_gpu(g), eg, bits, B, True, 3, 0)
    torch.cuda.synchronize()
    wc, ws, we = O.ef_compress(g, e, bits, B, True, 3, 0)
    _compare_blocks(n, bits, codes_np(c), scales_np(s), wc, ws, "ef")
    _compare_elems(n, f32_np(eg), we, "ef residual")


@pytest.mark.parametrize("bits", BITS)
def test_ef21_compress_nonfinite(bits):
    n = NB * B + 37
    rng = np.random.default_rng(10 + bits)
    g = _poison_f32(rng.standard_normal(n).astype(np.float32))
    h = (rng.standard_normal(n) * 1e-2).astype(np.float32)
    hg = f32_to_gpu(h)
    say(f"nonfinite ef21_compress bits={bits} n={n}")
    c, s = L.ef21_compress(f32_to_gpu(g), hg, bits, B, True, 4, 0)
    torch.cuda.synchronize()
    wc, ws, wh = O.ef21_compress(g, h, bits, B, True, 4, 0)
    _compare_blocks(n, bits, codes_np(c), scales_np(s), wc, ws, "ef21")
    _compare_elems(n, f32_np(hg), wh, "ef21 state")


@pytest.mark.parametrize("bits", BITS)
def test_hadamard_nonfinite(bits):
    n = NB * B
    x = _poison_f32(np.random.default_rng(20 + bits).standard_t(3, n).astype(np.float32))
    say(f"nonfinite hadamard compress bits={bits} n={n}")
    c, s = L.hadamard_quantize_pack(f32_to_gpu(x), bits, B, True, 5, 0)
    torch.cuda.synchronize()
    wc, ws = O.hadamard_quantize_pack(x, bits, B, True, 5, 0)
    _compare_blocks(n, bits, codes_np(c), scales_np(s), wc, ws, "hadamard")
    say(f"nonfinite hadamard decompress bits={bits} n={n}")
    y = L.hadamard_unpack_dequant(c, s, n, bits, B)
    torch.cuda.synchronize()
    _compare_elems(n, f32_np(y), O.hadamard_unpack_dequant(codes_np(c), scales_np(s), n, bits, B),
                   "hadamard values")


@pytest.mark.parametrize("bits", BITS)
def test_wdiff_nonfinite(bits):
    n = NB * B + 37
    rng = np.random.default_rng(30 + bits)
    w_old = O.f32_to_bf16_rne((rng.standard_normal(n) * 0.02).astype(np.float32))
    w_new = O.f32_to_bf16_rne(O.bf16_to_f32(w_old) + (rng.standard_normal(n) * 1e-3).astype(np.float32))
    w_new[BAD[0] * B + 5] = 0x7F80                         # +inf
    w_new[BAD[1] * B + 17] = 0x7FC0                        # NaN
    w_new[BAD[1] * B + 18] = 0xFF80                        # -inf
    say(f"nonfinite wdiff compress bits={bits} n={n}")
    c, s = L.wdiff_compress(bf16_to_gpu(w_new), bf16_to_gpu(w_old), bits, B)
    torch.cuda.synchronize()
    wc, ws = O.wdiff_compress(w_new, w_old, bits, B)
    _compare_blocks(n, bits, codes_np(c), scales_np(s), wc, ws, "wdiff")
    say(f"nonfinite wdiff apply bits={bits} n={n}")
    out = L.wdiff_apply(bf16_to_gpu(w_old), c, s, bits, B)
    torch.cuda.synchronize()
    _compare_elems(n, bf16_np(out), O.wdiff_apply(w_old, codes_np(c), scales_np(s), bits, B),
                   "wdiff apply")


@pytest.mark.parametrize("bits", BITS)
def test_nonfinite_scales_decompress_and_reduce(bits):
    """Peer scales of +inf and NaN (a corrupted message) in two blocks."""
    n = NB * B + 37
    P = 8
    pcs, pss = [], []
    for p in range(P):
        x = (np.random.default_rng(40 + p).standard_normal(n) * 10.0 ** (p % 3 - 1)).astype(np.float32)
        c, s = O.quantize_pack(x, bits, B)
        pcs.append(c)
        pss.append(s.copy())
    pss[2][BAD[0]] = 0x7C00                                # +inf
    pss[5][BAD[1]] = 0x7E00                                # NaN
    gc = [torch.from_numpy(c.view(np.int32)).cuda() for c in pcs]
    gs = [torch.from_numpy(s.view(np.float16)).cuda() for s in pss]
    say(f"nonfinite scales decompress bits={bits} n={n}")
    y = L.unpack_dequant(gc[2], gs[2], n, bits, B)
    torch.cuda.synchronize()
    _compare_elems(n, f32_np(y), O.unpack_dequant(pcs[2], pss[2], n, bits, B), "decompress")
    say(f"nonfinite scales reduce bits={bits} n={n}")
    c, s, tot = L.reduce_requant(gc, gs, n, bits, B, want_sum=True)
    torch.cuda.synchronize()
    wc, ws, wt, _ = O.reduce_requant_ex(pcs, pss, n, bits, B, bits, B, want_sum=True)
    _compare_blocks(n, bits, codes_np(c), scales_np(s), wc, ws, "reduce")
    _compare_elems(n, f32_np(tot), wt, "reduce sum")
    e = (np.random.default_rng(bits).standard_normal(n) * 1e-2).astype(np.float32)
    eg = f32_to_gpu(e)
    say(f"nonfinite scales reduce_ef bits={bits} n={n}")
    c, s, _ = L.reduce_requant_ef(gc, gs, n, bits, B, eg, bits > 1, 6, 0)
    torch.cuda.synchronize()
    wc, ws, _, we = O.reduce_requant_ex(pcs, pss, n, bits, B, bits, B, bits > 1, 6, 0, residual=e)
    _compare_blocks(n, bits, codes_np(c), scales_np(s), wc, ws, "reduce_ef")
    _compare_elems(n, f32_np(eg), we, "reduce_ef residual")
