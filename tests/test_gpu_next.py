"""GPU parity of the error-feedback variants and the mixed-width reduce,
through the C ABI, against the CPU oracle on the same seeded inputs:

* EF21 compress, chained over steps (state carried on the GPU and in the
  oracle independently);
* local reduce with stage-2 error feedback, chained over rounds;
* local reduce with fewer output bits than input bits (8 -> 4, 8 -> 2,
  4 -> 2) and different input/output block sizes, with and without the
  residual;
* compress and decompress with blockwise Hadamard smoothing (the GPU
  decompress is fed the GPU codes and checked against the oracle's
  decompress of the same codes).

Codes, scales, sums, residuals and states are compared bit for bit, at sizes
that span several tiles and a ragged tail (including a last output word whose
input words end early).
"""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import (assert_same, bf16_bits_of, codes_np, f32_np, mixed_input, say, scales_np,
                      to_gpu, f32_to_gpu)
from weight_communication_compression_amd import lowbit as L

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    L.lib()
    O.lib()
    yield
    torch.cuda.synchronize()


def _tile(bits, B):
    return max(64 * (32 // bits), B)


def _peers(P, n, bits, B, seed):
    pcs, pss, gc, gs = [], [], [], []
    for p in range(P):
        x = mixed_input(seed + p, n) if p % 2 else \
            (np.random.default_rng(seed + p).standard_normal(n) * 10.0 ** (p % 3 - 1)).astype(np.float32)
        c, s = O.quantize_pack(x, bits, B)
        pcs.append(c)
        pss.append(s)
        gc.append(torch.from_numpy(c.view(np.int32)).cuda())
        gs.append(torch.from_numpy(s.view(np.float16)).cuda())
    return pcs, pss, gc, gs


# ----------------------------------------------------------------- EF21 ----
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("sr", [False, True])
@pytest.mark.parametrize("B", [32, 128, 256, 2048])
@pytest.mark.parametrize("bits", [1, 2, 4, 8])
def test_ef21_compress_chained(bits, B, sr, dtype):
    n = 3 * _tile(bits, B) + B + 29
    rng = np.random.default_rng(bits * 7 + B)
    h_cpu = np.zeros(n, np.float32)
    h_gpu = torch.zeros(n, dtype=torch.float32, device="cuda")
    for step in range(3):
        g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
        gin = bf16_bits_of(g) if dtype == "bf16" else g
        say(f"ef21 bits={bits} B={B} sr={sr} {dtype} n={n} step={step}")
        c, s = L.ef21_compress(to_gpu(gin), h_gpu, bits, B, sr, 5 + step, B * 2)
        torch.cuda.synchronize()
        wc, ws, h_cpu = O.ef21_compress(gin, h_cpu, bits, B, sr, 5 + step, B * 2)
        assert_same(scales_np(s), ws, f"scales step {step}")
        assert_same(codes_np(c), wc, f"codes step {step}")
        assert_same(f32_np(h_gpu), h_cpu, f"state step {step}")


@pytest.mark.parametrize("n", [1, 5, 255, 257, 4096 + 3])
def test_ef21_small_and_ragged(n):
    g = mixed_input(77, n)
    h = mixed_input(78, n) * np.float32(1e-3)
    hg = f32_to_gpu(h)
    say(f"ef21 ragged n={n}")
    c, s = L.ef21_compress(f32_to_gpu(g), hg, 4, 128, True, 3, 0)
    torch.cuda.synchronize()
    wc, ws, wh = O.ef21_compress(g, h, 4, 128, True, 3, 0)
    assert_same(scales_np(s), ws, "scales")
    assert_same(codes_np(c), wc, "codes")
    assert_same(f32_np(hg), wh, "state")


# ----------------------------------------------------- stage-2 EF reduce ----
@pytest.mark.parametrize("want_sum", [False, True])
@pytest.mark.parametrize("P", [1, 3, 8, 16])
@pytest.mark.parametrize("sr", [False, True])
@pytest.mark.parametrize("B", [32, 128, 256, 4096])
@pytest.mark.parametrize("bits", [1, 2, 4, 8])
def test_reduce_stage2_ef_chained(bits, B, sr, P, want_sum):
    n = 2 * _tile(bits, B) + B + 45
    pcs, pss, gc, gs = _peers(P, n, bits, B, 500)
    e_cpu = (np.random.default_rng(bits + B).standard_normal(n) * 1e-2).astype(np.float32)
    e_gpu = f32_to_gpu(e_cpu)
    for rnd in range(2):
        say(f"reduce_ef bits={bits} B={B} sr={sr} P={P} sum={want_sum} n={n} round={rnd}")
        c, s, tot = L.reduce_requant_ef(gc, gs, n, bits, B, e_gpu, sr, 9 + rnd, B * 4,
                                        want_sum=want_sum, input_reused=rnd == 1)
        torch.cuda.synchronize()
        wc, ws, wt, e_cpu = O.reduce_requant_ex(pcs, pss, n, bits, B, bits, B, sr, 9 + rnd,
                                                B * 4, residual=e_cpu, want_sum=True)
        assert_same(scales_np(s), ws, f"scales round {rnd}")
        assert_same(codes_np(c), wc, f"codes round {rnd}")
        assert_same(f32_np(e_gpu), e_cpu, f"residual round {rnd}")
        if want_sum:
            assert_same(f32_np(tot), wt, f"sum round {rnd}")


# ------------------------------------------------ mixed widths / blocks ----
MIXED = [(8, 4), (8, 2), (4, 2)]
BLOCK_PAIRS = [(512, 128), (128, 128), (64, 256), (4096, 32), (32, 4096), (256, 64)]


@pytest.mark.parametrize("ef", [False, True])
@pytest.mark.parametrize("sr", [False, True])
@pytest.mark.parametrize("blocks", BLOCK_PAIRS)
@pytest.mark.parametrize("widths", MIXED)
def test_reduce_mixed(widths, blocks, sr, ef):
    bi, bo = widths
    Bi, Bo = blocks
    P = 5
    T = max(_tile(bo, Bo), Bi)
    for k, n in enumerate((3 * T + 37, 2 * T, 64 * (32 // bo) + 3)):
        pcs, pss, gc, gs = _peers(P, n, bi, Bi, 700 + bi + bo)
        e_cpu = (np.random.default_rng(n).standard_normal(n) * 1e-2).astype(np.float32) \
            if ef else None
        say(f"reduce mixed {bi}->{bo} B {Bi}->{Bo} sr={sr} ef={ef} n={n}")
        if ef:
            e_gpu = f32_to_gpu(e_cpu)
            c, s, tot = L.reduce_requant_ef(gc, gs, n, bi, Bi, e_gpu, sr, 4, 0, want_sum=True,
                                            out_bitwidth=bo, out_block_size=Bo,
                                            input_reused=k == 1)
        else:
            c, s, tot = L.reduce_requant(gc, gs, n, bi, Bi, sr, 4, 0, want_sum=True,
                                         out_bitwidth=bo, out_block_size=Bo, input_reused=k == 1)
        torch.cuda.synchronize()
        wc, ws, wt, we = O.reduce_requant_ex(pcs, pss, n, bi, Bi, bo, Bo, sr, 4, 0,
                                             residual=e_cpu, want_sum=True)
        assert_same(f32_np(tot), wt, f"sum n={n}")
        assert_same(scales_np(s), ws, f"scales n={n}")
        assert_same(codes_np(c), wc, f"codes n={n}")
        if ef:
            assert_same(f32_np(e_gpu), we, f"residual n={n}")


@pytest.mark.parametrize("widths", [(8, 8), (4, 4), (2, 2), (1, 1)])
def test_reduce_same_width_different_blocks(widths):
    b = widths[0]
    for Bi, Bo in [(512, 128), (64, 1024)]:
        n = 3 * max(_tile(b, Bo), Bi) + 11
        pcs, pss, gc, gs = _peers(4, n, b, Bi, 900)
        say(f"reduce same width b={b} B {Bi}->{Bo} n={n}")
        c, s, _ = L.reduce_requant(gc, gs, n, b, Bi, out_block_size=Bo)
        torch.cuda.synchronize()
        wc, ws, _, _ = O.reduce_requant_ex(pcs, pss, n, b, Bi, b, Bo)
        assert_same(scales_np(s), ws, "scales")
        assert_same(codes_np(c), wc, "codes")


def test_reduce_unsupported_pairs_raise():
    n = 1024
    pcs, pss, gc, gs = _peers(2, n, 4, 128, 1)
    for bo in (8, 1):
        with pytest.raises(L.LowbitError):
            L.reduce_requant(gc, gs, n, 4, 128, out_bitwidth=bo)


# ------------------------------------------------- Hadamard smoothing ----
HS_BLOCKS = [32, 64, 128, 256, 512, 1024, 2048, 4096]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("sr", [False, True])
@pytest.mark.parametrize("B", HS_BLOCKS)
@pytest.mark.parametrize("bits", [1, 2, 4, 8])
def test_hadamard_compress_decompress(bits, B, sr, dtype):
    T = _tile(bits, B)
    # whole blocks, and ragged ends: a partial last block is not transformed
    for i, n in enumerate(sorted({B, 3 * B, 4 * T + B, 9 * T, 5, B - 1, 3 * B + 1,
                                  4 * T + B + 37, 9 * T + B - 3})):
        x = mixed_input(3000 + bits * B + i, n) if i % 2 else \
            np.random.default_rng(i).standard_t(3, n).astype(np.float32)
        xin = bf16_bits_of(x) if dtype == "bf16" else x
        say(f"hadamard compress bits={bits} B={B} sr={sr} {dtype} n={n}")
        c, s = L.hadamard_quantize_pack(to_gpu(xin), bits, B, sr, 13, B * 2)
        torch.cuda.synchronize()
        wc, ws = O.hadamard_quantize_pack(xin, bits, B, sr, 13, B * 2)
        assert_same(scales_np(s), ws, f"scales n={n}")
        assert_same(codes_np(c), wc, f"codes n={n}")
        say(f"hadamard decompress bits={bits} B={B} n={n}")
        y = L.hadamard_unpack_dequant(c, s, n, bits, B)
        torch.cuda.synchronize()
        assert_same(f32_np(y), O.hadamard_unpack_dequant(wc, ws, n, bits, B), f"values n={n}")


@pytest.mark.parametrize("sr", [False, True])
@pytest.mark.parametrize("B", [32, 128, 4096])
@pytest.mark.parametrize("bits", [1, 2, 4, 8])
def test_hadamard_compress_input_reused_hint(bits, B, sr):
    """Streamed (default) and cached (LOWBIT_HINT_INPUT_REUSED) loads of the
    binary32 input give the same codes and scales."""
    T = _tile(bits, B)
    for i, n in enumerate([9 * T, 4 * T + B + 37]):
        x = np.random.default_rng(50 + i).standard_t(3, n).astype(np.float32)
        say(f"hadamard compress (input reused) bits={bits} B={B} sr={sr} n={n}")
        gx = to_gpu(x)
        c, s = L.hadamard_quantize_pack(gx, bits, B, sr, 21, 0, input_reused=True)
        c2, s2 = L.hadamard_quantize_pack(gx, bits, B, sr, 21, 0)
        torch.cuda.synchronize()
        wc, ws = O.hadamard_quantize_pack(x, bits, B, sr, 21, 0)
        for cc, ss in ((c, s), (c2, s2)):
            assert_same(scales_np(ss), ws, f"scales n={n}")
            assert_same(codes_np(cc), wc, f"codes n={n}")


def test_hadamard_size_rules_raise():
    x = torch.zeros(200, device="cuda")
    for B in (16, 96, 8192):
        with pytest.raises(L.LowbitError):
            L.hadamard_quantize_pack(x, 4, B)
    with pytest.raises(L.LowbitError):
        L.hadamard_quantize_pack(x, 3, 128)
