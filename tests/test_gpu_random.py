"""GPU parity on seeded random cases: each case draws a length (1 .. 2^18,
often ragged), a bitwidth, a block size, rounding, input type, seed and
global index offset, and runs one entry point of the C ABI against the
oracle on the same inputs, bit for bit.  The cases are fixed by their seeds,
so a failure names a reproducible case."""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import (assert_same, bf16_bits_of, bf16_np, codes_np, f32_np, f32_to_gpu,
                      mixed_input, say, scales_np, to_gpu)
from weight_communication_compression_amd import lowbit as L

pytestmark = pytest.mark.gpu

BITS = [1, 2, 4, 8]
BLOCKS = [32, 64, 128, 256, 512, 1024, 2048, 4096]
CASES = 24


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    L.lib()
    O.lib()
    yield
    torch.cuda.synchronize()


def _case(seed):
    g = np.random.default_rng(seed)
    n = int(g.integers(1, 1 << 18)) if g.random() < 0.8 else int(g.integers(1, 600))
    b = int(g.choice(BITS))
    B = int(g.choice(BLOCKS))
    sr = bool(g.random() < 0.5)
    dtype = "bf16" if g.random() < 0.3 else "f32"
    rseed = int(g.integers(0, 2 ** 63))
    off = B * int(g.integers(0, 1 << 40))
    x = mixed_input(seed, n) if g.random() < 0.5 else (g.standard_normal(n) * 1e-3).astype(np.float32)
    if dtype == "bf16":
        x = bf16_bits_of(x)
    return g, n, b, B, sr, dtype, rseed, off, x


@pytest.mark.parametrize("seed", range(CASES))
def test_random_compress_decompress(seed):
    _, n, b, B, sr, dtype, rseed, off, x = _case(1000 + seed)
    say(f"random compress seed={seed} n={n} b={b} B={B} sr={sr} {dtype} off={off}")
    c, s = L.quantize_pack(to_gpu(x), b, B, sr, rseed, off)
    y = L.unpack_dequant(c, s, n, b, B)
    torch.cuda.synchronize()
    wc, ws = O.quantize_pack(x, b, B, sr, rseed, off)
    assert_same(scales_np(s), ws, "scales")
    assert_same(codes_np(c), wc, "codes")
    assert_same(f32_np(y), O.unpack_dequant(wc, ws, n, b, B), "decompress")


@pytest.mark.parametrize("seed", range(CASES))
def test_random_error_feedback_and_ef21(seed):
    g, n, b, B, sr, dtype, rseed, off, x = _case(2000 + seed)
    e = (g.standard_normal(n) * 1e-4).astype(np.float32)
    say(f"random ef/ef21 seed={seed} n={n} b={b} B={B} sr={sr} {dtype}")
    ge, gh = f32_to_gpu(e), f32_to_gpu(e)
    c, s = L.ef_compress(to_gpu(x), ge, b, B, sr, rseed, off)
    c2, s2 = L.ef21_compress(to_gpu(x), gh, b, B, sr, rseed, off)
    torch.cuda.synchronize()
    wc, ws, we = O.ef_compress(x, e, b, B, sr, rseed, off)
    assert_same(codes_np(c), wc, "ef codes")
    assert_same(scales_np(s), ws, "ef scales")
    assert_same(f32_np(ge), we, "ef residual")
    wc, ws, wh = O.ef21_compress(x, e, b, B, sr, rseed, off)
    assert_same(codes_np(c2), wc, "ef21 codes")
    assert_same(scales_np(s2), ws, "ef21 scales")
    assert_same(f32_np(gh), wh, "ef21 state")


@pytest.mark.parametrize("seed", range(CASES))
def test_random_local_reduce(seed):
    g, n, b, B, sr, _, rseed, off, _ = _case(3000 + seed)
    P = int(g.integers(1, 17))
    bo = int(g.choice([w for w in BITS if w <= b and (w == b or b in (4, 8) and w in (2, 4))]))
    Bo = int(g.choice(BLOCKS))
    off = Bo * int(g.integers(0, 1 << 40))           # a multiple of the output block
    want_sum = bool(g.random() < 0.5)
    ef = bool(g.random() < 0.5)
    peers = [O.quantize_pack(mixed_input(seed * 31 + p, n), b, B) for p in range(P)]
    say(f"random reduce seed={seed} n={n} P={P} b={b}->{bo} B={B}->{Bo} sr={sr} ef={ef} "
        f"sum={want_sum}")
    gc = [torch.from_numpy(c.view(np.int32)).cuda() for c, _ in peers]
    gs = [torch.from_numpy(s.view(np.float16)).cuda() for _, s in peers]
    r = (g.standard_normal(n) * 1e-2).astype(np.float32)
    if ef:
        gr = f32_to_gpu(r)
        c, s, t = L.reduce_requant_ef(gc, gs, n, b, B, gr, sr, rseed, off, want_sum=want_sum,
                                      out_bitwidth=bo, out_block_size=Bo)
    else:
        c, s, t = L.reduce_requant(gc, gs, n, b, B, sr, rseed, off, want_sum=want_sum,
                                   out_bitwidth=bo, out_block_size=Bo)
    torch.cuda.synchronize()
    wc, ws, wt, we = O.reduce_requant_ex([c for c, _ in peers], [s for _, s in peers], n, b, B,
                                         bo, Bo, sr, rseed, off, residual=r if ef else None,
                                         want_sum=want_sum)
    assert_same(codes_np(c), wc, "codes")
    assert_same(scales_np(s), ws, "scales")
    if want_sum:
        assert_same(f32_np(t), wt, "sum")
    if ef:
        assert_same(f32_np(gr), we, "residual")


@pytest.mark.parametrize("seed", range(CASES))
def test_random_weight_difference_and_hadamard(seed):
    g, n, b, B, sr, dtype, rseed, off, x = _case(4000 + seed)
    w_old = (g.standard_normal(n) * 0.02).astype(np.float32)
    w_new = (w_old + g.standard_normal(n) * 1e-4).astype(np.float32)
    if dtype == "bf16":
        w_old, w_new = bf16_bits_of(w_old), bf16_bits_of(w_new)
    say(f"random wdiff/hadamard seed={seed} n={n} b={b} B={B} sr={sr} {dtype}")
    go = to_gpu(w_old)
    c, s = L.wdiff_compress(to_gpu(w_new), go, b, B, sr, rseed, off)
    out = L.wdiff_apply(go, c, s, b, B)
    hc, hs = L.hadamard_quantize_pack(to_gpu(x), b, B, sr, rseed, off)
    hy = L.hadamard_unpack_dequant(hc, hs, n, b, B)
    torch.cuda.synchronize()
    wc, ws = O.wdiff_compress(w_new, w_old, b, B, sr, rseed, off)
    assert_same(codes_np(c), wc, "wdiff codes")
    assert_same(scales_np(s), ws, "wdiff scales")
    want = O.wdiff_apply(w_old, wc, ws, b, B)
    assert_same(bf16_np(out) if dtype == "bf16" else f32_np(out), want, "apply")
    wc, ws = O.hadamard_quantize_pack(x, b, B, sr, rseed, off)
    assert_same(codes_np(hc), wc, "hadamard codes")
    assert_same(scales_np(hs), ws, "hadamard scales")
    assert_same(f32_np(hy), O.hadamard_unpack_dequant(wc, ws, n, b, B), "hadamard values")
