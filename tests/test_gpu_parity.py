"""GPU parity: every entry point of liblowbit (called through the C ABI via the
ctypes binding) against the CPU oracle on the same seeded inputs, at sizes
that span several tiles and a ragged tail.  Codes, scales and every float
output are compared bit for bit (the float bar, 1e-6 x block scale, is
checked as well and reported separately).
"""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import (assert_close_scaled, assert_same, bf16_bits_of, bf16_np, codes_np,
                      f32_np, f32_to_gpu, mixed_input, say, scale_per_element, scales_np,
                      to_gpu)
from weight_communication_compression_amd import lowbit as L

pytestmark = pytest.mark.gpu

BITS = [1, 2, 4, 8]
BLOCKS = [32, 64, 128, 256, 512, 1024, 2048, 4096]


def _tile(bits, B):
    row = 64 * (32 // bits)
    return max(row, B)


def _sizes(bits, B):
    T = _tile(bits, B)
    return sorted({1, 7, 33, B - 1, B + 1, 3 * T + 77, 5 * T, 10 * B + 13})


def _input(kind, n, seed, dtype):
    x = mixed_input(seed, n) if kind == "mixed" else \
        np.random.default_rng(seed).standard_normal(n).astype(np.float32)
    return bf16_bits_of(x) if dtype == "bf16" else x


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    L.lib()
    O.lib()
    yield
    torch.cuda.synchronize()


# -------------------------------------------------------------- compress --
@pytest.mark.parametrize("sr", [False, True])
@pytest.mark.parametrize("B", [32, 256, 4096])
@pytest.mark.parametrize("bits", BITS)
def test_quantize_input_reused_hint(bits, B, sr):
    """LOWBIT_HINT_INPUT_REUSED selects cached rather than streamed loads of
    the binary32 input of every plain compress; the codes and scales
    are the same."""
    for i, n in enumerate(_sizes(bits, B)):
        x = _input("mixed", n, 7000 * bits + B + i, "f32")
        say(f"quantize (input reused) bits={bits} B={B} sr={sr} n={n}")
        gx = to_gpu(x)
        c, s = L.quantize_pack(gx, bits, B, sr, 5, B * i, input_reused=True)
        c2, s2 = L.quantize_pack(gx, bits, B, sr, 5, B * i, input_reused=False)
        torch.cuda.synchronize()
        wc, ws = O.quantize_pack(x, bits, B, sr, 5, B * i)
        assert_same(scales_np(s), ws, f"scales n={n}")
        assert_same(codes_np(c), wc, f"codes n={n}")
        assert_same(scales_np(s2), ws, f"scales n={n}")
        assert_same(codes_np(c2), wc, f"codes n={n}")



@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("sr", [False, True])
@pytest.mark.parametrize("B", BLOCKS)
@pytest.mark.parametrize("bits", BITS)
def test_quantize_and_dequant(bits, B, sr, dtype):
    for i, n in enumerate(_sizes(bits, B)):
        x = _input("mixed", n, 1000 * bits + B + i, dtype)
        seed, off = 42 + i, B * (3 + i)
        say(f"quantize bits={bits} B={B} sr={sr} {dtype} n={n}")
        c, s = L.quantize_pack(to_gpu(x), bits, B, sr, seed, off)
        torch.cuda.synchronize()
        wc, ws = O.quantize_pack(x, bits, B, sr, seed, off)
        assert_same(scales_np(s), ws, f"scales n={n}")
        assert_same(codes_np(c), wc, f"codes n={n}")
        say(f"dequant bits={bits} B={B} n={n}")
        y = L.unpack_dequant(c, s, n, bits, B)
        torch.cuda.synchronize()
        wy = O.unpack_dequant(wc, ws, n, bits, B)
        assert_close_scaled(f32_np(y), wy, scale_per_element(ws, n, B), f"deq n={n}")
        assert_same(f32_np(y), wy, f"deq n={n}")


@pytest.mark.parametrize("bits", BITS)
def test_dequant_arbitrary_codes(bits):
    """Decompress of arbitrary words and scales (not produced by compress)."""
    B, n = 128, 128 * 37 + 5
    g = np.random.default_rng(bits)
    words = g.integers(0, 1 << 32, size=O.num_words(n, bits), dtype=np.uint64).astype(np.uint32)
    sc = np.exp(g.uniform(-12, 4, size=O.num_blocks(n, B))).astype(np.float16).view(np.uint16)
    sc[3] = 0
    say(f"dequant arbitrary bits={bits}")
    y = L.unpack_dequant(torch.from_numpy(words.view(np.int32)).cuda(),
                         torch.from_numpy(sc.view(np.float16)).cuda(), n, bits, B)
    torch.cuda.synchronize()
    assert_same(f32_np(y), O.unpack_dequant(words, sc, n, bits, B), "deq")


# ---------------------------------------------------------- error feedback --
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("sr", [False, True])
@pytest.mark.parametrize("B", [32, 128, 256, 1024, 4096])
@pytest.mark.parametrize("bits", BITS)
def test_ef_compress_chained(bits, B, sr, dtype):
    n = 5 * _tile(bits, B) + 3 * B + 29
    e_gpu = torch.zeros(n, dtype=torch.float32, device="cuda")
    e_ref = np.zeros(n, np.float32)
    for step in range(3):
        g = _input("mixed", n, 77 + step + bits, dtype)
        say(f"ef bits={bits} B={B} sr={sr} {dtype} n={n} step={step}")
        c, s = L.ef_compress(to_gpu(g), e_gpu, bits, B, sr, 2 + step, 0)
        torch.cuda.synchronize()
        wc, ws, e_ref = O.ef_compress(g, e_ref, bits, B, sr, 2 + step, 0)
        assert_same(scales_np(s), ws, f"scales step {step}")
        assert_same(codes_np(c), wc, f"codes step {step}")
        assert_close_scaled(f32_np(e_gpu), e_ref, scale_per_element(ws, n, B), "residual")
        assert_same(f32_np(e_gpu), e_ref, f"residual step {step}")


# ------------------------------------------------------------------ reduce --
@pytest.mark.parametrize("want_sum", [False, True])
@pytest.mark.parametrize("P", [1, 2, 3, 8, 16])
@pytest.mark.parametrize("sr", [False, True])
@pytest.mark.parametrize("B", [32, 128, 256, 2048])
@pytest.mark.parametrize("bits", BITS)
def test_reduce_requant(bits, B, sr, P, want_sum):
    n = 3 * _tile(bits, B) + B + 45
    pcs, pss, gc, gs = [], [], [], []
    for p in range(P):
        x = mixed_input(300 + p, n) if p % 2 else \
            np.random.default_rng(300 + p).standard_normal(n).astype(np.float32)
        c, s = O.quantize_pack(x, bits, B)
        pcs.append(c)
        pss.append(s)
        gc.append(torch.from_numpy(c.view(np.int32)).cuda())
        gs.append(torch.from_numpy(s.view(np.float16)).cuda())
    reused = P % 2 == 1      # LOWBIT_HINT_INPUT_REUSED: cached rather than streamed code loads
    say(f"reduce bits={bits} B={B} sr={sr} P={P} sum={want_sum} reused={reused} n={n}")
    c, s, tot = L.reduce_requant(gc, gs, n, bits, B, sr, 9, B * 5, want_sum=want_sum,
                                 input_reused=reused)
    torch.cuda.synchronize()
    wc, ws, wt = O.reduce_requant(pcs, pss, n, bits, B, bits, sr, 9, B * 5, want_sum=True)
    assert_same(scales_np(s), ws, "scales")
    assert_same(codes_np(c), wc, "codes")
    if want_sum:
        assert_same(f32_np(tot), wt, "sum")


def _controlled_peer(kind, bits, B, n, p, seed):
    """One peer's binary32 input whose blocks have an exactly chosen max |x|
    of 2^e (so the block scales' binary16 exponents differ across peers by
    the spread of e): 'limit' spreads e over 2^D (the widest the integer path
    of the 8-peer reduce takes: D = 5 at 4 bits, 3 at 8 bits), 'over' one
    step wider in one block in 40 (some waves take the integer path, others
    the binary32 one), 'subnormal' and 'mixed' reach binary16-
    subnormal scales, 'zeros' zeroes whole blocks of some peers (and some
    blocks of all peers)."""
    g = np.random.default_rng(seed)
    nb = -(-n // B)
    D = 5 if bits == 4 else 3
    e = {"normal": np.zeros(nb, np.int64),
         "limit": g.integers(0, D + 1, nb),
         "over": g.integers(0, D + 1, nb),
         "subnormal": g.integers(-24, -19, nb),
         "mixed": g.integers(-15, -15 + D + 1, nb),
         "zeros": g.integers(0, D + 1, nb)}[kind]
    bg = np.random.default_rng(seed // 100)          # the same for every peer
    if kind == "limit":
        e[::7] = D if p % 2 else 0                    # some blocks exactly at the limit
    if kind == "over":
        e[::40] = D + 1 if p == 3 else 0              # some blocks one past it
    x = g.uniform(-1.0, 1.0, n) * np.repeat(2.0 ** e, B)[:n]
    starts = np.arange(0, n, B)
    x[starts] = 2.0 ** e * np.where(g.random(nb) < 0.5, 1.0, -1.0)
    if kind == "zeros":
        zb = g.random(nb) < 0.3
        zb[bg.random(nb) < 0.2] = True                # zero in every peer
        for b in np.nonzero(zb)[0]:
            x[b * B:(b + 1) * B] = 0.0
    return x.astype(np.float32)


@pytest.mark.parametrize("kind", ["normal", "limit", "over", "subnormal", "mixed", "zeros"])
@pytest.mark.parametrize("sr", [False, True])
@pytest.mark.parametrize("B", [32, 64, 128, 256, 1024, 4096])
@pytest.mark.parametrize("bits", [4, 8])
def test_reduce_eight_peers_exact_sums(bits, B, sr, kind):
    """Eight peers (one per GPU of a node) whose block scales lie within or
    just outside the range in which the reduce forms the peer-ordered sums in
    integers: bit-identical to the oracle's binary32 sums either way, with and
    without the sum output, over several waves and a ragged tail."""
    n = 9 * _tile(bits, B) + B + 45
    pcs, pss, gc, gs = [], [], [], []
    for p in range(8):
        x = _controlled_peer(kind, bits, B, n, p, 100 * (bits * B) + p)
        c, s = O.quantize_pack(x, bits, B)
        pcs.append(c)
        pss.append(s)
        gc.append(torch.from_numpy(c.view(np.int32)).cuda())
        gs.append(torch.from_numpy(s.view(np.float16)).cuda())
    say(f"reduce 8 peers bits={bits} B={B} sr={sr} kind={kind} n={n}")
    wc, ws, wt = O.reduce_requant(pcs, pss, n, bits, B, bits, sr, 3, 0, want_sum=True)
    for want_sum, reused in ((False, False), (True, False), (False, True)):
        c, s, tot = L.reduce_requant(gc, gs, n, bits, B, sr, 3, 0, want_sum=want_sum,
                                     input_reused=reused)
        torch.cuda.synchronize()
        assert_same(scales_np(s), ws, "scales")
        assert_same(codes_np(c), wc, "codes")
        if want_sum:
            assert_same(f32_np(tot), wt, "sum")


# -------------------------------------------------------- weight difference --
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B", [32, 64, 128, 2048])
@pytest.mark.parametrize("bits", BITS)
def test_wdiff_compress_apply(bits, B, dtype):
    n = 4 * _tile(bits, B) + 2 * B + 11
    g = np.random.default_rng(bits * B)
    w_old = (g.standard_normal(n) * 0.02).astype(np.float32)
    w_new = (w_old + g.standard_normal(n) * 1e-4).astype(np.float32)
    if dtype == "bf16":
        w_old, w_new = bf16_bits_of(w_old), bf16_bits_of(w_new)
    say(f"wdiff bits={bits} B={B} {dtype} n={n}")
    go, gn = to_gpu(w_old), to_gpu(w_new)
    c, s = L.wdiff_compress(gn, go, bits, B)
    torch.cuda.synchronize()
    wc, ws = O.wdiff_compress(w_new, w_old, bits, B)
    assert_same(scales_np(s), ws, "scales")
    assert_same(codes_np(c), wc, "codes")
    say(f"wdiff apply bits={bits} B={B} {dtype} n={n}")
    out = L.wdiff_apply(go, c, s, bits, B)
    torch.cuda.synchronize()
    want = O.wdiff_apply(w_old, wc, ws, bits, B)
    got = bf16_np(out) if dtype == "bf16" else f32_np(out)
    assert_same(got, want, "apply")
    # in place: w_out is w_old
    say(f"wdiff apply in place bits={bits} B={B} {dtype}")
    L.wdiff_apply(go, c, s, bits, B, out=go)
    torch.cuda.synchronize()
    got = bf16_np(go) if dtype == "bf16" else f32_np(go)
    assert_same(got, want, "apply in place")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("rem", range(8))
def test_wdiff_apply_tail_lanes(rem, dtype):
    """8-bit apply: a lane covers 8 elements in two code words; with n % 8 in
    1..4 the tail lane's second word lies past the last code word and is not
    read."""
    bits, B = 8, 32
    n = 512 * 3 + 8 * 5 + rem
    g = np.random.default_rng(rem)
    w_old = (g.standard_normal(n) * 0.02).astype(np.float32)
    w_new = (w_old + g.standard_normal(n) * 1e-3).astype(np.float32)
    if dtype == "bf16":
        w_old, w_new = bf16_bits_of(w_old), bf16_bits_of(w_new)
    wc, ws = O.wdiff_compress(w_new, w_old, bits, B)
    c = torch.from_numpy(wc.view(np.int32)).cuda()
    s = torch.from_numpy(ws.view(np.float16)).cuda()
    say(f"wdiff apply tail bits={bits} {dtype} n={n}")
    out = L.wdiff_apply(to_gpu(w_old), c, s, bits, B)
    torch.cuda.synchronize()
    got = bf16_np(out) if dtype == "bf16" else f32_np(out)
    assert_same(got, O.wdiff_apply(w_old, wc, ws, bits, B), "apply")


# ------------------------------------------------------------- edge cases --
def test_zero_length_calls_launch_nothing():
    x = torch.empty(0, device="cuda")
    c, s = L.quantize_pack(x, 4, 128)
    assert c.numel() == 0 and s.numel() == 0
    y = L.unpack_dequant(c, s, 0, 4, 128)
    assert y.numel() == 0


@pytest.mark.parametrize("bits", BITS)
def test_special_blocks(bits):
    """All-zero blocks, negative zeros, exact-grid blocks, saturating scales,
    binary16-subnormal scales and binary32 subnormal inputs."""
    B = 64
    blocks = [np.zeros(B), -np.zeros(B), np.full(B, 1e30), np.full(B, -3e9),
              np.linspace(-7, 7, B) * 2.0 ** -20, np.full(B, 1e-40),
              np.r_[1e-45, np.zeros(B - 1)], np.linspace(-1, 1, B)]
    x = np.concatenate(blocks).astype(np.float32)
    for sr in (False, True):
        say(f"special bits={bits} sr={sr}")
        c, s = L.quantize_pack(to_gpu(x), bits, B, sr, 5, 0)
        torch.cuda.synchronize()
        wc, ws = O.quantize_pack(x, bits, B, sr, 5, 0)
        assert_same(scales_np(s), ws, "scales")
        assert_same(codes_np(c), wc, "codes")


@pytest.mark.parametrize("bits", BITS)
def test_nonfinite_inputs_terminate(bits):
    """inf and NaN inputs give some in-range codes; the call completes and the
    finite blocks are unaffected."""
    B, n = 128, 128 * 16
    x = np.random.default_rng(1).standard_normal(n).astype(np.float32)
    x[5] = np.inf
    x[200] = -np.inf
    x[300] = np.nan
    say(f"nonfinite bits={bits}")
    c, s = L.quantize_pack(to_gpu(x), bits, B, True, 1, 0)
    torch.cuda.synchronize()
    wc, ws = O.quantize_pack(x, bits, B, True, 1, 0)
    finite_blocks = [k for k in range(n // B) if np.all(np.isfinite(x[k * B:(k + 1) * B]))]
    per = 32 // bits
    for k in finite_blocks:
        a, b = k * B // per, (k + 1) * B // per
        assert_same(codes_np(c)[a:b], wc[a:b], f"block {k}")
        assert scales_np(s)[k] == ws[k]


@pytest.mark.parametrize("bits", BITS)
def test_index_offset_above_2_32(bits):
    B, n = 256, 256 * 40 + 7
    x = mixed_input(8, n)
    off = (1 << 32) - 256 * 20      # the buffer crosses global index 2^32
    say(f"offset>2^32 bits={bits}")
    c, s = L.quantize_pack(to_gpu(x), bits, B, True, 123456789012345, off)
    torch.cuda.synchronize()
    wc, ws = O.quantize_pack(x, bits, B, True, 123456789012345, off)
    assert_same(scales_np(s), ws, "scales")
    assert_same(codes_np(c), wc, "codes")


@pytest.mark.parametrize("bits", BITS)
def test_sharding_and_determinism_on_gpu(bits):
    """Chunked calls with index_offset give the bytes of one call, and two runs
    give identical bytes."""
    B = 256
    n = 64 * 2048 * 3 + 1234
    x = mixed_input(4, n)
    gx = to_gpu(x)
    say(f"sharding bits={bits}")
    c_all, s_all = L.quantize_pack(gx, bits, B, True, 42, 0)
    c2, s2 = L.quantize_pack(gx, bits, B, True, 42, 0)
    cuts = [0, 5 * B, 6 * B, 200 * B, n]
    cs, ss = [], []
    for a, b in zip(cuts[:-1], cuts[1:]):
        c, s = L.quantize_pack(gx[a:b], bits, B, True, 42, a)
        cs.append(c)
        ss.append(s)
    torch.cuda.synchronize()
    assert torch.equal(c_all, c2) and torch.equal(s_all, s2)
    assert torch.equal(torch.cat(ss), s_all)
    assert torch.equal(torch.cat(cs), c_all)


def test_runs_on_the_callers_stream():
    n, B = 1 << 16, 128
    x = mixed_input(2, n)
    side = torch.cuda.Stream()
    say("side stream")
    with torch.cuda.stream(side):
        gx = to_gpu(x)
        c, s = L.quantize_pack(gx, 4, B, True, 3, 0)
        y = L.unpack_dequant(c, s, n, 4, B)
    side.synchronize()
    wc, ws = O.quantize_pack(x, 4, B, True, 3, 0)
    assert_same(codes_np(c), wc, "codes")
    assert_same(f32_np(y), O.unpack_dequant(wc, ws, n, 4, B), "deq")


def test_copy_kernel():
    for n in [1, 3, 4, 1000, (1 << 20) + 3]:
        x = torch.randn(n, device="cuda")
        y = torch.empty_like(x)
        say(f"copy n={n}")
        L.copy_f32(x, y)
        torch.cuda.synchronize()
        assert torch.equal(x, y)


def test_xor_streams_reference_kernel():
    """The reduce-pattern bandwidth reference: out = XOR of the streams, for
    stream counts across the group of eight and sizes with a ragged wave."""
    for P, n in [(1, 1), (3, 127), (8, 128 * 1000), (9, 128 * 3 + 77), (16, (1 << 20) + 5)]:
        rng = np.random.default_rng(P * 1000 + n)
        hs = [rng.integers(0, 2 ** 32, n, dtype=np.uint32) for _ in range(P)]
        gs = [torch.from_numpy(h.view(np.int32)).cuda() for h in hs]
        out = torch.empty(n, dtype=torch.int32, device="cuda")
        say(f"xor_streams P={P} n={n}")
        L.xor_streams(gs, out)
        torch.cuda.synchronize()
        want = np.bitwise_xor.reduce(np.stack(hs), axis=0)
        assert_same(codes_np(out), want, f"xor P={P} n={n}")


def test_add_inplace_reference_kernel():
    """The EF-pattern bandwidth reference: y += x in binary32, in place, at
    sizes with a ragged last wave."""
    for n in [1, 7, 512, 512 * 3 + 100, (1 << 20) + 13]:
        rng = np.random.default_rng(n)
        xh = rng.standard_normal(n).astype(np.float32)
        yh = rng.standard_normal(n).astype(np.float32)
        x, y = f32_to_gpu(xh), f32_to_gpu(yh)
        say(f"add_inplace n={n}")
        L.add_inplace_f32(x, y)
        torch.cuda.synchronize()
        assert_same(f32_np(y), yh + xh, f"add n={n}")


@pytest.mark.parametrize("nt", [True, False])
@pytest.mark.parametrize("waves", [0, 8, 1000])
def test_stream_probe_kernel(waves, nt):
    """The memory-system probe: read (XOR of each 1024-word trip), write
    (i ^ value) and copy, one trip per wave and persistent grids of fewer and
    more waves than trips, streaming and plain stores."""
    for ntrips in [1, 37, 1025]:
        n = ntrips * 1024
        h = np.random.default_rng(ntrips + waves).integers(0, 2 ** 32, n, dtype=np.uint32)
        src = torch.from_numpy(h.view(np.int32)).cuda()
        rd = torch.full((ntrips,), -1, dtype=torch.int32, device="cuda")
        wr = torch.full((n,), -1, dtype=torch.int32, device="cuda")
        cp = torch.full((n,), -1, dtype=torch.int32, device="cuda")
        say(f"stream probe ntrips={ntrips} waves={waves} nt={nt}")
        L.stream_probe(L.PROBE_READ, rd, src, waves=waves, nontemporal=nt)
        L.stream_probe(L.PROBE_WRITE, wr, value=0x12345678, waves=waves, nontemporal=nt)
        L.stream_probe(L.PROBE_COPY, cp, src, waves=waves, nontemporal=nt)
        torch.cuda.synchronize()
        assert_same(codes_np(rd), np.bitwise_xor.reduce(h.reshape(ntrips, 1024), axis=1), "read")
        assert_same(codes_np(wr), np.arange(n, dtype=np.uint32) ^ np.uint32(0x12345678), "write")
        assert_same(codes_np(cp), h, "copy")


def _fold_reference(xh, bits):
    """The compress-volume reference's output, from its documented layout:
    groups of 2048 values as 8 rows x 64 lanes x 4, each lane's 32 values
    (row-major) XOR-folded into `bits` words."""
    n = xh.size
    pad = (-n) % 2048
    v = np.concatenate([xh.view(np.uint32), np.zeros(pad, np.uint32)])
    g = v.reshape(-1, 8, 64, 4).transpose(0, 2, 1, 3).reshape(-1, 64, bits, 32 // bits)
    return np.bitwise_xor.reduce(g, axis=3).reshape(-1)[:(n * bits + 31) // 32]


@pytest.mark.parametrize("bits", BITS)
def test_fold_reference_kernel(bits):
    """The compress-volume bandwidth reference at sizes with a ragged group."""
    for n in [1, 5, 2048, 2048 * 3 + 77, (1 << 20) + 13]:
        xh = np.random.default_rng(n + bits).standard_normal(n).astype(np.float32)
        x = f32_to_gpu(xh)
        say(f"fold bits={bits} n={n}")
        out = L.fold_f32(x, bits)
        torch.cuda.synchronize()
        assert_same(codes_np(out), _fold_reference(xh, bits), f"fold bits={bits} n={n}")
