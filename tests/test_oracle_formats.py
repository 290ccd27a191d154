"""Pins of the oracle's number formats, generator and bit packing.

Each test compares the oracle (plain C, ``oracle/lowbit_oracle.c``) with
something independent of it: numpy's and torch's own format conversions,
published MurmurHash3 test vectors, closed forms, and statistics.
"""
import numpy as np
import pytest
import torch


# ------------------------------------------------------------------ fp16 --
def test_f16_to_f32_all_patterns(oracle_mod):
    """All 65536 binary16 patterns widen exactly as numpy's float16 does."""
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = oracle_mod.f16_to_f32(h)
    want = h.view(np.float16).astype(np.float32)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))


def _pattern_chunks(lo_bits, hi_bits, chunk=1 << 24):
    for a in range(lo_bits, hi_bits, chunk):
        b = min(hi_bits, a + chunk)
        yield np.arange(a, b, dtype=np.uint64).astype(np.uint32).view(np.float32)


# binary32 exponent fields 0x60..0x90 cover everything from far below the
# smallest binary16 subnormal (2^-24) to above the overflow threshold (65520).
F16_RANGE = (0x60 << 23, 0x90 << 23)


def test_f32_to_f16_rne_exhaustive_range(oracle_mod):
    """Every binary32 pattern whose exponent is within reach of binary16 rounds
    exactly as numpy's float16 cast (IEEE round-to-nearest-even)."""
    with np.errstate(over="ignore"):
        for x in _pattern_chunks(*F16_RANGE):
            got = oracle_mod.f32_to_f16_rne(x)
            want = x.astype(np.float16).view(np.uint16)
            assert np.array_equal(got, want)
            got = oracle_mod.f32_to_f16_rne(-x)
            want = (-x).astype(np.float16).view(np.uint16)
            assert np.array_equal(got, want)


def test_f32_to_f16_rne_outside_range_sample(oracle_mod):
    g = np.random.default_rng(5)
    bits = g.integers(0, 1 << 32, size=1 << 22, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        want = x.astype(np.float16)
    got = oracle_mod.f32_to_f16_rne(x)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got.view(np.float16)), nan)
    assert np.array_equal(got[~nan], want.view(np.uint16)[~nan])


def test_f16_round_up_closed_form(oracle_mod):
    """Round-up scale conversion: the result h is the smallest binary16 value
    not below t, saturated at 65504 (checked with numpy's float16 values)."""
    f16max = np.float32(65504.0)
    # from 2^-63 (all of which rounds up to the smallest subnormal) to just
    # above 65536; the remaining patterns are sampled below.
    for x in _pattern_chunks(F16_RANGE[0], 0x47800000 + (1 << 20)):
        h = oracle_mod.f16_round_up(x)
        hv = h.view(np.float16).astype(np.float32)
        sat = x > f16max
        assert np.all(h[sat] == 0x7BFF)
        ok = ~sat
        assert np.all(hv[ok] >= x[ok])
        # the binary16 value just below h (h - 1 as a pattern) is below t
        prev = np.where(h[ok] > 0, h[ok] - 1, 0).astype(np.uint16).view(np.float16) \
            .astype(np.float32)
        assert np.all((h[ok] == 0) | (prev < x[ok]))
        assert np.all((h[ok] != 0) | (x[ok] == 0))


def test_f16_round_up_sample(oracle_mod):
    g = np.random.default_rng(11)
    x = g.integers(0, 0x7F800000, size=1 << 22, dtype=np.uint64).astype(np.uint32) \
        .view(np.float32)
    h = oracle_mod.f16_round_up(x)
    hv = h.view(np.float16).astype(np.float32)
    sat = x > np.float32(65504)
    assert np.all(h[sat] == 0x7BFF)
    assert np.all(hv[~sat] >= x[~sat])
    tiny = x < np.float32(2.0 ** -24)
    assert np.all(h[tiny & (x > 0)] == 1)


def test_f16_round_up_special_values(oracle_mod):
    x = np.array([0.0, np.inf, np.nan, 65504.0, 65505.0, 1e9, 2.0 ** -24, 2.0 ** -26],
                 np.float32)
    h = oracle_mod.f16_round_up(x)
    assert list(h) == [0x0000, 0x7BFF, 0x7BFF, 0x7BFF, 0x7BFF, 0x7BFF, 0x0001, 0x0001]


# ------------------------------------------------------------------ bf16 --
def test_bf16_rne_against_torch(oracle_mod):
    """binary32 -> bfloat16 RNE matches torch's CPU cast (strided sweep over all
    patterns plus every low-half pattern around a tie)."""
    step = 4099   # odd stride: visits every residue of the low 16 bits
    bits = np.arange(0, 1 << 32, step, dtype=np.uint64).astype(np.uint32)
    ties = (np.arange(1 << 16, dtype=np.uint32) << 16)[:, None] + \
        np.array([0x7FFF, 0x8000, 0x8001], np.uint32)[None, :]
    bits = np.concatenate([bits, ties.reshape(-1).astype(np.uint32)])
    x = bits.view(np.float32)
    got = oracle_mod.f32_to_bf16_rne(x)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    fin = np.isfinite(x)
    assert np.array_equal(got[fin], want[fin])
    # NaN stays NaN
    gw = (got[~fin & np.isnan(x)].astype(np.uint32) << 16).view(np.float32)
    assert np.all(np.isnan(gw))


def test_bf16_widen_exact(oracle_mod):
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = np.array([oracle_mod.lib().oracle_bf16_to_f32(int(v)) for v in h[::97]], np.float32)
    want = torch.from_numpy(h[::97].view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    fin = np.isfinite(want)
    assert np.array_equal(got[fin].view(np.uint32), want[fin].view(np.uint32))


# --------------------------------------------------------- the generator --
def _murmur3_x86_32(data: bytes, seed: int, fmix) -> int:
    """MurmurHash3_x86_32 body written here; the final avalanche is the
    oracle's fmix32.  Published test vectors of the whole hash therefore pin
    the oracle's finaliser."""
    c1, c2 = 0xCC9E2D51, 0x1B873593
    m32 = 0xFFFFFFFF

    def rotl(x, r):
        return ((x << r) | (x >> (32 - r))) & m32

    h = seed & m32
    n = len(data)
    nblk = n // 4
    for i in range(nblk):
        k = int.from_bytes(data[4 * i:4 * i + 4], "little")
        k = rotl((k * c1) & m32, 15)
        k = (k * c2) & m32
        h ^= k
        h = rotl(h, 13)
        h = (h * 5 + 0xE6546B64) & m32
    tail = data[4 * nblk:]
    k = 0
    if len(tail) >= 3:
        k ^= tail[2] << 16
    if len(tail) >= 2:
        k ^= tail[1] << 8
    if len(tail) >= 1:
        k ^= tail[0]
        k = rotl((k * c1) & m32, 15)
        k = (k * c2) & m32
        h ^= k
    h ^= n
    return int(fmix(np.array([h], np.uint32))[0])


# Published MurmurHash3_x86_32 test vectors (input, seed, hash).
MURMUR3_VECTORS = [
    (b"", 0, 0x00000000),
    (b"", 1, 0x514E28B7),
    (b"", 0xFFFFFFFF, 0x81F16F39),
    (b"\x00\x00\x00\x00", 0, 0x2362F9DE),
    (b"\xff\xff\xff\xff", 0, 0x76293B50),
    (b"\x21\x43\x65\x87", 0, 0xF55B516B),
    (b"\x21\x43\x65\x87", 0x5082EDEE, 0x2362F9DE),
    (b"\x21\x43\x65", 0, 0x7E4A8634),
    (b"\x21\x43", 0, 0xA0F7B07A),
    (b"\x21", 0, 0x72661CF4),
    (b"a", 0x9747B28C, 0x7FA09EA6),
    (b"aa", 0x9747B28C, 0x5D211726),
    (b"aaa", 0x9747B28C, 0x283E0130),
    (b"aaaa", 0x9747B28C, 0x5A97808A),
    (b"ab", 0x9747B28C, 0x74875592),
    (b"abc", 0x9747B28C, 0xC84A62DD),
    (b"abcd", 0x9747B28C, 0xF0478627),
    (b"Hello, world!", 0x9747B28C, 0x24884CBA),
    (b"The quick brown fox jumps over the lazy dog", 0x9747B28C, 0x2FA826CD),
]


@pytest.mark.parametrize("data,seed,want", MURMUR3_VECTORS)
def test_fmix32_published_vectors(oracle_mod, data, seed, want):
    assert _murmur3_x86_32(data, seed, oracle_mod.fmix32) == want


def test_sr_uniform_grid_and_range(oracle_mod):
    r = oracle_mod.sr_uniform(42, 0, 1 << 20)
    assert r.min() >= 0.0 and r.max() < 1.0
    assert np.array_equal(r * np.float32(1 << 24), np.floor(r * np.float32(1 << 24)))


def test_sr_uniform_statistics(oracle_mod):
    """Mean, variance and a 256-bin chi-square of 2^20 draws, for several seeds
    and for indices above 2^32 (the high half of the index is mixed in)."""
    n = 1 << 20
    for seed, i0 in [(0, 0), (42, 0), (7, (1 << 32) - (n // 2)), (123456789, 5 << 33)]:
        r = oracle_mod.sr_uniform(seed, i0, n).astype(np.float64)
        assert abs(r.mean() - 0.5) < 4 * np.sqrt(1 / 12 / n)
        assert abs(r.var() - 1 / 12) < 0.002
        counts = np.bincount((r * 256).astype(np.int64), minlength=256)
        chi2 = ((counts - n / 256) ** 2 / (n / 256)).sum()
        assert chi2 < 255 + 6 * np.sqrt(2 * 255)     # ~6 sigma
        # lag-1 correlation of consecutive indices
        c = np.corrcoef(r[:-1], r[1:])[0, 1]
        assert abs(c) < 5 / np.sqrt(n)


def test_sr_streams_differ(oracle_mod):
    a = oracle_mod.sr_uniform(1, 0, 4096)
    b = oracle_mod.sr_uniform(2, 0, 4096)
    c = oracle_mod.sr_uniform(1, 1 << 32, 4096)
    assert np.mean(a == b) < 0.01 and np.mean(a == c) < 0.01


def test_sr_bits_match_uniform(oracle_mod):
    for i in [0, 1, 2, 12345, (1 << 32) + 3]:
        h = oracle_mod.sr_bits(42, i)
        r = oracle_mod.sr_uniform(42, i, 1)[0]
        assert r == np.float32((h >> 8) / float(1 << 24))


# --------------------------------------------------------------- packing --
@pytest.mark.parametrize("n", [0, 1, 7, 31, 32, 33, 1000, 4099])
def test_pack_1bit_vs_packbits(oracle_mod, n):
    u = np.random.default_rng(n).integers(0, 2, size=n).astype(np.uint32)
    words = oracle_mod.pack_codes(u, 1)
    nw = (n + 31) // 32
    pb = np.packbits(u.astype(np.uint8), bitorder="little")
    pb = np.concatenate([pb, np.zeros(4 * nw - pb.size, np.uint8)])
    assert np.array_equal(words, pb.view("<u4"))


@pytest.mark.parametrize("n", [0, 1, 3, 4, 5, 1000, 4099])
def test_pack_8bit_vs_bytes(oracle_mod, n):
    u = np.random.default_rng(n).integers(0, 256, size=n).astype(np.uint32)
    words = oracle_mod.pack_codes(u, 8)
    nw = (n + 3) // 4
    b = np.concatenate([u.astype(np.uint8), np.zeros(4 * nw - n, np.uint8)])
    assert np.array_equal(words, b.view("<u4"))


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("n", [1, 15, 16, 17, 999, 4099])
def test_pack_2_4bit_vs_shifts(oracle_mod, bits, n):
    per = 32 // bits
    u = np.random.default_rng(n * bits).integers(0, 1 << bits, size=n).astype(np.uint64)
    pad = np.zeros((-n) % per, np.uint64)
    m = np.concatenate([u, pad]).reshape(-1, per)
    want = (m << (np.arange(per, dtype=np.uint64) * bits)[None, :]).sum(axis=1).astype(np.uint32)
    assert np.array_equal(oracle_mod.pack_codes(u.astype(np.uint32), bits), want)


@pytest.mark.parametrize("bits", [1, 2, 4, 8])
def test_pack_roundtrip(oracle_mod, bits):
    for n in [1, 33, 257, 10007]:
        u = np.random.default_rng(n).integers(0, 1 << bits, size=n).astype(np.uint32)
        w = oracle_mod.pack_codes(u, bits)
        assert w.size == (n * bits + 31) // 32
        assert np.array_equal(oracle_mod.unpack_codes(w, n, bits), u)
        # unused high bits of the last word are zero
        used = (n * bits) % 32
        if used:
            assert int(w[-1]) >> used == 0
