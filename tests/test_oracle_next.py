"""CPU pins of the oracle's error-feedback variants and mixed-width reduce.

* EF21 compress (bitscom README, "Backend Registration Options", mode
  "ef21"): d = fl(g - h), quantize d, h <- fl(h + deq).
* Stage-2 error feedback on the reduced shard (same section, mode
  "ef21_plus"): a = fl(sum + e), quantize a, e <- fl(a - deq).
* Mixed input/output bit counts and block sizes in the local reduce (SDP4Bit
  README, "Gradient Quantization Arguments": 8-bit intra-node and 4-bit
  inter-node gradient quantization with their own group sizes).

Every expected value is re-derived here with numpy from the definitions (a
numpy decoder of the packed format, float32 sums in peer order), or follows
from a property of the method (EF21's state converging to a constant
gradient), and is compared with the oracle.
"""
import numpy as np
import pytest
import torch


def _decode_numpy(words, scales, n, bits, block):
    """Packed codes + binary16 scales -> float32, from the format's definition:
    element i is bits [(i mod 32/b)*b, +b) of word i*b/32; q = u - 2^(b-1),
    value q*s (1 bit: u ? s : -s); s is the scale of block i // block."""
    per = 32 // bits
    sh = (np.arange(per, dtype=np.uint32) * bits)[None, :]
    u = ((np.asarray(words, np.uint32)[:, None] >> sh) & np.uint32((1 << bits) - 1)).reshape(-1)[:n]
    s = np.asarray(scales, np.uint16).view(np.float16).astype(np.float32)
    s = s[np.arange(n) // block]
    if bits == 1:
        return np.where(u == 1, s, -s).astype(np.float32)
    q = u.astype(np.int64) - (1 << (bits - 1))
    return (q.astype(np.float32) * s).astype(np.float32)


def _normal(seed, n, scale=1.0):
    return (np.random.default_rng(seed).standard_normal(n) * scale).astype(np.float32)


def _peers(oracle_mod, P, n, bits, block, seed=20):
    pcs, pss = [], []
    for p in range(P):
        x = _normal(seed + p, n, 10.0 ** (p % 3 - 1))
        c, s = oracle_mod.quantize_pack(x, bits, block)
        pcs.append(c)
        pss.append(s)
    return pcs, pss


def _sum_numpy(pcs, pss, n, bits, block):
    acc = None
    for c, s in zip(pcs, pss):
        d = _decode_numpy(c, s, n, bits, block)
        acc = d.copy() if acc is None else (acc + d).astype(np.float32)
    return acc


def _as_bf16_bits(x):
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _bf16_value(b):
    return (b.astype(np.uint32) << 16).view(np.float32)


# ------------------------------------------------------------- EF21 --------
@pytest.mark.parametrize("bits", [1, 2, 4, 8])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("sr", [False, True])
def test_ef21_rederived(oracle_mod, bits, dtype, sr):
    """codes = compress(fl(g - h)) with the pinned compress; the new state is
    fl(h + deq) with deq decoded by numpy."""
    n, B = 128 * 50 + 37, 128
    g = _normal(1, n, 1e-3)
    gin = _as_bf16_bits(g) if dtype == "bf16" else g
    gf = _bf16_value(gin) if dtype == "bf16" else g
    h = _normal(2, n, 5e-4)
    codes, scales, h_new = oracle_mod.ef21_compress(gin, h, bits, B, sr, 7, 0)
    d = (gf - h).astype(np.float32)
    cq, sq = oracle_mod.quantize_pack(d, bits, B, sr, 7, 0)
    assert np.array_equal(codes, cq) and np.array_equal(scales, sq)
    deq = _decode_numpy(codes, scales, n, bits, B)
    assert np.array_equal(h_new, (h + deq).astype(np.float32))


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_ef21_state_converges_to_constant_gradient(oracle_mod, bits):
    """With a fixed gradient, round-to-nearest EF21 shrinks each block's
    largest gap |g - h| by about a factor 2*qmax per step, so h reaches g
    within a few steps.  The bound per step: the scale is at most
    gap/qmax rounded up to binary16 (relative 2^-10, or up to the next
    multiple of 2^-24 once it is subnormal), the nearest-rounding error is at
    most s*(1/2 + (qmax+1)*2^-23), plus the binary32 roundings of g - h and
    h + deq."""
    n, B = 256 * 40, 256
    qmax = (1 << (bits - 1)) - 1
    g = _normal(3, n, 1e-2)
    h = np.zeros(n, np.float32)
    gap0 = np.abs(g - h).reshape(-1, B).max(axis=1)
    for step in range(4):
        _, _, h = oracle_mod.ef21_compress(g, h, bits, B)
        gap = np.abs(g.astype(np.float64) - h).reshape(-1, B).max(axis=1)
        s_max = gap0 * (1.0 + 2.0 ** -10) / qmax + 2.0 ** -24
        bound = s_max * (0.5 + (qmax + 1) * 2.0 ** -23) + \
            2.0 * np.spacing(np.abs(g)).reshape(-1, B).max(axis=1)
        assert np.all(gap <= bound), (step, float((gap / bound).max()))
        gap0 = gap


def test_ef21_zero_state_is_plain_compress(oracle_mod):
    """h = 0: the message is the plain compress of g and h becomes deq."""
    n, B = 64 * 33, 64
    g = _normal(4, n)
    codes, scales, h = oracle_mod.ef21_compress(g, np.zeros(n, np.float32), 4, B)
    cq, sq = oracle_mod.quantize_pack(g, 4, B)
    assert np.array_equal(codes, cq) and np.array_equal(scales, sq)
    assert np.array_equal(h, _decode_numpy(cq, sq, n, 4, B))


# ------------------------------------------------ stage-2 EF (reduce) --------
@pytest.mark.parametrize("bits", [1, 2, 4, 8])
@pytest.mark.parametrize("P", [1, 3, 8])
@pytest.mark.parametrize("sr", [False, True])
def test_reduce_stage2_ef_is_ef_on_the_sum(oracle_mod, bits, P, sr):
    """The reduce with a residual is error-feedback compress of the peer-order
    float32 sum (numpy), with the pinned EF compress; out_sum is the sum
    before the residual is added."""
    n, B = 128 * 30 + 77, 128
    pcs, pss = _peers(oracle_mod, P, n, bits, B)
    acc = _sum_numpy(pcs, pss, n, bits, B)
    e = _normal(9, n, 1e-3)
    codes, scales, total, e_new = oracle_mod.reduce_requant_ex(
        pcs, pss, n, bits, B, bits, B, sr, 11, 0, residual=e, want_sum=True)
    assert np.array_equal(total, acc)
    ce, se, ee = oracle_mod.ef_compress(acc, e, bits, B, sr, 11, 0)
    assert np.array_equal(codes, ce) and np.array_equal(scales, se)
    assert np.array_equal(e_new, ee)
    # and directly: e_new = fl(fl(acc + e) - deq)
    a = (acc + e).astype(np.float32)
    deq = _decode_numpy(codes, scales, n, bits, B)
    assert np.array_equal(e_new, (a - deq).astype(np.float32))


def test_reduce_stage2_zero_residual_matches_plain_reduce(oracle_mod):
    n, B = 256 * 20, 256
    pcs, pss = _peers(oracle_mod, 4, n, 4, B)
    c0, s0, _ = oracle_mod.reduce_requant(pcs, pss, n, 4, B, 4)
    c1, s1, _, e1 = oracle_mod.reduce_requant_ex(pcs, pss, n, 4, B, 4, B,
                                                 residual=np.zeros(n, np.float32))
    assert np.array_equal(c0, c1) and np.array_equal(s0, s1)
    acc = _sum_numpy(pcs, pss, n, 4, B)
    assert np.array_equal(e1, (acc - _decode_numpy(c1, s1, n, 4, B)).astype(np.float32))


def test_reduce_stage2_residual_carries_the_error(oracle_mod):
    """Over several rounds with the same peer data, the transmitted values
    plus the final residual add up to rounds x sum (up to the binary32
    roundings of the residual chain): nothing is lost."""
    n, B, rounds = 128 * 16, 128, 5
    pcs, pss = _peers(oracle_mod, 2, n, 2, B)
    acc = _sum_numpy(pcs, pss, n, 2, B).astype(np.float64)
    e = np.zeros(n, np.float32)
    sent = np.zeros(n, np.float64)
    slack = np.zeros(n, np.float64)
    for r in range(rounds):
        c, s, _, e = oracle_mod.reduce_requant_ex(pcs, pss, n, 2, B, 2, B, residual=e)
        sent += _decode_numpy(c, s, n, 2, B)
        slack += np.spacing(np.abs(acc) + np.abs(e)) * 2
    assert np.all(np.abs(sent + e - rounds * acc) <= slack)


# ------------------------------------------- mixed widths and blocks --------
@pytest.mark.parametrize("in_bits,in_block,out_bits,out_block", [
    (8, 512, 4, 128),      # the SDP4Bit default pair: 8-bit intra, 4-bit inter
    (8, 128, 4, 128),
    (8, 128, 2, 64),
    (4, 128, 2, 512),
    (4, 64, 8, 256),
    (2, 32, 4, 4096),
    (1, 256, 4, 128),
    (8, 4096, 1, 32),
])
@pytest.mark.parametrize("sr", [False, True])
def test_reduce_mixed_widths_rederived(oracle_mod, in_bits, in_block, out_bits, out_block, sr):
    """Peers packed with (in_bits, in_block) are decoded by numpy and summed in
    peer order; the output equals the pinned compress of that sum with
    (out_bits, out_block)."""
    n = 4096 * 3 + 160 + 7
    P = 5
    pcs, pss = _peers(oracle_mod, P, n, in_bits, in_block)
    acc = _sum_numpy(pcs, pss, n, in_bits, in_block)
    codes, scales, total, _ = oracle_mod.reduce_requant_ex(
        pcs, pss, n, in_bits, in_block, out_bits, out_block, sr, 5, 0, want_sum=True)
    assert np.array_equal(total, acc)
    cq, sq = oracle_mod.quantize_pack(acc, out_bits, out_block, sr, 5, 0)
    assert np.array_equal(codes, cq) and np.array_equal(scales, sq)


def test_reduce_mixed_with_residual(oracle_mod):
    n = 512 * 9 + 100
    pcs, pss = _peers(oracle_mod, 8, n, 8, 512)
    acc = _sum_numpy(pcs, pss, n, 8, 512)
    e = _normal(12, n, 1e-2)
    codes, scales, _, e_new = oracle_mod.reduce_requant_ex(pcs, pss, n, 8, 512, 4, 128,
                                                           residual=e)
    ce, se, ee = oracle_mod.ef_compress(acc, e, 4, 128)
    assert np.array_equal(codes, ce) and np.array_equal(scales, se) and np.array_equal(e_new, ee)


def test_reduce_ex_invalid_arguments(oracle_mod):
    n = 256
    pcs, pss = _peers(oracle_mod, 2, n, 8, 128)
    for args in [(8, 96, 4, 128), (8, 128, 3, 128), (8, 128, 4, 8192), (5, 128, 4, 128)]:
        with pytest.raises(ValueError):
            oracle_mod.reduce_requant_ex(pcs, pss, n, *args)
    with pytest.raises(ValueError):
        oracle_mod.reduce_requant_ex(pcs, pss, n, 8, 128, 4, 128, out_index_offset=64)
    with pytest.raises(ValueError):
        oracle_mod.reduce_requant_ex([], [], n, 8, 128, 4, 128)


# ---------------------------------------------------- Hadamard smoothing ----
# Pins of the blockwise Walsh-Hadamard transform against scipy's Sylvester
# matrix (an independent library routine), exact where the arithmetic is
# exact, and of the transform's purpose (smaller quantization error on data
# with outliers).
import scipy.linalg  # noqa: E402

HS_BLOCKS = [32, 64, 128, 256, 512, 1024, 2048, 4096]


def _hs_factors(B):
    L = B.bit_length() - 1
    return 2.0 ** -(L // 2), 2.0 ** -((L + 1) // 2)


@pytest.mark.parametrize("B", HS_BLOCKS)
def test_hadamard_is_sylvester_matrix_on_integers(oracle_mod, B):
    """Small integers keep every butterfly exact, so the binary32 transform
    must equal H_B @ x (scipy.linalg.hadamard, float64) times the stated
    power of two, bit for bit; the inverse restores x."""
    H = scipy.linalg.hadamard(B).astype(np.float64)
    fwd, inv = _hs_factors(B)
    rng = np.random.default_rng(B)
    x = rng.integers(-1000, 1000, size=3 * B).astype(np.float32)
    y = oracle_mod.hadamard_blocks(x, B)
    want = (x.reshape(-1, B).astype(np.float64) @ H.T * fwd).astype(np.float32).reshape(-1)
    assert np.array_equal(y, want)
    assert np.array_equal(oracle_mod.hadamard_blocks(y, B, inverse=True), x)
    # H is symmetric and H @ H = B * I: fwd * inv = 1 / B
    assert fwd * inv * B == 1.0


@pytest.mark.parametrize("B", [32, 128, 4096])
def test_hadamard_real_data_error_bound(oracle_mod, B):
    """On real data each output is within 2^L * 2^-24 * sum|x| (times the
    scaling) of the exact product: rounding errors of a stage reach each
    output once per later-stage path."""
    H = scipy.linalg.hadamard(B).astype(np.float64)
    fwd, _ = _hs_factors(B)
    x = _normal(31, 4 * B)
    y = oracle_mod.hadamard_blocks(x, B).astype(np.float64).reshape(-1, B)
    xb = x.reshape(-1, B).astype(np.float64)
    exact = xb @ H.T * fwd
    bound = B * 2.0 ** -24 * np.abs(xb).sum(axis=1, keepdims=True) * fwd
    assert np.all(np.abs(y - exact) <= bound)


@pytest.mark.parametrize("bits", [1, 2, 4, 8])
@pytest.mark.parametrize("B", [32, 128, 512, 4096])
@pytest.mark.parametrize("sr", [False, True])
def test_hadamard_compress_is_compress_of_transform(oracle_mod, bits, B, sr):
    """With exactly transformable (integer) inputs the smoothed compress is
    the pinned compress of H x (scipy, float64, exact)."""
    H = scipy.linalg.hadamard(B).astype(np.float64)
    fwd, _ = _hs_factors(B)
    x = np.random.default_rng(bits * B).integers(-300, 300, size=5 * B).astype(np.float32)
    y = (x.reshape(-1, B).astype(np.float64) @ H.T * fwd).astype(np.float32).reshape(-1)
    c, s = oracle_mod.hadamard_quantize_pack(x, bits, B, sr, 17, 2 * B)
    cq, sq = oracle_mod.quantize_pack(y, bits, B, sr, 17, 2 * B)
    assert np.array_equal(c, cq) and np.array_equal(s, sq)


@pytest.mark.parametrize("bits", [1, 2, 4, 8])
@pytest.mark.parametrize("B", HS_BLOCKS)
def test_hadamard_decompress_is_exact_matrix_product(oracle_mod, bits, B):
    """Decoded values of a block are integer multiples of its scale with
    |sum| <= B * 127 < 2^24 multiples, so the inverse butterflies are exact:
    the result equals (H @ deq) * 2^-ceil(L/2) computed in float64."""
    H = scipy.linalg.hadamard(B).astype(np.float64)
    _, inv = _hs_factors(B)
    x = mixed_input_np(41 + bits, 3 * B)
    c, s = oracle_mod.quantize_pack(x, bits, B)
    deq = _decode_numpy(c, s, x.size, bits, B).astype(np.float64)
    want = (deq.reshape(-1, B) @ H.T * inv).astype(np.float32).reshape(-1)
    got = oracle_mod.hadamard_unpack_dequant(c, s, x.size, bits, B)
    assert np.array_equal(got, want)


def mixed_input_np(seed, n):
    g = np.random.default_rng(seed)
    mag = 10.0 ** g.uniform(-6, 2, size=n // 32).repeat(32)
    return (g.standard_normal(n) * mag).astype(np.float32)


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("B", [64, 128, 512])
def test_hadamard_roundtrip_error_bound(oracle_mod, bits, B):
    """Round trip through smoothed compress/decompress: per block the L2 error
    is at most sqrt(B) * s * (1/2 + (qmax+1) 2^-23) (nearest rounding in the
    transformed domain, the transform orthonormal up to its scaling) plus
    binary32 slack; checked on blocks with one large outlier each."""
    qmax = (1 << (bits - 1)) - 1
    rng = np.random.default_rng(bits + B)
    x = rng.standard_normal(64 * B).astype(np.float32)
    x[rng.integers(0, B, size=64) + np.arange(64) * B] *= 200.0      # one outlier per block
    c, s = oracle_mod.hadamard_quantize_pack(x, bits, B)
    xh = oracle_mod.hadamard_unpack_dequant(c, s, x.size, bits, B)
    sc = s.view(np.float16).astype(np.float64)
    L = B.bit_length() - 1
    shrink = 2.0 ** (L / 2 - (L + 1) // 2)          # ||x^ - x|| = shrink * ||y^ - y||
    err = np.sqrt(((xh.astype(np.float64) - x).reshape(-1, B) ** 2).sum(axis=1))
    bound = shrink * np.sqrt(B) * sc * (0.5 + (qmax + 1) * 2.0 ** -23) + \
        1e-5 * np.sqrt((x.reshape(-1, B).astype(np.float64) ** 2).sum(axis=1))
    assert np.all(err <= bound)


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("B", [64, 128, 512])
def test_hadamard_lowers_error_on_heavy_tailed_data(oracle_mod, bits, B):
    """What the transform is for: on heavy-tailed (Student-t, 3 degrees of
    freedom) data, like the gradient buckets, the smoothed round trip has
    less than half the mean squared error of plain quantization at 4 and 8
    bits."""
    x = np.random.default_rng(bits + B).standard_t(3, 256 * B).astype(np.float32)
    c, s = oracle_mod.hadamard_quantize_pack(x, bits, B)
    xh = oracle_mod.hadamard_unpack_dequant(c, s, x.size, bits, B)
    cp, sp = oracle_mod.quantize_pack(x, bits, B)
    xp = oracle_mod.unpack_dequant(cp, sp, x.size, bits, B)
    mse_plain = float(((xp.astype(np.float64) - x) ** 2).mean())
    mse_hs = float(((xh.astype(np.float64) - x) ** 2).mean())
    assert mse_hs < 0.5 * mse_plain


@pytest.mark.parametrize("bits", [1, 2, 4, 8])
@pytest.mark.parametrize("B", [32, 128, 4096])
@pytest.mark.parametrize("rem", [1, 7, 31])
def test_hadamard_partial_last_block_is_plain(oracle_mod, bits, B, rem):
    """A last block of rem < B elements is compressed and decompressed without
    the transform: the whole blocks give what the smoothed codec gives on
    them alone, and the partial block gives what the pinned plain compress
    and decompress give on it, at its global index."""
    k = 3 if B < 4096 else 1
    n = k * B + rem
    x = np.random.default_rng(B + rem + bits).standard_t(3, n).astype(np.float32)
    c, s = oracle_mod.hadamard_quantize_pack(x, bits, B, True, 5, 4 * B)
    c0, s0 = oracle_mod.hadamard_quantize_pack(x[:k * B], bits, B, True, 5, 4 * B)
    ct, st = oracle_mod.quantize_pack(x[k * B:], bits, B, True, 5, 4 * B + k * B)
    w0 = k * B * bits // 32
    assert np.array_equal(c[:w0], c0) and np.array_equal(s[:k], s0)
    assert np.array_equal(c[w0:], ct) and np.array_equal(s[k:], st)
    y = oracle_mod.hadamard_unpack_dequant(c, s, n, bits, B)
    assert np.array_equal(y[:k * B], oracle_mod.hadamard_unpack_dequant(c0, s0, k * B, bits, B))
    assert np.array_equal(y[k * B:], oracle_mod.unpack_dequant(ct, st, rem, bits, B))
    t = oracle_mod.hadamard_blocks(x, B)
    assert np.array_equal(t[:k * B], oracle_mod.hadamard_blocks(x[:k * B], B))
    assert np.array_equal(t[k * B:], x[k * B:])


def test_hadamard_partial_only_block_is_plain(oracle_mod):
    """n < B: the single partial block is the plain codec's."""
    x = np.random.default_rng(3).standard_normal(100).astype(np.float32)
    c, s = oracle_mod.hadamard_quantize_pack(x, 4, 128)
    wc, ws = oracle_mod.quantize_pack(x, 4, 128)
    assert np.array_equal(c, wc) and np.array_equal(s, ws)
    assert np.array_equal(oracle_mod.hadamard_unpack_dequant(c, s, 100, 4, 128),
                          oracle_mod.unpack_dequant(wc, ws, 100, 4, 128))


def test_hadamard_handworked_stage_order(oracle_mod):
    """Worked by hand: B = 32, x = [1, 2^-24, -1, 2^-24, 0, ..., 0].
    Stride 1: fl(1 + 2^-24) = 1 (tie, to even), fl(1 - 2^-24) = 1 - 2^-24
    (exact), fl(-1 + 2^-24) = -1 + 2^-24 (exact), fl(-1 - 2^-24) = -1 (tie).
    Stride 2: y0 = 1 + (-1 + 2^-24) = 2^-24, y1 = (1 - 2^-24) + (-1) = -2^-24,
    y2 = 1 - (-1 + 2^-24) = 2 - 2^-24 -> 2 (tie, to even), y3 = (1 - 2^-24) -
    (-1) -> 2.  Strides 4..16 pair these with zeros and copy them, so the
    block is [2^-24, -2^-24, 2, 2] eight times, scaled by 2^-floor(5/2) = 1/4.
    The strides in the other order would give y0 = (1 - 1) + 2^-23 = 2^-23."""
    x = np.zeros(32, np.float32)
    x[0], x[1], x[2], x[3] = 1.0, 2.0 ** -24, -1.0, 2.0 ** -24
    want = np.tile(np.array([2.0 ** -26, -2.0 ** -26, 0.5, 0.5], np.float32), 8)
    assert np.array_equal(oracle_mod.hadamard_blocks(x, 32), want)
