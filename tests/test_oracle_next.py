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
