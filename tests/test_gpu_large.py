"""GPU parity beyond 2^31 elements: the element indices, word indices and
stochastic-rounding counters of the kernels are 64-bit.  bfloat16 buffers of
2^31 + 12345 elements (4.3 GB each) are generated on the GPU from an integer
hash of the element index (the same integer arithmetic reproduces any element
on the host) and compressed with stochastic rounding, decompressed, reduced
(two peers, with the sum) and error-feedback compressed; blocks sampled across
the buffers, including the last, partial one, are recomputed by the oracle
with their global index offset.
"""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import assert_same, codes_np, f32_np, say, scales_np, word_range
from weight_communication_compression_amd import lowbit as L

pytestmark = pytest.mark.gpu

N = (1 << 31) + 12345
B, BITS = 128, 4


def _bits_host(i: np.ndarray, salt: int = 0) -> np.ndarray:
    """bfloat16 pattern of element i from a multiplicative hash: a random
    sign and 0x3800 + 12 hashed bits (magnitudes between 2^-15 and 2^16)."""
    h = ((i.astype(np.uint64) + np.uint64(salt * 7919)) * np.uint64(0x9E3779B1)) & \
        np.uint64(0xFFFFFFFF)
    sign = (h >> np.uint64(31)) & np.uint64(1)
    body = (h >> np.uint64(7)) & np.uint64(0x0FFF)
    return ((sign << np.uint64(15)) | (np.uint64(0x3800) + body)).astype(np.uint16)


def _bits_gpu(n: int, salt: int = 0) -> torch.Tensor:
    out = torch.empty(n, dtype=torch.int16, device="cuda")
    chunk = 1 << 28
    for lo in range(0, n, chunk):
        i = torch.arange(lo, min(n, lo + chunk), dtype=torch.int64, device="cuda")
        h = ((i + salt * 7919) * 0x9E3779B1) & 0xFFFFFFFF
        sign = (h >> 31) & 1
        body = (h >> 7) & 0x0FFF
        v = (sign << 15) | (0x3800 + body)
        out[lo:lo + i.numel()] = (v - ((v >> 15) << 16)).to(torch.int16)   # as signed 16-bit
        del i, h, sign, body, v
    return out.view(torch.bfloat16)


def test_generator_matches_host():
    for salt in (0, 1):
        g = _bits_gpu(1 << 16, salt)
        want = _bits_host(np.arange(1 << 16, dtype=np.int64), salt)
        assert np.array_equal(g.view(torch.int16).cpu().numpy().view(np.uint16), want)


def _sample_blocks(nb):
    return np.unique(np.concatenate([np.linspace(0, nb - 1, 300).astype(np.int64),
                                     [(1 << 31) // B - 1, (1 << 31) // B, nb - 2, nb - 1]]))


def test_compress_decompress_beyond_2p31():
    say(f"large: generating {N} bfloat16 elements on the GPU")
    x = _bits_gpu(N)
    say("large: compress b4 B128 SR seed 9")
    c, s = L.quantize_pack(x, BITS, B, True, 9, 0)
    torch.cuda.synchronize()
    del x
    say("large: decompress")
    y = L.unpack_dequant(c, s, N, BITS, B)
    torch.cuda.synchronize()
    nb = -(-N // B)
    for k in _sample_blocks(nb):
        lo, hi = int(k) * B, min(N, (int(k) + 1) * B)
        xb = _bits_host(np.arange(lo, hi, dtype=np.int64))
        wc, ws = O.quantize_pack(xb, BITS, B, True, 9, lo)
        a, b = word_range(int(k), B, BITS, N)
        assert_same(codes_np(c[a:b]), wc, f"codes block {k}")
        assert_same(scales_np(s[k:k + 1]), ws, f"scale block {k}")
        assert_same(f32_np(y[lo:hi]), O.unpack_dequant(wc, ws, hi - lo, BITS, B),
                    f"values block {k}")


def test_reduce_and_error_feedback_beyond_2p31():
    nb = -(-N // B)
    say(f"large: two peers of {N} elements, compress b4 B128")
    peers = []
    for salt in (1, 2):
        x = _bits_gpu(N, salt)
        peers.append(L.quantize_pack(x, BITS, B))
        del x
    say("large: local reduce of the two peers, with the sum")
    rc, rs, tot = L.reduce_requant([p[0] for p in peers], [p[1] for p in peers], N, BITS, B,
                                   want_sum=True)
    torch.cuda.synchronize()
    ks = _sample_blocks(nb)
    for k in ks:
        lo, hi = int(k) * B, min(N, (int(k) + 1) * B)
        a, b = word_range(int(k), B, BITS, N)
        pc = [codes_np(p[0][a:b]) for p in peers]
        ps = [scales_np(p[1][k:k + 1]) for p in peers]
        for salt, (cc, ss) in zip((1, 2), zip(pc, ps)):
            wc, ws = O.quantize_pack(_bits_host(np.arange(lo, hi, dtype=np.int64), salt), BITS, B)
            assert_same(cc, wc, f"peer {salt} codes block {k}")
            assert_same(ss, ws, f"peer {salt} scale block {k}")
        wc, ws, wt = O.reduce_requant(pc, ps, hi - lo, BITS, B, BITS, want_sum=True)
        assert_same(codes_np(rc[a:b]), wc, f"reduce codes block {k}")
        assert_same(scales_np(rs[k:k + 1]), ws, f"reduce scale block {k}")
        assert_same(f32_np(tot[lo:hi]), wt, f"reduce sum block {k}")
    del peers, rc, rs, tot

    say("large: error-feedback compress, zero residual, b4 B128 SR seed 5")
    g = _bits_gpu(N, 3)
    e = torch.zeros(N, dtype=torch.float32, device="cuda")
    ec, es = L.ef_compress(g, e, BITS, B, True, 5, 0)
    torch.cuda.synchronize()
    for k in ks:
        lo, hi = int(k) * B, min(N, (int(k) + 1) * B)
        a, b = word_range(int(k), B, BITS, N)
        wc, ws, we = O.ef_compress(_bits_host(np.arange(lo, hi, dtype=np.int64), 3),
                                   np.zeros(hi - lo, np.float32), BITS, B, True, 5, lo)
        assert_same(codes_np(ec[a:b]), wc, f"ef codes block {k}")
        assert_same(scales_np(es[k:k + 1]), ws, f"ef scale block {k}")
        assert_same(f32_np(e[lo:hi]), we, f"ef residual block {k}")
