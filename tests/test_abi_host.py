"""Host-side checks of the C ABI (no GPU needed).

The library loads, exports every entry point ``include/lowbit.h`` declares,
computes sizes, and rejects invalid arguments before making any HIP call.
No test here launches a kernel.
"""
import ctypes
import os
import re

import pytest

from weight_communication_compression_amd import lowbit as lb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lowbit.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lowbit_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = _declared()
    assert "lowbit_quantize_pack" in names and len(names) >= 11
    L = ctypes.CDLL(lb.library_path)
    for name in names:
        assert hasattr(L, name), name


def test_version_and_status_strings():
    assert lb.lib().lowbit_version().startswith(b"lowbit ")
    for code, text in [(0, b"ok"), (1, b"invalid argument"), (2, b"unsupported combination"),
                       (3, b"device launch error"), (99, b"unknown status")]:
        assert lb.lib().lowbit_status_string(code) == text


@pytest.mark.parametrize("n", [0, 1, 7, 8, 31, 32, 33, 1 << 20, (1 << 40) + 3])
@pytest.mark.parametrize("bits", [1, 2, 4, 8])
def test_num_words(n, bits):
    assert lb.num_words(n, bits) == (n * bits + 31) // 32


@pytest.mark.parametrize("B", [32, 64, 128, 256, 512, 1024, 2048, 4096])
def test_num_blocks(B):
    for n in [0, 1, B - 1, B, B + 1, 1000 * B + 17]:
        assert lb.num_blocks(n, B) == -(-n // B)


def test_size_helpers_reject():
    L = lb.lib()
    for bits in [0, 3, 5, 16, -1]:
        assert L.lowbit_num_words(10, bits) == -1
    for B in [0, 16, 48, 8192, 100]:
        assert L.lowbit_num_blocks(10, B) == -1
    assert L.lowbit_num_words(-1, 4) == -1


def _qp(**kw):
    d = dict(bitwidth=4, block_size=128, stochastic=0, hints=0, seed=0, index_offset=0)
    d.update(kw)
    return lb.QParams(**d)


BAD_PARAMS = [dict(bitwidth=3), dict(bitwidth=16), dict(block_size=16), dict(block_size=96),
              dict(block_size=8192), dict(index_offset=64), dict(hints=2), dict(hints=-1)]


@pytest.mark.parametrize("bad", BAD_PARAMS)
def test_entry_points_reject_bad_params(bad):
    """Every entry point returns EINVAL for invalid options, before any HIP call
    (the pointers passed are NULL, so nothing could be launched anyway)."""
    L = lb.lib()
    qp = _qp(**bad)
    r = ctypes.byref(qp)
    assert L.lowbit_quantize_pack(None, 0, 100, r, None, None, None) == lb.EINVAL
    assert L.lowbit_unpack_dequant(None, None, 100, r, None, None) == lb.EINVAL
    assert L.lowbit_ef_compress(None, 0, None, 100, r, None, None, None) == lb.EINVAL
    assert L.lowbit_wdiff_compress(None, None, 0, 100, r, None, None, None) == lb.EINVAL
    assert L.lowbit_wdiff_apply(None, None, None, 100, r, None, 0, None) == lb.EINVAL
    good = _qp()
    assert L.lowbit_reduce_requant(None, None, 2, 100, r, ctypes.byref(good), None, None, None,
                                   None) == lb.EINVAL
    assert L.lowbit_reduce_requant(None, None, 2, 100, ctypes.byref(good), r, None, None, None,
                                   None) == lb.EINVAL
    assert L.lowbit_ef21_compress(None, 0, None, 100, r, None, None, None) == lb.EINVAL
    assert L.lowbit_hadamard_quantize_pack(None, 0, 128, r, None, None, None) == lb.EINVAL
    assert L.lowbit_hadamard_unpack_dequant(None, None, 128, r, None, None) == lb.EINVAL
    assert L.lowbit_reduce_requant_ef(None, None, 2, 100, r, ctypes.byref(good), None, None,
                                      None, None, None) == lb.EINVAL
    assert L.lowbit_reduce_requant_ef(None, None, 2, 100, ctypes.byref(good), r, None, None,
                                      None, None, None) == lb.EINVAL


def test_entry_points_reject_null_params_struct():
    L = lb.lib()
    assert L.lowbit_quantize_pack(None, 0, 100, None, None, None, None) == lb.EINVAL
    assert L.lowbit_unpack_dequant(None, None, 100, None, None, None) == lb.EINVAL


def test_null_pointers_and_negative_sizes():
    L = lb.lib()
    r = ctypes.byref(_qp())
    assert L.lowbit_quantize_pack(None, 0, 100, r, None, None, None) == lb.EINVAL
    assert L.lowbit_quantize_pack(None, 0, -1, r, None, None, None) == lb.EINVAL
    assert L.lowbit_quantize_pack(None, 7, 100, r, None, None, None) == lb.EINVAL   # dtype
    assert L.lowbit_ef_compress(None, 1, None, 100, r, None, None, None) == lb.EINVAL
    assert L.lowbit_copy_f32(None, None, 10, None) == lb.EINVAL
    assert L.lowbit_copy_f32(None, None, -10, None) == lb.EINVAL
    assert L.lowbit_fold_f32(None, 10, 4, None, None) == lb.EINVAL
    # memory-system probe: unknown op, a size that is not whole trips,
    # negative waves, null pointers
    assert L.lowbit_stream_probe_u32(3, None, None, 1024, 0, 0, 1, None) == lb.EINVAL
    assert L.lowbit_stream_probe_u32(0, None, None, 1000, 0, 0, 1, None) == lb.EINVAL
    assert L.lowbit_stream_probe_u32(1, None, None, 1024, 0, -1, 1, None) == lb.EINVAL
    assert L.lowbit_stream_probe_u32(1, None, None, 1024, 0, 0, 1, None) == lb.EINVAL
    assert L.lowbit_stream_probe_u32(2, None, None, 0, 0, 0, 1, None) == lb.OK
    assert L.lowbit_fold_f32(None, -1, 4, None, None) == lb.EINVAL
    assert L.lowbit_fold_f32(ctypes.c_void_p(0x1000), 10, 3, ctypes.c_void_p(0x2000), None) \
        == lb.EINVAL
    assert L.lowbit_fold_f32(ctypes.c_void_p(0x1008), 10, 4, ctypes.c_void_p(0x2000), None) \
        == lb.EINVAL
    assert L.lowbit_fold_f32(ctypes.c_void_p(0x1000), 10, 4, ctypes.c_void_p(0x2004), None) \
        == lb.EINVAL
    assert L.lowbit_fold_f32(None, 0, 4, None, None) == lb.OK
    streams = (ctypes.c_void_p * 2)(0x1000, 0x2000)
    sp = ctypes.cast(streams, ctypes.c_void_p)
    for ns in (0, -1, 17):
        assert L.lowbit_xor_streams_u32(sp, ns, 10, ctypes.c_void_p(0x3000), None) == lb.EINVAL
    assert L.lowbit_xor_streams_u32(sp, 2, -1, ctypes.c_void_p(0x3000), None) == lb.EINVAL
    assert L.lowbit_xor_streams_u32(None, 2, 10, ctypes.c_void_p(0x3000), None) == lb.EINVAL
    assert L.lowbit_xor_streams_u32(sp, 2, 10, None, None) == lb.EINVAL
    assert L.lowbit_xor_streams_u32(sp, 2, 10, ctypes.c_void_p(0x3002), None) == lb.EINVAL
    bad = (ctypes.c_void_p * 2)(0x1000, 0x2001)
    assert L.lowbit_xor_streams_u32(ctypes.cast(bad, ctypes.c_void_p), 2, 10,
                                    ctypes.c_void_p(0x3000), None) == lb.EINVAL
    nul = (ctypes.c_void_p * 2)(0x1000, None)
    assert L.lowbit_xor_streams_u32(ctypes.cast(nul, ctypes.c_void_p), 2, 10,
                                    ctypes.c_void_p(0x3000), None) == lb.EINVAL
    assert L.lowbit_xor_streams_u32(None, 1, 0, None, None) == lb.OK
    assert L.lowbit_add_inplace_f32(None, None, 10, None) == lb.EINVAL
    assert L.lowbit_add_inplace_f32(None, None, -1, None) == lb.EINVAL
    assert L.lowbit_add_inplace_f32(ctypes.c_void_p(0x1000), ctypes.c_void_p(0x2008), 10,
                                    None) == lb.EINVAL
    assert L.lowbit_add_inplace_f32(None, None, 0, None) == lb.OK


def test_misaligned_pointers_rejected():
    """Misaligned (never dereferenced) addresses are rejected on the host."""
    L = lb.lib()
    r = ctypes.byref(_qp())
    odd = ctypes.c_void_p(0x1008)        # 8-aligned, not 16-aligned
    ok4 = ctypes.c_void_p(0x2000)
    ok2 = ctypes.c_void_p(0x3000)
    assert L.lowbit_quantize_pack(odd, 0, 100, r, ok4, ok2, None) == lb.EINVAL
    assert L.lowbit_quantize_pack(ok4, 0, 100, r, ctypes.c_void_p(0x2002), ok2, None) == lb.EINVAL
    assert L.lowbit_quantize_pack(ok4, 0, 100, r, ok4, ctypes.c_void_p(0x3001), None) == lb.EINVAL
    assert L.lowbit_unpack_dequant(ok4, ok2, 100, r, odd, None) == lb.EINVAL


def test_zero_length_is_a_noop():
    L = lb.lib()
    r = ctypes.byref(_qp())
    assert L.lowbit_quantize_pack(None, 0, 0, r, None, None, None) == lb.OK
    assert L.lowbit_unpack_dequant(None, None, 0, r, None, None) == lb.OK
    assert L.lowbit_ef_compress(None, 0, None, 0, r, None, None, None) == lb.OK
    assert L.lowbit_wdiff_compress(None, None, 1, 0, r, None, None, None) == lb.OK
    assert L.lowbit_wdiff_apply(None, None, None, 0, r, None, 1, None) == lb.OK
    assert L.lowbit_reduce_requant(None, None, 1, 0, r, r, None, None, None, None) == lb.OK
    assert L.lowbit_reduce_requant_ef(None, None, 1, 0, r, r, None, None, None, None,
                                      None) == lb.OK
    assert L.lowbit_ef21_compress(None, 0, None, 0, r, None, None, None) == lb.OK
    assert L.lowbit_hadamard_quantize_pack(None, 0, 0, r, None, None, None) == lb.OK
    assert L.lowbit_hadamard_unpack_dequant(None, None, 0, r, None, None) == lb.OK


def test_hadamard_size_rules():
    L = lb.lib()
    # block sizes outside 32..4096 or not powers of two are rejected
    for B in (16, 96, 8192):
        bad = ctypes.byref(_qp(block_size=B))
        assert L.lowbit_hadamard_quantize_pack(None, 0, 256, bad, None, None, None) == lb.EINVAL
        assert L.lowbit_hadamard_unpack_dequant(None, None, 256, bad, None, None) == lb.EINVAL
    # any length, ragged or not, reaches the pointer checks (null -> EINVAL)
    # and n == 0 is a no-op
    r = ctypes.byref(_qp(block_size=128))
    for n in (200, 256, 4096 + 32):
        assert L.lowbit_hadamard_quantize_pack(None, 0, n, r, None, None, None) == lb.EINVAL
    assert L.lowbit_hadamard_quantize_pack(None, 0, 0, r, None, None, None) == lb.OK
    assert L.lowbit_copy_f32(None, None, 0, None) == lb.OK


def test_reduce_argument_rules():
    L = lb.lib()
    r = ctypes.byref(_qp())
    for npeers in [0, -1, 17, 100]:
        assert L.lowbit_reduce_requant(None, None, npeers, 10, r, r, None, None, None,
                                       None) == lb.EINVAL
        assert L.lowbit_reduce_requant_ef(None, None, npeers, 10, r, r, None, None, None,
                                          None, None) == lb.EINVAL
    # different block sizes are allowed: with NULL buffers the call reaches
    # the pointer checks
    other_block = ctypes.byref(_qp(block_size=256))
    assert L.lowbit_reduce_requant(None, None, 2, 10, r, other_block, None, None, None,
                                   None) == lb.EINVAL
    # bitwidth pairs: 8->4, 8->2, 4->2 are supported, the others are not
    for bi, bo in [(4, 8), (2, 4), (1, 2), (2, 1), (4, 1), (8, 1)]:
        qi, qo = ctypes.byref(_qp(bitwidth=bi)), ctypes.byref(_qp(bitwidth=bo))
        assert L.lowbit_reduce_requant(None, None, 2, 10, qi, qo, None, None, None,
                                       None) == lb.EUNSUPPORTED
        assert L.lowbit_reduce_requant_ef(None, None, 2, 10, qi, qo, None, None, None,
                                          None, None) == lb.EUNSUPPORTED
    for bi, bo in [(8, 4), (8, 2), (4, 2)]:
        qi, qo = ctypes.byref(_qp(bitwidth=bi)), ctypes.byref(_qp(bitwidth=bo))
        assert L.lowbit_reduce_requant(None, None, 2, 10, qi, qo, None, None, None,
                                       None) == lb.EINVAL
    # the stage-2 residual must be given
    ok = ctypes.c_void_p(0x4000)
    cp1 = (ctypes.c_void_p * 1)(ok)
    assert L.lowbit_reduce_requant_ef(ctypes.cast(cp1, ctypes.c_void_p),
                                      ctypes.cast(cp1, ctypes.c_void_p), 1, 10, r, r, None, ok,
                                      ok, None, None) == lb.EINVAL
    # mixed widths need peer codes aligned for the lane's vector load
    q8, q4 = ctypes.byref(_qp(bitwidth=8)), ctypes.byref(_qp(bitwidth=4))
    odd = (ctypes.c_void_p * 1)(ctypes.c_void_p(0x4004))
    assert L.lowbit_reduce_requant(ctypes.cast(odd, ctypes.c_void_p),
                                   ctypes.cast(cp1, ctypes.c_void_p), 1, 10, q8, q4, ok, ok,
                                   None, None) == lb.EINVAL
    # a NULL entry in the peer pointer arrays is rejected before launch
    ok = ctypes.c_void_p(0x4000)
    cp = (ctypes.c_void_p * 2)(ok, None)
    sp = (ctypes.c_void_p * 2)(ok, ok)
    assert L.lowbit_reduce_requant(ctypes.cast(cp, ctypes.c_void_p),
                                   ctypes.cast(sp, ctypes.c_void_p), 2, 10, r, r, ok, ok, None,
                                   None) == lb.EINVAL


def test_binding_rejects_host_tensors_and_bad_outputs():
    import torch
    x = torch.zeros(256)
    with pytest.raises(lb.LowbitError):
        lb.quantize_pack(x, 4, 128)
    with pytest.raises(lb.LowbitError):
        lb.quantize_pack(x, 3, 128)
    with pytest.raises(lb.LowbitError):      # undersized codes buffer
        lb.quantize_pack(x, 4, 128, codes=torch.zeros(3, dtype=torch.int32))
    with pytest.raises(lb.LowbitError):      # wrong scales dtype
        lb.quantize_pack(x, 4, 128, codes=torch.zeros(32, dtype=torch.int32),
                         scales=torch.zeros(2, dtype=torch.float32))
    with pytest.raises(lb.LowbitError):
        lb.unpack_dequant(torch.zeros(3, dtype=torch.int32), torch.zeros(2, dtype=torch.float16),
                          256, 4, 128)
