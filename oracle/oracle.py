"""numpy front end of the C oracle (``lowbit_oracle.c``) -- TEST INFRASTRUCTURE ONLY.

Every function takes and returns host numpy arrays and runs the plain scalar C
code one block at a time.  Nothing here touches a GPU and nothing here is used
by the product path.

Data conventions (the same wire format the method defines):
  * ``codes``  -- uint32 words, codes packed LSB-first by global element index;
  * ``scales`` -- uint16 holding binary16 bit patterns, one per block;
  * bfloat16 tensors are passed as uint16 bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

__all__ = [
    "build_oracle", "lib",
    "f16_to_f32", "f32_to_f16_rne", "f16_round_up", "bf16_to_f32", "f32_to_bf16_rne",
    "fmix32", "sr_key", "sr_bits", "sr_uniform",
    "num_words", "num_blocks", "pack_codes", "unpack_codes",
    "quantize_pack", "unpack_dequant", "ef_compress", "reduce_requant", "reduce_requant_ex",
    "ef21_compress", "hadamard_quantize_pack", "hadamard_unpack_dequant", "hadamard_blocks",
    "wdiff_compress", "wdiff_apply",
    "F32", "BF16",
]

F32 = 0
BF16 = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lowbit_oracle.c")
_LIB = os.path.join(_HERE, "liblowbit_oracle.so")
# A test of the pins themselves may point the wrapper at a deliberately
# broken build of the oracle (planted mistakes, CPU only).
_LIB_OVERRIDE = os.environ.get("LOWBIT_ORACLE_LIB")

# -ffp-contract=off: no fused multiply-add; -fexcess-precision=standard and
# SSE arithmetic (x86-64 default): every binary32 operation rounds once.
CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
          "-fexcess-precision=standard", "-fPIC", "-shared"]


def build_oracle(force: bool = False) -> str:
    """Compile the C oracle with gcc into ``oracle/liblowbit_oracle.so``."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        path = _LIB_OVERRIDE or _LIB
        if not _LIB_OVERRIDE and not os.path.exists(_LIB):
            build_oracle()
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i32, i64, u64, u32, u16 = (ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64,
                                   ctypes.c_uint32, ctypes.c_uint16)
        sig = {
            "oracle_f16_to_f32": (ctypes.c_float, [u16]),
            "oracle_f32_to_f16_rne": (u16, [ctypes.c_float]),
            "oracle_f16_round_up": (u16, [ctypes.c_float]),
            "oracle_bf16_to_f32": (ctypes.c_float, [u16]),
            "oracle_f32_to_bf16_rne": (u16, [ctypes.c_float]),
            "oracle_fmix32": (u32, [u32]),
            "oracle_sr_key": (u32, [u64]),
            "oracle_sr_bits": (u32, [u64, u64]),
            "oracle_sr_uniform": (ctypes.c_float, [u64, u64]),
            "oracle_num_words": (i64, [i64, i32]),
            "oracle_num_blocks": (i64, [i64, i32]),
            "oracle_pack_codes": (ctypes.c_int, [P, i64, i32, P]),
            "oracle_unpack_codes": (ctypes.c_int, [P, i64, i32, P]),
            "oracle_quantize_pack": (ctypes.c_int, [P, i32, i64, i32, i32, i32, u64, u64, P, P]),
            "oracle_unpack_dequant": (ctypes.c_int, [P, P, i64, i32, i32, P]),
            "oracle_ef_compress": (ctypes.c_int, [P, i32, P, i64, i32, i32, i32, u64, u64, P, P]),
            "oracle_reduce_requant": (ctypes.c_int, [P, P, i32, i64, i32, i32, i32, i32, u64, u64,
                                                     P, P, P]),
            "oracle_reduce_requant_ex": (ctypes.c_int, [P, P, i32, i64, i32, i32, i32, i32, i32,
                                                        u64, u64, P, P, P, P]),
            "oracle_ef21_compress": (ctypes.c_int, [P, i32, P, i64, i32, i32, i32, u64, u64, P, P]),
            "oracle_hadamard_quantize_pack": (ctypes.c_int, [P, i32, i64, i32, i32, i32, u64, u64,
                                                             P, P]),
            "oracle_hadamard_unpack_dequant": (ctypes.c_int, [P, P, i64, i32, i32, P]),
            "oracle_hadamard_blocks": (ctypes.c_int, [P, i64, i32, i32]),
            "oracle_wdiff_compress": (ctypes.c_int, [P, P, i32, i64, i32, i32, i32, u64, u64, P, P]),
            "oracle_wdiff_apply": (ctypes.c_int, [P, P, P, i64, i32, i32, P, i32]),
            "oracle_f32_to_f16_rne_array": (None, [P, i64, P]),
            "oracle_f16_round_up_array": (None, [P, i64, P]),
            "oracle_f16_to_f32_array": (None, [P, i64, P]),
            "oracle_f32_to_bf16_rne_array": (None, [P, i64, P]),
            "oracle_sr_uniform_array": (None, [u64, u64, i64, P]),
            "oracle_fmix32_array": (None, [P, i64, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise ValueError(f"oracle {what}: invalid arguments (status {rc})")


# ---------------------------------------------------------------- scalars --
def f16_to_f32(h) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, np.float32)
    lib().oracle_f16_to_f32_array(_ptr(h), h.size, _ptr(out))
    return out


def f32_to_f16_rne(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().oracle_f32_to_f16_rne_array(_ptr(x), x.size, _ptr(out))
    return out


def f16_round_up(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().oracle_f16_round_up_array(_ptr(x), x.size, _ptr(out))
    return out


def bf16_to_f32(h) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    return (h.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_rne(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().oracle_f32_to_bf16_rne_array(_ptr(x), x.size, _ptr(out))
    return out


def fmix32(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.uint32)
    out = np.empty(x.shape, np.uint32)
    lib().oracle_fmix32_array(_ptr(x), x.size, _ptr(out))
    return out


def sr_key(seed: int) -> int:
    return int(lib().oracle_sr_key(seed))


def sr_bits(seed: int, i: int) -> int:
    return int(lib().oracle_sr_bits(seed, i))


def sr_uniform(seed: int, i0: int, n: int) -> np.ndarray:
    out = np.empty(n, np.float32)
    lib().oracle_sr_uniform_array(seed, i0, n, _ptr(out))
    return out


# ---------------------------------------------------------------- packing --
def num_words(n: int, bits: int) -> int:
    return int(lib().oracle_num_words(n, bits))


def num_blocks(n: int, block: int) -> int:
    return int(lib().oracle_num_blocks(n, block))


def pack_codes(u, bits: int) -> np.ndarray:
    u = np.ascontiguousarray(u, dtype=np.uint32)
    words = np.empty(max(num_words(u.size, bits), 0), np.uint32)
    _check(lib().oracle_pack_codes(_ptr(u), u.size, bits, _ptr(words)), "pack_codes")
    return words


def unpack_codes(words, n: int, bits: int) -> np.ndarray:
    words = np.ascontiguousarray(words, dtype=np.uint32)
    u = np.empty(n, np.uint32)
    _check(lib().oracle_unpack_codes(_ptr(words), n, bits, _ptr(u)), "unpack_codes")
    return u


# ------------------------------------------------------------- the method --
def _as_input(x):
    """float32 -> (F32, array); uint16 (bfloat16 bits) -> (BF16, array)."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.float32:
        return F32, x
    if x.dtype == np.uint16:
        return BF16, x
    raise TypeError("oracle inputs are float32 or uint16 (bfloat16 bits)")


def quantize_pack(x, bits: int, block: int, stochastic: bool = False, seed: int = 0,
                  index_offset: int = 0):
    """x -> (codes uint32[num_words], scales uint16[num_blocks])."""
    dt, x = _as_input(x)
    n = x.size
    codes = np.empty(num_words(n, bits), np.uint32)
    scales = np.empty(num_blocks(n, block), np.uint16)
    _check(lib().oracle_quantize_pack(_ptr(x), dt, n, bits, block, int(stochastic), seed,
                                      index_offset, _ptr(codes), _ptr(scales)), "quantize_pack")
    return codes, scales


def unpack_dequant(codes, scales, n: int, bits: int, block: int) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint32)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    y = np.empty(n, np.float32)
    _check(lib().oracle_unpack_dequant(_ptr(codes), _ptr(scales), n, bits, block, _ptr(y)),
           "unpack_dequant")
    return y


def ef_compress(g, residual, bits: int, block: int, stochastic: bool = False, seed: int = 0,
                index_offset: int = 0):
    """Returns (codes, scales, new_residual); the input residual is not modified."""
    dt, g = _as_input(g)
    n = g.size
    e = np.array(residual, dtype=np.float32, copy=True)
    assert e.size == n
    codes = np.empty(num_words(n, bits), np.uint32)
    scales = np.empty(num_blocks(n, block), np.uint16)
    _check(lib().oracle_ef_compress(_ptr(g), dt, _ptr(e), n, bits, block, int(stochastic), seed,
                                    index_offset, _ptr(codes), _ptr(scales)), "ef_compress")
    return codes, scales, e


def reduce_requant(peer_codes, peer_scales, n: int, in_bits: int, block: int, out_bits: int,
                   out_stochastic: bool = False, out_seed: int = 0, out_index_offset: int = 0,
                   want_sum: bool = False):
    """Returns (codes, scales, sum_or_None)."""
    P = len(peer_codes)
    pc = [np.ascontiguousarray(c, dtype=np.uint32) for c in peer_codes]
    ps = [np.ascontiguousarray(s, dtype=np.uint16) for s in peer_scales]
    cp = (ctypes.c_void_p * max(P, 1))(*[_ptr(c) for c in pc])
    sp = (ctypes.c_void_p * max(P, 1))(*[_ptr(s) for s in ps])
    codes = np.empty(num_words(n, out_bits), np.uint32)
    scales = np.empty(num_blocks(n, block), np.uint16)
    total = np.empty(n, np.float32) if want_sum else None
    _check(lib().oracle_reduce_requant(ctypes.cast(cp, ctypes.c_void_p),
                                       ctypes.cast(sp, ctypes.c_void_p), P, n, in_bits, block,
                                       out_bits, int(out_stochastic), out_seed, out_index_offset,
                                       _ptr(codes), _ptr(scales),
                                       _ptr(total) if want_sum else None), "reduce_requant")
    return codes, scales, total


def reduce_requant_ex(peer_codes, peer_scales, n: int, in_bits: int, in_block: int,
                      out_bits: int, out_block: int, out_stochastic: bool = False,
                      out_seed: int = 0, out_index_offset: int = 0, residual=None,
                      want_sum: bool = False):
    """General local reduce: separate input/output widths and block sizes and
    an optional stage-2 residual.  Returns (codes, scales, sum_or_None,
    new_residual_or_None); the input residual is not modified."""
    P = len(peer_codes)
    pc = [np.ascontiguousarray(c, dtype=np.uint32) for c in peer_codes]
    ps = [np.ascontiguousarray(s, dtype=np.uint16) for s in peer_scales]
    cp = (ctypes.c_void_p * max(P, 1))(*[_ptr(c) for c in pc])
    sp = (ctypes.c_void_p * max(P, 1))(*[_ptr(s) for s in ps])
    codes = np.empty(num_words(n, out_bits), np.uint32)
    scales = np.empty(num_blocks(n, out_block), np.uint16)
    total = np.empty(n, np.float32) if want_sum else None
    e = None
    if residual is not None:
        e = np.array(residual, dtype=np.float32, copy=True)
        assert e.size == n
    _check(lib().oracle_reduce_requant_ex(ctypes.cast(cp, ctypes.c_void_p),
                                          ctypes.cast(sp, ctypes.c_void_p), P, n, in_bits,
                                          in_block, out_bits, out_block, int(out_stochastic),
                                          out_seed, out_index_offset,
                                          _ptr(e) if e is not None else None, _ptr(codes),
                                          _ptr(scales), _ptr(total) if want_sum else None),
           "reduce_requant_ex")
    return codes, scales, total, e


def ef21_compress(g, state, bits: int, block: int, stochastic: bool = False, seed: int = 0,
                  index_offset: int = 0):
    """Returns (codes, scales, new_state); the input state is not modified."""
    dt, g = _as_input(g)
    n = g.size
    h = np.array(state, dtype=np.float32, copy=True)
    assert h.size == n
    codes = np.empty(num_words(n, bits), np.uint32)
    scales = np.empty(num_blocks(n, block), np.uint16)
    _check(lib().oracle_ef21_compress(_ptr(g), dt, _ptr(h), n, bits, block, int(stochastic),
                                      seed, index_offset, _ptr(codes), _ptr(scales)),
           "ef21_compress")
    return codes, scales, h


def hadamard_quantize_pack(x, bits: int, block: int, stochastic: bool = False, seed: int = 0,
                           index_offset: int = 0):
    """Blockwise Hadamard transform, then compress (a partial last block is
    compressed untransformed).  Returns (codes, scales)."""
    dt, x = _as_input(x)
    n = x.size
    codes = np.empty(num_words(n, bits), np.uint32)
    scales = np.empty(num_blocks(n, block), np.uint16)
    _check(lib().oracle_hadamard_quantize_pack(_ptr(x), dt, n, bits, block, int(stochastic),
                                               seed, index_offset, _ptr(codes), _ptr(scales)),
           "hadamard_quantize_pack")
    return codes, scales


def hadamard_unpack_dequant(codes, scales, n: int, bits: int, block: int) -> np.ndarray:
    """Decompress, then the inverse blockwise Hadamard transform (not on a
    partial last block)."""
    codes = np.ascontiguousarray(codes, dtype=np.uint32)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    y = np.empty(n, np.float32)
    _check(lib().oracle_hadamard_unpack_dequant(_ptr(codes), _ptr(scales), n, bits, block,
                                                _ptr(y)), "hadamard_unpack_dequant")
    return y


def hadamard_blocks(x, block: int, inverse: bool = False) -> np.ndarray:
    """The scaled blockwise transform alone on a copy of x (whole blocks; a
    partial last block is left as it is)."""
    y = np.array(x, dtype=np.float32, copy=True)
    _check(lib().oracle_hadamard_blocks(_ptr(y), y.size, block, int(inverse)), "hadamard_blocks")
    return y


def wdiff_compress(w_new, w_old, bits: int, block: int, stochastic: bool = False, seed: int = 0,
                   index_offset: int = 0):
    dt, w_new = _as_input(w_new)
    dt2, w_old = _as_input(w_old)
    assert dt == dt2 and w_new.size == w_old.size
    n = w_new.size
    codes = np.empty(num_words(n, bits), np.uint32)
    scales = np.empty(num_blocks(n, block), np.uint16)
    _check(lib().oracle_wdiff_compress(_ptr(w_new), _ptr(w_old), dt, n, bits, block,
                                       int(stochastic), seed, index_offset, _ptr(codes),
                                       _ptr(scales)), "wdiff_compress")
    return codes, scales


def wdiff_apply(w_old, codes, scales, bits: int, block: int) -> np.ndarray:
    dt, w_old = _as_input(w_old)
    n = w_old.size
    codes = np.ascontiguousarray(codes, dtype=np.uint32)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    out = np.empty(n, w_old.dtype)
    _check(lib().oracle_wdiff_apply(_ptr(w_old), _ptr(codes), _ptr(scales), n, bits, block,
                                    _ptr(out), dt), "wdiff_apply")
    return out
