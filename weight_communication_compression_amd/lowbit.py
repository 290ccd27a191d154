"""Thin ctypes binding of liblowbit (the C ABI in ``include/lowbit.h``).

Argument marshalling only: every step of the codec runs in the gfx950 HIP
kernels behind the C ABI.  torch is used for device memory (tensors) and for
the current HIP stream.  If the library is missing or a call fails, a
``LowbitError`` is raised -- there is no CPU fallback.

Wire format of the returned tensors:
  codes  -- torch.int32 holding the packed uint32 words (bit patterns)
  scales -- torch.float16, one binary16 scale per block
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

__all__ = [
    "LowbitError", "lib", "library_path", "num_words", "num_blocks", "QParams",
    "quantize_pack", "unpack_dequant", "ef_compress", "reduce_requant",
    "wdiff_compress", "wdiff_apply", "copy_f32", "xor_streams", "add_inplace_f32", "fold_f32",
    "stream_probe", "PROBE_READ", "PROBE_WRITE", "PROBE_COPY",
    "OK", "EINVAL", "EUNSUPPORTED", "EDEVICE", "F32", "BF16", "HINT_INPUT_REUSED",
]

OK, EINVAL, EUNSUPPORTED, EDEVICE = 0, 1, 2, 3
PROBE_READ, PROBE_WRITE, PROBE_COPY = 0, 1, 2
F32, BF16 = 0, 1
HINT_INPUT_REUSED = 1        # lowbit_qparams.hints: the input is read again soon

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "liblowbit.so")


class LowbitError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        name = {1: "invalid argument", 2: "unsupported combination",
                3: "device launch error"}.get(status, f"status {status}")
        super().__init__(f"{what}: {name}")


class QParams(ctypes.Structure):
    """lowbit_qparams"""
    _fields_ = [("bitwidth", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("stochastic", ctypes.c_int32), ("hints", ctypes.c_int32),
                ("seed", ctypes.c_uint64), ("index_offset", ctypes.c_uint64)]


_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """Load liblowbit.so (built in-tree by ``build.py``); raise if absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise LowbitError(-1, f"{library_path} is not built (run __graft_entry__.build())")
        L = ctypes.CDLL(library_path)
        P, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        QP = ctypes.POINTER(QParams)
        sigs = {
            "lowbit_num_words": (i64, [i64, i32]),
            "lowbit_num_blocks": (i64, [i64, i32]),
            "lowbit_status_string": (ctypes.c_char_p, [ctypes.c_int]),
            "lowbit_version": (ctypes.c_char_p, []),
            "lowbit_quantize_pack": (ctypes.c_int, [P, ctypes.c_int, i64, QP, P, P, P]),
            "lowbit_unpack_dequant": (ctypes.c_int, [P, P, i64, QP, P, P]),
            "lowbit_ef_compress": (ctypes.c_int, [P, ctypes.c_int, P, i64, QP, P, P, P]),
            "lowbit_ef21_compress": (ctypes.c_int, [P, ctypes.c_int, P, i64, QP, P, P, P]),
            "lowbit_hadamard_quantize_pack": (ctypes.c_int, [P, ctypes.c_int, i64, QP, P, P, P]),
            "lowbit_hadamard_unpack_dequant": (ctypes.c_int, [P, P, i64, QP, P, P]),
            "lowbit_reduce_requant": (ctypes.c_int, [P, P, i32, i64, QP, QP, P, P, P, P]),
            "lowbit_reduce_requant_ef": (ctypes.c_int, [P, P, i32, i64, QP, QP, P, P, P, P, P]),
            "lowbit_wdiff_compress": (ctypes.c_int, [P, P, ctypes.c_int, i64, QP, P, P, P]),
            "lowbit_wdiff_apply": (ctypes.c_int, [P, P, P, i64, QP, P, ctypes.c_int, P]),
            "lowbit_copy_f32": (ctypes.c_int, [P, P, i64, P]),
            "lowbit_xor_streams_u32": (ctypes.c_int, [P, i32, i64, P, P]),
            "lowbit_add_inplace_f32": (ctypes.c_int, [P, P, i64, P]),
            "lowbit_fold_f32": (ctypes.c_int, [P, i64, i32, P, P]),
            "lowbit_stream_probe_u32": (ctypes.c_int, [i32, P, P, i64, ctypes.c_uint32, i32, i32, P]),
        }
        for name, (res, args) in sigs.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def num_words(n: int, bitwidth: int) -> int:
    v = lib().lowbit_num_words(n, bitwidth)
    if v < 0:
        raise LowbitError(EINVAL, "num_words")
    return int(v)


def num_blocks(n: int, block_size: int) -> int:
    v = lib().lowbit_num_blocks(n, block_size)
    if v < 0:
        raise LowbitError(EINVAL, "num_blocks")
    return int(v)


# ------------------------------------------------------------ marshalling --
def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise LowbitError(EINVAL, f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _dev(t: torch.Tensor, what: str) -> int:
    if not t.is_cuda:
        raise LowbitError(EINVAL, f"{what} must be a GPU tensor")
    if not t.is_contiguous():
        raise LowbitError(EINVAL, f"{what} must be contiguous")
    return t.data_ptr()


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _qp(bitwidth, block_size, stochastic=False, seed=0, index_offset=0, hints=0) -> QParams:
    return QParams(int(bitwidth), int(block_size), int(bool(stochastic)), int(hints),
                   int(seed) & (2 ** 64 - 1), int(index_offset))


def _check(status: int, what: str) -> None:
    if status != OK:
        raise LowbitError(status, what)


def _need_codes(t: torch.Tensor, n: int, bitwidth: int, what: str) -> None:
    if t.dtype != torch.int32 or t.numel() < num_words(n, bitwidth):
        raise LowbitError(EINVAL, f"{what} must be int32 with >= {num_words(n, bitwidth)} words")


def _need_scales(t: torch.Tensor, n: int, block_size: int, what: str) -> None:
    if t.dtype != torch.float16 or t.numel() < num_blocks(n, block_size):
        raise LowbitError(EINVAL,
                          f"{what} must be float16 with >= {num_blocks(n, block_size)} entries")


def _out_codes(n, bitwidth, like, codes):
    if codes is None:
        codes = torch.empty(num_words(n, bitwidth), dtype=torch.int32, device=like.device)
    _need_codes(codes, n, bitwidth, "codes")
    return codes


def _out_scales(n, block_size, like, scales):
    if scales is None:
        scales = torch.empty(num_blocks(n, block_size), dtype=torch.float16, device=like.device)
    _need_scales(scales, n, block_size, "scales")
    return scales


# -------------------------------------------------------------- the codec --
def quantize_pack(x: torch.Tensor, bitwidth: int, block_size: int, stochastic: bool = False,
                  seed: int = 0, index_offset: int = 0, codes: Optional[torch.Tensor] = None,
                  scales: Optional[torch.Tensor] = None, input_reused: bool = False):
    """Compress x (float32 or bfloat16) -> (codes int32[num_words], scales float16[num_blocks]).

    input_reused: the caller reads x again soon (LOWBIT_HINT_INPUT_REUSED), so
    it is kept in the caches rather than streamed."""
    n = x.numel()
    codes = _out_codes(n, bitwidth, x, codes)
    scales = _out_scales(n, block_size, x, scales)
    qp = _qp(bitwidth, block_size, stochastic, seed, index_offset,
             HINT_INPUT_REUSED if input_reused else 0)
    _check(lib().lowbit_quantize_pack(_dev(x, "x"), _dtype_code(x), n, ctypes.byref(qp),
                                      _dev(codes, "codes"), _dev(scales, "scales"), _stream(x)),
           "lowbit_quantize_pack")
    return codes, scales


def unpack_dequant(codes: torch.Tensor, scales: torch.Tensor, n: int, bitwidth: int,
                   block_size: int, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Decompress -> float32[n]."""
    _need_codes(codes, n, bitwidth, "codes")
    _need_scales(scales, n, block_size, "scales")
    if out is None:
        out = torch.empty(n, dtype=torch.float32, device=codes.device)
    if out.dtype != torch.float32 or out.numel() < n:
        raise LowbitError(EINVAL, "out must be float32 with >= n elements")
    qp = _qp(bitwidth, block_size)
    _check(lib().lowbit_unpack_dequant(_dev(codes, "codes"), _dev(scales, "scales"), n,
                                       ctypes.byref(qp), _dev(out, "out"), _stream(codes)),
           "lowbit_unpack_dequant")
    return out


def hadamard_quantize_pack(x: torch.Tensor, bitwidth: int, block_size: int,
                           stochastic: bool = False, seed: int = 0, index_offset: int = 0,
                           codes: Optional[torch.Tensor] = None,
                           scales: Optional[torch.Tensor] = None, input_reused: bool = False):
    """Blockwise Walsh-Hadamard transform of x, then compress; a partial last
    block (x.numel() not a multiple of block_size) is compressed untransformed.

    input_reused: as for quantize_pack (LOWBIT_HINT_INPUT_REUSED)."""
    n = x.numel()
    codes = _out_codes(n, bitwidth, x, codes)
    scales = _out_scales(n, block_size, x, scales)
    qp = _qp(bitwidth, block_size, stochastic, seed, index_offset,
             HINT_INPUT_REUSED if input_reused else 0)
    _check(lib().lowbit_hadamard_quantize_pack(_dev(x, "x"), _dtype_code(x), n, ctypes.byref(qp),
                                               _dev(codes, "codes"), _dev(scales, "scales"),
                                               _stream(x)), "lowbit_hadamard_quantize_pack")
    return codes, scales


def hadamard_unpack_dequant(codes: torch.Tensor, scales: torch.Tensor, n: int, bitwidth: int,
                            block_size: int, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Decompress, then the inverse blockwise transform -> float32[n]."""
    _need_codes(codes, n, bitwidth, "codes")
    _need_scales(scales, n, block_size, "scales")
    if out is None:
        out = torch.empty(n, dtype=torch.float32, device=codes.device)
    if out.dtype != torch.float32 or out.numel() < n:
        raise LowbitError(EINVAL, "out must be float32 with >= n elements")
    qp = _qp(bitwidth, block_size)
    _check(lib().lowbit_hadamard_unpack_dequant(_dev(codes, "codes"), _dev(scales, "scales"), n,
                                                ctypes.byref(qp), _dev(out, "out"),
                                                _stream(codes)), "lowbit_hadamard_unpack_dequant")
    return out


def ef_compress(g: torch.Tensor, residual: torch.Tensor, bitwidth: int, block_size: int,
                stochastic: bool = False, seed: int = 0, index_offset: int = 0,
                codes: Optional[torch.Tensor] = None, scales: Optional[torch.Tensor] = None):
    """Error-feedback compress; `residual` (float32[n]) is updated in place."""
    n = g.numel()
    if residual.dtype != torch.float32 or residual.numel() != n:
        raise LowbitError(EINVAL, "residual must be float32 with g.numel() elements")
    codes = _out_codes(n, bitwidth, g, codes)
    scales = _out_scales(n, block_size, g, scales)
    qp = _qp(bitwidth, block_size, stochastic, seed, index_offset)
    _check(lib().lowbit_ef_compress(_dev(g, "g"), _dtype_code(g), _dev(residual, "residual"), n,
                                    ctypes.byref(qp), _dev(codes, "codes"),
                                    _dev(scales, "scales"), _stream(g)), "lowbit_ef_compress")
    return codes, scales


def ef21_compress(g: torch.Tensor, state: torch.Tensor, bitwidth: int, block_size: int,
                  stochastic: bool = False, seed: int = 0, index_offset: int = 0,
                  codes: Optional[torch.Tensor] = None, scales: Optional[torch.Tensor] = None):
    """EF21 compress of g - state; `state` (float32[n]) becomes state + deq, in place."""
    n = g.numel()
    if state.dtype != torch.float32 or state.numel() != n:
        raise LowbitError(EINVAL, "state must be float32 with g.numel() elements")
    codes = _out_codes(n, bitwidth, g, codes)
    scales = _out_scales(n, block_size, g, scales)
    qp = _qp(bitwidth, block_size, stochastic, seed, index_offset)
    _check(lib().lowbit_ef21_compress(_dev(g, "g"), _dtype_code(g), _dev(state, "state"), n,
                                      ctypes.byref(qp), _dev(codes, "codes"),
                                      _dev(scales, "scales"), _stream(g)), "lowbit_ef21_compress")
    return codes, scales


def _reduce(peer_codes, peer_scales, n, bitwidth, block_size, stochastic, seed, index_offset,
            out_codes, out_scales, out_sum, want_sum, out_bitwidth, out_block_size, residual,
            input_reused=False):
    P = len(peer_codes)
    if P != len(peer_scales):
        raise LowbitError(EINVAL, "peer_codes and peer_scales differ in length")
    if P < 1:
        raise LowbitError(EINVAL, "reduce_requant needs at least one peer")
    ob = bitwidth if out_bitwidth is None else out_bitwidth
    oB = block_size if out_block_size is None else out_block_size
    for c, sc in zip(peer_codes, peer_scales):
        _need_codes(c, n, bitwidth, "peer codes")
        _need_scales(sc, n, block_size, "peer scales")
    like = peer_codes[0]
    out_codes = _out_codes(n, ob, like, out_codes)
    out_scales = _out_scales(n, oB, like, out_scales)
    if want_sum and out_sum is None:
        out_sum = torch.empty(n, dtype=torch.float32, device=like.device)
    if out_sum is not None and (out_sum.dtype != torch.float32 or out_sum.numel() < n):
        raise LowbitError(EINVAL, "out_sum must be float32 with >= n elements")
    cp = (ctypes.c_void_p * P)(*[_dev(c, "peer codes") for c in peer_codes])
    sp = (ctypes.c_void_p * P)(*[_dev(s, "peer scales") for s in peer_scales])
    qi = _qp(bitwidth, block_size, hints=HINT_INPUT_REUSED if input_reused else 0)
    qo = _qp(ob, oB, stochastic, seed, index_offset)
    tail = (_dev(out_codes, "out_codes"), _dev(out_scales, "out_scales"),
            _dev(out_sum, "out_sum") if out_sum is not None else None, _stream(like))
    if residual is None:
        _check(lib().lowbit_reduce_requant(ctypes.cast(cp, ctypes.c_void_p),
                                           ctypes.cast(sp, ctypes.c_void_p), P, n,
                                           ctypes.byref(qi), ctypes.byref(qo), *tail),
               "lowbit_reduce_requant")
    else:
        if residual.dtype != torch.float32 or residual.numel() != n:
            raise LowbitError(EINVAL, "residual must be float32 with n elements")
        _check(lib().lowbit_reduce_requant_ef(ctypes.cast(cp, ctypes.c_void_p),
                                              ctypes.cast(sp, ctypes.c_void_p), P, n,
                                              ctypes.byref(qi), ctypes.byref(qo),
                                              _dev(residual, "residual"), *tail),
               "lowbit_reduce_requant_ef")
    return out_codes, out_scales, out_sum


def reduce_requant(peer_codes: Sequence[torch.Tensor], peer_scales: Sequence[torch.Tensor],
                   n: int, bitwidth: int, block_size: int, stochastic: bool = False,
                   seed: int = 0, index_offset: int = 0, out_codes=None, out_scales=None,
                   out_sum=None, want_sum: bool = False, out_bitwidth: Optional[int] = None,
                   out_block_size: Optional[int] = None, input_reused: bool = False):
    """Local reduce: dequantize npeers chunks packed with (bitwidth,
    block_size), sum in peer order, requantize with (out_bitwidth,
    out_block_size) (default: the same) and the rounding options.
    input_reused: the caller reads the peers' codes again soon
    (LOWBIT_HINT_INPUT_REUSED), so they are not streamed; results are the same.

    Returns (codes, scales, sum_or_None)."""
    return _reduce(peer_codes, peer_scales, n, bitwidth, block_size, stochastic, seed,
                   index_offset, out_codes, out_scales, out_sum, want_sum, out_bitwidth,
                   out_block_size, None, input_reused)


def reduce_requant_ef(peer_codes: Sequence[torch.Tensor], peer_scales: Sequence[torch.Tensor],
                      n: int, bitwidth: int, block_size: int, residual: torch.Tensor,
                      stochastic: bool = False, seed: int = 0, index_offset: int = 0,
                      out_codes=None, out_scales=None, out_sum=None, want_sum: bool = False,
                      out_bitwidth: Optional[int] = None, out_block_size: Optional[int] = None,
                      input_reused: bool = False):
    """Local reduce with stage-2 error feedback: the sum plus `residual`
    (float32[n], updated in place) is requantized.  Returns (codes, scales,
    sum_or_None); the sum is taken before the residual is added.
    input_reused: as for reduce_requant."""
    if residual is None:
        raise LowbitError(EINVAL, "reduce_requant_ef needs a residual")
    return _reduce(peer_codes, peer_scales, n, bitwidth, block_size, stochastic, seed,
                   index_offset, out_codes, out_scales, out_sum, want_sum, out_bitwidth,
                   out_block_size, residual, input_reused)


def wdiff_compress(w_new: torch.Tensor, w_old: torch.Tensor, bitwidth: int, block_size: int,
                   stochastic: bool = False, seed: int = 0, index_offset: int = 0,
                   codes=None, scales=None):
    """Compress the weight difference w_new - w_old."""
    n = w_new.numel()
    if w_old.dtype != w_new.dtype or w_old.numel() != n:
        raise LowbitError(EINVAL, "w_new and w_old must match in dtype and size")
    codes = _out_codes(n, bitwidth, w_new, codes)
    scales = _out_scales(n, block_size, w_new, scales)
    qp = _qp(bitwidth, block_size, stochastic, seed, index_offset)
    _check(lib().lowbit_wdiff_compress(_dev(w_new, "w_new"), _dev(w_old, "w_old"),
                                       _dtype_code(w_new), n, ctypes.byref(qp),
                                       _dev(codes, "codes"), _dev(scales, "scales"),
                                       _stream(w_new)), "lowbit_wdiff_compress")
    return codes, scales


def wdiff_apply(w_old: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor, bitwidth: int,
                block_size: int, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """w_out = w_old + deq (rounded to w_old's dtype); `out` may be w_old itself."""
    n = w_old.numel()
    _need_codes(codes, n, bitwidth, "codes")
    _need_scales(scales, n, block_size, "scales")
    if out is None:
        out = torch.empty_like(w_old)
    if out.dtype != w_old.dtype or out.numel() != n:
        raise LowbitError(EINVAL, "out must match w_old")
    qp = _qp(bitwidth, block_size)
    _check(lib().lowbit_wdiff_apply(_dev(w_old, "w_old"), _dev(codes, "codes"),
                                    _dev(scales, "scales"), n, ctypes.byref(qp),
                                    _dev(out, "out"), _dtype_code(w_old), _stream(w_old)),
           "lowbit_wdiff_apply")
    return out


def copy_f32(x: torch.Tensor, y: torch.Tensor) -> torch.Tensor:
    """Plain float32 copy kernel (bandwidth reference, not a codec step)."""
    if x.dtype != torch.float32 or y.dtype != torch.float32 or y.numel() != x.numel():
        raise LowbitError(EINVAL, "copy_f32 needs two float32 tensors of equal size")
    _check(lib().lowbit_copy_f32(_dev(x, "x"), _dev(y, "y"), x.numel(), _stream(x)),
           "lowbit_copy_f32")
    return y


def add_inplace_f32(x: torch.Tensor, y: torch.Tensor) -> torch.Tensor:
    """y += x in place (float32), with the error-feedback compress's access
    pattern (bandwidth reference for that kernel, not a codec step)."""
    if x.dtype != torch.float32 or y.dtype != torch.float32 or y.numel() != x.numel():
        raise LowbitError(EINVAL, "add_inplace_f32 needs two float32 tensors of equal size")
    _check(lib().lowbit_add_inplace_f32(_dev(x, "x"), _dev(y, "y"), x.numel(), _stream(y)),
           "lowbit_add_inplace_f32")
    return y


def xor_streams(streams: Sequence[torch.Tensor], out: torch.Tensor) -> torch.Tensor:
    """out = XOR of the int32 streams, read with the local reduce's access
    pattern (bandwidth reference for the reduce, not a codec step)."""
    P = len(streams)
    n = out.numel()
    if out.dtype != torch.int32 or any(t.dtype != torch.int32 or t.numel() != n for t in streams):
        raise LowbitError(EINVAL, "xor_streams needs int32 tensors of equal size")
    if not 1 <= P <= 16:
        raise LowbitError(EINVAL, "xor_streams needs 1 to 16 streams")
    sp = (ctypes.c_void_p * P)(*[_dev(t, "stream") for t in streams])
    _check(lib().lowbit_xor_streams_u32(ctypes.cast(sp, ctypes.c_void_p), P, n, _dev(out, "out"),
                                        _stream(out)), "lowbit_xor_streams_u32")
    return out


def fold_f32(x: torch.Tensor, bitwidth: int, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Compress-volume bandwidth reference (not a codec step): reads the
    float32 x, writes num_words(x.numel(), bitwidth) int32 words of XOR folds."""
    if x.dtype != torch.float32:
        raise LowbitError(EINVAL, "fold_f32 needs a float32 tensor")
    n = x.numel()
    nw = num_words(n, bitwidth)
    if out is None:
        out = torch.empty(nw, dtype=torch.int32, device=x.device)
    elif out.dtype != torch.int32 or out.numel() < nw:
        raise LowbitError(EINVAL, f"out must be int32 with >= {nw} words")
    _check(lib().lowbit_fold_f32(_dev(x, "x"), n, int(bitwidth), _dev(out, "out"), _stream(x)),
           "lowbit_fold_f32")
    return out


def stream_probe(op: int, dst: torch.Tensor, src: Optional[torch.Tensor] = None, value: int = 0,
                 waves: int = 0, nontemporal: bool = True) -> torch.Tensor:
    """Memory-system probe (not a codec step), on int32 tensors viewed as
    32-bit words: PROBE_READ writes dst[t] = XOR of trip t (1024 words) of
    src, PROBE_WRITE dst[i] = i ^ value, PROBE_COPY dst = src.  waves = 0:
    one trip per wave; > 0: a persistent grid of that many waves."""
    nwords = src.numel() if op != PROBE_WRITE else dst.numel()
    for t, name in ((dst, "dst"), (src, "src")):
        if t is not None and t.dtype != torch.int32:
            raise LowbitError(EINVAL, f"{name} must be int32")
    if op == PROBE_READ and dst.numel() < nwords // 1024:
        raise LowbitError(EINVAL, "dst too small")
    if op == PROBE_COPY and dst.numel() < nwords:
        raise LowbitError(EINVAL, "dst too small")
    sp = _dev(src, "src") if src is not None else None
    _check(lib().lowbit_stream_probe_u32(int(op), sp, _dev(dst, "dst"), nwords,
                                         int(value) & 0xFFFFFFFF, int(waves), int(bool(nontemporal)),
                                         _stream(dst)), "lowbit_stream_probe_u32")
    return dst
