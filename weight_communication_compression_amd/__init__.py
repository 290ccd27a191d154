"""MI355X-native blockwise low-bit compression of training communication buffers.

The codec (compress, decompress, error-feedback and EF21 compress, local
reduce + requantize with optional stage-2 error feedback and fewer output bits,
Hadamard-smoothed compress/decompress, weight-difference compress/apply) runs in hand-written gfx950 HIP
kernels behind the C ABI of ``liblowbit.so`` (declared in ``include/lowbit.h``);
``lowbit`` is its thin Python binding.  ``synth`` holds the seeded synthetic
input recipes.
"""
from .lowbit import (  # noqa: F401
    LowbitError, QParams, add_inplace_f32, copy_f32, ef21_compress, ef_compress,
    hadamard_quantize_pack, hadamard_unpack_dequant, lib, library_path, num_blocks, num_words,
    quantize_pack, reduce_requant, reduce_requant_ef, unpack_dequant, wdiff_apply, wdiff_compress,
    xor_streams,
)

__version__ = "0.1.0"
