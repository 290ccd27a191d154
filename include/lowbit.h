/*
 * lowbit.h -- C ABI of liblowbit: blockwise low-bit compression of training
 * communication buffers on AMD Instinct MI355X (gfx950).
 *
 * The operations are the codec stages of a low-bit data-parallel exchange:
 *
 *   compress   : buffer -> one binary16 scale per block + b-bit codes packed
 *                LSB-first into 32-bit words          (bitscom README,
 *                "Implemented Features": blockwise quantization with per-block
 *                FP16 scales; 1/2/4/8-bit codes; bit-packing; stochastic
 *                rounding; compress/decompress helpers)
 *   decompress : codes + scales -> binary32            (same section)
 *   error-feedback compress: compress (g + e), keep e <- (g + e) - deq(...)
 *                (bitscom README, "Implemented Features" and "Backend
 *                Registration Options": the legacy mode on the first-stage
 *                quantization)
 *   Hadamard smoothing: blockwise Walsh-Hadamard transform before compress
 *                and after decompress (SDP4Bit README, "Gradient Quantization
 *                Arguments")
 *   EF21 compress: compress (g - h), keep h <- h + deq(...) (bitscom README,
 *                "Backend Registration Options": the "ef21" mode)
 *   local reduce + requantize: the middle stage of a low-bit all-reduce
 *                (all-to-all -> local reduce -> all-gather; bitscom README,
 *                "Implemented Features"), optionally with error feedback on
 *                the reduced shard (same page, "Backend Registration
 *                Options": "ef21_plus") and with fewer output bits than input
 *                bits (SDP4Bit README, "Gradient Quantization Arguments":
 *                8-bit intra-node, 4-bit inter-node codes)
 *   weight-difference compress / apply (SDP4Bit README, "Overview" and
 *                "Weight Quantization Arguments")
 *
 * Wire format (shared by every entry point):
 *   codes  : uint32_t[lowbit_num_words(n, b)], little-endian words; element i
 *            occupies bits [(i mod 32/b) * b, +b) of word i / (32/b); bits of
 *            the last word past element n-1 are 0.  For b >= 2 the stored code
 *            is u = q + 2^(b-1) with q in [-(2^(b-1)-1), 2^(b-1)-1]; for b = 1
 *            it is u = 1 for x >= 0 (including -0.0) and 0 otherwise.
 *   scales : uint16_t[lowbit_num_blocks(n, B)], binary16 bit patterns, one per
 *            block of B consecutive elements (the last block may be shorter).
 *            b >= 2: s = smallest binary16 >= fl(max|x| / (2^(b-1)-1));
 *            b = 1 : s = smallest binary16 >= fl(sum|x| / n_valid), the sum
 *            taken over the block by an adjacent-pairs tree; both saturate at
 *            65504.  Dequantized value: q * s (b >= 2), u ? s : -s (b = 1).
 *   rounding: v = fl(x * fl(1/s)); round to nearest (ties to even) or
 *            stochastic q = floor(fl(v + r)), r = (h >> 8) * 2^-24 with
 *            h = fmix32(lo32(i) ^ fmix32(hi32(i) ^ K(seed))), i the global
 *            element index (index_offset + position), fmix32 the MurmurHash3
 *            finaliser and K(seed) = fmix32(lo32(seed) ^ fmix32(hi32(seed) ^
 *            0x9E3779B9)); then q is clamped to the grid.
 *
 * Conventions:
 *   - Pointers named as device pointers must be device memory (HBM) visible to
 *     the current HIP device; `peer_codes` / `peer_scales` themselves are host
 *     arrays holding device pointers.  The caller allocates and owns every
 *     buffer, including the error-feedback residual; the library allocates
 *     nothing and keeps no state between calls.
 *   - Alignment: element buffers (x, g, residual, state, w_*, y) 16 bytes,
 *     codes 4 bytes (peer codes of a mixed-width reduce: 4 * b_in/b_out
 *     bytes), scales 2 bytes.
 *   - Launches are asynchronous on `stream` (0 = the null stream).  Argument
 *     errors are reported synchronously and nothing is launched.  A launch
 *     failure returns LOWBIT_EDEVICE.  No call aborts or throws.
 *   - n == 0 is a no-op returning LOWBIT_OK.
 *   - Outputs must not alias inputs, except `residual` / `state` (in/out by
 *     design) and w_out == w_old in lowbit_wdiff_apply.
 *   - Non-finite inputs give unspecified (but in-range) codes; calls still
 *     terminate normally.
 */
#ifndef LOWBIT_H
#define LOWBIT_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    LOWBIT_OK = 0,
    LOWBIT_EINVAL = 1,        /* invalid argument; nothing launched            */
    LOWBIT_EUNSUPPORTED = 2,  /* valid but not built into this library         */
    LOWBIT_EDEVICE = 3        /* the HIP runtime reported a launch error       */
} lowbit_status;

typedef enum {
    LOWBIT_F32 = 0,           /* IEEE binary32                                 */
    LOWBIT_BF16 = 1           /* bfloat16, widened exactly to binary32         */
} lowbit_dtype;

/* Quantizer options (bitscom README, "Backend Registration Options": bitwidth
 * and block size; "Implemented Features": stochastic rounding). */

/* lowbit_qparams.hints: the caller reads the input again soon (for example
 * it compresses the same buffer at another bitwidth next, or decompresses the
 * peers' codes after reducing them): keep it in the caches.  Without it the
 * input is streamed where the access pattern allows (non-temporal loads), which
 * is faster for data read once: the binary32 input of the plain and the
 * Hadamard-smoothed compress (lowbit_quantize_pack,
 * lowbit_hadamard_quantize_pack) and the peers' code words of the local reduce
 * (taken from in_p of lowbit_reduce_requant and lowbit_reduce_requant_ef).
 * Accepted by every entry point; the others ignore it. */
#define LOWBIT_HINT_INPUT_REUSED 1
typedef struct {
    int32_t  bitwidth;        /* b: 1, 2, 4 or 8                                */
    int32_t  block_size;      /* B: power of two in [32, 4096]                  */
    int32_t  stochastic;      /* 0: nearest, ties to even; 1: stochastic
                                 rounding (ignored when b == 1)                 */
    int32_t  hints;           /* cache hints, LOWBIT_HINT_* bits (0: none); they
                                 change how data moves through the caches,
                                 never a result                                 */
    uint64_t seed;            /* stochastic-rounding key                        */
    uint64_t index_offset;    /* global index of element 0; a multiple of B.
                                 Only the random numbers depend on it, so a
                                 buffer split at block boundaries and
                                 compressed in pieces gives the same bytes.    */
} lowbit_qparams;

/* ceil(n * b / 32), or -1 for invalid arguments. */
int64_t lowbit_num_words(int64_t n, int32_t bitwidth);
/* ceil(n / B), or -1 for invalid arguments. */
int64_t lowbit_num_blocks(int64_t n, int32_t block_size);
/* static, human-readable name of a status code */
const char* lowbit_status_string(lowbit_status status);
/* library version string, e.g. "lowbit 0.1.0 gfx950" */
const char* lowbit_version(void);

/*
 * Compress (bitscom README, "Implemented Features": blockwise FP16-scaled
 * quantization to 1/2/4/8 bits with bit-packing, optional stochastic
 * rounding).
 *   x      : device, n elements of type xt
 *   codes  : device, lowbit_num_words(n, p->bitwidth) words (written)
 *   scales : device, lowbit_num_blocks(n, p->block_size) binary16 (written)
 * EINVAL: p == NULL, bad bitwidth/block_size, unknown hint bits, index_offset
 * not a multiple of block_size, n < 0, NULL or misaligned pointer with n > 0,
 * unknown dtype.
 */
lowbit_status lowbit_quantize_pack(const void* x, lowbit_dtype xt, int64_t n,
                                   const lowbit_qparams* p, uint32_t* codes, uint16_t* scales,
                                   hipStream_t stream);

/*
 * Decompress (bitscom README, "Implemented Features": unpacking and
 * dequantization, the decompress helper).
 *   codes, scales : device, as written by a compress call with the same
 *                   bitwidth and block_size (seed/index_offset/stochastic are
 *                   not used)
 *   y             : device, n binary32 values (written); y_i = q_i * s, exact.
 */
lowbit_status lowbit_unpack_dequant(const uint32_t* codes, const uint16_t* scales, int64_t n,
                                    const lowbit_qparams* p, float* y, hipStream_t stream);

/*
 * Compress with Hadamard smoothing (SDP4Bit README, "Gradient Quantization
 * Arguments": a Hadamard transform before gradient quantization lowers the
 * quantization error).  Each block of B elements is first transformed by the
 * Sylvester-ordered Walsh-Hadamard matrix -- butterflies (a, b) -> (fl(a+b),
 * fl(a-b)) of stride 1, 2, ..., B/2 in that order on binary32 values -- and
 * multiplied by 2^-floor(L/2), L = log2 B; the result is compressed as by
 * lowbit_quantize_pack (same wire format, same rounding options).  The local
 * reduce is linear and works on such codes unchanged.  When n is not a
 * multiple of block_size, the last, partial block is compressed without the
 * transform, exactly as lowbit_quantize_pack compresses it (the pages give
 * the transform for whole blocks only).
 */
lowbit_status lowbit_hadamard_quantize_pack(const void* x, lowbit_dtype xt, int64_t n,
                                            const lowbit_qparams* p, uint32_t* codes,
                                            uint16_t* scales, hipStream_t stream);

/*
 * Decompress with the inverse smoothing: dequantize, apply the same
 * butterflies per block and multiply by 2^-ceil(L/2) (the two scalings
 * multiply to 1/B, so the pair of transforms is the identity in exact
 * arithmetic).  A partial last block (n not a multiple of block_size) is
 * decompressed without the inverse transform, as lowbit_unpack_dequant does.
 */
lowbit_status lowbit_hadamard_unpack_dequant(const uint32_t* codes, const uint16_t* scales,
                                             int64_t n, const lowbit_qparams* p, float* y,
                                             hipStream_t stream);

/*
 * Error-feedback compress, legacy mode (bitscom README, "Implemented
 * Features": error feedback in first-stage quantization; "Backend
 * Registration Options": legacy mode).  For every element
 *     a = fl(g + e);  (codes, scales) = compress(a);  e <- fl(a - deq)
 *   g        : device, n elements of type gt (read)
 *   residual : device, n binary32 (read and overwritten); zero it before the
 *              first step.
 */
lowbit_status lowbit_ef_compress(const void* g, lowbit_dtype gt, float* residual, int64_t n,
                                 const lowbit_qparams* p, uint32_t* codes, uint16_t* scales,
                                 hipStream_t stream);

/*
 * EF21 compress (bitscom README, "Backend Registration Options": the "ef21"
 * mode of the first-stage quantization; the update is the published EF21
 * one).  For every element
 *     d = fl(g - h);  (codes, scales) = compress(d);  h <- fl(h + deq)
 *   g     : device, n elements of type gt (read)
 *   state : device, n binary32 (read and overwritten); the worker's EF21
 *           state h, zero before the first step.  Receivers track the sum of
 *           the states by adding the reduced messages (lowbit_wdiff_apply
 *           with wt = LOWBIT_F32 computes that fl(h + deq)).
 */
lowbit_status lowbit_ef21_compress(const void* g, lowbit_dtype gt, float* state, int64_t n,
                                   const lowbit_qparams* p, uint32_t* codes, uint16_t* scales,
                                   hipStream_t stream);

/*
 * Local reduce + requantize of a low-bit all-reduce (bitscom README,
 * "Implemented Features": all-to-all -> local reduce -> all-gather).  The
 * npeers chunks cover the same n elements; each is dequantized with in_p
 * (its bitwidth and block size) and summed in binary32 in peer order,
 *     acc = d_0;  acc = fl(acc + d_p), p = 1 .. npeers-1,
 * and acc is compressed with out_p.  in_p and out_p may differ in block size
 * and, for the pairs 8 -> 4, 8 -> 2 and 4 -> 2, in bitwidth (SDP4Bit README,
 * "Gradient Quantization Arguments": 8-bit intra-node codes requantized to
 * 4 bits for the inter-node step).  Only in_p's bitwidth and block_size are
 * used.
 *   peer_codes, peer_scales : HOST arrays of npeers DEVICE pointers
 *   out_sum                 : device, n binary32 (written) or NULL to skip
 * EINVAL additionally: npeers outside [1, 16].  EUNSUPPORTED: any other pair
 * of different bitwidths.
 */
lowbit_status lowbit_reduce_requant(const uint32_t* const* peer_codes,
                                    const uint16_t* const* peer_scales, int32_t npeers, int64_t n,
                                    const lowbit_qparams* in_p, const lowbit_qparams* out_p,
                                    uint32_t* out_codes, uint16_t* out_scales, float* out_sum,
                                    hipStream_t stream);

/*
 * Local reduce with stage-2 error feedback (bitscom README, "Backend
 * Registration Options": "ef21_plus" adds error feedback to the quantization
 * of the reduced shard).  As lowbit_reduce_requant, then per element
 *     a = fl(acc + e);  (out_codes, out_scales) = compress(a);  e <- fl(a - deq)
 *   residual : device, n binary32 (read and overwritten), zero before the
 *              first step; must not be NULL.
 *   out_sum  : receives acc (before e is added), or NULL.
 */
lowbit_status lowbit_reduce_requant_ef(const uint32_t* const* peer_codes,
                                       const uint16_t* const* peer_scales, int32_t npeers,
                                       int64_t n, const lowbit_qparams* in_p,
                                       const lowbit_qparams* out_p, float* residual,
                                       uint32_t* out_codes, uint16_t* out_scales, float* out_sum,
                                       hipStream_t stream);

/*
 * Weight-difference compress (SDP4Bit README, "Overview": weights are sent
 * as quantized differences; "Weight Quantization Arguments": bit count and
 * group size).  d = fl(w_new - w_old) is compressed with p.
 *   w_new, w_old : device, n elements of type wt
 */
lowbit_status lowbit_wdiff_compress(const void* w_new, const void* w_old, lowbit_dtype wt,
                                    int64_t n, const lowbit_qparams* p, uint32_t* codes,
                                    uint16_t* scales, hipStream_t stream);

/*
 * Weight-difference apply, the receiving side of the same scheme:
 *     w_out = to_wt(fl(w_old + deq)),  to_wt = identity (F32) or RNE (BF16).
 *   w_old, w_out : device, n elements of type wt; w_out may equal w_old.
 */
lowbit_status lowbit_wdiff_apply(const void* w_old, const uint32_t* codes, const uint16_t* scales,
                                 int64_t n, const lowbit_qparams* p, void* w_out, lowbit_dtype wt,
                                 hipStream_t stream);

/*
 * Measurement aid, not a step of the method: y[i] = x[i] for n binary32
 * values, with the same launch shape as the codec kernels.  Used to measure
 * the achievable HBM copy bandwidth and to scale hardware byte counters.
 */
lowbit_status lowbit_copy_f32(const float* x, float* y, int64_t n, hipStream_t stream);

/*
 * Measurement aid, not a step of the method: y[i] = fl(y[i] + x[i]) in place
 * for n binary32 values, with the error-feedback compress's access pattern
 * (two streams read, the second rewritten in place, the same per-wave trip)
 * and none of its arithmetic or code writes: the practical ceiling of the
 * error-feedback compress.
 *   x, y : device, n binary32 values each, 16-byte aligned; y is read and
 *          overwritten; x must not overlap y.
 * Errors: EINVAL for n < 0 or a null or misaligned pointer when n > 0;
 * n == 0 is a no-op.
 */
lowbit_status lowbit_add_inplace_f32(const float* x, float* y, int64_t n, hipStream_t stream);

/*
 * Measurement aid, not a step of the method: out[w] = XOR over the nstreams
 * streams of streams[p][w], for nwords 32-bit words.  It reads its inputs with
 * the local reduce's access pattern (every stream at the same offsets, one
 * 4-byte word per lane) and does none of its arithmetic, so its rate is what
 * HBM delivers for that pattern: the practical ceiling of the reduce.
 *   streams : host array of nstreams device pointers (1 <= nstreams <= 16),
 *             each 4-byte aligned and nwords words long.
 *   out     : device, nwords words; must not alias a stream.
 * Errors: EINVAL for nstreams outside [1, 16], nwords < 0, or a null or
 * misaligned pointer when nwords > 0; nwords == 0 is a no-op.
 */
lowbit_status lowbit_xor_streams_u32(const uint32_t* const* streams, int32_t nstreams,
                                     int64_t nwords, uint32_t* out, hipStream_t stream);

/*
 * Measurement aid, not a step of the method: reads n binary32 values and
 * writes ceil(n*bitwidth/32) 32-bit words -- the byte volume of a compress at
 * that bitwidth, less its scales (2/B bytes per value) -- with coalesced
 * 16-byte loads, one store per lane, and no arithmetic beyond XOR: the
 * practical ceiling of the compress kernels.  Values are taken in groups of
 * 2048 (8 rows of 256, four consecutive values per lane and row); lane l of
 * group g writes words (64g + l)*bitwidth + k, k < bitwidth, word k being the
 * XOR of the bit patterns of the lane's values 4r + j (r the row, j < 4) with
 * (4r + j) / (32/bitwidth) == k.  Values past n read as 0; words at or past
 * ceil(n*bitwidth/32) are not written.
 *   x   : device, n binary32 values, 16-byte aligned.
 *   out : device, ceil(n*bitwidth/32) words, 16-byte aligned; must not
 *         overlap x.
 * Errors: EINVAL for bitwidth outside {1, 2, 4, 8}, n < 0, or a null or
 * misaligned pointer when n > 0; n == 0 is a no-op.
 */
lowbit_status lowbit_fold_f32(const float* x, int64_t n, int32_t bitwidth, uint32_t* out,
                              hipStream_t stream);

/*
 * Measurement aid, not a step of the method: one pass over nwords 32-bit
 * words with a chosen grid and store policy, the probe behind the codec
 * kernels' launch shape (one trip per wave rather than a persistent grid) and
 * their streaming stores.  A trip is 1024 consecutive words, four coalesced
 * 16-byte pieces per lane.
 *   op LOWBIT_PROBE_READ  : dst[t] = XOR of the words of trip t of src
 *                           (nwords / 1024 words written);
 *   op LOWBIT_PROBE_WRITE : dst[i] = (i mod 2^32) ^ value (src unused);
 *   op LOWBIT_PROBE_COPY  : dst[i] = src[i].
 *   waves       : 0 -- one trip per wave over the whole buffer (the codec
 *                 kernels' shape); > 0 -- a persistent grid of that many waves
 *                 (rounded up to whole workgroups of four) looping over the
 *                 trips.
 *   nontemporal : nonzero -- streaming (non-temporal) stores; 0 -- plain.
 *   src, dst    : device, 16-byte aligned; must not overlap.
 * Errors: EINVAL for an unknown op, nwords < 0 or not a multiple of 1024,
 * waves < 0, or a null or misaligned pointer that the op uses when
 * nwords > 0; nwords == 0 is a no-op.
 */
#define LOWBIT_PROBE_READ 0
#define LOWBIT_PROBE_WRITE 1
#define LOWBIT_PROBE_COPY 2
lowbit_status lowbit_stream_probe_u32(int32_t op, const uint32_t* src, uint32_t* dst,
                                      int64_t nwords, uint32_t value, int32_t waves,
                                      int32_t nontemporal, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LOWBIT_H */
