/*
 * lowbit_oracle.c -- plain, slow CPU oracle for blockwise low-bit compression
 * of training communication buffers.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  The product path
 * (the HIP library and its Python binding) never calls into it, and the two
 * share no code: no headers, helpers, tables or constants.
 *
 * What is computed, and where it is described:
 *   - bitscom README, section "Implemented Features": quantization to 1, 2, 4
 *     or 8 bits, bit-packing and unpacking, stochastic rounding, blockwise
 *     quantization with one FP16 scale per block, the compress/decompress
 *     helpers, the low-bit all-reduce as all-to-all -> local reduce ->
 *     all-gather, and error feedback on the first-stage quantization.
 *   - bitscom README, section "Backend Registration Options": the options
 *     bitwidth / block_size / error feedback, and the "legacy" error-feedback
 *     mode applied to the first-stage quantization.
 *   - the same section: the "ef21" mode of the first-stage quantization and
 *     the "ef21_plus" mode, which adds error feedback to the quantization of
 *     the reduced shard.
 *   - SDP4Bit README, section "Overview": quantizing weight differences
 *     instead of weights; section "Weight Quantization Arguments": the bit
 *     count and group (block) size of weight quantization; section "Gradient
 *     Quantization Arguments": separate bit counts and group sizes for the
 *     intra-node and the inter-node gradient quantization, and the Hadamard
 *     transform applied before gradient quantization.
 *
 * The pages fix no formulas.  Each step below follows the plainest reading;
 * every reading is numbered (R1..R16, R23..R26) where it is used and listed
 * in the design notes of the repository.
 *
 * Arithmetic: IEEE binary32 with round-to-nearest-even, one operation at a
 * time.  Build with  -O2 -ffp-contract=off -fno-fast-math  so that no
 * product is fused into a sum and no excess precision is used.  Nothing here
 * is vectorised, blocked or reordered: blocks are visited in order and the
 * elements of a block one by one.
 */
#include <stdint.h>
#include <string.h>
#include <math.h>
#include <stdlib.h>

#define ORACLE_OK 0
#define ORACLE_EINVAL 1

/* ------------------------------------------------------------------------ */
/* Bit views of binary32                                                     */
/* ------------------------------------------------------------------------ */
static uint32_t f32_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float bits_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* ------------------------------------------------------------------------ */
/* binary16 (IEEE half) conversions, written from the format definition:     */
/* 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits; exponent field 0 */
/* holds subnormals k * 2^-24, field 31 holds inf/NaN.                       */
/* ------------------------------------------------------------------------ */

/* binary16 bit pattern -> binary32 value (always exact). */
float oracle_f16_to_f32(uint16_t h)
{
    uint32_t sign = (uint32_t)(h >> 15) & 1u;
    uint32_t expo = (uint32_t)(h >> 10) & 0x1Fu;
    uint32_t frac = (uint32_t)h & 0x3FFu;
    float mag;
    if (expo == 0) {
        mag = ldexpf((float)frac, -24);              /* subnormal or zero */
    } else if (expo == 31) {
        mag = (frac == 0) ? INFINITY : NAN;
    } else {
        mag = ldexpf((float)(1024u + frac), (int)expo - 25);  /* 1.f * 2^(e-15) */
    }
    return sign ? -mag : mag;
}

/* binary32 -> binary16, round to nearest, ties to even, subnormals kept,
 * overflow to infinity.  Works on the exact value m * 2^e of the input. */
uint16_t oracle_f32_to_f16_rne(float f)
{
    uint32_t u = f32_bits(f);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    uint32_t expo = (u >> 23) & 0xFFu;
    uint32_t frac = u & 0x7FFFFFu;
    if (expo == 0xFF) {
        if (frac == 0) return (uint16_t)(sign | 0x7C00u);
        return (uint16_t)(sign | 0x7E00u);           /* any NaN -> quiet NaN */
    }
    /* exact value = m * 2^(E - 23), m an integer below 2^24 */
    uint32_t m;
    int E;
    if (expo == 0) { m = frac; E = -126; } else { m = frac | 0x800000u; E = (int)expo - 127; }
    if (m == 0) return sign;
    /* normalise so that bit 23 of m is set (subnormal binary32 inputs) */
    while ((m & 0x800000u) == 0) { m <<= 1; E -= 1; }
    if (E > 15) return (uint16_t)(sign | 0x7C00u);   /* >= 2^16: overflow */
    uint32_t k;       /* magnitude in units of the target spacing */
    uint32_t shift;   /* bits of m dropped */
    uint32_t result;
    if (E >= -14) {
        /* normal range: spacing 2^(E-10); keep 11 significant bits */
        shift = 13;
        k = m >> shift;
        uint32_t rem = m & ((1u << shift) - 1u);
        uint32_t half = 1u << (shift - 1);
        if (rem > half || (rem == half && (k & 1u))) k += 1;
        /* k in [1024, 2048]; 2048 carries into the exponent */
        result = ((uint32_t)(E + 15) << 10) + (k - 1024u);
        if (result >= 0x7C00u) result = 0x7C00u;     /* rounded up to infinity */
    } else {
        /* subnormal range: spacing 2^-24; value/2^-24 = m * 2^(E - 23 + 24) */
        shift = (uint32_t)(-(E + 1));                /* >= 14 */
        if (shift > 25) {
            k = 0;                                   /* below 2^-25: rounds to 0 */
        } else {
            k = m >> shift;
            uint32_t rem = m & ((1u << shift) - 1u);
            uint32_t half = 1u << (shift - 1);
            if (rem > half || (rem == half && (k & 1u))) k += 1;
        }
        result = k;                                  /* k == 1024 is the smallest normal */
    }
    return (uint16_t)(sign | result);
}

/* R4: the stored scale is the smallest binary16 value >= t (rounding toward
 * +infinity), saturated to the largest finite binary16 (65504).  Any t that is
 * not below 65504, and any NaN, gives 65504.  t is a non-negative statistic. */
uint16_t oracle_f16_round_up(float t)
{
    uint16_t h = oracle_f32_to_f16_rne(t);
    if (oracle_f16_to_f32(h) < t) h = (uint16_t)(h + 1u);
    if (h > 0x7BFFu) h = 0x7BFFu;
    return h;
}

/* bfloat16: the upper half of a binary32 pattern.  Widening is exact. */
float oracle_bf16_to_f32(uint16_t h)
{
    return bits_f32((uint32_t)h << 16);
}

/* binary32 -> bfloat16, round to nearest, ties to even (NaN stays NaN). */
uint16_t oracle_f32_to_bf16_rne(float f)
{
    uint32_t u = f32_bits(f);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x7FFFFFu) != 0)
        return (uint16_t)((u >> 16) | 0x40u);
    uint32_t upper = u >> 16;
    uint32_t rem = u & 0xFFFFu;
    if (rem > 0x8000u || (rem == 0x8000u && (upper & 1u))) upper += 1;
    return (uint16_t)upper;
}

/* ------------------------------------------------------------------------ */
/* Counter-based random numbers for stochastic rounding (R9).               */
/* The pages name stochastic rounding (bitscom README, "Implemented          */
/* Features") but no generator.  The generator used is the 32-bit finaliser  */
/* of MurmurHash3 (public domain, Austin Appleby), keyed by the seed and    */
/* applied to the global element index.                                      */
/* ------------------------------------------------------------------------ */
uint32_t oracle_fmix32(uint32_t h)
{
    h ^= h >> 16;
    h *= 0x85EBCA6Bu;
    h ^= h >> 13;
    h *= 0xC2B2AE35u;
    h ^= h >> 16;
    return h;
}

/* key of a 64-bit seed */
uint32_t oracle_sr_key(uint64_t seed)
{
    uint32_t lo = (uint32_t)seed;
    uint32_t hi = (uint32_t)(seed >> 32);
    return oracle_fmix32(lo ^ oracle_fmix32(hi ^ 0x9E3779B9u));
}

/* 32 random bits of global element index i under a seed */
uint32_t oracle_sr_bits(uint64_t seed, uint64_t i)
{
    uint32_t key = oracle_sr_key(seed);
    uint32_t lo = (uint32_t)i;
    uint32_t hi = (uint32_t)(i >> 32);
    return oracle_fmix32(lo ^ oracle_fmix32(hi ^ key));
}

/* R8: uniform r in [0, 1) on the 2^-24 grid: the top 24 bits of the hash */
float oracle_sr_uniform(uint64_t seed, uint64_t i)
{
    uint32_t h = oracle_sr_bits(seed, i);
    return (float)(h >> 8) * (1.0f / 16777216.0f);
}

/* ------------------------------------------------------------------------ */
/* Bit packing (bitscom README, "Implemented Features": packing/unpacking). */
/* R13: codes are laid out by global element index, LSB first, 32/b codes   */
/* per little-endian uint32 word: element i sits in bits                    */
/* [(i mod (32/b)) * b, +b) of word i / (32/b).  Unused bits are 0.          */
/* ------------------------------------------------------------------------ */
int64_t oracle_num_words(int64_t n, int32_t bits) { return (n * bits + 31) / 32; }
int64_t oracle_num_blocks(int64_t n, int32_t block) { return (n + block - 1) / block; }

static void put_code(uint32_t* words, int64_t i, int bits, uint32_t u)
{
    int64_t per_word = 32 / bits;
    int64_t w = i / per_word;
    int sh = (int)(i % per_word) * bits;
    words[w] |= u << sh;
}

static uint32_t get_code(const uint32_t* words, int64_t i, int bits)
{
    int64_t per_word = 32 / bits;
    int64_t w = i / per_word;
    int sh = (int)(i % per_word) * bits;
    uint32_t mask = (bits == 32) ? 0xFFFFFFFFu : ((1u << bits) - 1u);
    return (words[w] >> sh) & mask;
}

static int valid_bits(int32_t b) { return b == 1 || b == 2 || b == 4 || b == 8; }
static int valid_block(int32_t B)
{
    return B >= 32 && B <= 4096 && (B & (B - 1)) == 0;
}

/* pack raw codes u[0..n) (each < 2^b) into words[0..num_words) */
int oracle_pack_codes(const uint32_t* u, int64_t n, int32_t bits, uint32_t* words)
{
    if (!valid_bits(bits) || n < 0) return ORACLE_EINVAL;
    int64_t nw = oracle_num_words(n, bits);
    for (int64_t w = 0; w < nw; ++w) words[w] = 0;
    for (int64_t i = 0; i < n; ++i) put_code(words, i, bits, u[i]);
    return ORACLE_OK;
}

int oracle_unpack_codes(const uint32_t* words, int64_t n, int32_t bits, uint32_t* u)
{
    if (!valid_bits(bits) || n < 0) return ORACLE_EINVAL;
    for (int64_t i = 0; i < n; ++i) u[i] = get_code(words, i, bits);
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* The blockwise quantizer                                                   */
/* ------------------------------------------------------------------------ */

/* R11: sum of |x| over a block for the 1-bit scale, by the adjacent-pairs
 * tree over the B leaf positions of the block (positions past the valid
 * elements are +0):  T(lo, hi) = T(lo, mid) + T(mid, hi). */
static float tree_abs_sum(const float* a, int64_t nvalid, int64_t lo, int64_t hi)
{
    if (hi - lo == 1) return (lo < nvalid) ? fabsf(a[lo]) : 0.0f;
    int64_t mid = lo + (hi - lo) / 2;
    float left = tree_abs_sum(a, nvalid, lo, mid);
    float right = tree_abs_sum(a, nvalid, mid, hi);
    return left + right;
}

static int qmax_of(int bits) { return (bits == 1) ? 1 : (1 << (bits - 1)) - 1; }

/*
 * Quantize one block a[0..nvalid) (nvalid <= span = B) whose first element
 * has global element index gidx.  Writes the codes into the packed word array
 * (element j of the block goes to array position pos0 + j), returns the
 * binary16 scale and, when deq != NULL, the dequantized values.
 *
 *   b >= 2 (R1): symmetric grid q in [-qmax, qmax], qmax = 2^(b-1) - 1.
 *       statistic  amax = max |a_j|
 *       t          = fl(amax / qmax)
 *   b == 1 (R3): sign code, scale = mean |a_j| of the block.
 *       statistic  S = tree sum of |a_j| (R11)
 *       t          = fl(S / nvalid)
 *   s16 = f16_round_up(t) (R4, R5); s = value of s16;
 *   inv = fl(1 / s), or 0 when s == 0 (R6).
 *   b >= 2, per element: v = fl(a_j * inv)
 *       round to nearest (R7): q = rint(v)  (ties to even)
 *       stochastic (R8):       q = floor(fl(v + r_j)), r_j from R9
 *       q = min(max(q, -qmax), qmax) (R10); stored code u = q + 2^(b-1) (R2)
 *       dequantized value q * s
 *   b == 1: u = 1 if a_j >= 0 (so -0 -> 1) else 0; dequantized u ? s : -s.
 */
static uint16_t quantize_block(const float* a, int64_t nvalid, int64_t span, int bits,
                                    int stochastic, uint64_t seed, uint64_t gidx,
                                    uint32_t* words, int64_t pos0, float* deq)
{
    int qmax = qmax_of(bits);
    float t;
    if (bits == 1) {
        float S = tree_abs_sum(a, nvalid, 0, span);
        t = S / (float)nvalid;
    } else {
        float amax = 0.0f;
        for (int64_t j = 0; j < nvalid; ++j) {
            float m = fabsf(a[j]);
            if (m > amax) amax = m;
        }
        t = amax / (float)qmax;
    }
    uint16_t s16 = oracle_f16_round_up(t);
    float s = oracle_f16_to_f32(s16);
    float inv = (s != 0.0f) ? 1.0f / s : 0.0f;

    for (int64_t j = 0; j < nvalid; ++j) {
        uint32_t u;
        float d;
        if (bits == 1) {
            u = (a[j] >= 0.0f) ? 1u : 0u;
            d = u ? s : -s;
        } else {
            float v = a[j] * inv;
            float q;
            if (stochastic) {
                float r = oracle_sr_uniform(seed, gidx + (uint64_t)j);
                float y = v + r;
                q = floorf(y);
            } else {
                q = rintf(v);
            }
            q = fmaxf(q, (float)-qmax);
            q = fminf(q, (float)qmax);
            int qi = (int)q;
            u = (uint32_t)(qi + (1 << (bits - 1)));
            d = (float)qi * s;
        }
        put_code(words, pos0 + j, bits, u);
        if (deq) deq[j] = d;
    }
    return s16;
}

/* dequantize one code with its block scale (exact in binary32) */
static float dequant_code(uint32_t u, int bits, float s)
{
    if (bits == 1) return u ? s : -s;
    int q = (int)u - (1 << (bits - 1));
    return (float)q * s;
}

/* element loader: dtype 0 = binary32, 1 = bfloat16 (widened exactly) */
static float load_elem(const void* p, int dtype, int64_t i)
{
    if (dtype == 0) return ((const float*)p)[i];
    return oracle_bf16_to_f32(((const uint16_t*)p)[i]);
}

static int check_q(int32_t bits, int32_t block, int64_t n, uint64_t index_offset)
{
    if (!valid_bits(bits) || !valid_block(block) || n < 0) return ORACLE_EINVAL;
    if (index_offset % (uint64_t)block != 0) return ORACLE_EINVAL;
    return ORACLE_OK;
}

/*
 * compress: x[0..n) (binary32 or bfloat16) -> packed codes + one binary16
 * scale per block.  Element k of x has global index index_offset + k; this
 * index only feeds the stochastic-rounding generator.
 */
int oracle_quantize_pack(const void* x, int32_t dtype, int64_t n, int32_t bits, int32_t block,
                         int32_t stochastic, uint64_t seed, uint64_t index_offset,
                         uint32_t* codes, uint16_t* scales)
{
    int rc = check_q(bits, block, n, index_offset);
    if (rc) return rc;
    int64_t nw = oracle_num_words(n, bits);
    for (int64_t w = 0; w < nw; ++w) codes[w] = 0;
    float* a = (float*)malloc(sizeof(float) * (size_t)block);
    if (!a) return ORACLE_EINVAL;
    int64_t nb = oracle_num_blocks(n, block);
    for (int64_t k = 0; k < nb; ++k) {
        int64_t lo = k * block;
        int64_t nvalid = (n - lo < block) ? (n - lo) : block;
        for (int64_t j = 0; j < nvalid; ++j) a[j] = load_elem(x, dtype, lo + j);
        scales[k] = quantize_block(a, nvalid, block, bits, bits == 1 ? 0 : stochastic,
                                        seed, index_offset + (uint64_t)lo, codes, lo, NULL);
    }
    free(a);
    return ORACLE_OK;
}

/* decompress: packed codes + scales -> binary32 (bitscom README,
 * "Implemented Features": dequantize / decompress). */
int oracle_unpack_dequant(const uint32_t* codes, const uint16_t* scales, int64_t n,
                          int32_t bits, int32_t block, float* y)
{
    if (!valid_bits(bits) || !valid_block(block) || n < 0) return ORACLE_EINVAL;
    for (int64_t i = 0; i < n; ++i) {
        float s = oracle_f16_to_f32(scales[i / block]);
        y[i] = dequant_code(get_code(codes, i, bits), bits, s);
    }
    return ORACLE_OK;
}

/*
 * Hadamard smoothing (SDP4Bit README, "Gradient Quantization Arguments": a
 * Hadamard transform of the gradient before quantization lowers the
 * quantization error; "Overview": the two-level gradient smooth
 * quantization).  R26: each block of B elements is transformed by the
 * Sylvester-ordered Walsh-Hadamard matrix (H_1 = [1], H_2m = [[H_m, H_m],
 * [H_m, -H_m]]), computed in binary32 by butterflies of stride 1, 2, ..., B/2
 * in that order, each butterfly (a, b) -> (fl(a + b), fl(a - b)).  The
 * forward result is multiplied by 2^-floor(L/2) and the inverse by
 * 2^-ceil(L/2), L = log2 B, so the pair is the identity in exact arithmetic
 * and both scalings are exact.  R27: the pages give the transform for whole
 * quantization blocks only; a last block of fewer than B elements (n not a
 * multiple of B) is compressed and decompressed without it, exactly as the
 * plain compress and decompress treat a partial block.
 */
static void walsh_hadamard(float* t, int64_t B)
{
    for (int64_t h = 1; h < B; h <<= 1)
        for (int64_t i = 0; i < B; i += 2 * h)
            for (int64_t j = i; j < i + h; ++j) {
                float a = t[j], b = t[j + h];
                t[j] = a + b;
                t[j + h] = a - b;
            }
}

static int log2_of(int64_t B)
{
    int L = 0;
    while (((int64_t)1 << L) < B) ++L;
    return L;
}

int oracle_hadamard_quantize_pack(const void* x, int32_t dtype, int64_t n, int32_t bits,
                                  int32_t block, int32_t stochastic, uint64_t seed,
                                  uint64_t index_offset, uint32_t* codes, uint16_t* scales)
{
    int rc = check_q(bits, block, n, index_offset);
    if (rc) return rc;
    int64_t nw = oracle_num_words(n, bits);
    for (int64_t w = 0; w < nw; ++w) codes[w] = 0;
    float* a = (float*)malloc(sizeof(float) * (size_t)block);
    if (!a) return ORACLE_EINVAL;
    float f = ldexpf(1.0f, -(log2_of(block) / 2));
    int64_t nb = oracle_num_blocks(n, block);
    for (int64_t k = 0; k < nb; ++k) {
        int64_t lo = k * block;
        int64_t nvalid = (n - lo < block) ? (n - lo) : block;
        for (int64_t j = 0; j < nvalid; ++j) a[j] = load_elem(x, dtype, lo + j);
        if (nvalid == block) {              /* a partial last block is not transformed */
            walsh_hadamard(a, block);
            for (int64_t j = 0; j < block; ++j) a[j] = a[j] * f;
        }
        scales[k] = quantize_block(a, nvalid, block, bits, bits == 1 ? 0 : stochastic, seed,
                                   index_offset + (uint64_t)lo, codes, lo, NULL);
    }
    free(a);
    return ORACLE_OK;
}

int oracle_hadamard_unpack_dequant(const uint32_t* codes, const uint16_t* scales, int64_t n,
                                   int32_t bits, int32_t block, float* y)
{
    if (!valid_bits(bits) || !valid_block(block) || n < 0) return ORACLE_EINVAL;
    float f = ldexpf(1.0f, -((log2_of(block) + 1) / 2));
    for (int64_t lo = 0; lo < n; lo += block) {
        float s = oracle_f16_to_f32(scales[lo / block]);
        int64_t nvalid = (n - lo < block) ? (n - lo) : block;
        for (int64_t j = 0; j < nvalid; ++j)
            y[lo + j] = dequant_code(get_code(codes, lo + j, bits), bits, s);
        if (nvalid == block) {              /* a partial last block is not transformed */
            walsh_hadamard(y + lo, block);
            for (int64_t j = 0; j < block; ++j) y[lo + j] = y[lo + j] * f;
        }
    }
    return ORACLE_OK;
}

/* The transform alone (forward: inverse = 0, inverse: inverse = 1), on the
 * whole blocks of x in place (a partial last block is left as it is). */
int oracle_hadamard_blocks(float* x, int64_t n, int32_t block, int32_t inverse)
{
    if (!valid_block(block) || n < 0) return ORACLE_EINVAL;
    int L = log2_of(block);
    float f = ldexpf(1.0f, inverse ? -((L + 1) / 2) : -(L / 2));
    for (int64_t lo = 0; lo + block <= n; lo += block) {
        walsh_hadamard(x + lo, block);
        for (int64_t j = 0; j < block; ++j) x[lo + j] = x[lo + j] * f;
    }
    return ORACLE_OK;
}

/*
 * Error-feedback compress (bitscom README, "Implemented Features" and
 * "Backend Registration Options": the legacy mode applied to the first-stage
 * quantization).  R14:
 *   a_i = fl(g_i + e_i); quantize a; e_i <- fl(a_i - deq_i).
 * The residual e is binary32, owned by the caller, updated in place.
 */
int oracle_ef_compress(const void* g, int32_t dtype, float* e, int64_t n, int32_t bits,
                       int32_t block, int32_t stochastic, uint64_t seed, uint64_t index_offset,
                       uint32_t* codes, uint16_t* scales)
{
    int rc = check_q(bits, block, n, index_offset);
    if (rc) return rc;
    int64_t nw = oracle_num_words(n, bits);
    for (int64_t w = 0; w < nw; ++w) codes[w] = 0;
    float* a = (float*)malloc(sizeof(float) * (size_t)block);
    float* d = (float*)malloc(sizeof(float) * (size_t)block);
    if (!a || !d) { free(a); free(d); return ORACLE_EINVAL; }
    int64_t nb = oracle_num_blocks(n, block);
    for (int64_t k = 0; k < nb; ++k) {
        int64_t lo = k * block;
        int64_t nvalid = (n - lo < block) ? (n - lo) : block;
        for (int64_t j = 0; j < nvalid; ++j) a[j] = load_elem(g, dtype, lo + j) + e[lo + j];
        scales[k] = quantize_block(a, nvalid, block, bits, bits == 1 ? 0 : stochastic,
                                        seed, index_offset + (uint64_t)lo, codes, lo, d);
        for (int64_t j = 0; j < nvalid; ++j) e[lo + j] = a[j] - d[j];
    }
    free(a);
    free(d);
    return ORACLE_OK;
}

/*
 * EF21 compress (bitscom README, "Backend Registration Options": the "ef21"
 * error-feedback mode of the first-stage quantization; the page names the
 * mode only, so the update follows the published EF21 method: each worker
 * keeps a state h, sends the compressed difference between its gradient and
 * h, and moves h by what it sent).  R23:
 *   d_i = fl(g_i - h_i); quantize d; h_i <- fl(h_i + deq_i).
 * The state h is binary32, owned by the caller, updated in place.
 */
int oracle_ef21_compress(const void* g, int32_t dtype, float* h, int64_t n, int32_t bits,
                         int32_t block, int32_t stochastic, uint64_t seed, uint64_t index_offset,
                         uint32_t* codes, uint16_t* scales)
{
    int rc = check_q(bits, block, n, index_offset);
    if (rc) return rc;
    int64_t nw = oracle_num_words(n, bits);
    for (int64_t w = 0; w < nw; ++w) codes[w] = 0;
    float* d = (float*)malloc(sizeof(float) * (size_t)block);
    float* q = (float*)malloc(sizeof(float) * (size_t)block);
    if (!d || !q) { free(d); free(q); return ORACLE_EINVAL; }
    int64_t nb = oracle_num_blocks(n, block);
    for (int64_t k = 0; k < nb; ++k) {
        int64_t lo = k * block;
        int64_t nvalid = (n - lo < block) ? (n - lo) : block;
        for (int64_t j = 0; j < nvalid; ++j) d[j] = load_elem(g, dtype, lo + j) - h[lo + j];
        scales[k] = quantize_block(d, nvalid, block, bits, bits == 1 ? 0 : stochastic,
                                   seed, index_offset + (uint64_t)lo, codes, lo, q);
        for (int64_t j = 0; j < nvalid; ++j) h[lo + j] = h[lo + j] + q[j];
    }
    free(d);
    free(q);
    return ORACLE_OK;
}

/*
 * Local reduce of the low-bit all-reduce (bitscom README, "Implemented
 * Features": all-to-all -> local reduce -> all-gather).  npeers chunks of the
 * same n elements, each packed with (in_bits, in_block), are dequantized and
 * summed in binary32 in peer order (R15):
 *     acc = d_0;  acc = fl(acc + d_p) for p = 1 .. npeers-1
 * where d_p of element i uses peer p's scale of input block i / in_block.
 * The sum is quantized again with (out_bits, out_block, out_stochastic,
 * out_seed, out_index_offset).  out_sum, when not NULL, receives acc.
 *
 * Mixed widths and block sizes (SDP4Bit README, "Gradient Quantization
 * Arguments": separate bit counts and group sizes for the intra-node and the
 * inter-node gradient quantization, 8 and 4 bits by default) are the same
 * computation with in_bits != out_bits or in_block != out_block (R24).
 *
 * Stage-2 error feedback (bitscom README, "Backend Registration Options":
 * the "ef21_plus" mode also applies error feedback to the quantization of
 * the reduced shard) when residual is not NULL, R25 (R14 on the sum):
 *     a_i = fl(acc_i + e_i); quantize a; e_i <- fl(a_i - deq_i).
 * out_sum still receives acc (before the residual is added).
 */
int oracle_reduce_requant_ex(const uint32_t* const* peer_codes,
                             const uint16_t* const* peer_scales, int32_t npeers, int64_t n,
                             int32_t in_bits, int32_t in_block, int32_t out_bits,
                             int32_t out_block, int32_t out_stochastic, uint64_t out_seed,
                             uint64_t out_index_offset, float* residual, uint32_t* out_codes,
                             uint16_t* out_scales, float* out_sum)
{
    if (npeers < 1 || npeers > 16) return ORACLE_EINVAL;
    int rc = check_q(in_bits, in_block, n, 0);
    if (rc) return rc;
    rc = check_q(out_bits, out_block, n, out_index_offset);
    if (rc) return rc;
    int64_t nw = oracle_num_words(n, out_bits);
    for (int64_t w = 0; w < nw; ++w) out_codes[w] = 0;
    float* a = (float*)malloc(sizeof(float) * (size_t)out_block);
    float* q = (float*)malloc(sizeof(float) * (size_t)out_block);
    if (!a || !q) { free(a); free(q); return ORACLE_EINVAL; }
    int64_t nb = oracle_num_blocks(n, out_block);
    for (int64_t k = 0; k < nb; ++k) {
        int64_t lo = k * out_block;
        int64_t nvalid = (n - lo < out_block) ? (n - lo) : out_block;
        for (int64_t j = 0; j < nvalid; ++j) {
            int64_t i = lo + j;
            float acc = 0.0f;
            for (int32_t p = 0; p < npeers; ++p) {
                float s = oracle_f16_to_f32(peer_scales[p][i / in_block]);
                float d = dequant_code(get_code(peer_codes[p], i, in_bits), in_bits, s);
                acc = (p == 0) ? d : acc + d;
            }
            if (out_sum) out_sum[i] = acc;
            a[j] = residual ? acc + residual[i] : acc;
        }
        out_scales[k] = quantize_block(a, nvalid, out_block, out_bits,
                                       out_bits == 1 ? 0 : out_stochastic, out_seed,
                                       out_index_offset + (uint64_t)lo, out_codes, lo,
                                       residual ? q : NULL);
        if (residual)
            for (int64_t j = 0; j < nvalid; ++j) residual[lo + j] = a[j] - q[j];
    }
    free(a);
    free(q);
    return ORACLE_OK;
}

/* The plain local reduce: one block size for input and output, no residual. */
int oracle_reduce_requant(const uint32_t* const* peer_codes, const uint16_t* const* peer_scales,
                          int32_t npeers, int64_t n, int32_t in_bits, int32_t block,
                          int32_t out_bits, int32_t out_stochastic, uint64_t out_seed,
                          uint64_t out_index_offset, uint32_t* out_codes, uint16_t* out_scales,
                          float* out_sum)
{
    return oracle_reduce_requant_ex(peer_codes, peer_scales, npeers, n, in_bits, block, out_bits,
                                    block, out_stochastic, out_seed, out_index_offset, NULL,
                                    out_codes, out_scales, out_sum);
}

/*
 * Weight-difference compress (SDP4Bit README, "Overview": weights are
 * communicated as quantized differences; "Weight Quantization Arguments":
 * bit count and group size).  R16:  d_i = fl(w_new_i - w_old_i), quantized
 * blockwise like any other buffer.
 */
int oracle_wdiff_compress(const void* w_new, const void* w_old, int32_t dtype, int64_t n,
                          int32_t bits, int32_t block, int32_t stochastic, uint64_t seed,
                          uint64_t index_offset, uint32_t* codes, uint16_t* scales)
{
    int rc = check_q(bits, block, n, index_offset);
    if (rc) return rc;
    int64_t nw = oracle_num_words(n, bits);
    for (int64_t w = 0; w < nw; ++w) codes[w] = 0;
    float* a = (float*)malloc(sizeof(float) * (size_t)block);
    if (!a) return ORACLE_EINVAL;
    int64_t nb = oracle_num_blocks(n, block);
    for (int64_t k = 0; k < nb; ++k) {
        int64_t lo = k * block;
        int64_t nvalid = (n - lo < block) ? (n - lo) : block;
        for (int64_t j = 0; j < nvalid; ++j)
            a[j] = load_elem(w_new, dtype, lo + j) - load_elem(w_old, dtype, lo + j);
        scales[k] = quantize_block(a, nvalid, block, bits, bits == 1 ? 0 : stochastic,
                                        seed, index_offset + (uint64_t)lo, codes, lo, NULL);
    }
    free(a);
    return ORACLE_OK;
}

/*
 * Weight-difference apply (receiver side of the same scheme):
 *     w_out_i = round_to_dtype(fl(w_old_i + deq_i))
 * with round_to_dtype = identity for binary32 and RNE to bfloat16 otherwise.
 * w_out may be the same buffer as w_old.
 */
int oracle_wdiff_apply(const void* w_old, const uint32_t* codes, const uint16_t* scales,
                       int64_t n, int32_t bits, int32_t block, void* w_out, int32_t dtype)
{
    if (!valid_bits(bits) || !valid_block(block) || n < 0) return ORACLE_EINVAL;
    for (int64_t i = 0; i < n; ++i) {
        float s = oracle_f16_to_f32(scales[i / block]);
        float d = dequant_code(get_code(codes, i, bits), bits, s);
        float w = load_elem(w_old, dtype, i) + d;
        if (dtype == 0) ((float*)w_out)[i] = w;
        else ((uint16_t*)w_out)[i] = oracle_f32_to_bf16_rne(w);
    }
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Array helpers used only by the pinning tests                             */
/* ------------------------------------------------------------------------ */
void oracle_f32_to_f16_rne_array(const float* x, int64_t n, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f32_to_f16_rne(x[i]);
}
void oracle_f16_round_up_array(const float* x, int64_t n, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f16_round_up(x[i]);
}
void oracle_f16_to_f32_array(const uint16_t* h, int64_t n, float* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f16_to_f32(h[i]);
}
void oracle_f32_to_bf16_rne_array(const float* x, int64_t n, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f32_to_bf16_rne(x[i]);
}
void oracle_sr_uniform_array(uint64_t seed, uint64_t i0, int64_t n, float* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_sr_uniform(seed, i0 + (uint64_t)i);
}
void oracle_fmix32_array(const uint32_t* x, int64_t n, uint32_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_fmix32(x[i]);
}
