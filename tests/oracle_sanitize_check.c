/*
 * Memory and undefined-behaviour check of the CPU oracle: every entry point of
 * oracle/lowbit_oracle.c runs on buffers allocated to their exact documented
 * sizes (ragged lengths, every bitwidth and block size, stochastic rounding,
 * residuals, sums, mixed widths, both input types), built with AddressSanitizer
 * and UndefinedBehaviorSanitizer by the test that compiles this file.  Values
 * are not checked here (the pins do that); an out-of-bounds access, a use of
 * freed memory or undefined arithmetic aborts the program.  Prints OK.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

float oracle_f16_to_f32(uint16_t h);
uint16_t oracle_f32_to_f16_rne(float f);
uint16_t oracle_f16_round_up(float t);
float oracle_bf16_to_f32(uint16_t h);
uint16_t oracle_f32_to_bf16_rne(float f);
uint32_t oracle_fmix32(uint32_t h);
float oracle_sr_uniform(uint64_t seed, uint64_t i);
int64_t oracle_num_words(int64_t n, int32_t bits);
int64_t oracle_num_blocks(int64_t n, int32_t block);
int oracle_pack_codes(const uint32_t* u, int64_t n, int32_t bits, uint32_t* words);
int oracle_unpack_codes(const uint32_t* words, int64_t n, int32_t bits, uint32_t* u);
int oracle_quantize_pack(const void* x, int32_t dtype, int64_t n, int32_t bits, int32_t block,
                         int32_t stochastic, uint64_t seed, uint64_t index_offset,
                         uint32_t* codes, uint16_t* scales);
int oracle_unpack_dequant(const uint32_t* codes, const uint16_t* scales, int64_t n,
                          int32_t bits, int32_t block, float* y);
int oracle_hadamard_quantize_pack(const void* x, int32_t dtype, int64_t n, int32_t bits,
                                  int32_t block, int32_t stochastic, uint64_t seed,
                                  uint64_t index_offset, uint32_t* codes, uint16_t* scales);
int oracle_hadamard_unpack_dequant(const uint32_t* codes, const uint16_t* scales, int64_t n,
                                   int32_t bits, int32_t block, float* y);
int oracle_hadamard_blocks(float* x, int64_t n, int32_t block, int32_t inverse);
int oracle_ef_compress(const void* g, int32_t dtype, float* e, int64_t n, int32_t bits,
                       int32_t block, int32_t stochastic, uint64_t seed, uint64_t index_offset,
                       uint32_t* codes, uint16_t* scales);
int oracle_ef21_compress(const void* g, int32_t dtype, float* h, int64_t n, int32_t bits,
                         int32_t block, int32_t stochastic, uint64_t seed, uint64_t index_offset,
                         uint32_t* codes, uint16_t* scales);
int oracle_reduce_requant_ex(const uint32_t* const* peer_codes,
                             const uint16_t* const* peer_scales, int32_t npeers, int64_t n,
                             int32_t in_bits, int32_t in_block, int32_t out_bits,
                             int32_t out_block, int32_t out_stochastic, uint64_t out_seed,
                             uint64_t out_index_offset, float* residual, uint32_t* out_codes,
                             uint16_t* out_scales, float* out_sum);
int oracle_wdiff_compress(const void* w_new, const void* w_old, int32_t dtype, int64_t n,
                          int32_t bits, int32_t block, int32_t stochastic, uint64_t seed,
                          uint64_t index_offset, uint32_t* codes, uint16_t* scales);
int oracle_wdiff_apply(const void* w_old, const uint32_t* codes, const uint16_t* scales,
                       int64_t n, int32_t bits, int32_t block, void* w_out, int32_t dtype);

static uint64_t rng = 0x243F6A8885A308D3ull;
static uint32_t next32(void)
{
    rng ^= rng << 13;
    rng ^= rng >> 7;
    rng ^= rng << 17;
    return (uint32_t)(rng >> 16);
}

/* values of mixed magnitudes, with zeros and a few huge and tiny ones */
static float value(void)
{
    uint32_t r = next32();
    float v = ((float)(r & 0xFFFF) / 32768.0f - 1.0f);
    switch (r >> 28) {
        case 0: return 0.0f;
        case 1: return v * 1e-30f;
        case 2: return v * 6e4f;
        default: return v;
    }
}

/* n elements of dtype (0: binary32, 1: bfloat16 bit patterns), exact size */
static void* input(int dtype, int64_t n)
{
    if (dtype == 0) {
        float* x = (float*)malloc(sizeof(float) * (size_t)(n ? n : 1));
        for (int64_t i = 0; i < n; ++i) x[i] = value();
        return x;
    }
    uint16_t* x = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(n ? n : 1));
    for (int64_t i = 0; i < n; ++i) x[i] = oracle_f32_to_bf16_rne(value());
    return x;
}

static int fail = 0;
static void expect_ok(int rc, const char* what)
{
    if (rc != 0) {
        printf("unexpected status %d from %s\n", rc, what);
        fail = 1;
    }
}

int main(void)
{
    const int bitsv[4] = {1, 2, 4, 8};
    const int blocks[5] = {32, 64, 128, 1024, 4096};
    const int64_t lens[6] = {1, 7, 33, 255, 4096, 4096 * 2 + 77};

    for (int bi = 0; bi < 4; ++bi)
        for (int k = 0; k < 5; ++k)
            for (int li = 0; li < 6; ++li)
                for (int dt = 0; dt < 2; ++dt) {
                    const int b = bitsv[bi], B = blocks[k], sr = (li + dt) & 1;
                    const int64_t n = lens[li];
                    const int64_t nw = oracle_num_words(n, b), nb = oracle_num_blocks(n, B);
                    void* x = input(dt, n);
                    void* x2 = input(dt, n);
                    uint32_t* c = (uint32_t*)malloc(sizeof(uint32_t) * (size_t)nw);
                    uint16_t* s = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)nb);
                    float* y = (float*)malloc(sizeof(float) * (size_t)n);
                    float* e = (float*)calloc((size_t)n, sizeof(float));
                    uint32_t* u = (uint32_t*)malloc(sizeof(uint32_t) * (size_t)n);

                    expect_ok(oracle_quantize_pack(x, dt, n, b, B, sr, 42, (uint64_t)B * 3, c, s),
                              "quantize_pack");
                    expect_ok(oracle_unpack_dequant(c, s, n, b, B, y), "unpack_dequant");
                    expect_ok(oracle_unpack_codes(c, n, b, u), "unpack_codes");
                    expect_ok(oracle_pack_codes(u, n, b, c), "pack_codes");
                    expect_ok(oracle_hadamard_quantize_pack(x, dt, n, b, B, sr, 7, 0, c, s),
                              "hadamard_quantize_pack");
                    expect_ok(oracle_hadamard_unpack_dequant(c, s, n, b, B, y),
                              "hadamard_unpack_dequant");
                    expect_ok(oracle_hadamard_blocks(y, n, B, 1), "hadamard_blocks");
                    expect_ok(oracle_ef_compress(x, dt, e, n, b, B, sr, 3, 0, c, s), "ef_compress");
                    expect_ok(oracle_ef21_compress(x, dt, e, n, b, B, sr, 4, 0, c, s),
                              "ef21_compress");
                    expect_ok(oracle_wdiff_compress(x, x2, dt, n, b, B, sr, 5, 0, c, s),
                              "wdiff_compress");
                    void* w = dt == 0 ? malloc(sizeof(float) * (size_t)n)
                                      : malloc(sizeof(uint16_t) * (size_t)n);
                    expect_ok(oracle_wdiff_apply(x2, c, s, n, b, B, w, dt), "wdiff_apply");

                    /* local reduce of 3 peers, same and lower output widths and
                     * another output block size, with and without residual and sum */
                    const uint32_t* pc[3];
                    const uint16_t* ps[3];
                    uint32_t* own_c[3];
                    uint16_t* own_s[3];
                    for (int p = 0; p < 3; ++p) {
                        own_c[p] = (uint32_t*)malloc(sizeof(uint32_t) * (size_t)nw);
                        own_s[p] = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)nb);
                        void* xp = input(0, n);
                        expect_ok(oracle_quantize_pack(xp, 0, n, b, B, 0, 0, 0, own_c[p], own_s[p]),
                                  "peer quantize_pack");
                        free(xp);
                        pc[p] = own_c[p];
                        ps[p] = own_s[p];
                    }
                    for (int ob = 0; ob <= bi; ++ob) {
                        const int bo = bitsv[ob];
                        const int Bo = blocks[(k + ob) % 5];
                        const int64_t onw = oracle_num_words(n, bo), onb = oracle_num_blocks(n, Bo);
                        uint32_t* oc = (uint32_t*)malloc(sizeof(uint32_t) * (size_t)onw);
                        uint16_t* os = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)onb);
                        float* sum = (float*)malloc(sizeof(float) * (size_t)n);
                        float* res = (float*)calloc((size_t)n, sizeof(float));
                        expect_ok(oracle_reduce_requant_ex(pc, ps, 3, n, b, B, bo, Bo, sr, 9, 0,
                                                           (ob & 1) ? res : NULL, oc, os,
                                                           (ob & 1) ? NULL : sum),
                                  "reduce_requant_ex");
                        free(oc);
                        free(os);
                        free(sum);
                        free(res);
                    }
                    for (int p = 0; p < 3; ++p) {
                        free(own_c[p]);
                        free(own_s[p]);
                    }
                    free(w);
                    free(x);
                    free(x2);
                    free(c);
                    free(s);
                    free(y);
                    free(e);
                    free(u);
                }

    /* conversions over a sweep of bit patterns, including NaN and infinities */
    for (uint64_t i = 0; i < (1ull << 32); i += 65537) {
        uint32_t v = (uint32_t)i;
        float f;
        memcpy(&f, &v, sizeof f);
        (void)oracle_f32_to_f16_rne(f);
        (void)oracle_f16_round_up(f < 0 ? -f : f);
        (void)oracle_f32_to_bf16_rne(f);
        (void)oracle_f16_to_f32((uint16_t)v);
        (void)oracle_bf16_to_f32((uint16_t)v);
        (void)oracle_fmix32(v);
        (void)oracle_sr_uniform(i, i * 2654435761ull);
    }

    /* invalid arguments return a status without touching the buffers */
    if (oracle_quantize_pack(NULL, 0, 10, 3, 128, 0, 0, 0, NULL, NULL) == 0) fail = 1;
    if (oracle_quantize_pack(NULL, 0, 10, 4, 100, 0, 0, 0, NULL, NULL) == 0) fail = 1;
    if (oracle_unpack_dequant(NULL, NULL, -1, 4, 128, NULL) == 0) fail = 1;
    if (oracle_reduce_requant_ex(NULL, NULL, 0, 10, 4, 128, 4, 128, 0, 0, 0, NULL, NULL, NULL,
                                 NULL) == 0)
        fail = 1;

    if (fail) return 1;
    printf("OK\n");
    return 0;
}
