/* Drives every oracle function on small inputs, for an AddressSanitizer /
 * UndefinedBehaviorSanitizer build (test infrastructure).  Exit status 0 and
 * no sanitizer report is the pass condition; the numeric checks here are only
 * coarse sanity checks (the values are pinned by the Python tests). */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int orc_mcg_value(uint32_t state, uint32_t mcg);
void orc_stream_states(const uint16_t *words, int nwords, int K, uint16_t *states);
double orc_e4m3_rne(double x);
double orc_codebook_value(uint32_t state, uint32_t mcg, int codebook);
void orc_decode_tile(const uint16_t *words, int K, uint32_t mcg, int codebook, float *vals);
void orc_decode_matrix(const uint16_t *codes, int in, int out, int K, uint32_t mcg, int codebook, float *dst);
int64_t orc_tile_position(int order, int in, int out, int tk, int tn);
int orc_decode_matrix_order(const uint16_t *codes, int in, int out, int K, uint32_t mcg, int codebook, int order,
                            float *dst);
void orc_expand_block_scales(const uint16_t *block, int EA, int H, int I, uint16_t *const *suh,
                             uint16_t *const *svh);
void orc_router_logits(const uint16_t *x, int x_dtype, int64_t T, int H, const uint16_t *Wr, const float *bias,
                       int E, float *logits);
void orc_topk_softmax(const float *logits, int64_t T, int E, int k, int32_t *idx, double *w);
void orc_segments(const int32_t *idx, int64_t T, int k, int E, int32_t *counts, int32_t *offsets,
                  int32_t *sorted_ids, int32_t *pos);
void orc_sylvester(int n, int8_t *Hm);
void orc_rotate(double *v, int len, const int8_t *s);
int orc_layer(int H, int I, int E, int k, int K, uint32_t mcg, int codebook, int x_dtype, const uint16_t *x,
              const int64_t *tok, int64_t n_tok, const uint16_t *router_w, const float *bias,
              const uint16_t *const *codes, const uint16_t *const *suh, const uint16_t *const *svh,
              const uint16_t *const *shared, const int32_t *ktab, const int8_t *signs, int shared_trellis,
              int32_t *idx_out, double *w_out, double *out, int nthreads);

static uint32_t rng_state = 12345u;
static uint16_t rnd16(void)
{
    rng_state = rng_state * 1664525u + 1013904223u;
    return (uint16_t)(rng_state >> 16);
}

static uint16_t *words(size_t n)
{
    uint16_t *w = (uint16_t *)malloc(n * sizeof(uint16_t));
    for (size_t i = 0; i < n; ++i)
        w[i] = rnd16();
    return w;
}

/* fp16 bits of a small positive value (exponent 0x0D: 2^-2 .. 2^-1) */
static uint16_t f16_small(void) { return (uint16_t)(0x3400 | (rnd16() & 0x3FF)); }

#define CHECK(c) do { if (!(c)) { fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); return 1; } } while (0)

int main(void)
{
    const uint32_t mcg = 0x9E3779B1u;
    CHECK(orc_mcg_value(0, mcg) == -254);
    for (int K = 2; K <= 4; ++K) {
        uint16_t *w = words(16 * K);
        uint16_t st[256];
        float vals[256];
        orc_stream_states(w, 16 * K, K, st);
        orc_decode_tile(w, K, mcg, 1, vals);
        for (int j = 0; j < 256; ++j)
            CHECK(fabsf(vals[j]) <= 4.0f);
        free(w);
        const int in = 48, out = 256;
        uint16_t *m = words((size_t)(in / 16) * (out / 16) * 16 * K);
        float *d = (float *)malloc(sizeof(float) * in * out);
        orc_decode_matrix(m, in, out, K, mcg, 0, d);
        for (int order = 0; order <= 2; ++order)
            CHECK(orc_decode_matrix_order(m, in, out, K, mcg, 0, order, d) == 0);
        CHECK(orc_decode_matrix_order(m, in, out, K, mcg, 0, 9, d) == -1);
        CHECK(orc_tile_position(2, in, out, 2, 15) == (15 / 8) * 3 * 8 + 2 * 8 + 7);
        free(m);
        free(d);
    }
    CHECK(orc_e4m3_rne(1000.0) == 448.0);
    CHECK(orc_codebook_value(0, mcg, 0) == -254.0 / 64.0);

    /* a layer with every option: per-tensor widths, rotation, trellis shared
     * expert, dense shared expert, router bias; then the plain layer */
    const int H = 256, I = 128, E = 8, k = 2, T = 5, EA = E + 1;
    uint16_t *x = (uint16_t *)malloc(sizeof(uint16_t) * T * H);
    for (int i = 0; i < T * H; ++i)
        x[i] = f16_small() ^ (uint16_t)((rnd16() & 1) << 15);
    uint16_t *rw = (uint16_t *)malloc(sizeof(uint16_t) * E * H);
    for (int i = 0; i < E * H; ++i)
        rw[i] = f16_small() ^ (uint16_t)((rnd16() & 1) << 15);
    float bias[8] = {0.1f, -0.2f, 0.3f, 0, 0, 0, NAN, 0};
    int32_t ktab[3 * 9];
    for (int i = 0; i < 3 * EA; ++i)
        ktab[i] = 2 + (int)(rnd16() % 3);
    const uint16_t *codes[3 * 9];
    uint16_t *own[3 * 9];
    for (int p = 0; p < 3; ++p)
        for (int e = 0; e < EA; ++e) {
            own[p * EA + e] = words((size_t)(H / 16) * (I / 16) * 16 * ktab[p * EA + e]);
            codes[p * EA + e] = own[p * EA + e];
        }
    uint16_t *suh[3], *svh[3], *shared[3];
    for (int p = 0; p < 3; ++p) {
        int n_in = p < 2 ? H : I, n_out = p < 2 ? I : H;
        suh[p] = (uint16_t *)malloc(sizeof(uint16_t) * EA * n_in);
        svh[p] = (uint16_t *)malloc(sizeof(uint16_t) * EA * n_out);
        for (int i = 0; i < EA * n_in; ++i)
            suh[p][i] = f16_small();
        for (int i = 0; i < EA * n_out; ++i)
            svh[p][i] = f16_small();
        shared[p] = (uint16_t *)malloc(sizeof(uint16_t) * H * I);
        for (int i = 0; i < H * I; ++i)
            shared[p][i] = (uint16_t)(f16_small() - 0x0C00);
    }
    uint16_t block[9 * 3 * 2];
    for (int i = 0; i < 9 * 3 * 2; ++i)
        block[i] = f16_small();
    orc_expand_block_scales(block, EA, H, I, suh, svh);
    int8_t signs[2 * 256];
    for (int i = 0; i < 2 * H; ++i)
        signs[i] = (rnd16() & 1) ? 1 : -1;
    int8_t hm[128 * 128];
    orc_sylvester(128, hm);
    double v[256];
    for (int i = 0; i < 256; ++i)
        v[i] = i;
    orc_rotate(v, 256, signs);
    int64_t tok[5] = {0, 1, 2, 3, 4};
    int32_t idx[5 * 2];
    double w[5 * 2], out[5 * 256];
    CHECK(orc_layer(H, I, E, k, 2, mcg, 1, 1, x, tok, T, rw, bias, codes, (const uint16_t *const *)suh,
                    (const uint16_t *const *)svh, (const uint16_t *const *)shared, ktab, signs, 1, idx, w, out,
                    2) == 0);
    for (int i = 0; i < T * k; ++i)
        CHECK(idx[i] >= 0 && idx[i] < E && idx[i] != 6);
    for (int p = 0; p < 3; ++p)
        for (int e = 0; e < E; ++e)
            ktab[p * E + e] = 3;   /* a uniform-width layer without the shared expert */
    const uint16_t *codes8[3 * 8];
    uint16_t *own8[3 * 8];
    for (int p = 0; p < 3; ++p)
        for (int e = 0; e < E; ++e) {
            own8[p * E + e] = words((size_t)(H / 16) * (I / 16) * 16 * 3);
            codes8[p * E + e] = own8[p * E + e];
        }
    CHECK(orc_layer(H, I, E, k, 3, mcg, 0, 2, x, tok, T, rw, NULL, codes8, (const uint16_t *const *)suh,
                    (const uint16_t *const *)svh, NULL, NULL, NULL, 0, idx, w, out, 1) == 0);
    /* every expert's gate at width 7: rejected before any decode */
    for (int e = 0; e < E; ++e)
        ktab[e] = 7;
    CHECK(orc_layer(H, I, E, k, 3, mcg, 0, 2, x, tok, T, rw, NULL, codes8, (const uint16_t *const *)suh,
                    (const uint16_t *const *)svh, NULL, ktab, NULL, 0, idx, w, out, 1) == -1);

    float lg[5 * 8];
    orc_router_logits(x, 2, T, H, rw, bias, E, lg);
    orc_topk_softmax(lg, T, E, k, idx, w);
    int32_t counts[8], offsets[9], sorted_ids[10], pos[10];
    orc_segments(idx, T, k, E, counts, offsets, sorted_ids, pos);
    CHECK(offsets[E] == T * k);

    for (int i = 0; i < 3 * EA; ++i)
        free(own[i]);
    for (int i = 0; i < 3 * E; ++i)
        free(own8[i]);
    for (int p = 0; p < 3; ++p) {
        free(suh[p]);
        free(svh[p]);
        free(shared[p]);
    }
    free(x);
    free(rw);
    printf("oracle driver: ok\n");
    return 0;
}
