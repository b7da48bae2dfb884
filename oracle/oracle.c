/*
 * CPU oracle for one EXL3 trellis-coded MoE layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  It shares no code,
 * header, table or constant generator with the HIP library; it is a plain,
 * slow, direct statement of what the layer computes.
 *
 * Sources (page titles; each function cites the passage it follows):
 *   [p1] "GLM-5.3-Flash EXL3 (~2.1 bpw, SM70 tile order)", header paragraph:
 *        EXL3 tensors are packed 16-bit trellis words holding 16/K weights each.
 *   [p2] "GLM-5.3 Flash EXL3 for 2x DGX Sparks", "Cold prefill (E3 grouped MoE)"
 *        (gather, gate/up + SwiGLU, down + scatter, device segment tables) and
 *        "What runs" (the routed experts are EXL3 trellis tensors with their
 *        side vectors, read through the MCG codebook).
 *   [p3] "GLM-5.3-Flash EXL3 K2", "What is in the shards": per expert tensor
 *        `suh`, `svh`, `trellis` and a (1,) int32 `mcg`.
 *   [p4] "GLM-5.3-Flash . exlr8 (K2/K3/K4)": opening paragraph (round every
 *        codebook value to FP8 E4M3, nearest-even, saturating, before the side
 *        vectors) and "Loading" (4096 x 128 gate/up halves, 288 experts top-8,
 *        one shared expert).
 *   [p5] "GLM-5.3-Flash-EXL3-TR3-3.5bpw": shared expert left unquantized; its
 *        settings table gives every routed-expert tensor its own width (K3 or
 *        K4), which the tensor's payload shape carries.
 *   [p4] "Index slices" and "Calibration": per layer, one pair of int8 sign
 *        vectors over the hidden size (`signs` [2, 4096]) and the 128x128
 *        Hadamard matrix as a primitive of the format; "Loading": the shared
 *        expert stored as trellis expert 288 after the routed ones, each
 *        projection in halves of 128 intermediate channels.
 *
 * Where the pages are silent the readings below are this project's own and
 * are listed with their reasons in the design notes:
 *   value map   h = (mcg * s) mod 2^32; v = sum_{i=0..3} ((h >> (8i+1)) & 127) - 254;
 *               c = v / 64
 *   stream      a tile's 16K words form a 256K-bit stream, most significant
 *               bit of word 0 first; state j is the 16 bits starting at bit
 *               j*K, read circularly (tail-biting) and first bit most significant
 *   tile order  state j of a tile sits at input row 16*tk + (j % 16) and output
 *               column 16*tn + (j / 16); tile (tk, tn) starts at word
 *               (tk * (out/16) + tn) * 16K of the expert's [in/16][out/16] grid
 *   side vecs   W[k][n] = suh[k] * c[k][n] * svh[n]
 *   router      fp32 logits in a fixed order (64 lane partial sums, then a
 *               halving tree), top-k by (logit desc, index asc; a NaN logit
 *               ranks as -inf), softmax over the k chosen logits
 *   segments    stable counting sort of a = t*k + j by expert
 *   combine     out[t] = sum_j w[t][j] * y[t][j] + shared(x[t])
 *   rotation    optional: the trellis experts work in a rotated basis of the
 *               hidden dimension, x' = R(s0 * x) and out = s1 * R(expert sum),
 *               R the block-diagonal 128x128 Hadamard matrix over 2^(7/2),
 *               s0, s1 the layer's two sign vectors; the router and the fp16
 *               shared expert see x itself
 *   widths      optional: a width K per (projection, expert) tensor
 *   shared      optional: a trellis-coded shared expert stored as expert E
 *               after the routed ones, added with weight 1 in the experts'
 *               basis
 *
 * Precision: routing decides integers, so logits are fp32 in the fixed order,
 * every step a fused multiply-add (the exact product added to the partial sum
 * with one rounding to fp32).  Everything after routing is carried in fp64.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_DT_F32 0
#define ORC_DT_F16 1
#define ORC_DT_BF16 2
#define ORC_CB_MCG 0
#define ORC_CB_MCG_E4M3 1

/* IEEE binary16 -> double, from the format definition (bias 15, 10-bit mantissa). */
double orc_f16_to_double(uint16_t h)
{
    int sign = h >> 15, ex = (h >> 10) & 0x1F, man = h & 0x3FF;
    double v;
    if (ex == 0)
        v = ldexp((double)man, -24);
    else if (ex == 31)
        v = man ? NAN : INFINITY;
    else
        v = ldexp((double)(man | 0x400), ex - 25);
    return sign ? -v : v;
}

/* bfloat16 = the upper 16 bits of an IEEE binary32. */
double orc_bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

static double act_to_double(uint16_t bits, int dtype)
{
    return dtype == ORC_DT_BF16 ? orc_bf16_to_double(bits) : orc_f16_to_double(bits);
}

/* Codebook value map: multiplicative congruential hash of the 16-bit state
 * with the tensor's `mcg` multiplier ([p3] "What is in the shards"; [p2]
 * "What runs": codebook MCG), then the sum of four 7-bit fields of the hash,
 * centred.  Returns v in [-254, 254]; the weight value is v / 64. */
int orc_mcg_value(uint32_t state, uint32_t mcg)
{
    uint32_t h = (uint32_t)(((uint64_t)mcg * (uint64_t)state) & 0xFFFFFFFFu);
    int sum = 0;
    for (int i = 0; i < 4; ++i)
        sum += (int)((h >> (8 * i + 1)) & 0x7Fu);
    return sum - 254;
}

/* States of a tail-biting K-bit trellis stream held in `nwords` 16-bit words
 * ([p1] header: each word holds 16/K weights).  There are 16*nwords/K states;
 * state j is the 16-bit window starting at stream bit j*K, wrapping at the end
 * of the stream, first bit most significant.  Stream bit p is bit 15 - p%16
 * of word p/16. */
void orc_stream_states(const uint16_t *words, int nwords, int K, uint16_t *states)
{
    int B = 16 * nwords, n = B / K;
    for (int j = 0; j < n; ++j) {
        uint32_t s = 0;
        for (int t = 0; t < 16; ++t) {
            int p = (j * K + t) % B;
            uint32_t bit = (words[p / 16] >> (15 - p % 16)) & 1u;
            s = (s << 1) | bit;
        }
        states[j] = (uint16_t)s;
    }
}

/* OCP FP8 E4M3FN rounding ([p4] opening paragraph: nearest-even, saturating).
 * E4M3FN has 3 mantissa bits, exponent bias 7, smallest normal 2^-6,
 * subnormal spacing 2^-9, largest finite 448 and no infinities. */
double orc_e4m3_rne(double x)
{
    if (x != x || x == 0.0)
        return x;
    double a = fabs(x);
    int e2;
    frexp(a, &e2);            /* a = f * 2^e2 with f in [0.5, 1) */
    int ex = e2 - 1;          /* floor(log2 a) */
    if (ex < -6)
        ex = -6;              /* subnormal range shares the 2^-9 spacing */
    double q = ldexp(1.0, ex - 3);
    double r = rint(a / q) * q;   /* default rounding mode: ties to even */
    if (r > 448.0)
        r = 448.0;
    return copysign(r, x);
}

/* Decoded weight value of one state, before the side vectors: c = v / 64, or
 * its E4M3 rounding for the exlr8 codebook variant ([p4]). */
double orc_codebook_value(uint32_t state, uint32_t mcg, int codebook)
{
    double c = (double)orc_mcg_value(state, mcg) / 64.0;
    return codebook == ORC_CB_MCG_E4M3 ? orc_e4m3_rne(c) : c;
}

/* Decode one 16x16 tile (16K words) into 256 values indexed by state j. */
void orc_decode_tile(const uint16_t *words, int K, uint32_t mcg, int codebook, float *vals)
{
    uint16_t st[256];
    orc_stream_states(words, 16 * K, K, st);
    for (int j = 0; j < 256; ++j)
        vals[j] = (float)orc_codebook_value(st[j], mcg, codebook);
}

/* Decode a whole [in][out] projection stored as an [in/16][out/16] grid of
 * tiles into a dense row-major fp32 matrix (every value is exact in fp32). */
void orc_decode_matrix(const uint16_t *codes, int in, int out, int K, uint32_t mcg,
                       int codebook, float *dst)
{
    int ntn = out / 16, ntk = in / 16;
#pragma omp parallel for schedule(static)
    for (int tk = 0; tk < ntk; ++tk) {
        float vals[256];
        for (int tn = 0; tn < ntn; ++tn) {
            const uint16_t *w = codes + ((size_t)tk * ntn + tn) * 16 * (size_t)K;
            orc_decode_tile(w, K, mcg, codebook, vals);
            for (int j = 0; j < 256; ++j) {
                int r = j % 16, c = j / 16;
                dst[(size_t)(16 * tk + r) * out + 16 * tn + c] = vals[j];
            }
        }
    }
}

/* Tile orders a checkpoint may store a projection's [in/16][out/16] tile grid
 * in ([p1] header: a column-major tile order recorded in the quantization
 * config, which the loader reorders to the kernels' own layout; [p4]
 * "Loading": each projection in halves of 128 intermediate channels).  The
 * function gives the position, in units of one tile, of tile (tk, tn):
 *   0  row-major grid:    tk * (out/16) + tn (the layout every kernel reads)
 *   1  column-major grid: tn * (in/16) + tk
 *   2  groups of 128 output columns stored one after another, each a
 *      row-major grid of in/16 x 8 tiles: (tn/8) * (in/16) * 8 + tk * 8 + tn%8
 *      (a gate or up half of 4096 x 128; a down half, which splits the input
 *      dimension, is order 0)
 * Returns -1 for an unknown order. */
int64_t orc_tile_position(int order, int in, int out, int tk, int tn)
{
    int64_t ntk = in / 16, ntn = out / 16;
    switch (order) {
    case 0: return (int64_t)tk * ntn + tn;
    case 1: return (int64_t)tn * ntk + tk;
    case 2: return (int64_t)(tn / 8) * ntk * 8 + (int64_t)tk * 8 + tn % 8;
    default: return -1;
    }
}

/* Dense decode of a projection whose tiles are stored in `order`. */
int orc_decode_matrix_order(const uint16_t *codes, int in, int out, int K, uint32_t mcg,
                            int codebook, int order, float *dst)
{
    if (orc_tile_position(order, in, out, 0, 0) < 0 || (order == 2 && out % 128))
        return -1;
    int ntn = out / 16, ntk = in / 16;
#pragma omp parallel for schedule(static)
    for (int tk = 0; tk < ntk; ++tk) {
        float vals[256];
        for (int tn = 0; tn < ntn; ++tn) {
            const uint16_t *w = codes + orc_tile_position(order, in, out, tk, tn) * 16 * (int64_t)K;
            orc_decode_tile(w, K, mcg, codebook, vals);
            for (int j = 0; j < 256; ++j)
                dst[(size_t)(16 * tk + j % 16) * out + 16 * tn + j / 16] = vals[j];
        }
    }
    return 0;
}

/* Side vectors from the exlr8 block table ([p4] "Index slices": F16 block
 * scales [EA][3][H/128] per layer; "Loading": 32 per projection at hidden
 * 4096).  This project's reading: a scale covers 128 channels of the hidden
 * dimension, the input of gate and up and the output of down; the
 * intermediate side carries no scale (1).
 *   suh_g[e][k] = block[e][0][k/128]   suh_u[e][k] = block[e][1][k/128]
 *   svh_d[e][m] = block[e][2][m/128]   svh_g = svh_u = suh_d = 1
 * suh[p], svh[p] as in orc_layer ([EA][in], [EA][out]). */
void orc_expand_block_scales(const uint16_t *block, int EA, int H, int I, uint16_t *const *suh,
                             uint16_t *const *svh)
{
    const uint16_t one = 0x3C00; /* fp16 1.0 */
    int nb = H / 128;
    for (int e = 0; e < EA; ++e) {
        for (int k = 0; k < H; ++k) {
            suh[0][(size_t)e * H + k] = block[((size_t)e * 3 + 0) * nb + k / 128];
            suh[1][(size_t)e * H + k] = block[((size_t)e * 3 + 1) * nb + k / 128];
            svh[2][(size_t)e * H + k] = block[((size_t)e * 3 + 2) * nb + k / 128];
        }
        for (int n = 0; n < I; ++n) {
            svh[0][(size_t)e * I + n] = one;
            svh[1][(size_t)e * I + n] = one;
            suh[2][(size_t)e * I + n] = one;
        }
    }
}

/* One accumulation step of a router partial sum: p + x * w with a single
 * rounding to fp32 (a fused multiply-add).  The product of a bf16 or fp16
 * activation and an fp16 weight has at most 22 significant bits, so it is
 * exact in double.  The double sum is then either exact (the leading bits of
 * the two terms lie within 28 places of each other) or the smaller term is
 * below 2^-3 of half an fp32 ulp of the larger, which is itself an fp32 number;
 * in both cases rounding the double sum to float gives
 * the correctly rounded fp32 value of p + x * w.  Where the product is a normal
 * fp32 number it is exact in fp32 as well, and the step equals a separate
 * multiply and add; the two differ only for products below fp32's normal
 * range. */
static float fused_step(float p, float x, float w) { return (float)((double)p + (double)x * (double)w); }

/* Router logits in fp32 ([p1] "Recipe" and [p4] "Intended use": routers stay
 * in source precision because routing is sensitive).  For each (t, e): 64
 * partial sums p[l] accumulate x[t][64i+l] * Wr[e][64i+l] for i = 0, 1, ...
 * in order, one fused step each; then p[l] += p[l+d] for d = 32, 16, 8, 4,
 * 2, 1; logit = p[0] (+ bias[e]). */
void orc_router_logits(const uint16_t *x, int x_dtype, int64_t T, int H, const uint16_t *Wr,
                       const float *bias, int E, float *logits)
{
    /* every bf16 / fp16 value is exact in fp32 */
    float *wf = (float *)malloc(sizeof(float) * (size_t)E * H);
    for (size_t i = 0; i < (size_t)E * H; ++i)
        wf[i] = (float)orc_f16_to_double(Wr[i]);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = 0; t < T; ++t) {
        float *xf = (float *)malloc(sizeof(float) * H);
        for (int hh = 0; hh < H; ++hh)
            xf[hh] = (float)act_to_double(x[t * H + hh], x_dtype);
        for (int e = 0; e < E; ++e) {
            const float *we = wf + (size_t)e * H;
            float p[64];
            for (int l = 0; l < 64; ++l)
                p[l] = 0.0f;
            for (int i = 0; i < H / 64; ++i)
                for (int l = 0; l < 64; ++l)
                    p[l] = fused_step(p[l], xf[64 * i + l], we[64 * i + l]);
            for (int d = 32; d >= 1; d /= 2)
                for (int l = 0; l < d; ++l)
                    p[l] = p[l] + p[l + d];
            logits[t * E + e] = bias ? p[0] + bias[e] : p[0];
        }
        free(xf);
    }
    free(wf);
}

/* Top-k of each token's logits by (logit descending, expert ascending), and
 * softmax weights over the k chosen logits ([p4] "Loading": 288 experts with
 * top-8 routing), computed in fp64 from the fp32 logits.  The pages do not
 * say how a NaN logit ranks; here it ranks as -inf (below every number, tied
 * with -inf and, like any tie, broken by the lower expert index), so every
 * chosen index is a valid expert.  The softmax takes the ranked values: a NaN
 * logit enters it as -inf. */
static double rank_key(float v) { return v != v ? -INFINITY : (double)v; }

void orc_topk_softmax(const float *logits, int64_t T, int E, int k, int32_t *idx, double *w)
{
    char *chosen = (char *)malloc((size_t)E);
    for (int64_t t = 0; t < T; ++t) {
        const float *l = logits + t * E;
        memset(chosen, 0, (size_t)E);
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e)
                if (!chosen[e] && (best < 0 || rank_key(l[e]) > rank_key(l[best])))
                    best = e;
            chosen[best] = 1;
            idx[t * k + j] = best;
        }
        double l0 = rank_key(l[idx[t * k]]), sum = 0.0;
        for (int j = 0; j < k; ++j)
            sum += exp(rank_key(l[idx[t * k + j]]) - l0);
        for (int j = 0; j < k; ++j)
            w[t * k + j] = exp(rank_key(l[idx[t * k + j]]) - l0) / sum;
    }
    free(chosen);
}

/* Segment tables ([p2] "Cold prefill (E3 grouped MoE)": device-side segment
 * tables in place of a per-expert host loop): counts per expert, exclusive
 * offsets (E+1 entries), the slots a = t*k + j grouped by expert ascending and
 * by a ascending within an expert, and pos[a], the inverse permutation. */
void orc_segments(const int32_t *idx, int64_t T, int k, int E, int32_t *counts,
                  int32_t *offsets, int32_t *sorted_ids, int32_t *pos)
{
    int64_t n = T * k;
    int32_t *fill = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
    for (int e = 0; e < E; ++e)
        counts[e] = 0;
    for (int64_t a = 0; a < n; ++a)
        counts[idx[a]]++;
    offsets[0] = 0;
    for (int e = 0; e < E; ++e)
        offsets[e + 1] = offsets[e] + counts[e];
    for (int e = 0; e < E; ++e)
        fill[e] = offsets[e];
    for (int64_t a = 0; a < n; ++a) {
        int32_t p = fill[idx[a]]++;
        sorted_ids[p] = (int32_t)a;
        pos[a] = p;
    }
    free(fill);
}

/* Hadamard matrix of order n (a power of two) by Sylvester's construction:
 * H_1 = [1], H_2m = [[H_m, H_m], [H_m, -H_m]] ([p4] "Calibration": the 128x128
 * Hadamard matrix is one of the format's primitives).  Hm is n x n int8. */
void orc_sylvester(int n, int8_t *Hm)
{
    Hm[0] = 1;
    for (int m = 1; m < n; m *= 2)
        for (int i = 0; i < m; ++i)
            for (int j = 0; j < m; ++j) {
                int8_t v = Hm[i * n + j];
                Hm[i * n + j + m] = v;
                Hm[(i + m) * n + j] = v;
                Hm[(i + m) * n + j + m] = (int8_t)-v;
            }
}

/* Block rotation of a vector of length len (a multiple of 128), optionally
 * after an elementwise sign vector: u = s * v (s NULL: u = v), then each block
 * of 128 is replaced by H_128 u_block / sqrt(128), a matrix product with the
 * Sylvester matrix.  H_128 is symmetric and H_128 H_128 = 128 I, so the
 * rotation is orthonormal and its own inverse. */
void orc_rotate(double *v, int len, const int8_t *s)
{
    int8_t Hm[128 * 128];
    orc_sylvester(128, Hm);
    double u[128];
    for (int b = 0; b < len; b += 128) {
        for (int j = 0; j < 128; ++j)
            u[j] = s ? (double)s[b + j] * v[b + j] : v[b + j];
        for (int i = 0; i < 128; ++i) {
            double acc = 0.0;
            for (int j = 0; j < 128; ++j)
                acc += (double)Hm[i * 128 + j] * u[j];
            v[b + i] = acc / sqrt(128.0);
        }
    }
}

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* Routed rows of one trellis expert: for each listed row r (token row tr[r]
 * of xin, weight wr[r]) ([p2] "Cold prefill": gate/up + SwiGLU, then down +
 * scatter):
 *   g[n] = svh_g[n] * sum_k xin[k] suh_g[k] c_g[k][n]       (u likewise)
 *   h[n] = silu(g[n]) * u[n]
 *   y[m] = svh_d[m] * sum_n h[n] suh_d[n] c_d[n][m]
 *   acc[tr[r]] += wr[r] * y
 * c_p is the expert's decoded projection p at width Kp[p]. */
static void expert_rows(int H, int I, const int Kp[3], uint32_t mcg, int codebook,
                        const uint16_t *const cw[3], const uint16_t *suh_g, const uint16_t *suh_u,
                        const uint16_t *suh_d, const uint16_t *svh_g, const uint16_t *svh_u,
                        const uint16_t *svh_d, const double *xin, const int64_t *tr,
                        const double *wr, int64_t nr, double *acc)
{
    float *cg = (float *)malloc(sizeof(float) * (size_t)H * I);
    float *cu = (float *)malloc(sizeof(float) * (size_t)H * I);
    float *cd = (float *)malloc(sizeof(float) * (size_t)I * H);
    double *xs_g = (double *)malloc(sizeof(double) * H);
    double *xs_u = (double *)malloc(sizeof(double) * H);
    double *hs = (double *)malloc(sizeof(double) * I);
    double *y = (double *)malloc(sizeof(double) * H);
    orc_decode_matrix(cw[0], H, I, Kp[0], mcg, codebook, cg);
    orc_decode_matrix(cw[1], H, I, Kp[1], mcg, codebook, cu);
    orc_decode_matrix(cw[2], I, H, Kp[2], mcg, codebook, cd);
    for (int64_t r = 0; r < nr; ++r) {
        const double *xt = xin + tr[r] * H;
        for (int kk = 0; kk < H; ++kk) {
            xs_g[kk] = xt[kk] * orc_f16_to_double(suh_g[kk]);
            xs_u[kk] = xt[kk] * orc_f16_to_double(suh_u[kk]);
        }
        /* columns in blocks of 64 so that each pass over k reads rows */
#pragma omp parallel for schedule(static)
        for (int n0 = 0; n0 < I; n0 += 64) {
            int nn = I - n0 < 64 ? I - n0 : 64;
            double sg[64], su[64];
            for (int c = 0; c < nn; ++c)
                sg[c] = su[c] = 0.0;
            for (int kk = 0; kk < H; ++kk) {
                const float *rg = cg + (size_t)kk * I + n0, *ru = cu + (size_t)kk * I + n0;
                for (int c = 0; c < nn; ++c) {
                    sg[c] += xs_g[kk] * (double)rg[c];
                    su[c] += xs_u[kk] * (double)ru[c];
                }
            }
            for (int c = 0; c < nn; ++c) {
                int n = n0 + c;
                double g = sg[c] * orc_f16_to_double(svh_g[n]);
                double u = su[c] * orc_f16_to_double(svh_u[n]);
                hs[n] = silu(g) * u * orc_f16_to_double(suh_d[n]);
            }
        }
#pragma omp parallel for schedule(static)
        for (int m0 = 0; m0 < H; m0 += 64) {
            int mm = H - m0 < 64 ? H - m0 : 64;
            double sacc[64];
            for (int c = 0; c < mm; ++c)
                sacc[c] = 0.0;
            for (int n = 0; n < I; ++n) {
                const float *rd = cd + (size_t)n * H + m0;
                for (int c = 0; c < mm; ++c)
                    sacc[c] += hs[n] * (double)rd[c];
            }
            for (int c = 0; c < mm; ++c)
                y[m0 + c] = sacc[c] * orc_f16_to_double(svh_d[m0 + c]);
        }
        double *at = acc + tr[r] * H;
        for (int m = 0; m < H; ++m)
            at[m] += wr[r] * y[m];
    }
    free(cg);
    free(cu);
    free(cd);
    free(xs_g);
    free(xs_u);
    free(hs);
    free(y);
}

/*
 * The layer for a subset of tokens, in fp64 after routing.
 *
 *   E               routed experts; the trellis tensors hold EA = E experts,
 *                   or EA = E + 1 with shared_trellis (the shared expert is
 *                   stored as expert E after the routed ones, [p4] "Loading")
 *   codes[p*EA + e] words of expert e, projection p (0 gate, 1 up, 2 down);
 *                   may be NULL for routed experts no selected token routes to
 *   K, ktab         width of every tensor: ktab[p*EA + e] when ktab is not
 *                   NULL ([p5] settings table: every tensor its own width),
 *                   K otherwise
 *   suh[p], svh[p]  fp16 [EA][in], [EA][out]
 *   signs           NULL, or int8 [2][H] sign vectors ([p4] "Index slices"):
 *                   the trellis experts then see x' = R(signs[0] * x) and the
 *                   layer adds signs[1] * R(their weighted sum), R the
 *                   orthonormal block rotation of orc_rotate
 *   shared[p]       fp16 nn.Linear weights (gate/up [I][H], down [H][I]) or
 *                   NULL: the unquantized shared expert ([p1] "Recipe"; [p5]),
 *                   added with weight 1 on x itself:
 *                   out[t] += Wd (silu(Wg x) * (Wu x))
 *
 * Routing (logits, top-k, softmax) always reads x.  Each selected token's k
 * routed experts are added with their routing weights, the trellis shared
 * expert with weight 1 (expert_rows).
 *
 * Returns 0, or -1 if a needed expert's codes are NULL or a width is not 2, 3
 * or 4.
 */
int orc_layer(int H, int I, int E, int k, int K, uint32_t mcg, int codebook, int x_dtype,
              const uint16_t *x, const int64_t *tok, int64_t n_tok, const uint16_t *router_w,
              const float *bias, const uint16_t *const *codes, const uint16_t *const *suh,
              const uint16_t *const *svh, const uint16_t *const *shared, const int32_t *ktab,
              const int8_t *signs, int shared_trellis, int32_t *idx_out, double *w_out,
              double *out, int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    const int EA = E + (shared_trellis ? 1 : 0);
    float *lg = (float *)malloc(sizeof(float) * (size_t)E);
    for (int64_t i = 0; i < n_tok; ++i) {
        orc_router_logits(x + tok[i] * H, x_dtype, 1, H, router_w, bias, E, lg);
        orc_topk_softmax(lg, 1, E, k, idx_out + i * k, w_out + i * k);
    }
    free(lg);

    /* the trellis experts' input rows, rotated when sign vectors are given */
    double *xin = (double *)malloc(sizeof(double) * (size_t)n_tok * H);
    double *acc = (double *)calloc((size_t)n_tok * H, sizeof(double));
    for (int64_t ti = 0; ti < n_tok; ++ti) {
        for (int kk = 0; kk < H; ++kk)
            xin[ti * H + kk] = act_to_double(x[tok[ti] * H + kk], x_dtype);
        if (signs)
            orc_rotate(xin + ti * H, H, signs);
    }
    int64_t *tr = (int64_t *)malloc(sizeof(int64_t) * (size_t)(n_tok * k + n_tok + 1));
    double *wr = (double *)malloc(sizeof(double) * (size_t)(n_tok * k + n_tok + 1));
    int rc = 0;

    for (int e = 0; e < EA && rc == 0; ++e) {
        int64_t nr = 0;
        if (e < E) {
            for (int64_t a = 0; a < n_tok * k; ++a)
                if (idx_out[a] == e) {
                    tr[nr] = a / k;
                    wr[nr] = w_out[a];
                    ++nr;
                }
        } else {
            for (int64_t ti = 0; ti < n_tok; ++ti) {
                tr[nr] = ti;
                wr[nr] = 1.0;
                ++nr;
            }
        }
        if (nr == 0)
            continue;
        int Kp[3];
        const uint16_t *cw[3];
        for (int p = 0; p < 3; ++p) {
            Kp[p] = ktab ? ktab[p * EA + e] : K;
            cw[p] = codes[p * EA + e];
            if (!cw[p] || Kp[p] < 2 || Kp[p] > 4)
                rc = -1;
        }
        if (rc)
            break;
        expert_rows(H, I, Kp, mcg, codebook, cw, suh[0] + (size_t)e * H, suh[1] + (size_t)e * H,
                    suh[2] + (size_t)e * I, svh[0] + (size_t)e * I, svh[1] + (size_t)e * I,
                    svh[2] + (size_t)e * H, xin, tr, wr, nr, acc);
    }

    for (int64_t ti = 0; ti < n_tok && rc == 0; ++ti) {
        double *at = acc + ti * H;
        if (signs) {
            orc_rotate(at, H, NULL);
            for (int m = 0; m < H; ++m)
                at[m] *= (double)signs[H + m];
        }
        memcpy(out + ti * H, at, sizeof(double) * H);
    }

    if (rc == 0 && shared && shared[0] && shared[1] && shared[2]) {
        double *xs = (double *)malloc(sizeof(double) * H);
        double *hs = (double *)malloc(sizeof(double) * I);
        for (int64_t ti = 0; ti < n_tok; ++ti) {
            const uint16_t *xt = x + tok[ti] * H;
            for (int kk = 0; kk < H; ++kk)
                xs[kk] = act_to_double(xt[kk], x_dtype);
#pragma omp parallel for schedule(static)
            for (int n = 0; n < I; ++n) {
                double sg = 0.0, su = 0.0;
                const uint16_t *wg = shared[0] + (size_t)n * H, *wu = shared[1] + (size_t)n * H;
                for (int kk = 0; kk < H; ++kk) {
                    sg += orc_f16_to_double(wg[kk]) * xs[kk];
                    su += orc_f16_to_double(wu[kk]) * xs[kk];
                }
                hs[n] = silu(sg) * su;
            }
#pragma omp parallel for schedule(static)
            for (int m = 0; m < H; ++m) {
                double sacc = 0.0;
                const uint16_t *wd = shared[2] + (size_t)m * I;
                for (int n = 0; n < I; ++n)
                    sacc += orc_f16_to_double(wd[n]) * hs[n];
                out[ti * H + m] += sacc;
            }
        }
        free(xs);
        free(hs);
    }

    free(xin);
    free(acc);
    free(tr);
    free(wr);
    return rc;
}
