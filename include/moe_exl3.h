/*
 * moe_exl3.h -- C ABI of the MI355X (gfx950) library for one MoE layer whose
 * routed experts are EXL3 K-bit trellis codes.
 *
 * What the layer computes (page "GLM-5.3 Flash EXL3 for 2x DGX Sparks",
 * section "Cold prefill (E3 grouped MoE)": gather, gate/up + SwiGLU, down +
 * scatter, built from device-side segment tables with no host sync; page
 * "GLM-5.3-Flash . exlr8 (K2/K3/K4)", section "Loading": 288 routed experts,
 * top-8, hidden 4096, expert intermediate 2048, one shared expert):
 *
 *   logits[t][e] = sum_h x[t][h] * router_w[e][h] (+ router_bias[e])   (fp32,
 *                  fixed order: 64 lane partial sums over h = 64i + l, added
 *                  in order of i, then a halving tree over l)
 *   idx[t][0..k) = top-k experts by (logit desc, expert asc)
 *   w[t][j]      = softmax of the k chosen logits
 *   for each (t, j), e = idx[t][j]:
 *     g = (x[t] * suh_g[e]) C_g[e] * svh_g[e]        u likewise
 *     y = ((silu(g) * u) * suh_d[e]) C_d[e] * svh_d[e]
 *   out[t] = sum_j w[t][j] y[t][j]  +  Wd (silu(Wg x[t]) * (Wu x[t]))   (shared)
 *
 * C_p[e] is the dense [in][out] matrix of decoded codebook values c = v/64.
 *
 * Trellis code layout (page "GLM-5.3-Flash EXL3 (~2.1 bpw, SM70 tile order)",
 * header: packed 16-bit words, 16/K weights each; page "GLM-5.3-Flash EXL3
 * K2", "What is in the shards": trellis, suh, svh, (1,) int32 mcg):
 *   codes[p]   uint16 [E][in/16][out/16][16*K]: one 16x16 tile per 16*K words,
 *              tiles row-major over (input block, output block).
 *   tile       a 256*K-bit stream, word 0 first, most significant bit first;
 *              state j = the 16 bits starting at bit j*K, wrapping inside the
 *              tile; state j is the weight at input row j % 16 and output
 *              column j / 16 of the tile.
 *   value      h = (mcg * state) mod 2^32;
 *              v = sum_{i=0..3} ((h >> (8i+1)) & 127) - 254;  c = v / 64.
 *   E4M3       with MOE_EXL3_CB_MCG_E4M3, c is rounded to OCP FP8 E4M3FN
 *              (nearest-even, saturating) before the side vectors (page
 *              "GLM-5.3-Flash . exlr8 (K2/K3/K4)", opening paragraph).
 *   gate, up   in = hidden, out = inter;  down: in = inter, out = hidden.
 *
 * Conventions for every entry point:
 *   - Pointers marked "device" point to device memory of the current HIP
 *     device, are owned by the caller and must stay valid until the work
 *     queued on `stream` has finished.  The library never allocates, frees or
 *     synchronises.  Apart from the per-GPU scratch array of
 *     moe_exl3_layer_noalloc (see there) it keeps no mutable global state, so
 *     calls on different streams are independent as long as each call has its
 *     own workspace.
 *   - `stream` is a hipStream_t (NULL = the null stream).
 *   - Return value: 0 on success or a negative MOE_EXL3_ERR_* code.  All
 *     argument checks run before the first launch; on error nothing is
 *     launched.  Faults inside kernels surface at the caller's next
 *     synchronisation, as HIP errors.
 *   - Device pointers must be 16-byte aligned (MOE_EXL3_ERR_MISALIGNED).
 */
#ifndef MOE_EXL3_H
#define MOE_EXL3_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_EXL3_ABI_VERSION 2

/* error codes */
#define MOE_EXL3_OK 0
#define MOE_EXL3_ERR_INVALID_ARG (-1)   /* NULL pointer, negative size, shape rule broken */
#define MOE_EXL3_ERR_UNSUPPORTED (-2)   /* K, dtype, codebook or size outside the kernels' range */
#define MOE_EXL3_ERR_WORKSPACE (-3)     /* workspace smaller than moe_exl3_workspace_size() */
#define MOE_EXL3_ERR_MISALIGNED (-4)    /* a device pointer is not 16-byte aligned */
#define MOE_EXL3_ERR_HIP (-5)           /* a launch failed (hipGetLastError) */

/* element types */
#define MOE_EXL3_DT_F32 0
#define MOE_EXL3_DT_F16 1
#define MOE_EXL3_DT_BF16 2
#define MOE_EXL3_DT_FP8 3   /* OCP E4M3FN bit patterns, one byte per value */
#define MOE_EXL3_DT_GEMV_F16 4   /* moe_exl3_decode only: fp16 128*c + 1532, the
                                    decode-fused GEMV's dot-product operand */
#define MOE_EXL3_DT_MFMA_BIASED_F16 5   /* moe_exl3_decode only, CB_MCG only: fp16
                                    128*c + 1532 from the gate/up MFMA's decoder
                                    of one-block (at most 32-row) tiles */

/* codebooks */
#define MOE_EXL3_CB_MCG 0
#define MOE_EXL3_CB_MCG_E4M3 1

/* desc.flags */
#define MOE_EXL3_HAS_SHARED (1u << 0)       /* add the fp16 shared expert */
#define MOE_EXL3_HAS_ROUTER_BIAS (1u << 1)  /* add router_bias to the logits */
#define MOE_EXL3_FORCE_GEMV (1u << 2)       /* raise the GEMV row threshold to its maximum, 8
                                               rows: experts with more rows still run on MFMA
                                               tiles, and with hidden > 8192 (the GEMV's LDS
                                               limit) every expert does */
#define MOE_EXL3_FORCE_MFMA (1u << 3)       /* every routed expert on the MFMA path */
#define MOE_EXL3_FP8_MFMA (1u << 4)         /* routed MFMA GEMMs in fp8 (needs CB_MCG_E4M3, hidden and
                                               inter % 256 == 0 and hidden <= 8192) */
#define MOE_EXL3_DEBUG_CHECKS (1u << 5)     /* extra launches that check the routing tables and
                                               the finiteness of x into the status word */
#define MOE_EXL3_DETERMINISTIC_COMBINE (1u << 6) /* accepted, always in effect: the k slot rows of
                                               a token and the shared expert are summed in
                                               fp32 in a fixed order, so the same inputs give
                                               the same bits on every call */
/*
 * Format variants (page "GLM-5.3-Flash . exlr8 (K2/K3/K4)"; page
 * "GLM-5.3-Flash-EXL3-TR3-3.5bpw"):
 *   HADAMARD        the trellis experts work in a rotated basis of the hidden
 *                   dimension ("Calibration": the 128x128 Hadamard matrix is a
 *                   format primitive; "Index slices": one pair of int8 sign
 *                   vectors over the hidden size per layer, weights.signs).
 *                   The experts read x' = R(s0 * x) and the layer adds
 *                   s1 * R(their weighted sum), R the block-diagonal matrix of
 *                   128x128 Sylvester-Hadamard blocks over sqrt(128).  The
 *                   router and the fp16 shared expert read x itself.  x' is
 *                   rounded to fp16 once.
 *   SHARED_TRELLIS  a trellis-coded shared expert stored as expert E after the
 *                   routed ones ("Loading": the shared expert is expert 288):
 *                   codes, suh and svh hold E + 1 experts, and expert E is
 *                   added for every token with weight 1, in the trellis
 *                   experts' basis.  Needs n_experts <= 1016.
 *   PER_TENSOR_K    every (projection, expert) tensor has its own width (the
 *                   TR3-3.5bpw settings table: each routed-expert tensor K3 or
 *                   K4): weights.k_tab and weights.code_tab replace desc.K and
 *                   codes[] (see moe_exl3_weights).
 */
#define MOE_EXL3_HADAMARD (1u << 7)
#define MOE_EXL3_SHARED_TRELLIS (1u << 8)
#define MOE_EXL3_PER_TENSOR_K (1u << 9)

/*
 * Status word.  Every moe_exl3_layer / moe_exl3_route call clears the int32
 * at byte MOE_EXL3_STATUS_OFFSET of its workspace in its first launch; later
 * launches set these bits in it.  It is valid once the call's work on the
 * stream has finished (the caller synchronises and reads it).  With a bit
 * other than ACT_RANGE set the outputs are unspecified.
 */
#define MOE_EXL3_STATUS_OFFSET 8
#define MOE_EXL3_STATUS_BAD_INDEX (1u << 0)      /* an expert index outside [0, E) reached the
                                                    segment tables (left out of them) */
#define MOE_EXL3_STATUS_TILE_OVERFLOW (1u << 1)  /* more MFMA row tiles than the workspace holds
                                                    (the list was cut) */
#define MOE_EXL3_STATUS_ACT_RANGE (1u << 2)      /* a finite bf16 activation beyond the fp16 range
                                                    (|x| >= 65520) became inf in the fp16 copy the
                                                    expert GEMMs read */
#define MOE_EXL3_STATUS_COUNTS (1u << 3)         /* DEBUG_CHECKS: counts do not sum to T*k */
#define MOE_EXL3_STATUS_TABLES (1u << 4)         /* DEBUG_CHECKS: offsets, sorted_ids or pos are
                                                    not the stable sort of idx */
#define MOE_EXL3_STATUS_NONFINITE_X (1u << 5)    /* DEBUG_CHECKS: x holds an inf or NaN */
#define MOE_EXL3_STATUS_BAD_WIDTH (1u << 6)      /* PER_TENSOR_K: a k_tab entry outside {2, 3, 4} */

/*
 * Layer description.  Shape rules: hidden is a multiple of 256, inter a
 * multiple of 128, both at most 16384; n_experts is a multiple of 8 and at
 * most 1024; 1 <= top_k <= min(n_experts, 16); K in {2, 3, 4}; act_dtype is
 * F16 or BF16; T * top_k < 2^31.
 *
 * Activation range: the expert GEMMs and the shared expert read an fp16 copy
 * of bf16 activations, exact for |x| in [2^-14, 65504]; smaller values round
 * as fp16 subnormals, and finite values of magnitude 65520 or more become inf
 * (flagged as MOE_EXL3_STATUS_ACT_RANGE).  The router reads x itself.
 * NaN logits rank below every number (as -inf, ties to the lower expert), so
 * the chosen experts are always valid; a token whose chosen logits are all
 * -inf or NaN gets NaN routing weights.
 */
typedef struct moe_exl3_desc {
    int32_t hidden;         /* H */
    int32_t inter;          /* I, expert (and shared expert) intermediate size */
    int32_t n_experts;      /* E */
    int32_t top_k;          /* k */
    int32_t K;              /* trellis bits per weight */
    int32_t codebook;       /* MOE_EXL3_CB_* */
    uint32_t mcg;           /* codebook multiplier (bit pattern of the int32 `mcg`) */
    int32_t act_dtype;      /* dtype of x and out */
    uint32_t flags;         /* MOE_EXL3_* flags */
    int32_t gemv_max_rows;  /* experts with at most this many routed rows use the
                               GEMV path (at most 8); 0 selects the default: 8 for
                               calls of at most 8 tokens (every expert on the GEMV
                               path), else 2 */
} moe_exl3_desc;

/*
 * Layer weights.  All device pointers, contiguous, row-major.  EA is the
 * number of trellis-coded experts: E, or E + 1 with SHARED_TRELLIS.
 */
typedef struct moe_exl3_weights {
    const uint16_t *codes[3];   /* gate, up, down: [EA][in/16][out/16][16K]; not read
                                   with PER_TENSOR_K */
    const uint16_t *suh[3];     /* fp16 [EA][in]  input-channel side vectors */
    const uint16_t *svh[3];     /* fp16 [EA][out] output-channel side vectors */
    const uint16_t *router_w;   /* fp16 [E][H] */
    const float *router_bias;   /* fp32 [E], read only with HAS_ROUTER_BIAS */
    const uint16_t *shared_w[3];/* fp16 nn.Linear weights: gate/up [I][H], down [H][I];
                                   read only with HAS_SHARED */
    const int8_t *signs;        /* int8 [2][H] (+1 / -1): s0 = signs[0], s1 = signs[1];
                                   read only with HADAMARD */
    const uint64_t *code_tab;   /* PER_TENSOR_K: device array [3][EA] of device addresses,
                                   the [in/16][out/16][16 K] words of tensor (p, e), each
                                   16-byte aligned */
    const int32_t *k_tab;       /* PER_TENSOR_K: device int32 [3][EA], the width of tensor
                                   (p, e), each 2, 3 or 4 (an entry outside that range
                                   sets MOE_EXL3_STATUS_BAD_WIDTH and the tensor is read
                                   as zero) */
} moe_exl3_weights;

/* ABI version (MOE_EXL3_ABI_VERSION). */
int moe_exl3_version(void);

/* Static description of an error code; never NULL. */
const char *moe_exl3_strerror(int code);

/*
 * Workspace bytes needed by moe_exl3_layer / moe_exl3_route for up to
 * `max_tokens` tokens (page "GLM-5.3 Flash EXL3 for 2x DGX Sparks", "Cold
 * prefill": the grouped path keeps a caller-visible scratch of gathered rows).
 * Host-only; touches no device.
 */
int moe_exl3_workspace_size(const moe_exl3_desc *desc, int64_t max_tokens, size_t *bytes);

/*
 * One MoE layer.  x: device [T][H] act_dtype; out: device [T][H] act_dtype,
 * must not overlap x.  T = 0 is a no-op.  The workspace is device memory of at
 * least moe_exl3_workspace_size(desc, T) bytes, 256-byte aligned; its content
 * on entry is ignored and on exit unspecified.
 */
int moe_exl3_layer(const moe_exl3_desc *desc, const moe_exl3_weights *weights, const void *x,
                   int64_t T, void *out, void *workspace, size_t ws_bytes, void *stream);

/*
 * moe_exl3_layer for callers that cannot allocate memory (code under HIP
 * graph capture, serving loops or harnesses that forbid hipMalloc): the
 * workspace is a device array of MOE_EXL3_SCRATCH_BYTES inside the library,
 * one per GPU, held from the first call on that GPU until the process ends.
 * The call itself allocates and frees nothing.  Every call on one GPU uses
 * the same array, so calls that overlap on one GPU (other streams, other
 * threads) race and must be ordered by the caller; the layer needs nothing
 * of the array's previous contents.  Returns MOE_EXL3_ERR_WORKSPACE when
 * moe_exl3_workspace_size(desc, T) exceeds MOE_EXL3_SCRATCH_BYTES (about 500
 * tokens at hidden 4096, inter 2048, top-8), MOE_EXL3_ERR_HIP when the array's
 * address cannot be taken; otherwise the same contract as moe_exl3_layer.
 * The status word sits at MOE_EXL3_STATUS_OFFSET of the array and is not
 * readable by the caller.
 */
#define MOE_EXL3_SCRATCH_BYTES (64u << 20)
int moe_exl3_layer_noalloc(const moe_exl3_desc *desc, const moe_exl3_weights *weights, const void *x,
                           int64_t T, void *out, void *stream);

/*
 * Routing and segment tables only (the layer's first steps, exposed for
 * bit-exact checks).  Outputs are device buffers:
 *   idx [T][k] int32, w [T][k] fp32 (softmax over the chosen logits),
 *   counts [E], offsets [E+1] (exclusive scan of counts),
 *   sorted_ids [T*k]: slots a = t*k + j grouped by expert ascending, and by a
 *   ascending within an expert; pos [T*k]: the inverse (sorted_ids[pos[a]] = a).
 * Any output pointer may be NULL except idx.
 */
int moe_exl3_route(const moe_exl3_desc *desc, const moe_exl3_weights *weights, const void *x,
                   int64_t T, int32_t *idx, float *w, int32_t *counts, int32_t *offsets,
                   int32_t *sorted_ids, int32_t *pos, void *workspace, size_t ws_bytes,
                   void *stream);

/*
 * moe_exl3_layer with timing hooks, for benchmarks and profilers: events[i]
 * (caller-created hipEvent_t handles) is recorded on `stream` right before
 * launch step i, and events[MOE_EXL3_STEP_END] after the last step.  Steps
 * skipped for this call are still recorded (at the same point).  n_events must
 * be MOE_EXL3_STEP_END + 1 and every handle non-NULL (else INVALID_ARG).  With
 * T = 0 nothing is launched or recorded.  Same contract as moe_exl3_layer
 * otherwise.
 */
#define MOE_EXL3_STEP_ROUTE_LOGITS 0
#define MOE_EXL3_STEP_TOPK 1
#define MOE_EXL3_STEP_SEGMENTS 2
#define MOE_EXL3_STEP_CONVERT_X 3
#define MOE_EXL3_STEP_GEMV_GATEUP 4
#define MOE_EXL3_STEP_MFMA_GATEUP 5
#define MOE_EXL3_STEP_GEMV_DOWN 6
#define MOE_EXL3_STEP_MFMA_DOWN 7
#define MOE_EXL3_STEP_SHARED 8
#define MOE_EXL3_STEP_COMBINE 9
#define MOE_EXL3_STEP_END 10
int moe_exl3_layer_profiled(const moe_exl3_desc *desc, const moe_exl3_weights *weights,
                            const void *x, int64_t T, void *out, void *workspace, size_t ws_bytes,
                            void *stream, void *const *events, int n_events);

/*
 * Dense decode of one trellis-coded [n_in][n_out] matrix (no side vectors),
 * for the bit-exact check of the decode (page "GLM-5.3-Flash EXL3 (~2.1 bpw,
 * SM70 tile order)", header: packed 16-bit words, 16/K weights each).  Each
 * dst_dtype runs the fragment decoder of one kernel of the layer:
 *   F16       dst = c in fp16, from the gate/up MFMA's decoder (exact)
 *   BF16      dst = c in bf16, from the down MFMA's decoder (exact)
 *   FP8       dst = E4M3FN bits of c, from the fp8 MFMA's decoder (exact for
 *             the E4M3 codebook; CB_MCG values are rounded to E4M3)
 *   GEMV_F16  dst = 128 c + 1532 in fp16, the decode-fused GEMV's operand (exact)
 *   MFMA_BIASED_F16  dst = 128 c + 1532 in fp16, from the gate/up MFMA's decoder
 *             of one-block tiles (exact; CB_MCG only, else UNSUPPORTED: with
 *             the E4M3 codebook those tiles use the F16 decoder)
 *   F32       dst = c in fp32 (exact)
 * codes: device [n_in/16][n_out/16][16K] uint16; dst: device, row-major.
 * n_in and n_out are positive multiples of 16.
 */
int moe_exl3_decode(const uint16_t *codes, int32_t n_in, int32_t n_out, int32_t K, uint32_t mcg,
                    int32_t codebook, void *dst, int32_t dst_dtype, void *stream);

/*
 * Load-time tile reorder of `count` trellis tensors, each an [n_in/16][n_out/16]
 * grid of 16x16 tiles (16 K words per tile), from a stored tile order into the
 * row-major grid every kernel reads (page "GLM-5.3-Flash EXL3 (~2.1 bpw, SM70
 * tile order)", header: the checkpoint's column-major tile order is reordered
 * by the loader into the kernels' layout; page "GLM-5.3-Flash . exlr8
 * (K2/K3/K4)", "Loading": each projection in halves of 128 intermediate
 * channels).  A tile is a self-contained trellis stream, so this is a byte
 * copy of whole tiles; the tiles' own content is unchanged.  Position, in
 * tiles, of tile (tk, tn) in src:
 *   ORDER_ROWMAJOR     tk * (n_out/16) + tn  (the kernels' order: a plain copy)
 *   ORDER_COLMAJOR     tn * (n_in/16) + tk
 *   ORDER_COLGROUPS128 (tn/8) * (n_in/16) * 8 + tk * 8 + tn % 8: groups of 128
 *                      output columns one after another, each row-major (a
 *                      gate or up projection stored as halves of 4096 x 128;
 *                      a down projection split by input rows is ROWMAJOR).
 *                      Needs n_out % 128 == 0.
 * src, dst: device, count * (n_in/16) * (n_out/16) * 16 K uint16 each,
 * 16-byte aligned, not overlapping.  count >= 1; n_in, n_out positive
 * multiples of 16; K in {2, 3, 4}.
 */
#define MOE_EXL3_ORDER_ROWMAJOR 0
#define MOE_EXL3_ORDER_COLMAJOR 1
#define MOE_EXL3_ORDER_COLGROUPS128 2
int moe_exl3_repack(const uint16_t *src, uint16_t *dst, int32_t count, int32_t n_in, int32_t n_out, int32_t K,
                    int32_t src_order, void *stream);

/*
 * Per-channel side vectors from block scales (page "GLM-5.3-Flash . exlr8
 * (K2/K3/K4)", "Index slices": an F16 block table [EA][3][hidden/128] per
 * layer, the shared expert as its last row; "Loading": 32 block scales per
 * projection at hidden 4096).  A scale covers 128 channels of the hidden
 * dimension, which is the input of gate and up and the output of down:
 *   suh[0][e][k] = block[e][0][k/128]   suh[1][e][k] = block[e][1][k/128]
 *   svh[2][e][m] = block[e][2][m/128]
 * and the intermediate-side vectors svh[0], svh[1], suh[2] are set to 1.
 * block: device fp16 [n_trellis][3][hidden/128]; suh, svh: host arrays of 3
 * device pointers to the fp16 vectors laid out as in moe_exl3_weights
 * (suh[p] [n_trellis][in], svh[p] [n_trellis][out]).  hidden is a positive
 * multiple of 128, inter positive, n_trellis >= 1; pointers 16-byte aligned.
 */
int moe_exl3_expand_block_scales(const uint16_t *block, int32_t n_trellis, int32_t hidden, int32_t inter,
                                 uint16_t *const *suh, uint16_t *const *svh, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_EXL3_H */
