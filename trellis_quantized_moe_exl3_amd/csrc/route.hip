// Routing (fp32 router logits in a fixed order, top-k, softmax) and
// device-side segment tables (page "GLM-5.3 Flash EXL3 for 2x DGX Sparks",
// "Cold prefill (E3 grouped MoE)": segment tables built on the device, no
// per-expert launches, no host sync).
#include <algorithm>

#include "common.h"
#include "gemm.h"
#include "internal.h"

namespace moe {

// ---------------------------------------------------------------- router logits
// Fixed order: 64 partial sums p[l] over channels h = 64i + l, each
// accumulated in order of i, then the halving tree p[l] += p[l + d],
// d = 32 .. 1, and the bias.  Each step is one fused multiply-add (a single
// rounding; a product of two 16-bit floats is exact in fp32 unless it falls
// below fp32's normal range).  Two kernels compute it: one
// (token, expert) pair per 32 lanes for few tokens, and tiles of pairs on the
// matrix cores for many.

// The first launch of every call clears the status word of the workspace
// header; later launches only set bits in it.
MOE_DEV void clear_status(WsHeader *hdr)
{
    if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0)
        hdr->status = 0;
}

// Few tokens: 32 lanes per (token, expert) pair, lane m owning the partial
// sums l = 2m and 2m + 1 (one dword of each row per chunk i), so a call with
// a few thousand pairs still fills every SIMD and each lane keeps a whole
// group of kPairChunk chunks of loads in flight.  The tree runs as lane
// shuffles (d = 32 .. 2: lane m += lane m + d/2) and one in-lane add (d = 1).
constexpr int kPairChunk = 32;

template <bool BF16>
__global__ __launch_bounds__(256) void route_logits_pairs_kernel(const uint16_t *__restrict__ x, int64_t T,
                                                                 int H, const uint16_t *__restrict__ Wr,
                                                                 const float *__restrict__ bias, int E,
                                                                 float *__restrict__ logits, WsHeader *hdr)
{
    clear_status(hdr);
    const int64_t pair = (int64_t)blockIdx.x * 8 + (threadIdx.x >> 5);
    const int m = threadIdx.x & 31;
    const bool ok = pair < T * E;
    const int64_t t = ok ? pair / E : 0;   // rows past the last pair read row 0
    const int e = ok ? (int)(pair % E) : 0;
    const uint32_t *xr = (const uint32_t *)(x + t * H) + m;
    const uint32_t *wr = (const uint32_t *)(Wr + (int64_t)e * H) + m;
    const int n = H / 64;
    float p0 = 0.0f, p1 = 0.0f;
    for (int i0 = 0; i0 < n; i0 += kPairChunk) {
        uint32_t xv[kPairChunk], wv[kPairChunk];
#pragma unroll
        for (int c = 0; c < kPairChunk; ++c)
            if (i0 + c < n) {
                xv[c] = xr[32 * (i0 + c)];
                wv[c] = wr[32 * (i0 + c)];
            }
#pragma unroll
        for (int c = 0; c < kPairChunk; ++c)
            if (i0 + c < n) {
                float x0, x1;
                if (BF16) {
                    x0 = __uint_as_float(xv[c] << 16);
                    x1 = __uint_as_float(xv[c] & 0xFFFF0000u);
                } else {
                    x0 = f16_to_f32((uint16_t)(xv[c] & 0xFFFFu));
                    x1 = f16_to_f32((uint16_t)(xv[c] >> 16));
                }
                p0 = __builtin_fmaf(x0, f16_to_f32((uint16_t)(wv[c] & 0xFFFFu)), p0);
                p1 = __builtin_fmaf(x1, f16_to_f32((uint16_t)(wv[c] >> 16)), p1);
            }
    }
#pragma unroll
    for (int d = 16; d >= 1; d >>= 1) {
        p0 = p0 + __shfl_down(p0, d, 32);
        p1 = p1 + __shfl_down(p1, d, 32);
    }
    if (m == 0 && ok) {
        const float r = p0 + p1;
        logits[t * E + e] = bias ? r + bias[e] : r;
    }
}

// Many tokens, on the matrix cores.  v_mfma_f32_16x16x1_4b_f32 has k = 1: each
// instruction adds exactly one product to each accumulator, and its four
// 16 x 16 blocks carry four of the 64 partial-sum chains of every (token,
// expert) pair of a 16 x 16 tile.  Instruction q (q = 0..15) of a 64-channel
// chunk i adds x[64i + l] * w[64i + l] to chain l = q + 16b of block b = 0..3;
// the lanes of block b supply token (A) and expert (B) rows 0..15.  The
// product is exact in fp32, so every accumulation step rounds once, the order
// over i is the plain one, and the halving tree over l runs on the finished
// chains.
//
// A block of four wavefronts computes 16 tokens x 32 experts.  Wavefronts 2s
// and 2s + 1 own experts 16s .. 16s + 15; wavefront 2s + h issues
// instructions q = 8h .. 8h + 7 of every chunk, so its lane (b, row c) needs
// channels 64i + 16b + 8h .. + 7 of token row c and of expert row 16s + c.
// Chains q, q + 16, q + 32, q + 48 of a pair then sit in one lane of one
// wavefront (block b in registers 4b .. 4b + 3, lane 16 (row / 4) + column,
// register row % 4): the tree steps d = 32, 16 are in-lane adds, d = 8 adds
// wavefront 2s + 1's sums to wavefront 2s's through LDS, and d = 4, 2, 1 are
// in-lane again.  128 accumulator registers per wavefront, two wavefronts per
// SIMD.
//
// Each step of 128 channels (two chunks) the block copies its 16 token rows
// and 32 expert rows into one stage of an LDS ring with LDS-direct loads in
// which 16 lanes read 256 contiguous bytes of one row, so every cache line a
// load touches is used whole, and each staged activation row serves 32
// experts.  (Loading the operands straight into registers touched 16 rows per
// instruction and half of each line, and the texture addresser stalled.)
// Piece p (16 bytes, channels 8p .. 8p + 7 of the step) of row r sits in slot
// p ^ (r & 15) of the row's 16, so the 16 lanes that read one piece of 16
// rows hit 16 distinct 4-bank groups.  The step's 32 operands are widened to
// fp32 before its 16 MFMAs, which then issue back to back.
constexpr int kRlTok = 16, kRlExp = 32;
constexpr int kRlStages = 6;                      // ring depth; loads run 5 steps ahead
constexpr int kRlSlots = (kRlTok + kRlExp) * 16;  // 16-byte slots per stage
constexpr int kRlLoads = kRlSlots / 256;          // LDS-direct loads per lane per step

// element q (0..7) of 8 activations packed in 16 bytes, widened to fp32
template <bool BF16>
MOE_DEV float act_elem(const u32x4 &v, int q)
{
    const uint32_t d = v[q >> 1];
    if (BF16)
        return __uint_as_float((q & 1) ? (d & 0xFFFF0000u) : (d << 16));
    return f16_to_f32((uint16_t)((q & 1) ? (d >> 16) : (d & 0xFFFFu)));
}

MOE_DEV float w_elem(const u32x4 &v, int q)
{
    const uint32_t d = v[q >> 1];
    return f16_to_f32((uint16_t)((q & 1) ? (d >> 16) : (d & 0xFFFFu)));
}

template <bool BF16>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void route_logits_mfma_kernel(
    const uint16_t *__restrict__ x, int64_t T, int H, const uint16_t *__restrict__ Wr,
    const float *__restrict__ bias, int E, float *__restrict__ logits, WsHeader *hdr, int n_tt, int n_et)
{
    __shared__ u32x4 ring_mem[kRlStages * kRlSlots];   // 72 KiB
    LDS_AS u32x4 *ring = (LDS_AS u32x4 *)ring_mem;
    clear_status(hdr);
    int tt, et;
    xcd_map((int)blockIdx.x, n_et, tt, et);   // the expert tiles of a token tile share one XCD's L2
    if (tt >= n_tt)
        return;
    const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)), l = threadIdx.x & 63;
    const int sx = w >> 1, h = w & 1, b = l >> 4, c = l & 15;
    const int64_t t0 = (int64_t)tt * kRlTok;
    const int e0 = et * kRlExp;
    const int nt = (int)std::min<int64_t>(kRlTok, T - t0), ne = std::min(kRlExp, E - e0);
    // rows past the last token / expert read zeros through the ranges; their
    // sums are never stored
    const __amdgpu_buffer_rsrc_t xs = buf_rsrc(x + t0 * H, (uint32_t)(nt * H * 2));
    const __amdgpu_buffer_rsrc_t ws = buf_rsrc(Wr + (int64_t)e0 * H, (uint32_t)(ne * H * 2));
    const __amdgpu_buffer_rsrc_t none = buf_rsrc(x, 0);
    // load k of wavefront w fills slots 64j .. 64j + 63 of a stage, j = 3w + k:
    // stage row 4j + l / 16 (token rows 0..15, then expert rows), slot l % 16
    // of that row, which holds piece (l % 16) ^ (row & 15)
    uint32_t loff[kRlLoads];
    __amdgpu_buffer_rsrc_t lrs[kRlLoads];
#pragma unroll
    for (int k = 0; k < kRlLoads; ++k) {
        const int j = kRlLoads * w + k, r = 4 * j + (l >> 4);
        const bool tok = 4 * j < kRlTok;   // the same for the whole wavefront
        const int rr = tok ? r : r - kRlTok;
        lrs[k] = tok ? xs : ws;
        loff[k] = (uint32_t)(rr * H * 2 + 16 * ((l & 15) ^ (rr & 15)));
    }
    const int nst = H / 128;
    // Every step issues the same loads; those past the last step go through a
    // zero-range descriptor (no memory access) into a stage nobody reads, so
    // one wait count holds on every path.
    auto load = [&](int g, int slot) {
        LDS_AS u32x4 *st = ring + slot * kRlSlots;
#pragma unroll
        for (int k = 0; k < kRlLoads; ++k) {
            const __amdgpu_buffer_rsrc_t rs = g < nst ? lrs[k] : none;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS_AS void *)(st + 64 * (kRlLoads * w + k)), 16,
                                                     loff[k] + 256u * (uint32_t)g, 0, 0, 0);
        }
    };
    // the lane's operand slots: piece 8i + 2b + h (chunk i of the step) of
    // token row c and of expert row 16 sx + c
    const int xsl0 = 16 * c + ((2 * b + h) ^ c), xsl1 = 16 * c + ((8 + 2 * b + h) ^ c);
    const int wsl0 = 16 * (kRlTok + 16 * sx) + xsl0, wsl1 = 16 * (kRlTok + 16 * sx) + xsl1;
    f32x16 acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q)
        acc[q] = (f32x16){};
#pragma unroll
    for (int j = 0; j < kRlStages - 1; ++j)
        load(j, j);
    int cur = 0, prev = kRlStages - 1;
    for (int g = 0; g < nst; ++g) {
        __builtin_amdgcn_sched_barrier(0);
        wait_vmcnt<(kRlStages - 2) * kRlLoads>();   // this step's loads are done
        __builtin_amdgcn_s_barrier();     // ... for every wavefront, and nobody reads step g - 1 any more
        load(g + kRlStages - 1, prev);    // into step g - 1's stage
        const LDS_AS u32x4 *st = ring + cur * kRlSlots;
        prev = cur;
        cur = cur + 1 == kRlStages ? 0 : cur + 1;
        const u32x4 xv0 = st[xsl0], wv0 = st[wsl0], xv1 = st[xsl1], wv1 = st[wsl1];
        __builtin_amdgcn_sched_barrier(0);   // all four reads go out before the first MFMA
        float a0[8], b0[8], a1[8], b1[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            a0[q] = act_elem<BF16>(xv0, q);
            b0[q] = w_elem(wv0, q);
            a1[q] = act_elem<BF16>(xv1, q);
            b1[q] = w_elem(wv1, q);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < 8; ++q)
            acc[q] = __builtin_amdgcn_mfma_f32_16x16x1f32(a0[q], b0[q], acc[q], 0, 0, 0);
#pragma unroll
        for (int q = 0; q < 8; ++q)
            acc[q] = __builtin_amdgcn_mfma_f32_16x16x1f32(a1[q], b1[q], acc[q], 0, 0, 0);
    }
    wait_vmcnt<0>();   // the trailing zero-range loads still write LDS
    __syncthreads();   // the ring is free: it holds the exchange below
    f32x4 u[8];
#pragma unroll
    for (int q = 0; q < 8; ++q)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            u[q][r] = (acc[q][r] + acc[q][8 + r]) + (acc[q][4 + r] + acc[q][12 + r]);
    LDS_AS f32x4 *xch = (LDS_AS f32x4 *)ring + sx * 8 * 64;
    if (h == 1) {
#pragma unroll
        for (int q = 0; q < 8; ++q)
            xch[64 * q + l] = u[q];
    }
    __syncthreads();
    if (h == 1)
        return;
#pragma unroll
    for (int q = 0; q < 8; ++q)
        u[q] = u[q] + xch[64 * q + l];
#pragma unroll
    for (int d = 4; d >= 1; d >>= 1)
#pragma unroll
        for (int q = 0; q < d; ++q)
            u[q] = u[q] + u[q + d];
    const int e = e0 + 16 * sx + c;
    if (e < E) {
        const float be = bias ? bias[e] : 0.0f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t t = t0 + 4 * b + r;
            if (t < T)
                logits[t * E + e] = bias ? u[0][r] + be : u[0][r];
        }
    }
}

hipError_t launch_route_logits(const uint16_t *x, bool bf16, int64_t T, int H, const uint16_t *Wr,
                               const float *bias, int E, float *logits, WsHeader *hdr, hipStream_t s)
{
    // many tokens: 16 x 32 tiles on the matrix cores, in 128-channel steps
    // (the layer's hidden size is a multiple of 256); few tokens: one (token,
    // expert) pair per 32 lanes so that enough wavefronts stream the router
    // weights
    if (H % 128)
        return hipErrorInvalidValue;
    if (T > 64) {
        const int n_tt = (int)((T + kRlTok - 1) / kRlTok), n_et = (E + kRlExp - 1) / kRlExp;
        const unsigned grid = (unsigned)(((n_tt + 7) / 8) * 8 * n_et);
        if (bf16)
            route_logits_mfma_kernel<true><<<grid, 256, 0, s>>>(x, T, H, Wr, bias, E, logits, hdr, n_tt, n_et);
        else
            route_logits_mfma_kernel<false><<<grid, 256, 0, s>>>(x, T, H, Wr, bias, E, logits, hdr, n_tt, n_et);
    } else {
        const unsigned grid = (unsigned)((T * E + 7) / 8);
        if (bf16) route_logits_pairs_kernel<true><<<grid, 256, 0, s>>>(x, T, H, Wr, bias, E, logits, hdr);
        else route_logits_pairs_kernel<false><<<grid, 256, 0, s>>>(x, T, H, Wr, bias, E, logits, hdr);
    }
    return hipGetLastError();
}

// ----------------------------------------------------------------- top-k, softmax
// One wavefront per token.  Lane l holds the logits of experts l, l + 64, ...
// (NPER slots, enough for E).  k rounds: each lane offers its best remaining
// (logit, expert), a DPP reduction finds the wave maximum, and a ballot of the
// lanes holding it names the winner (the lowest expert among ties, which needs
// a second reduction only when several lanes tie).  A NaN logit ranks as -inf:
// no NaN reaches the reductions, so while any lane still holds an expert the
// ballot is never empty and the winner is always a valid expert.

// v <- op(v, v of the lane the DPP control names); rows outside row_mask
// keep their own value (op(v, v) = v).
template <int CTRL, int ROW_MASK>
MOE_DEV float dpp_fmax(float v)
{
    const int o = __builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, ROW_MASK, 0xF, false);
    return fmaxf(v, __int_as_float(o));
}
template <int CTRL, int ROW_MASK>
MOE_DEV int dpp_imin(int v)
{
    return min(v, __builtin_amdgcn_update_dpp(v, v, CTRL, ROW_MASK, 0xF, false));
}

// Wave-wide maximum / minimum (all 64 lanes active), read from lane 63:
// xor 1 and xor 2 inside quads, mirrored halves of 8 and 16 lanes, then the
// last lane of rows 0 and 2 into rows 1 and 3, and of row 1 into rows 2, 3.
MOE_DEV float wave_max(float v)
{
    v = dpp_fmax<0xB1, 0xF>(v);    // quad_perm [1, 0, 3, 2]
    v = dpp_fmax<0x4E, 0xF>(v);    // quad_perm [2, 3, 0, 1]
    v = dpp_fmax<0x141, 0xF>(v);   // row_half_mirror
    v = dpp_fmax<0x140, 0xF>(v);   // row_mirror
    v = dpp_fmax<0x142, 0xA>(v);   // row_bcast15
    v = dpp_fmax<0x143, 0xC>(v);   // row_bcast31
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
MOE_DEV int wave_min(int v)
{
    v = dpp_imin<0xB1, 0xF>(v);
    v = dpp_imin<0x4E, 0xF>(v);
    v = dpp_imin<0x141, 0xF>(v);
    v = dpp_imin<0x140, 0xF>(v);
    v = dpp_imin<0x142, 0xA>(v);
    v = dpp_imin<0x143, 0xC>(v);
    return __builtin_amdgcn_readlane(v, 63);
}

constexpr int kNoExpert = 0x7fffffff;

// Top-k and softmax of token t by the calling wavefront (all 64 lanes).
template <int NPER>
MOE_DEV void topk_token(const float *__restrict__ logits, int64_t t, int E, int k, int32_t *__restrict__ idx,
                        float *__restrict__ w, int32_t *sidx = nullptr)
{
    const int l = threadIdx.x & 63;
    float v[NPER];
    int key[NPER];
#pragma unroll
    for (int i = 0; i < NPER; ++i) {
        const int e = l + 64 * i;
        const bool ok = e < E;
        const float lv = ok ? logits[t * E + e] : -INFINITY;
        v[i] = lv != lv ? -INFINITY : lv;
        key[i] = ok ? e : kNoExpert;
    }
    // lane j keeps pick j (k <= 16 lanes); the softmax then runs across lanes
    float myv = -INFINITY, top = -INFINITY;
    int myi = 0;
    for (int j = 0; j < k; ++j) {
        // the lane's best remaining: slots are in ascending expert order, so
        // the strict compare keeps the lowest expert among equal logits
        float bv = -INFINITY;
        int bi = kNoExpert;
#pragma unroll
        for (int i = 0; i < NPER; ++i) {
            if (key[i] != kNoExpert && (bi == kNoExpert || v[i] > bv)) {
                bv = v[i];
                bi = key[i];
            }
        }
        const float m = wave_max(bi == kNoExpert ? -INFINITY : bv);
        const uint64_t tie = __ballot(bi != kNoExpert && bv == m);
        int win;
        if (__popcll(tie) == 1)
            win = __builtin_amdgcn_readlane(bi, __builtin_ctzll(tie));
        else
            win = wave_min(((tie >> l) & 1) ? bi : kNoExpert);
        if (l == j) {
            myv = m;
            myi = win;
        }
        if (j == 0)
            top = m;
        if ((win & 63) == l) {
#pragma unroll
            for (int i = 0; i < NPER; ++i)
                if (key[i] == win)
                    key[i] = kNoExpert;
        }
    }
    // softmax over the k picks: one exponential per lane, the sum by a fixed
    // butterfly over the wavefront (lanes past k add zero), then every pick
    // stored by its own lane
    const float ex = l < k ? expf(myv - top) : 0.0f;
    float sum = ex;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        sum += __shfl_xor(sum, off, 64);
    if (l < k) {
        idx[t * k + l] = myi;
        w[t * k + l] = ex / sum;
        if (sidx)
            sidx[t * k + l] = myi;
    }
}

template <int NPER>
__global__ __launch_bounds__(256) void topk_kernel(const float *__restrict__ logits, int64_t T,
                                                   int E, int k, int32_t *__restrict__ idx,
                                                   float *__restrict__ w)
{
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T)   // whole wavefronts leave
        return;
    topk_token<NPER>(logits, t, E, k, idx, w);
}

hipError_t launch_topk(const float *logits, int64_t T, int E, int k, int32_t *idx, float *w,
                       hipStream_t s)
{
    const unsigned grid = (unsigned)((T + 3) / 4);
    const int nper = (E + 63) / 64;   // E <= 1024
    if (nper <= 1)
        topk_kernel<1><<<grid, 256, 0, s>>>(logits, T, E, k, idx, w);
    else if (nper <= 2)
        topk_kernel<2><<<grid, 256, 0, s>>>(logits, T, E, k, idx, w);
    else if (nper <= 5)
        topk_kernel<5><<<grid, 256, 0, s>>>(logits, T, E, k, idx, w);
    else if (nper <= 8)
        topk_kernel<8><<<grid, 256, 0, s>>>(logits, T, E, k, idx, w);
    else
        topk_kernel<16><<<grid, 256, 0, s>>>(logits, T, E, k, idx, w);
    return hipGetLastError();
}

// ---------------------------------------------------------------- segment tables
// Stable counting sort of the slots a = t*k + j by expert, in three launches:
//  1. per-block expert histograms of kSegChunk consecutive slots;
//  2. one block: per-expert running sums over blocks, counts, exclusive
//     offsets, and the work lists (GEMV experts, MFMA row tiles);
//  3. per block, slots in order: eight wavefronts each rank a span of the
//     block's slots, inside each 64-slot chunk from ballots; position =
//     block base + earlier spans' counts + rank.

// An expert index outside [0, E) (impossible from topk_token; a guard against
// a corrupted table) is left out of every table and flagged in the status word.
MOE_DEV bool valid_expert(int e, int E) { return (unsigned)e < (unsigned)E; }

MOE_DEV void flag_status(WsHeader *hdr, uint32_t bits) { atomicOr((unsigned *)&hdr->status, bits); }

__global__ __launch_bounds__(256) void seg_hist_kernel(const int32_t *__restrict__ idx, int64_t n,
                                                       int E, int32_t *__restrict__ bhist, WsHeader *hdr)
{
    extern __shared__ int32_t hist[];
    for (int e = threadIdx.x; e < E; e += blockDim.x)
        hist[e] = 0;
    __syncthreads();
    const int64_t a0 = (int64_t)blockIdx.x * kSegChunk;
    for (int i = threadIdx.x; i < kSegChunk; i += blockDim.x) {
        const int64_t a = a0 + i;
        if (a < n) {
            const int e = idx[a];
            if (valid_expert(e, E))
                atomicAdd(&hist[e], 1);
            else
                flag_status(hdr, MOE_EXL3_STATUS_BAD_INDEX);
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x)
        bhist[(int64_t)blockIdx.x * E + e] = hist[e];
}

// Block-wide exclusive scan of one value per thread (blockDim.x == 1024).
__device__ int block_exclusive_scan(int v, int *total)
{
    __shared__ int wsum[16];
    const int l = threadIdx.x & 63, wv = threadIdx.x >> 6;
    int incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(incl, off, 64);
        if (l >= off)
            incl += o;
    }
    if (l == 63)
        wsum[wv] = incl;
    __syncthreads();
    int base = 0, tot = 0;
    for (int i = 0; i < 16; ++i) {
        if (i < wv)
            base += wsum[i];
        tot += wsum[i];
    }
    __syncthreads();
    *total = tot;
    return base + incl - v;
}

// Three block-wide exclusive scans at once (blockDim.x == 1024), for counts
// whose block totals stay below 2^21: packed as 21-bit fields of one 64-bit
// value, no carry crosses a field, so each field scans exactly.
__device__ void block_exclusive_scan3(const int v[3], int ex[3], int tot[3])
{
    __shared__ uint64_t wsum3[16];
    const int l = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const uint64_t p = (uint64_t)v[0] | ((uint64_t)v[1] << 21) | ((uint64_t)v[2] << 42);
    uint64_t incl = p;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint64_t o = __shfl_up(incl, off, 64);
        if (l >= off)
            incl += o;
    }
    if (l == 63)
        wsum3[wv] = incl;
    __syncthreads();
    uint64_t base = 0, all = 0;
    for (int i = 0; i < 16; ++i) {
        if (i < wv)
            base += wsum3[i];
        all += wsum3[i];
    }
    __syncthreads();
    const uint64_t e = base + incl - p;
    constexpr uint64_t kMask = (1ull << 21) - 1;
#pragma unroll
    for (int f = 0; f < 3; ++f) {
        ex[f] = (int)((e >> (21 * f)) & kMask);
        tot[f] = (int)((all >> (21 * f)) & kMask);
    }
}

// The GEMV expert list and the MFMA tile list (expert, first row), written by
// the thread of expert e.  The tile list holds at most max_tiles entries (the
// host's bound on the tiles a call can produce); a longer one is cut there and
// flagged.
MOE_DEV void write_work_lists(int e, bool gemv, int gpos, int ng, int nt, int tpos, int ntt, int tile_m,
                              int max_tiles, int32_t *__restrict__ glist, int32_t *__restrict__ tiles,
                              WsHeader *hdr)
{
    if (gemv)
        glist[gpos] = e;
    for (int m = 0; m < nt; ++m) {
        if (tpos + m >= max_tiles)
            break;
        tiles[2 * (tpos + m)] = e;
        tiles[2 * (tpos + m) + 1] = m * tile_m;
    }
    if (e == 0) {
        hdr->n_gemv = ng;
        hdr->n_tiles = min(ntt, max_tiles);
        if (ntt > max_tiles)
            flag_status(hdr, MOE_EXL3_STATUS_TILE_OVERFLOW);
    }
}

// The slots of the trellis shared expert: slot nr + t is token t's, with
// routing weight 1, and sits at position nr + t of the sorted list (the
// expert follows every routed one).
MOE_DEV void write_extra_slots(int64_t nr, int64_t T, int32_t *__restrict__ sorted, int32_t *__restrict__ pos,
                               float *__restrict__ w)
{
    for (int64_t t = threadIdx.x; t < T; t += blockDim.x) {
        sorted[nr + t] = (int32_t)(nr + t);
        pos[nr + t] = (int32_t)(nr + t);
        w[nr + t] = 1.0f;
    }
}

__global__ __launch_bounds__(1024) void seg_scan_kernel(int32_t *__restrict__ bhist, int nblk, int E, int64_t T,
                                                        int64_t nr, bool extra, int gemv_rows, int tile_m,
                                                        int max_tiles, int32_t *__restrict__ counts,
                                                        int32_t *__restrict__ offsets,
                                                        int32_t *__restrict__ sorted, int32_t *__restrict__ pos,
                                                        float *__restrict__ w,
                                                        int32_t *__restrict__ glist,
                                                        int32_t *__restrict__ tiles,
                                                        WsHeader *__restrict__ hdr)
{
    const int e = threadIdx.x;   // E + extra <= 1024
    const int EA = E + (extra ? 1 : 0);
    int c = 0;
    if (e < E) {
        // per-chunk counts -> running bases, 16 chunks' loads in flight at a time
        constexpr int kG = 16;
        for (int b0 = 0; b0 < nblk; b0 += kG) {
            int v[kG];
#pragma unroll
            for (int j = 0; j < kG; ++j)
                v[j] = b0 + j < nblk ? bhist[(int64_t)(b0 + j) * E + e] : 0;
#pragma unroll
            for (int j = 0; j < kG; ++j)
                if (b0 + j < nblk) {
                    bhist[(int64_t)(b0 + j) * E + e] = c;
                    c += v[j];
                }
        }
    } else if (e < EA) {
        c = (int)T;
    }
    int tot;
    const int off = block_exclusive_scan(e < EA ? c : 0, &tot);
    if (e < EA) {
        counts[e] = c;
        offsets[e] = off;
    }
    if (e == 0)
        offsets[EA] = tot;
    const bool gemv = e < EA && c > 0 && c <= gemv_rows;
    const int nt = (e < EA && c > gemv_rows) ? (c + tile_m - 1) / tile_m : 0;
    int ng, ntt;
    const int gpos = block_exclusive_scan(gemv ? 1 : 0, &ng);
    const int tpos = block_exclusive_scan(nt, &ntt);
    write_work_lists(e, gemv, gpos, ng, nt, tpos, ntt, tile_m, max_tiles, glist, tiles, hdr);
    if (extra)
        write_extra_slots(nr, T, sorted, pos, w);
}

// Scatter of one kSegChunk-slot block by kScatterWaves wavefronts, wavefront
// w taking the block's slots w * kScatterSpan .. + kScatterSpan - 1 in order.
// Each wavefront first counts its span per expert; the bases of wavefront w
// are then the block's base plus the counts of wavefronts 0 .. w - 1, so the
// spans rank independently and the order stays the stable one.
constexpr int kScatterWaves = 8;
constexpr int kScatterSpan = kSegChunk / kScatterWaves;   // a multiple of 64

__global__ __launch_bounds__(64 * kScatterWaves) void seg_scatter_kernel(const int32_t *__restrict__ idx, int64_t n,
                                                                        int E, const int32_t *__restrict__ bhist,
                                                                        const int32_t *__restrict__ offsets,
                                                                        int32_t *__restrict__ sorted,
                                                                        int32_t *__restrict__ pos)
{
    extern __shared__ int32_t base[];   // [kScatterWaves][E]
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    for (int i = threadIdx.x; i < kScatterWaves * E; i += 64 * kScatterWaves)
        base[i] = 0;
    const int64_t a0 = (int64_t)blockIdx.x * kSegChunk + (int64_t)w * kScatterSpan;
    int nbits = 0;
    while ((1 << nbits) < E)
        ++nbits;
    const uint64_t below = (l == 0) ? 0ull : (~0ull >> (64 - l));
    // the span's expert ids are loaded up front (one round trip), the ranking
    // below then runs on registers and LDS only
    constexpr int kIter = kScatterSpan / 64;
    int ev[kIter];
#pragma unroll
    for (int c = 0; c < kIter; ++c) {
        const int64_t a = a0 + 64 * c + l;
        ev[c] = a < n ? idx[a] : 0;
    }
    __syncthreads();
    int32_t *wb = base + w * E;
#pragma unroll
    for (int c = 0; c < kIter; ++c) {
        const int64_t a = a0 + 64 * c + l;
        if (a < n && valid_expert(ev[c], E))
            atomicAdd(&wb[ev[c]], 1);
    }
    __syncthreads();
    // counts -> bases: the block's base of expert e, then the wavefronts'
    // spans in order
    for (int e = threadIdx.x; e < E; e += 64 * kScatterWaves) {
        int run = bhist[(int64_t)blockIdx.x * E + e] + offsets[e];
        for (int v = 0; v < kScatterWaves; ++v) {
            const int cnt = base[v * E + e];
            base[v * E + e] = run;
            run += cnt;
        }
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < kIter; ++c) {
        const int64_t a = a0 + 64 * c + l;
        if (a - l >= n)   // wavefront-uniform: the rest of the span is past the end
            break;
        const int e = ev[c];
        const bool valid = a < n && valid_expert(e, E);
        uint64_t m = __ballot(valid);
        for (int b = 0; b < nbits; ++b) {
            const bool bit = (e >> b) & 1;
            const uint64_t bb = __ballot(bit);
            m &= bit ? bb : ~bb;
        }
        // the wavefront's LDS operations run in order: every lane reads its
        // expert's base before the last lane of that expert advances it
        if (valid) {
            const int p = wb[e] + __popcll(m & below);
            sorted[p] = (int32_t)a;
            pos[a] = p;
        }
        __builtin_amdgcn_wave_barrier();
        if (valid && (m >> l) == 1ull)   // last lane of its expert in this chunk
            wb[e] += __popcll(m);
        __builtin_amdgcn_wave_barrier();
    }
}

hipError_t launch_segments(const int32_t *idx, int64_t T, int k, int E, bool extra, int nblk, int gemv_rows,
                           int tile_m, int max_tiles, int32_t *bhist, int32_t *counts, int32_t *offsets,
                           int32_t *sorted, int32_t *pos, float *w, int32_t *glist, int32_t *tiles,
                           WsHeader *hdr, hipStream_t s)
{
    const int64_t n = T * k;
    const size_t lds = sizeof(int32_t) * (size_t)E;
    seg_hist_kernel<<<nblk, 256, lds, s>>>(idx, n, E, bhist, hdr);
    seg_scan_kernel<<<1, 1024, 0, s>>>(bhist, nblk, E, T, n, extra, gemv_rows, tile_m, max_tiles, counts,
                                       offsets, sorted, pos, w, glist, tiles, hdr);
    seg_scatter_kernel<<<nblk, 64 * kScatterWaves, kScatterWaves * lds, s>>>(idx, n, E, bhist, offsets, sorted, pos);
    return hipGetLastError();
}

// ---------------------------------------------------------------- debug checks
// One block: thread e walks expert e's segment and checks that it holds
// counts[e] slots, in increasing order, each routed to e, with pos its
// inverse; the counts must sum to n.  Every table value is range-checked
// before it is used as an index.
__global__ __launch_bounds__(1024) void debug_tables_kernel(const int32_t *__restrict__ idx, int64_t n, int E,
                                                            const int32_t *__restrict__ counts,
                                                            const int32_t *__restrict__ offsets,
                                                            const int32_t *__restrict__ sorted,
                                                            const int32_t *__restrict__ pos, WsHeader *hdr)
{
    __shared__ long long total;
    if (threadIdx.x == 0)
        total = 0;
    __syncthreads();
    bool bad = false;
    long long mine = 0;
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        const int c = counts[e], o0 = offsets[e], o1 = offsets[e + 1];
        mine += c;
        if (o1 - o0 != c || o0 < 0 || o1 > n || o0 > o1) {
            bad = true;
            continue;
        }
        int prev = -1;
        for (int p = o0; p < o1; ++p) {
            const int a = sorted[p];
            if (a <= prev || a >= n || idx[a] != e || pos[a] != p) {
                bad = true;
                break;
            }
            prev = a;
        }
    }
    atomicAdd((unsigned long long *)&total, (unsigned long long)mine);
    if (bad)
        flag_status(hdr, MOE_EXL3_STATUS_TABLES);
    __syncthreads();
    if (threadIdx.x == 0 && (total != n || offsets[0] != 0 || offsets[E] != n))
        flag_status(hdr, MOE_EXL3_STATUS_COUNTS);
}

// Grid-stride check that every activation is finite.
__global__ __launch_bounds__(256) void debug_finite_kernel(const uint16_t *__restrict__ x, int64_t n, uint32_t expo,
                                                           WsHeader *hdr)
{
    bool bad = false;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
        bad |= (x[i] & expo) == expo;
    if (bad)
        flag_status(hdr, MOE_EXL3_STATUS_NONFINITE_X);
}

hipError_t launch_debug_checks(const uint16_t *x, bool bf16, int64_t T, int H, int k, int E,
                               const int32_t *idx, const int32_t *counts, const int32_t *offsets,
                               const int32_t *sorted, const int32_t *pos, WsHeader *hdr, hipStream_t s)
{
    debug_tables_kernel<<<1, 1024, 0, s>>>(idx, T * k, E, counts, offsets, sorted, pos, hdr);
    const int64_t n = T * H;
    const unsigned grid = (unsigned)std::min<int64_t>(2048, (n + 255) / 256);
    debug_finite_kernel<<<grid, 256, 0, s>>>(x, n, bf16 ? 0x7F80u : 0x7C00u, hdr);
    return hipGetLastError();
}

// ---------------------------------------------------------------- decode-sized calls
// One block of 1024 threads runs the whole routing tail of a decode-sized call
// (T <= kSmallRouteTokens, T * k <= kSegChunk) in one launch: top-k and
// softmax (one wavefront per token), the expert histogram, counts, offsets
// and work lists (as seg_scan_kernel with a single chunk), the stable scatter
// (as seg_scatter_kernel, by wavefront 0 alone), and, when x16 is given, the
// bf16 -> fp16 copy of the activations.
template <int NPER>
__global__ __launch_bounds__(1024) void route_small_kernel(
    const float *__restrict__ logits, int64_t T, int E, int k, bool extra, int gemv_rows, int tile_m, int max_tiles,
    int32_t *__restrict__ idx, float *__restrict__ w, int32_t *__restrict__ counts,
    int32_t *__restrict__ offsets, int32_t *__restrict__ sorted, int32_t *__restrict__ pos,
    int32_t *__restrict__ glist, int32_t *__restrict__ tiles, WsHeader *__restrict__ hdr,
    const uint16_t *__restrict__ x, int H, uint16_t *__restrict__ x16)
{
    __shared__ int32_t sidx[kSegChunk];
    __shared__ int32_t hist[1024];
    const int wv = threadIdx.x >> 6, l = threadIdx.x & 63;
    // up to 8 tokens, wavefronts 8..15 have no token to rank: they copy the
    // activations while wavefronts 0..T-1 run top-k
    const bool split = T <= 8;
    if (!split || wv < 8)
        for (int64_t t = wv; t < T; t += 16)
            topk_token<NPER>(logits, t, E, k, idx, w, sidx);
    if (x16 && (!split || wv >= 8)) {
        const int64_t n8 = T * H / 8;
        const int first = split ? (int)threadIdx.x - 512 : (int)threadIdx.x, step = split ? 512 : 1024;
        bool over = false;
        // all loads of a round of kCopyBatch pieces go out before its first
        // store: one memory latency per round rather than one per piece
        constexpr int kCopyBatch = 8;
        for (int64_t i0 = first; i0 < n8; i0 += (int64_t)kCopyBatch * step) {
            u32x4 v[kCopyBatch];
#pragma unroll
            for (int j = 0; j < kCopyBatch; ++j) {
                const int64_t i = i0 + (int64_t)j * step;
                v[j] = i < n8 ? ((const u32x4 *)x)[i] : (u32x4){0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int j = 0; j < kCopyBatch; ++j) {
                const int64_t i = i0 + (int64_t)j * step;
                if (i < n8)
                    ((u32x4 *)x16)[i] = bf16x8_to_f16x8(v[j], over);
            }
        }
        if (over)
            flag_status(hdr, MOE_EXL3_STATUS_ACT_RANGE);
    }
    hist[threadIdx.x] = 0;
    __syncthreads();
    const int n = (int)(T * k);
    for (int a = threadIdx.x; a < n; a += 1024) {
        if (valid_expert(sidx[a], E))
            atomicAdd(&hist[sidx[a]], 1);
        else
            flag_status(hdr, MOE_EXL3_STATUS_BAD_INDEX);
    }
    __syncthreads();
    const int e = threadIdx.x;   // E + extra <= 1024
    const int EA = E + (extra ? 1 : 0);
    const int c = e < E ? hist[e] : e < EA ? (int)T : 0;
    const bool gemv = e < EA && c > 0 && c <= gemv_rows;
    const int nt = (e < EA && c > gemv_rows) ? (c + tile_m - 1) / tile_m : 0;
    // offsets, GEMV list positions and tile list positions in one scan (every
    // block total is at most T * k + T <= 2 kSegChunk < 2^21)
    const int sv[3] = {c, gemv ? 1 : 0, nt};
    int sx[3], st[3];
    block_exclusive_scan3(sv, sx, st);
    const int off = sx[0];
    if (e < EA) {
        counts[e] = c;
        offsets[e] = off;
    }
    if (e == 0)
        offsets[EA] = st[0];
    write_work_lists(e, gemv, sx[1], st[1], nt, sx[2], st[2], tile_m, max_tiles, glist, tiles, hdr);
    if (extra)
        write_extra_slots((int64_t)n, T, sorted, pos, w);
    __syncthreads();
    hist[threadIdx.x] = off;   // running base of every expert
    __syncthreads();
    if (wv == 0) {
        int nbits = 0;
        while ((1 << nbits) < E)
            ++nbits;
        const uint64_t below = (l == 0) ? 0ull : (~0ull >> (64 - l));
        for (int c0 = 0; c0 < n; c0 += 64) {
            const int a = c0 + l;
            const int ea = a < n ? sidx[a] : 0;
            const bool valid = a < n && valid_expert(ea, E);
            uint64_t m = __ballot(valid);
            for (int b = 0; b < nbits; ++b) {
                const bool bit = (ea >> b) & 1;
                const uint64_t bb = __ballot(bit);
                m &= bit ? bb : ~bb;
            }
            // the wavefront's LDS operations run in order: every lane reads
            // the base before the last lane of its expert advances it
            const int p = valid ? hist[ea] + __popcll(m & below) : 0;
            if (valid) {
                sorted[p] = a;
                pos[a] = p;
            }
            __builtin_amdgcn_wave_barrier();
            if (valid && (m >> l) == 1ull)   // last lane of its expert in this chunk
                hist[ea] += __popcll(m);
            __builtin_amdgcn_wave_barrier();
        }
    }
}

hipError_t launch_route_small(const float *logits, int64_t T, int E, int k, bool extra, int gemv_rows, int tile_m,
                              int max_tiles, int32_t *idx, float *w, int32_t *counts, int32_t *offsets,
                              int32_t *sorted, int32_t *pos, int32_t *glist, int32_t *tiles, WsHeader *hdr,
                              const uint16_t *x, int H, uint16_t *x16, hipStream_t s)
{
    const int nper = (E + 63) / 64;   // E <= 1024
#define MOE_ROUTE_SMALL(NP) \
    route_small_kernel<NP><<<1, 1024, 0, s>>>(logits, T, E, k, extra, gemv_rows, tile_m, max_tiles, idx, w, \
                                              counts, offsets, sorted, pos, glist, tiles, hdr, x, H, x16)
    if (nper <= 1) MOE_ROUTE_SMALL(1);
    else if (nper <= 2) MOE_ROUTE_SMALL(2);
    else if (nper <= 5) MOE_ROUTE_SMALL(5);
    else if (nper <= 8) MOE_ROUTE_SMALL(8);
    else MOE_ROUTE_SMALL(16);
#undef MOE_ROUTE_SMALL
    return hipGetLastError();
}

}  // namespace moe
