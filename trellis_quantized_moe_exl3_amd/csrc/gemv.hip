// Decode-fused GEMV path for experts with few routed rows (decode-sized
// steps; page "GLM-5.3 Flash EXL3 for 2x DGX Sparks", "What runs": one fused
// launch per layer for decode-sized steps, trellis decoded inside the matmul;
// page "GLM-5.3-Flash EXL3 (~2.1 bpw, SM70 tile order)", "Speed": direct
// per-lane window loads with a deep prefetch).
//
// Each lane decodes eight consecutive input rows of one output column from
// two code dwords into packed fp16 pairs, which are its B operand of one
// v_mfma_f32_32x32x16_f16 per tile row, so a wavefront streams a pair of
// 16-column tiles and every output column stays in one lane.  The code stream is read once per pass of up to two routed rows (once
// per expert at the default split); it is the only large HBM traffic of a
// decode-sized step.  The dense shared expert's decode-sized GEMV lives here
// too, as blocks of its own launches or of the routed ones.
#include <algorithm>
#include <initializer_list>

#include "common.h"
#include "gemm.h"
#include "internal.h"
#include "trellis.h"

namespace moe {

constexpr int kGemvU = 4;      // tile rows per prefetch group
constexpr int kGemvPass = 2;   // routed rows per pass over the codes
constexpr int kStageIt = 2;    // 16-byte pieces per thread and row in one staging round
constexpr int kNontemporal = 2;   // buffer-load cache policy: the nt bit

// 1532 * (row sum), the re-centring of the biased decoded values.
constexpr float kBias2 = 1532.0f;

// A wavefront-uniform value of a routing table an earlier launch wrote, read
// through the scalar cache (the tables are read-only here): its wait does
// not hold up the vector loads in flight, as a vector load's would.
MOE_DEV int32_t ld_uniform(const int32_t *p)
{
    return *(const __attribute__((address_space(4))) int32_t *)p;
}

// Deterministic block reduction (256 threads) of N floats per thread, all
// in one pair of barriers: entry i is summed, or maximised where bit i of
// MAXMASK is set.  Every lane of the butterfly ends with the same value; the
// four wavefront results are combined as ((w0 + w1) + w2) + w3.
template <int N, unsigned MAXMASK = 0u>
MOE_DEV void block_reduce256(float v[N], float (*part)[4])
{
#pragma unroll
    for (int i = 0; i < N; ++i)
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            const float o = __shfl_xor(v[i], off, 64);
            v[i] = ((MAXMASK >> i) & 1u) ? fmaxf(v[i], o) : v[i] + o;
        }
    __syncthreads();
    if ((threadIdx.x & 63) == 0)
#pragma unroll
        for (int i = 0; i < N; ++i)
            part[i][threadIdx.x >> 6] = v[i];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < N; ++i)
        v[i] = ((MAXMASK >> i) & 1u) ? fmaxf(fmaxf(part[i][0], part[i][1]), fmaxf(part[i][2], part[i][3]))
                                     : ((part[i][0] + part[i][1]) + part[i][2]) + part[i][3];
}

// The code stream of one wavefront: tile rows [tk0, tk1) of the lane's
// fragment, through a buffer resource over the wavefront's 16-column tile
// pair: the lane's two dwords sit at fixed byte offsets v0, v1 inside a tile
// row and the tile row at a scalar offset, so a load costs no vector address
// arithmetic.  Two register sets of kGemvU tile rows alternate, one decoding
// while the other fills.  The loads do not depend on the width, so the first
// two groups can go out (prime) as soon as the expert is known, ahead of the
// staging of the pass's activations.  The stream is read once per pass and
// never again in the call: the loads carry the nontemporal hint (cache
// policy 2), which measured 1% (K = 2) and 2% (K = 4) off the 8-token layer.
struct GemvCodes {
    __amdgpu_buffer_rsrc_t rs;
    uint32_t v0, v1, rowb;
    int tk0, tk1;
    uint32_t A[kGemvU][2], B[kGemvU][2];

    MOE_DEV void load(uint32_t (&buf)[kGemvU][2], int g)
    {
#pragma unroll
        for (int u = 0; u < kGemvU; ++u) {
            const int so = (g + u) * (int)rowb;
            buf[u][0] = __builtin_amdgcn_raw_buffer_load_b32(rs, v0, so, kNontemporal);
            buf[u][1] = __builtin_amdgcn_raw_buffer_load_b32(rs, v1, so, kNontemporal);
        }
    }
    // tk0, tk1 are wavefront-uniform: every branch of the stream is scalar.
    // tk1 - tk0 is a positive multiple of kGemvU (an even one for every
    // shape the library accepts, so the single-group tail is kept only for
    // generality).  Every load is issued unconditionally: a group past the
    // wave's range reloads its last group (in range, just read, never used),
    // so no load sits behind a branch and the two register sets need no
    // copies to merge loaded and kept values.
    MOE_DEV void prime()
    {
        load(A, tk0);
        load(B, min(tk0 + kGemvU, tk1 - kGemvU));
    }
};

// Accumulate x . (2v + 1532) of the primed stream on the matrix cores.  The
// lane's fragment (eight input rows kk + 8h .. + 7 of column 16 ts + c) is
// exactly its B operand of v_mfma_f32_32x32x16_f16 (column l % 32, k-half
// l / 32), and its A operand is the same eight inputs of activation row
// l % 32, read from LDS at arow + kk (arow: the lane's row, already offset by
// 8h).  Rows past the pass's routed rows carry any in-range data: their
// output rows are never read.  The accumulator d holds, in lanes 0..31, the
// column's sum for activation row r in register r (r < 4); the MFMA adds both
// k-halves.
template <int K, int CB>
MOE_DEV void gemv_stream_mfma(GemvCodes &cs, int q, uint32_t m_lo, uint32_t m_hi, const f16 *arow, f32x16 &d)
{
    auto run = [&](const uint32_t(&buf)[kGemvU][2], int g) {
#pragma unroll
        for (int u = 0; u < kGemvU; ++u) {
            f16x2 wp[4];
            frag_biased_pairs<K, CB>(buf[u][0], buf[u][1], q, m_lo, m_hi, wp);
            const f16x8 av = *(const f16x8 *)(arow + 16 * (g + u));
            d = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, __builtin_bit_cast(f16x8, wp), d, 0, 0, 0);
        }
    };
    const int tk1 = cs.tk1, glast = tk1 - kGemvU;
    int g = cs.tk0;
    for (; g + 2 * kGemvU <= tk1; g += 2 * kGemvU) {
        run(cs.A, g);
        cs.load(cs.A, min(g + 2 * kGemvU, glast));
        run(cs.B, g + kGemvU);
        cs.load(cs.B, min(g + 3 * kGemvU, glast));
    }
    if (g < tk1)
        run(cs.A, g);
}

template <int K, int CB>
MOE_DEV void gemv_stream_mfma_k(int kw, GemvCodes &cs, int q, uint32_t m_lo, uint32_t m_hi, const f16 *arow,
                                f32x16 &d)
{
    if constexpr (K > 0) {
        gemv_stream_mfma<K, CB>(cs, q, m_lo, m_hi, arow, d);
    } else {
        if (kw == 4)
            gemv_stream_mfma<4, CB>(cs, q, m_lo, m_hi, arow, d);
        else if (kw == 3)
            gemv_stream_mfma<3, CB>(cs, q, m_lo, m_hi, arow, d);
        else
            gemv_stream_mfma<2, CB>(cs, q, m_lo, m_hi, arow, d);
    }
}

// ------------------------------------------------------------ shared expert GEMV
// Dense fp16 weights in nn.Linear layout [out][in]; one wavefront per weight
// row (gate/up: the gate and the up row of one channel), four per block.  The
// input dimension is walked in slabs of kShSlab channels: the block stages
// the slab of all TT token rows (a power of two >= T; rows past T and
// channels past the end are zero) in LDS once, so every token row is read
// from L2 once per block instead of once per wavefront, while each lane
// streams its 16-byte weight chunks k = 8l + 512c of the slab (the next
// slab's chunks are loaded before the current one is used).
constexpr int kShSlab = 2048;
constexpr int kShChunks = kShSlab / 512;

// Sum over the wavefront (all lanes active), the result in every lane.
MOE_DEV float wave_sum(float v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        v += __shfl_xor(v, off, 64);
    return v;
}

MOE_DEV float dot8(const f16x8 &a, const f16x8 &b, float s)
{
#pragma unroll
    for (int j = 0; j < 8; j += 2)
        s = __builtin_amdgcn_fdot2((f16x2){a[j], a[j + 1]}, (f16x2){b[j], b[j + 1]}, s, false);
    return s;
}

// Rows [0, TT) of the slab [kb, kb + kShSlab) of a [T][n] fp16 matrix into LDS
// (zeros past T or n), by all 256 threads of the block: every thread issues
// all of its loads before its first LDS write, so the slab costs one memory
// latency rather than one per load.
template <int TT>
MOE_DEV void stage_slab(const uint16_t *__restrict__ src, int T, int n, int kb, f16 *xs)
{
    constexpr int kPer = TT * kShSlab / 8 / 256;   // 16-byte pieces per thread
    f16x8 v[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int i = threadIdx.x + 256 * j;
        const int t = i / (kShSlab / 8), k = kb + 8 * (i % (kShSlab / 8));
        const bool in = t < T && k < n;
        const f16x8 a = *(const f16x8 *)(src + (in ? (int64_t)t * n + k : 0));
        v[j] = in ? a : (f16x8){};
    }
#pragma unroll
    for (int j = 0; j < kPer; ++j)
        *(f16x8 *)(xs + 8 * (threadIdx.x + 256 * j)) = v[j];
}

// The lane's weight chunks of one slab of row r (zeros past the row end).
MOE_DEV void load_chunks(const uint16_t *__restrict__ r, int n, int kb, int l, f16x8 v[kShChunks])
{
#pragma unroll
    for (int c = 0; c < kShChunks; ++c) {
        const int k0 = kb + 512 * c + 8 * l;
        const f16x8 a = *(const f16x8 *)(r + (k0 < n ? k0 : 0));
        v[c] = k0 < n ? a : (f16x8){};
    }
}

// Shared-expert gate/up rows 4 rb .. 4 rb + 3 (xs: TT * kShSlab halves of LDS).
template <int TT>
MOE_DEV void shared_gateup_block(const uint16_t *__restrict__ x16, int T, int H, int I,
                                 const uint16_t *__restrict__ wg, const uint16_t *__restrict__ wu,
                                 uint16_t *__restrict__ sh, int rb, f16 *xs)
{
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    const int n = min(rb * 4 + w, I - 1);   // spare wavefronts repeat the last row
    float acc[2][TT];
#pragma unroll
    for (int t = 0; t < TT; ++t)
        acc[0][t] = acc[1][t] = 0.0f;
    const uint16_t *gr = wg + (int64_t)n * H, *ur = wu + (int64_t)n * H;
    f16x8 vg[kShChunks], vu[kShChunks];
    load_chunks(gr, H, 0, l, vg);
    load_chunks(ur, H, 0, l, vu);
    for (int kb = 0; kb < H; kb += kShSlab) {
        __syncthreads();   // the previous slab's LDS reads are done
        stage_slab<TT>(x16, T, H, kb, xs);
        __syncthreads();
        f16x8 cg[kShChunks], cu[kShChunks];
#pragma unroll
        for (int c = 0; c < kShChunks; ++c) {
            cg[c] = vg[c];
            cu[c] = vu[c];
        }
        if (kb + kShSlab < H) {
            load_chunks(gr, H, kb + kShSlab, l, vg);
            load_chunks(ur, H, kb + kShSlab, l, vu);
        }
#pragma unroll
        for (int t = 0; t < TT; ++t) {
            f16x8 xv[kShChunks];
#pragma unroll
            for (int c = 0; c < kShChunks; ++c)
                xv[c] = *(const f16x8 *)(xs + t * kShSlab + 512 * c + 8 * l);
            float g = acc[0][t], u = acc[1][t];
#pragma unroll
            for (int c = 0; c < kShChunks; ++c) {
                g = dot8(cg[c], xv[c], g);
                u = dot8(cu[c], xv[c], u);
            }
            acc[0][t] = g;
            acc[1][t] = u;
        }
    }
    const bool own = rb * 4 + w < I;
#pragma unroll
    for (int t = 0; t < TT; ++t) {
        const float g = wave_sum(acc[0][t]), u = wave_sum(acc[1][t]);
        if (own && l == 0 && t < T)
            sh[(int64_t)t * I + n] = f32_to_f16_bits(silu_f(g) * u);
    }
}

// Shared-expert down rows 4 rb .. 4 rb + 3 (hs: TT * kShSlab halves of LDS).
template <int TT>
MOE_DEV void shared_down_block(const uint16_t *__restrict__ sh, int T, int H, int I,
                               const uint16_t *__restrict__ wd, float *__restrict__ sy, int rb, f16 *hs)
{
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    const int m = min(rb * 4 + w, H - 1);
    float acc[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t)
        acc[t] = 0.0f;
    const uint16_t *dr = wd + (int64_t)m * I;
    f16x8 vd[kShChunks];
    load_chunks(dr, I, 0, l, vd);
    for (int kb = 0; kb < I; kb += kShSlab) {
        __syncthreads();
        stage_slab<TT>(sh, T, I, kb, hs);
        __syncthreads();
        f16x8 cd[kShChunks];
#pragma unroll
        for (int c = 0; c < kShChunks; ++c)
            cd[c] = vd[c];
        if (kb + kShSlab < I)
            load_chunks(dr, I, kb + kShSlab, l, vd);
#pragma unroll
        for (int t = 0; t < TT; ++t) {
            f16x8 hv[kShChunks];
#pragma unroll
            for (int c = 0; c < kShChunks; ++c)
                hv[c] = *(const f16x8 *)(hs + t * kShSlab + 512 * c + 8 * l);
            float v = acc[t];
#pragma unroll
            for (int c = 0; c < kShChunks; ++c)
                v = dot8(cd[c], hv[c], v);
            acc[t] = v;
        }
    }
    const bool own = rb * 4 + w < H;
#pragma unroll
    for (int t = 0; t < TT; ++t) {
        const float v = wave_sum(acc[t]);
        if (own && l == 0 && t < T)
            sy[(int64_t)t * H + m] = v;
    }
}

template <int TT>
__global__ __launch_bounds__(256) void shared_gemv_gateup_kernel(const uint16_t *__restrict__ x16, int T, int H,
                                                                 int I, const uint16_t *__restrict__ wg,
                                                                 const uint16_t *__restrict__ wu,
                                                                 uint16_t *__restrict__ sh)
{
    __shared__ __align__(16) f16 xs[TT * kShSlab];
    shared_gateup_block<TT>(x16, T, H, I, wg, wu, sh, (int)blockIdx.x, xs);
}

template <int TT>
__global__ __launch_bounds__(256) void shared_gemv_down_kernel(const uint16_t *__restrict__ sh, int T, int H,
                                                               int I, const uint16_t *__restrict__ wd,
                                                               float *__restrict__ sy)
{
    __shared__ __align__(16) f16 hs[TT * kShSlab];
    shared_down_block<TT>(sh, T, H, I, wd, sy, (int)blockIdx.x, hs);
}

// Shared-expert work inside a routed GEMV launch: grid rows past the routed
// experts' (blockIdx.y >= max_list) carry its blocks of 4 weight rows (T <= 8:
// TT picked at run time).
MOE_DEV bool shared_in_gemv(const GroupArgs &a, const SharedArgs &sa, int max_list, bool gateup, f16 *smem)
{
    if ((int)blockIdx.y < max_list)
        return false;
    const int rb = ((int)blockIdx.y - max_list) * (int)gridDim.x + (int)blockIdx.x;
    const int T = (int)a.T;
    if (gateup) {
        if (rb * 4 < a.I) {
            if (T <= 1) shared_gateup_block<1>(sa.x16, T, a.H, a.I, sa.w[0], sa.w[1], sa.h, rb, smem);
            else if (T <= 2) shared_gateup_block<2>(sa.x16, T, a.H, a.I, sa.w[0], sa.w[1], sa.h, rb, smem);
            else if (T <= 4) shared_gateup_block<4>(sa.x16, T, a.H, a.I, sa.w[0], sa.w[1], sa.h, rb, smem);
            else shared_gateup_block<8>(sa.x16, T, a.H, a.I, sa.w[0], sa.w[1], sa.h, rb, smem);
        }
    } else if (rb * 4 < a.H) {
        if (T <= 1) shared_down_block<1>(sa.h, T, a.H, a.I, sa.w[2], sa.y, rb, smem);
        else if (T <= 2) shared_down_block<2>(sa.h, T, a.H, a.I, sa.w[2], sa.y, rb, smem);
        else if (T <= 4) shared_down_block<4>(sa.h, T, a.H, a.I, sa.w[2], sa.y, rb, smem);
        else shared_down_block<8>(sa.h, T, a.H, a.I, sa.w[2], sa.y, rb, smem);
    }
    return true;
}

// gate/up + SwiGLU.  Block = CP pairs of 16-column tiles of one expert for
// both projections; wavefront w = 2p + j streams projection p, over input
// half j (CP = 1: one tile pair) or over all inputs for tile pair j (CP = 2).
// Rows are processed kGemvPass at a time: x * suh of the pass's rows in LDS
// (fp16, both projections), one MFMA per tile row for all of the pass's rows.
// The partial sums of the two halves meet in LDS and are added in a fixed
// order.  The launch takes CP = 2 (longer streams per wavefront amortise the
// staging of x * suh) unless that leaves fewer routed blocks than the GPU
// holds at once; then CP = 1 doubles the blocks.
template <int K, int CB, int CP>
__global__ __launch_bounds__(256, 4) void gemv_gateup_kernel(GroupArgs a, int max_list, SharedArgs sa)
{
    static_assert(CP == 1 || CP == 2, "gate/up tile pairs per block");
    constexpr int kGuCols = 32 * CP, kGuKH = 2 / CP;
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ float part[2 * kGemvPass][4];
    __shared__ float rsum[2][kGemvPass];
    __shared__ float psum[2][kGuKH][kGemvPass][kGuCols];   // [projection][half][row][column]
    if (shared_in_gemv(a, sa, max_list, true, (f16 *)smem))
        return;
    // experts vary slowest: the blocks of the listed experts dispatch before
    // those past the list's end, which only check the count and leave (the
    // list entry is read with the count: li < max_list is inside the list)
    const int li = blockIdx.y;
    const int n_gemv = ld_uniform(&a.hdr->n_gemv), e = ld_uniform(a.glist + li);
    if (li >= n_gemv)
        return;
    const int H = a.H, I = a.I;
    const int n0 = blockIdx.x * kGuCols;
    f16 *xs = (f16 *)smem;   // [2][kGemvPass][H]

    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), l = threadIdx.x & 63;
    const int pr = w >> 1, kh = kGuKH == 2 ? (w & 1) : 0, cp = CP == 2 ? (w & 1) : 0;
    const int c = l & 15, ts = (l >> 4) & 1, h = l >> 5;
    // the block's tile pair in every tile row of expert e's projection pr
    const TensorCodes tcs = tensor_codes<K>(a, pr, e, H, I);
    const int kw = K > 0 ? K : __builtin_amdgcn_readfirstlane(tcs.K);
    int d0, d1, q;
    frag_pos_rt(kw, c, h, d0, d1, q);
    const uint32_t rowb = (uint32_t)(I / 16) * 32u * kw;
    const __amdgpu_buffer_rsrc_t rs =
        buf_rsrc(tcs.base + (n0 / 16) * 8 * kw, tcs.bytes ? tcs.bytes - (uint32_t)(n0 / 16) * 32u * kw : 0u);
    const uint32_t tb = (uint32_t)(2 * cp + ts) * 8u * kw;
    const uint32_t m_lo = a.mcg & 0xFFFFu, m_hi = a.mcg >> 16;
    const int ntk = H / 16;
    GemvCodes cs;
    cs.rs = rs;
    cs.v0 = 4u * (tb + d0);
    cs.v1 = 4u * (tb + d1);
    cs.rowb = rowb;
    cs.tk0 = kh * (ntk / kGuKH);
    cs.tk1 = cs.tk0 + ntk / kGuKH;
    const int R = ld_uniform(a.counts + e);
    const int p0 = ld_uniform(a.offsets + e);
    // one round of staging: the pieces ch = threadIdx.x + 256 (it0 + it)
    auto load_suh = [&](f16x8 (&sv)[2][kStageIt], int it0) {
#pragma unroll
        for (int it = 0; it < kStageIt; ++it) {
            const int ch = threadIdx.x + 256 * (it0 + it);
#pragma unroll
            for (int pp = 0; pp < 2; ++pp)
                sv[pp][it] = ch < H / 8 ? *(const f16x8 *)(a.suh[pp] + (int64_t)e * H + 8 * ch) : (f16x8){};
        }
    };

    for (int r0 = 0; r0 < R; r0 += kGemvPass) {
        const int nr = min(kGemvPass, R - r0);
        // x * suh of the pass's rows for both projections, and their sums.
        // The rows' slot ids (rows past nr read the last row's) and the first
        // round's suh pieces go out first, then the code stream's first
        // groups, so the codes load while the slot -> token -> activation
        // chain runs; every x piece of a round is loaded before the first
        // product.
        int32_t slot[kGemvPass];
#pragma unroll
        for (int r = 0; r < kGemvPass; ++r)
            slot[r] = ld_uniform(a.sorted + p0 + r0 + min(r, nr - 1));
        f16x8 sv0[2][kStageIt];
        load_suh(sv0, 0);
        cs.prime();
        // (keeps the first use of the slot ids, and so their wait, below the
        // code loads)
        __builtin_amdgcn_sched_barrier(0);
        int64_t tok[kGemvPass];
#pragma unroll
        for (int r = 0; r < kGemvPass; ++r)
            tok[r] = slot_token(slot[r], a.nr, a.k);
        float sums[2 * kGemvPass] = {};
        for (int it0 = 0; 256 * it0 < H / 8; it0 += kStageIt) {
            f16x8 sv[2][kStageIt], xv[kGemvPass][kStageIt];
            if (it0 == 0) {
#pragma unroll
                for (int pp = 0; pp < 2; ++pp)
#pragma unroll
                    for (int it = 0; it < kStageIt; ++it)
                        sv[pp][it] = sv0[pp][it];
            } else {
                load_suh(sv, it0);
            }
#pragma unroll
            for (int it = 0; it < kStageIt; ++it) {
                const int ch = threadIdx.x + 256 * (it0 + it);
#pragma unroll
                for (int r = 0; r < kGemvPass; ++r)
                    xv[r][it] = ch < H / 8 && r < nr ? *(const f16x8 *)(a.x16 + tok[r] * H + 8 * ch) : (f16x8){};
            }
#pragma unroll
            for (int pp = 0; pp < 2; ++pp)
#pragma unroll
                for (int r = 0; r < kGemvPass; ++r)
#pragma unroll
                    for (int it = 0; it < kStageIt; ++it) {
                        const int ch = threadIdx.x + 256 * (it0 + it);
                        if (r >= nr || ch >= H / 8)
                            continue;
                        const f16x8 pv = xv[r][it] * sv[pp][it];
                        *(f16x8 *)(xs + ((size_t)pp * kGemvPass + r) * H + 8 * ch) = pv;
#pragma unroll
                        for (int j = 0; j < 8; ++j)
                            sums[pp * kGemvPass + r] += (float)pv[j];
                    }
        }
        block_reduce256<2 * kGemvPass>(sums, part);
        if (threadIdx.x == 0)
#pragma unroll
            for (int i = 0; i < 2 * kGemvPass; ++i)
                rsum[i / kGemvPass][i % kGemvPass] = sums[i];
        __syncthreads();

        // lane l's activation row: l % 32 for the pass's rows, the last one
        // for the rest (in range; their output rows are not read)
        const int ar = min(l & 31, nr - 1);
        const f16 *arow = xs + ((size_t)pr * kGemvPass + ar) * H + 8 * h;
        f32x16 d = {};
        gemv_stream_mfma_k<K, CB>(kw, cs, q, m_lo, m_hi, arow, d);
#pragma unroll
        for (int r = 0; r < kGemvPass; ++r)
            if (r < nr && h == 0)
                psum[pr][kh][r][32 * cp + 16 * ts + c] = d[r];
        __syncthreads();
        if (threadIdx.x < nr * kGuCols) {
            const int r = threadIdx.x / kGuCols, cc = threadIdx.x % kGuCols;
            const int col = n0 + cc;
            const float sg = kGuKH == 2 ? psum[0][0][r][cc] + psum[0][kGuKH - 1][r][cc] : psum[0][0][r][cc];
            const float su = kGuKH == 2 ? psum[1][0][r][cc] + psum[1][kGuKH - 1][r][cc] : psum[1][0][r][cc];
            const float g = (sg - kBias2 * rsum[0][r]) * (f16_to_f32(a.svh[0][(int64_t)e * I + col]) * (1.0f / 128.0f));
            const float u = (su - kBias2 * rsum[1][r]) * (f16_to_f32(a.svh[1][(int64_t)e * I + col]) * (1.0f / 128.0f));
            const float hv = silu_f(g) * u * f16_to_f32(a.suh[2][(int64_t)e * I + col]);
            a.hbuf[(int64_t)(p0 + r0 + r) * I + col] = f32_to_bf16_bits(hv);
        }
        __syncthreads();
    }
}

// down + routing weight.  Block = CP pairs of 16-column tiles of one
// expert; the input rows are split into S = 4 / CP (fewer for small inter
// sizes) ranges of a multiple of kGemvU tile rows, and wavefront w streams
// range w / CP of tile pair w % CP.  The pass's h rows sit
// in LDS as fp16, each scaled by a power of two that brings its largest
// magnitude into [2^14, 2^15): every bf16 value within 2^28 of the row
// maximum converts exactly, so the fp16 MFMA serves here as in gate/up, and
// the scale comes off the finished sum.
// Range sums meet in LDS and are added in a fixed order.  The launch takes
// CP = 4 (each wavefront streams every input row of its pair; faster than
// one or two when the grid fills the GPU) unless that leaves fewer routed
// blocks than the GPU holds at once; then the smallest CP (2 or 1) that
// fills it, or 1.
template <int K, int CB, int CP>
__global__ __launch_bounds__(256, 4) void gemv_down_kernel(GroupArgs a, int max_list, SharedArgs sa)
{
    static_assert(CP == 1 || CP == 2 || CP == 4, "down tile pairs per block");
    constexpr int kDownCP = CP, kDownCols = 32 * CP, kDownS = 4 / CP;
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ float part[2 * kGemvPass][4];
    __shared__ float rsum[kGemvPass];
    __shared__ int rexp[kGemvPass];
    __shared__ float psum[kDownS][kGemvPass][kDownCols];   // [range][row][column]
    if (shared_in_gemv(a, sa, max_list, false, (f16 *)smem))
        return;
    const int li = blockIdx.y;
    const int n_gemv = ld_uniform(&a.hdr->n_gemv), e = ld_uniform(a.glist + li);
    if (li >= n_gemv)
        return;
    const int H = a.H, I = a.I;
    const int m0 = blockIdx.x * kDownCols;
    f16 *hs = (f16 *)smem;   // [kGemvPass][I]

    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), l = threadIdx.x & 63;
    const int cp = w % kDownCP, kr = w / kDownCP;
    const int c = l & 15, ts = (l >> 4) & 1, h = l >> 5;
    const TensorCodes tcs = tensor_codes<K>(a, 2, e, I, H);
    const int kw = K > 0 ? K : __builtin_amdgcn_readfirstlane(tcs.K);
    int d0, d1, q;
    frag_pos_rt(kw, c, h, d0, d1, q);
    const uint32_t rowb = (uint32_t)(H / 16) * 32u * kw;
    const __amdgpu_buffer_rsrc_t rs =
        buf_rsrc(tcs.base + (m0 / 16) * 8 * kw, tcs.bytes ? tcs.bytes - (uint32_t)(m0 / 16) * 32u * kw : 0u);
    const uint32_t tb = (uint32_t)(2 * cp + ts) * 8u * kw;
    const uint32_t m_lo = a.mcg & 0xFFFFu, m_hi = a.mcg >> 16;
    // I % 128 == 0, so ntk is a multiple of kGemvU and S = 1 always fits
    const int ntk = I / 16;
    const int S = (kDownS >= 4 && ntk % (4 * kGemvU) == 0) ? 4 : (kDownS >= 2 && ntk % (2 * kGemvU) == 0) ? 2 : 1;
    GemvCodes cs;
    cs.rs = rs;
    cs.v0 = 4u * (tb + d0);
    cs.v1 = 4u * (tb + d1);
    cs.rowb = rowb;
    // wavefronts past the S ranges (kr >= S) stream nothing; their primed
    // loads read range 0 (in range, never used), so the prime needs no branch
    cs.tk0 = kr < S ? kr * (ntk / S) : 0;
    cs.tk1 = cs.tk0 + ntk / S;
    const int R = ld_uniform(a.counts + e);
    const int p0 = ld_uniform(a.offsets + e);
    // one round of h pieces ch = threadIdx.x + 256 (it0 + it) of the pass's rows
    auto load_h = [&](u32x4 (&raw)[kGemvPass][kStageIt], int r0, int nr, int it0) {
#pragma unroll
        for (int r = 0; r < kGemvPass; ++r)
#pragma unroll
            for (int it = 0; it < kStageIt; ++it) {
                const int ch = threadIdx.x + 256 * (it0 + it);
                raw[r][it] = r < nr && ch < I / 8 ? *(const u32x4 *)(a.hbuf + (int64_t)(p0 + r0 + r) * I + 8 * ch)
                                                  : (u32x4){0u, 0u, 0u, 0u};
            }
    };

    for (int r0 = 0; r0 < R; r0 += kGemvPass) {
        const int nr = min(kGemvPass, R - r0);
        // per row: the largest magnitude and the sum, in one reduction.  The
        // first round's pieces (all of a row up to I = 256 * 8 * kStageIt)
        // go out before the code stream's first groups and are kept for the
        // conversion below.
        float red[2 * kGemvPass] = {};   // [2r] max |h|, [2r + 1] sum h
        u32x4 held[kGemvPass][kStageIt];
        load_h(held, r0, nr, 0);
        cs.prime();
        __builtin_amdgcn_sched_barrier(0);
        for (int it0 = 0; 256 * it0 < I / 8; it0 += kStageIt) {
            u32x4 raw[kGemvPass][kStageIt];
            if (it0 == 0) {
#pragma unroll
                for (int r = 0; r < kGemvPass; ++r)
#pragma unroll
                    for (int it = 0; it < kStageIt; ++it)
                        raw[r][it] = held[r][it];
            } else {
                load_h(raw, r0, nr, it0);
            }
#pragma unroll
            for (int r = 0; r < kGemvPass; ++r)
#pragma unroll
                for (int it = 0; it < kStageIt; ++it)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float lo = __uint_as_float(raw[r][it][j] << 16),
                                    hi = __uint_as_float(raw[r][it][j] & 0xFFFF0000u);
                        red[2 * r] = fmaxf(red[2 * r], fmaxf(fabsf(lo), fabsf(hi)));
                        red[2 * r + 1] += lo + hi;
                    }
        }
        block_reduce256<2 * kGemvPass, 0x5u>(red, part);
        int ex[kGemvPass];
#pragma unroll
        for (int r = 0; r < kGemvPass; ++r) {
            // red * 2^ex in [2^14, 2^15); zero, inf and NaN rows keep scale 1
            const float mx = red[2 * r];
            ex[r] = (mx > 0.0f && mx < __builtin_inff()) ? 15 - __builtin_amdgcn_frexp_expf(mx) : 0;
        }
        // the scaled fp16 rows into LDS: the first round from the kept
        // pieces, later rounds (I > 256 * 8 * kStageIt) loaded again
        for (int it0 = 0; 256 * it0 < I / 8; it0 += kStageIt) {
            u32x4 raw[kGemvPass][kStageIt];
            if (it0 == 0) {
#pragma unroll
                for (int r = 0; r < kGemvPass; ++r)
#pragma unroll
                    for (int it = 0; it < kStageIt; ++it)
                        raw[r][it] = held[r][it];
            } else {
                load_h(raw, r0, nr, it0);
            }
#pragma unroll
            for (int r = 0; r < kGemvPass; ++r)
#pragma unroll
                for (int it = 0; it < kStageIt; ++it) {
                    const int ch = threadIdx.x + 256 * (it0 + it);
                    if (r >= nr || ch >= I / 8)
                        continue;
                    f16x8 hv;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        hv[2 * j] = (f16)__builtin_ldexpf(__uint_as_float(raw[r][it][j] << 16), ex[r]);
                        hv[2 * j + 1] = (f16)__builtin_ldexpf(__uint_as_float(raw[r][it][j] & 0xFFFF0000u), ex[r]);
                    }
                    *(f16x8 *)(hs + (size_t)r * I + 8 * ch) = hv;
                }
        }
        if (threadIdx.x == 0)
#pragma unroll
            for (int r = 0; r < kGemvPass; ++r) {
                rsum[r] = __builtin_ldexpf(red[2 * r + 1], ex[r]);
                rexp[r] = ex[r];
            }
        __syncthreads();

        const int ar = min(l & 31, nr - 1);
        const f16 *arow = hs + (size_t)ar * I + 8 * h;
        f32x16 d = {};
        if (kr < S)
            gemv_stream_mfma_k<K, CB>(kw, cs, q, m_lo, m_hi, arow, d);
#pragma unroll
        for (int r = 0; r < kGemvPass; ++r)
            if (kr < S && r < nr && h == 0)
                psum[kr][r][32 * cp + 16 * ts + c] = d[r];
        __syncthreads();
        if (threadIdx.x < nr * kDownCols) {
            const int r = threadIdx.x / kDownCols, cc = threadIdx.x % kDownCols;
            const int m = m0 + cc;
            float raw = psum[0][r][cc];
            if (S == 2)
                raw += psum[1 % kDownS][r][cc];
            else if (S == 4)
                raw = (psum[0][r][cc] + psum[1 % kDownS][r][cc]) + (psum[2 % kDownS][r][cc] + psum[3 % kDownS][r][cc]);
            const float tot = __builtin_ldexpf(raw - kBias2 * rsum[r], -rexp[r]);
            const int slot = a.sorted[p0 + r0 + r];
            const float svh = f16_to_f32(a.svh[2][(int64_t)e * H + m]) * (1.0f / 128.0f);
            a.ybuf[(int64_t)slot * H + m] = f32_to_bf16_bits(tot * svh * a.w[slot]);
        }
        __syncthreads();
    }
}

// Extra grid rows (of ncols blocks each) for the shared expert's blocks of 4
// weight rows out of n, and the LDS they need (TT token rows of a slab).
static unsigned shared_rows_of(const SharedArgs *sh, int n, int ncols)
{
    return sh ? (unsigned)((n / 4 + ncols - 1) / ncols) : 0u;
}

static size_t shared_lds_of(const SharedArgs *sh, int64_t T)
{
    const int tt = T <= 1 ? 1 : T <= 2 ? 2 : T <= 4 ? 4 : 8;
    return sh ? sizeof(f16) * tt * kShSlab : 0;
}

// Blocks of 256 threads the GPU holds at once at four wavefronts per SIMD.
constexpr int kResidentBlocks = 1024;

template <int K, int CB, int CP>
struct GateupKernel {
    static void go(dim3 grid, size_t lds, hipStream_t s, const GroupArgs &a, int max_list, const SharedArgs &sa)
    {
        gemv_gateup_kernel<K, CB, CP><<<grid, 256, lds, s>>>(a, max_list, sa);
    }
};
template <int K, int CB, int CP>
struct DownKernel {
    static void go(dim3 grid, size_t lds, hipStream_t s, const GroupArgs &a, int max_list, const SharedArgs &sa)
    {
        gemv_down_kernel<K, CB, CP><<<grid, 256, lds, s>>>(a, max_list, sa);
    }
};

// the kernel instance for the call's width and codebook
template <template <int, int, int> class KERNEL, int CP>
static void gemv_dispatch(dim3 grid, size_t lds, hipStream_t s, const GroupArgs &a, int max_list,
                          const SharedArgs &sa)
{
    if (a.code_tab && a.cb == 0) KERNEL<0, 0, CP>::go(grid, lds, s, a, max_list, sa);
    else if (a.code_tab) KERNEL<0, 1, CP>::go(grid, lds, s, a, max_list, sa);
    else if (a.K == 2 && a.cb == 0) KERNEL<2, 0, CP>::go(grid, lds, s, a, max_list, sa);
    else if (a.K == 3 && a.cb == 0) KERNEL<3, 0, CP>::go(grid, lds, s, a, max_list, sa);
    else if (a.K == 4 && a.cb == 0) KERNEL<4, 0, CP>::go(grid, lds, s, a, max_list, sa);
    else if (a.K == 2) KERNEL<2, 1, CP>::go(grid, lds, s, a, max_list, sa);
    else if (a.K == 3) KERNEL<3, 1, CP>::go(grid, lds, s, a, max_list, sa);
    else KERNEL<4, 1, CP>::go(grid, lds, s, a, max_list, sa);
}

// Tile pairs per block: the largest of `cps` (descending) whose routed grid
// of max_list experts fills the resident blocks, else the smallest.
static int gemv_cp(int max_list, int ncols, std::initializer_list<int> cps)
{
    int cp = 1;
    for (int c : cps) {
        cp = c;
        if ((int64_t)max_list * (ncols / (32 * c)) >= kResidentBlocks)
            break;
    }
    return cp;
}

template <int CP>
static void gateup_cp(const GroupArgs &a, int max_list, const SharedArgs *sh, hipStream_t s)
{
    // I % 128 == 0: whole blocks of 4 shared rows
    const unsigned nx = (unsigned)(a.I / (32 * CP));
    dim3 grid(nx, max_list + shared_rows_of(sh, a.I, (int)nx));
    const size_t lds = std::max(sizeof(f16) * 2 * kGemvPass * a.H, shared_lds_of(sh, a.T));
    gemv_dispatch<GateupKernel, CP>(grid, lds, s, a, max_list, sh ? *sh : SharedArgs{});
}

template <int CP>
static void down_cp(const GroupArgs &a, int max_list, const SharedArgs *sh, hipStream_t s)
{
    // H % 256 == 0: whole blocks of 4 shared rows
    const unsigned nx = (unsigned)(a.H / (32 * CP));
    dim3 grid(nx, max_list + shared_rows_of(sh, a.H, (int)nx));
    const size_t lds = std::max(sizeof(f16) * kGemvPass * a.I, shared_lds_of(sh, a.T));
    gemv_dispatch<DownKernel, CP>(grid, lds, s, a, max_list, sh ? *sh : SharedArgs{});
}

hipError_t launch_gemv_gateup(const GroupArgs &a, int max_list, const SharedArgs *sh, hipStream_t s)
{
    if (max_list <= 0)
        return hipSuccess;
    if (gemv_cp(max_list, a.I, {2, 1}) == 2)
        gateup_cp<2>(a, max_list, sh, s);
    else
        gateup_cp<1>(a, max_list, sh, s);
    return hipGetLastError();
}

hipError_t launch_gemv_down(const GroupArgs &a, int max_list, const SharedArgs *sh, hipStream_t s)
{
    if (max_list <= 0)
        return hipSuccess;
    const int cp = gemv_cp(max_list, a.H, {4, 2, 1});
    if (cp == 4)
        down_cp<4>(a, max_list, sh, s);
    else if (cp == 2)
        down_cp<2>(a, max_list, sh, s);
    else
        down_cp<1>(a, max_list, sh, s);
    return hipGetLastError();
}

template <int TT>
static void shared_gemv_launch(const uint16_t *x16, int T, int H, int I, const uint16_t *wg,
                               const uint16_t *wu, const uint16_t *wd, uint16_t *sh, float *sy,
                               hipStream_t s)
{
    shared_gemv_gateup_kernel<TT><<<(I + 3) / 4, 256, 0, s>>>(x16, T, H, I, wg, wu, sh);
    shared_gemv_down_kernel<TT><<<(H + 3) / 4, 256, 0, s>>>(sh, T, H, I, wd, sy);
}

hipError_t launch_shared_gemv(const uint16_t *x16, int T, int H, int I, const uint16_t *wg,
                              const uint16_t *wu, const uint16_t *wd, uint16_t *sh, float *sy,
                              hipStream_t s)
{
    // 1 <= T <= kSharedGemvMaxTokens (16)
    if (T <= 1) shared_gemv_launch<1>(x16, T, H, I, wg, wu, wd, sh, sy, s);
    else if (T <= 2) shared_gemv_launch<2>(x16, T, H, I, wg, wu, wd, sh, sy, s);
    else if (T <= 4) shared_gemv_launch<4>(x16, T, H, I, wg, wu, wd, sh, sy, s);
    else if (T <= 8) shared_gemv_launch<8>(x16, T, H, I, wg, wu, wd, sh, sy, s);
    else shared_gemv_launch<16>(x16, T, H, I, wg, wu, wd, sh, sy, s);
    return hipGetLastError();
}

}  // namespace moe
