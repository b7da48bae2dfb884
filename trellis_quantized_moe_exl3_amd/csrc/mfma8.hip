// FP8 MFMA path of the E4M3-rounded codebook (page "GLM-5.3-Flash . exlr8
// (K2/K3/K4)", opening paragraph: every codebook value rounded to FP8 E4M3;
// "Loading": prefill runs on FP8 tensor cores).
//
// The decoded weight of this codebook IS an E4M3 number, so the B operand is
// exact: each lane decodes its 32 k-values straight to E4M3 bytes.  The
// activations carry the side vectors and a dynamic per-row scale:
//   gate/up : A_p[row] = E4M3(x[t] * suh_p[e] / s_p[row]), s_p = the least
//             power of two >= amax / 448, for p = gate, up (one row per
//             routed slot, sorted order);
//             g = acc_g * s_g * svh_g, u = acc_u * s_u * svh_u,
//             h = silu(g) * u * suh_down -> bf16 (as on the 16-bit path)
//   down    : A[row] = E4M3(h[row] / s_h[row]);  y = acc * s_h * svh_d * w.
// MFMA: v_mfma_scale_f32_32x32x64_f8f6f4 with unit block scales, 64 input
// channels per pipeline stage.  Lane l holds A row l % 32 / B column l % 32
// and the 32 channels 32 (l / 32) .. + 31 of the stage (any assignment of
// channels to (lane half, byte) works as long as A and B agree); D register
// r holds row 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32.
//
// Block = 8 wavefronts (two per SIMD): gate/up -> waves 0-3 gate, 4-7 up,
// 32 columns each; down -> 32 columns per wave.  The A stages of one
// or both operands go through a 4-slot LDS ring (LDS-direct loads, same
// 64-byte-row swizzle as the 16-bit path); B comes from code dwords in
// registers, prefetched 3 stages ahead, decoded one stage ahead.
#include "common.h"
#include "gemm.h"
#include "internal.h"
#include "trellis.h"

namespace moe {

constexpr int k8BM = kTileM;          // rows per work tile
constexpr int k8MB = k8BM / 32;       // 32-row MFMA blocks
constexpr int k8BK = 64;              // input channels (bytes of an A row) per stage
constexpr int k8Stage = k8BM * k8BK;  // bytes of one operand stage: 16 KiB
constexpr int k8Threads = 512;

template <bool GATEUP>
struct Traits8 {
    static constexpr int kOps = GATEUP ? 2 : 1;          // A operands in the ring
    static constexpr int kSlotBytes = kOps * k8Stage;
    static constexpr int kNA = 2 * kOps;                 // LDS-direct loads per wave and stage
    static constexpr int kNB = 8;                        // code dwords per column group and stage
    static constexpr int kBlockN = GATEUP ? 128 : 256;   // block columns at one group per wave
};

MOE_DEV f32x16 mfma8(i32x8 a, i32x8 b, f32x16 c)
{
    // operand formats 0 = FP8 E4M3; block scales 127 = 2^0
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

template <bool GATEUP, int K>
struct Tile8 {
    using TR = Traits8<GATEUP>;
    int w, l, c, ts, kh, pr;
    int rows, p0, e, col, Kdim;
    __amdgpu_buffer_rsrc_t arsrc[2], anull, brsrc, bnull;
    uint32_t aoff[2];      // LDS-direct: global byte offset of the lane's 16-byte piece
    uint32_t aread[2];     // LDS byte offsets of the lane's two 16-byte A pieces
    uint32_t boff[4];      // code dwords (d0, d1 of k-half 0; d0, d1 of k-half 1)
    uint32_t rstride;      // bytes between tile rows
    int qa, qb;
    uint32_t m_lo, m_hi;

    template <int CM>
    struct BRaw {
        uint32_t c[2][CM][4];   // [tile row of the lane's pair][column group][dword]
    };

    MOE_DEV void load_a(int s, int nst, LDS_AS uint8_t *ring)
    {
#pragma unroll
        for (int op = 0; op < TR::kOps; ++op) {
            const __amdgpu_buffer_rsrc_t rs = s < nst ? arsrc[op] : anull;
#pragma unroll
            for (int j = 0; j < 2; ++j)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rs, (LDS_AS void *)(ring + op * k8Stage + (32 * w + 16 * j) * k8BK), 16, aoff[j], s * k8BK, 0, 0);
        }
    }

    // the lane's tile rows of stage s: 4 s + 2 kh + r (2 kh is in boff)
    template <int CM>
    MOE_DEV void load_b(int s, int nst, BRaw<CM> &br)
    {
        const __amdgpu_buffer_rsrc_t rs = s < nst ? brsrc : bnull;
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int so = (4 * s + r) * (int)rstride;
#pragma unroll
            for (int cm = 0; cm < CM; ++cm) {
                const uint32_t go = (uint32_t)(cm * 2 * Tile<K>::kBytes);   // 32 columns on
#pragma unroll
                for (int d = 0; d < 4; ++d)
                    br.c[r][cm][d] = __builtin_amdgcn_raw_buffer_load_b32(rs, boff[d] + go, so, 0);
            }
        }
    }

    // B operand of column group cm: bytes k = 16 r + 8 h + t of the lane's 32
    template <int CM>
    MOE_DEV i32x8 decode(const BRaw<CM> &br, int cm) const
    {
        i32x8 b;
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const u32x2 lo = frag_decode_fp8<K>(br.c[r][cm][0], br.c[r][cm][1], qa, m_lo, m_hi);
            const u32x2 hi = frag_decode_fp8<K>(br.c[r][cm][2], br.c[r][cm][3], qb, m_lo, m_hi);
            b[4 * r + 0] = (int)lo[0];
            b[4 * r + 1] = (int)lo[1];
            b[4 * r + 2] = (int)hi[0];
            b[4 * r + 3] = (int)hi[1];
        }
        return b;
    }

    template <int NMB>
    MOE_DEV static void interleave()
    {
        constexpr int kV = (NMB >= 8) ? 12 : 96 / NMB;
#pragma unroll
        for (int i = 0; i < NMB; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, kV, 0);
        }
    }

    // One pipeline stage (ring slot SLOT = s % 4): wait for this wave's loads
    // of stage s, barrier, prefetch stage s + 3, read the A fragments, then
    // the MFMAs of each column group while the next group (or group 0 of
    // stage s + 1, carried in dk0) is decoded.  "At most 2 (NA + NB)
    // outstanding" proves the loads of stage s are done (loads complete in
    // issue order; every stage issues the same loads).
    template <int NMB, int CM, int SLOT>
    MOE_DEV void stage(int s, int nst, LDS_AS uint8_t *rg, LDS_AS uint8_t *rgp, const BRaw<CM> &bcur,
                       const BRaw<CM> &bnext, BRaw<CM> &bpf, i32x8 &dk0, f32x16 acc[k8MB])
    {
        constexpr int NA = TR::kNA, NB = TR::kNB * CM;
        __builtin_amdgcn_sched_barrier(0);
        wait_vmcnt<2 * (NA + NB)>();
        __builtin_amdgcn_s_barrier();
        load_a(s + 3, nst, rgp);
        load_b<CM>(s + 3, nst, bpf);
        const LDS_AS char *A = (const LDS_AS char *)rg + (GATEUP ? pr : 0) * k8Stage;
        i32x8 dcur = dk0;
#pragma unroll
        for (int f = 0; f < CM; ++f) {
            const i32x8 b = dcur;
            if (f + 1 < CM)
                dcur = decode<CM>(bcur, f + 1);
            else
                dcur = decode<CM>(bnext, 0);
            // A fragments are read right before their MFMA (registers are
            // scarce: 8 registers per fragment)
#pragma unroll
            for (int i = 0; i < NMB; ++i) {
                const u32x4 x0 = *(const LDS_AS u32x4 *)(A + aread[0] + i * 32 * k8BK);
                const u32x4 x1 = *(const LDS_AS u32x4 *)(A + aread[1] + i * 32 * k8BK);
                const i32x8 af = (i32x8){(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3],
                                         (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
                acc[f * NMB + i] = mfma8(af, b, acc[f * NMB + i]);
            }
            interleave<NMB>();
        }
        dk0 = dcur;
    }

    template <int NMB, int CM>
    MOE_DEV void run(LDS_AS uint8_t *r0, LDS_AS uint8_t *r1, LDS_AS uint8_t *r2, LDS_AS uint8_t *r3,
                     f32x16 acc[k8MB])
    {
        const int nst = Kdim / k8BK;   // a multiple of 4 (hidden, inter % 256 == 0 on this path)
        BRaw<CM> b0, b1, b2, b3;
        load_a(0, nst, r0);
        load_b<CM>(0, nst, b0);
        load_a(1, nst, r1);
        load_b<CM>(1, nst, b1);
        load_a(2, nst, r2);
        load_b<CM>(2, nst, b2);
        i32x8 dk0 = decode<CM>(b0, 0);
        for (int s = 0; s < nst; s += 4) {
            stage<NMB, CM, 0>(s, nst, r0, r3, b0, b1, b3, dk0, acc);
            stage<NMB, CM, 1>(s + 1, nst, r1, r0, b1, b2, b0, dk0, acc);
            stage<NMB, CM, 2>(s + 2, nst, r2, r1, b2, b3, b1, dk0, acc);
            stage<NMB, CM, 3>(s + 3, nst, r3, r2, b3, b0, b2, dk0, acc);
        }
        wait_vmcnt<0>();   // the trailing zero-range loads still write LDS
    }
};

template <bool GATEUP, int K, int NMB, int CM>
MOE_DEV void tile8_body(Tile8<GATEUP, K> &g, const GroupArgs &a, int n0, uint8_t *ring0, uint8_t *ring1,
                        uint8_t *ring2, uint8_t *ring3)
{
    using TR = Traits8<GATEUP>;
    constexpr int NB = NMB * CM;
    static_assert(NB <= k8MB, "accumulator blocks");
    const int Nout = GATEUP ? a.I : a.H;
    const int H = a.H, I = a.I;
    g.col = n0 + 32 * CM * (GATEUP ? (g.w & 3) : g.w) + 16 * g.ts + g.c;
    {
        int d0, d1, q;
        const int64_t per_expert = (int64_t)(g.Kdim / 16) * (Nout / 16) * Tile<K>::kBytes;
        g.rstride = (uint32_t)((Nout / 16) * Tile<K>::kBytes);
        g.brsrc = buf_rsrc((const char *)a.codes[g.pr] + g.e * per_expert, (uint32_t)per_expert);
        g.bnull = buf_rsrc((const char *)a.codes[g.pr], 0);
        const uint32_t base = (uint32_t)((g.col / 16) * Tile<K>::kBytes) + 2u * g.kh * g.rstride;
        frag_pos<K>(g.c, 0, d0, d1, q);
        g.qa = q;
        g.boff[0] = base + 4 * d0;
        g.boff[1] = base + 4 * d1;
        frag_pos<K>(g.c, 1, d0, d1, q);
        g.qb = q;
        g.boff[2] = base + 4 * d0;
        g.boff[3] = base + 4 * d1;
    }

    LDS_AS uint8_t *R0 = (LDS_AS uint8_t *)ring0, *R1 = (LDS_AS uint8_t *)ring1;
    LDS_AS uint8_t *R2 = (LDS_AS uint8_t *)ring2, *R3 = (LDS_AS uint8_t *)ring3;
    f32x16 acc[k8MB];
#pragma unroll
    for (int i = 0; i < k8MB; ++i)
        acc[i] = (f32x16){};
    g.template run<NMB, CM>(R0, R1, R2, R3, acc);
    __syncthreads();   // every wave is done with the rings (reused below)

    const int h = g.kh, rows = g.rows, e = g.e, p0 = g.p0;
    const int mblocks = (rows + 31) >> 5;
    if constexpr (GATEUP) {
        // the tile's row scales through LDS (one row per thread, in the second
        // half of ring 0, which the exchange below leaves alone)
        LDS_AS float *sgs = (LDS_AS float *)(R0 + k8Stage);
        LDS_AS float *sus = sgs + k8BM;
        if ((int)threadIdx.x < rows) {
            sgs[threadIdx.x] = a.sg8[p0 + threadIdx.x];
            sus[threadIdx.x] = a.su8[p0 + threadIdx.x];
        }
        __syncthreads();
        // gate wavefront w and up wavefront w + 4 hold the same columns.  In
        // rounds of four accumulator blocks, the up wavefront hands its scaled
        // values (acc * row scale * svh) of the first two blocks to the gate
        // wavefront through LDS and the gate wavefront its scaled values of
        // the last two to the up wavefront; each then finishes its two blocks
        const int cg = g.w & 3;
        float *ex = cg == 0 ? (float *)ring0 : cg == 1 ? (float *)ring1 : cg == 2 ? (float *)ring2 : (float *)ring3;
        const LDS_AS float *rsm = sgs + (g.pr == 0 ? 0 : k8BM);   // this projection's row scales
#pragma unroll
        for (int round = 0; round < (NB + 3) / 4; ++round) {
#pragma unroll
            for (int b = 4 * round; b < 4 * round + 4 && b < NB; ++b) {
                const int cm = b / NMB, i = b % NMB;
                const bool mine = (g.pr == 0) == ((b & 3) < 2);
                if (!mine && i < mblocks) {
                    const float sv = f16_to_f32(a.svh[g.pr][(int64_t)e * I + g.col + 32 * cm]);
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int row = min(32 * i + 8 * (r >> 2) + 4 * h + (r & 3), rows - 1);
                        ex[((b & 3) * 16 + r) * 64 + g.l] = acc[b][r] * rsm[row] * sv;
                    }
                }
            }
            __syncthreads();
#pragma unroll
            for (int b = 4 * round; b < 4 * round + 4 && b < NB; ++b) {
                const int cm = b / NMB, i = b % NMB;
                const int col = g.col + 32 * cm;
                const bool mine = (g.pr == 0) == ((b & 3) < 2);
                if (mine && i < mblocks) {
                    const float sv = f16_to_f32(a.svh[g.pr][(int64_t)e * I + col]);
                    const float sd = f16_to_f32(a.suh[2][(int64_t)e * I + col]);
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int row = 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
                        if (row < rows) {
                            const float own = acc[b][r] * rsm[row] * sv;
                            const float other = ex[((b & 3) * 16 + r) * 64 + g.l];
                            const float gv = g.pr == 0 ? own : other;
                            const float uv = g.pr == 0 ? other : own;
                            a.hbuf[(int64_t)(p0 + row) * I + col] = f32_to_bf16_bits(silu_f(gv) * uv * sd);
                        }
                    }
                }
            }
            __syncthreads();
        }
    } else {
        // the tile's slot ids and per-row factors (row scale times routing
        // weight) through LDS (one row per thread; the rings are free now)
        // rather than as dependent global loads for every accumulator element
        LDS_AS int *slots = (LDS_AS int *)R0;
        LDS_AS float *rw = (LDS_AS float *)(R0 + 4 * k8BM);
        if ((int)threadIdx.x < rows) {
            const int slot = a.sorted[p0 + threadIdx.x];
            slots[threadIdx.x] = slot;
            // the row scale is a power of two, so folding it into the routing
            // weight rounds the same way as applying the two in turn
            rw[threadIdx.x] = a.sh8[p0 + threadIdx.x] * a.w[slot];
        }
        __syncthreads();
        // each wavefront turns a 32 x 32 accumulator block into bf16 rows in
        // its own 2 KiB of ring 1, then stores 16 bytes per lane of a row
        LDS_AS uint16_t *tw = (LDS_AS uint16_t *)R1 + 1024 * g.w;
        const int lc = g.l & 31;
#pragma unroll
        for (int cm = 0; cm < CM; ++cm) {
            const int col = g.col + 32 * cm;
            const float sv = f16_to_f32(a.svh[2][(int64_t)e * H + col]);
#pragma unroll
            for (int i = 0; i < NMB; ++i) {
                if (i < mblocks) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int rl = 8 * (r >> 2) + 4 * h + (r & 3);
                        tw[rl * 32 + lc] = f32_to_bf16_bits(acc[cm * NMB + i][r] * sv * rw[32 * i + rl]);
                    }
#pragma unroll
                    for (int q = 0; q < 2; ++q) {
                        const int rl = (g.l >> 2) + 16 * q, row = 32 * i + rl;
                        const u32x4 v = *(const LDS_AS u32x4 *)(tw + rl * 32 + 8 * (g.l & 3));
                        if (row < rows)
                            *(u32x4 *)(a.ybuf + (int64_t)slots[row] * H + (col - lc) + 8 * (g.l & 3)) = v;
                    }
                }
            }
        }
    }
}

template <bool GATEUP, int K>
__global__ __launch_bounds__(k8Threads, 1) void gemm8_kernel(GroupArgs a, int nslices)
{
    using TR = Traits8<GATEUP>;
    // four ring slots (distinct LDS objects: the compiler tells their
    // LDS-direct writes apart)
    __shared__ __align__(16) uint8_t ring0[TR::kSlotBytes];
    __shared__ __align__(16) uint8_t ring1[TR::kSlotBytes];
    __shared__ __align__(16) uint8_t ring2[TR::kSlotBytes];
    __shared__ __align__(16) uint8_t ring3[TR::kSlotBytes];

    Tile8<GATEUP, K> g;
    g.w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    g.l = threadIdx.x & 63;
    g.Kdim = GATEUP ? a.H : a.I;

    int ti, slice;
    xcd_map(blockIdx.x, nslices, ti, slice);
    if (ti >= a.hdr->n_tiles)
        return;
    g.e = a.tiles[2 * ti];
    const int m0 = a.tiles[2 * ti + 1];
    g.rows = min(k8BM, a.counts[g.e] - m0);
    g.p0 = a.offsets[g.e] + m0;
    const int mblocks = (g.rows + 31) >> 5;
    // one column group per wavefront (the prefetched code dwords of a second
    // group would not fit next to 128 accumulator registers)
    const int n0 = slice * TR::kBlockN;

    // ---- A rows of the tile (contiguous in sorted order)
    {
        const uint8_t *src0 = GATEUP ? a.a8g : a.h8;
        const uint8_t *src1 = GATEUP ? a.a8u : a.h8;
        const uint32_t bytes = (uint32_t)((int64_t)g.rows * g.Kdim);
        g.arsrc[0] = buf_rsrc(src0 + (int64_t)g.p0 * g.Kdim, bytes);
        g.arsrc[1] = buf_rsrc(src1 + (int64_t)g.p0 * g.Kdim, bytes);
        g.anull = buf_rsrc(src0, 0);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int r = 32 * g.w + 16 * j + (g.l >> 2);
            const int rc = min(r, g.rows - 1);   // rows past the tile's end repeat its last row
            const int piece = a_slot(r, g.l & 3);
            g.aoff[j] = (uint32_t)(rc * g.Kdim + 16 * piece);
        }
        g.kh = g.l >> 5;
        const int r = g.l & 31;
#pragma unroll
        for (int j = 0; j < 2; ++j)
            g.aread[j] = (uint32_t)(r * k8BK + 16 * a_slot(r, 2 * g.kh + j));
    }
    g.c = g.l & 15;
    g.ts = (g.l >> 4) & 1;
    g.pr = GATEUP ? (g.w >> 2) : 2;
    g.m_lo = a.mcg & 0xFFFFu;
    g.m_hi = a.mcg >> 16;

    if (mblocks <= 2) {
        tile8_body<GATEUP, K, 2, 1>(g, a, n0, ring0, ring1, ring2, ring3);
    } else if (mblocks <= 4) {
        tile8_body<GATEUP, K, 4, 1>(g, a, n0, ring0, ring1, ring2, ring3);
    } else if (mblocks <= 6) {
        tile8_body<GATEUP, K, 6, 1>(g, a, n0, ring0, ring1, ring2, ring3);
    } else {
        tile8_body<GATEUP, K, 8, 1>(g, a, n0, ring0, ring1, ring2, ring3);
    }
}

template <bool GATEUP>
static hipError_t launch8(const GroupArgs &a, int max_tiles, hipStream_t s)
{
    if (max_tiles <= 0)
        return hipSuccess;
    const int nslices = (GATEUP ? a.I : a.H) / Traits8<GATEUP>::kBlockN;
    const unsigned grid = (unsigned)(((max_tiles + 7) / 8) * 8 * nslices);
    if (a.K == 2) gemm8_kernel<GATEUP, 2><<<grid, k8Threads, 0, s>>>(a, nslices);
    else if (a.K == 3) gemm8_kernel<GATEUP, 3><<<grid, k8Threads, 0, s>>>(a, nslices);
    else gemm8_kernel<GATEUP, 4><<<grid, k8Threads, 0, s>>>(a, nslices);
    return hipGetLastError();
}

hipError_t launch_mfma8_gateup(const GroupArgs &a, int max_tiles, hipStream_t s)
{
    return launch8<true>(a, max_tiles, s);
}

hipError_t launch_mfma8_down(const GroupArgs &a, int max_tiles, hipStream_t s)
{
    return launch8<false>(a, max_tiles, s);
}

// ------------------------------------------------------------ row quantizers
// Row scale: the least power of two s with amax / s <= 448 (the largest
// finite E4M3 value), found exactly from amax = m 2^e, m in [0.5, 1), and
// 448 = 0.875 2^9.  The scaled convert below takes its scale as a power of
// two (only the exponent of the fp32 operand counts) and does not saturate
// (anything past 464 becomes NaN), so both properties matter.  An all-zero
// row gets scale 1.
MOE_DEV float e4m3_row_scale(float amax)
{
    if (!(amax > 0.0f))
        return 1.0f;
    int e;
    const float m = frexpf(amax, &e);
    return ldexpf(1.0f, e - 9 + (m > 0.875f ? 1 : 0));
}

// eight fp32 values / s -> eight E4M3 bytes, nearest-even (s a power of two:
// the division is exact)
MOE_DEV u32x2 e4m3_pack8(const float v[8], float s)
{
    u32x2 o;
#pragma unroll
    for (int d = 0; d < 2; ++d) {
        s16x2 w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32((s16x2){0, 0}, v[4 * d], v[4 * d + 1], s, false);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, v[4 * d + 2], v[4 * d + 3], s, true);
        o[d] = __builtin_bit_cast(uint32_t, w);
    }
    return o;
}

// Wave-wide maximum of a non-negative float (all 64 lanes hold the result).
MOE_DEV float wave_max64(float v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

// One wavefront per routed slot a (slot order, four per block), written as
// row p = pos[a] of the sorted order: x[t] * suh_p[e] for gate and up, each
// scaled by its row amax / 448 and rounded to E4M3.  The row's expert is its slot's top-k expert (for the
// trellis shared expert's slots past the routed ones, the last expert).  Lane
// l holds the 16-byte pieces l, l + 64, ... of the three rows (at most NC of
// them: H <= 512 NC) between the amax reduction and the conversion; the
// products are exact in fp32 and formed again for the conversion.
template <int NC>
__global__ __launch_bounds__(256) void quant_gateup_kernel(GroupArgs a, int64_t n)
{
    // rows in slot order (the k slots of a token side by side, so its
    // activation row is read once from memory), each written at its sorted
    // position
    const int64_t slot = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (slot >= n)
        return;
    const int l = threadIdx.x & 63, H = a.H;
    const int64_t p = a.pos[slot];
    // a slot left out of the tables (an expert index outside [0, E), flagged
    // in the status word) has no position: nothing is written for it
    if ((uint64_t)p >= (uint64_t)n)
        return;
    const int64_t t = slot_token(slot, a.nr, a.k);
    // (clamped: an index outside the table, which the segment kernels flag
    // in the status word, still reads inside the side-vector arrays)
    const int e = slot < a.nr ? min(max(a.idx[slot], 0), a.E - 1) : a.E - 1;
    // lane l takes 32-byte pieces 64c + l of the row (16 channels each: the
    // fp8 path's hidden sizes are multiples of 256), so each projection's
    // quantized piece leaves in one 16-byte store
    constexpr int NP = (NC + 1) / 2;
    const f16x8 *xr = (const f16x8 *)(a.x16 + t * H);
    const f16x8 *sg = (const f16x8 *)(a.suh[0] + (int64_t)e * H);
    const f16x8 *su = (const f16x8 *)(a.suh[1] + (int64_t)e * H);
    const int np = H / 16;
    f16x8 xv[NP][2], gv[NP][2], uv[NP][2];
#pragma unroll
    for (int c = 0; c < NP; ++c) {
        const int q = 64 * c + l < np ? 64 * c + l : np - 1;   // in bounds; past np never used
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            xv[c][hh] = xr[2 * q + hh];
            gv[c][hh] = sg[2 * q + hh];
            uv[c][hh] = su[2 * q + hh];
        }
    }
    float mg = 0.0f, mu = 0.0f;
#pragma unroll
    for (int c = 0; c < NP; ++c)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (64 * c + l < np) {
                    mg = fmaxf(mg, fabsf((float)xv[c][hh][j] * (float)gv[c][hh][j]));
                    mu = fmaxf(mu, fabsf((float)xv[c][hh][j] * (float)uv[c][hh][j]));
                }
    const float s_g = e4m3_row_scale(wave_max64(mg));
    const float s_u = e4m3_row_scale(wave_max64(mu));
#pragma unroll
    for (int c = 0; c < NP; ++c) {
        const int q = 64 * c + l;
        if (q >= np)
            break;
        u32x4 og, ou;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            float vg[8], vu[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                vg[j] = (float)xv[c][hh][j] * (float)gv[c][hh][j];
                vu[j] = (float)xv[c][hh][j] * (float)uv[c][hh][j];
            }
            const u32x2 pg = e4m3_pack8(vg, s_g), pu = e4m3_pack8(vu, s_u);
            og[2 * hh] = pg[0];
            og[2 * hh + 1] = pg[1];
            ou[2 * hh] = pu[0];
            ou[2 * hh + 1] = pu[1];
        }
        __builtin_nontemporal_store(og, (u32x4 *)(a.a8g + p * H + 16 * q));
        __builtin_nontemporal_store(ou, (u32x4 *)(a.a8u + p * H + 16 * q));
    }
    if (l == 0) {
        a.sg8[p] = s_g;
        a.su8[p] = s_u;
    }
}

// One wavefront per routed row p, four rows per block: h[p] (bf16, already
// times suh_down; I <= 512 NC) scaled by its amax / 448 and rounded to E4M3.
template <int NC>
__global__ __launch_bounds__(256) void quant_h_kernel(GroupArgs a, int64_t n)
{
    const int64_t p = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (p >= n)
        return;
    const int l = threadIdx.x & 63, I = a.I;
    const u32x4 *hr = (const u32x4 *)(a.hbuf + p * I);
    const int np = I / 8;
    u32x4 raw[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c)
        raw[c] = hr[64 * c + l < np ? 64 * c + l : np - 1];
    float m = 0.0f;
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (64 * c + l < np)
                m = fmaxf(m, fmaxf(fabsf(__uint_as_float(raw[c][j] << 16)),
                               fabsf(__uint_as_float(raw[c][j] & 0xFFFF0000u))));
    const float s = e4m3_row_scale(wave_max64(m));
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        if (64 * c + l >= np)
            break;
        float v[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[2 * j] = __uint_as_float(raw[c][j] << 16);
            v[2 * j + 1] = __uint_as_float(raw[c][j] & 0xFFFF0000u);
        }
        *(u32x2 *)(a.h8 + p * I + 8 * (64 * c + l)) = e4m3_pack8(v, s);
    }
    if (l == 0)
        a.sh8[p] = s;
}

// Rows of `width` channels (a multiple of 8, at most 512 * 16 for gate/up and
// 512 * 32 for h): NC = pieces per lane, rounded up to a power of two.
template <template <int> class KERNEL>
static hipError_t launch_rows(const GroupArgs &a, int64_t n, int width, int max_nc, hipStream_t s)
{
    if (n <= 0)
        return hipSuccess;
    const int need = (width / 8 + 63) / 64;
    if (width % 8 || need > max_nc)
        return hipErrorInvalidValue;
    const unsigned grid = (unsigned)((n + 3) / 4);
    if (need <= 1) KERNEL<1>::launch(grid, a, n, s);
    else if (need <= 2) KERNEL<2>::launch(grid, a, n, s);
    else if (need <= 4) KERNEL<4>::launch(grid, a, n, s);
    else if (need <= 8) KERNEL<8>::launch(grid, a, n, s);
    else if (need <= 16) KERNEL<16>::launch(grid, a, n, s);
    else KERNEL<32>::launch(grid, a, n, s);
    return hipGetLastError();
}

template <int NC>
struct QuantGateup {
    static void launch(unsigned grid, const GroupArgs &a, int64_t n, hipStream_t s)
    {
        if constexpr (NC <= 16)   // (three rows of 32 pieces per lane would not fit in registers)
            quant_gateup_kernel<NC><<<grid, 256, 0, s>>>(a, n);
    }
};
template <int NC>
struct QuantH {
    static void launch(unsigned grid, const GroupArgs &a, int64_t n, hipStream_t s)
    {
        quant_h_kernel<NC><<<grid, 256, 0, s>>>(a, n);
    }
};

hipError_t launch_quant_gateup(const GroupArgs &a, int64_t n, hipStream_t s)
{
    return launch_rows<QuantGateup>(a, n, a.H, kQuantMaxHidden / 512, s);
}

hipError_t launch_quant_h(const GroupArgs &a, int64_t n, hipStream_t s)
{
    return launch_rows<QuantH>(a, n, a.I, 32, s);
}

}  // namespace moe
