// MFMA path for experts with many routed rows (prefill chunks; page
// "GLM-5.3 Flash EXL3 for 2x DGX Sparks", "Cold prefill (E3 grouped MoE)":
// gather, gate/up + SwiGLU, down + scatter from device segment tables).
//
// One work tile = (expert, 256 routed rows, a column slice).  The A operand
// (activation rows) is staged through LDS, double buffered, 64 input channels
// per stage.  The B operand never touches LDS: each lane decodes its own MFMA
// B fragment (8 consecutive input rows of one output column) straight from two
// code dwords into registers, so a wavefront decodes only the columns it owns
// and no decoded weight is ever written anywhere.
//
//   gate/up : A = x (fp16) gathered through the sorted slot list; B = 2v * suh
//             (fp16, exact 2v times fp16 suh); v_mfma_f32_32x32x16_f16;
//             epilogue g = acc * svh / 128, h = silu(g) * u * suh_down -> bf16
//   down    : A = h rows (bf16, contiguous per expert); B = 2v (bf16, exact);
//             v_mfma_f32_32x32x16_bf16; epilogue y = acc * svh / 128 * w -> fp32
//             row of the slot, summed per token by the combine kernel
//   shared  : the same loop with dense fp16 nn.Linear weights as B.
//
// MFMA 32x32x16 (16-bit inputs) lane layout, lane l: A row l%32, k 8*(l/32)+0..7;
// B column l%32, k 8*(l/32)+0..7; D register r holds row 8*(r/4) + 4*(l/32) + r%4,
// column l%32.
#include "common.h"
#include "internal.h"
#include "trellis.h"

namespace moe {

constexpr int kBM = kTileM;    // rows per work tile
constexpr int kMB = kBM / 32;  // 32-row MFMA blocks per work tile
constexpr int kBK = 64;        // input channels per stage
constexpr int kLdsRow = kBK + 8;   // fp16/bf16 elements per LDS row (16-byte pad)

enum Mode { GATEUP_TRELLIS = 0, DOWN_TRELLIS = 1, GATEUP_DENSE = 2, DOWN_DENSE = 3 };

template <int MODE>
struct ModeTraits {
    static constexpr bool kTrellis = MODE == GATEUP_TRELLIS || MODE == DOWN_TRELLIS;
    static constexpr bool kGateUp = MODE == GATEUP_TRELLIS || MODE == GATEUP_DENSE;
    static constexpr bool kBF16 = MODE == DOWN_TRELLIS;   // MFMA input type
    // columns per wavefront (gate/up: 32 gate + 32 up; down: 64)
    static constexpr int kWaveN = 64;
    static constexpr int kBlockN = kGateUp ? 4 * 32 : 4 * 64;   // output columns per block
};

struct GemmArgs {
    GroupArgs g;
    // dense (shared expert) operands
    const uint16_t *dA;      // [T][Kdim] fp16 rows
    const uint16_t *dB[2];   // nn.Linear [N][Kdim] fp16
    uint16_t *dOutH;         // shared gate/up output [T][I] fp16
    float *dOutY;            // shared down output [T][H] fp32
    int64_t T;
};

template <int MODE>
MOE_DEV f32x16 mfma_step(u32x4 a, u32x4 b, f32x16 c)
{
    if (ModeTraits<MODE>::kBF16)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                        __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                   __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

template <int MODE, int K, int CB>
__global__ __launch_bounds__(256, 1) void group_gemm_kernel(GemmArgs args)
{
    using TR = ModeTraits<MODE>;
    const GroupArgs &a = args.g;
    __shared__ __align__(16) uint16_t As[2][kBM * kLdsRow];

    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int H = a.H, I = a.I;
    const int Kdim = TR::kGateUp ? H : I;
    const int Nout = TR::kGateUp ? I : H;

    // ---- work tile
    int e = 0, rows, p0 = 0;
    int64_t t0 = 0;
    if (TR::kTrellis) {
        const int ti = blockIdx.x;
        if (ti >= a.hdr->n_tiles)
            return;
        e = a.tiles[2 * ti];
        const int m0 = a.tiles[2 * ti + 1];
        const int cnt = a.counts[e];
        rows = min(kBM, cnt - m0);
        p0 = a.offsets[e] + m0;
    } else {
        t0 = (int64_t)blockIdx.x * kBM;
        rows = (int)min<int64_t>(kBM, args.T - t0);
    }
    const int n0 = blockIdx.y * TR::kBlockN;

    // ---- A loader: thread -> 16-byte chunk `ach` of rows arow + 32 i
    const int ach = tid & 7, arow = tid >> 3;
    const uint16_t *asrc[kMB];
#pragma unroll
    for (int i = 0; i < kMB; ++i) {
        const int r = arow + 32 * i;
        const uint16_t *p = nullptr;
        if (r < rows) {
            if (MODE == GATEUP_TRELLIS)
                p = a.x16 + (int64_t)(a.sorted[p0 + r] / a.k) * H;
            else if (MODE == DOWN_TRELLIS)
                p = a.hbuf + (int64_t)(p0 + r) * I;
            else
                p = args.dA + (t0 + r) * (int64_t)Kdim;
        }
        asrc[i] = p;
    }
    u32x4 areg[kMB];
    auto load_a = [&](int s) {
#pragma unroll
        for (int i = 0; i < kMB; ++i)
            areg[i] = asrc[i] ? *(const u32x4 *)(asrc[i] + s * kBK + 8 * ach) : (u32x4){0, 0, 0, 0};
    };
    auto store_a = [&](int buf) {
#pragma unroll
        for (int i = 0; i < kMB; ++i)
            *(u32x4 *)(&As[buf][(arow + 32 * i) * kLdsRow + 8 * ach]) = areg[i];
    };

    // ---- B source: lane -> (column c of tile ts, k-half h)
    const int c = l & 15, ts = (l >> 4) & 1, h = l >> 5;
    // two B fragments per k-step: gate/up -> (gate, up) of the same 32 columns;
    // down -> two adjacent 32-column blocks
    int colb[2];
    if (TR::kGateUp) {
        colb[0] = colb[1] = n0 + 32 * w + 16 * ts + c;
    } else {
        colb[0] = n0 + 64 * w + 16 * ts + c;
        colb[1] = colb[0] + 32;
    }
    int d0 = 0, d1 = 0, q = 0;
    const uint32_t *cbase[2] = {nullptr, nullptr};
    int64_t rstride = 0;
    const uint16_t *dbase[2] = {nullptr, nullptr};
    if (TR::kTrellis) {
        frag_pos<K>(c, h, d0, d1, q);
        const int64_t per_expert = (int64_t)(Kdim / 16) * (Nout / 16) * Tile<K>::kDwords;
        rstride = (int64_t)(Nout / 16) * Tile<K>::kDwords;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int pr = TR::kGateUp ? j : 2;
            const int tn = colb[j] / 16;
            cbase[j] = (const uint32_t *)a.codes[pr] + e * per_expert + (int64_t)tn * Tile<K>::kDwords;
        }
    } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const uint16_t *W = TR::kGateUp ? args.dB[j] : args.dB[0];
            dbase[j] = W + (int64_t)colb[j] * Kdim + 8 * h;
        }
    }
    // raw B words of one stage: trellis 2 dwords per (fragment, k-step);
    // dense 16 bytes per (fragment, k-step)
    const uint16_t *suh_e[2] = {nullptr, nullptr};
    if constexpr (MODE == GATEUP_TRELLIS) {
        suh_e[0] = a.suh[0] + (int64_t)e * H + 8 * h;
        suh_e[1] = a.suh[1] + (int64_t)e * H + 8 * h;
    }
    // trellis: 2 code dwords per (fragment, k-step) [+ 8 suh values for gate/up];
    // dense: 16 weight bytes per (fragment, k-step)
    uint32_t craw[2][4][2];
    u32x4 draw[2][4];
    auto load_b = [&](int s) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) {
                if constexpr (TR::kTrellis) {
                    const uint32_t *tile = cbase[j] + (int64_t)(4 * s + kt) * rstride;
                    craw[j][kt][0] = tile[d0];
                    craw[j][kt][1] = tile[d1];
                    if constexpr (MODE == GATEUP_TRELLIS)
                        draw[j][kt] = *(const u32x4 *)(suh_e[j] + s * kBK + 16 * kt);
                } else {
                    draw[j][kt] = *(const u32x4 *)(dbase[j] + s * kBK + 16 * kt);
                }
            }
    };
    const uint32_t m_lo = a.mcg & 0xFFFFu, m_hi = a.mcg >> 16;

    f32x16 acc[kMB][2];
#pragma unroll
    for (int i = 0; i < kMB; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
            acc[i][j] = (f32x16){};

    const int nst = Kdim / kBK;
    load_a(0);
    load_b(0);
    store_a(0);
    __syncthreads();
    for (int s = 0; s < nst; ++s) {
        const int buf = s & 1;
        uint32_t cr[2][4][2];
        u32x4 dr[2][4];
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) {
                cr[j][kt][0] = craw[j][kt][0];
                cr[j][kt][1] = craw[j][kt][1];
                dr[j][kt] = draw[j][kt];
            }
        if (s + 1 < nst) {
            load_a(s + 1);
            load_b(s + 1);
        }
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            u32x4 bfrag[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                if constexpr (MODE == GATEUP_TRELLIS) {
                    const f16x8 v = frag_decode_f16<K, CB>(cr[j][kt][0], cr[j][kt][1], q, m_lo, m_hi);
                    bfrag[j] = __builtin_bit_cast(u32x4, v * __builtin_bit_cast(f16x8, dr[j][kt]));
                } else if constexpr (MODE == DOWN_TRELLIS) {
                    bfrag[j] = __builtin_bit_cast(u32x4, frag_decode_bf16<K, CB>(cr[j][kt][0], cr[j][kt][1], q, m_lo, m_hi));
                } else {
                    bfrag[j] = dr[j][kt];
                }
            }
#pragma unroll
            for (int i = 0; i < kMB; ++i) {
                const u32x4 af = *(const u32x4 *)(&As[buf][(32 * i + (l & 31)) * kLdsRow + 16 * kt + 8 * h]);
                acc[i][0] = mfma_step<MODE>(af, bfrag[0], acc[i][0]);
                acc[i][1] = mfma_step<MODE>(af, bfrag[1], acc[i][1]);
            }
        }
        if (s + 1 < nst)
            store_a(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue
    if (TR::kGateUp) {
        const int n = colb[0];
        float sg = 1.0f, su = 1.0f, sd = 1.0f;
        if (MODE == GATEUP_TRELLIS) {
            sg = f16_to_f32(a.svh[0][(int64_t)e * I + n]) * (1.0f / 128.0f);
            su = f16_to_f32(a.svh[1][(int64_t)e * I + n]) * (1.0f / 128.0f);
            sd = f16_to_f32(a.suh[2][(int64_t)e * I + n]);
        }
#pragma unroll
        for (int i = 0; i < kMB; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
                if (row < rows) {
                    const float g = acc[i][0][r] * sg, u = acc[i][1][r] * su;
                    const float hv = silu_f(g) * u * sd;
                    if (MODE == GATEUP_TRELLIS)
                        a.hbuf[(int64_t)(p0 + row) * I + n] = f32_to_bf16_bits(hv);
                    else
                        args.dOutH[(t0 + row) * I + n] = f32_to_f16_bits(hv);
                }
            }
    } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int m = colb[j];
            const float sv = MODE == DOWN_TRELLIS ? f16_to_f32(a.svh[2][(int64_t)e * H + m]) * (1.0f / 128.0f) : 1.0f;
#pragma unroll
            for (int i = 0; i < kMB; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
                    if (row < rows) {
                        if (MODE == DOWN_TRELLIS) {
                            const int slot = a.sorted[p0 + row];
                            a.ybuf[(int64_t)slot * H + m] = acc[i][j][r] * sv * a.w[slot];
                        } else {
                            args.dOutY[(t0 + row) * H + m] = acc[i][j][r];
                        }
                    }
                }
        }
    }
}

template <int MODE>
static hipError_t launch_mode(const GemmArgs &ga, dim3 grid, hipStream_t s)
{
    const GroupArgs &a = ga.g;
    if (ModeTraits<MODE>::kTrellis) {
        if (a.K == 2 && a.cb == 0) group_gemm_kernel<MODE, 2, 0><<<grid, 256, 0, s>>>(ga);
        else if (a.K == 3 && a.cb == 0) group_gemm_kernel<MODE, 3, 0><<<grid, 256, 0, s>>>(ga);
        else if (a.K == 4 && a.cb == 0) group_gemm_kernel<MODE, 4, 0><<<grid, 256, 0, s>>>(ga);
        else if (a.K == 2) group_gemm_kernel<MODE, 2, 1><<<grid, 256, 0, s>>>(ga);
        else if (a.K == 3) group_gemm_kernel<MODE, 3, 1><<<grid, 256, 0, s>>>(ga);
        else group_gemm_kernel<MODE, 4, 1><<<grid, 256, 0, s>>>(ga);
    } else {
        group_gemm_kernel<MODE, 2, 0><<<grid, 256, 0, s>>>(ga);
    }
    return hipGetLastError();
}

hipError_t launch_mfma_gateup(const GroupArgs &a, int max_tiles, hipStream_t s)
{
    if (max_tiles <= 0)
        return hipSuccess;
    GemmArgs ga{};
    ga.g = a;
    return launch_mode<GATEUP_TRELLIS>(ga, dim3(max_tiles, a.I / ModeTraits<GATEUP_TRELLIS>::kBlockN), s);
}

hipError_t launch_mfma_down(const GroupArgs &a, int max_tiles, hipStream_t s)
{
    if (max_tiles <= 0)
        return hipSuccess;
    GemmArgs ga{};
    ga.g = a;
    return launch_mode<DOWN_TRELLIS>(ga, dim3(max_tiles, a.H / ModeTraits<DOWN_TRELLIS>::kBlockN), s);
}

hipError_t launch_shared_gateup(const uint16_t *x16, int64_t T, int H, int I, const uint16_t *wg,
                                const uint16_t *wu, uint16_t *sh, hipStream_t s)
{
    GemmArgs ga{};
    ga.g.H = H;
    ga.g.I = I;
    ga.dA = x16;
    ga.dB[0] = wg;
    ga.dB[1] = wu;
    ga.dOutH = sh;
    ga.T = T;
    const dim3 grid((unsigned)((T + kBM - 1) / kBM), I / ModeTraits<GATEUP_DENSE>::kBlockN);
    return launch_mode<GATEUP_DENSE>(ga, grid, s);
}

hipError_t launch_shared_down(const uint16_t *sh, int64_t T, int H, int I, const uint16_t *wd,
                              float *sy, hipStream_t s)
{
    GemmArgs ga{};
    ga.g.H = H;
    ga.g.I = I;
    ga.dA = sh;
    ga.dB[0] = wd;
    ga.dOutY = sy;
    ga.T = T;
    const dim3 grid((unsigned)((T + kBM - 1) / kBM), H / ModeTraits<DOWN_DENSE>::kBlockN);
    return launch_mode<DOWN_DENSE>(ga, grid, s);
}

// ---------------------------------------------------------------- small kernels
// bf16 activations -> fp16 (exact for |x| in the fp16 normal range).
__global__ __launch_bounds__(256) void convert_x_kernel(const uint16_t *__restrict__ x, int64_t n8,
                                                        uint16_t *__restrict__ x16)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n8)
        return;
    const u32x4 v = ((const u32x4 *)x)[i];
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float lo = __uint_as_float(v[j] << 16), hi = __uint_as_float(v[j] & 0xFFFF0000u);
        o[j] = (uint32_t)f32_to_f16_bits(lo) | ((uint32_t)f32_to_f16_bits(hi) << 16);
    }
    ((u32x4 *)x16)[i] = o;
}

hipError_t launch_convert_x(const uint16_t *x, bool bf16, int64_t n, uint16_t *x16, hipStream_t s)
{
    (void)bf16;
    const int64_t n8 = n / 8;
    convert_x_kernel<<<(unsigned)((n8 + 255) / 256), 256, 0, s>>>(x, n8, x16);
    return hipGetLastError();
}

// out[t] = shared[t] + sum_j ybuf[t*k + j], cast to the activation dtype.
template <bool BF16>
__global__ __launch_bounds__(256) void combine_kernel(const float *__restrict__ ybuf,
                                                      const float *__restrict__ sy, int64_t T, int H,
                                                      int k, uint16_t *__restrict__ out)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;   // 4 outputs per thread
    const int64_t n4 = T * H / 4;
    if (i >= n4)
        return;
    const int64_t t = (4 * i) / H, m = (4 * i) % H;
    f32x4 s = sy ? *(const f32x4 *)(sy + t * H + m) : (f32x4){0, 0, 0, 0};
    for (int j = 0; j < k; ++j)
        s += *(const f32x4 *)(ybuf + (t * k + j) * H + m);
    uint32_t o0, o1;
    if (BF16) {
        o0 = (uint32_t)f32_to_bf16_bits(s[0]) | ((uint32_t)f32_to_bf16_bits(s[1]) << 16);
        o1 = (uint32_t)f32_to_bf16_bits(s[2]) | ((uint32_t)f32_to_bf16_bits(s[3]) << 16);
    } else {
        o0 = (uint32_t)f32_to_f16_bits(s[0]) | ((uint32_t)f32_to_f16_bits(s[1]) << 16);
        o1 = (uint32_t)f32_to_f16_bits(s[2]) | ((uint32_t)f32_to_f16_bits(s[3]) << 16);
    }
    *(u32x2 *)(out + t * H + m) = (u32x2){o0, o1};
}

hipError_t launch_combine(const float *ybuf, const float *sy, int64_t T, int H, int k, bool bf16,
                          uint16_t *out, hipStream_t s)
{
    const int64_t n4 = T * H / 4;
    const unsigned grid = (unsigned)((n4 + 255) / 256);
    if (bf16)
        combine_kernel<true><<<grid, 256, 0, s>>>(ybuf, sy, T, H, k, out);
    else
        combine_kernel<false><<<grid, 256, 0, s>>>(ybuf, sy, T, H, k, out);
    return hipGetLastError();
}

}  // namespace moe
