// Decode-fused GEMV path for experts with few routed rows (decode-sized
// steps; page "GLM-5.3 Flash EXL3 for 2x DGX Sparks", "What runs": one fused
// launch per layer for decode-sized steps, trellis decoded inside the matmul;
// page "GLM-5.3-Flash EXL3 (~2.1 bpw, SM70 tile order)", "Speed": direct
// per-lane window loads with a deep prefetch).
//
// Each lane decodes eight consecutive input rows of one output column from
// two code dwords and feeds them to fp16/bf16 dot products, so a wavefront
// streams two tiles per step and every output column stays in one lane.  The
// code stream is read exactly once per expert; it is the only large HBM
// traffic of a decode-sized step.
#include "common.h"
#include "internal.h"
#include "trellis.h"

namespace moe {

constexpr int kGemvU = 8;   // tile rows per prefetch group

// gate/up + SwiGLU.  Block = 4 wavefronts = (gate, up) x 2 tile pairs = 64
// output columns of one expert; grid.x walks the GEMV expert list.
template <int K, int CB>
__global__ __launch_bounds__(256) void gemv_gateup_kernel(GroupArgs a, int rows_cap)
{
    extern __shared__ __align__(16) unsigned char smem[];
    const int li = blockIdx.x;
    if (li >= a.hdr->n_gemv)
        return;
    const int H = a.H, I = a.I;
    const int e = a.glist[li];
    const int R = a.counts[e];
    const int p0 = a.offsets[e];
    const int n0 = blockIdx.y * 64;
    f16 *xs = (f16 *)smem;      // [2][rows_cap][H]
    float *gu = (float *)smem;  // [2][rows_cap][64], reuses xs after the main loop

    // x * suh for both projections, fp16
    const int nchunk = H / 8;
    for (int i = threadIdx.x; i < 2 * R * nchunk; i += 256) {
        const int pr = i / (R * nchunk), rem = i % (R * nchunk);
        const int r = rem / nchunk, ch = rem % nchunk;
        const int t = a.sorted[p0 + r] / a.k;
        const f16x8 xv = *(const f16x8 *)(a.x16 + (int64_t)t * H + 8 * ch);
        const f16x8 sv = *(const f16x8 *)(a.suh[pr] + (int64_t)e * H + 8 * ch);
        *(f16x8 *)(xs + ((size_t)pr * rows_cap + r) * H + 8 * ch) = xv * sv;
    }
    __syncthreads();

    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    const int pr = w >> 1, tp = w & 1;
    const int c = l & 15, ts = (l >> 4) & 1, h = l >> 5;
    const int tn = n0 / 16 + 2 * tp + ts;
    int d0, d1, q;
    frag_pos<K>(c, h, d0, d1, q);
    const int64_t per_expert = (int64_t)(H / 16) * (I / 16) * Tile<K>::kDwords;
    const uint32_t *cb = (const uint32_t *)a.codes[pr] + e * per_expert + (int64_t)tn * Tile<K>::kDwords;
    const int64_t rstride = (int64_t)(I / 16) * Tile<K>::kDwords;
    const uint32_t m_lo = a.mcg & 0xFFFFu, m_hi = a.mcg >> 16;
    const f16 *xsp = xs + (size_t)pr * rows_cap * H + 8 * h;

    float acc[kGemvMaxRows];
#pragma unroll
    for (int r = 0; r < kGemvMaxRows; ++r)
        acc[r] = 0.0f;

    const int ntk = H / 16;
    uint32_t nx[kGemvU][2];
#pragma unroll
    for (int u = 0; u < kGemvU; ++u) {
        nx[u][0] = cb[u * rstride + d0];
        nx[u][1] = cb[u * rstride + d1];
    }
    for (int g = 0; g < ntk; g += kGemvU) {
        uint32_t cu[kGemvU][2];
#pragma unroll
        for (int u = 0; u < kGemvU; ++u) {
            cu[u][0] = nx[u][0];
            cu[u][1] = nx[u][1];
        }
        if (g + kGemvU < ntk) {
            const uint32_t *nb = cb + (int64_t)(g + kGemvU) * rstride;
#pragma unroll
            for (int u = 0; u < kGemvU; ++u) {
                nx[u][0] = nb[u * rstride + d0];
                nx[u][1] = nb[u * rstride + d1];
            }
        }
#pragma unroll
        for (int u = 0; u < kGemvU; ++u) {
            const f16x8 v = frag_decode_f16<K, CB>(cu[u][0], cu[u][1], q, m_lo, m_hi);
            const int kk = 16 * (g + u);
#pragma unroll
            for (int r = 0; r < kGemvMaxRows; ++r) {
                if (r < R && r < rows_cap) {
                    const f16x8 xv = *(const f16x8 *)(xsp + (size_t)r * H + kk);
                    float s = acc[r];
                    s = __builtin_amdgcn_fdot2((f16x2){v[0], v[1]}, (f16x2){xv[0], xv[1]}, s, false);
                    s = __builtin_amdgcn_fdot2((f16x2){v[2], v[3]}, (f16x2){xv[2], xv[3]}, s, false);
                    s = __builtin_amdgcn_fdot2((f16x2){v[4], v[5]}, (f16x2){xv[4], xv[5]}, s, false);
                    s = __builtin_amdgcn_fdot2((f16x2){v[6], v[7]}, (f16x2){xv[6], xv[7]}, s, false);
                    acc[r] = s;
                }
            }
        }
    }
    // the two k-halves of a column sit in lanes l and l ^ 32
    const int col = 16 * (2 * tp + ts) + c;
    const float svh = f16_to_f32(a.svh[pr][(int64_t)e * I + n0 + col]) * (1.0f / 128.0f);
    float tot[kGemvMaxRows];
#pragma unroll
    for (int r = 0; r < kGemvMaxRows; ++r)
        tot[r] = acc[r] + __shfl_xor(acc[r], 32, 64);
    __syncthreads();   // every wavefront is done reading xs
#pragma unroll
    for (int r = 0; r < kGemvMaxRows; ++r) {
        if (r < R && r < rows_cap) {
            if (h == 0)
                gu[((size_t)pr * rows_cap + r) * 64 + col] = tot[r] * svh;
        }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < R * 64; i += 256) {
        const int r = i / 64, cc = i % 64;
        const float g = gu[(size_t)r * 64 + cc];
        const float u = gu[((size_t)rows_cap + r) * 64 + cc];
        const float hv = silu_f(g) * u * f16_to_f32(a.suh[2][(int64_t)e * I + n0 + cc]);
        a.hbuf[(int64_t)(p0 + r) * I + n0 + cc] = f32_to_bf16_bits(hv);
    }
}

// down + routing-weighted scatter.  Block = 4 wavefronts x 2 tiles = 128
// output columns of one expert.
template <int K, int CB>
__global__ __launch_bounds__(256) void gemv_down_kernel(GroupArgs a, int rows_cap)
{
    extern __shared__ __align__(16) unsigned char smem[];
    const int li = blockIdx.x;
    if (li >= a.hdr->n_gemv)
        return;
    const int H = a.H, I = a.I;
    const int e = a.glist[li];
    const int R = a.counts[e];
    const int p0 = a.offsets[e];
    const int m0 = blockIdx.y * 128;
    uint16_t *hs = (uint16_t *)smem;   // [rows_cap][I] bf16
    const int nchunk = I / 8;
    for (int i = threadIdx.x; i < R * nchunk; i += 256) {
        const int r = i / nchunk, ch = i % nchunk;
        *(u32x4 *)(hs + (size_t)r * I + 8 * ch) = *(const u32x4 *)(a.hbuf + (int64_t)(p0 + r) * I + 8 * ch);
    }
    __syncthreads();

    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    const int c = l & 15, ts = (l >> 4) & 1, h = l >> 5;
    const int tn = m0 / 16 + 2 * w + ts;
    int d0, d1, q;
    frag_pos<K>(c, h, d0, d1, q);
    const int64_t per_expert = (int64_t)(I / 16) * (H / 16) * Tile<K>::kDwords;
    const uint32_t *cb = (const uint32_t *)a.codes[2] + e * per_expert + (int64_t)tn * Tile<K>::kDwords;
    const int64_t rstride = (int64_t)(H / 16) * Tile<K>::kDwords;
    const uint32_t m_lo = a.mcg & 0xFFFFu, m_hi = a.mcg >> 16;
    const uint16_t *hsp = hs + 8 * h;

    float acc[kGemvMaxRows];
#pragma unroll
    for (int r = 0; r < kGemvMaxRows; ++r)
        acc[r] = 0.0f;
    const int ntk = I / 16;
    uint32_t nx[kGemvU][2];
#pragma unroll
    for (int u = 0; u < kGemvU; ++u) {
        nx[u][0] = cb[u * rstride + d0];
        nx[u][1] = cb[u * rstride + d1];
    }
    for (int g = 0; g < ntk; g += kGemvU) {
        uint32_t cu[kGemvU][2];
#pragma unroll
        for (int u = 0; u < kGemvU; ++u) {
            cu[u][0] = nx[u][0];
            cu[u][1] = nx[u][1];
        }
        if (g + kGemvU < ntk) {
            const uint32_t *nb = cb + (int64_t)(g + kGemvU) * rstride;
#pragma unroll
            for (int u = 0; u < kGemvU; ++u) {
                nx[u][0] = nb[u * rstride + d0];
                nx[u][1] = nb[u * rstride + d1];
            }
        }
#pragma unroll
        for (int u = 0; u < kGemvU; ++u) {
            const bf16x8 v = frag_decode_bf16<K, CB>(cu[u][0], cu[u][1], q, m_lo, m_hi);
            const int kk = 16 * (g + u);
#pragma unroll
            for (int r = 0; r < kGemvMaxRows; ++r) {
                if (r < R && r < rows_cap) {
                    const bf16x8 hv = *(const bf16x8 *)(hsp + (size_t)r * I + kk);
                    float s = acc[r];
                    s = __builtin_amdgcn_fdot2_f32_bf16((bf16x2){v[0], v[1]}, (bf16x2){hv[0], hv[1]}, s, false);
                    s = __builtin_amdgcn_fdot2_f32_bf16((bf16x2){v[2], v[3]}, (bf16x2){hv[2], hv[3]}, s, false);
                    s = __builtin_amdgcn_fdot2_f32_bf16((bf16x2){v[4], v[5]}, (bf16x2){hv[4], hv[5]}, s, false);
                    s = __builtin_amdgcn_fdot2_f32_bf16((bf16x2){v[6], v[7]}, (bf16x2){hv[6], hv[7]}, s, false);
                    acc[r] = s;
                }
            }
        }
    }
    const int m = m0 + 32 * w + 16 * ts + c;
    const float svh = f16_to_f32(a.svh[2][(int64_t)e * H + m]) * (1.0f / 128.0f);
#pragma unroll
    for (int r = 0; r < kGemvMaxRows; ++r) {
        if (r < R && r < rows_cap) {
            const float tot = acc[r] + __shfl_xor(acc[r], 32, 64);
            if (h == 0) {
                const int slot = a.sorted[p0 + r];
                a.ybuf[(int64_t)slot * H + m] = tot * svh * a.w[slot];
            }
        }
    }
}

hipError_t launch_gemv_gateup(const GroupArgs &a, int max_list, int rows_cap, hipStream_t s)
{
    if (max_list <= 0)
        return hipSuccess;
    dim3 grid(max_list, a.I / 64);
    const size_t lds = sizeof(f16) * 2 * rows_cap * a.H;
    if (a.K == 2 && a.cb == 0) gemv_gateup_kernel<2, 0><<<grid, 256, lds, s>>>(a, rows_cap);
    else if (a.K == 3 && a.cb == 0) gemv_gateup_kernel<3, 0><<<grid, 256, lds, s>>>(a, rows_cap);
    else if (a.K == 4 && a.cb == 0) gemv_gateup_kernel<4, 0><<<grid, 256, lds, s>>>(a, rows_cap);
    else if (a.K == 2) gemv_gateup_kernel<2, 1><<<grid, 256, lds, s>>>(a, rows_cap);
    else if (a.K == 3) gemv_gateup_kernel<3, 1><<<grid, 256, lds, s>>>(a, rows_cap);
    else gemv_gateup_kernel<4, 1><<<grid, 256, lds, s>>>(a, rows_cap);
    return hipGetLastError();
}

hipError_t launch_gemv_down(const GroupArgs &a, int max_list, int rows_cap, hipStream_t s)
{
    if (max_list <= 0)
        return hipSuccess;
    dim3 grid(max_list, a.H / 128);
    const size_t lds = sizeof(uint16_t) * rows_cap * a.I;
    if (a.K == 2 && a.cb == 0) gemv_down_kernel<2, 0><<<grid, 256, lds, s>>>(a, rows_cap);
    else if (a.K == 3 && a.cb == 0) gemv_down_kernel<3, 0><<<grid, 256, lds, s>>>(a, rows_cap);
    else if (a.K == 4 && a.cb == 0) gemv_down_kernel<4, 0><<<grid, 256, lds, s>>>(a, rows_cap);
    else if (a.K == 2) gemv_down_kernel<2, 1><<<grid, 256, lds, s>>>(a, rows_cap);
    else if (a.K == 3) gemv_down_kernel<3, 1><<<grid, 256, lds, s>>>(a, rows_cap);
    else gemv_down_kernel<4, 1><<<grid, 256, lds, s>>>(a, rows_cap);
    return hipGetLastError();
}

// ------------------------------------------------------------ shared expert GEMV
// Dense fp16 weights in nn.Linear layout [out][in]; one wavefront streams
// whole weight rows in 16-byte chunks and reduces across lanes at the end.
constexpr int kShRows = 4;   // weight rows (gate+up pairs, or down rows) per wavefront

__global__ __launch_bounds__(256) void shared_gemv_gateup_kernel(const uint16_t *__restrict__ x16,
                                                                 int T, int H, int I,
                                                                 const uint16_t *__restrict__ wg,
                                                                 const uint16_t *__restrict__ wu,
                                                                 uint16_t *__restrict__ sh)
{
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    const int n0 = (blockIdx.x * 4 + w) * kShRows;
    if (n0 >= I)
        return;
    float acc[2][kShRows][kSharedGemvMaxTokens];
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int r = 0; r < kShRows; ++r)
#pragma unroll
            for (int t = 0; t < kSharedGemvMaxTokens; ++t)
                acc[p][r][t] = 0.0f;
    for (int k0 = 8 * l; k0 < H; k0 += 512) {
        f16x8 wv[2][kShRows];
#pragma unroll
        for (int r = 0; r < kShRows; ++r) {
            wv[0][r] = *(const f16x8 *)(wg + (int64_t)(n0 + r) * H + k0);
            wv[1][r] = *(const f16x8 *)(wu + (int64_t)(n0 + r) * H + k0);
        }
#pragma unroll
        for (int t = 0; t < kSharedGemvMaxTokens; ++t) {
            if (t < T) {
                const f16x8 xv = *(const f16x8 *)(x16 + (int64_t)t * H + k0);
#pragma unroll
                for (int p = 0; p < 2; ++p)
#pragma unroll
                    for (int r = 0; r < kShRows; ++r) {
                        float s = acc[p][r][t];
#pragma unroll
                        for (int j = 0; j < 8; j += 2)
                            s = __builtin_amdgcn_fdot2((f16x2){wv[p][r][j], wv[p][r][j + 1]},
                                                       (f16x2){xv[j], xv[j + 1]}, s, false);
                        acc[p][r][t] = s;
                    }
            }
        }
    }
#pragma unroll
    for (int t = 0; t < kSharedGemvMaxTokens; ++t) {
        if (t < T) {
#pragma unroll
            for (int r = 0; r < kShRows; ++r) {
                float g = acc[0][r][t], u = acc[1][r][t];
#pragma unroll
                for (int off = 32; off >= 1; off >>= 1) {
                    g += __shfl_xor(g, off, 64);
                    u += __shfl_xor(u, off, 64);
                }
                if (l == 0)
                    sh[(int64_t)t * I + n0 + r] = f32_to_f16_bits(silu_f(g) * u);
            }
        }
    }
}

__global__ __launch_bounds__(256) void shared_gemv_down_kernel(const uint16_t *__restrict__ sh, int T,
                                                               int H, int I,
                                                               const uint16_t *__restrict__ wd,
                                                               float *__restrict__ sy)
{
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    const int m0 = (blockIdx.x * 4 + w) * kShRows;
    if (m0 >= H)
        return;
    float acc[kShRows][kSharedGemvMaxTokens];
#pragma unroll
    for (int r = 0; r < kShRows; ++r)
#pragma unroll
        for (int t = 0; t < kSharedGemvMaxTokens; ++t)
            acc[r][t] = 0.0f;
    for (int k0 = 8 * l; k0 < I; k0 += 512) {
        f16x8 wv[kShRows];
#pragma unroll
        for (int r = 0; r < kShRows; ++r)
            wv[r] = *(const f16x8 *)(wd + (int64_t)(m0 + r) * I + k0);
#pragma unroll
        for (int t = 0; t < kSharedGemvMaxTokens; ++t) {
            if (t < T) {
                const f16x8 hv = *(const f16x8 *)(sh + (int64_t)t * I + k0);
#pragma unroll
                for (int r = 0; r < kShRows; ++r) {
                    float s = acc[r][t];
#pragma unroll
                    for (int j = 0; j < 8; j += 2)
                        s = __builtin_amdgcn_fdot2((f16x2){wv[r][j], wv[r][j + 1]},
                                                   (f16x2){hv[j], hv[j + 1]}, s, false);
                    acc[r][t] = s;
                }
            }
        }
    }
#pragma unroll
    for (int t = 0; t < kSharedGemvMaxTokens; ++t) {
        if (t < T) {
#pragma unroll
            for (int r = 0; r < kShRows; ++r) {
                float v = acc[r][t];
#pragma unroll
                for (int off = 32; off >= 1; off >>= 1)
                    v += __shfl_xor(v, off, 64);
                if (l == 0)
                    sy[(int64_t)t * H + m0 + r] = v;
            }
        }
    }
}

hipError_t launch_shared_gemv(const uint16_t *x16, int T, int H, int I, const uint16_t *wg,
                              const uint16_t *wu, const uint16_t *wd, uint16_t *sh, float *sy,
                              hipStream_t s)
{
    const int rows_per_block = 4 * kShRows;
    shared_gemv_gateup_kernel<<<(I + rows_per_block - 1) / rows_per_block, 256, 0, s>>>(x16, T, H, I, wg, wu, sh);
    shared_gemv_down_kernel<<<(H + rows_per_block - 1) / rows_per_block, 256, 0, s>>>(sh, T, H, I, wd, sy);
    return hipGetLastError();
}

}  // namespace moe
