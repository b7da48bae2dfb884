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

constexpr int kGemvU = 8;      // tile rows per prefetch group
constexpr int kGemvPass = 2;   // routed rows per pass over the codes

// 1532 * (row sum), the re-centring of the biased decoded values.
constexpr float kBias2 = 1532.0f;

// Deterministic block sum (256 threads) of one float per thread.
MOE_DEV float block_sum256(float v, float *part)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        v += __shfl_xor(v, off, 64);
    __syncthreads();
    if ((threadIdx.x & 63) == 0)
        part[threadIdx.x >> 6] = v;
    __syncthreads();
    return ((part[0] + part[1]) + part[2]) + part[3];
}

// Each lane decodes a fragment of tile rows and accumulates x * (2v + 1532)
// into acc[r] with one v_fma_mix_f32 per weight and row (fp16 operands, exact
// products, fp32 accumulation).  Code words are prefetched kGemvU tile rows
// ahead.  XS(r, kk) returns the 8 activation values of row r at input rows
// kk + 8h .. kk + 8h + 7 for the lane.
template <int K, int CB, int NR, class XS>
MOE_DEV void gemv_stream(const uint32_t *cb, int64_t rstride, int ntk, int d0, int d1, int q,
                         uint32_t m_lo, uint32_t m_hi, int nr, XS xs, float acc[NR])
{
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
            uint32_t st[8];
            frag_states<K>(cu[u][0], cu[u][1], q, st);
            f16 wv[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                if (CB == CB_MCG) {
                    wv[t] = __builtin_bit_cast(f16, (uint16_t)value2_biased_f16bits(st[t], m_lo, m_hi));
                } else {
                    wv[t] = (f16)(e4m3_value2(value2_f32(st[t], m_lo, m_hi)) + kBias2);
                }
            }
            const int kk = 16 * (g + u);
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                if (r < nr) {
                    float xv[8];
                    xs(r, kk, xv);
                    float s = acc[r];
#pragma unroll
                    for (int t = 0; t < 8; ++t)
                        s = __builtin_fmaf((float)wv[t], xv[t], s);
                    acc[r] = s;
                }
            }
        }
    }
}

// gate/up + SwiGLU.  Block = 4 wavefronts = (gate, up) x 2 tile pairs = 64
// output columns of one expert; grid.x walks the GEMV expert list.  Rows are
// processed kGemvPass at a time (x * suh of the pass in LDS, fp16).
template <int K, int CB>
__global__ __launch_bounds__(256) void gemv_gateup_kernel(GroupArgs a)
{
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ float part[4];
    __shared__ float rsum[2][kGemvPass];
    __shared__ float gu[2][kGemvPass][64];
    const int li = blockIdx.x;
    if (li >= a.hdr->n_gemv)
        return;
    const int H = a.H, I = a.I;
    const int e = a.glist[li];
    const int R = a.counts[e];
    const int p0 = a.offsets[e];
    const int n0 = blockIdx.y * 64;
    f16 *xs = (f16 *)smem;   // [2][kGemvPass][H]

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
    const int col = 16 * (2 * tp + ts) + c;
    const float svh = f16_to_f32(a.svh[pr][(int64_t)e * I + n0 + col]) * (1.0f / 128.0f);

    for (int r0 = 0; r0 < R; r0 += kGemvPass) {
        const int nr = min(kGemvPass, R - r0);
        // x * suh of the pass's rows for both projections, and their sums
        for (int pp = 0; pp < 2; ++pp)
            for (int r = 0; r < nr; ++r) {
                const int t = a.sorted[p0 + r0 + r] / a.k;
                float sum = 0.0f;
                for (int ch = threadIdx.x; ch < H / 8; ch += 256) {
                    const f16x8 xv = *(const f16x8 *)(a.x16 + (int64_t)t * H + 8 * ch);
                    const f16x8 sv = *(const f16x8 *)(a.suh[pp] + (int64_t)e * H + 8 * ch);
                    const f16x8 pv = xv * sv;
                    *(f16x8 *)(xs + ((size_t)pp * kGemvPass + r) * H + 8 * ch) = pv;
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        sum += (float)pv[j];
                }
                const float tot = block_sum256(sum, part);
                if (threadIdx.x == 0)
                    rsum[pp][r] = tot;
            }
        __syncthreads();

        float acc[kGemvPass] = {};
        const f16 *xsp = xs + (size_t)pr * kGemvPass * H + 8 * h;
        gemv_stream<K, CB, kGemvPass>(cb, rstride, H / 16, d0, d1, q, m_lo, m_hi, nr,
                                      [&](int r, int kk, float xv[8]) {
                                          const f16x8 v = *(const f16x8 *)(xsp + (size_t)r * H + kk);
#pragma unroll
                                          for (int t = 0; t < 8; ++t)
                                              xv[t] = (float)v[t];
                                      },
                                      acc);
        // the two k-halves of a column sit in lanes l and l ^ 32
#pragma unroll
        for (int r = 0; r < kGemvPass; ++r) {
            const float tot = acc[r] + __shfl_xor(acc[r], 32, 64);
            if (r < nr && h == 0)
                gu[pr][r][col] = (tot - kBias2 * rsum[pr][r]) * svh;
        }
        __syncthreads();
        if (threadIdx.x < nr * 64) {
            const int r = threadIdx.x >> 6, cc = threadIdx.x & 63;
            const float g = gu[0][r][cc], u = gu[1][r][cc];
            const float hv = silu_f(g) * u * f16_to_f32(a.suh[2][(int64_t)e * I + n0 + cc]);
            a.hbuf[(int64_t)(p0 + r0 + r) * I + n0 + cc] = f32_to_bf16_bits(hv);
        }
        __syncthreads();
    }
}

// down + routing-weighted scatter.  Block = 4 wavefronts x 2 tiles = 128
// output columns of one expert.  h * suh_down rows of the pass in LDS, fp32.
template <int K, int CB>
__global__ __launch_bounds__(256) void gemv_down_kernel(GroupArgs a)
{
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ float part[4];
    __shared__ float rsum[kGemvPass];
    const int li = blockIdx.x;
    if (li >= a.hdr->n_gemv)
        return;
    const int H = a.H, I = a.I;
    const int e = a.glist[li];
    const int R = a.counts[e];
    const int p0 = a.offsets[e];
    const int m0 = blockIdx.y * 128;
    float *hs = (float *)smem;   // [kGemvPass][I]

    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    const int c = l & 15, ts = (l >> 4) & 1, h = l >> 5;
    const int tn = m0 / 16 + 2 * w + ts;
    int d0, d1, q;
    frag_pos<K>(c, h, d0, d1, q);
    const int64_t per_expert = (int64_t)(I / 16) * (H / 16) * Tile<K>::kDwords;
    const uint32_t *cb = (const uint32_t *)a.codes[2] + e * per_expert + (int64_t)tn * Tile<K>::kDwords;
    const int64_t rstride = (int64_t)(H / 16) * Tile<K>::kDwords;
    const uint32_t m_lo = a.mcg & 0xFFFFu, m_hi = a.mcg >> 16;
    const int m = m0 + 32 * w + 16 * ts + c;
    const float svh = f16_to_f32(a.svh[2][(int64_t)e * H + m]) * (1.0f / 128.0f);

    for (int r0 = 0; r0 < R; r0 += kGemvPass) {
        const int nr = min(kGemvPass, R - r0);
        for (int r = 0; r < nr; ++r) {
            float sum = 0.0f;
            for (int ch = threadIdx.x; ch < I / 8; ch += 256) {
                const u32x4 raw = *(const u32x4 *)(a.hbuf + (int64_t)(p0 + r0 + r) * I + 8 * ch);
                f32x4 lo, hi;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float v0 = __uint_as_float(raw[j] << 16), v1 = __uint_as_float(raw[j] & 0xFFFF0000u);
                    sum += v0 + v1;
                    if (j < 2) {
                        lo[2 * j] = v0;
                        lo[2 * j + 1] = v1;
                    } else {
                        hi[2 * j - 4] = v0;
                        hi[2 * j - 3] = v1;
                    }
                }
                *(f32x4 *)(hs + (size_t)r * I + 8 * ch) = lo;
                *(f32x4 *)(hs + (size_t)r * I + 8 * ch + 4) = hi;
            }
            const float tot = block_sum256(sum, part);
            if (threadIdx.x == 0)
                rsum[r] = tot;
        }
        __syncthreads();

        float acc[kGemvPass] = {};
        const float *hsp = hs + 8 * h;
        gemv_stream<K, CB, kGemvPass>(cb, rstride, I / 16, d0, d1, q, m_lo, m_hi, nr,
                                      [&](int r, int kk, float xv[8]) {
                                          const f32x4 v0 = *(const f32x4 *)(hsp + (size_t)r * I + kk);
                                          const f32x4 v1 = *(const f32x4 *)(hsp + (size_t)r * I + kk + 4);
#pragma unroll
                                          for (int t = 0; t < 4; ++t) {
                                              xv[t] = v0[t];
                                              xv[t + 4] = v1[t];
                                          }
                                      },
                                      acc);
#pragma unroll
        for (int r = 0; r < kGemvPass; ++r) {
            const float tot = acc[r] + __shfl_xor(acc[r], 32, 64);
            if (r < nr && h == 0) {
                const int slot = a.sorted[p0 + r0 + r];
                a.ybuf[(int64_t)slot * H + m] = f32_to_bf16_bits((tot - kBias2 * rsum[r]) * svh * a.w[slot]);
            }
        }
        __syncthreads();
    }
}

hipError_t launch_gemv_gateup(const GroupArgs &a, int max_list, hipStream_t s)
{
    if (max_list <= 0)
        return hipSuccess;
    dim3 grid(max_list, a.I / 64);
    const size_t lds = sizeof(f16) * 2 * kGemvPass * a.H;
    if (a.K == 2 && a.cb == 0) gemv_gateup_kernel<2, 0><<<grid, 256, lds, s>>>(a);
    else if (a.K == 3 && a.cb == 0) gemv_gateup_kernel<3, 0><<<grid, 256, lds, s>>>(a);
    else if (a.K == 4 && a.cb == 0) gemv_gateup_kernel<4, 0><<<grid, 256, lds, s>>>(a);
    else if (a.K == 2) gemv_gateup_kernel<2, 1><<<grid, 256, lds, s>>>(a);
    else if (a.K == 3) gemv_gateup_kernel<3, 1><<<grid, 256, lds, s>>>(a);
    else gemv_gateup_kernel<4, 1><<<grid, 256, lds, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_gemv_down(const GroupArgs &a, int max_list, hipStream_t s)
{
    if (max_list <= 0)
        return hipSuccess;
    dim3 grid(max_list, a.H / 128);
    const size_t lds = sizeof(float) * kGemvPass * a.I;
    if (a.K == 2 && a.cb == 0) gemv_down_kernel<2, 0><<<grid, 256, lds, s>>>(a);
    else if (a.K == 3 && a.cb == 0) gemv_down_kernel<3, 0><<<grid, 256, lds, s>>>(a);
    else if (a.K == 4 && a.cb == 0) gemv_down_kernel<4, 0><<<grid, 256, lds, s>>>(a);
    else if (a.K == 2) gemv_down_kernel<2, 1><<<grid, 256, lds, s>>>(a);
    else if (a.K == 3) gemv_down_kernel<3, 1><<<grid, 256, lds, s>>>(a);
    else gemv_down_kernel<4, 1><<<grid, 256, lds, s>>>(a);
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
