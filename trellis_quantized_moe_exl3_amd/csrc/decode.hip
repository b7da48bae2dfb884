// Dense decode of one trellis-coded matrix, for the bit-exact check of the
// decode (page "GLM-5.3-Flash EXL3 (~2.1 bpw, SM70 tile order)", header:
// packed 16-bit words holding 16/K weights each).  Every output mode runs the
// very fragment decoder of one kernel of the layer, so checking a mode checks
// the values that kernel feeds to its arithmetic:
//   F16       frag_decode_f16  (the gate/up MFMA B operand, 2v in fp16)
//   BF16      frag_decode_bf16 (the down MFMA B operand, 2v in bf16)
//   FP8       frag_decode_fp8  (the fp8 MFMA B operand, E4M3 bytes of c)
//   GEMV_F16  frag_biased_pairs (the decode-fused GEMV's MFMA operand,
//             fp16 2v + 1532, stored as is)
//   MFMA_BIASED_F16  frag_decode_f16_biased (the gate/up MFMA operand on
//             one-block tiles, mcg codebook: fp16 2v + 1532, stored as is)
//   F32       frag_decode_f32  (2v in fp32)
// The 16-bit and fp32 modes store c = 2v / 128; the division is by a power
// of two and exact in every one of these types.
#include "common.h"
#include "internal.h"
#include "trellis.h"

namespace moe {

enum { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2, DT_FP8 = 3, DT_GEMV_F16 = 4, DT_MFMA_BIASED_F16 = 5 };

// 256 threads = 8 tiles; thread -> (tile, column c, k-half h).
template <int K, int CB, int DT>
__global__ __launch_bounds__(256) void decode_kernel(const uint32_t *__restrict__ codes, int n_in,
                                                     int n_out, uint32_t m_lo, uint32_t m_hi,
                                                     void *__restrict__ dst)
{
    const int ntn = n_out / 16;
    const int64_t ntiles = (int64_t)(n_in / 16) * ntn;
    const int64_t ti = (int64_t)blockIdx.x * 8 + (threadIdx.x >> 5);
    if (ti >= ntiles)
        return;
    const int f = threadIdx.x & 31, c = f & 15, h = f >> 4;
    const int tk = (int)(ti / ntn), tn = (int)(ti % ntn);
    int d0, d1, q;
    frag_pos<K>(c, h, d0, d1, q);
    const uint32_t *tile = codes + ti * Tile<K>::kDwords;
    const uint32_t D0 = tile[d0], D1 = tile[d1];
    const int col = 16 * tn + c;
    auto at = [&](int t) { return (int64_t)(16 * tk + 8 * h + t) * n_out + col; };
    if constexpr (DT == DT_FP8) {
        // either codebook: the bytes are the E4M3 rounding of c
        const u32x2 b8 = frag_decode_fp8<K>(D0, D1, q, m_lo, m_hi);
#pragma unroll
        for (int t = 0; t < 8; ++t)
            ((uint8_t *)dst)[at(t)] = (uint8_t)(b8[t >> 2] >> (8 * (t & 3)));
    } else if constexpr (DT == DT_F16) {
        const f16x8 v = frag_decode_f16<K, CB>(D0, D1, q, m_lo, m_hi);
#pragma unroll
        for (int t = 0; t < 8; ++t)
            ((f16 *)dst)[at(t)] = v[t] * (f16)(1.0f / 128.0f);
    } else if constexpr (DT == DT_BF16) {
        const bf16x8 v = frag_decode_bf16<K, CB>(D0, D1, q, m_lo, m_hi);
#pragma unroll
        for (int t = 0; t < 8; ++t)
            ((uint16_t *)dst)[at(t)] = f32_to_bf16_bits((float)v[t] * (1.0f / 128.0f));
    } else if constexpr (DT == DT_GEMV_F16) {
        f16x2 wp[4];
        frag_biased_pairs<K, CB>(D0, D1, q, m_lo, m_hi, wp);
#pragma unroll
        for (int t = 0; t < 8; ++t)
            ((f16 *)dst)[at(t)] = wp[t / 2][t & 1];
    } else if constexpr (DT == DT_MFMA_BIASED_F16) {
        const f16x8 v = frag_decode_f16_biased<K>(D0, D1, q, m_lo, m_hi);
#pragma unroll
        for (int t = 0; t < 8; ++t)
            ((f16 *)dst)[at(t)] = v[t];
    } else {
        float v2[8];
        frag_decode_f32<K, CB>(D0, D1, q, m_lo, m_hi, v2);
#pragma unroll
        for (int t = 0; t < 8; ++t)
            ((float *)dst)[at(t)] = v2[t] * (1.0f / 128.0f);
    }
}

template <int K, int CB>
static hipError_t decode_dt(const uint16_t *codes, int n_in, int n_out, uint32_t mcg, void *dst,
                            int dt, hipStream_t s)
{
    const int64_t ntiles = (int64_t)(n_in / 16) * (n_out / 16);
    const unsigned grid = (unsigned)((ntiles + 7) / 8);
    const uint32_t *c32 = (const uint32_t *)codes;
    const uint32_t lo = mcg & 0xFFFFu, hi = mcg >> 16;
    switch (dt) {
    case DT_F32: decode_kernel<K, CB, DT_F32><<<grid, 256, 0, s>>>(c32, n_in, n_out, lo, hi, dst); break;
    case DT_F16: decode_kernel<K, CB, DT_F16><<<grid, 256, 0, s>>>(c32, n_in, n_out, lo, hi, dst); break;
    case DT_BF16: decode_kernel<K, CB, DT_BF16><<<grid, 256, 0, s>>>(c32, n_in, n_out, lo, hi, dst); break;
    case DT_GEMV_F16: decode_kernel<K, CB, DT_GEMV_F16><<<grid, 256, 0, s>>>(c32, n_in, n_out, lo, hi, dst); break;
    case DT_MFMA_BIASED_F16:
        decode_kernel<K, CB, DT_MFMA_BIASED_F16><<<grid, 256, 0, s>>>(c32, n_in, n_out, lo, hi, dst);
        break;
    default: decode_kernel<K, CB, DT_FP8><<<grid, 256, 0, s>>>(c32, n_in, n_out, lo, hi, dst); break;
    }
    return hipGetLastError();
}

hipError_t launch_decode(const uint16_t *codes, int n_in, int n_out, int K, uint32_t mcg, int cb,
                         void *dst, int dst_dtype, hipStream_t s)
{
    if (K == 2)
        return cb ? decode_dt<2, CB_MCG_E4M3>(codes, n_in, n_out, mcg, dst, dst_dtype, s)
                  : decode_dt<2, CB_MCG>(codes, n_in, n_out, mcg, dst, dst_dtype, s);
    if (K == 3)
        return cb ? decode_dt<3, CB_MCG_E4M3>(codes, n_in, n_out, mcg, dst, dst_dtype, s)
                  : decode_dt<3, CB_MCG>(codes, n_in, n_out, mcg, dst, dst_dtype, s);
    return cb ? decode_dt<4, CB_MCG_E4M3>(codes, n_in, n_out, mcg, dst, dst_dtype, s)
              : decode_dt<4, CB_MCG>(codes, n_in, n_out, mcg, dst, dst_dtype, s);
}

// ---------------------------------------------------------------- load-time layout
// Tile-grid reorder (page "GLM-5.3-Flash EXL3 (~2.1 bpw, SM70 tile order)",
// header: the checkpoint's column-major tile order is reordered by the loader
// into the kernels' layout; page "GLM-5.3-Flash . exlr8 (K2/K3/K4)",
// "Loading": projections stored in halves of 128 intermediate channels).
// A tile is a self-contained 32K-byte trellis stream, so reordering whole
// tiles is a byte copy: dst holds tile (tk, tn) at tk * (n_out/16) + tn.
// One thread moves 16 bytes; 2K threads one tile.
__device__ int64_t src_tile(int order, int ntk, int ntn, int tk, int tn)
{
    if (order == 1)
        return (int64_t)tn * ntk + tk;
    if (order == 2)
        return (int64_t)(tn / 8) * ntk * 8 + (int64_t)tk * 8 + tn % 8;
    return (int64_t)tk * ntn + tn;
}

__global__ __launch_bounds__(256) void repack_kernel(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst,
                                                     int64_t n16, int ntk, int ntn, int per_tile, int order)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n16)
        return;
    const int64_t grid = (int64_t)ntk * ntn;
    const int64_t tensor = i / (grid * per_tile);
    const int64_t r = i % (grid * per_tile);
    const int64_t dt = r / per_tile;
    const int piece = (int)(r % per_tile);
    const int tk = (int)(dt / ntn), tn = (int)(dt % ntn);
    dst[i] = src[(tensor * grid + src_tile(order, ntk, ntn, tk, tn)) * per_tile + piece];
}

hipError_t launch_repack(const uint16_t *src, uint16_t *dst, int count, int n_in, int n_out, int K, int order,
                         hipStream_t s)
{
    const int per_tile = 2 * K;   // 16-byte pieces in a 32K-byte tile
    const int64_t n16 = (int64_t)count * (n_in / 16) * (n_out / 16) * per_tile;
    repack_kernel<<<(unsigned)((n16 + 255) / 256), 256, 0, s>>>((const u32x4 *)src, (u32x4 *)dst, n16, n_in / 16,
                                                                 n_out / 16, per_tile, order);
    return hipGetLastError();
}

// Block scales -> per-channel side vectors (page "GLM-5.3-Flash . exlr8
// (K2/K3/K4)", "Index slices": an F16 block table [EA][3][H/128] per layer,
// one scale per 128 hidden channels of each projection).  The hidden channels
// are the input of gate and up and the output of down: suh_g[e][k] =
// block[e][0][k/128], suh_u[e][k] = block[e][1][k/128], svh_d[e][m] =
// block[e][2][m/128]; the intermediate side (svh_g, svh_u, suh_d) is 1.
// One thread per channel of one expert.
__global__ __launch_bounds__(256) void expand_scales_kernel(const uint16_t *__restrict__ block, int EA, int H, int I,
                                                            uint16_t *__restrict__ sg, uint16_t *__restrict__ su,
                                                            uint16_t *__restrict__ sd, uint16_t *__restrict__ vg,
                                                            uint16_t *__restrict__ vu, uint16_t *__restrict__ vd)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t nh = (int64_t)EA * H, ni = (int64_t)EA * I;
    const uint16_t one = 0x3C00;   // fp16 1.0
    if (i < nh) {
        const int64_t e = i / H;
        const int k = (int)(i % H), nb = H / 128;
        sg[i] = block[(e * 3 + 0) * nb + k / 128];
        su[i] = block[(e * 3 + 1) * nb + k / 128];
        vd[i] = block[(e * 3 + 2) * nb + k / 128];
    }
    if (i < ni) {
        vg[i] = one;
        vu[i] = one;
        sd[i] = one;
    }
}

hipError_t launch_expand_scales(const uint16_t *block, int EA, int H, int I, uint16_t *const suh[3],
                                uint16_t *const svh[3], hipStream_t s)
{
    const int64_t n = (int64_t)EA * (H > I ? H : I);
    expand_scales_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(block, EA, H, I, suh[0], suh[1], suh[2], svh[0],
                                                                     svh[1], svh[2]);
    return hipGetLastError();
}

}  // namespace moe
