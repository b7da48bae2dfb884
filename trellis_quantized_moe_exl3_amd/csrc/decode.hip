// Dense decode of one trellis-coded matrix (the bit-exact check of the decode
// that every GEMM kernel uses).  Same fragment decoder as the GEMM kernels.
#include "common.h"
#include "internal.h"
#include "trellis.h"

namespace moe {

enum { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2, DT_FP8 = 3 };

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
    if (DT == DT_FP8) {
        // the same fragment decoder as the fp8 MFMA path (either codebook:
        // the bytes are the E4M3 rounding of c)
        const u32x2 b8 = frag_decode_fp8<K>(D0, D1, q, m_lo, m_hi);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int64_t o = (int64_t)(16 * tk + 8 * h + t) * n_out + col;
            ((uint8_t *)dst)[o] = (uint8_t)(b8[t >> 2] >> (8 * (t & 3)));
        }
        return;
    }
    float v2[8];
    frag_decode_f32<K, CB>(D0, D1, q, m_lo, m_hi, v2);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const int64_t o = (int64_t)(16 * tk + 8 * h + t) * n_out + col;
        const float cval = v2[t] * (1.0f / 128.0f);   // c = 2v / 128, exact
        if (DT == DT_F32)
            ((float *)dst)[o] = cval;
        else if (DT == DT_F16)
            ((uint16_t *)dst)[o] = f32_to_f16_bits(cval);
        else if (DT == DT_BF16)
            ((uint16_t *)dst)[o] = f32_to_bf16_bits(cval);
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

}  // namespace moe
