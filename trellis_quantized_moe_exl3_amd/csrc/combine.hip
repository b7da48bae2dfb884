// Elementwise passes of the layer around the expert GEMMs: the bf16 -> fp16
// copy of the activations, the rotation of the trellis experts' input
// (page "GLM-5.3-Flash . exlr8 (K2/K3/K4)", "Calibration": the 128 x 128
// Hadamard matrix; "Index slices": the layer's two sign vectors) and the
// per-token combine of the routed slot rows with the shared expert's output
// (the scatter half of "down + scatter", page "GLM-5.3 Flash EXL3 for 2x DGX
// Sparks", "Cold prefill (E3 grouped MoE)").  All three are HBM-bound
// streams of 16-byte pieces.
#include "common.h"
#include "internal.h"

namespace moe {

// ---------------------------------------------------------------- small kernels
// bf16 activations -> fp16 (exact for |x| in the fp16 normal range; a finite
// value past the fp16 range is flagged in the status word).
__global__ __launch_bounds__(256) void convert_x_kernel(const uint16_t *__restrict__ x, int64_t n8,
                                                        uint16_t *__restrict__ x16, WsHeader *hdr)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n8)
        return;
    bool over = false;
    ((u32x4 *)x16)[i] = bf16x8_to_f16x8(((const u32x4 *)x)[i], over);
    if (over)
        atomicOr((unsigned *)&hdr->status, MOE_EXL3_STATUS_ACT_RANGE);
}

hipError_t launch_convert_x(const uint16_t *x, int64_t n, uint16_t *x16, WsHeader *hdr, hipStream_t s)
{
    const int64_t n8 = n / 8;
    convert_x_kernel<<<(unsigned)((n8 + 255) / 256), 256, 0, s>>>(x, n8, x16, hdr);
    return hipGetLastError();
}

// ---------------------------------------------------------------- rotation
// The experts' basis rotation (page "GLM-5.3-Flash . exlr8 (K2/K3/K4)",
// "Calibration": the 128x128 Hadamard matrix; "Index slices": the layer's two
// int8 sign vectors over the hidden size).  Sixteen lanes hold one block of
// 128 consecutive channels, eight per lane: the transform runs as three
// butterfly stages inside the lane (channel distance 1, 2, 4) and four across
// the 16 lanes (distance 8, 16, 32, 64: lane l pairs with l ^ m), each
// (a, b) -> (a + b, a - b) with a the lower channel, in fp32; the result is
// scaled by 1 / sqrt(128).  The Sylvester matrix is symmetric, so the same
// transform serves both sides.
MOE_DEV void fwht128(float v[8], int lane16)
{
#pragma unroll
    for (int d = 1; d < 8; d <<= 1)
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (!(i & d)) {
                const float a = v[i], b = v[i + d];
                v[i] = a + b;
                v[i + d] = a - b;
            }
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) {
        const bool hi = lane16 & m;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float p = __shfl_xor(v[i], m, 64);
            v[i] = hi ? p - v[i] : v[i] + p;
        }
    }
    constexpr float kScale = 0.08838834764831845f;   // 1 / sqrt(128)
#pragma unroll
    for (int i = 0; i < 8; ++i)
        v[i] *= kScale;
}

// xr[t] = fp16(R(s0 * x[t])): the rotated copy of the activations the trellis
// experts read.  One thread per 8 channels; 16 consecutive threads = one
// 128-channel block of one token (hidden is a multiple of 256, so no block
// straddles a token and every wavefront holds whole blocks).
template <bool BF16>
__global__ __launch_bounds__(256) void rotate_x_kernel(const uint16_t *__restrict__ x, int64_t n8, int H,
                                                       const int8_t *__restrict__ s0, uint16_t *__restrict__ xr,
                                                       WsHeader *hdr)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n8)   // n8 is a multiple of 16: whole 16-lane groups leave
        return;
    const int m = (int)((8 * i) % H);
    const u32x4 raw = ((const u32x4 *)x)[i];
    const uint2 sg = *(const uint2 *)(s0 + m);
    float v[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        v[2 * j] = act_to_f32<BF16>((uint16_t)(raw[j] & 0xFFFFu));
        v[2 * j + 1] = act_to_f32<BF16>((uint16_t)(raw[j] >> 16));
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int8_t sj = (int8_t)(((j < 4 ? sg.x : sg.y) >> (8 * (j & 3))) & 0xFF);
        v[j] = sj < 0 ? -v[j] : v[j];
    }
    fwht128(v, (int)(i & 15));
    u32x4 o;
    bool over = false;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t a = f32_to_f16_bits(v[2 * j]), b = f32_to_f16_bits(v[2 * j + 1]);
        over |= (a & 0x7FFFu) == 0x7C00u || (b & 0x7FFFu) == 0x7C00u;
        o[j] = a | (b << 16);
    }
    ((u32x4 *)xr)[i] = o;
    if (over)
        atomicOr((unsigned *)&hdr->status, MOE_EXL3_STATUS_ACT_RANGE);
}

hipError_t launch_rotate_x(const uint16_t *x, bool bf16, int64_t T, int H, const int8_t *s0, uint16_t *xr,
                           WsHeader *hdr, hipStream_t s)
{
    const int64_t n8 = T * H / 8;
    const unsigned grid = (unsigned)((n8 + 255) / 256);
    if (bf16)
        rotate_x_kernel<true><<<grid, 256, 0, s>>>(x, n8, H, s0, xr, hdr);
    else
        rotate_x_kernel<false><<<grid, 256, 0, s>>>(x, n8, H, s0, xr, hdr);
    return hipGetLastError();
}

// ---------------------------------------------------------------- combine
// out[t] = shared[t] + s1 * R(sum_j ybuf[t*k + j] (+ ybuf[T*k + t]))
// ybuf holds bf16 slot rows (routing weight applied); the routed rows of a
// token, then the trellis shared expert's row when there is one (slot T*k + t,
// weight 1), are summed in fp32 in that fixed order: deterministic.  With
// sign vectors the sum is rotated back (R, then s1) before the fp16 shared
// expert's fp32 row is added; then the cast to the activation dtype.  8
// outputs per thread (16 threads per 128-channel block when rotating).  Slot
// rows and shared rows are read once, with nontemporal loads: the 7168-token
// layer's combine went 0.121 -> 0.098 ms with them (the rate of a plain
// streaming read).
template <bool BF16, bool ROT>
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t *__restrict__ ybuf,
                                                      const float *__restrict__ sy, int64_t T, int H,
                                                      int k, int extra, const int8_t *__restrict__ s1,
                                                      uint16_t *__restrict__ out)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t n8 = T * H / 8;
    if (i >= n8)
        return;
    const int64_t t = (8 * i) / H, m = (8 * i) % H;
    float s[8];
#pragma unroll
    for (int q = 0; q < 8; ++q)
        s[q] = 0.0f;
    // all slot rows are loaded before the first add (k + 1 <= 17), then
    // summed in slot order
    constexpr int kMaxK = 17;
    u32x4 v[kMaxK];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
        if (j < k)
            v[j] = __builtin_nontemporal_load((const u32x4 *)(ybuf + (t * k + j) * H + m));
        else if (j == k && extra)
            v[j] = __builtin_nontemporal_load((const u32x4 *)(ybuf + (T * k + t) * H + m));
    }
#pragma unroll
    for (int j = 0; j < kMaxK; ++j)
        if (j < k + extra) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                s[2 * q] += __uint_as_float(v[j][q] << 16);
                s[2 * q + 1] += __uint_as_float(v[j][q] & 0xFFFF0000u);
            }
        }
    if constexpr (ROT) {
        fwht128(s, (int)(i & 15));
        const uint2 sg = *(const uint2 *)(s1 + m);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int8_t sj = (int8_t)(((j < 4 ? sg.x : sg.y) >> (8 * (j & 3))) & 0xFF);
            s[j] = sj < 0 ? -s[j] : s[j];
        }
    }
    if (sy) {
        const f32x4 a = __builtin_nontemporal_load((const f32x4 *)(sy + t * H + m)),
                    b = __builtin_nontemporal_load((const f32x4 *)(sy + t * H + m + 4));
        s[0] += a[0]; s[1] += a[1]; s[2] += a[2]; s[3] += a[3];
        s[4] += b[0]; s[5] += b[1]; s[6] += b[2]; s[7] += b[3];
    }
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        if (BF16)
            o[q] = (uint32_t)f32_to_bf16_bits(s[2 * q]) | ((uint32_t)f32_to_bf16_bits(s[2 * q + 1]) << 16);
        else
            o[q] = (uint32_t)f32_to_f16_bits(s[2 * q]) | ((uint32_t)f32_to_f16_bits(s[2 * q + 1]) << 16);
    }
    *(u32x4 *)(out + t * H + m) = o;
}

hipError_t launch_combine(const uint16_t *ybuf, const float *sy, int64_t T, int H, int k, bool extra,
                          const int8_t *s1, bool bf16, uint16_t *out, hipStream_t s)
{
    const int64_t n8 = T * H / 8;
    const unsigned grid = (unsigned)((n8 + 255) / 256);
    const int ex = extra ? 1 : 0;
    if (bf16) {
        if (s1) combine_kernel<true, true><<<grid, 256, 0, s>>>(ybuf, sy, T, H, k, ex, s1, out);
        else combine_kernel<true, false><<<grid, 256, 0, s>>>(ybuf, sy, T, H, k, ex, s1, out);
    } else {
        if (s1) combine_kernel<false, true><<<grid, 256, 0, s>>>(ybuf, sy, T, H, k, ex, s1, out);
        else combine_kernel<false, false><<<grid, 256, 0, s>>>(ybuf, sy, T, H, k, ex, s1, out);
    }
    return hipGetLastError();
}

}  // namespace moe
