// Trellis decode on gfx950: K-bit tail-biting streams in 16x16 tiles, mcg
// codebook (optionally E4M3-rounded).
//
// Storage (page "GLM-5.3-Flash EXL3 (~2.1 bpw, SM70 tile order)", header:
// packed 16-bit words holding 16/K weights each; page "GLM-5.3-Flash EXL3 K2",
// "What is in the shards": per-tensor `trellis`, `suh`, `svh`, int32 `mcg`):
//   * a tile is 16*K little-endian 16-bit words = 8*K dwords = 256*K bits;
//   * the stream reads word 0 first, most significant bit first;
//   * state j (0..255) is the 16-bit window starting at stream bit j*K, read
//     circularly inside the tile (tail-biting);
//   * state j holds the weight at input row j % 16, output column j / 16 of
//     the tile, so eight consecutive states are eight consecutive input rows of
//     one output column: exactly the eight k-values one lane feeds to an MFMA
//     operand or to a dot product;
//   * value map: h = (mcg * s) mod 2^32, v = sum_{i<4} ((h >> (8i+1)) & 127) - 254,
//     weight c = v / 64 (E4M3 variant: c rounded to FP8 E4M3, nearest-even;
//     page "GLM-5.3-Flash . exlr8 (K2/K3/K4)", opening paragraph).
//
// A lane "fragment" is (tile column c in 0..15, k-half h in 0..1): states
// j = 16c + 8h + t for t = 0..7.  Its 7K+16 window bits start at bit K*(16c+8h)
// and always fit in two consecutive dwords of the tile (the second one wraps to
// dword 0 at the end of the tile).
//
// Instruction budget per weight (gfx950): one bit-field extract for the
// window (plus a byte permute per fragment), one 32-bit multiply for the
// hash, one AND and one SAD for the four-field sum (the SAD of the second
// state of a pair writes the high half, so packing is free), then half an op
// to re-centre two fp16 values.
#pragma once

#include "common.h"

namespace moe {

template <int K>
struct Tile {
    static constexpr int kDwords = 8 * K;
    static constexpr int kBytes = 32 * K;
};

// First/second dword of a lane fragment and the bit offset inside the first.
template <int K>
MOE_DEV void frag_pos(int c, int h, int &d0, int &d1, int &q)
{
    const int b0 = K * (16 * c + 8 * h);
    d0 = b0 >> 5;
    q = b0 & 31;
    d1 = (d0 + 1 == Tile<K>::kDwords) ? 0 : d0 + 1;
}

// v_perm_b32 selector (src0 = D0, src1 = D1) that assembles the 32 stream
// bits starting at stream byte b (0..4) of the dword pair, first stream bit
// most significant.  Stream byte j of the pair (word 0 first, high byte
// first) is v_perm byte 5, 4, 7, 6, 1, 0, 3, 2.
MOE_DEV uint32_t frag_sel(int b)
{
    return __builtin_bswap32((uint32_t)(0x0203000106070405ull >> (8 * b)));
}

// The eight 16-bit states of a fragment from its two raw dwords, each in the
// low 16 bits of st[t] with the upper bits clear.  A fragment starts at a
// multiple of 8 stream bits (K * 8 * (2c + h)), so one byte permute yields
// the 32 bits from its first state on and one bit-field extract per state
// picks a window; states past bit 16 come from a second permute that starts
// one (K = 3) or two (K = 4) bytes further.  The selectors depend on q only.
template <int K>
MOE_DEV void frag_states(uint32_t D0, uint32_t D1, int q, uint32_t st[8])
{
    constexpr int kC = K == 4 ? 2 : 1;   // byte offset of the second permute
    const int b = q >> 3;
    const uint32_t A = __builtin_amdgcn_perm(D0, D1, frag_sel(b));
    const uint32_t C = K == 2 ? 0u : __builtin_amdgcn_perm(D0, D1, frag_sel(b + kC));
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const int o = K * t;   // window start relative to the fragment
        st[t] = o <= 16 ? __builtin_amdgcn_ubfe(A, 16 - o, 16) : __builtin_amdgcn_ubfe(C, 16 + 8 * kC - o, 16);
    }
}

// frag_states at a run-time width kw (2, 3 or 4, wave-uniform), for kernels
// whose width comes from a per-tensor table.  States 0..4 start at most 16
// bits into the fragment (K * t <= 16) and come from the first permute for
// every width; states 5..7 come from the second permute (one or two bytes
// further) where K * t > 16, which costs one select each.
MOE_DEV void frag_states_rt(uint32_t D0, uint32_t D1, int q, int kw, uint32_t st[8])
{
    const int kC = kw == 4 ? 2 : 1;
    const int b = q >> 3;
    const uint32_t A = __builtin_amdgcn_perm(D0, D1, frag_sel(b));
    const uint32_t C = __builtin_amdgcn_perm(D0, D1, frag_sel(b + kC));
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const int o = kw * t;
        if (t < 5)
            st[t] = __builtin_amdgcn_ubfe(A, 16 - o, 16);
        else
            st[t] = o <= 16 ? __builtin_amdgcn_ubfe(A, 16 - o, 16) : __builtin_amdgcn_ubfe(C, 16 + 8 * kC - o, 16);
    }
}

// frag_states<K> for K > 0, frag_states_rt(kw) for K = 0.
template <int K>
MOE_DEV void frag_states_k(uint32_t D0, uint32_t D1, int q, int kw, uint32_t st[8])
{
    if constexpr (K > 0)
        frag_states<K>(D0, D1, q, st);
    else
        frag_states_rt(D0, D1, q, kw, st);
}

// (mcg * s) mod 2^32 for a 16-bit state s (upper bits clear): one
// v_mul_lo_u32 (measured at 5.4-6.4 cycles per wavefront instruction on
// gfx950, against about 4 for a plain VALU operation).
MOE_DEV uint32_t mcg_hash(uint32_t s, uint32_t m_lo, uint32_t m_hi)
{
    return s * (m_lo | (m_hi << 16));
}

// base + 2 * sum of the four 7-bit fields (bits 1..7 of every byte of h).
MOE_DEV uint32_t field_sum2(uint32_t h, uint32_t base)
{
    return __builtin_amdgcn_sad_u8(h & 0xFEFEFEFEu, 0u, base);
}

// 2v as an exact fp32 value.
MOE_DEV float value2_f32(uint32_t s, uint32_t m_lo, uint32_t m_hi)
{
    // bits 0x4B000000 + n are the float 2^23 + n (n < 2^23)
    const float r = __uint_as_float(field_sum2(mcg_hash(s, m_lo, m_hi), 0x4B000000u));
    return r - 8389116.0f;   // 2^23 + 508
}

// E4M3 rounding of c = 2v / 128, returned as 128 * c8 (exact in fp32).
MOE_DEV float e4m3_value2(float v2)
{
    const uint32_t b = __builtin_amdgcn_cvt_pk_fp8_f32(v2 * (1.0f / 128.0f), 0.0f, 0, false);
    return __builtin_amdgcn_cvt_f32_fp8(b, 0) * 128.0f;
}

enum { CB_MCG = 0, CB_MCG_E4M3 = 1 };

typedef short s16x2 __attribute__((ext_vector_type(2)));

// Two states -> the fp16 pair (2v0 + 1532, 2v1 + 1532), exact: bits 0x6400 + n
// are the half 1024 + n (n < 1024); the low half gets 0x6400 + 2 (field sum
// of s0) from v_sad_u8, the high half 0x6400 + 2 (field sum of s1) from
// v_sad_hi_u8, which adds its sum shifted left by 16 (no carry: 0x6400 + 508
// < 2^16).
MOE_DEV uint32_t value2_pair_biased(uint32_t s0, uint32_t s1, uint32_t m_lo, uint32_t m_hi)
{
    const uint32_t ra = field_sum2(mcg_hash(s0, m_lo, m_hi), 0x64006400u);
    return __builtin_amdgcn_sad_hi_u8(mcg_hash(s1, m_lo, m_hi) & 0xFEFEFEFEu, 0u, ra);
}

// The fp16 pair (2v0, 2v1), exact.
MOE_DEV f16x2 value2_pair_f16(uint32_t s0, uint32_t s1, uint32_t m_lo, uint32_t m_hi)
{
    return __builtin_bit_cast(f16x2, value2_pair_biased(s0, s1, m_lo, m_hi)) - (f16x2){(f16)1532.0f, (f16)1532.0f};
}

// E4M3 rounding of a pair c = 2v / 128: both values to FP8 E4M3 (nearest
// even; |c| < 4, far from saturation) with one scaled convert, which divides
// by 128, and back with one that multiplies by 128: the fp16 pair
// 128 * E4M3(c), exact (even integers of at most 4 significant bits).
MOE_DEV f16x2 e4m3_pair_f16(f16x2 v2)
{
    const s16x2 b = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16((s16x2){0, 0}, v2, 128.0f, false);
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(__builtin_bit_cast(uint32_t, b), 128.0f, false);
}

// Fragment -> eight exact fp16 values of 2v (or 128 * E4M3(v/64)).
template <int K, int CB>
MOE_DEV f16x8 frag_decode_f16(uint32_t D0, uint32_t D1, int q, uint32_t m_lo, uint32_t m_hi, int kw = K)
{
    uint32_t st[8];
    frag_states_k<K>(D0, D1, q, kw, st);
    f16x8 out;
#pragma unroll
    for (int t = 0; t < 8; t += 2) {
        f16x2 v = value2_pair_f16(st[t], st[t + 1], m_lo, m_hi);
        if (CB == CB_MCG_E4M3)
            v = e4m3_pair_f16(v);
        out[t] = v[0];
        out[t + 1] = v[1];
    }
    return out;
}

// Fragment -> eight fp16 values of 2v + 1532 (mcg codebook; exact integers
// in [1020, 2044]) at the run-time window width kw when K = 0: the biased
// form whose bias the MFMA gate/up kernel takes off per row.
template <int K>
MOE_DEV f16x8 frag_decode_f16_biased(uint32_t D0, uint32_t D1, int q, uint32_t m_lo, uint32_t m_hi, int kw = K)
{
    uint32_t st[8];
    frag_states_k<K>(D0, D1, q, kw, st);
    u32x4 pk;
#pragma unroll
    for (int t = 0; t < 8; t += 2)
        pk[t / 2] = value2_pair_biased(st[t], st[t + 1], m_lo, m_hi);
    return __builtin_bit_cast(f16x8, pk);
}

// Fragment -> eight exact bf16 values of 2v (or 128 * E4M3(v/64)).
template <int K, int CB>
MOE_DEV bf16x8 frag_decode_bf16(uint32_t D0, uint32_t D1, int q, uint32_t m_lo, uint32_t m_hi, int kw = K)
{
    uint32_t st[8];
    frag_states_k<K>(D0, D1, q, kw, st);
    u32x4 pk;
#pragma unroll
    for (int t = 0; t < 8; t += 2) {
        if (CB == CB_MCG_E4M3) {
            // E4M3 bytes of the pair, widened to bf16 with the factor 128
            const s16x2 b = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(
                (s16x2){0, 0}, value2_pair_f16(st[t], st[t + 1], m_lo, m_hi), 128.0f, false);
            pk[t / 2] = __builtin_bit_cast(
                uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(__builtin_bit_cast(uint32_t, b), 128.0f, false));
        } else {
            const float a = value2_f32(st[t], m_lo, m_hi);
            const float b = value2_f32(st[t + 1], m_lo, m_hi);
            // |2v| <= 512 has at most 8 significant bits: truncation is exact
            pk[t / 2] = __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
        }
    }
    return __builtin_bit_cast(bf16x8, pk);
}

// Fragment -> eight FP8 E4M3 bytes of c = v / 64 (nearest-even, saturating;
// the E4M3 codebook value itself), state t in byte t % 4 of dword t / 4.
// The scaled convert divides the fp16 pair 2v by 128 before rounding.
template <int K>
MOE_DEV u32x2 frag_decode_fp8(uint32_t D0, uint32_t D1, int q, uint32_t m_lo, uint32_t m_hi)
{
    uint32_t st[8];
    frag_states<K>(D0, D1, q, st);
    u32x2 out;
#pragma unroll
    for (int d = 0; d < 2; ++d) {
        s16x2 w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16((s16x2){0, 0},
                                                           value2_pair_f16(st[4 * d], st[4 * d + 1], m_lo, m_hi),
                                                           128.0f, false);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(w, value2_pair_f16(st[4 * d + 2], st[4 * d + 3], m_lo, m_hi),
                                                     128.0f, true);
        out[d] = __builtin_bit_cast(uint32_t, w);
    }
    return out;
}

// Fragment -> the eight decoded values as fp16 pairs of 2v + 1532 (exact:
// integers in [1020, 2044]), the B operand of the decode-fused GEMV's MFMA
// (which subtracts 1532 * sum(x) once per output).  mcg: the
// biased pair straight from the field sums; E4M3: 128 * c8 + 1532 (128 * c8
// is an even integer: E4M3 keeps 4 significant bits of the integer v).
template <int K, int CB>
MOE_DEV void frag_biased_pairs(uint32_t D0, uint32_t D1, int q, uint32_t m_lo, uint32_t m_hi, f16x2 wp[4])
{
    uint32_t st[8];
    frag_states<K>(D0, D1, q, st);
#pragma unroll
    for (int t = 0; t < 8; t += 2) {
        if (CB == CB_MCG)
            wp[t / 2] = __builtin_bit_cast(f16x2, value2_pair_biased(st[t], st[t + 1], m_lo, m_hi));
        else
            wp[t / 2] = e4m3_pair_f16(value2_pair_f16(st[t], st[t + 1], m_lo, m_hi)) +
                        (f16x2){(f16)1532.0f, (f16)1532.0f};
    }
}

// Fragment -> eight fp32 values of 2v (or 128 * E4M3(v/64)).
template <int K, int CB>
MOE_DEV void frag_decode_f32(uint32_t D0, uint32_t D1, int q, uint32_t m_lo, uint32_t m_hi, float out[8])
{
    uint32_t st[8];
    frag_states<K>(D0, D1, q, st);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const float v = value2_f32(st[t], m_lo, m_hi);
        out[t] = CB == CB_MCG_E4M3 ? e4m3_value2(v) : v;
    }
}

}  // namespace moe
