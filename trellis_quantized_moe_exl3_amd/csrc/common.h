// Shared device/host definitions of the HIP library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef _Float16 f16;
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

#define MOE_DEV __device__ __forceinline__

MOE_DEV float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
MOE_DEV float f16_to_f32(uint16_t h) { return (float)__builtin_bit_cast(f16, h); }

// Round-to-nearest-even fp32 -> bf16 bits (inputs are finite).
MOE_DEV uint16_t f32_to_bf16_bits(float f)
{
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}

MOE_DEV uint16_t f32_to_f16_bits(float f)
{
    return __builtin_bit_cast(uint16_t, (f16)f);
}

// Activation element -> fp32 (activation dtype is fp16 or bf16).
template <bool BF16>
MOE_DEV float act_to_f32(uint16_t v)
{
    return BF16 ? bf16_to_f32(v) : f16_to_f32(v);
}

// Eight bf16 activations (raw 16-byte piece) -> eight fp16 (round to nearest
// even; exact in fp16's normal range).  `over` is set when a finite value lies
// beyond the fp16 range and became infinite.
MOE_DEV u32x4 bf16x8_to_f16x8(u32x4 v, bool &over)
{
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float lo = __uint_as_float(v[j] << 16), hi = __uint_as_float(v[j] & 0xFFFF0000u);
        const uint32_t a = f32_to_f16_bits(lo), b = f32_to_f16_bits(hi);
        // fp16 infinity (0x7C00 after the sign) from a finite bf16 (exponent
        // field below 0xFF)
        over |= ((a & 0x7FFFu) == 0x7C00u && (v[j] & 0x7F80u) != 0x7F80u) ||
                ((b & 0x7FFFu) == 0x7C00u && (v[j] & 0x7F800000u) != 0x7F800000u);
        o[j] = a | (b << 16);
    }
    return o;
}

// Token of routed-table slot a: a / k for the nr = T * k routed slots, a - nr
// for the trellis shared expert's slots that follow them.
MOE_DEV int64_t slot_token(int64_t a, int64_t nr, int k) { return a < nr ? a / k : a - nr; }

// Wavefront size on CDNA.
constexpr int kWave = 64;

// silu(z) = z / (1 + e^-z) with the hardware reciprocal (about 1 ulp)
MOE_DEV float silu_f(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }
