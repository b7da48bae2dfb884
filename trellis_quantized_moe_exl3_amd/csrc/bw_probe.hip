// Streaming-read probe: the HBM read bandwidth a plain kernel reaches on this
// GPU, the "achievable" figure next to the 8 TB/s specification in the
// benchmark's bandwidth fractions.  Not part of the layer library.
//
// Each thread reads 16-byte pieces in a grid-stride loop, eight nontemporal
// loads in flight, and folds them with XOR; one word per block is written so
// the loads cannot be removed.  Of the variants measured (4, 8 or 16 loads in
// flight, plain or nontemporal, grid-stride or one contiguous range per block,
// 1024 to 16384 blocks of 256 threads), this one read fastest, at 16384 blocks.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kInFlight = 8;

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4 *__restrict__ src, int64_t n16,
                                                          uint32_t *__restrict__ sink)
{
    const int64_t stride = (int64_t)gridDim.x * 256;
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (; i + (kInFlight - 1) * stride < n16; i += kInFlight * stride) {
        u32x4 v[kInFlight];
#pragma unroll
        for (int u = 0; u < kInFlight; ++u)
            v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < kInFlight; ++u)
            acc ^= v[u];
    }
    for (; i < n16; i += stride)
        acc ^= src[i];
    __shared__ uint32_t red[256];
    red[threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = 0;
        for (int t = 0; t < 256; ++t)
            r ^= red[t];
        sink[blockIdx.x] = r;
    }
}

extern "C" int moe_exl3_bw_stream_read(const void *src, int64_t bytes, uint32_t *sink, int blocks, void *stream)
{
    if (!src || !sink || bytes < 16 || blocks < 1 || ((uintptr_t)src & 15))
        return -1;
    stream_read_kernel<<<blocks, 256, 0, (hipStream_t)stream>>>((const u32x4 *)src, bytes / 16, sink);
    return hipGetLastError() == hipSuccess ? 0 : -5;
}
