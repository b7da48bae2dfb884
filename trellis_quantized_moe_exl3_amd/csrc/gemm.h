// Helpers shared by the MFMA expert kernels (fp16/bf16 and fp8).
#pragma once

#include "common.h"
#include "internal.h"

namespace moe {

#define LDS_AS __attribute__((address_space(3)))

// Blocks are dealt to the 8 XCDs round-robin (block L runs on XCD L % 8).
// Map block L so that every column slice of a row tile lands on one XCD and
// the slices of a tile are consecutive there: the tile's A rows are then
// fetched into that XCD's L2 once and reused by all its slices.
MOE_DEV void xcd_map(int L, int nslices, int &tile, int &slice)
{
    const int x = L & 7, j = L >> 3;
    tile = (j / nslices) * 8 + x;
    slice = j % nslices;
}

// Raw buffer resource over `bytes` bytes at p (loads past the end return 0).
MOE_DEV __amdgpu_buffer_rsrc_t buf_rsrc(const void *p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, (int)bytes, 0x00020000);
}

// s_waitcnt with only the vector-memory counter limited to n (gfx9 encoding:
// vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14).
template <int N>
MOE_DEV void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | 0x70 | 0xF00 | ((N >> 4) << 14));
}

// LDS layout of one A stage: row r is 64 bytes = four 16-byte pieces; the
// piece holding k-offset 8p is stored in slot p ^ ((r >> 2) & 3), which makes
// the 16-lane reads of an MFMA A fragment (16 consecutive rows, one piece)
// hit 16 distinct 4-bank groups.
MOE_DEV int a_slot(int r, int p) { return p ^ ((r >> 2) & 3); }

// First/second dword of a lane fragment (column c, k-half h) of a tile at
// width K, and the bit offset inside the first (the run-time form of
// frag_pos<K>, for kernels whose width is read per tensor).
MOE_DEV void frag_pos_rt(int K, int c, int h, int &d0, int &d1, int &q)
{
    const int b0 = K * (16 * c + 8 * h);
    d0 = b0 >> 5;
    q = b0 & 31;
    d1 = (d0 + 1 == 8 * K) ? 0 : d0 + 1;
}

// The code words of tensor (p, e), an [n_in/16][n_out/16] tile grid.
//   K > 0, no tables:   every tensor has width K and is slice e of codes[p].
//   K > 0, tables:      the tensor's own address; its table width must be K
//                       (the caller dispatched on it), otherwise the width
//                       was invalid.
//   K = 0 (tables):     the address and the width from the tables.
// An invalid width sets the status bit and the tensor is read through an
// empty range (as zero words, at width 2).
struct TensorCodes {
    const uint32_t *base;
    uint32_t bytes;   // of the tensor (0: nothing may be read)
    int K;
};

// A wave-uniform 64-bit address as such: values loaded from memory are not
// known to be uniform, and a buffer descriptor built from a non-uniform base
// turns every load through it into a waterfall loop.
MOE_DEV const uint32_t *uniform_ptr(const void *p)
{
    const uint64_t v = (uint64_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (const uint32_t *)(((uint64_t)hi << 32) | lo);
}

MOE_DEV int table_width(const GroupArgs &a, int p, int e)
{
    const int kw = a.k_tab[p * a.E + e];
    return (kw >= 2 && kw <= 4) ? kw : 0;
}

template <int K>
MOE_DEV TensorCodes tensor_codes(const GroupArgs &a, int p, int e, int n_in, int n_out)
{
    TensorCodes t;
    const uint32_t grid_bytes = (uint32_t)((n_in / 16) * (n_out / 16) * 32);
    if (!a.code_tab) {
        t.K = K;
        t.bytes = grid_bytes * K;
        t.base = uniform_ptr((const char *)a.codes[p] + (int64_t)e * t.bytes);
        return t;
    }
    const int kw = table_width(a, p, e);
    const bool ok = K > 0 ? kw == K : kw != 0;
    if (!ok)
        atomicOr((unsigned *)&const_cast<WsHeader *>(a.hdr)->status, MOE_EXL3_STATUS_BAD_WIDTH);
    t.K = __builtin_amdgcn_readfirstlane(K > 0 ? K : (ok ? kw : 2));
    t.bytes = __builtin_amdgcn_readfirstlane(ok ? grid_bytes * t.K : 0u);
    t.base = uniform_ptr((const void *)a.code_tab[p * a.E + e]);
    return t;
}

}  // namespace moe
