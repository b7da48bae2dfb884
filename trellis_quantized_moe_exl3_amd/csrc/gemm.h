// Helpers shared by the MFMA expert kernels (fp16/bf16 and fp8).
#pragma once

#include "common.h"

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

}  // namespace moe
