// Internal launchers shared by the host entry points (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe_exl3.h"

namespace moe {

// Rows of one MFMA work tile (an expert's routed rows are cut into tiles of
// this many rows) and columns of one gate/up (per projection) and down work
// tile.
constexpr int kTileM = 256;
constexpr int kGateUpN = 128;
constexpr int kDownN = 256;
// Entries of the routing table handled by one segment-table block.
constexpr int kSegChunk = 2048;
// Largest per-expert row count the GEMV path accepts (rows beyond two per
// pass re-stream the expert's codes), and the default threshold.
constexpr int kGemvMaxRows = 8;
constexpr int kGemvDefaultRows = 2;
// The GEMV blocks keep two rows of activations in LDS within 64 KiB: fp16
// x * suh of both projections for gate/up (8 H bytes), fp16 h for down
// (4 I bytes).
constexpr int kGemvMaxHidden = 8192;
constexpr int kGemvMaxInter = 16384;
// The fp8 path's activation quantizer holds a row's x and two suh rows in
// registers, one wavefront per row: hidden sizes up to this.
constexpr int kQuantMaxHidden = 8192;
// Tokens up to which one block runs the whole routing tail (top-k, segment
// tables, activation copy) in a single launch.
constexpr int kSmallRouteTokens = 64;
// Tokens up to which the shared expert runs as a GEMV.
constexpr int kSharedGemvMaxTokens = 16;
// Up to this many tokens the shared-expert GEMV blocks run inside the routed
// GEMV launches (the bound keeps their registers within those kernels').
constexpr int kSharedGemvMergeTokens = 8;

// Small header at the start of the workspace, written by the routing and
// segment kernels.  status sits at byte MOE_EXL3_STATUS_OFFSET.
struct WsHeader {
    int32_t n_gemv;    // experts on the GEMV path
    int32_t n_tiles;   // MFMA work tiles
    int32_t status;    // MOE_EXL3_STATUS_* bits of this call
    int32_t pad[13];
};
static_assert(offsetof(WsHeader, status) == MOE_EXL3_STATUS_OFFSET, "status word offset");

struct Plan {
    int64_t T;
    int nblk;        // segment-table blocks
    int max_tiles;   // upper bound on MFMA work tiles
    size_t hdr, logits, idx, w, counts, offsets, bhist, sorted, pos, glist, tiles, x16, xr16, hbuf,
        ybuf, sh, sy, a8g, a8u, h8, sg8, su8, sh8, total;
};

hipError_t launch_route_logits(const uint16_t *x, bool bf16, int64_t T, int H, const uint16_t *Wr,
                               const float *bias, int E, float *logits, WsHeader *hdr, hipStream_t s);
hipError_t launch_topk(const float *logits, int64_t T, int E, int k, int32_t *idx, float *w,
                       hipStream_t s);
// With `extra`, expert E (the trellis shared expert) joins the tables with
// the T slots T*k + t, routing weight 1.
hipError_t launch_segments(const int32_t *idx, int64_t T, int k, int E, bool extra, int nblk, int gemv_rows,
                           int tile_m, int max_tiles, int32_t *bhist, int32_t *counts, int32_t *offsets,
                           int32_t *sorted, int32_t *pos, float *w, int32_t *glist, int32_t *tiles,
                           WsHeader *hdr, hipStream_t s);

hipError_t launch_route_small(const float *logits, int64_t T, int E, int k, bool extra, int gemv_rows, int tile_m,
                              int max_tiles, int32_t *idx, float *w, int32_t *counts, int32_t *offsets, int32_t *sorted,
                              int32_t *pos, int32_t *glist, int32_t *tiles, WsHeader *hdr,
                              const uint16_t *x, int H, uint16_t *x16, hipStream_t s);

hipError_t launch_decode(const uint16_t *codes, int n_in, int n_out, int K, uint32_t mcg, int cb,
                         void *dst, int dst_dtype, hipStream_t s);
hipError_t launch_repack(const uint16_t *src, uint16_t *dst, int count, int n_in, int n_out, int K, int order,
                         hipStream_t s);
hipError_t launch_expand_scales(const uint16_t *block, int EA, int H, int I, uint16_t *const suh[3],
                                uint16_t *const svh[3], hipStream_t s);

struct GroupArgs {
    const uint16_t *codes[3];
    const uint16_t *suh[3];
    const uint16_t *svh[3];
    int H, I, k, K, cb;
    int E;          // experts in the segment tables: the routed ones (+ the trellis shared expert)
    int64_t T;
    int64_t nr;     // routed slots T * k; slots nr + t belong to the trellis shared expert
    // per-tensor widths (PER_TENSOR_K; NULL otherwise): [3][E] device
    // addresses of each tensor's codes and its width
    const uint64_t *code_tab;
    const int32_t *k_tab;
    uint32_t mcg;
    const int32_t *counts, *offsets, *sorted, *glist, *tiles;
    const int32_t *idx;      // top-k expert of every routed slot [T*k]
    const int32_t *pos;      // inverse of sorted: the sorted position of slot a
    const WsHeader *hdr;
    const float *w;          // routing weights [T*k]
    const uint16_t *x16;     // fp16 activations [T][H]
    uint16_t *hbuf;          // bf16 [T*k][I], sorted order, h * suh_down
    uint16_t *ybuf;          // bf16 [T*k][H], slot order, w * y
    // fp8 MFMA path (E4M3 codebook): per routed row in sorted order
    uint8_t *a8g, *a8u;      // E4M3 [T*k][H]: x * suh_gate / sg8, x * suh_up / su8
    uint8_t *h8;             // E4M3 [T*k][I]: h / sh8
    float *sg8, *su8, *sh8;  // row scales (least power of two >= row amax / 448)
};

hipError_t launch_convert_x(const uint16_t *x, int64_t n, uint16_t *x16, WsHeader *hdr, hipStream_t s);
// DEBUG_CHECKS: consistency of the routing tables and finiteness of x, into
// the status word.
hipError_t launch_debug_checks(const uint16_t *x, bool bf16, int64_t T, int H, int k, int E,
                               const int32_t *idx, const int32_t *counts, const int32_t *offsets,
                               const int32_t *sorted, const int32_t *pos, WsHeader *hdr, hipStream_t s);
// The dense shared expert, when its work rides along in the routed MFMA or
// GEMV launches (x16 [T][H] fp16, w = gate, up, down nn.Linear fp16, h [T][I]
// fp16 gate/up output, y [T][H] fp32 down output).
struct SharedArgs {
    const uint16_t *x16;
    const uint16_t *w[3];
    uint16_t *h;
    float *y;
};
// With sh set (1 <= T <= kSharedGemvMergeTokens), the shared expert's GEMV
// rows run as extra blocks after the routed ones.
hipError_t launch_gemv_gateup(const GroupArgs &a, int max_list, const SharedArgs *sh, hipStream_t s);
hipError_t launch_gemv_down(const GroupArgs &a, int max_list, const SharedArgs *sh, hipStream_t s);
hipError_t launch_mfma_gateup(const GroupArgs &a, int max_tiles, const SharedArgs *sh, hipStream_t s);
hipError_t launch_mfma_down(const GroupArgs &a, int max_tiles, const SharedArgs *sh, hipStream_t s);
hipError_t launch_quant_gateup(const GroupArgs &a, int64_t n, hipStream_t s);
hipError_t launch_quant_h(const GroupArgs &a, int64_t n, hipStream_t s);
hipError_t launch_mfma8_gateup(const GroupArgs &a, int max_tiles, hipStream_t s);
hipError_t launch_mfma8_down(const GroupArgs &a, int max_tiles, hipStream_t s);

hipError_t launch_shared_gateup(const uint16_t *x16, int64_t T, int H, int I, const uint16_t *wg,
                                const uint16_t *wu, uint16_t *sh, hipStream_t s);
hipError_t launch_shared_down(const uint16_t *sh, int64_t T, int H, int I, const uint16_t *wd,
                              float *sy, hipStream_t s);
hipError_t launch_shared_gemv(const uint16_t *x16, int T, int H, int I, const uint16_t *wg,
                              const uint16_t *wu, const uint16_t *wd, uint16_t *sh, float *sy,
                              hipStream_t s);
// out = sy + s1 * R(routed slot rows (+ the trellis shared expert's row));
// without s1 no rotation.
hipError_t launch_combine(const uint16_t *ybuf, const float *sy, int64_t T, int H, int k, bool extra,
                          const int8_t *s1, bool bf16, uint16_t *out, hipStream_t s);
// xr = fp16(R(s0 * x)), the rotated activations of the trellis experts.
hipError_t launch_rotate_x(const uint16_t *x, bool bf16, int64_t T, int H, const int8_t *s0, uint16_t *xr,
                           WsHeader *hdr, hipStream_t s);

}  // namespace moe
