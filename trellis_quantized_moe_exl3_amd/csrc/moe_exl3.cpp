// Host side of the C ABI: argument checks, workspace plan, launch sequence.
// Declarations and the full contract are in include/moe_exl3.h.
#include "moe_exl3.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>

#include "internal.h"

using namespace moe;

// Workspace of moe_exl3_layer_noalloc: a device array of the library, one
// copy per GPU, held until the process ends.  Its name is a host-side stand-in
// in host code; only the address hipGetSymbolAddress returns for the current
// device may reach a kernel or a copy.
static __device__ __align__(256) unsigned char scratch[MOE_EXL3_SCRATCH_BYTES];

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// The routed-row threshold between the GEMV and MFMA paths for a call of T
// tokens.  No expert receives more rows than there are tokens (a token's k
// experts are distinct), so with the default threshold a call of at most
// kGemvMaxRows tokens puts every expert on the GEMV path and needs no MFMA
// launch at all.
int gemv_rows_of(const moe_exl3_desc &d, int64_t T)
{
    // the GEMV blocks keep two rows of activations in LDS (64 KiB at most)
    const int cap = kGemvMaxRows;
    if ((d.flags & MOE_EXL3_FORCE_MFMA) || d.hidden > kGemvMaxHidden || d.inter > kGemvMaxInter)
        return 0;
    if (d.flags & MOE_EXL3_FORCE_GEMV)
        return cap;
    if (d.gemv_max_rows > 0)
        return std::min(d.gemv_max_rows, cap);
    return T <= cap ? cap : kGemvDefaultRows;
}

int check_desc(const moe_exl3_desc *d)
{
    if (!d)
        return MOE_EXL3_ERR_INVALID_ARG;
    if (d->hidden <= 0 || d->inter <= 0 || d->n_experts <= 0 || d->top_k <= 0)
        return MOE_EXL3_ERR_INVALID_ARG;
    if (d->hidden % 256 || d->inter % 128 || d->n_experts % 8)
        return MOE_EXL3_ERR_INVALID_ARG;
    if (d->hidden > 16384 || d->inter > 16384 || d->n_experts > 1024 || d->top_k > 16 ||
        d->top_k > d->n_experts)
        return MOE_EXL3_ERR_UNSUPPORTED;
    if (d->K < 2 || d->K > 4)
        return MOE_EXL3_ERR_UNSUPPORTED;
    if (d->codebook != MOE_EXL3_CB_MCG && d->codebook != MOE_EXL3_CB_MCG_E4M3)
        return MOE_EXL3_ERR_UNSUPPORTED;
    if (d->act_dtype != MOE_EXL3_DT_F16 && d->act_dtype != MOE_EXL3_DT_BF16)
        return MOE_EXL3_ERR_UNSUPPORTED;
    if (d->gemv_max_rows < 0)
        return MOE_EXL3_ERR_INVALID_ARG;
    // fp8 MFMA: only the E4M3 codebook (its values are exact in E4M3), and
    // whole 4-stage pipeline rounds of 64 input channels
    if ((d->flags & MOE_EXL3_FP8_MFMA) &&
        (d->codebook != MOE_EXL3_CB_MCG_E4M3 || d->hidden % 256 || d->inter % 256 || d->hidden > kQuantMaxHidden))
        return MOE_EXL3_ERR_UNSUPPORTED;
    if ((d->flags & MOE_EXL3_FORCE_GEMV) && (d->flags & MOE_EXL3_FORCE_MFMA))
        return MOE_EXL3_ERR_INVALID_ARG;
    // fp8 MFMA kernels read one width per launch
    if ((d->flags & MOE_EXL3_FP8_MFMA) && (d->flags & MOE_EXL3_PER_TENSOR_K))
        return MOE_EXL3_ERR_UNSUPPORTED;
    // the segment kernels keep one thread per table expert (1024)
    if ((d->flags & MOE_EXL3_SHARED_TRELLIS) && d->n_experts + 1 > 1024)
        return MOE_EXL3_ERR_UNSUPPORTED;
    return MOE_EXL3_OK;
}

// Trellis-coded experts in the tensors and the segment tables.
int trellis_experts(const moe_exl3_desc &d) { return d.n_experts + ((d.flags & MOE_EXL3_SHARED_TRELLIS) ? 1 : 0); }

// Slots of the segment tables: T * k routed, + T of the trellis shared expert.
int64_t table_slots(const moe_exl3_desc &d, int64_t T)
{
    return T * d.top_k + ((d.flags & MOE_EXL3_SHARED_TRELLIS) ? T : 0);
}

int check_weights(const moe_exl3_desc &d, const moe_exl3_weights *w, bool routing_only)
{
    if (!w || !w->router_w)
        return MOE_EXL3_ERR_INVALID_ARG;
    if ((d.flags & MOE_EXL3_HAS_ROUTER_BIAS) && !w->router_bias)
        return MOE_EXL3_ERR_INVALID_ARG;
    if (!aligned16(w->router_w) || ((d.flags & MOE_EXL3_HAS_ROUTER_BIAS) && !aligned16(w->router_bias)))
        return MOE_EXL3_ERR_MISALIGNED;
    if (routing_only)
        return MOE_EXL3_OK;
    const bool ptk = d.flags & MOE_EXL3_PER_TENSOR_K;
    if (ptk && (!w->code_tab || !w->k_tab))
        return MOE_EXL3_ERR_INVALID_ARG;
    if (ptk && (!aligned16(w->code_tab) || !aligned16(w->k_tab)))
        return MOE_EXL3_ERR_MISALIGNED;
    if (d.flags & MOE_EXL3_HADAMARD) {
        if (!w->signs)
            return MOE_EXL3_ERR_INVALID_ARG;
        if (!aligned16(w->signs))
            return MOE_EXL3_ERR_MISALIGNED;
    }
    for (int p = 0; p < 3; ++p) {
        if ((!ptk && !w->codes[p]) || !w->suh[p] || !w->svh[p])
            return MOE_EXL3_ERR_INVALID_ARG;
        if ((!ptk && !aligned16(w->codes[p])) || !aligned16(w->suh[p]) || !aligned16(w->svh[p]))
            return MOE_EXL3_ERR_MISALIGNED;
        if (d.flags & MOE_EXL3_HAS_SHARED) {
            if (!w->shared_w[p])
                return MOE_EXL3_ERR_INVALID_ARG;
            if (!aligned16(w->shared_w[p]))
                return MOE_EXL3_ERR_MISALIGNED;
        }
    }
    return MOE_EXL3_OK;
}

// The GEMM kernels read activations, h rows, codes and shared weights through
// 32-bit buffer offsets: every such buffer must stay below 2 GiB.
bool buffers_addressable(const moe_exl3_desc &d, int64_t T)
{
    const int64_t lim = (int64_t)1 << 31;
    const int64_t slots = table_slots(d, T);
    return T * d.hidden * 2 < lim && slots * d.inter * 2 < lim && slots * d.hidden * 2 < lim &&
           T * d.inter * 2 < lim && (int64_t)d.hidden * d.inter * 2 < lim;
}

Plan make_plan(const moe_exl3_desc &d, int64_t T)
{
    Plan p{};
    p.T = T;
    const int64_t n = T * d.top_k;         // routed slots
    const int64_t ns = table_slots(d, T);  // + the trellis shared expert's
    const int E = d.n_experts, EA = trellis_experts(d);
    p.nblk = (int)std::max<int64_t>(1, (n + kSegChunk - 1) / kSegChunk);
    const int g = gemv_rows_of(d, T);
    // experts with more than g rows (at most ns / (g + 1)) each add one
    // partial tile to the ns / kTileM full ones
    const int64_t heavy = std::min<int64_t>(EA, ns / (g + 1));
    p.max_tiles = T <= g ? 0 : (int)std::max<int64_t>(0, std::min<int64_t>(ns / kTileM + heavy, ns));
    size_t o = 0;
    auto take = [&](size_t bytes) {
        const size_t at = o;
        o = align_up(o + bytes);
        return at;
    };
    p.hdr = take(sizeof(WsHeader));
    p.logits = take(sizeof(float) * (size_t)T * E);
    p.idx = take(sizeof(int32_t) * (size_t)n);
    p.w = take(sizeof(float) * (size_t)ns);
    p.counts = take(sizeof(int32_t) * (size_t)EA);
    p.offsets = take(sizeof(int32_t) * (size_t)(EA + 1));
    p.bhist = take(sizeof(int32_t) * (size_t)p.nblk * E);
    p.sorted = take(sizeof(int32_t) * (size_t)ns);
    p.pos = take(sizeof(int32_t) * (size_t)ns);
    p.glist = take(sizeof(int32_t) * (size_t)EA);
    p.tiles = take(sizeof(int32_t) * 2 * (size_t)std::max(1, p.max_tiles));
    p.x16 = take(d.act_dtype == MOE_EXL3_DT_BF16 ? sizeof(uint16_t) * (size_t)T * d.hidden : 0);
    p.xr16 = take((d.flags & MOE_EXL3_HADAMARD) ? sizeof(uint16_t) * (size_t)T * d.hidden : 0);
    p.hbuf = take(sizeof(uint16_t) * (size_t)ns * d.inter);
    p.ybuf = take(sizeof(uint16_t) * (size_t)ns * d.hidden);
    const bool sh = d.flags & MOE_EXL3_HAS_SHARED;
    p.sh = take(sh ? sizeof(uint16_t) * (size_t)T * d.inter : 0);
    p.sy = take(sh ? sizeof(float) * (size_t)T * d.hidden : 0);
    const bool f8 = d.flags & MOE_EXL3_FP8_MFMA;
    p.a8g = take(f8 ? (size_t)ns * d.hidden : 0);
    p.a8u = take(f8 ? (size_t)ns * d.hidden : 0);
    p.h8 = take(f8 ? (size_t)ns * d.inter : 0);
    p.sg8 = take(f8 ? sizeof(float) * (size_t)ns : 0);
    p.su8 = take(f8 ? sizeof(float) * (size_t)ns : 0);
    p.sh8 = take(f8 ? sizeof(float) * (size_t)ns : 0);
    p.total = o;
    return p;
}

template <class T>
T *at(void *ws, size_t off)
{
    return (T *)((char *)ws + off);
}

// Records events[step] when timing hooks were given.
struct Marks {
    void *const *ev = nullptr;
    hipStream_t s = nullptr;
    bool mark(int step) const
    {
        return !ev || hipEventRecord((hipEvent_t)ev[step], s) == hipSuccess;
    }
};

// Routing steps a1-a3.  Decode-sized calls (T <= kSmallRouteTokens, one
// segment chunk) run everything after the logits in one single-block launch,
// which also writes the fp16 copy of bf16 activations when x16 is given (then
// *converted is set).
int run_route(const moe_exl3_desc &d, const moe_exl3_weights &w, const void *x, int64_t T,
              void *ws, const Plan &p, hipStream_t s, const Marks &mk = Marks(),
              uint16_t *x16 = nullptr, bool *converted = nullptr)
{
    const bool bf16 = d.act_dtype == MOE_EXL3_DT_BF16;
    const float *bias = (d.flags & MOE_EXL3_HAS_ROUTER_BIAS) ? w.router_bias : nullptr;
    if (!mk.mark(MOE_EXL3_STEP_ROUTE_LOGITS))
        return MOE_EXL3_ERR_HIP;
    WsHeader *hdr = at<WsHeader>(ws, p.hdr);
    if (launch_route_logits((const uint16_t *)x, bf16, T, d.hidden, w.router_w, bias, d.n_experts,
                            at<float>(ws, p.logits), hdr, s) != hipSuccess)
        return MOE_EXL3_ERR_HIP;
    const bool debug = d.flags & MOE_EXL3_DEBUG_CHECKS;
    const bool extra = d.flags & MOE_EXL3_SHARED_TRELLIS;
    auto checks = [&]() {
        return !debug || launch_debug_checks((const uint16_t *)x, bf16, T, d.hidden, d.top_k, d.n_experts,
                                             at<int32_t>(ws, p.idx), at<int32_t>(ws, p.counts),
                                             at<int32_t>(ws, p.offsets), at<int32_t>(ws, p.sorted),
                                             at<int32_t>(ws, p.pos), hdr, s) == hipSuccess;
    };
    if (!mk.mark(MOE_EXL3_STEP_TOPK))
        return MOE_EXL3_ERR_HIP;
    if (T <= kSmallRouteTokens && p.nblk == 1) {
        if (launch_route_small(at<float>(ws, p.logits), T, d.n_experts, d.top_k, extra, gemv_rows_of(d, T), kTileM,
                               p.max_tiles, at<int32_t>(ws, p.idx), at<float>(ws, p.w), at<int32_t>(ws, p.counts),
                               at<int32_t>(ws, p.offsets), at<int32_t>(ws, p.sorted), at<int32_t>(ws, p.pos),
                               at<int32_t>(ws, p.glist), at<int32_t>(ws, p.tiles), hdr,
                               (const uint16_t *)x, d.hidden, x16, s) != hipSuccess ||
            !checks() || !mk.mark(MOE_EXL3_STEP_SEGMENTS))
            return MOE_EXL3_ERR_HIP;
        if (converted)
            *converted = x16 != nullptr;
        return MOE_EXL3_OK;
    }
    if (launch_topk(at<float>(ws, p.logits), T, d.n_experts, d.top_k, at<int32_t>(ws, p.idx),
                    at<float>(ws, p.w), s) != hipSuccess)
        return MOE_EXL3_ERR_HIP;
    if (!mk.mark(MOE_EXL3_STEP_SEGMENTS))
        return MOE_EXL3_ERR_HIP;
    if (launch_segments(at<int32_t>(ws, p.idx), T, d.top_k, d.n_experts, extra, p.nblk, gemv_rows_of(d, T),
                        kTileM, p.max_tiles, at<int32_t>(ws, p.bhist), at<int32_t>(ws, p.counts),
                        at<int32_t>(ws, p.offsets), at<int32_t>(ws, p.sorted),
                        at<int32_t>(ws, p.pos), at<float>(ws, p.w), at<int32_t>(ws, p.glist),
                        at<int32_t>(ws, p.tiles), hdr, s) != hipSuccess ||
        !checks())
        return MOE_EXL3_ERR_HIP;
    return MOE_EXL3_OK;
}

// Device address of `scratch` on the current device, taken once per device.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch[kMaxDevices];

int scratch_of_current_device(void **ptr)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return MOE_EXL3_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return MOE_EXL3_ERR_HIP;
        g_scratch[dev] = p;
    }
    *ptr = g_scratch[dev];
    return MOE_EXL3_OK;
}

}  // namespace

extern "C" {

int moe_exl3_version(void) { return MOE_EXL3_ABI_VERSION; }

const char *moe_exl3_strerror(int code)
{
    switch (code) {
    case MOE_EXL3_OK: return "ok";
    case MOE_EXL3_ERR_INVALID_ARG: return "invalid argument (null pointer, negative size or shape rule)";
    case MOE_EXL3_ERR_UNSUPPORTED: return "unsupported K, dtype, codebook, flag or size";
    case MOE_EXL3_ERR_WORKSPACE: return "workspace too small";
    case MOE_EXL3_ERR_MISALIGNED: return "device pointer not 16-byte aligned (workspace: 256-byte)";
    case MOE_EXL3_ERR_HIP: return "HIP launch error";
    default: return "unknown error";
    }
}

int moe_exl3_workspace_size(const moe_exl3_desc *desc, int64_t max_tokens, size_t *bytes)
{
    const int rc = check_desc(desc);
    if (rc)
        return rc;
    if (!bytes || max_tokens < 0)
        return MOE_EXL3_ERR_INVALID_ARG;
    if (max_tokens * desc->top_k >= ((int64_t)1 << 31) || !buffers_addressable(*desc, max_tokens))
        return MOE_EXL3_ERR_UNSUPPORTED;
    *bytes = make_plan(*desc, max_tokens).total;
    return MOE_EXL3_OK;
}

int moe_exl3_route(const moe_exl3_desc *desc, const moe_exl3_weights *weights, const void *x,
                   int64_t T, int32_t *idx, float *w, int32_t *counts, int32_t *offsets,
                   int32_t *sorted_ids, int32_t *pos, void *workspace, size_t ws_bytes, void *stream)
{
    int rc = check_desc(desc);
    if (rc)
        return rc;
    if (T < 0)
        return MOE_EXL3_ERR_INVALID_ARG;
    if (T * desc->top_k >= ((int64_t)1 << 31))
        return MOE_EXL3_ERR_UNSUPPORTED;
    if (T == 0)
        return MOE_EXL3_OK;
    rc = check_weights(*desc, weights, true);
    if (rc)
        return rc;
    if (!x || !idx || !workspace)
        return MOE_EXL3_ERR_INVALID_ARG;
    if (!aligned16(x) || ((uintptr_t)workspace % kAlign))
        return MOE_EXL3_ERR_MISALIGNED;
    const Plan p = make_plan(*desc, T);
    if (ws_bytes < p.total)
        return MOE_EXL3_ERR_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    rc = run_route(*desc, *weights, x, T, workspace, p, s);
    if (rc)
        return rc;
    const int64_t n = T * desc->top_k;
    const int E = desc->n_experts;
    struct Cp { void *dst; size_t off, bytes; } cps[] = {
        {idx, p.idx, sizeof(int32_t) * (size_t)n},
        {w, p.w, sizeof(float) * (size_t)n},
        {counts, p.counts, sizeof(int32_t) * (size_t)E},
        {offsets, p.offsets, sizeof(int32_t) * (size_t)(E + 1)},
        {sorted_ids, p.sorted, sizeof(int32_t) * (size_t)n},
        {pos, p.pos, sizeof(int32_t) * (size_t)n},
    };
    for (const Cp &c : cps)
        if (c.dst && hipMemcpyAsync(c.dst, at<char>(workspace, c.off), c.bytes, hipMemcpyDeviceToDevice, s) != hipSuccess)
            return MOE_EXL3_ERR_HIP;
    return MOE_EXL3_OK;
}

static int run_layer(const moe_exl3_desc *desc, const moe_exl3_weights *weights, const void *x,
                     int64_t T, void *out, void *workspace, size_t ws_bytes, void *stream,
                     void *const *events)
{
    int rc = check_desc(desc);
    if (rc)
        return rc;
    if (T < 0)
        return MOE_EXL3_ERR_INVALID_ARG;
    if (T * desc->top_k >= ((int64_t)1 << 31) || !buffers_addressable(*desc, T))
        return MOE_EXL3_ERR_UNSUPPORTED;
    if (T == 0)
        return MOE_EXL3_OK;
    rc = check_weights(*desc, weights, false);
    if (rc)
        return rc;
    if (!x || !out || !workspace)
        return MOE_EXL3_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(out) || ((uintptr_t)workspace % kAlign))
        return MOE_EXL3_ERR_MISALIGNED;
    const size_t xbytes = sizeof(uint16_t) * (size_t)T * desc->hidden;
    if ((const char *)out < (const char *)x + xbytes && (const char *)x < (const char *)out + xbytes)
        return MOE_EXL3_ERR_INVALID_ARG;
    const Plan p = make_plan(*desc, T);
    if (ws_bytes < p.total)
        return MOE_EXL3_ERR_WORKSPACE;
    const moe_exl3_desc &d = *desc;
    const moe_exl3_weights &wt = *weights;
    hipStream_t s = (hipStream_t)stream;
    void *ws = workspace;

    Marks mk;
    mk.ev = events;
    mk.s = s;
    const bool bf16 = d.act_dtype == MOE_EXL3_DT_BF16;
    bool converted = false;
    rc = run_route(d, wt, x, T, ws, p, s, mk, bf16 ? at<uint16_t>(ws, p.x16) : nullptr, &converted);
    if (rc)
        return rc;
    if (!mk.mark(MOE_EXL3_STEP_CONVERT_X))
        return MOE_EXL3_ERR_HIP;
    const uint16_t *x16 = (const uint16_t *)x;
    if (bf16) {
        if (!converted &&
            launch_convert_x((const uint16_t *)x, T * d.hidden, at<uint16_t>(ws, p.x16), at<WsHeader>(ws, p.hdr), s) !=
                hipSuccess)
            return MOE_EXL3_ERR_HIP;
        x16 = at<uint16_t>(ws, p.x16);
    }
    // the trellis experts' activations: x in fp16, or its rotation
    const bool rot = d.flags & MOE_EXL3_HADAMARD;
    const uint16_t *xe16 = x16;
    if (rot) {
        if (launch_rotate_x((const uint16_t *)x, bf16, T, d.hidden, wt.signs, at<uint16_t>(ws, p.xr16),
                            at<WsHeader>(ws, p.hdr), s) != hipSuccess)
            return MOE_EXL3_ERR_HIP;
        xe16 = at<uint16_t>(ws, p.xr16);
    }
    GroupArgs ga{};
    for (int i = 0; i < 3; ++i) {
        ga.codes[i] = wt.codes[i];
        ga.suh[i] = wt.suh[i];
        ga.svh[i] = wt.svh[i];
    }
    ga.H = d.hidden;
    ga.I = d.inter;
    ga.E = trellis_experts(d);
    ga.nr = T * d.top_k;
    if (d.flags & MOE_EXL3_PER_TENSOR_K) {
        ga.code_tab = wt.code_tab;
        ga.k_tab = wt.k_tab;
    }
    ga.k = d.top_k;
    ga.T = T;
    ga.K = d.K;
    ga.cb = d.codebook;
    ga.mcg = d.mcg;
    ga.counts = at<int32_t>(ws, p.counts);
    ga.offsets = at<int32_t>(ws, p.offsets);
    ga.sorted = at<int32_t>(ws, p.sorted);
    ga.idx = at<int32_t>(ws, p.idx);
    ga.pos = at<int32_t>(ws, p.pos);
    ga.glist = at<int32_t>(ws, p.glist);
    ga.tiles = at<int32_t>(ws, p.tiles);
    ga.hdr = at<WsHeader>(ws, p.hdr);
    ga.w = at<float>(ws, p.w);
    ga.x16 = xe16;
    ga.hbuf = at<uint16_t>(ws, p.hbuf);
    ga.ybuf = at<uint16_t>(ws, p.ybuf);
    const bool f8 = d.flags & MOE_EXL3_FP8_MFMA;
    if (f8) {
        ga.a8g = at<uint8_t>(ws, p.a8g);
        ga.a8u = at<uint8_t>(ws, p.a8u);
        ga.h8 = at<uint8_t>(ws, p.h8);
        ga.sg8 = at<float>(ws, p.sg8);
        ga.su8 = at<float>(ws, p.su8);
        ga.sh8 = at<float>(ws, p.sh8);
    }
    const int g = gemv_rows_of(d, T);
    const int64_t n = table_slots(d, T);
    const int max_list = g > 0 ? (int)std::min<int64_t>(trellis_experts(d), n) : 0;

    // The shared expert: a dot-product GEMV for up to kSharedGemvMaxTokens
    // tokens, whose blocks run at the end of the routed GEMV launches for up to
    // kSharedGemvMergeTokens (the memory-bound shared rows fill the second,
    // partly empty round of the VALU-bound routed blocks); otherwise its dense
    // tiles ride along in the routed 16-bit MFMA launches (filling the CUs
    // their last routed tiles leave idle), or, on the fp8 path, run in
    // launches of their own.
    const bool shared = d.flags & MOE_EXL3_HAS_SHARED;
    uint16_t *sh = shared ? at<uint16_t>(ws, p.sh) : nullptr;
    float *sy = shared ? at<float>(ws, p.sy) : nullptr;
    SharedArgs sa{};
    if (shared) {
        sa.x16 = x16;
        for (int i = 0; i < 3; ++i)
            sa.w[i] = wt.shared_w[i];
        sa.h = sh;
        sa.y = sy;
    }
    const bool merged = shared && !f8 && T > kSharedGemvMaxTokens;
    const bool gemv_merged = shared && T <= kSharedGemvMergeTokens && max_list > 0;
    const SharedArgs *sap = merged ? &sa : nullptr;
    const SharedArgs *sgp = gemv_merged ? &sa : nullptr;

    // fp8: the activation rows are quantized at the end of the convert step,
    // the h rows at the start of the GEMV down step
    if (f8 && launch_quant_gateup(ga, n, s) != hipSuccess)
        return MOE_EXL3_ERR_HIP;
    if (!mk.mark(MOE_EXL3_STEP_GEMV_GATEUP) || launch_gemv_gateup(ga, max_list, sgp, s) != hipSuccess ||
        !mk.mark(MOE_EXL3_STEP_MFMA_GATEUP) ||
        (f8 ? launch_mfma8_gateup(ga, p.max_tiles, s) : launch_mfma_gateup(ga, p.max_tiles, sap, s)) != hipSuccess ||
        !mk.mark(MOE_EXL3_STEP_GEMV_DOWN) || (f8 && launch_quant_h(ga, n, s) != hipSuccess) ||
        launch_gemv_down(ga, max_list, sgp, s) != hipSuccess ||
        !mk.mark(MOE_EXL3_STEP_MFMA_DOWN) ||
        (f8 ? launch_mfma8_down(ga, p.max_tiles, s) : launch_mfma_down(ga, p.max_tiles, sap, s)) != hipSuccess ||
        !mk.mark(MOE_EXL3_STEP_SHARED))
        return MOE_EXL3_ERR_HIP;

    if (shared && !merged && !gemv_merged) {
        hipError_t e;
        if (T <= kSharedGemvMaxTokens)
            e = launch_shared_gemv(x16, (int)T, d.hidden, d.inter, wt.shared_w[0], wt.shared_w[1],
                                   wt.shared_w[2], sh, sy, s);
        else {
            e = launch_shared_gateup(x16, T, d.hidden, d.inter, wt.shared_w[0], wt.shared_w[1], sh, s);
            if (e == hipSuccess)
                e = launch_shared_down(sh, T, d.hidden, d.inter, wt.shared_w[2], sy, s);
        }
        if (e != hipSuccess)
            return MOE_EXL3_ERR_HIP;
    }
    if (!mk.mark(MOE_EXL3_STEP_COMBINE) ||
        launch_combine(at<uint16_t>(ws, p.ybuf), sy, T, d.hidden, d.top_k, d.flags & MOE_EXL3_SHARED_TRELLIS,
                       rot ? wt.signs + d.hidden : nullptr, bf16, (uint16_t *)out, s) != hipSuccess ||
        !mk.mark(MOE_EXL3_STEP_END))
        return MOE_EXL3_ERR_HIP;
    return MOE_EXL3_OK;
}

int moe_exl3_layer(const moe_exl3_desc *desc, const moe_exl3_weights *weights, const void *x,
                   int64_t T, void *out, void *workspace, size_t ws_bytes, void *stream)
{
    return run_layer(desc, weights, x, T, out, workspace, ws_bytes, stream, nullptr);
}

int moe_exl3_layer_noalloc(const moe_exl3_desc *desc, const moe_exl3_weights *weights, const void *x, int64_t T,
                           void *out, void *stream)
{
    int rc = check_desc(desc);
    if (rc)
        return rc;
    if (T < 0)
        return MOE_EXL3_ERR_INVALID_ARG;
    if (T == 0)
        return MOE_EXL3_OK;
    size_t need = 0;
    rc = moe_exl3_workspace_size(desc, T, &need);
    if (rc)
        return rc;
    if (need > (size_t)MOE_EXL3_SCRATCH_BYTES)
        return MOE_EXL3_ERR_WORKSPACE;
    void *ws = nullptr;
    rc = scratch_of_current_device(&ws);
    if (rc)
        return rc;
    return run_layer(desc, weights, x, T, out, ws, (size_t)MOE_EXL3_SCRATCH_BYTES, stream, nullptr);
}

int moe_exl3_layer_profiled(const moe_exl3_desc *desc, const moe_exl3_weights *weights,
                            const void *x, int64_t T, void *out, void *workspace, size_t ws_bytes,
                            void *stream, void *const *events, int n_events)
{
    if (!events || n_events != MOE_EXL3_STEP_END + 1)
        return MOE_EXL3_ERR_INVALID_ARG;
    for (int i = 0; i < n_events; ++i)
        if (!events[i])
            return MOE_EXL3_ERR_INVALID_ARG;
    return run_layer(desc, weights, x, T, out, workspace, ws_bytes, stream, events);
}


int moe_exl3_decode(const uint16_t *codes, int32_t n_in, int32_t n_out, int32_t K, uint32_t mcg,
                    int32_t codebook, void *dst, int32_t dst_dtype, void *stream)
{
    if (!codes || !dst || n_in <= 0 || n_out <= 0 || n_in % 16 || n_out % 16)
        return MOE_EXL3_ERR_INVALID_ARG;
    if (K < 2 || K > 4 || (codebook != MOE_EXL3_CB_MCG && codebook != MOE_EXL3_CB_MCG_E4M3) ||
        dst_dtype < MOE_EXL3_DT_F32 || dst_dtype > MOE_EXL3_DT_MFMA_BIASED_F16 ||
        (dst_dtype == MOE_EXL3_DT_MFMA_BIASED_F16 && codebook != MOE_EXL3_CB_MCG))
        return MOE_EXL3_ERR_UNSUPPORTED;
    if (!aligned16(codes) || !aligned16(dst))
        return MOE_EXL3_ERR_MISALIGNED;
    if (launch_decode(codes, n_in, n_out, K, mcg, codebook, dst, dst_dtype, (hipStream_t)stream) != hipSuccess)
        return MOE_EXL3_ERR_HIP;
    return MOE_EXL3_OK;
}

int moe_exl3_repack(const uint16_t *src, uint16_t *dst, int32_t count, int32_t n_in, int32_t n_out, int32_t K,
                    int32_t src_order, void *stream)
{
    if (!src || !dst || count < 1 || n_in <= 0 || n_out <= 0 || n_in % 16 || n_out % 16)
        return MOE_EXL3_ERR_INVALID_ARG;
    if (K < 2 || K > 4 || src_order < MOE_EXL3_ORDER_ROWMAJOR || src_order > MOE_EXL3_ORDER_COLGROUPS128 ||
        (src_order == MOE_EXL3_ORDER_COLGROUPS128 && n_out % 128))
        return MOE_EXL3_ERR_UNSUPPORTED;
    if (!aligned16(src) || !aligned16(dst))
        return MOE_EXL3_ERR_MISALIGNED;
    const int64_t bytes = (int64_t)count * (n_in / 16) * (n_out / 16) * 32 * K;
    if ((const char *)dst < (const char *)src + bytes && (const char *)src < (const char *)dst + bytes)
        return MOE_EXL3_ERR_INVALID_ARG;
    if (launch_repack(src, dst, count, n_in, n_out, K, src_order, (hipStream_t)stream) != hipSuccess)
        return MOE_EXL3_ERR_HIP;
    return MOE_EXL3_OK;
}

int moe_exl3_expand_block_scales(const uint16_t *block, int32_t n_trellis, int32_t hidden, int32_t inter,
                                 uint16_t *const *suh, uint16_t *const *svh, void *stream)
{
    if (!block || !suh || !svh || n_trellis < 1 || hidden <= 0 || hidden % 128 || inter <= 0)
        return MOE_EXL3_ERR_INVALID_ARG;
    if (!aligned16(block))
        return MOE_EXL3_ERR_MISALIGNED;
    for (int p = 0; p < 3; ++p) {
        if (!suh[p] || !svh[p])
            return MOE_EXL3_ERR_INVALID_ARG;
        if (!aligned16(suh[p]) || !aligned16(svh[p]))
            return MOE_EXL3_ERR_MISALIGNED;
    }
    if (launch_expand_scales(block, n_trellis, hidden, inter, suh, svh, (hipStream_t)stream) != hipSuccess)
        return MOE_EXL3_ERR_HIP;
    return MOE_EXL3_OK;
}

}  // extern "C"
