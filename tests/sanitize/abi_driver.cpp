// Calls every C-ABI entry point with arguments its host-side checks must
// reject (no launch, no device touched), for an AddressSanitizer /
// UndefinedBehaviorSanitizer build of the host code (test infrastructure).
// The kernel launchers are replaced by stubs that abort: reaching one fails.
#include <stdio.h>
#include <stdlib.h>

#include "moe_exl3.h"

#define CHECK(c) do { if (!(c)) { fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); return 1; } } while (0)

int main()
{
    moe_exl3_desc d = {4096, 2048, 288, 8, 2, MOE_EXL3_CB_MCG, 0x9E3779B1u, MOE_EXL3_DT_BF16,
                       MOE_EXL3_HAS_SHARED | MOE_EXL3_HAS_ROUTER_BIAS, 0};
    size_t bytes = 0;
    CHECK(moe_exl3_workspace_size(&d, 7168, &bytes) == MOE_EXL3_OK && bytes > 0);
    CHECK(moe_exl3_workspace_size(&d, -1, &bytes) == MOE_EXL3_ERR_INVALID_ARG);
    CHECK(moe_exl3_workspace_size(nullptr, 8, &bytes) == MOE_EXL3_ERR_INVALID_ARG);
    CHECK(moe_exl3_workspace_size(&d, (int64_t)1 << 40, &bytes) == MOE_EXL3_ERR_UNSUPPORTED);
    moe_exl3_desc bad = d;
    bad.hidden = 100;
    CHECK(moe_exl3_workspace_size(&bad, 8, &bytes) == MOE_EXL3_ERR_INVALID_ARG);
    bad = d;
    bad.K = 5;
    CHECK(moe_exl3_workspace_size(&bad, 8, &bytes) == MOE_EXL3_ERR_UNSUPPORTED);
    bad = d;
    bad.flags |= MOE_EXL3_FP8_MFMA;
    CHECK(moe_exl3_workspace_size(&bad, 8, &bytes) == MOE_EXL3_ERR_UNSUPPORTED);
    bad = d;
    bad.flags |= MOE_EXL3_SHARED_TRELLIS;
    bad.n_experts = 1024;
    CHECK(moe_exl3_workspace_size(&bad, 8, &bytes) == MOE_EXL3_ERR_UNSUPPORTED);
    for (uint32_t f = 0; f < (1u << 10); f += 7) {
        moe_exl3_desc v = d;
        v.flags = f;
        size_t b = 0;
        const int rc = moe_exl3_workspace_size(&v, 300, &b);
        CHECK(rc == MOE_EXL3_OK || rc == MOE_EXL3_ERR_INVALID_ARG || rc == MOE_EXL3_ERR_UNSUPPORTED);
    }

    // the layer: every rejection path before the first launch
    moe_exl3_weights w = {};
    alignas(256) static unsigned char fake[4096];
    // the host checks compare and align-check addresses but never dereference
    // device pointers: x and out are distinct aligned addresses far apart
    const void *x = (const void *)(uintptr_t)0x10000000u;
    void *out = (void *)(uintptr_t)0x20000000u;
    CHECK(moe_exl3_layer(&d, nullptr, x, 8, out, fake, sizeof fake, nullptr) == MOE_EXL3_ERR_INVALID_ARG);
    CHECK(moe_exl3_layer(&d, &w, x, 8, out, fake, sizeof fake, nullptr) == MOE_EXL3_ERR_INVALID_ARG);
    CHECK(moe_exl3_layer(&d, &w, x, -3, out, fake, sizeof fake, nullptr) == MOE_EXL3_ERR_INVALID_ARG);
    CHECK(moe_exl3_layer(&d, &w, x, 0, out, fake, sizeof fake, nullptr) == MOE_EXL3_OK);
    for (int p = 0; p < 3; ++p) {
        w.codes[p] = (const uint16_t *)fake;
        w.suh[p] = (const uint16_t *)fake;
        w.svh[p] = (const uint16_t *)fake;
        w.shared_w[p] = (const uint16_t *)fake;
    }
    w.router_w = (const uint16_t *)fake;
    w.router_bias = (const float *)fake;
    // misaligned activation, overlapping output, small workspace
    CHECK(moe_exl3_layer(&d, &w, (const char *)x + 2, 8, out, fake, sizeof fake, nullptr) == MOE_EXL3_ERR_MISALIGNED);
    CHECK(moe_exl3_layer(&d, &w, x, 8, (void *)x, fake, sizeof fake, nullptr) == MOE_EXL3_ERR_INVALID_ARG);
    CHECK(moe_exl3_layer(&d, &w, x, 8, out, fake, 16, nullptr) == MOE_EXL3_ERR_WORKSPACE);
    moe_exl3_desc dh = d;
    dh.flags |= MOE_EXL3_HADAMARD;
    CHECK(moe_exl3_layer(&dh, &w, x, 8, out, fake, sizeof fake, nullptr) == MOE_EXL3_ERR_INVALID_ARG);
    moe_exl3_desc dk = d;
    dk.flags |= MOE_EXL3_PER_TENSOR_K;
    CHECK(moe_exl3_layer(&dk, &w, x, 8, out, fake, sizeof fake, nullptr) == MOE_EXL3_ERR_INVALID_ARG);
    void *ev[MOE_EXL3_STEP_END + 1] = {};
    CHECK(moe_exl3_layer_profiled(&d, &w, x, 8, out, fake, sizeof fake, nullptr, ev, 3) ==
          MOE_EXL3_ERR_INVALID_ARG);
    CHECK(moe_exl3_layer_profiled(&d, &w, x, 8, out, fake, sizeof fake, nullptr, ev, MOE_EXL3_STEP_END + 1) ==
          MOE_EXL3_ERR_INVALID_ARG);

    // routing, decode, repack, block scales
    int32_t *idx = (int32_t *)(fake + 2048);
    CHECK(moe_exl3_route(&d, &w, x, 8, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, fake, sizeof fake,
                         nullptr) == MOE_EXL3_ERR_INVALID_ARG);
    CHECK(moe_exl3_route(&d, &w, x, 8, idx, nullptr, nullptr, nullptr, nullptr, nullptr, fake, 16, nullptr) ==
          MOE_EXL3_ERR_WORKSPACE);
    const uint16_t *c = (const uint16_t *)fake;
    CHECK(moe_exl3_decode(c, 15, 16, 2, 1u, 0, out, MOE_EXL3_DT_F32, nullptr) == MOE_EXL3_ERR_INVALID_ARG);
    CHECK(moe_exl3_decode(c, 16, 16, 5, 1u, 0, out, MOE_EXL3_DT_F32, nullptr) == MOE_EXL3_ERR_UNSUPPORTED);
    CHECK(moe_exl3_decode(c, 16, 16, 2, 1u, 0, out, 9, nullptr) == MOE_EXL3_ERR_UNSUPPORTED);
    CHECK(moe_exl3_decode(c, 16, 16, 2, 1u, 1, out, MOE_EXL3_DT_MFMA_BIASED_F16, nullptr) == MOE_EXL3_ERR_UNSUPPORTED);
    CHECK(moe_exl3_decode(c, 16, 16, 2, 1u, 0, (char *)out + 1, MOE_EXL3_DT_F32, nullptr) == MOE_EXL3_ERR_MISALIGNED);
    uint16_t *dst = (uint16_t *)(fake + 2048);
    CHECK(moe_exl3_repack(c, dst, 0, 16, 16, 2, 0, nullptr) == MOE_EXL3_ERR_INVALID_ARG);
    CHECK(moe_exl3_repack(c, dst, 1, 16, 16, 2, 7, nullptr) == MOE_EXL3_ERR_UNSUPPORTED);
    CHECK(moe_exl3_repack(c, dst, 1, 16, 48, 2, MOE_EXL3_ORDER_COLGROUPS128, nullptr) == MOE_EXL3_ERR_UNSUPPORTED);
    CHECK(moe_exl3_repack(c, (uint16_t *)c, 1, 16, 16, 2, 0, nullptr) == MOE_EXL3_ERR_INVALID_ARG);
    uint16_t *sv[3] = {dst, dst, nullptr};
    CHECK(moe_exl3_expand_block_scales(c, 1, 128, 128, sv, sv, nullptr) == MOE_EXL3_ERR_INVALID_ARG);
    CHECK(moe_exl3_expand_block_scales(c, 1, 100, 128, sv, sv, nullptr) == MOE_EXL3_ERR_INVALID_ARG);
    CHECK(moe_exl3_version() == MOE_EXL3_ABI_VERSION);
    for (int code = -6; code <= 1; ++code)
        CHECK(moe_exl3_strerror(code) != nullptr);
    printf("abi driver: ok\n");
    return 0;
}
