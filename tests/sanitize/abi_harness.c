/*
 * Host harness of the k3moe C ABI's host code (argument checks, workspace
 * planning, pack and cache argument checks), linked against the library's
 * host objects built with AddressSanitizer and UndefinedBehaviorSanitizer.
 * It runs where no GPU is present: every call below must return its status
 * before touching a device (or report K3MOE_EHIP when the only thing left
 * is a device call), and none may read or write outside its arguments.
 * Sizes include the extremes of int32 so that any unchecked overflow in the
 * size arithmetic is reported.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "k3moe.h"

static int g_fail = 0;
#define CHECK(c, msg)                                                         \
    do {                                                                      \
        if (!(c)) {                                                           \
            fprintf(stderr, "FAIL %s:%d: %s\n", __FILE__, __LINE__, msg);     \
            ++g_fail;                                                         \
        }                                                                     \
    } while (0)

static k3moe_config cfg(int32_t d, int32_t E, int32_t k, int32_t f, int32_t T, uint32_t flags)
{
    k3moe_config c = {d, E, k, f, T, flags};
    return c;
}

int main(void)
{
    for (int s = -6; s <= 2; ++s)
        CHECK(k3moe_status_str(s) != NULL && k3moe_status_str(s)[0] != 0, "status string");

    /* workspace planning over valid, malformed and extreme configs */
    const int32_t big = 2147483647;
    const k3moe_config cases[] = {
        cfg(128, 8, 2, 256, 1, 0),       cfg(7168, 896, 16, 2048, 4096, 0),
        cfg(7168, 896, 16, 2048, 32768, 0), cfg(7168, 896, 16, 2048, 32769, 0),
        cfg(100, 8, 2, 256, 1, 0),       cfg(128, 8, 9, 256, 1, 0),
        cfg(128, 8, 2, 256, 0, 0),       cfg(128, 8, 2, 256, 1, 2),
        cfg(big, 8, 2, 256, 1, 0),       cfg(128, big, 2, 256, 1, 0),
        cfg(128, 8, 2, big, 1, 0),       cfg(128, 4096, 64, 4096, big, 0),
        cfg(8192, 4096, 64, 4096, 1 << 12, 0), cfg(-128, 8, 2, 256, 1, 0),
        cfg(128, -8, 2, 256, 1, 0),      cfg(128, 8, -2, 256, 1, 0),
        cfg(128, 8, 2, 256, 1, K3MOE_FLAG_BIAS_SELECT_ONLY), cfg(128, 8, 2, 256, 1, 0x80000001u),
    };
    const int64_t want_ok[] = {1, 1, 1, 0, 0, 0, 0, 0, 0, 0, 0, 0, 1, 0, 0, 0, 1, 0};
    for (size_t i = 0; i < sizeof(cases) / sizeof(cases[0]); ++i) {
        const int64_t n = k3moe_workspace_bytes(&cases[i]);
        CHECK(want_ok[i] ? n > 0 : n < 0, "workspace_bytes validation");
    }
    CHECK(k3moe_workspace_bytes(NULL) < 0, "workspace_bytes(NULL)");

    /* tiled scale sizes, including overflow-sized shapes */
    CHECK(k3moe_tiled_scale_bytes(1, 16, 128) == 256, "tiled scale bytes");
    CHECK(k3moe_tiled_scale_bytes(896, 2048, 7168) > 0, "tiled scale bytes, K3 gate");
    CHECK(k3moe_tiled_scale_bytes(0, 16, 128) == 0, "tiled scale bytes, n = 0");
    CHECK(k3moe_tiled_scale_bytes(1, 15, 128) == 0, "tiled scale bytes, R % 16");
    CHECK(k3moe_tiled_scale_bytes(1, 16, 100) == 0, "tiled scale bytes, K % 128");
    (void)k3moe_tiled_scale_bytes(big, big - 15, big - 127);

    /* pack: argument checks before any device call */
    static uint8_t buf[4096] __attribute__((aligned(16)));
    uint8_t *p = buf, *mis = buf + 1;
    CHECK(k3moe_pack_mxfp4(NULL, p, 1, 16, 128, p, p, NULL) == K3MOE_EINVAL, "pack NULL");
    CHECK(k3moe_pack_mxfp4(mis, p, 1, 16, 128, p, p, NULL) == K3MOE_EINVAL, "pack misaligned");
    CHECK(k3moe_pack_mxfp4(p, p, 1, 15, 128, p, p, NULL) == K3MOE_EINVAL, "pack R % 16");
    CHECK(k3moe_pack_mxfp4(p, p, 0, 16, 128, p, p, NULL) == K3MOE_EINVAL, "pack n = 0");
    CHECK(k3moe_pack_mxfp4(p, p, 1, 16, -128, p, p, NULL) == K3MOE_EINVAL, "pack K < 0");

    /* create: argument checks, then a device call that fails without a GPU */
    k3moe_weights w = {(const float *)p, NULL, p, p, p, p, p, p};
    k3moe_weights wmis = w;
    wmis.up_s = mis;
    k3moe_weights wnull = w;
    wnull.down_q = NULL;
    k3moe *h = (k3moe *)(uintptr_t)1;
    const k3moe_config good = cfg(2048, 64, 8, 1024, 8, 0);
    const k3moe_config bad = cfg(2048, 64, 80, 1024, 8, 0);
    CHECK(k3moe_create(&good, &w, 0, NULL) == K3MOE_EINVAL, "create out NULL");
    CHECK(k3moe_create(NULL, &w, 0, &h) == K3MOE_EINVAL && h == NULL, "create cfg NULL");
    CHECK(k3moe_create(&bad, &w, 0, &h) == K3MOE_EINVAL, "create bad cfg");
    CHECK(k3moe_create(&good, &wmis, 0, &h) == K3MOE_EINVAL, "create misaligned weights");
    CHECK(k3moe_create(&good, &wnull, 0, &h) == K3MOE_EINVAL, "create NULL weights");
    const int rc = k3moe_create(&good, &w, 0, &h);
    CHECK((rc == K3MOE_EHIP || rc == K3MOE_EINVAL) && h == NULL, "create without a GPU");
    k3moe_destroy(NULL);

    /* entry points on a NULL handle */
    CHECK(k3moe_layer_forward(NULL, p, 1, (float *)p, NULL, NULL, NULL) == K3MOE_EINVAL, "forward NULL");
    CHECK(k3moe_route(NULL, p, 1, NULL, (int32_t *)p, (float *)p, NULL) == K3MOE_EINVAL, "route NULL");
    CHECK(k3moe_group(NULL, (int32_t *)p, 1, (int32_t *)p, (int32_t *)p, (int32_t *)p, NULL) == K3MOE_EINVAL,
          "group NULL");
    CHECK(k3moe_experts_forward(NULL, p, 1, (int32_t *)p, (float *)p, (float *)p, NULL) == K3MOE_EINVAL,
          "experts NULL");
    CHECK(k3moe_profile_begin(NULL, 4) == K3MOE_EINVAL, "profile_begin NULL");
    CHECK(k3moe_profile_begin_stages(NULL, 4, 1u << K3MOE_STAGE_GATEUP) == K3MOE_EINVAL,
          "profile_begin_stages NULL");
    float ms[K3MOE_NUM_STAGES];
    int32_t launches[K3MOE_NUM_STAGES];
    CHECK(k3moe_profile_end(NULL, ms, launches) == K3MOE_EINVAL, "profile_end NULL");

    /* the no-allocation forward: everything is checked on the host first */
    CHECK(k3moe_layer_forward_noalloc(NULL, &w, p, 1, (float *)p, NULL, NULL, NULL) == K3MOE_EINVAL,
          "noalloc cfg NULL");
    CHECK(k3moe_layer_forward_noalloc(&good, &w, p, 9, (float *)p, NULL, NULL, NULL) == K3MOE_EINVAL,
          "noalloc T > max");
    CHECK(k3moe_layer_forward_noalloc(&good, &w, p, 5, (float *)p, NULL, NULL, NULL) ==
              K3MOE_EUNSUPPORTED, "noalloc T > 4");
    CHECK(k3moe_layer_forward_noalloc(&good, &w, p, 1, (float *)p, (int32_t *)p, NULL, NULL) ==
              K3MOE_EINVAL, "noalloc idx without gate");
    const k3moe_config wide = cfg(4096, 4096, 64, 4096, 4, 0);
    CHECK(k3moe_layer_forward_noalloc(&wide, &w, p, 4, (float *)p, NULL, NULL, NULL) ==
              K3MOE_EUNSUPPORTED, "noalloc beyond its scratch");
    CHECK(k3moe_layer_forward_noalloc(&good, &w, p, 0, (float *)p, NULL, NULL, NULL) == K3MOE_OK,
          "noalloc T = 0");

    /* the expert cache: argument checks, stats and destroy on NULL */
    k3moe_host_weights hw = {(const float *)p, NULL, p, p, p, p, p, p};
    k3moe_cache *c = (k3moe_cache *)(uintptr_t)1;
    CHECK(k3moe_cache_create(&good, NULL, 16, 0, &c) == K3MOE_EINVAL && c == NULL, "cache weights NULL");
    CHECK(k3moe_cache_create(&good, &hw, 7, 0, &c) == K3MOE_EINVAL, "cache slots < k");
    CHECK(k3moe_cache_create(&good, &hw, 65, 0, &c) == K3MOE_EINVAL, "cache slots > E");
    CHECK(k3moe_cache_create(&bad, &hw, 16, 0, &c) == K3MOE_EINVAL, "cache bad cfg");
    int64_t a, b2, c2, d2;
    CHECK(k3moe_cache_stats(NULL, &a, &b2, &c2, &d2) == K3MOE_EINVAL, "cache stats NULL");
    CHECK(k3moe_cache_prefetch_stats(NULL, &a, &b2) == K3MOE_EINVAL, "prefetch stats NULL");
    CHECK(k3moe_cache_forward(NULL, p, 1, (float *)p, NULL, NULL, NULL) == K3MOE_EINVAL, "cache forward NULL");
    int32_t ids[2] = {0, 1};
    CHECK(k3moe_cache_prefetch(NULL, ids, 2, NULL) == K3MOE_EINVAL, "prefetch NULL");
    CHECK(k3moe_cache_create_ex(&good, &hw, 16, 0, 2u, &c) == K3MOE_EINVAL && c == NULL,
          "cache unknown flags");
    CHECK(k3moe_cache_create_ex(&good, NULL, 16, 0, K3MOE_CACHE_DEVICE_PLAN, &c) == K3MOE_EINVAL,
          "device-planned cache weights NULL");
    CHECK(k3moe_cache_prefetch_device(NULL, ids, 2, NULL) == K3MOE_EINVAL, "device prefetch NULL");
    CHECK(k3moe_cache_device_counters(NULL, &a, &b2) == K3MOE_EINVAL, "device counters NULL");
    k3moe_cache_destroy(NULL);

    if (g_fail) {
        fprintf(stderr, "%d checks failed\n", g_fail);
        return 1;
    }
    printf("abi harness: all checks passed\n");
    return 0;
}
