// Drives the C ABI's host logic (validation, dispatch, error messages, the slot allocator)
// under the address and undefined-behaviour sanitizers, against the launcher stand-ins of
// api_stub.cpp. Exits nonzero on the first unexpected status; the sanitizers abort on any
// memory or undefined-behaviour error.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "../../include/mamba1.h"
#include "../../include/mamba2.h"

extern int g_launches;

static int g_fail = 0;
#define EXPECT(cond)                                                              \
    do {                                                                          \
        if (!(cond)) {                                                            \
            std::fprintf(stderr, "%s:%d: expected %s (last error: %s)\n", __FILE__, \
                         __LINE__, #cond, mamba2_last_error());                   \
            g_fail = 1;                                                           \
        }                                                                         \
    } while (0)

int main() {
    // fake device addresses: never dereferenced by the host code or the stubs
    alignas(16) static char arena[1 << 12];
    void *g = arena, *g2 = arena + 256, *g3 = arena + 512;
    const int32_t *ix = reinterpret_cast<const int32_t *>(arena + 1024);
    void *mis = arena + 4;
    mamba2_dims d{128, 64, 128, 8, 4, 128, MAMBA2_BF16, MAMBA2_BF16, MAMBA2_BF16, MAMBA2_BF16};
    mamba2_dims d32 = d;
    d32.state_dtype = MAMBA2_F32;

    EXPECT(mamba2_check_dims(&d) == MAMBA2_OK);
    EXPECT(mamba2_check_dims(nullptr) == MAMBA2_ERR_INVALID_ARG);
    mamba2_dims bad = d;
    bad.ngroups = 3;
    EXPECT(mamba2_check_dims(&bad) == MAMBA2_ERR_INVALID_ARG);
    bad = d;
    bad.act_dtype = 7;
    EXPECT(mamba2_check_dims(&bad) == MAMBA2_ERR_INVALID_ARG);
    EXPECT(mamba2_ssm_slot_bytes(&d) == 2u * 1024 * 1024);
    EXPECT(mamba2_ssm_slot_bytes(&bad) == 0);
    size_t ws = 0;
    EXPECT(mamba2_prefill_workspace_bytes(&d32, 32768, &ws) == MAMBA2_OK && ws > 0);
    EXPECT(mamba2_chunk_scan_workspace_bytes(&d, -1, 1, &ws) == MAMBA2_ERR_INVALID_ARG);

    // decode: valid calls reach the launchers, invalid ones are refused before
    int before = g_launches;
    EXPECT(mamba2_conv1d_update(&d, g, static_cast<const float *>(g2), nullptr, g, g2, 16, ix, 4, nullptr) ==
           MAMBA2_ERR_INVALID_ARG);  // output aliases the input
    EXPECT(mamba2_conv1d_update(&d, g, static_cast<const float *>(g2), nullptr, g3, g2, 16, ix, 4, nullptr) ==
           MAMBA2_OK);
    EXPECT(mamba2_state_update(&d, g, g2, static_cast<const float *>(g3), static_cast<const float *>(g3),
                               static_cast<const float *>(g3), nullptr, g2, g, 16, ix, 4, nullptr) == MAMBA2_OK);
    EXPECT(mamba2_state_update(&d, mis, g2, static_cast<const float *>(g3), static_cast<const float *>(g3),
                               static_cast<const float *>(g3), nullptr, g2, g, 16, ix, 4, nullptr) ==
           MAMBA2_ERR_INVALID_ARG);
    EXPECT(std::strstr(mamba2_last_error(), "aligned") != nullptr);
    EXPECT(mamba2_state_update(&d, g, g2, static_cast<const float *>(g3), static_cast<const float *>(g3),
                               static_cast<const float *>(g3), nullptr, g2, g, -5, ix, 4, nullptr) ==
           MAMBA2_ERR_INVALID_ARG);
    EXPECT(std::strstr(mamba2_last_error(), "num_slots") != nullptr);
    EXPECT(mamba2_state_update_multi(&d, g, g2, static_cast<const float *>(g3), static_cast<const float *>(g3),
                                     static_cast<const float *>(g3), nullptr, g2, g, 16, ix, ix, 4, 3, nullptr) ==
           MAMBA2_OK);
    EXPECT(mamba2_conv1d_update_multi(&d, g, static_cast<const float *>(g2), nullptr, g3, g2, 16, ix,
                                      reinterpret_cast<const int32_t *>(arena + 2), 4, 3, nullptr) ==
           MAMBA2_ERR_INVALID_ARG);  // misaligned destination table
    EXPECT(g_launches > before);

    // prefill: chunk scan with and without a workspace, the fused call, the mixed call
    const float *f = static_cast<const float *>(g3);
    EXPECT(mamba2_conv1d_fwd(&d32, g, f, nullptr, g3, g2, 8, ix, 4, 1000, ix, nullptr, nullptr) == MAMBA2_OK);
    EXPECT(mamba2_chunk_scan_fwd(&d32, g, g2, f, f, f, nullptr, g3, g, 8, ix, 4, 1000, ix, nullptr, nullptr, 0,
                                 nullptr) == MAMBA2_OK);
    EXPECT(mamba2_chunk_scan_fwd(&d32, g, g2, f, f, f, nullptr, g3, g, 8, ix, 0, 5, ix, nullptr, nullptr, 0,
                                 nullptr) == MAMBA2_ERR_INVALID_ARG);
    size_t need = 0;
    EXPECT(mamba2_prefill_workspace_bytes(&d32, 1000, &need) == MAMBA2_OK);
    EXPECT(mamba2_prefill_fwd(&d32, g, g2, nullptr, f, nullptr, f, f, f, nullptr, 1e-5f, 0, g3, g, g2, 8, ix, 4,
                              1000, ix, nullptr, arena + 3072, need, nullptr) == MAMBA2_OK);
    EXPECT(mamba2_prefill_fwd(&d32, g, g2, nullptr, f, nullptr, f, f, f, nullptr, 1e-5f, 0, g3, g, g2, 8, ix, 4,
                              1000, ix, nullptr, arena + 3072, need - 1, nullptr) == MAMBA2_ERR_WORKSPACE);
    EXPECT(mamba2_prefill_fwd(&d32, g, g2, nullptr, f, nullptr, f, f, f, f, 1e-5f, 100, g3, g, g2, 8, ix, 4, 1000,
                              ix, nullptr, arena + 3072, need, nullptr) == MAMBA2_ERR_UNSUPPORTED);
    EXPECT(mamba2_prefill_fwd_noalloc(&d32, g, g2, nullptr, f, nullptr, f, f, f, nullptr, 1e-5f, 0, g3, g, g2, 8,
                                      ix, 4, 1000, ix, nullptr, nullptr) == MAMBA2_OK);
    EXPECT(mamba2_prefill_fwd_noalloc(&d32, g, g2, nullptr, f, nullptr, f, f, f, nullptr, 1e-5f, 0, g3, g, g2, 8,
                                      ix, 4, 1 << 20, ix, nullptr, nullptr) == MAMBA2_ERR_WORKSPACE);
    EXPECT(std::strstr(mamba2_last_error(), "static scratch") != nullptr);
    EXPECT(mamba2_mixed_fwd(&d32, g, g2, nullptr, f, nullptr, f, f, f, g3, g3, g, g2, 8, ix, 4, 1000, ix, nullptr,
                            ix, 16, arena + 3072, need, nullptr) == MAMBA2_OK);
    EXPECT(mamba2_gated_rmsnorm(&d, g, g2, f, 1e-5f, 0, g3, 7, nullptr) == MAMBA2_OK);
    EXPECT(mamba2_gated_rmsnorm(&d, g, g2, f, -1.0f, 0, g3, 7, nullptr) == MAMBA2_ERR_INVALID_ARG);

    // Mamba-1
    mamba1_dims d1{8192, 16, 1, MAMBA2_BF16, MAMBA2_F32, MAMBA2_BF16};
    EXPECT(mamba1_selective_scan_fwd(&d1, g, g2, f, g, g2, f, nullptr, f, 1, g3, g, 4, ix, 4, 100, ix, nullptr,
                                     nullptr) == MAMBA2_OK);
    EXPECT(mamba1_selective_state_update(&d1, g, g2, f, g, g2, f, nullptr, f, 1, g, g2, 4, ix, 4, nullptr) ==
           MAMBA2_ERR_INVALID_ARG);  // y aliases u
    d1.dstate = 32;
    EXPECT(mamba1_selective_state_update(&d1, g, g2, f, g, g2, f, nullptr, f, 1, g3, g2, 4, ix, 4, nullptr) ==
           MAMBA2_ERR_UNSUPPORTED);

    // slot checks
    EXPECT(mamba2_check_slot_indices(ix, 8, 16, reinterpret_cast<uint32_t *>(g3), nullptr) == MAMBA2_OK);
    EXPECT(mamba2_check_slot_indices(ix, -1, 16, reinterpret_cast<uint32_t *>(g3), nullptr) ==
           MAMBA2_ERR_INVALID_ARG);
    EXPECT(mamba2_read_slot_errors(reinterpret_cast<uint32_t *>(g3), 1, nullptr) == MAMBA2_OK);

    // allocator: fill, exhaust, free, double free, out-of-range free, many allocators
    for (int round = 0; round < 3; ++round) {
        mamba2_slots *s = nullptr;
        const int n = 1000 + round;
        EXPECT(mamba2_slots_create(n, &s) == MAMBA2_OK && s);
        std::vector<int32_t> got;
        for (int i = 0; i < n; ++i) {
            int32_t v = -1;
            EXPECT(mamba2_slot_alloc(s, &v) == MAMBA2_OK);
            got.push_back(v);
        }
        int32_t v = -1;
        EXPECT(mamba2_slot_alloc(s, &v) == MAMBA2_ERR_NO_SLOT);
        EXPECT(mamba2_slots_in_use(s) == n);
        for (int i = 0; i < n; i += 2) EXPECT(mamba2_slot_free(s, got[i]) == MAMBA2_OK);
        EXPECT(mamba2_slot_free(s, got[0]) == MAMBA2_ERR_NO_SLOT);
        EXPECT(mamba2_slot_free(s, n) == MAMBA2_ERR_NO_SLOT);
        EXPECT(mamba2_slot_free(s, -1) == MAMBA2_ERR_NO_SLOT);
        EXPECT(mamba2_slots_in_use(s) == n / 2);
        mamba2_slots_destroy(s);
    }
    mamba2_slots *s = reinterpret_cast<mamba2_slots *>(1);
    EXPECT(mamba2_slots_create(0, &s) == MAMBA2_ERR_INVALID_ARG && s == nullptr);
    EXPECT(mamba2_slots_create(5, nullptr) == MAMBA2_ERR_INVALID_ARG);
    EXPECT(mamba2_slot_alloc(nullptr, nullptr) == MAMBA2_ERR_INVALID_ARG);
    mamba2_slots_destroy(nullptr);
    for (int st = -1; st <= 6; ++st) EXPECT(mamba2_status_string(st) != nullptr);
    EXPECT(std::strlen(mamba2_version()) > 0);

    if (!g_fail) std::printf("api driver: ok (%d launches reached)\n", g_launches);
    return g_fail;
}
