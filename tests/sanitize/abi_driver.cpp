// Drives the C ABI's host-side paths -- argument validation, workspace sizing, ring set-up
// and the chunk-aware growth schedule -- for a host build of the library with
// AddressSanitizer and UndefinedBehaviorSanitizer.  Every compute call here is rejected
// by validation before anything is enqueued, so no GPU is needed and no device pointer is
// dereferenced (FAKE is never touched).
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "hf.h"

static int failures = 0;
#define EXPECT(cond)                                                      \
    do {                                                                  \
        if (!(cond)) {                                                    \
            std::fprintf(stderr, "abi driver: line %d: %s\n", __LINE__, #cond); \
            ++failures;                                                   \
        }                                                                 \
    } while (0)

int main() {
    void *const FAKE = reinterpret_cast<void *>(0x10000);
    EXPECT(hf_abi_version() == HF_ABI_VERSION);
    for (int s = 0; s <= 7; ++s) EXPECT(hf_status_str(static_cast<hf_status>(s)) != nullptr);

    hf_dims d{1, 12, 128, 1560, 3, 6, 64, 64};
    size_t ws = 0, ws2 = 0, bws = 0;
    EXPECT(hf_workspace_size(&d, 37, &ws) == HF_OK && ws > 0);
    EXPECT(hf_workspace_size(&d, 147, &ws2) == HF_OK && ws2 >= ws);
    EXPECT(hf_workspace_size(nullptr, 37, &ws2) == HF_ERR_NULL);
    EXPECT(hf_backward_workspace_size(&d, 37, &bws) == HF_OK && bws > 0);
    const hf_dims bad[] = {{1, 12, 96, 1560, 3, 6, 64, 64}, {1, 12, 128, 1561, 3, 6, 64, 64},
                           {1, 12, 128, 1560, 3, 2, 64, 64}, {0, 12, 128, 1560, 3, 6, 64, 64},
                           {1, 12, 128, 1560, 3, 6, 48, 64}, {1, 12, 128, 1560, 3, 6, 64, 24}};
    for (const hf_dims &b : bad) EXPECT(hf_workspace_size(&b, 1, &ws2) != HF_OK && std::strlen(hf_last_error()) > 0);

    hf_kv_ring ring{};
    EXPECT(hf_ring_init(&d, FAKE, FAKE, &ring) == HF_OK && ring.head == 0 && ring.n_committed == 0);
    EXPECT(hf_ring_init(&d, nullptr, FAKE, &ring) == HF_ERR_NULL);
    ring.n_committed = 3;

    // selection: top_k out of range, ring state out of range, workspace too small
    int32_t *const idx = static_cast<int32_t *>(FAKE);
    EXPECT(hf_block_select(&d, FAKE, &ring, 0, idx, nullptr, FAKE, ws, nullptr) == HF_ERR_SHAPE);
    EXPECT(hf_block_select(&d, FAKE, &ring, 148, idx, nullptr, FAKE, ws, nullptr) == HF_ERR_SHAPE);
    EXPECT(hf_block_select(&d, FAKE, &ring, 37, idx, nullptr, FAKE, ws - 1, nullptr) == HF_ERR_WORKSPACE);
    EXPECT(hf_block_select(&d, nullptr, &ring, 37, idx, nullptr, FAKE, ws, nullptr) == HF_ERR_NULL);
    hf_kv_ring bad_ring = ring;
    bad_ring.head = 6;
    EXPECT(hf_block_select(&d, FAKE, &bad_ring, 37, idx, nullptr, FAKE, ws, nullptr) == HF_ERR_RING_STATE);
    bad_ring = ring;
    bad_ring.n_committed = 4;
    EXPECT(hf_block_select(&d, FAKE, &bad_ring, 37, idx, nullptr, FAKE, ws, nullptr) == HF_ERR_RING_STATE);
    EXPECT(hf_block_select_hier(&d, FAKE, &ring, 0, 37, idx, nullptr, nullptr, nullptr, FAKE, ws, nullptr) != HF_OK);

    float *const fp = static_cast<float *>(FAKE);
    EXPECT(hf_sparse_window_attn(&d, FAKE, &ring, idx, 0, fp, fp, 1e-6f, fp, FAKE, ws, nullptr) == HF_ERR_SHAPE);
    EXPECT(hf_sparse_window_attn(&d, FAKE, &ring, idx, 37, fp, nullptr, 1e-6f, fp, FAKE, ws, nullptr) != HF_OK);
    EXPECT(hf_sparse_window_attn_lse(&d, FAKE, &ring, idx, 37, fp, fp, 1e-6f, fp, nullptr, FAKE, ws, nullptr) == HF_ERR_NULL);
    const hf_rope bad_rope{24, 3, 10000.f};
    EXPECT(hf_sparse_window_attn_rope(&d, FAKE, &ring, idx, 37, fp, fp, 1e-6f, &bad_rope, fp, FAKE, ws, nullptr) != HF_OK);
    EXPECT(hf_linear_absorb(&d, FAKE, FAKE, -1, fp, fp, FAKE, ws, nullptr) != HF_OK);
    EXPECT(hf_hybrid_step(&d, FAKE, FAKE, FAKE, &ring, 37, 1u, fp, fp, 1e-6f, idx, fp, FAKE, ws - 1, nullptr, nullptr) ==
           HF_ERR_WORKSPACE);
    EXPECT(hf_hybrid_step(&d, nullptr, FAKE, FAKE, &ring, 37, 1u, fp, fp, 1e-6f, idx, fp, FAKE, ws, nullptr, nullptr) ==
           HF_ERR_NULL);
    EXPECT(hf_hybrid_step_rope(&d, FAKE, FAKE, FAKE, &ring, 37, 1u, fp, fp, 1e-6f, &bad_rope, idx, fp, FAKE, ws, nullptr,
                               nullptr) != HF_OK);
    hf_dims big = d;
    big.B = 8;
    big.H = 16;
    EXPECT(hf_hybrid_step_noalloc(&big, FAKE, FAKE, FAKE, &ring, 37, 1u, fp, fp, 1e-6f, idx, fp, nullptr, nullptr) ==
           HF_ERR_UNSUPPORTED);
    EXPECT(hf_hybrid_attn_backward(&d, FAKE, &ring, idx, 37, fp, fp, 1e-6f, fp, fp, fp, fp, fp, fp, fp, fp, FAKE,
                                   bws - 1, nullptr) == HF_ERR_WORKSPACE);
    EXPECT(hf_linear_absorb_backward(&d, FAKE, FAKE, -1, fp, fp, fp, fp, FAKE, bws, nullptr) != HF_OK);

    // the chunk-aware growth schedule: host arithmetic end to end
    const int32_t nkb[16] = {74, 147, 147, 147, 147, 147, 147, 147, 147, 147, 147, 147, 147, 147, 147, 147};
    int32_t top_k[16];
    double sp[16], beta = -1.0;
    EXPECT(hf_cag_schedule(16, nkb, 0.9, 0.75, 0.95, top_k, sp, &beta) == HF_OK);
    EXPECT(top_k[0] == 74 && beta >= 0.0 && std::isfinite(beta));
    for (int i = 1; i < 16; ++i) EXPECT(top_k[i] >= 1 && top_k[i] <= nkb[i] && sp[i] >= sp[i - 1]);
    EXPECT(hf_cag_schedule(0, nkb, 0.9, 0.75, 0.95, top_k, sp, &beta) != HF_OK);
    EXPECT(hf_cag_schedule(16, nkb, 0.9, 1.5, 0.95, top_k, sp, &beta) != HF_OK);
    EXPECT(hf_cag_schedule(16, nullptr, 0.9, 0.75, 0.95, top_k, sp, &beta) == HF_ERR_NULL);

    if (failures) return 1;
    std::puts("abi driver: ok");
    return 0;
}
