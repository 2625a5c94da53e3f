// Host-layer driver for the AddressSanitizer build of the library (host code
// only; no GPU and no kernel launch). It walks every entry point through its
// argument checks and, with the allocation cap set to 0, through the
// allocation-failure paths of plan creation and the CSR build, so that the
// sanitizer sees the host code that validates, creates and tears down plans.
// Exit status 0 and "host layer ok" on success.
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "gnn_attn.h"
#include "gnn_reduce.h"
#include "gnn_reorder.h"
#include "gnn_spmm.h"

#define CHECK(cond)                                                            \
    do {                                                                       \
        if (!(cond)) {                                                         \
            std::fprintf(stderr, "FAIL %s:%d: %s\n", __FILE__, __LINE__, #cond); \
            return 1;                                                          \
        }                                                                      \
    } while (0)

int main() {
    // aligned fake device addresses: never dereferenced on these paths
    void *A = reinterpret_cast<void *>(0x10000);
    const int32_t *I = static_cast<const int32_t *>(A);
    int32_t *Iw = static_cast<int32_t *>(A);
    const char *c = reinterpret_cast<const char *>(A);
    for (int s = -8; s <= 1; ++s) CHECK(std::strlen(gnn_status_string(s)) > 0);
    CHECK(std::strlen(gnn_status_string(99)) > 0);

    // attention calls
    CHECK(gnn_attn_fwd(nullptr, I, I, 10, 20, 2, 24, A, A, A, A, nullptr, 0.f, GNN_F32, nullptr) == GNN_ERR_UNSUPPORTED);
    CHECK(gnn_attn_fwd(nullptr, I, I, -1, 20, 2, 32, A, A, A, A, nullptr, 0.f, GNN_F32, nullptr) == GNN_ERR_INVALID_ARG);
    CHECK(gnn_attn_fwd(nullptr, I, I, 10, 20, 2, 32, c + 4, A, A, A, nullptr, 0.f, GNN_F32, nullptr) ==
          GNN_ERR_ALIGNMENT);
    CHECK(gnn_attn_fwd(nullptr, I, I, 0, 0, 2, 32, A, A, A, A, nullptr, 0.f, GNN_F32, nullptr) == GNN_OK);
    CHECK(gnn_attn_fwd_noalloc(nullptr, I, I, 10, 20, 2, 32, nullptr, A, A, A, nullptr, 0.f, GNN_F32, nullptr) ==
          GNN_ERR_INVALID_ARG);
    CHECK(gnn_attn_fwd_noalloc(nullptr, I, I, 10, 20, 2, 32, A, A, A, (void *)(c + 8), nullptr, 0.f, GNN_BF16,
                               nullptr) == GNN_ERR_ALIGNMENT);
    CHECK(gnn_attn_fwd_noalloc(nullptr, I, I, 0, 0, 2, 32, A, A, A, A, nullptr, 0.f, GNN_F32, nullptr) == GNN_OK);
    CHECK(gatv2_attn_fwd(nullptr, I, I, 10, 20, 2, 32, A, A, A, nullptr, 0.2f, A, nullptr, GNN_F32, nullptr) ==
          GNN_ERR_INVALID_ARG);
    CHECK(gnn_attn_bwd(nullptr, I, I, 10, 20, 2, 32, A, A, A, A, A, (const float *)A, A, A, A, 0.f, GNN_F32,
                       nullptr) == GNN_ERR_INVALID_ARG);
    CHECK(gatv2_attn_bwd(nullptr, I, I, 10, 20, 2, 32, A, A, A, (const float *)A, 0.2f, A, (const float *)A, A, A,
                         nullptr, (float *)A, GNN_F32, nullptr) == GNN_ERR_INVALID_ARG);
    // reduction, reordering, SpMM
    CHECK(gnn_reduce_fwd(nullptr, I, I, 10, 20, 6, A, A, Iw, GNN_REDUCE_MAX, GNN_MSG_SRC, GNN_F32, nullptr) ==
          GNN_ERR_UNSUPPORTED);
    CHECK(gnn_reduce_bwd(nullptr, I, I, 10, 20, 8, A, I, A, GNN_MSG_SRC, GNN_F32, nullptr) == GNN_ERR_INVALID_ARG);
    CHECK(gnn_reorder(I, I, 10, 20, (gnn_order_t)2, Iw, nullptr) == GNN_ERR_INVALID_ARG);
    CHECK(gnn_permute_graph(I, I, 10, 20, nullptr, Iw, Iw, nullptr) == GNN_ERR_INVALID_ARG);
    CHECK(gnn_permute_rows(A, (void *)(c + 16), 10, 24, I, 0, nullptr) == GNN_ERR_UNSUPPORTED);
    CHECK(gnn_spmm_prepare(nullptr, GNN_NORM_GCN, nullptr) == GNN_ERR_INVALID_ARG);
    CHECK(gnn_spmm(nullptr, I, I, 10, 20, 8, A, A, 0, GNN_F32, nullptr) == GNN_ERR_INVALID_ARG);

    // plans: options and arguments
    gnn_plan_opts o;
    CHECK(gnn_plan_opts_default(&o) == GNN_OK && o.light_threshold == 512 && o.waves_per_group == 4);
    CHECK(gnn_plan_opts_default(nullptr) == GNN_ERR_INVALID_ARG);
    gnn_plan_t h = nullptr;
    CHECK(gnn_plan_create(nullptr, I, 10, 20, nullptr, nullptr, &h) == GNN_ERR_INVALID_ARG);
    o.waves_per_group = 3;
    CHECK(gnn_plan_create(I, I, 10, 20, &o, nullptr, &h) == GNN_ERR_INVALID_ARG);
    CHECK(gnn_plan_export(nullptr, nullptr) == GNN_ERR_INVALID_ARG);
    CHECK(gnn_plan_destroy(nullptr) == GNN_ERR_INVALID_ARG);
    CHECK(gnn_plan_set_timing(nullptr, 1) == GNN_ERR_INVALID_ARG);
    int32_t n = 0;
    CHECK(gnn_plan_timing_read(nullptr, 0, nullptr, nullptr, nullptr, &n) == GNN_ERR_INVALID_ARG);

    // allocation failure: with the cap at 0 every device allocation is refused
    // before hipMalloc; plan creation (for every option set) and the CSR
    // build must fail cleanly, free what they built and leave *plan_out alone
    setenv("GNN_ALLOC_CAP_BYTES", "0", 1);
    for (int csc = 0; csc < 2; ++csc) {
        for (float tau : {0.0f, 0.75f}) {
            gnn_plan_opts_default(&o);
            o.want_csc = csc;
            o.tile_density = tau;
            h = nullptr;
            CHECK(gnn_plan_create(I, I, 10, 20, &o, nullptr, &h) == GNN_ERR_OOM);
            CHECK(h == nullptr);
            CHECK(std::strstr(gnn_status_string(GNN_ERR_OOM), "GNN_ALLOC_CAP_BYTES") != nullptr);
        }
    }
    int64_t e = 0;
    CHECK(gnn_csr_build(I, I, 5, 3, 1, Iw, Iw, 10, &e, nullptr) == GNN_ERR_OOM);
    unsetenv("GNN_ALLOC_CAP_BYTES");
    std::printf("host layer ok\n");
    return 0;
}
