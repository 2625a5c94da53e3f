// Host-side internals shared by the library's translation units.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "../../include/gnn_attn.h"

namespace gnn {

// Remember the last HIP failure for gnn_status_string.
void set_hip_error(hipError_t e, const char *what);

#define GNN_HIP(call)                                   \
    do {                                                \
        hipError_t e_ = (call);                         \
        if (e_ != hipSuccess) {                         \
            ::gnn::set_hip_error(e_, #call);            \
            return e_ == hipErrorOutOfMemory ? GNN_ERR_OOM : GNN_ERR_HIP; \
        }                                               \
    } while (0)

#define GNN_TRY(expr)                 \
    do {                              \
        int s_ = (expr);              \
        if (s_ != GNN_OK) return s_;  \
    } while (0)

// Device buffer with size accounting.
struct DevBuf {
    void *p = nullptr;
    size_t bytes = 0;
};

int dev_alloc(DevBuf &b, size_t bytes);
void dev_free(DevBuf &b);

template <class T>
T *as(const DevBuf &b) { return reinterpret_cast<T *>(b.p); }

// Degree buckets of one CSR-like structure (in-degree over the CSR, or
// out-degree over the transposed adjacency).
struct Buckets {
    int32_t n_light = 0, n_heavy = 0, n_groups = 0;
    DevBuf light, heavy, groups, partial_ofs;
};

// Per-kernel timing log.
struct TimingRec {
    int kind;
    hipEvent_t a, b;
};

enum KernelKind {
    K_FWD_MAIN = 0,
    K_FWD_MERGE,
    K_GAT_MAIN,
    K_GAT_MERGE,
    K_BWD_DST_MAIN,
    K_BWD_DST_MERGE,
    K_BWD_SRC_MAIN,
    K_BWD_SRC_MERGE,
    K_TILE_FWD,
    K_TILE_BWD,
    K_NUM_KINDS
};
extern const char *kKernelNames[K_NUM_KINDS];

struct Timer {
    bool enabled = false;
    std::vector<TimingRec> log;
    std::vector<hipEvent_t> pool;
    hipEvent_t get();
    int begin(int kind, hipStream_t s, TimingRec &r);
    int end(TimingRec &r, hipStream_t s);
    ~Timer();
};

}  // namespace gnn

struct gnn_plan_s {
    int32_t n_nodes = 0;
    int64_t n_edges = 0;
    const int32_t *indptr = nullptr, *indices = nullptr;   // caller's arrays (not owned)
    gnn_plan_opts opts{};
    gnn::Buckets fwd;          // in-degree buckets over the CSR
    bool has_csc = false;
    gnn::DevBuf cindptr, cindices;
    gnn::Buckets bwd;          // out-degree buckets over the transposed adjacency
    // tiles
    bool has_tiles = false;
    int32_t n_tiles = 0, tile_min_nnz = 0;
    int64_t n_residual = 0;
    gnn::DevBuf tile_rc, tile_mask, tile_ptr, rindptr, rindices;
    // workspace (heavy partials, backward statistics), grows on demand
    gnn::DevBuf ws;
    int64_t largest_ws = 0;
    gnn::Timer timer;
    int64_t structure_bytes() const;
};

namespace gnn {
// plan workspace of at least `bytes` (kept, grown on demand)
int plan_workspace(gnn_plan_s *p, size_t bytes, hipStream_t s, void **out);

// device-wide exclusive scan of int32 (in may equal out); returns the total in *total_dev (int32 device scalar)
int scan_exclusive(const int32_t *in, int32_t *out, int64_t n, int32_t *total_dev, hipStream_t s);
// LSD radix sort of 64-bit keys on bits [0, bits); result in keys (tmp: same size scratch)
int radix_sort_u64(uint64_t *keys, uint64_t *tmp, int64_t n, int bits, hipStream_t s);
// bucket a CSR-like structure
int build_buckets(const int32_t *indptr, int32_t n, int32_t T, int32_t C, int32_t W, Buckets &b,
                  hipStream_t s);
}  // namespace gnn
