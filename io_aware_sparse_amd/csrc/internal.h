// Host-side internals shared by the library's translation units.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "../../include/gnn_attn.h"

namespace gnn {

// Size limits. Edge positions are int32 in the kernels, which add up to one
// chunk group (C * W entries) and two steps of 64 entries to a position inside
// a row; the headroom below keeps every such sum below 2^31.
constexpr int64_t kMaxGroupSpan = 1ll << 20;                 // C * W
constexpr int64_t kMaxEdges = (1ll << 31) - (1ll << 21);     // E

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
    // launch order of the light list, as gnn_plan_opts::sched_order asks (order
    // 0 is a copy of the light list); kernel results do not depend on it
    DevBuf sched;
    // the light list in the packed launch order (descending ceil(degree / 4),
    // ties by ascending id), for kernels that pack several rows per wave
    DevBuf by_degree;
    // light rows of more than kLongRow entries; in the packed order they are
    // the first n_long entries of by_degree
    int32_t n_long = 0;
};

// The forward's heavy rows cut at the boundaries of 8 equal source-id ranges
// and then into groups of at most C entries, each streamed by one wave:
// every group reads sources of one range only. Launch slot i*8 + r holds the
// i-th group of range r (-1 when range r has fewer); the kernels give block b
// the slots of range b % 8, and blocks are dealt to the 8 XCDs round-robin,
// so each XCD gathers from one eighth of the table and its L2 holds much more
// of what it reads. Partial slots stay per node and contiguous (partial_ofs),
// so the merge is unchanged.
struct XSplit {
    int32_t n_groups = 0, n_slots = 0;
    DevBuf groups, partial_ofs, order;
};
// the forward uses the split groups when one range's gathered rows take at most this
constexpr int64_t kXsplitMaxRangeBytes = 12ll << 20;

// A light row longer than this gets a wave of its own in the packed SpMM and
// attention-forward launches rather than a share of one (a packed row steps
// through its entries a few at a time, so the longest rows would set the
// kernel's duration).
constexpr int32_t kLongRow = 128;

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
    K_TILE_BWD_DST,
    K_TILE_BWD_SRC,
    K_GAT_BWD_DST_MAIN,
    K_GAT_BWD_DST_MERGE,
    K_GAT_BWD_SRC_MAIN,
    K_GAT_BWD_SRC_MERGE,
    K_GAT_DATT,
    K_RED_INIT,
    K_RED_MAIN,
    K_RED_FINAL,
    K_RED_BWD_MAIN,
    K_RED_BWD_MERGE,
    K_SPMM_MAIN,
    K_SPMM_MERGE,
    K_SPMM_T_MAIN,
    K_SPMM_T_MERGE,
    K_SPMM_WSB,
    K_SPMM_T_WSB,
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
    bool rows_sorted = false;  // every row's sources in non-decreasing order (checked at creation)
    gnn_plan_opts opts{};
    gnn::Buckets fwd;          // in-degree buckets over the CSR
    gnn::XSplit xsplit;        // the forward's heavy rows split at source ranges (see XSplit)
    bool has_csc = false;
    gnn::DevBuf cindptr, cindices;
    gnn::Buckets bwd;          // out-degree buckets over the transposed adjacency
    // 16x16 tiles: tile list by (row block, col block), residual CSR, the
    // light rows outside tiled row blocks; for the backward also the tiles
    // ordered by column block, the transposed residual and the light sources
    // outside tiled column blocks
    bool has_tiles = false;
    int32_t n_tiles = 0, tile_min_nnz = 0, n_trb = 0, n_light_nt = 0, n_tcb = 0, n_c_light_nt = 0;
    int64_t n_residual = 0;
    gnn::DevBuf tile_rc, tile_mask, tile_ptr, trb, rindptr, rindices, light_nt;
    gnn::DevBuf ctile, ctile_ptr, tcb, rcindptr, rcindices, c_light_nt;
    // cached SpMM weights (CSR order; transposed-adjacency order with the transpose), -1: none;
    // and each light row's entry range [e0, e1) in the descending-degree launch order (int2
    // [n_light]; over the transposed adjacency too), so a packed wave reads its rows' ranges
    // without first reading the row ids
    int32_t spmm_norm = -1;
    gnn::DevBuf spmm_w, spmm_cw, spmm_rng, spmm_crng;
    // tiled plans: cached weights of the residual entries (residual CSR order;
    // transposed-residual order with the transpose)
    gnn::DevBuf spmm_rw, spmm_rcw;
    // workspace (heavy partials, backward statistics), grows on demand
    gnn::DevBuf ws;
    int64_t largest_ws = 0;
    gnn::Timer timer;
    // every structure array the plan owns (the workspace excluded)
    std::vector<gnn::DevBuf *> structures();
    int64_t structure_bytes();
};

namespace gnn {
// plan workspace of at least `bytes` (kept, grown on demand)
int plan_workspace(gnn_plan_s *p, size_t bytes, hipStream_t s, void **out);

int64_t cdiv(int64_t a, int64_t b);
dim3 grid1d(int64_t n, int t = 256);
int bits_for(int64_t n);
// int32 scratch elements needed by scan_rec / radix_sort on n elements
int64_t scan_scratch(int64_t n);
int64_t sort_scratch(int64_t n);
// device-wide exclusive scan of int32 (in may equal out); *total_dev receives the sum
int scan_rec(const int32_t *in, int32_t *out, int64_t n, int32_t *total_dev, int32_t *scratch, hipStream_t s);
// stable LSD radix sort of 64-bit keys on bits [0, bits) (tmp: same-size scratch);
// an optional int32 payload moves with its key
int radix_sort(uint64_t *keys, uint64_t *tmp, int64_t n, int bits, int32_t *scratch, hipStream_t s,
               int32_t *vals = nullptr, int32_t *vtmp = nullptr);
// sorted (row << nb | col) keys -> rowptr [n_rows+1] / col [<= cap]; dedupe drops repeated keys
int emit_structure(uint64_t *keys, int64_t n, int nb, int dedupe, int32_t n_rows, int32_t *rowptr, int32_t *col,
                   int64_t cap, int32_t *flags, int32_t *pos, int32_t *total_dev, int32_t *scratch, hipStream_t s);
// indptr monotone from 0 to e, every index in [0, n): GNN_OK, else GNN_ERR_BAD_GRAPH (synchronises s)
int validate_csr(const int32_t *indptr, const int32_t *indices, int32_t n, int64_t e, hipStream_t s);
__global__ void k_set_i32(int32_t *p, int32_t v);
__global__ void k_fill_i32(int32_t *p, int64_t n, int32_t v);   // p[0..n) = v
// transpose a CSR (indptr/indices over n rows) into cindptr/cindices
int build_transpose(const int32_t *indptr, const int32_t *indices, int32_t n, int64_t e, DevBuf &cindptr,
                    DevBuf &cindices, hipStream_t s);
// bucket a CSR-like structure (by_degree: also the light list by descending degree)
int build_buckets(const int32_t *indptr, int32_t n, int32_t T, int32_t C, int32_t W, int32_t sched_order,
                  Buckets &b, hipStream_t s, bool by_degree = false);
// 16x16 tile census of the plan's graph (fills the plan's tile arrays)
int build_tiles(gnn_plan_s *p, int32_t min_nnz, hipStream_t s);

// Checked builds (GNN_CHECKED): each compute entry point validates its graph
// after the argument checks (checked_graph) and, after its kernels, reads and
// clears every source file's index flag (finish_call): GNN_ERR_BAD_GRAPH when
// a kernel met an index outside [0, N). Other builds: no-ops.
int index_fault_attn(hipStream_t s);
int index_fault_gat(hipStream_t s);
int index_fault_tile(hipStream_t s);
int index_fault_reduce(hipStream_t s);
int index_fault_spmm(hipStream_t s);
int take_index_faults(hipStream_t s);

inline int checked_graph(const int32_t *indptr, const int32_t *indices, int32_t n, int64_t e, hipStream_t s) {
#ifdef GNN_CHECKED
    return n > 0 ? validate_csr(indptr, indices, n, e, s) : GNN_OK;
#else
    (void)indptr, (void)indices, (void)n, (void)e, (void)s;
    return GNN_OK;
#endif
}

inline int finish_call(int rc, hipStream_t s) {
#ifdef GNN_CHECKED
    return rc != GNN_OK ? rc : take_index_faults(s);
#else
    (void)s;
    return rc;
#endif
}
}  // namespace gnn
