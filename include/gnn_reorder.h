/*
 * gnn_reorder.h: graph reordering for gather locality (C ABI).
 *
 * "On Efficient Scaling of GNNs via IO-Aware Layers Implementations",
 * technical summary, Methodology (graph reordering revisited for the kernels'
 * parallelisation strategies, neighbour-parallel versus feature-parallel:
 * gather-dominated kernels gain on high-degree graphs, little on low-degree or
 * tiny ones).
 *
 * Conventions as in gnn_attn.h: DEVICE pointers owned by the caller, status
 * codes returned, validation on the host before any kernel. These calls are
 * preprocessing: they allocate temporary device memory and synchronise
 * `stream` before returning. The graph is a CSR by destination (indptr int32
 * [N+1], indices int32 [E]); it is checked as in gnn_plan_create
 * (GNN_ERR_BAD_GRAPH when indptr is not monotone from 0 to E or an index is
 * outside [0, N)).
 */
#ifndef GNN_REORDER_H
#define GNN_REORDER_H

#include "gnn_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Degree of a node below: its row's entries plus the entries naming it
 * (in-degree + out-degree, repeated entries counted). */
typedef enum {
    GNN_ORDER_DEGREE = 0, /* descending degree, ties by ascending id */
    GNN_ORDER_RCM = 1     /* reverse Cuthill-McKee on the symmetrised graph: components in the order of
                             their smallest (degree, id) member, each searched breadth first from it,
                             a node's unvisited neighbours taken in ascending (degree, id); the whole
                             visiting order reversed */
} gnn_order_t;

/*
 * Node order for relabelling: perm[new id] = old id, int32 [N], written to
 * device memory. Deterministic (independent of scheduling). RCM labels
 * components by min-rank hooking with pointer jumping (about log2 of the
 * largest component's diameter sweeps) and then searches breadth first one
 * level at a time; both are O(E) per step with one host synchronisation.
 * Both loops are capped: label sweeps at 64 + 8 * ceil(log2(N + 1)), search
 * levels at 65,536 (a component deeper than that from its start, e.g. a
 * path of more than 65,537 nodes); reaching a cap returns
 * GNN_ERR_UNSUPPORTED (degree order has no such limit). The environment
 * variables GNN_RCM_MAX_SWEEPS and GNN_RCM_MAX_LEVELS (positive integers)
 * override the caps.
 * GNN_ERR_INVALID_ARG for bad sizes or method.
 * Source: technical summary, Methodology (graph reordering revisited for
 * neighbour- and feature-parallel kernels).
 */
int gnn_reorder(const int32_t *indptr, const int32_t *indices, int32_t N, int64_t E, gnn_order_t method,
                int32_t *perm /*[N]*/, hipStream_t stream);

/*
 * The relabelled graph: new row r is old row perm[r], every source j renamed
 * to the new id of j, each row sorted ascending; repeated entries are kept.
 * new_indptr [N+1], new_indices [E] (caller-allocated). perm must name every
 * node exactly once, else GNN_ERR_INVALID_ARG.
 * Source: as gnn_reorder (applying a reordering to the graph).
 */
int gnn_permute_graph(const int32_t *indptr, const int32_t *indices, int32_t N, int64_t E, const int32_t *perm,
                      int32_t *new_indptr, int32_t *new_indices, hipStream_t stream);

/*
 * Feature rows in the new order: dst[r] = src[perm[r]] (back = 0), or back to
 * the old order: dst[perm[r]] = src[r] (back = 1). Rows of row_bytes bytes
 * (a multiple of 16, else GNN_ERR_UNSUPPORTED); src and dst distinct (when
 * N > 0 and row_bytes > 0; empty tables may both be null) and 16-byte aligned
 * (GNN_ERR_ALIGNMENT). perm is checked to name every node once
 * (GNN_ERR_INVALID_ARG); the copy itself is asynchronous on `stream`. N == 0
 * or row_bytes == 0: nothing to do, GNN_OK.
 * Source: as gnn_reorder (applying a reordering to the node features).
 */
int gnn_permute_rows(const void *src, void *dst, int32_t N, int64_t row_bytes, const int32_t *perm, int32_t back,
                     hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* GNN_REORDER_H */
