/*
 * gnn_reduce.h: degree-aware neighbourhood max / min reduction (C ABI).
 *
 * "On Efficient Scaling of GNNs via IO-Aware Layers Implementations",
 * technical summary, Methodology (reduction-based aggregations): a per-edge
 * computation followed by a reduction over the neighbourhood (min/max
 * pooling); nodes split by a degree threshold into light ones, served by a
 * feature-parallel kernel, and heavy ones, whose edge lists are cut into
 * chunks reduced in parallel and merged with atomic operations on packed
 * (value, index) pairs.
 *
 * Conventions are those of gnn_attn.h: every array pointer is a DEVICE pointer
 * owned by the caller; calls are asynchronous on `stream`; they return a
 * gnn_status_t, validate on the host before any HIP call, and allocate
 * nothing but the plan's workspace (grown on demand, kept by the plan).
 * The graph is a CSR by destination (indptr int32 [N+1], indices int32 [E]:
 * row i lists the sources j of edges j -> i). The plan, when given, must
 * have been created on the same indptr / indices arrays.
 */
#ifndef GNN_REDUCE_H
#define GNN_REDUCE_H

#include "gnn_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { GNN_REDUCE_MAX = 0, GNN_REDUCE_MIN = 1 } gnn_reduce_op_t;

/* Per-edge message of entry (i, j): the source row, or the source row minus
 * the destination row (one fp32 subtraction per feature). */
typedef enum { GNN_MSG_SRC = 0, GNN_MSG_DIFF = 1 } gnn_msg_t;

/*
 * Neighbourhood max / min with the winning source:
 *   m_ij[f] = X[j,f] (GNN_MSG_SRC) or X[j,f] - X[i,f] (GNN_MSG_DIFF)
 *   out[i,f] = max (GNN_REDUCE_MAX) or min (GNN_REDUCE_MIN) of m_ij[f] over
 *              the entries of row i
 *   arg[i,f] = the smallest source j attaining it
 * Values compare as floats (-0 == +0; the stored value is the winner's own,
 * sign of zero included); NaN inputs are not supported. Empty rows give
 * out 0 and arg -1. The result is exact: no rounding except the one fp32
 * subtraction of GNN_MSG_DIFF and, for bf16, the rounding of that difference
 * to bf16 (nearest even) on output.
 *   X, out: [N, F] row-major in `dtype` (GNN_F32 or GNN_BF16); F*sizeof(dtype)
 *           must be a multiple of 16 bytes, else GNN_ERR_UNSUPPORTED.
 *   arg:    int32 [N, F] or NULL (then not written).
 *   plan:   NULL runs every row on the light kernel (one wave per row and
 *           feature group); with a plan, rows of degree > light_threshold run
 *           as chunk groups merged by 64-bit atomic max / min and the plan
 *           workspace holds n_heavy * F * 8 bytes. The result does not depend
 *           on the plan or on the order of the atomics.
 *   Errors: GNN_ERR_INVALID_ARG (sizes, NULL arrays, op / msg, plan built on
 *   other arrays), GNN_ERR_ALIGNMENT (X, out or arg not 16-byte aligned),
 *   GNN_ERR_OOM / GNN_ERR_HIP.
 * Source: technical summary, Methodology, reduction-based aggregations (a
 * per-edge computation followed by a neighbourhood min/max; degree-aware
 * light/heavy tiling; heavy partials merged by packed (value, index) atomics).
 */
int gnn_reduce_fwd(gnn_plan_t plan, const int32_t *indptr, const int32_t *indices, int32_t N, int64_t E, int32_t F,
                   const void *X, void *out, int32_t *arg /*nullable*/, gnn_reduce_op_t op, gnn_msg_t msg,
                   gnn_dtype_t dtype, hipStream_t stream);

/*
 * Gradient of gnn_reduce_fwd with respect to X through the winners arg
 * (as returned by the forward on the same graph):
 *   dX[j,f] = sum of dOut[i,f] over the rows i with arg[i,f] == j
 *             (a source listed several times in a row receives it once)
 *             - dOut[j,f] for GNN_MSG_DIFF when row j is not empty.
 * Summed in fp32 in a fixed order (no float atomics): bitwise reproducible.
 *   dOut, dX: [N, F] in `dtype` (dX rounded to bf16, nearest even, for bf16);
 *   arg: int32 [N, F]. All three 16-byte aligned.
 *   plan: required, created with want_csc (the transposed adjacency and its
 *         out-degree buckets); heavy sources use n_groups * F * 4 bytes of
 *         workspace. GNN_ERR_INVALID_ARG without a plan, GNN_ERR_UNSUPPORTED
 *         when it has no transposed adjacency.
 * Source: the training pass of the same reduction layer (technical summary,
 * Methodology); the gradient is the chain rule through the winners.
 */
int gnn_reduce_bwd(gnn_plan_t plan, const int32_t *indptr, const int32_t *indices, int32_t N, int64_t E, int32_t F,
                   const void *dOut, const int32_t *arg, void *dX, gnn_msg_t msg, gnn_dtype_t dtype,
                   hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* GNN_REDUCE_H */
