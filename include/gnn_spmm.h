/*
 * gnn_spmm.h: cached SpMM aggregation for GCN / GraphConv layers (C ABI).
 *
 * "On Efficient Scaling of GNNs via IO-Aware Layers Implementations",
 * technical summary, Methodology (SpMM-based convolutions H' = sigma(A H W):
 * graph-specific metadata such as normalised weights is cached and the
 * transposed adjacency is precomputed for the backward pass).
 *
 * Conventions as in gnn_attn.h (DEVICE pointers owned by the caller, status
 * codes, host validation before any kernel, asynchronous on `stream`). The
 * dense feature transform (H W) is an ordinary GEMM and is not part of this
 * library; this is the sparse aggregation.
 */
#ifndef GNN_SPMM_H
#define GNN_SPMM_H

#include "gnn_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Weight of entry (row i, source j); indeg(v) = number of entries in row v,
 * self-loops included when the CSR holds them (the degrees of A + I). */
typedef enum {
    GNN_NORM_SUM = 0,  /* 1                              (GraphConv, sum aggregation) */
    GNN_NORM_MEAN = 1, /* 1 / indeg(i)                   (mean aggregation)           */
    GNN_NORM_GCN = 2   /* 1 / sqrt(indeg(i) * indeg(j))  (GCN symmetric normalisation; 0 when
                          source j has no entries of its own, as indeg(j)^-1/2 is taken as 0) */
} gnn_norm_t;

/*
 * Compute and cache the per-entry weights of `norm` in the plan (fp32, in CSR
 * order and, when the plan was created with want_csc, in transposed-adjacency
 * order), replacing any earlier cache. Allocates 4*E bytes per order on the
 * first call; later calls rewrite those buffers in place, ordered after
 * earlier work on `stream` (products still running on another stream race
 * with it). GNN_ERR_INVALID_ARG for a NULL plan or an unknown norm.
 * Source: technical summary, Methodology, SpMM-based convolutions
 * (graph-specific metadata such as normalised weights cached once).
 */
int gnn_spmm_prepare(gnn_plan_t plan, gnn_norm_t norm, hipStream_t stream);

/*
 * Y = A_w X (transpose = 0) or Y = A_w^T X (transpose = 1, the gradient of the
 * former with respect to X; needs the plan's transposed adjacency, else
 * GNN_ERR_UNSUPPORTED), A_w the N x N matrix with entry (i, j) the summed
 * weights of row i's entries naming j.
 *   X, Y: [N, F] row-major in `dtype` (GNN_F32 or GNN_BF16), 16-byte aligned;
 *         F * sizeof(dtype) a multiple of 16 bytes (else GNN_ERR_UNSUPPORTED).
 *   plan: required, created on these indptr / indices arrays and prepared with
 *         gnn_spmm_prepare (else GNN_ERR_INVALID_ARG).
 * fp32 accumulation in a fixed order (no atomics: bitwise reproducible), Y
 * rounded to the storage type (nearest even). Heavy rows use n_groups * F * 4
 * bytes of plan workspace.
 * On a plan created with tile_density > 0 (a 16x16 tile census), when F is a
 * multiple of 16 and a row is at most 256 bytes, the tiled 16-row blocks
 * (16-column blocks for the transpose) run on the block kernel: the tiles'
 * products on the matrix cores in fp32 (weights from the in-degrees, the
 * same expression as the cached ones), then the blocks' residual entries
 * with cached weights (gnn_spmm_prepare caches them for tiled plans, 4 bytes
 * per residual entry and order); other rows run as above.
 * Source: technical summary, Methodology, SpMM-based convolutions (the
 * aggregation of H' = sigma(A H W); the transposed adjacency precomputed for
 * the backward pass; the Weighted Block Sparse option for the matrix units
 * on locally dense graphs).
 */
int gnn_spmm(gnn_plan_t plan, const int32_t *indptr, const int32_t *indices, int32_t N, int64_t E, int32_t F,
             const void *X, void *Y, int32_t transpose, gnn_dtype_t dtype, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* GNN_SPMM_H */
