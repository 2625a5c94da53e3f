/*
 * gnn_attn.h — C ABI of the fused CSR neighbourhood-attention library for
 * AMD MI355X (gfx950).
 *
 * The operations follow "On Efficient Scaling of GNNs via IO-Aware Layers
 * Implementations" (technical summary, Methodology):
 *   - attention-based layers (Graph Transformer, GATv2) computed by fused CSR
 *     kernels that score, softmax-normalise and aggregate in one streaming
 *     pass over each node's neighbours;
 *   - the forward pass keeps running softmax statistics in registers (online
 *     softmax) so no edge-wise logits are written;
 *   - the backward pass caches a compact per-node statistic (log-sum-exp)
 *     instead of edge weights and recomputes the weights on the fly;
 *   - degree-aware tiling: nodes split into light and heavy sets by a degree
 *     threshold, heavy neighbour lists cut into edge chunks reduced in
 *     parallel;
 *   - graph metadata (buckets, transposed adjacency) built once and cached
 *     for reuse in a plan.
 *
 * Conventions for every call below
 *   - Pointers are DEVICE pointers owned by the caller unless marked "host".
 *     The library never frees caller memory and keeps no caller pointer past
 *     the call, except that a plan does not copy indptr/indices: the arrays
 *     passed to gnn_plan_create must stay alive and unchanged while the plan
 *     is used with them.
 *   - Graphs are CSR by destination: row i (indices[indptr[i] .. indptr[i+1]))
 *     lists the sources j of the edges j -> i; the softmax of node i runs
 *     over those in-neighbours. indptr is int32 [N+1] with indptr[0] = 0 and
 *     indptr[N] = E; indices is int32 [E], each in [0, N). Multigraph entries
 *     are each counted.
 *   - Node features Q, K, V, O and every gradient are [N, H, D] contiguous
 *     row-major: element (i, h, d) at offset (i*H + h)*D + d, all in one
 *     dtype (fp32 or bf16). Arithmetic is fp32; bf16 results are rounded to
 *     nearest-even. LSE is fp32 [N, H] in natural-log units.
 *   - D must be 16, 32, 64 or 128; H >= 1. Feature pointers must be 16-byte
 *     aligned. E <= 2^31 - 2^21 (2,145,386,496; GNN_ERR_INVALID_ARG above).
 *   - A node with no in-edges gets O = 0, LSE = -inf and zero gradients.
 *   - Attention calls are asynchronous on `stream` and do not synchronise
 *     the host, with one exception: a call on a plan whose workspace is
 *     smaller than the call needs (the first call at a larger H*D, or the
 *     first backward) synchronises `stream` once before replacing it.
 *     gnn_csr_build and gnn_plan_create synchronise `stream` once to read
 *     back counts.
 *   - Every call returns a gnn_status_t; argument errors are detected on the
 *     host before any HIP call is made. No exception crosses the ABI.
 *   - A plan may be used by one stream at a time (it owns reusable
 *     workspace); different plans are independent.
 *   - Device memory the library allocates itself (plan arrays, workspace,
 *     temporaries) fails with GNN_ERR_OOM when hipMalloc does. Test hook:
 *     when the environment variable GNN_ALLOC_CAP_BYTES holds a non-negative
 *     integer, every such allocation larger than it is refused the same way
 *     before hipMalloc is called (read at each allocation); everything the
 *     failing call had allocated is freed, and gnn_status_string names the cap.
 */
#ifndef GNN_ATTN_H
#define GNN_ATTN_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { GNN_F32 = 0, GNN_BF16 = 1 } gnn_dtype_t;

typedef enum {
    GNN_OK = 0,
    GNN_ERR_INVALID_ARG = -1,  /* null pointer, negative size, inconsistent sizes   */
    GNN_ERR_UNSUPPORTED = -2,  /* D not in {16,32,64,128}, unknown dtype, plan lacks a part */
    GNN_ERR_ALIGNMENT = -3,    /* feature pointer not 16-byte aligned                 */
    GNN_ERR_OOM = -4,          /* device allocation failed                            */
    GNN_ERR_HIP = -5,          /* a HIP runtime call failed (see gnn_status_string)   */
    GNN_ERR_BAD_GRAPH = -6,    /* indptr/indices inconsistent or out of range         */
    GNN_ERR_SCRATCH = -7       /* gnn_attn_fwd_noalloc: problem exceeds its fixed scratch */
} gnn_status_t;

typedef struct gnn_plan_s *gnn_plan_t;   /* opaque; owns its device arrays */

/*
 * Plan options (degree-aware tiling, technical summary, Methodology).
 * The pages name a degree threshold but give no value; these are tunables.
 */
typedef struct {
    int32_t light_threshold; /* T: in-degree <= T is light (one wave per node); default 512   */
    int32_t chunk;           /* C: edges per wave on a heavy row; default 512, >= 1,
                                C * waves_per_group <= 2^20                                        */
    int32_t waves_per_group; /* W: waves per heavy workgroup, merged in LDS; 1, 2, 4 or 8; default 4 */
    float tile_density;      /* tau: a 16x16 block with >= tau*256 edges becomes a dense tile;
                                <= 0 disables the tile path; default 0                         */
    int32_t want_csc;        /* build the transposed adjacency and its out-degree buckets,
                                needed by gnn_attn_bwd; default 0                               */
    int32_t sched_order;     /* launch order of light nodes; ties always by ascending id.
                                0 = ascending id; 1 = descending degree; 2 (default) = nodes
                                of degree > max(1, light_threshold/4) first, by descending
                                floor(log2(degree)), then the rest by id. Outputs do not
                                depend on it                                                   */
    int32_t xcd_split;       /* 1 (default): also cut the heavy rows at the boundaries of 8
                                equal source-id ranges into groups of at most C entries,
                                each reading one range and streamed by one wave, and launch
                                them so that the 8 XCDs each take one range (their L2s then
                                hold what they gather);
                                the forward and the GATv2 backward's destination pass use
                                them when the gathered rows (K, plus V unless it aliases K)
                                of N/8 nodes take at most 12 MiB and all heads fit one head
                                group; results differ from the plain groups by rounding only.
                                0: not built. Needs sorted rows                             */
} gnn_plan_opts;

/* Fill *opts with the defaults above. Returns GNN_ERR_INVALID_ARG if opts is NULL. */
int gnn_plan_opts_default(gnn_plan_opts *opts /*host*/);

/*
 * Canonical CSR by destination from a COO edge list (edge src[k] -> dst[k]).
 * Rows ascend by destination, each row's sources ascend, duplicate pairs are
 * removed, and with add_self_loops != 0 every node has the pair (i, i)
 * exactly once. Device radix sort on 64-bit (dst, src) keys, then
 * de-duplication and row boundaries; bit-exact and deterministic.
 *   src, dst      int32 [n_edges_in], device; each in [0, n_nodes)
 *   indptr        int32 [n_nodes+1], device, written
 *   indices       int32 [cap], device, written up to min(E, cap)
 *   n_edges_out   host; receives E (the number of unique edges)
 * Errors: GNN_ERR_BAD_GRAPH if an endpoint is out of range; GNN_ERR_INVALID_ARG
 * if E > cap (indptr is then complete, indices truncated). Temporary device
 * memory (about 20 bytes per input edge) is allocated and freed inside.
 * Synchronises `stream` once.
 * Source: the fused CSR attention kernels (technical summary, Methodology,
 * attention-based layers) take the graph as CSR; by destination so a node's
 * softmax runs over its in-neighbours (the workload descriptions).
 */
int gnn_csr_build(const int32_t *src, const int32_t *dst, int64_t n_edges_in, int32_t n_nodes,
                  int32_t add_self_loops, int32_t *indptr, int32_t *indices, int64_t cap,
                  int64_t *n_edges_out /*host*/, hipStream_t stream);

/*
 * Build a plan for one CSR graph: validates indptr/indices (monotone,
 * indptr[N] = E, indices in range), splits nodes into light/heavy by
 * in-degree with the heavy chunk-group table, and, as opts ask, the
 * transposed adjacency with out-degree buckets and the 16x16 tile census.
 * opts NULL means defaults. Synchronises `stream` once. *plan_out is set only
 * on success.
 * Source: technical summary, Methodology: degree-aware tiling (light and
 * heavy node sets by a degree threshold, heavy neighbour lists cut into edge
 * chunks reduced in parallel), graph metadata cached once and reused, the
 * transposed adjacency precomputed for the backward pass, 16x16 block tiles
 * for locally dense neighbourhoods.
 */
int gnn_plan_create(const int32_t *indptr, const int32_t *indices, int32_t n_nodes, int64_t n_edges,
                    const gnn_plan_opts *opts /*host, nullable*/, hipStream_t stream,
                    gnn_plan_t *plan_out /*host*/);

/* Counts and device pointers of a plan's arrays (read-only views, owned by the plan).
 * Tiles follow the 16x16 block-sparse tiles of the attention layers (technical
 * summary, Methodology): a (row block, column block) pair of aligned 16-node
 * blocks becomes a tile when it holds >= tile_min_nnz distinct positions and
 * neither block contains a node of degree > T (in-degree for rows, out-degree
 * for sources); the first copy of each position in a tile is covered by the
 * tile's mask and every other edge stays in the residual CSR. */
typedef struct {
    int32_t n_nodes;
    int64_t n_edges;
    int32_t light_threshold, chunk, waves_per_group;
    /* in-degree buckets over the CSR */
    int32_t n_light, n_heavy, n_groups;
    const int32_t *light_ids;   /* [n_light]   ascending node ids with deg <= T          */
    const int32_t *heavy_ids;   /* [n_heavy]   ascending node ids with deg > T           */
    const int32_t *groups;      /* [n_groups][3] (node, e0, e1), e1 - e0 <= C*W          */
    const int32_t *partial_ofs; /* [n_heavy+1] group range of each heavy node            */
    /* transposed adjacency and out-degree buckets (want_csc) */
    int32_t has_csc;
    const int32_t *cindptr;     /* [N+1] */
    const int32_t *cindices;    /* [E]   destinations of each source, ascending          */
    int32_t c_n_light, c_n_heavy, c_n_groups;
    const int32_t *c_light_ids, *c_heavy_ids, *c_groups, *c_partial_ofs;
    /* 16x16 tiles (tile_density > 0) */
    int32_t has_tiles, n_tiles, tile_min_nnz;
    const int32_t *tile_rc;     /* [n_tiles][2] (row block, col block), ascending       */
    const uint64_t *tile_mask;  /* [n_tiles][4] bit (dst%16)*16 + (src%16), word = bit/64 */
    const int32_t *tile_ptr;    /* [ceil(N/16)+1] tiles of each row block               */
    const int32_t *rindptr;     /* [N+1] residual CSR (edges outside tiles)             */
    const int32_t *rindices;    /* [n_residual]                                         */
    int64_t n_residual;
    int32_t n_trb, n_light_nt, n_tcb, n_c_light_nt;
    const int32_t *trb;         /* [n_trb] row blocks holding tiles, ascending           */
    const int32_t *light_nt;    /* [n_light_nt] light nodes outside tiled row blocks     */
    const int32_t *ctile;       /* [n_tiles] tile ids ordered by (col block, row block)  */
    const int32_t *ctile_ptr;   /* [ceil(N/16)+1] range of each column block in ctile   */
    const int32_t *tcb;         /* [n_tcb] column blocks holding tiles (want_csc)        */
    const int32_t *rcindptr;    /* [N+1] transposed residual (want_csc)                  */
    const int32_t *rcindices;   /* [n_residual]                                          */
    const int32_t *c_light_nt;  /* [n_c_light_nt] light sources outside tiled column blocks */
    /* device memory owned by the plan */
    const int32_t *light_sched;   /* [n_light]   launch order of the light nodes          */
    const int32_t *c_light_sched; /* [c_n_light] launch order of the light sources        */
    int64_t structure_bytes;    /* buckets, transposed adjacency, tiles                 */
    int64_t workspace_bytes;    /* heavy partials and backward statistics (grows lazily) */
    int64_t largest_workspace_alloc;
    int32_t rows_sorted;        /* 1: every CSR row lists its sources in non-decreasing order */
    const int32_t *light_by_degree; /* [n_light] light nodes in the order of the launches that pack
                                       several rows per wave: descending ceil(in-degree / 4),
                                       ties by ascending id (whatever sched_order is) */
    const int32_t *c_light_by_degree; /* [c_n_light] the same over out-degrees (with want_csc) */
    int32_t spmm_norm;          /* gnn_norm_t cached by gnn_spmm_prepare, -1: none          */
    const float *spmm_w;        /* [n_edges] cached SpMM weights in CSR order (or NULL)     */
    const float *spmm_cw;       /* [n_edges] the same in transposed-adjacency order (or NULL) */
    int32_t n_long_light;       /* light nodes of in-degree above 128: the first entries of
                                   light_by_degree, each given a wave of its own by the packed
                                   SpMM and attention-forward launches */
    int32_t c_n_long_light;     /* the same over out-degrees and c_light_by_degree (want_csc) */
    /* source-range split of the heavy rows (xcd_split; n_xsplit_groups = 0: none) */
    int32_t n_xsplit_groups, n_xsplit_slots;
    const int32_t *xsplit_groups;      /* [n_xsplit_groups][3] (node, e0, e1): for each heavy node
                                          in heavy_ids order, its entries of each source range r
                                          (sources in [r*ceil(N/8), (r+1)*ceil(N/8)), r = 0..7, in
                                          order) cut into ceil(len / C) near-equal groups,
                                          group j = [a + len*j/k, a + len*(j+1)/k)              */
    const int32_t *xsplit_partial_ofs; /* [n_heavy+1] group range of each heavy node             */
    const int32_t *xsplit_order;       /* [n_xsplit_slots] launch slot i*8 + r: the i-th group of
                                          range r, or -1; n_xsplit_slots = 8 * the largest count */
} gnn_plan_info;

int gnn_plan_export(gnn_plan_t plan, gnn_plan_info *info /*host*/);
int gnn_plan_destroy(gnn_plan_t plan);

/*
 * Graph-Transformer attention forward: for each node i and head h,
 *   s_ij = scale * <Q[i,h,:], K[j,h,:]> over j in row i,
 *   O[i,h,:] = sum_j softmax_j(s_ij) V[j,h,:],  LSE[i,h] = ln sum_j exp(s_ij).
 * One streaming pass with an online softmax; no per-edge value reaches
 * memory. plan NULL runs every node on the light (one wave per node) path;
 * otherwise the plan's buckets are used and must describe this graph.
 * scale <= 0 means 1/sqrt(D). LSE may be NULL.
 * Source: technical summary, Methodology, attention-based layers, forward
 * pass: score, softmax normalisation and aggregation fused in one streaming
 * pass over the neighbours, running statistics in registers (online
 * softmax), no edge-wise logits written; the per-node log-sum-exp is kept
 * for the backward pass.
 */
int gnn_attn_fwd(gnn_plan_t plan, const int32_t *indptr, const int32_t *indices, int32_t N, int64_t E,
                 int32_t H, int32_t D, const void *Q, const void *K, const void *V, void *O,
                 float *LSE /*nullable*/, float scale, gnn_dtype_t dtype, hipStream_t stream);

/*
 * Graph-Transformer attention forward that allocates no device memory, for
 * callers that cannot allocate: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc. Same arguments, operation and
 * results as gnn_attn_fwd (bitwise identical outputs for the same inputs and
 * plan); the caller passes O (and LSE, nullable) already allocated.
 *   Scratch: the heavy rows' partial states go to a fixed device buffer of
 *   GNN_NOALLOC_SCRATCH_BYTES (16 MiB) that the library holds on each GPU it
 *   runs on until the process ends, instead of the plan workspace, which this
 *   call never grows. A call needs n_groups * (H*D + 2*H) * 4 bytes of it
 *   (n_groups: the plan's heavy chunk groups; 0 without a plan, without heavy
 *   rows, or on the tile path's tiled rows); a larger need returns
 *   GNN_ERR_SCRATCH before anything is launched.
 *   Sharing: every call on one GPU uses that GPU's buffer, which keeps the
 *   last call's contents. Calls that overlap in time on one GPU (two streams,
 *   or two host threads) race and give undefined results: serialise them.
 *   Nothing in the buffer needs to start at zero (every partial a call reads
 *   is written earlier in the same call).
 *   Per-kernel timing must be off on the plan (GNN_ERR_UNSUPPORTED otherwise).
 *   The first call on a device looks up the buffer's device address with the
 *   device current (hipGetSymbolAddress); later calls make no such lookup.
 */
#define GNN_NOALLOC_SCRATCH_BYTES (16u << 20)
int gnn_attn_fwd_noalloc(gnn_plan_t plan, const int32_t *indptr, const int32_t *indices, int32_t N, int64_t E,
                         int32_t H, int32_t D, const void *Q, const void *K, const void *V, void *O,
                         float *LSE /*nullable*/, float scale, gnn_dtype_t dtype, hipStream_t stream);

/*
 * Graph-Transformer attention backward from the cached LSE (the forward's
 * output for the same inputs): weights are recomputed per edge as
 * p_ij = exp(s_ij - LSE_i), and with dp_ij = <dO_i, V_j>,
 * Delta_i = sum_j p_ij dp_ij (which equals <dO_i, O_i> for the exact O):
 *   dQ_i = scale * sum_j p_ij (dp_ij - Delta_i) K_j        (destination pass, CSR)
 *   dK_j = scale * sum_i p_ij (dp_ij - Delta_i) Q_i        (source pass, CSC)
 *   dV_j = sum_i p_ij dO_i
 * The destination pass forms Delta_i from the recomputed weights in the same
 * sweep that accumulates dQ_i, so a bf16-rounded O never enters the
 * gradients; O is therefore not read and may be NULL (it is kept in the
 * signature so callers can pass the forward's outputs unchanged).
 * The plan must have been created with want_csc. No atomics: results are
 * bitwise reproducible for the same inputs and plan. dQ, dK, dV must not
 * alias inputs.
 * Source: technical summary, Methodology, attention-based layers, backward
 * pass: a compact per-node statistic (the log-sum-exp) is cached instead of
 * the edge weights, which are recomputed on the fly; the transposed
 * adjacency (cached metadata) serves the source-side gradients.
 */
int gnn_attn_bwd(gnn_plan_t plan, const int32_t *indptr, const int32_t *indices, int32_t N, int64_t E,
                 int32_t H, int32_t D, const void *Q, const void *K, const void *V, const void *O,
                 const void *dO, const float *LSE, void *dQ, void *dK, void *dV, float scale,
                 gnn_dtype_t dtype, hipStream_t stream);

/*
 * GATv2 attention forward (the GATv2 layer named by the pages):
 *   s_ij = sum_d att[h,d] * LeakyReLU(K[j,h,d] + Q[i,h,d]),
 *   LeakyReLU(x) = x for x >= 0, negative_slope * x otherwise,
 * with Q = W_d x (destination projection) and K = W_s x (source projection)
 * given; O[i,h,:] = sum_j softmax_j(s_ij) V[j,h,:], where V is normally the
 * same buffer as K (then one row is gathered per edge). att is fp32 [H, D].
 * No score scaling. LSE may be NULL; plan as for gnn_attn_fwd.
 * Source: technical summary, Methodology (GATv2 among the attention-based
 * layers computed by the fused streaming pass) and Results (GATv2 speed and
 * peak-memory figures); the score is GATv2's, as the workload descriptions
 * give it.
 */
int gatv2_attn_fwd(gnn_plan_t plan, const int32_t *indptr, const int32_t *indices, int32_t N, int64_t E,
                   int32_t H, int32_t D, const void *Q, const void *K, const void *V, const float *att,
                   float negative_slope, void *O, float *LSE /*nullable*/, gnn_dtype_t dtype,
                   hipStream_t stream);

/*
 * GATv2 attention backward from the cached LSE (the forward's LSE for the same
 * inputs; weights recomputed per edge as p_ij = exp(s_ij - LSE_i), as for the
 * Graph Transformer). With z = K[j] + Q[i], phi = LeakyReLU(negative_slope),
 * dp_ij = <dO_i, V_j>, Delta_i = sum_j p_ij dp_ij, ds_ij = p_ij (dp_ij - Delta_i):
 *   dQ_i   = sum_j ds_ij att * phi'(z_ij)           (destination projection XD)
 *   dK_j   = sum_i ds_ij att * phi'(z_ij)           (source projection XS)
 *            + sum_i p_ij dO_i  when V is the same buffer as K
 *   dV_j   = sum_i p_ij dO_i    when V is a separate buffer (dV may be NULL otherwise)
 *   d_att  = sum over all edges of ds_ij phi(z_ij)  (fp32 [H, D], overwritten;
 *            zero for a graph without edges, N == 0 included)
 * phi'(z) = 1 for z >= 0 and negative_slope otherwise (the forward's branch).
 * The plan must have been created with want_csc. No atomics: d_att is a
 * fixed-order sum and every output is bitwise reproducible. The plan
 * workspace grows by N*H*D fp32 for the per-node d_att rows.
 * Source: technical summary, Methodology (the backward pass's log-sum-exp
 * recompute, applied to GATv2) and Results (GATv2 training memory); the
 * gradient is the chain rule of the GATv2 score.
 */
int gatv2_attn_bwd(gnn_plan_t plan, const int32_t *indptr, const int32_t *indices, int32_t N, int64_t E,
                   int32_t H, int32_t D, const void *Q, const void *K, const void *V, const float *att,
                   float negative_slope, const void *dO, const float *LSE, void *dQ, void *dK,
                   void *dV /*nullable when V == K*/, float *d_att, gnn_dtype_t dtype, hipStream_t stream);

/*
 * Per-kernel timing on a plan (for measurement tools). When enabled, every
 * attention call on the plan records HIP events around each kernel it
 * launches, on the call's stream. gnn_plan_timing_read synchronises on the
 * recorded events, reports for each kernel kind the number of launches and
 * their summed duration in milliseconds, and clears the log.
 *   names[k]: static strings owned by the library.
 */
int gnn_plan_set_timing(gnn_plan_t plan, int32_t enable);
int gnn_plan_timing_read(gnn_plan_t plan, int32_t cap, const char **names /*host [cap]*/,
                         int32_t *launches /*host [cap]*/, double *total_ms /*host [cap]*/,
                         int32_t *n_out /*host*/);

/*
 * 1 when this library is the checked build (compiled with GNN_CHECKED, the
 * debugging variant), else 0. In the checked build every compute call also
 * validates its indptr / indices as gnn_plan_create does (after the argument
 * checks; the allocation-free forward skips this, as the check allocates), and
 * its kernels check every graph index before using it as a node-table row: an
 * index outside [0, N) is replaced by row 0, so no access leaves the tables,
 * and the call returns GNN_ERR_BAD_GRAPH after its kernels (it synchronises
 * the stream to read the kernels' flags, so no call of the checked build can
 * be captured into a HIP graph). Results of good graphs are the same as the
 * normal build's.
 * For: debugging callers' graph arrays and the library itself; not for speed.
 */
int gnn_build_checked(void);

/* Human-readable text for a status code (includes the last HIP error for GNN_ERR_HIP). */
const char *gnn_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* GNN_ATTN_H */
