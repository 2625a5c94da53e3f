// Cached SpMM aggregation for GCN / GraphConv layers: Y = A_w X and its
// transpose (the backward), with the per-entry weights cached in the plan.
//
// "On Efficient Scaling of GNNs via IO-Aware Layers Implementations",
// technical summary, Methodology (SpMM-based convolutions H' = sigma(A H W):
// graph-specific metadata such as normalised weights cached, the transposed
// adjacency precomputed for the backward pass).
//
// Weights of entry (row i, source j): 1 (GNN_NORM_SUM), 1/indeg(i)
// (GNN_NORM_MEAN) or 1/sqrt(indeg(i) indeg(j)) (GNN_NORM_GCN; 0 when source j
// has no entries of its own), indeg the number of row entries (self-loops
// included when the CSR holds them),
// computed once in fp32 by gnn_spmm_prepare, in CSR order and, when the plan
// has the transposed adjacency, in its order too.
//
// The product uses the degree-aware layout of the other kernels: a lane holds
// one 16-byte slice of a feature row; light rows run from the packed-order
// list 4 per wave when a row spans at most 16 lanes (256 bytes), 2 per wave
// with 10 edges per step in fp32 (8 in bf16) when it spans 17-32 lanes (512
// bytes), else one per wave; the packed waves read each row's entry range
// from a record cached by gnn_spmm_prepare, alongside the row id (rows are
// short: one dependent load fewer before the gathers). The light rows of more
// than 128 entries, which head the packed list, get a wave each in the same
// launch (all its edge groups on one row), so the longest light rows take
// half or a quarter of the steps they would take packed; heavy rows run as
// the plan's chunk groups, their W waves summed in LDS and the groups summed
// in ascending order by a second pass. On a plan with a tile census the
// tiled 16-row blocks run on the block kernel further down (the Weighted
// Block Sparse option: tile products on the matrix cores, then the blocks'
// residual entries). fp32 accumulation, output rounded to the storage type;
// no atomics, so the result is bitwise reproducible. The transposed product
// (dX = A_w^T dY) is the same kernels over the transposed structures.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>

#include "attn_core.h"
#include "gnn_spmm.h"

namespace gnn {

// weight of entry (destination i, source j) from their in-degrees
__device__ __forceinline__ float spmm_weight(int norm, float di, float dj) {
    if (norm == GNN_NORM_MEAN) return 1.f / di;
    if (norm == GNN_NORM_GCN) return dj > 0.f ? 1.f / sqrtf(di * dj) : 0.f;   // a source without entries: nothing
    return 1.f;
}

__device__ __forceinline__ float in_degree(const int32_t *indptr, int32_t v) {
    return (float)(indptr[v + 1] - indptr[v]);
}

// weights in CSR order: one wave per row
__global__ void k_spmm_w_rows(const int32_t *indptr, const int32_t *indices, int32_t n, int norm, float *w) {
    const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / kWave;
    const int lane = threadIdx.x % kWave;
    if (i >= n) return;
    const int32_t e0 = indptr[i], e1 = indptr[i + 1];
    const float di = (float)(e1 - e0);
    for (int32_t e = e0 + lane; e < e1; e += kWave)
        w[e] = spmm_weight(norm, di, norm == GNN_NORM_GCN ? in_degree(indptr, checked_index(indices[e], n)) : 0.f);
}

// weights in transposed order: the entries of source j name destinations i
__global__ void k_spmm_w_cols(const int32_t *indptr, const int32_t *cindptr, const int32_t *cindices, int32_t n,
                              int norm, float *cw) {
    const int64_t j = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / kWave;
    const int lane = threadIdx.x % kWave;
    if (j >= n) return;
    const float dj = in_degree(indptr, (int32_t)j);
    for (int32_t e = cindptr[j] + lane; e < cindptr[j + 1]; e += kWave)
        cw[e] = spmm_weight(norm, in_degree(indptr, checked_index(cindices[e], n)), dj);
}

// weights of a tiled plan's residual entries, in the order of a residual
// structure (rptr, ridx) whose rows are destinations (residual CSR) or
// sources (transposed residual); degrees from the full CSR
__global__ void k_spmm_w_res(const int32_t *indptr, const int32_t *rptr, const int32_t *ridx, int32_t n, int norm,
                             int rows_are_dst, float *w) {
    const int64_t r = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / kWave;
    const int lane = threadIdx.x % kWave;
    if (r >= n) return;
    const float dr = in_degree(indptr, (int32_t)r);
    for (int32_t e = rptr[r] + lane; e < rptr[r + 1]; e += kWave) {
        const float dother = in_degree(indptr, checked_index(ridx[e], n));
        w[e] = rows_are_dst ? spmm_weight(norm, dr, dother) : spmm_weight(norm, dother, dr);
    }
}

struct SpGeom {
    int32_t N = 0, F = 0, L = 0, lr_shift = 0, G = 1, NFG = 1;
};

// entry range of each light row, in the order of the list `light`
__global__ void k_spmm_ranges(const int32_t *indptr, const int32_t *light, int32_t n_light, int2 *rng) {
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k < n_light) {
        const int32_t v = light[k];
        rng[k] = make_int2(indptr[v], indptr[v + 1]);
    }
}

struct SpParams {
    SpGeom g;
    const int32_t *indptr, *indices;   // CSR, or the transposed adjacency for the transposed product
    const float *w;                    // weights in the same order
    const void *X;
    void *Y;
    const int32_t *light;
    const int2 *rng;                   // entry range of each entry of `light` (packed launches), or null
    int32_t n_light;
    int32_t n_long;                    // packed launches: the first n_long rows get a wave each
    const int32_t *groups;
    int32_t n_groups;
    const int32_t *heavy, *partial_ofs;
    int32_t n_heavy;
    int32_t C, W;
    float *part;                       // [n_groups][F] group partials
};

template <int NV, int RPW>
struct SpLane {
    int lane, rg0, g, c, slice;
    bool act;
    int64_t col;
    __device__ __forceinline__ SpLane(const SpGeom &G, int fg) {
        lane = lane_id();
        rg0 = lane & ~(kWave / RPW - 1);
        g = (lane - rg0) >> G.lr_shift;
        c = lane & ((1 << G.lr_shift) - 1);
        slice = fg * kWave + c;
        act = slice < G.L;
        col = (int64_t)slice * NV;
    }
};

// acc = sum over entries [e0, e1) of w_e * X[j_e] (this lane's slice), edge
// groups of the row summed by a xor tree (every group lane ends with the sum)
template <class T, int U, int RPW>
__device__ __forceinline__ void sp_stream(const SpParams &P, const SpLane<Vec<T>::N, RPW> &lp, int e0, int e1,
                                          float (&acc)[Vec<T>::N]) {
    using VT = Vec<T>;
    constexpr int NV = VT::N;
    constexpr int kLanesRG = kWave / RPW;
    const SpGeom &G = P.g;
    const int64_t F = G.F;
#pragma unroll
    for (int k = 0; k < NV; ++k) acc[k] = 0.f;
    const int GR = G.G / RPW;
    const int S = min(kLanesRG, GR * U);
    const int UE = S / GR;
    const int li = lp.lane - lp.rg0;
    int jn = -1;
    float wn = 0.f;
    if (li < S && e0 + li < e1) {
        jn = checked_index(P.indices[e0 + li], G.N);
        wn = P.w[e0 + li];
    }
    for (int base = e0; RPW == 1 ? base < e1 : __any(base < e1); base += S) {
        const int jc = jn;
        const float wc = wn;
        jn = -1;
        wn = 0.f;
        if (li < S && base + S + li < e1) {
            jn = checked_index(P.indices[base + S + li], G.N);
            wn = P.w[base + S + li];
        }
        int j[U];
        float wu[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int src = lp.rg0 + u * GR + lp.g;
            j[u] = (u < UE) ? __shfl(jc, src, kWave) : -1;
            wu[u] = (u < UE) ? __shfl(wc, src, kWave) : 0.f;
        }
        typename VT::raw r[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool ok = lp.act & (j[u] >= 0);
            const int row = ok ? j[u] : 0;
            const int64_t col = ok ? lp.col : 0;
            r[u] = load_vec<T>(P.X, (int64_t)row * F + col);
            wu[u] = ok ? wu[u] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float x[NV];
            VT::unpack(r[u], x);
#pragma unroll
            for (int k = 0; k < NV; ++k) acc[k] = fmaf(wu[u], x[k], acc[k]);
        }
    }
    for (int off = 1 << G.lr_shift; off < kLanesRG; off <<= 1) {
#pragma unroll
        for (int k = 0; k < NV; ++k) acc[k] += xor_lane(acc[k], off);
    }
}

// TR marks the transposed product; the code is the same, the two launches
// get distinct kernel symbols so that profiles tell them apart.
template <class T, int U, int RPW, bool TR>
__global__ __launch_bounds__(512) void k_spmm_main(SpParams P) {
    using VT = Vec<T>;
    constexpr int NV = VT::N;
    extern __shared__ float lds[];
    const SpGeom &G = P.g;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int heavy_blocks = P.n_groups * G.NFG;
    float acc[NV];
    if ((int)blockIdx.x < heavy_blocks) {
        const int grp = blockIdx.x / G.NFG, fg = blockIdx.x % G.NFG;
        const int g0 = P.groups[3 * grp + 1], g1 = P.groups[3 * grp + 2];
        const int e0 = min(g1, g0 + w * P.C), e1 = min(g1, e0 + P.C);
        const SpLane<NV, 1> lp(G, fg);
        sp_stream<T, U, 1>(P, lp, e0, e1, acc);
        const int LR = 1 << G.lr_shift;
        float *mine = lds + ((size_t)w * LR + lp.lane) * NV;
        if (lp.lane < LR) {
#pragma unroll
            for (int k = 0; k < NV; ++k) mine[k] = acc[k];
        }
        __syncthreads();
        if (w != 0 || lp.lane >= LR || !lp.act) return;
        for (int v = 1; v < P.W; ++v) {
            const float *o = lds + ((size_t)v * LR + lp.lane) * NV;
#pragma unroll
            for (int k = 0; k < NV; ++k) acc[k] += o[k];
        }
#pragma unroll
        for (int k = 0; k < NV; ++k) P.part[(int64_t)grp * G.F + lp.col + k] = acc[k];
        return;
    }
    const int64_t item = (int64_t)(blockIdx.x - heavy_blocks) * P.W + w;
    int node, fg = 0;
    if (RPW == 1) {
        const int64_t ni = item / G.NFG;
        if (ni >= P.n_light) return;
        fg = (int)(item % G.NFG);
        node = P.light ? P.light[ni] : (int)ni;
    } else {
        if (item < P.n_long) {
            // a long row at the head of the packed list: the whole wave, all its edge groups
            node = P.light[item];
            const int2 r = P.rng[item];
            const SpLane<NV, 1> lp(G, 0);
            sp_stream<T, U, 1>(P, lp, r.x, r.y, acc);
            if (lp.g != 0 || !lp.act) return;
            store_vec_nt<T>(P.Y, (int64_t)node * G.F + lp.col, VT::pack(acc));
            return;
        }
        const int64_t ni0 = P.n_long + (item - P.n_long) * RPW;
        if (ni0 >= P.n_light) return;
        const int64_t ni = ni0 + (lane_id() / (kWave / RPW));
        node = ni < P.n_light ? P.light[ni] : -1;
        if (P.rng) {
            // the row's range from the cached records, loaded alongside the row id rather than after it
            const int2 r = ni < P.n_light ? P.rng[ni] : make_int2(0, 0);
            const SpLane<NV, RPW> lp(G, fg);
            sp_stream<T, U, RPW>(P, lp, r.x, r.y, acc);
            if (lp.g != 0 || !lp.act || node < 0) return;
            store_vec_nt<T>(P.Y, (int64_t)node * G.F + lp.col, VT::pack(acc));
            return;
        }
    }
    const SpLane<NV, RPW> lp(G, fg);
    const int e0 = node >= 0 ? P.indptr[node] : 0, e1 = node >= 0 ? P.indptr[node + 1] : 0;
    sp_stream<T, U, RPW>(P, lp, e0, e1, acc);
    if (lp.g != 0 || !lp.act || node < 0) return;
    store_vec_nt<T>(P.Y, (int64_t)node * G.F + lp.col, VT::pack(acc));
}

// heavy rows: the groups' partials summed in ascending group order
template <class T>
__global__ void k_spmm_merge(SpParams P) {
    using VT = Vec<T>;
    constexpr int NV = VT::N;
    const SpGeom &G = P.g;
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= (int64_t)P.n_heavy * G.L) return;
    const int h = (int)(t / G.L);
    const int64_t col = (int64_t)(t % G.L) * NV;
    float acc[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) acc[k] = 0.f;
    for (int grp = P.partial_ofs[h]; grp < P.partial_ofs[h + 1]; ++grp) {
        const float *p = P.part + (int64_t)grp * G.F + col;
#pragma unroll
        for (int k = 0; k < NV; ++k) acc[k] += p[k];
    }
    store_vec<T>(P.Y, (int64_t)P.heavy[h] * G.F + col, VT::pack(acc));
}

static SpGeom sp_geom(int32_t N, int32_t F, gnn_dtype_t dt) {
    SpGeom g;
    g.N = N;
    g.F = F;
    g.L = (int32_t)(((int64_t)F * (dt == GNN_BF16 ? 2 : 4)) / 16);
    if (g.L <= kWave) {
        int sh = 0;
        while ((1 << sh) < g.L) ++sh;
        g.lr_shift = sh;
        g.G = kWave >> sh;
    } else {
        g.lr_shift = 6;
        g.G = 1;
        g.NFG = (g.L + kWave - 1) / kWave;
    }
    return g;
}

template <class T, int RPW, bool TR, int U = 4>
static int launch_spmm_main(gnn_plan_t plan, const SpParams &P, int kind, hipStream_t s) {
    constexpr int NV = Vec<T>::N;
    const int64_t light_waves = RPW == 1 ? (int64_t)P.n_light * P.g.NFG
                                         : P.n_long + ((int64_t)P.n_light - P.n_long + RPW - 1) / RPW;
    const int64_t blocks = (int64_t)P.n_groups * P.g.NFG + (light_waves + P.W - 1) / P.W;
    if (blocks >= (1ll << 31)) return GNN_ERR_INVALID_ARG;
    const size_t lds = P.n_groups ? (size_t)P.W * (1 << P.g.lr_shift) * NV * sizeof(float) : 0;
    return launch(plan, kind, k_spmm_main<T, U, RPW, TR>, dim3((unsigned)blocks), dim3(64 * P.W), lds, s, P);
}

template <class T, bool TR>
static int run_spmm(gnn_plan_t plan, SpParams &P, const int32_t *by_degree, const int2 *rng, int32_t n_long,
                    hipStream_t s) {
    const int k_main = TR ? K_SPMM_T_MAIN : K_SPMM_MAIN, k_merge = TR ? K_SPMM_T_MERGE : K_SPMM_MERGE;
    if (by_degree && P.g.NFG == 1 && P.g.G >= 2) {
        SpParams Q = P;
        Q.light = by_degree;
        Q.rng = rng;
        Q.n_long = rng ? n_long : 0;
        // two rows per wave: 10 entries per step in fp32 (on the mean-degree-8 power-law
        // graph 9, 11 and 12 measured slower, and 8 slower still), 8 in bf16
        constexpr int U2 = Vec<T>::bytes == 4 ? 10 : 8;
        if (P.g.G >= 4) GNN_TRY((launch_spmm_main<T, 4, TR>(plan, Q, k_main, s)));
        else GNN_TRY((launch_spmm_main<T, 2, TR, U2>(plan, Q, k_main, s)));
    } else {
        GNN_TRY((launch_spmm_main<T, 1, TR>(plan, P, k_main, s)));
    }
    const int64_t nm = (int64_t)P.n_heavy * P.g.L;
    if (nm) GNN_TRY(launch(plan, k_merge, k_spmm_merge<T>, grid1d(nm), dim3(256), 0, s, P));
    return GNN_OK;
}

// ------------------------------------------------- 16x16 block tiles (WSB)
//
// On a plan with a tile census, each tiled 16-row block (a 16-column block for
// the transposed product) runs in one 4-wave workgroup. Tile phase: per tile,
// the 16 gathered rows of X are staged in LDS as fp32 and the block product
// Y_b += W_t X_t runs on the matrix cores as 16x16x4 fp32 MFMA steps (wave w
// takes the 16-feature chunks w and w + 4), with W_t built in registers from
// the tile's bit mask and the entries' weights (from the in-degrees, the same
// expression as the cached weights). The 16 x F block result goes through LDS
// to the CSR lane geometry (4 rows per wave, 16-byte slices), which streams
// the block's residual entries with the cached residual weights, adds the
// tile result and writes the row once. fp32 throughout, one rounding to the
// storage type; no atomics.

typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

constexpr int kWsbWaves = 4;

struct WsbArgs {
    const int32_t *blocks;      // tiled row blocks (product) or column blocks (transposed product)
    int32_t n_blocks;
    const int32_t *tile_ptr;    // tile range of each block
    const int32_t *tile_ids;    // null: tiles in range order; else tile ids (by column block)
    const int32_t *tile_rc;     // (row block, column block) per tile
    const uint64_t *tile_mask;  // 4 words per tile, bit (dst % 16) * 16 + (src % 16)
    const int32_t *rptr, *ridx; // residual structure
    const float *rw;            // residual weights
    const int32_t *indptr;      // the CSR (in-degrees for the tile weights)
    int32_t norm;
};

// fp32 row stride of the staged block, 16 (mod 64) floats: the four rows one
// operand read touches start 16 banks apart
__host__ __device__ constexpr int wsb_stride(int F) { return F + ((16 - F) % 64 + 64) % 64; }

static size_t wsb_lds(int F) { return (size_t)(16 * wsb_stride(F) + 16 * (F + 4) + 16) * sizeof(float); }

// rows of at most 16 lanes (the residual pass packs 4 rows per wave) and whole 16-feature chunks
static bool wsb_supported(const SpGeom &g) { return g.F % 16 == 0 && g.L <= 16; }

template <class T, int U, bool TR>
__global__ __launch_bounds__(kWsbWaves * kWave) void k_spmm_wsb(SpParams P, WsbArgs A) {
    using VT = Vec<T>;
    constexpr int NV = VT::N;
    extern __shared__ float lds[];
    const SpGeom &G = P.g;
    const int F = G.F, N = G.N;
    const int xstride = wsb_stride(F), hstride = F + 4;
    float *xs = lds;                                   // [16][xstride] staged gathered rows
    float *hand = lds + 16 * xstride;                  // [16][hstride] tile result per output row
    float *gdeg = hand + 16 * hstride;                 // [16] in-degrees of the gathered rows
    const int blk = A.blocks[blockIdx.x];
    const int row0 = blk * 16;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), l = lane_id();
    const int m = l & 15, kq = l >> 4;
    const int nch = F / 16;
    f32x4_t acc[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // this lane's A-operand row: output row m of the block
    const float dout = row0 + m < N ? in_degree(A.indptr, row0 + m) : 0.f;
    const int t0 = A.tile_ptr[blk], t1 = A.tile_ptr[blk + 1];
    for (int t = t0; t < t1; ++t) {
        const int tid = A.tile_ids ? A.tile_ids[t] : t;
        const int s0 = 16 * A.tile_rc[2 * tid + (TR ? 0 : 1)];   // first gathered row
        __syncthreads();                                          // the previous tile's operands are read
        const int nvec = F / NV;
        for (int v = threadIdx.x; v < 16 * nvec; v += kWsbWaves * kWave) {
            const int r = v / nvec, c = (v % nvec) * NV;
            float x[NV];
            if (s0 + r < N) {
                VT::unpack(load_vec<T>(P.X, (int64_t)(s0 + r) * F + c), x);
            } else {
#pragma unroll
                for (int k = 0; k < NV; ++k) x[k] = 0.f;
            }
#pragma unroll
            for (int k = 0; k < NV; ++k) xs[r * xstride + c + k] = x[k];
        }
        if (threadIdx.x < 16) gdeg[threadIdx.x] = s0 + (int)threadIdx.x < N ? in_degree(A.indptr, s0 + threadIdx.x) : 0.f;
        const uint64_t w0 = A.tile_mask[4 * tid], w1 = A.tile_mask[4 * tid + 1], w2 = A.tile_mask[4 * tid + 2],
                       w3 = A.tile_mask[4 * tid + 3];
        __syncthreads();
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            // A operand of this step: lane (m, kq) holds W[m][4 st + kq]
            const int k = 4 * st + kq;
            const int bit = TR ? k * 16 + m : m * 16 + k;
            const uint64_t word = (bit >> 6) == 0 ? w0 : (bit >> 6) == 1 ? w1 : (bit >> 6) == 2 ? w2 : w3;
            const bool on = (word >> (bit & 63)) & 1ull;
            const float dg = gdeg[k];
            const float a = on ? (TR ? spmm_weight(A.norm, dg, dout) : spmm_weight(A.norm, dout, dg)) : 0.f;
#pragma unroll
            for (int ci = 0; ci < 2; ++ci) {
                const int c = w + kWsbWaves * ci;
                // B operand: lane (m, kq) holds X_t[4 st + kq][16 c + m]
                if (c < nch) acc[ci] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, xs[k * xstride + 16 * c + m], acc[ci], 0, 0, 0);
            }
        }
    }
    // D layout: lane (m, kq) holds rows 4 kq + i of column 16 c + m
#pragma unroll
    for (int ci = 0; ci < 2; ++ci) {
        const int c = w + kWsbWaves * ci;
        if (c < nch) {
#pragma unroll
            for (int i = 0; i < 4; ++i) hand[(4 * kq + i) * hstride + 16 * c + m] = acc[ci][i];
        }
    }
    __syncthreads();
    // residual entries: wave w takes the block's rows 4w .. 4w + 3
    const SpLane<NV, 4> lp(G, 0);
    const int r = 4 * w + (l >> 4);
    const int node = row0 + r;
    const int e0 = node < N ? A.rptr[node] : 0, e1 = node < N ? A.rptr[node + 1] : 0;
    SpParams Q = P;
    Q.indices = A.ridx;
    Q.w = A.rw;
    float y[NV];
    sp_stream<T, U, 4>(Q, lp, e0, e1, y);
    if (lp.g != 0 || !lp.act || node >= N) return;
#pragma unroll
    for (int k = 0; k < NV; ++k) y[k] += hand[r * hstride + lp.col + k];
    store_vec_nt<T>(P.Y, (int64_t)node * F + lp.col, VT::pack(y));
}

template <class T, bool TR>
static int launch_wsb(gnn_plan_t plan, const SpParams &P, const WsbArgs &A, hipStream_t s) {
    return launch(plan, TR ? K_SPMM_T_WSB : K_SPMM_WSB, k_spmm_wsb<T, 4, TR>, dim3((unsigned)A.n_blocks),
                  dim3(kWsbWaves * kWave), wsb_lds(P.g.F), s, P, A);
}

template <class T, bool TR>
static int run_spmm_tiled(gnn_plan_t plan, SpParams &P, const WsbArgs &A, hipStream_t s) {
    GNN_TRY((run_spmm<T, TR>(plan, P, nullptr, nullptr, 0, s)));
    return launch_wsb<T, TR>(plan, P, A, s);
}

// this file's kernels' index flag (checked builds)
GNN_INDEX_FAULT_READER(index_fault_spmm)

}  // namespace gnn

using namespace gnn;

extern "C" {

int gnn_spmm_prepare(gnn_plan_t plan, gnn_norm_t norm, hipStream_t stream) {
    if (!plan) return GNN_ERR_INVALID_ARG;
    if (norm != GNN_NORM_SUM && norm != GNN_NORM_MEAN && norm != GNN_NORM_GCN) return GNN_ERR_INVALID_ARG;
    const int32_t n = plan->n_nodes;
    const int64_t e = plan->n_edges;
    const size_t bytes = (size_t)std::max<int64_t>(e, 1) * 4;
    // a later call rewrites the cached weights in place (stream-ordered after
    // earlier products on the same stream), never freeing a buffer in use
    if (plan->spmm_w.bytes != bytes) GNN_TRY(dev_alloc(plan->spmm_w, bytes));
    if (n > 0)
        hipLaunchKernelGGL(k_spmm_w_rows, grid1d((int64_t)n * kWave), dim3(256), 0, stream, plan->indptr,
                           plan->indices, n, (int)norm, as<float>(plan->spmm_w));
    // entry ranges of the light rows in descending-degree order (graph structure only: built once)
    const size_t rb = (size_t)std::max(plan->fwd.n_light, 1) * sizeof(int2);
    if (plan->spmm_rng.bytes != rb) {
        GNN_TRY(dev_alloc(plan->spmm_rng, rb));
        if (plan->fwd.n_light > 0)
            hipLaunchKernelGGL(k_spmm_ranges, grid1d(plan->fwd.n_light), dim3(256), 0, stream, plan->indptr,
                               as<int32_t>(plan->fwd.by_degree), plan->fwd.n_light, as<int2>(plan->spmm_rng));
    }
    if (plan->has_csc) {
        if (plan->spmm_cw.bytes != bytes) GNN_TRY(dev_alloc(plan->spmm_cw, bytes));
        if (n > 0)
            hipLaunchKernelGGL(k_spmm_w_cols, grid1d((int64_t)n * kWave), dim3(256), 0, stream, plan->indptr,
                               as<int32_t>(plan->cindptr), as<int32_t>(plan->cindices), n, (int)norm,
                               as<float>(plan->spmm_cw));
        const size_t cb = (size_t)std::max(plan->bwd.n_light, 1) * sizeof(int2);
        if (plan->spmm_crng.bytes != cb) {
            GNN_TRY(dev_alloc(plan->spmm_crng, cb));
            if (plan->bwd.n_light > 0)
                hipLaunchKernelGGL(k_spmm_ranges, grid1d(plan->bwd.n_light), dim3(256), 0, stream,
                                   as<int32_t>(plan->cindptr), as<int32_t>(plan->bwd.by_degree), plan->bwd.n_light,
                                   as<int2>(plan->spmm_crng));
        }
    }
    if (plan->has_tiles) {
        // a tiled plan's residual entries (their weights, in residual order)
        const size_t rbytes = (size_t)std::max<int64_t>(plan->n_residual, 1) * 4;
        if (plan->spmm_rw.bytes != rbytes) GNN_TRY(dev_alloc(plan->spmm_rw, rbytes));
        if (n > 0)
            hipLaunchKernelGGL(k_spmm_w_res, grid1d((int64_t)n * kWave), dim3(256), 0, stream, plan->indptr,
                               as<int32_t>(plan->rindptr), as<int32_t>(plan->rindices), n, (int)norm, 1,
                               as<float>(plan->spmm_rw));
        if (plan->has_csc) {
            if (plan->spmm_rcw.bytes != rbytes) GNN_TRY(dev_alloc(plan->spmm_rcw, rbytes));
            if (n > 0)
                hipLaunchKernelGGL(k_spmm_w_res, grid1d((int64_t)n * kWave), dim3(256), 0, stream, plan->indptr,
                                   as<int32_t>(plan->rcindptr), as<int32_t>(plan->rcindices), n, (int)norm, 0,
                                   as<float>(plan->spmm_rcw));
        }
    }
    GNN_HIP(hipGetLastError());
    plan->spmm_norm = (int32_t)norm;
    return GNN_OK;
}

static int spmm_impl(gnn_plan_t plan, const int32_t *indptr, const int32_t *indices, int32_t N, int64_t E, int32_t F,
             const void *X, void *Y, int32_t transpose, gnn_dtype_t dtype, hipStream_t stream) {
    if (!plan || N < 0 || E < 0 || F < 1 || !indptr || (E > 0 && !indices)) return GNN_ERR_INVALID_ARG;
    if (plan->n_nodes != N || plan->n_edges != E || plan->indptr != indptr || plan->indices != indices)
        return GNN_ERR_INVALID_ARG;
    if (dtype != GNN_F32 && dtype != GNN_BF16) return GNN_ERR_UNSUPPORTED;
    if (((int64_t)F * (dtype == GNN_BF16 ? 2 : 4)) % 16) return GNN_ERR_UNSUPPORTED;
    if ((int64_t)N * F >= (1ll << 40)) return GNN_ERR_INVALID_ARG;
    if (plan->spmm_norm < 0) return GNN_ERR_INVALID_ARG;            // gnn_spmm_prepare first
    if (transpose && !plan->has_csc) return GNN_ERR_UNSUPPORTED;
    if (N > 0 && (!X || !Y)) return GNN_ERR_INVALID_ARG;
    if (!aligned16(X) || !aligned16(Y)) return GNN_ERR_ALIGNMENT;
    if (N == 0) return GNN_OK;
    GNN_TRY(checked_graph(indptr, indices, N, E, stream));
    SpParams P{};
    P.g = sp_geom(N, F, dtype);
    P.X = X;
    P.Y = Y;
    const Buckets &b = transpose ? plan->bwd : plan->fwd;
    P.indptr = transpose ? as<int32_t>(plan->cindptr) : indptr;
    P.indices = transpose ? as<int32_t>(plan->cindices) : indices;
    P.w = as<float>(transpose ? plan->spmm_cw : plan->spmm_w);
    P.light = as<int32_t>(b.sched);
    P.n_light = b.n_light;
    P.groups = as<int32_t>(b.groups);
    P.n_groups = b.n_groups;
    P.heavy = as<int32_t>(b.heavy);
    P.partial_ofs = as<int32_t>(b.partial_ofs);
    P.n_heavy = b.n_heavy;
    P.C = plan->opts.chunk;
    P.W = plan->opts.waves_per_group;
    if (P.n_groups) {
        void *ws = nullptr;
        GNN_TRY(plan_workspace(plan, (size_t)P.n_groups * F * sizeof(float), stream, &ws));
        P.part = (float *)ws;
    }
    if (plan->has_tiles && wsb_supported(P.g)) {
        // tiled blocks on the block kernel; the light rows outside them (one
        // per wave) and the heavy rows on the CSR kernel
        P.light = as<int32_t>(transpose ? plan->c_light_nt : plan->light_nt);
        P.n_light = transpose ? plan->n_c_light_nt : plan->n_light_nt;
        WsbArgs A{};
        A.blocks = as<int32_t>(transpose ? plan->tcb : plan->trb);
        A.n_blocks = transpose ? plan->n_tcb : plan->n_trb;
        A.tile_ptr = as<int32_t>(transpose ? plan->ctile_ptr : plan->tile_ptr);
        A.tile_ids = transpose ? as<int32_t>(plan->ctile) : nullptr;
        A.tile_rc = as<int32_t>(plan->tile_rc);
        A.tile_mask = as<uint64_t>(plan->tile_mask);
        A.rptr = as<int32_t>(transpose ? plan->rcindptr : plan->rindptr);
        A.ridx = as<int32_t>(transpose ? plan->rcindices : plan->rindices);
        A.rw = as<float>(transpose ? plan->spmm_rcw : plan->spmm_rw);
        A.indptr = indptr;
        A.norm = plan->spmm_norm;
        if (dtype == GNN_BF16)
            return transpose ? run_spmm_tiled<bf16_tag, true>(plan, P, A, stream)
                             : run_spmm_tiled<bf16_tag, false>(plan, P, A, stream);
        return transpose ? run_spmm_tiled<float, true>(plan, P, A, stream)
                         : run_spmm_tiled<float, false>(plan, P, A, stream);
    }
    const int32_t *by_degree = as<int32_t>(b.by_degree);
    const int2 *rng = as<int2>(transpose ? plan->spmm_crng : plan->spmm_rng);
    if (dtype == GNN_BF16)
        return transpose ? run_spmm<bf16_tag, true>(plan, P, by_degree, rng, b.n_long, stream)
                         : run_spmm<bf16_tag, false>(plan, P, by_degree, rng, b.n_long, stream);
    return transpose ? run_spmm<float, true>(plan, P, by_degree, rng, b.n_long, stream)
                     : run_spmm<float, false>(plan, P, by_degree, rng, b.n_long, stream);
}

int gnn_spmm(gnn_plan_t plan, const int32_t *indptr, const int32_t *indices, int32_t N, int64_t E, int32_t F,
             const void *X, void *Y, int32_t transpose, gnn_dtype_t dtype, hipStream_t stream) {
    return finish_call(spmm_impl(plan, indptr, indices, N, E, F, X, Y, transpose, dtype, stream), stream);
}

}  // extern "C"
