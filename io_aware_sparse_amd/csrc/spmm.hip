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
// one 16-byte slice of a feature row; light rows run from the
// packed-order list 4 per wave when a row spans at most 16 lanes
// (256 bytes), 2 per wave with 10 edges per step in fp32 (8 in bf16) when it
// spans 17-32 lanes (512 bytes), else one per wave; the packed waves read each row's entry
// range from a record cached by gnn_spmm_prepare, alongside the row id
// (rows are short: one dependent load fewer before the gathers). The light
// rows of more than 128 entries, which head the packed list, get a wave each
// in the same launch (all its edge groups on one row), so the longest light
// rows take half or a quarter of the steps they would take packed; heavy
// rows run as the plan's chunk groups, their W waves
// summed in LDS and the groups summed in ascending order by a second pass.
// fp32 accumulation, output rounded to the storage type; no atomics, so the
// result is bitwise reproducible. The transposed product (dX = A_w^T dY) is
// the same kernel over the transposed adjacency and its buckets.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>

#include "attn_core.h"
#include "gnn_spmm.h"

namespace gnn {

// weights in CSR order: one wave per row
__global__ void k_spmm_w_rows(const int32_t *indptr, const int32_t *indices, int32_t n, int norm, float *w) {
    const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / kWave;
    const int lane = threadIdx.x % kWave;
    if (i >= n) return;
    const int32_t e0 = indptr[i], e1 = indptr[i + 1];
    const float di = (float)(e1 - e0);
    for (int32_t e = e0 + lane; e < e1; e += kWave) {
        float v = 1.f;
        if (norm == GNN_NORM_MEAN) v = 1.f / di;
        if (norm == GNN_NORM_GCN) {
            const int32_t j = indices[e];
            const float dj = (float)(indptr[j + 1] - indptr[j]);
            v = dj > 0.f ? 1.f / sqrtf(di * dj) : 0.f;      // a source without entries contributes nothing
        }
        w[e] = v;
    }
}

// weights in transposed order: the entries of source j name destinations i
__global__ void k_spmm_w_cols(const int32_t *indptr, const int32_t *cindptr, const int32_t *cindices, int32_t n,
                              int norm, float *cw) {
    const int64_t j = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / kWave;
    const int lane = threadIdx.x % kWave;
    if (j >= n) return;
    const float dj = (float)(indptr[j + 1] - indptr[j]);
    for (int32_t e = cindptr[j] + lane; e < cindptr[j + 1]; e += kWave) {
        const int32_t i = cindices[e];
        const float di = (float)(indptr[i + 1] - indptr[i]);
        float v = 1.f;
        if (norm == GNN_NORM_MEAN) v = 1.f / di;
        if (norm == GNN_NORM_GCN) v = dj > 0.f ? 1.f / sqrtf(di * dj) : 0.f;
        cw[e] = v;
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
        jn = P.indices[e0 + li];
        wn = P.w[e0 + li];
    }
    for (int base = e0; RPW == 1 ? base < e1 : __any(base < e1); base += S) {
        const int jc = jn;
        const float wc = wn;
        jn = -1;
        wn = 0.f;
        if (li < S && base + S + li < e1) {
            jn = P.indices[base + S + li];
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
    GNN_HIP(hipGetLastError());
    plan->spmm_norm = (int32_t)norm;
    return GNN_OK;
}

int gnn_spmm(gnn_plan_t plan, const int32_t *indptr, const int32_t *indices, int32_t N, int64_t E, int32_t F,
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
    const int32_t *by_degree = as<int32_t>(b.by_degree);
    const int2 *rng = as<int2>(transpose ? plan->spmm_crng : plan->spmm_rng);
    if (dtype == GNN_BF16)
        return transpose ? run_spmm<bf16_tag, true>(plan, P, by_degree, rng, b.n_long, stream)
                         : run_spmm<bf16_tag, false>(plan, P, by_degree, rng, b.n_long, stream);
    return transpose ? run_spmm<float, true>(plan, P, by_degree, rng, b.n_long, stream)
                     : run_spmm<float, false>(plan, P, by_degree, rng, b.n_long, stream);
}

}  // extern "C"
