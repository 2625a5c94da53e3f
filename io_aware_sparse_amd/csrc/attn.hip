// Fused CSR neighbourhood attention kernels for gfx950.
//
// "On Efficient Scaling of GNNs via IO-Aware Layers Implementations",
// technical summary, Methodology (attention-based layers): one streaming pass
// over each node's neighbours computes the scores, the softmax normalisation
// and the value aggregation; the forward keeps running statistics in
// registers (online softmax) so no edge logit is written; the backward reads
// a cached per-node log-sum-exp and recomputes every weight on the fly.
// Degree-aware tiling (same section): light nodes (in-degree <= T) take one
// wavefront each (two per wavefront for rows of 257-512 bytes in the
// forward); heavy nodes are cut into chunk groups whose waves each
// stream <= C edges, merge their partial (m, l, acc) states in LDS, write one
// partial per group, and a second pass merges a node's partials.
//
// Lane geometry. A node's feature row is H*D elements. One lane holds one
// 16-byte vector (4 fp32 or 8 bf16) of it, so a head occupies LH = D*s/16
// lanes and a wave covers HW = min(H, 64/LH) heads ("head group"). The LR
// lanes of one row (HW*LH rounded up to a power of two) form an edge group;
// the wave runs G = 64/LR edge groups side by side, each on different edges
// of the same node, and merges them at the end. Each group gathers U edges
// per step, so a wave keeps G*U row gathers in flight. Per-head dot products
// are reduced across LH lanes with DPP moves. Scores are kept in log2 units
// (the scale is pre-multiplied by log2 e) so exp2 is a single instruction.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <mutex>

#include "attn_core.h"

namespace gnn {

// Heavy blocks at the head of the forward launch: one per (chunk group, head
// group), or, in XCD order, 8 per W rows of slots (n_slots is 8 times the
// largest range's group count)
__host__ __device__ inline int64_t fwd_heavy_blocks(const FwdParams &P) {
    return P.gperm ? 8 * (((int64_t)P.n_slots / 8 + P.W - 1) / P.W) : (int64_t)P.n_slots * P.g.NHG;
}

// a heavy group's partial online-softmax state (acc; m and l per head)
template <int NV>
__device__ __forceinline__ void write_partial(const FwdParams &P, const LanePos &lp, int grp, const SoftState<NV> &st) {
    const int64_t rowlen = (int64_t)P.g.H * P.g.D;
#pragma unroll
    for (int k = 0; k < NV; ++k) P.ws_acc[(int64_t)grp * rowlen + lp.col + k] = st.acc[k];
    if (lp.dv == 0) {
        P.ws_ml[((int64_t)grp * P.g.H + lp.h) * 2 + 0] = st.m;
        P.ws_ml[((int64_t)grp * P.g.H + lp.h) * 2 + 1] = st.l;
    }
}

// RPW > 1: the light rows run RPW per wave (rows of at most 64/RPW lanes).
template <class T, int LH, int MODE, int U, int RPW>
__global__ __launch_bounds__(512) void k_fwd_main(FwdParams P) {
    using VT = Vec<T>;
    constexpr int NV = VT::N;
    extern __shared__ float lds[];
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int heavy_blocks = (int)fwd_heavy_blocks(P);
    if ((int)blockIdx.x < heavy_blocks) {
        if (P.gperm) {
            // XCD-ordered source-range groups (one head group): the block that
            // dispatch puts on XCD r = blockIdx % 8 takes the next W groups of
            // range r, one per wave; a wave streams its whole group and writes
            // its own partial state (no barrier on this path)
            const int slot = ((int)(blockIdx.x / 8) * P.W + w) * 8 + (int)(blockIdx.x % 8);
            const int grp = slot < P.n_slots ? P.gperm[slot] : -1;
            if (grp < 0) return;
            const LanePos lp = lane_pos<LH, NV>(P.g, 0);
            SoftState<NV> st;
            fwd_stream<T, LH, MODE, U>(P, lp, P.groups[3 * grp], P.groups[3 * grp + 1], P.groups[3 * grp + 2], st);
            if (lp.lane < (1 << P.g.lr_shift) && lp.act) write_partial(P, lp, grp, st);
            return;
        }
        const int grp = blockIdx.x / P.g.NHG, hg = blockIdx.x % P.g.NHG;
        const int node = P.groups[3 * grp], g0 = P.groups[3 * grp + 1], g1 = P.groups[3 * grp + 2];
        const int e0 = min(g1, g0 + w * P.C), e1 = min(g1, e0 + P.C);
        const LanePos lp = lane_pos<LH, NV>(P.g, hg);
        SoftState<NV> st;
        fwd_stream<T, LH, MODE, U>(P, lp, node, e0, e1, st);
        // LDS merge of the W waves (ascending wave order)
        const int LR = 1 << P.g.lr_shift;
        float *mine = lds + (size_t)w * LR * (NV + 2);
        if (lp.lane < LR) {
            mine[lp.lane * (NV + 2) + 0] = st.m;
            mine[lp.lane * (NV + 2) + 1] = st.l;
#pragma unroll
            for (int k = 0; k < NV; ++k) mine[lp.lane * (NV + 2) + 2 + k] = st.acc[k];
        }
        __syncthreads();
        if (w != 0 || lp.lane >= LR) return;
        for (int v = 1; v < P.W; ++v) {
            const float *o = lds + ((size_t)v * LR + lp.lane) * (NV + 2);
            float a2[NV];
#pragma unroll
            for (int k = 0; k < NV; ++k) a2[k] = o[2 + k];
            merge_state(st, o[0], o[1], a2);
        }
        if (lp.act) write_partial(P, lp, grp, st);
        return;
    }
    // the packed rows come from the descending-degree list, which has no id
    // locality for an XCD-aware order to keep; one-row waves follow the plan's
    // launch order, mostly id order, and take the XCD-aware block order
    const int64_t lblock = blockIdx.x - heavy_blocks;
    const int64_t item = (RPW > 1 ? lblock : xcd_block(lblock, gridDim.x - heavy_blocks)) * P.W + w;
    if (RPW > 1) {                        // RPW rows of the light list per wave (NHG == 1)
        if (item < P.n_long) {
            // a long row at the head of the packed list: the whole wave, all its edge groups
            const int node = P.light[item];
            const int e0 = P.indptr[node], e1 = P.indptr[node + 1];
            const LanePos lp = lane_pos<LH, NV>(P.g, 0);
            SoftState<NV> st;
            fwd_stream<T, LH, MODE, U>(P, lp, node, e0, e1, st);
            write_out<T, NV>(P, lp, node, st);
            return;
        }
        const int64_t ni0 = P.n_long + (item - P.n_long) * RPW;
        if (ni0 >= P.n_light) return;
        const int64_t ni = ni0 + lane_id() / (kWave / RPW);
        const int node = ni < P.n_light ? P.light[ni] : -1;
        const int e0 = node >= 0 ? P.indptr[node] : 0, e1 = node >= 0 ? P.indptr[node + 1] : 0;
        const LanePos lp = lane_pos<LH, NV, RPW>(P.g, 0);
        SoftState<NV> st;
        fwd_stream<T, LH, MODE, U, RPW>(P, lp, node < 0 ? 0 : node, e0, e1, st);
        if (node >= 0) write_out<T, NV>(P, lp, node, st);
        return;
    }
    const int64_t ni = item / P.g.NHG;
    if (ni >= P.n_light) return;
    const int hg = (int)(item % P.g.NHG);
    const int node = P.light ? P.light[ni] : (int)ni;
    const int e0 = P.indptr[node], e1 = P.indptr[node + 1];
    const LanePos lp = lane_pos<LH, NV>(P.g, hg);
    SoftState<NV> st;
    fwd_stream<T, LH, MODE, U>(P, lp, node, e0, e1, st);
    write_out<T, NV>(P, lp, node, st);
}

// Second pass: one 4-wave workgroup per (heavy node, head group) merges the
// node's partials in a fixed order: wave w takes partials p0 + w*G + g
// (stride 4G), merges them in sequence, the wave's groups merge by a fixed
// xor tree, and wave 0 merges the four wave states in ascending order.
constexpr int kMergeWaves = 4;

template <class T, int LH>
__global__ __launch_bounds__(256) void k_fwd_merge(FwdParams P) {
    using VT = Vec<T>;
    constexpr int NV = VT::N;
    __shared__ float red[kMergeWaves][kWave][NV + 2];
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int k = (int)(blockIdx.x / P.g.NHG), hg = (int)(blockIdx.x % P.g.NHG);
    const int node = P.heavy[k];
    const int p0 = P.partial_ofs[k], p1 = P.partial_ofs[k + 1];
    const LanePos lp = lane_pos<LH, NV>(P.g, hg);
    const int64_t rowlen = (int64_t)P.g.H * P.g.D;
    SoftState<NV> st;
    st.m = kNegInf;
    st.l = 0.f;
#pragma unroll
    for (int q = 0; q < NV; ++q) st.acc[q] = 0.f;
    if (lp.act) {
        for (int p = p0 + w * P.g.G + lp.g; p < p1; p += kMergeWaves * P.g.G) {
            float a2[NV];
#pragma unroll
            for (int q = 0; q < NV; ++q) a2[q] = P.ws_acc[(int64_t)p * rowlen + lp.col + q];
            merge_state(st, P.ws_ml[((int64_t)p * P.g.H + lp.h) * 2], P.ws_ml[((int64_t)p * P.g.H + lp.h) * 2 + 1], a2);
        }
    }
    merge_groups(st, P.g.lr_shift);
    red[w][lp.lane][0] = st.m;
    red[w][lp.lane][1] = st.l;
#pragma unroll
    for (int q = 0; q < NV; ++q) red[w][lp.lane][2 + q] = st.acc[q];
    __syncthreads();
    if (w != 0) return;
    for (int v = 1; v < kMergeWaves; ++v) {
        float a2[NV];
#pragma unroll
        for (int q = 0; q < NV; ++q) a2[q] = red[v][lp.lane][2 + q];
        merge_state(st, red[v][lp.lane][0], red[v][lp.lane][1], a2);
    }
    write_out<T, NV>(P, lp, node, st);
}

// Heavy partial layout per group slot: A [H*D], B [H*D], Delta [H].
template <class T, int LH, int U>
__global__ __launch_bounds__(512) void k_bwd_dst_main(BwdParams P) {
    using VT = Vec<T>;
    constexpr int NV = VT::N;
    extern __shared__ float lds[];
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int heavy_blocks = P.a_n_groups * P.g.NHG;
    const int64_t rowlen = (int64_t)P.g.H * P.g.D;
    if ((int)blockIdx.x < heavy_blocks) {
        const int grp = blockIdx.x / P.g.NHG, hg = blockIdx.x % P.g.NHG;
        const int node = P.a_groups[3 * grp], g0 = P.a_groups[3 * grp + 1], g1 = P.a_groups[3 * grp + 2];
        const int e0 = min(g1, g0 + w * P.C), e1 = min(g1, e0 + P.C);
        const LanePos lp = lane_pos<LH, NV>(P.g, hg);
        float x[3][NV];
        float lse2;
        bwd_dst_stream<T, LH, U>(P, lp, node, e0, e1, x[0], x[1], x[2][0], lse2);
#pragma unroll
        for (int k = 1; k < NV; ++k) x[2][k] = 0.f;
        if (!lds_sum_waves<NV, 3>(lds, w, P.W, lp.lane, 1 << P.g.lr_shift, x) || !lp.act) return;
        float *slot = P.ws_a + (int64_t)grp * (2 * rowlen + P.g.H);
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            slot[lp.col + k] = x[0][k];
            slot[rowlen + lp.col + k] = x[1][k];
        }
        if (lp.dv == 0) slot[2 * rowlen + lp.h] = x[2][0];
        return;
    }
    const int64_t item = xcd_block(blockIdx.x - heavy_blocks, gridDim.x - heavy_blocks) * P.W + w;
    const int64_t ni = item / P.g.NHG;
    if (ni >= P.a_n_light) return;
    const int hg = (int)(item % P.g.NHG);
    const int node = P.a_light[ni];
    const LanePos lp = lane_pos<LH, NV>(P.g, hg);
    float A[NV], B[NV];
    float dsum, lse2;
    bwd_dst_stream<T, LH, U>(P, lp, node, P.indptr[node], P.indptr[node + 1], A, B, dsum, lse2);
    if (lp.g != 0 || !lp.act) return;
    store_dq<T, NV>(P, lp, node, A, B, dsum, lse2);
}

template <class T, int LH>
__global__ __launch_bounds__(256) void k_bwd_dst_merge(BwdParams P) {
    using VT = Vec<T>;
    constexpr int NV = VT::N;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t item = (int64_t)blockIdx.x * (blockDim.x / kWave) + w;
    if (item >= (int64_t)P.a_n_heavy * P.g.NHG) return;
    const int k = (int)(item / P.g.NHG), hg = (int)(item % P.g.NHG);
    const int node = P.a_heavy[k];
    const int p0 = P.a_ofs[k], p1 = P.a_ofs[k + 1];
    const LanePos lp = lane_pos<LH, NV>(P.g, hg);
    const int64_t rowlen = (int64_t)P.g.H * P.g.D;
    float A[NV], B[NV];
    float dsum = 0.f, lse2 = kNegInf;
#pragma unroll
    for (int q = 0; q < NV; ++q) A[q] = B[q] = 0.f;
    if (lp.act) {
        for (int p = p0 + lp.g; p < p1; p += P.g.G) {
            const float *slot = P.ws_a + (int64_t)p * (2 * rowlen + P.g.H);
#pragma unroll
            for (int q = 0; q < NV; ++q) {
                A[q] += slot[lp.col + q];
                B[q] += slot[rowlen + lp.col + q];
            }
            dsum += slot[2 * rowlen + lp.h];
        }
        lse2 = P.LSE[(int64_t)node * P.g.H + lp.h] * kLog2e;
    }
    sum_groups(A, P.g.lr_shift);
    sum_groups(B, P.g.lr_shift);
    for (int off = 1 << P.g.lr_shift; off < kWave; off <<= 1) dsum += xor_lane(dsum, off);
    if (lp.g != 0 || !lp.act) return;
    store_dq<T, NV>(P, lp, node, A, B, dsum, lse2);
}

template <class T, int LH, int U>
__global__ __launch_bounds__(512) void k_bwd_src_main(BwdParams P) {
    using VT = Vec<T>;
    constexpr int NV = VT::N;
    extern __shared__ float lds[];
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int heavy_blocks = P.b_n_groups * P.g.NHG;
    const int64_t rowlen = (int64_t)P.g.H * P.g.D;
    if ((int)blockIdx.x < heavy_blocks) {
        const int grp = blockIdx.x / P.g.NHG, hg = blockIdx.x % P.g.NHG;
        const int node = P.b_groups[3 * grp], g0 = P.b_groups[3 * grp + 1], g1 = P.b_groups[3 * grp + 2];
        const int e0 = min(g1, g0 + w * P.C), e1 = min(g1, e0 + P.C);
        const LanePos lp = lane_pos<LH, NV>(P.g, hg);
        float x[2][NV];
        bwd_src_stream<T, LH, U>(P, lp, node, e0, e1, x[0], x[1]);
        if (!lds_sum_waves<NV, 2>(lds, w, P.W, lp.lane, 1 << P.g.lr_shift, x) || !lp.act) return;
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            P.ws_b[((int64_t)grp * 2 + 0) * rowlen + lp.col + k] = x[0][k];
            P.ws_b[((int64_t)grp * 2 + 1) * rowlen + lp.col + k] = x[1][k];
        }
        return;
    }
    const int64_t item = xcd_block(blockIdx.x - heavy_blocks, gridDim.x - heavy_blocks) * P.W + w;
    const int64_t ni = item / P.g.NHG;
    if (ni >= P.b_n_light) return;
    const int hg = (int)(item % P.g.NHG);
    const int node = P.b_light[ni];
    const LanePos lp = lane_pos<LH, NV>(P.g, hg);
    float dk[NV], dv[NV];
    bwd_src_stream<T, LH, U>(P, lp, node, P.cindptr[node], P.cindptr[node + 1], dk, dv);
    if (lp.g != 0 || !lp.act) return;
    store_scaled<T, NV>(P.dK, (int64_t)node * rowlen + lp.col, dk, P.scale);
    store_scaled<T, NV>(P.dV, (int64_t)node * rowlen + lp.col, dv, 1.f);
}

template <class T, int LH>
__global__ __launch_bounds__(256) void k_bwd_src_merge(BwdParams P) {
    using VT = Vec<T>;
    constexpr int NV = VT::N;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t item = (int64_t)blockIdx.x * (blockDim.x / kWave) + w;
    if (item >= (int64_t)P.b_n_heavy * P.g.NHG) return;
    const int k = (int)(item / P.g.NHG), hg = (int)(item % P.g.NHG);
    const int node = P.b_heavy[k];
    const int p0 = P.b_ofs[k], p1 = P.b_ofs[k + 1];
    const LanePos lp = lane_pos<LH, NV>(P.g, hg);
    const int64_t rowlen = (int64_t)P.g.H * P.g.D;
    float dk[NV], dv[NV];
#pragma unroll
    for (int q = 0; q < NV; ++q) dk[q] = dv[q] = 0.f;
    if (lp.act) {
        for (int p = p0 + lp.g; p < p1; p += P.g.G) {
#pragma unroll
            for (int q = 0; q < NV; ++q) {
                dk[q] += P.ws_b[((int64_t)p * 2 + 0) * rowlen + lp.col + q];
                dv[q] += P.ws_b[((int64_t)p * 2 + 1) * rowlen + lp.col + q];
            }
        }
    }
    sum_groups(dk, P.g.lr_shift);
    sum_groups(dv, P.g.lr_shift);
    if (lp.g != 0 || !lp.act) return;
    store_scaled<T, NV>(P.dK, (int64_t)node * rowlen + lp.col, dk, P.scale);
    store_scaled<T, NV>(P.dV, (int64_t)node * rowlen + lp.col, dv, 1.f);
}

// ======================================================================
// host side
// ======================================================================

template <class T, int LH, int MODE, int U, int RPW>
static int launch_fwd_main(gnn_plan_t plan, const FwdParams &P, hipStream_t s) {
    constexpr int NV = Vec<T>::N;
    const int kind_main = MODE == M_GT ? K_FWD_MAIN : K_GAT_MAIN;
    const int64_t light_waves = RPW == 1 ? (int64_t)P.n_light * P.g.NHG
                                         : P.n_long + ((int64_t)P.n_light - P.n_long + RPW - 1) / RPW;
    const int64_t blocks = fwd_heavy_blocks(P) + (light_waves + P.W - 1) / P.W;
    if (blocks >= (1ll << 31)) return GNN_ERR_INVALID_ARG;
    const size_t lds = P.n_groups ? (size_t)P.W * (1 << P.g.lr_shift) * (NV + 2) * sizeof(float) : 0;
    return launch(plan, kind_main, k_fwd_main<T, LH, MODE, U, RPW>, dim3((unsigned)blocks), dim3(64 * P.W), lds, s,
                  P);
}

// Light rows of 257-512 bytes (two edge groups per wave) on a plan run from
// the packed-order list, 2 per wave with 8 edges per step (GATv2) or 7 (GT:
// 88 instead of 97 VGPRs for fp32, five waves per SIMD instead of four), so
// each row keeps about the edges per step it would have alone and a wave has
// twice the rows in flight; the rows of more than 128 edges at the head of
// that list take a wave each (both edge groups, 16 or 14 edges per step), so
// the longest light rows do not set the kernel's duration. Otherwise one
// (row, head group) per wave, 4 edges per group and step.
template <class T, int LH, int MODE>
static int run_fwd(gnn_plan_t plan, FwdParams &P, const int32_t *by_degree, hipStream_t s) {
    const int kind_merge = MODE == M_GT ? K_FWD_MERGE : K_GAT_MERGE;
    if (by_degree && P.g.NHG == 1 && P.g.G == 2) {
        FwdParams Q = P;
        Q.light = by_degree;
        Q.n_long = plan->fwd.n_long;
        GNN_TRY((launch_fwd_main<T, LH, MODE, MODE == M_GT ? 7 : 8, 2>(plan, Q, s)));
    } else {
        GNN_TRY((launch_fwd_main<T, LH, MODE, 4, 1>(plan, P, s)));
    }
    if (P.n_heavy) {
        const int64_t mb = (int64_t)P.n_heavy * P.g.NHG;
        GNN_TRY(launch(plan, kind_merge, k_fwd_merge<T, LH>, dim3((unsigned)mb), dim3(64 * kMergeWaves), 0, s, P));
    }
    return GNN_OK;
}

template <int MODE>
static int dispatch_fwd(gnn_plan_t plan, FwdParams &P, const int32_t *by_degree, gnn_dtype_t dt, int D,
                        hipStream_t s) {
    if (dt == GNN_F32) {
        switch (D) {
            case 16: return run_fwd<float, 4, MODE>(plan, P, by_degree, s);
            case 32: return run_fwd<float, 8, MODE>(plan, P, by_degree, s);
            case 64: return run_fwd<float, 16, MODE>(plan, P, by_degree, s);
            case 128: return run_fwd<float, 32, MODE>(plan, P, by_degree, s);
        }
    } else {
        switch (D) {
            case 16: return run_fwd<bf16_tag, 2, MODE>(plan, P, by_degree, s);
            case 32: return run_fwd<bf16_tag, 4, MODE>(plan, P, by_degree, s);
            case 64: return run_fwd<bf16_tag, 8, MODE>(plan, P, by_degree, s);
            case 128: return run_fwd<bf16_tag, 16, MODE>(plan, P, by_degree, s);
        }
    }
    return GNN_ERR_UNSUPPORTED;
}

// fixed_ws: when non-null, the heavy partials go there (at most fixed_bytes)
// instead of the plan workspace, and nothing is allocated.
static int fwd_common(gnn_plan_t plan, const int32_t *indptr, const int32_t *indices, int32_t N, int64_t E,
                      int32_t H, int32_t D, const void *Q, const void *K, const void *V, void *O, float *LSE,
                      const float *att, float slope, float mul, int mode, gnn_dtype_t dtype, hipStream_t s,
                      float *fixed_ws = nullptr, size_t fixed_bytes = 0) {
    GNN_TRY(check_common(plan, indptr, indices, N, E, H, D, dtype));
    if (N > 0 && (!Q || !K || !V || !O)) return GNN_ERR_INVALID_ARG;
    if (mode != M_GT && N > 0 && !att) return GNN_ERR_INVALID_ARG;
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O)) return GNN_ERR_ALIGNMENT;
    if (mode != M_GT && !aligned16(att)) return GNN_ERR_ALIGNMENT;
    if (N == 0) return GNN_OK;
    if (!fixed_ws) GNN_TRY(checked_graph(indptr, indices, N, E, s));   // the allocation-free path skips it
    FwdParams P{};
    const int LH = lanes_per_head(dtype, D);
    P.g = make_geom(N, H, D, LH);
    P.indptr = indptr;
    P.indices = indices;
    P.Q = Q;
    P.K = K;
    P.V = V;
    P.O = O;
    P.LSE = LSE;
    P.att = att;
    P.slope = slope;
    P.mul = mul;
    if (plan) {
        P.light = as<int32_t>(plan->fwd.sched);
        P.n_light = plan->fwd.n_light;
        P.groups = as<int32_t>(plan->fwd.groups);
        P.n_groups = plan->fwd.n_groups;
        P.heavy = as<int32_t>(plan->fwd.heavy);
        P.partial_ofs = as<int32_t>(plan->fwd.partial_ofs);
        P.n_heavy = plan->fwd.n_heavy;
        P.gperm = nullptr;
        P.n_slots = P.n_groups;
        // heavy rows split at source ranges, XCD-ordered: worth it when one
        // range's gathered rows come near an XCD's L2 (a 6.4 MiB range of a
        // 51 MiB table gathers about twice as fast as the whole table; 22 MiB
        // ranges gain nothing), and only with one head group, whose blocks
        // are the launch slots themselves
        const int64_t gathered = (int64_t)N * H * D * (dtype == GNN_BF16 ? 2 : 4) * (mode == M_GAT_ALIAS ? 1 : 2);
        if (plan->xsplit.n_groups && P.g.NHG == 1 && (gathered + 7) / 8 <= kXsplitMaxRangeBytes) {
            P.groups = as<int32_t>(plan->xsplit.groups);
            P.n_groups = plan->xsplit.n_groups;
            P.partial_ofs = as<int32_t>(plan->xsplit.partial_ofs);
            P.gperm = as<int32_t>(plan->xsplit.order);
            P.n_slots = plan->xsplit.n_slots;
        }
        P.C = plan->opts.chunk;
        P.W = plan->opts.waves_per_group;
        if (P.n_groups) {
            const size_t rowlen = (size_t)H * D;
            const size_t bytes = (size_t)P.n_groups * (rowlen + 2 * H) * sizeof(float);
            void *ws = fixed_ws;
            if (fixed_ws) {
                if (bytes > fixed_bytes) return GNN_ERR_SCRATCH;
            } else {
                GNN_TRY(plan_workspace(plan, bytes, s, &ws));
            }
            P.ws_acc = (float *)ws;
            P.ws_ml = P.ws_acc + (size_t)P.n_groups * rowlen;
        }
    } else {
        P.light = nullptr;
        P.n_light = N;
        P.W = 4;
        P.C = 1;
    }
    // tiled plan: the CSR kernels take the light rows outside tiled row
    // blocks, the tile kernel the tiled blocks (tiles + residual edges)
    const bool tiles = plan && plan->has_tiles && mode == M_GT && tile_supported(dtype, D);
    if (tiles) {
        P.light = as<int32_t>(plan->light_nt);
        P.n_light = plan->n_light_nt;
        GNN_TRY(dispatch_fwd<M_GT>(plan, P, nullptr, dtype, D, s));   // light rows outside tiled blocks: one per wave
        return launch_tile_fwd(plan, P, D, s);
    }
    const int32_t *by_degree = plan ? as<int32_t>(plan->fwd.by_degree) : nullptr;
    if (mode == M_GT) return dispatch_fwd<M_GT>(plan, P, by_degree, dtype, D, s);
    if (mode == M_GAT_ALIAS) return dispatch_fwd<M_GAT_ALIAS>(plan, P, by_degree, dtype, D, s);
    return dispatch_fwd<M_GAT_SEPV>(plan, P, by_degree, dtype, D, s);
}

template <class T, int LH>
static int run_bwd(gnn_plan_t plan, BwdParams &P, hipStream_t s, bool tiles) {
    constexpr int U = 2;
    constexpr int NV = Vec<T>::N;
    const int LR = 1 << P.g.lr_shift;
    {
        const int64_t lb = ((int64_t)P.a_n_light * P.g.NHG + P.W - 1) / P.W;
        const int64_t blocks = (int64_t)P.a_n_groups * P.g.NHG + lb;
        if (blocks >= (1ll << 31)) return GNN_ERR_INVALID_ARG;
        const size_t lds = P.a_n_groups ? (size_t)P.W * LR * 3 * NV * sizeof(float) : 0;
        GNN_TRY(launch(plan, K_BWD_DST_MAIN, k_bwd_dst_main<T, LH, U>, dim3((unsigned)blocks), dim3(64 * P.W), lds, s,
                       P));
        if (P.a_n_heavy)
            GNN_TRY(launch(plan, K_BWD_DST_MERGE, k_bwd_dst_merge<T, LH>,
                           dim3((unsigned)(((int64_t)P.a_n_heavy * P.g.NHG + 3) / 4)), dim3(256), 0, s, P));
        if (tiles) GNN_TRY(launch_tile_bwd_dst(plan, P, P.g.D, s));
    }
    {
        const int64_t lb = ((int64_t)P.b_n_light * P.g.NHG + P.W - 1) / P.W;
        const int64_t blocks = (int64_t)P.b_n_groups * P.g.NHG + lb;
        if (blocks >= (1ll << 31)) return GNN_ERR_INVALID_ARG;
        const size_t lds = P.b_n_groups ? (size_t)P.W * LR * 2 * NV * sizeof(float) : 0;
        GNN_TRY(launch(plan, K_BWD_SRC_MAIN, k_bwd_src_main<T, LH, U>, dim3((unsigned)blocks), dim3(64 * P.W), lds, s,
                       P));
        if (P.b_n_heavy)
            GNN_TRY(launch(plan, K_BWD_SRC_MERGE, k_bwd_src_merge<T, LH>,
                           dim3((unsigned)(((int64_t)P.b_n_heavy * P.g.NHG + 3) / 4)), dim3(256), 0, s, P));
        if (tiles) GNN_TRY(launch_tile_bwd_src(plan, P, P.g.D, s));
    }
    return GNN_OK;
}

// ---------------------------------------------------------------------------
// Allocation-free forward. The heavy rows' partial states live in this
// file-scope device array instead of the plan workspace. In host code the
// name `scratch` is only a host-side stand-in for the symbol: its device
// address is looked up once per device (hipGetSymbolAddress, with that device
// current) and only that address is passed to kernels. Every call on a GPU
// shares that GPU's copy.
// ---------------------------------------------------------------------------
static __device__ __align__(256) float scratch[GNN_NOALLOC_SCRATCH_BYTES / sizeof(float)];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static float *g_scratch_dev[kMaxDevices] = {};

// device address of the current device's copy of `scratch`
static int scratch_on_current_device(float **out) {
    int dev = 0;
    GNN_HIP(hipGetDevice(&dev));
    if (dev < 0 || dev >= kMaxDevices) return GNN_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void *p = nullptr;
        GNN_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
        if (!p) return GNN_ERR_HIP;
        g_scratch_dev[dev] = static_cast<float *>(p);
    }
    *out = g_scratch_dev[dev];
    return GNN_OK;
}

// this file's kernels' index flag (checked builds)
GNN_INDEX_FAULT_READER(index_fault_attn)

}  // namespace gnn

using namespace gnn;

extern "C" {

int gnn_attn_fwd(gnn_plan_t plan, const int32_t *indptr, const int32_t *indices, int32_t N, int64_t E, int32_t H,
                 int32_t D, const void *Q, const void *K, const void *V, void *O, float *LSE, float scale,
                 gnn_dtype_t dtype, hipStream_t stream) {
    const float sc = scale > 0.f ? scale : (float)(1.0 / std::sqrt((double)std::max(D, 1)));
    return finish_call(fwd_common(plan, indptr, indices, N, E, H, D, Q, K, V, O, LSE, nullptr, 0.f, sc * kLog2e, M_GT,
                                  dtype, stream),
                       stream);
}

int gnn_attn_fwd_noalloc(gnn_plan_t plan, const int32_t *indptr, const int32_t *indices, int32_t N, int64_t E,
                         int32_t H, int32_t D, const void *Q, const void *K, const void *V, void *O, float *LSE,
                         float scale, gnn_dtype_t dtype, hipStream_t stream) {
    // argument checks first, so that a rejected call never touches the device
    GNN_TRY(check_common(plan, indptr, indices, N, E, H, D, dtype));
    if (N > 0 && (!Q || !K || !V || !O)) return GNN_ERR_INVALID_ARG;
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O)) return GNN_ERR_ALIGNMENT;
    if (plan && plan->timer.enabled) return GNN_ERR_UNSUPPORTED;   // event records are not allocation-free
    if (N == 0) return GNN_OK;
    float *buf = nullptr;
    GNN_TRY(scratch_on_current_device(&buf));
    const float sc = scale > 0.f ? scale : (float)(1.0 / std::sqrt((double)std::max(D, 1)));
    return finish_call(fwd_common(plan, indptr, indices, N, E, H, D, Q, K, V, O, LSE, nullptr, 0.f, sc * kLog2e, M_GT,
                                  dtype, stream, buf, GNN_NOALLOC_SCRATCH_BYTES),
                       stream);
}

int gatv2_attn_fwd(gnn_plan_t plan, const int32_t *indptr, const int32_t *indices, int32_t N, int64_t E,
                   int32_t H, int32_t D, const void *Q, const void *K, const void *V, const float *att,
                   float negative_slope, void *O, float *LSE, gnn_dtype_t dtype, hipStream_t stream) {
    const int mode = (V == K) ? M_GAT_ALIAS : M_GAT_SEPV;
    return finish_call(fwd_common(plan, indptr, indices, N, E, H, D, Q, K, V, O, LSE, att, negative_slope, 1.f, mode,
                                  dtype, stream),
                       stream);
}

static int attn_bwd_impl(gnn_plan_t plan, const int32_t *indptr, const int32_t *indices, int32_t N, int64_t E, int32_t H,
                 int32_t D, const void *Q, const void *K, const void *V, const void *O, const void *dO,
                 const float *LSE, void *dQ, void *dK, void *dV, float scale, gnn_dtype_t dtype,
                 hipStream_t stream) {
    if (!plan) return GNN_ERR_INVALID_ARG;
    GNN_TRY(check_common(plan, indptr, indices, N, E, H, D, dtype));
    if (!plan->has_csc) return GNN_ERR_UNSUPPORTED;
    if (N > 0 && (!Q || !K || !V || !dO || !LSE || !dQ || !dK || !dV)) return GNN_ERR_INVALID_ARG;
    for (const void *p : {Q, K, V, dO, (const void *)dQ, (const void *)dK, (const void *)dV})
        if (!aligned16(p)) return GNN_ERR_ALIGNMENT;
    if (N == 0) return GNN_OK;
    GNN_TRY(checked_graph(indptr, indices, N, E, stream));
    const float sc = scale > 0.f ? scale : (float)(1.0 / std::sqrt((double)D));
    BwdParams P{};
    fill_bwd_params(plan, P, indptr, indices, N, H, D, Q, K, V, dO, LSE, dQ, dK, dV, sc, dtype);
    const size_t rowlen = (size_t)H * D;
    const size_t n_stat = (size_t)N * H * 2;
    const size_t n_a = (size_t)P.a_n_groups * (2 * rowlen + H), n_b = (size_t)P.b_n_groups * 2 * rowlen;
    void *ws = nullptr;
    GNN_TRY(plan_workspace(plan, (n_stat + n_a + n_b) * sizeof(float), stream, &ws));
    P.stat = (float2 *)ws;
    P.ws_a = (float *)ws + n_stat;
    P.ws_b = P.ws_a + n_a;
    const bool tiles = plan->has_tiles && tile_supported(dtype, D);
    if (tiles) {
        P.a_light = as<int32_t>(plan->light_nt);
        P.a_n_light = plan->n_light_nt;
        P.b_light = as<int32_t>(plan->c_light_nt);
        P.b_n_light = plan->n_c_light_nt;
    }
    if (dtype == GNN_F32) {
        switch (D) {
            case 16: return run_bwd<float, 4>(plan, P, stream, false);
            case 32: return run_bwd<float, 8>(plan, P, stream, false);
            case 64: return run_bwd<float, 16>(plan, P, stream, false);
            case 128: return run_bwd<float, 32>(plan, P, stream, false);
        }
    } else {
        switch (D) {
            case 16: return run_bwd<bf16_tag, 2>(plan, P, stream, tiles);
            case 32: return run_bwd<bf16_tag, 4>(plan, P, stream, tiles);
            case 64: return run_bwd<bf16_tag, 8>(plan, P, stream, tiles);
            case 128: return run_bwd<bf16_tag, 16>(plan, P, stream, tiles);
        }
    }
    return GNN_ERR_UNSUPPORTED;
}

int gnn_attn_bwd(gnn_plan_t plan, const int32_t *indptr, const int32_t *indices, int32_t N, int64_t E, int32_t H,
                 int32_t D, const void *Q, const void *K, const void *V, const void *O, const void *dO,
                 const float *LSE, void *dQ, void *dK, void *dV, float scale, gnn_dtype_t dtype,
                 hipStream_t stream) {
    return finish_call(attn_bwd_impl(plan, indptr, indices, N, E, H, D, Q, K, V, O, dO, LSE, dQ, dK, dV, scale, dtype, stream), stream);
}

}  // extern "C"
