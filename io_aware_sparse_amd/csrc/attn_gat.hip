// GATv2 attention backward from the cached LSE.
//
// "On Efficient Scaling of GNNs via IO-Aware Layers Implementations",
// technical summary, Methodology (attention-based layers, backward pass):
// compact per-node statistics (log-sum-exp) are cached instead of edge
// weights, and the weights are recomputed on the fly. Applied to the GATv2
// layer the pages name. Per head, with z = xs_j + xd_i,
// phi = LeakyReLU(slope), s_ij = sum_d a_d phi(z_d), p_ij = exp(s_ij - LSE_i),
// dp_ij = <dO_i, v_j>, Delta_i = sum_j p_ij dp_ij, ds = p (dp - Delta):
//   dXD_i = sum_j ds_ij a phi'(z_ij)           destination pass (CSR)
//   da    = sum_ij ds_ij phi(z_ij)              destination pass + column sum
//   dXS_j = sum_i ds_ij a phi'(z_ij) (+ dV_j when V is XS)   source pass (CSC)
//   dV_j  = sum_i p_ij dO_i
// The destination pass accumulates A = sum p dp g, B = sum p g (g = a phi'),
// C = sum p dp phi, E = sum p phi and Delta in one sweep and forms
// dXD = A - Delta B and da_i = C - Delta E, so Delta comes from the same
// recomputed weights. Per-node da_i rows are summed over nodes by a fixed-order
// column reduction: no atomics, bitwise reproducible.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>

#include "attn_core.h"

namespace gnn {

struct GatBwdParams {
    BwdParams b;          // graph, buckets, Q = XD, K = XS, V, dO, LSE, dQ = dXD, dK = dXS, dV, stat, ws
    const float *att;
    float slope;
    float *da_nodes;      // [N][H*D] per-node d_att contributions
    float *da_part;       // [n_chunks][H*D] column-sum partials
    float *d_att;         // [H][D] output
    int32_t n_chunks;
    const int32_t *a_gperm;   // nullable: destination-pass launch slot -> heavy group (-1: none)
    int32_t a_n_slots;        // destination-pass heavy launch slots (b.a_n_groups without a_gperm)
};

// heavy blocks at the head of the destination-pass launch (as in the forward:
// one per (chunk group, head group), or 8 per W rows of XCD-ordered slots)
__host__ __device__ inline int64_t gat_dst_heavy_blocks(const GatBwdParams &GP) {
    return GP.a_gperm ? 8 * (((int64_t)GP.a_n_slots / 8 + GP.b.W - 1) / GP.b.W)
                      : (int64_t)GP.a_n_slots * GP.b.g.NHG;
}

template <class T, int LH, bool SEPV, int U>
__device__ __forceinline__ void gat_dst_stream(const GatBwdParams &GP, const LanePos &lp, int node, int e0, int e1,
                                               float (&A)[Vec<T>::N], float (&B)[Vec<T>::N], float (&Cc)[Vec<T>::N],
                                               float (&Ee)[Vec<T>::N], float &dsum, float &lse2) {
    using VT = Vec<T>;
    constexpr int NV = VT::N;
    const BwdParams &P = GP.b;
    const Geom &G = P.g;
    const int64_t rowlen = (int64_t)G.H * G.D;
    float xd[NV], dof[NV], an[NV], al[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) xd[k] = dof[k] = an[k] = al[k] = A[k] = B[k] = Cc[k] = Ee[k] = 0.f;
    dsum = 0.f;
    lse2 = -INFINITY;
    if (lp.act) {
        VT::unpack(load_vec<T>(P.Q, (int64_t)node * rowlen + lp.col), xd);
        VT::unpack(load_vec<T>(P.dO, (int64_t)node * rowlen + lp.col), dof);
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            an[k] = GP.att[lp.col + k];
            al[k] = an[k] * kLog2e;
        }
        lse2 = P.LSE[(int64_t)node * G.H + lp.h] * kLog2e;
    }
    const float slope = GP.slope;
    const int S = min(kWave, G.G * U);
    const int UE = S / G.G;
    int jn = (lp.lane < S && e0 + lp.lane < e1) ? checked_index(P.indices[e0 + lp.lane], G.N) : -1;
    for (int base = e0; base < e1; base += S) {
        const int jc = jn;
        if (base + S < e1) jn = (lp.lane < S && base + S + lp.lane < e1) ? checked_index(P.indices[base + S + lp.lane], G.N) : -1;
        int j[U];
#pragma unroll
        for (int u = 0; u < U; ++u) j[u] = (u < UE) ? __shfl(jc, u * G.G + lp.g, kWave) : -1;
        typename VT::raw xr[U], vr[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool ok = lp.act && j[u] >= 0;
            xr[u] = ok ? load_vec<T>(P.K, (int64_t)j[u] * rowlen + lp.col) : VT::zero();
            if (SEPV) vr[u] = ok ? load_vec<T>(P.V, (int64_t)j[u] * rowlen + lp.col) : VT::zero();
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float xs[NV], vf[NV], ph[NV], gd[NV];
            VT::unpack(xr[u], xs);
            VT::unpack(SEPV ? vr[u] : xr[u], vf);
            float ts = 0.f, tp = 0.f;
#pragma unroll
            for (int k = 0; k < NV; ++k) {
                const float z = xs[k] + xd[k];
                ph[k] = z >= 0.f ? z : slope * z;
                gd[k] = z >= 0.f ? an[k] : slope * an[k];
                ts = fmaf(al[k], ph[k], ts);
                tp = fmaf(dof[k], vf[k], tp);
            }
            ts = group_sum<LH>(ts);
            tp = group_sum<LH>(tp);
            const float p = (j[u] >= 0) ? fast_exp2(ts - lse2) : 0.f;
            const float pd = p * tp;
            dsum += pd;
#pragma unroll
            for (int k = 0; k < NV; ++k) {
                A[k] = fmaf(pd, gd[k], A[k]);
                B[k] = fmaf(p, gd[k], B[k]);
                Cc[k] = fmaf(pd, ph[k], Cc[k]);
                Ee[k] = fmaf(p, ph[k], Ee[k]);
            }
        }
    }
    sum_groups(A, G.lr_shift);
    sum_groups(B, G.lr_shift);
    sum_groups(Cc, G.lr_shift);
    sum_groups(Ee, G.lr_shift);
    for (int off = 1 << G.lr_shift; off < kWave; off <<= 1) dsum += xor_lane(dsum, off);
}

template <class T, int NV>
__device__ __forceinline__ void gat_dst_finish(const GatBwdParams &GP, const LanePos &lp, int node,
                                               const float (&A)[NV], const float (&B)[NV], const float (&Cc)[NV],
                                               const float (&Ee)[NV], float dsum, float lse2) {
    const BwdParams &P = GP.b;
    const int64_t off = (int64_t)node * P.g.H * P.g.D + lp.col;
    float gx[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        gx[k] = fmaf(-dsum, B[k], A[k]);
        GP.da_nodes[off + k] = fmaf(-dsum, Ee[k], Cc[k]);
    }
    store_scaled<T, NV>(P.dQ, off, gx, 1.f);
    if (lp.dv == 0) P.stat[(int64_t)node * P.g.H + lp.h] = make_float2(lse2, dsum);
}

// heavy partial slot: A, B, C, E [4][H*D], Delta [H]
template <class T, int LH, bool SEPV, int U>
__global__ __launch_bounds__(512) void k_gat_bwd_dst_main(GatBwdParams GP) {
    using VT = Vec<T>;
    constexpr int NV = VT::N;
    extern __shared__ float lds[];
    const BwdParams &P = GP.b;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int heavy_blocks = (int)gat_dst_heavy_blocks(GP);
    const int64_t rowlen = (int64_t)P.g.H * P.g.D;
    if ((int)blockIdx.x < heavy_blocks) {
        int grp, e0, e1, hg = 0;
        if (GP.a_gperm) {
            // XCD-ordered source-range groups, one per wave (as in the forward)
            const int slot = ((int)(blockIdx.x / 8) * P.W + w) * 8 + (int)(blockIdx.x % 8);
            grp = slot < GP.a_n_slots ? GP.a_gperm[slot] : -1;
            if (grp < 0) return;
            e0 = P.a_groups[3 * grp + 1];
            e1 = P.a_groups[3 * grp + 2];
        } else {
            grp = blockIdx.x / P.g.NHG;
            hg = blockIdx.x % P.g.NHG;
            const int g0 = P.a_groups[3 * grp + 1], g1 = P.a_groups[3 * grp + 2];
            e0 = min(g1, g0 + w * P.C);
            e1 = min(g1, e0 + P.C);
        }
        const int node = P.a_groups[3 * grp];
        const LanePos lp = lane_pos<LH, NV>(P.g, hg);
        float x[5][NV];
        float lse2;
        gat_dst_stream<T, LH, SEPV, U>(GP, lp, node, e0, e1, x[0], x[1], x[2], x[3], x[4][0], lse2);
#pragma unroll
        for (int k = 1; k < NV; ++k) x[4][k] = 0.f;
        if (GP.a_gperm) {
            if (lp.lane >= (1 << P.g.lr_shift) || !lp.act) return;    // no barrier on this path
        } else if (!lds_sum_waves<NV, 5>(lds, w, P.W, lp.lane, 1 << P.g.lr_shift, x) || !lp.act) {
            return;
        }
        float *slot = P.ws_a + (int64_t)grp * (4 * rowlen + P.g.H);
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int k = 0; k < NV; ++k) slot[a * rowlen + lp.col + k] = x[a][k];
        if (lp.dv == 0) slot[4 * rowlen + lp.h] = x[4][0];
        return;
    }
    const int64_t item = (int64_t)(blockIdx.x - heavy_blocks) * P.W + w;
    const int64_t ni = item / P.g.NHG;
    if (ni >= P.a_n_light) return;
    const int hg = (int)(item % P.g.NHG);
    const int node = P.a_light[ni];
    const LanePos lp = lane_pos<LH, NV>(P.g, hg);
    float A[NV], B[NV], Cc[NV], Ee[NV];
    float dsum, lse2;
    gat_dst_stream<T, LH, SEPV, U>(GP, lp, node, P.indptr[node], P.indptr[node + 1], A, B, Cc, Ee, dsum, lse2);
    if (lp.g != 0 || !lp.act) return;
    gat_dst_finish<T, NV>(GP, lp, node, A, B, Cc, Ee, dsum, lse2);
}

template <class T, int LH>
__global__ __launch_bounds__(256) void k_gat_bwd_dst_merge(GatBwdParams GP) {
    using VT = Vec<T>;
    constexpr int NV = VT::N;
    extern __shared__ float lds[];
    const BwdParams &P = GP.b;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int nw = blockDim.x / kWave;
    // one block per (heavy node, head group): wave w takes partials
    // p0 + w*G + g, stepping nw*G, so a hub's long list is summed by nw
    // waves at once; the waves are then summed in LDS in ascending order
    const int64_t item = blockIdx.x;
    if (item >= (int64_t)P.a_n_heavy * P.g.NHG) return;      // the whole block
    const int k = (int)(item / P.g.NHG), hg = (int)(item % P.g.NHG);
    const int node = P.a_heavy[k];
    const int p0 = P.a_ofs[k], p1 = P.a_ofs[k + 1];
    const LanePos lp = lane_pos<LH, NV>(P.g, hg);
    const int64_t rowlen = (int64_t)P.g.H * P.g.D;
    float x[5][NV];                  // A, B, C, E and (Delta, 0, ...)
    float lse2 = -INFINITY;
#pragma unroll
    for (int a = 0; a < 5; ++a)
#pragma unroll
        for (int q = 0; q < NV; ++q) x[a][q] = 0.f;
    if (lp.act) {
        for (int p = p0 + w * P.g.G + lp.g; p < p1; p += nw * P.g.G) {
            const float *slot = P.ws_a + (int64_t)p * (4 * rowlen + P.g.H);
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int q = 0; q < NV; ++q) x[a][q] += slot[a * rowlen + lp.col + q];
            x[4][0] += slot[4 * rowlen + lp.h];
        }
        lse2 = P.LSE[(int64_t)node * P.g.H + lp.h] * kLog2e;
    }
#pragma unroll
    for (int a = 0; a < 4; ++a) sum_groups(x[a], P.g.lr_shift);
    for (int off = 1 << P.g.lr_shift; off < kWave; off <<= 1) x[4][0] += xor_lane(x[4][0], off);
    if (!lds_sum_waves<NV, 5>(lds, w, nw, lp.lane, 1 << P.g.lr_shift, x) || !lp.act) return;
    gat_dst_finish<T, NV>(GP, lp, node, x[0], x[1], x[2], x[3], x[4][0], lse2);
}

template <class T, int LH, bool SEPV, int U>
__device__ __forceinline__ void gat_src_stream(const GatBwdParams &GP, const LanePos &lp, int node, int e0, int e1,
                                               float (&dxs)[Vec<T>::N], float (&dv)[Vec<T>::N]) {
    using VT = Vec<T>;
    constexpr int NV = VT::N;
    const BwdParams &P = GP.b;
    const Geom &G = P.g;
    const int64_t rowlen = (int64_t)G.H * G.D;
    float xs[NV], vf[NV], an[NV], al[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) xs[k] = vf[k] = an[k] = al[k] = dxs[k] = dv[k] = 0.f;
    if (lp.act) {
        VT::unpack(load_vec<T>(P.K, (int64_t)node * rowlen + lp.col), xs);
        VT::unpack(load_vec<T>(SEPV ? P.V : P.K, (int64_t)node * rowlen + lp.col), vf);
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            an[k] = GP.att[lp.col + k];
            al[k] = an[k] * kLog2e;
        }
    }
    const float slope = GP.slope;
    const int S = min(kWave, G.G * U);
    const int UE = S / G.G;
    int jn = (lp.lane < S && e0 + lp.lane < e1) ? checked_index(P.cindices[e0 + lp.lane], G.N) : -1;
    for (int base = e0; base < e1; base += S) {
        const int jc = jn;
        if (base + S < e1) jn = (lp.lane < S && base + S + lp.lane < e1) ? checked_index(P.cindices[base + S + lp.lane], G.N) : -1;
        int i[U];
#pragma unroll
        for (int u = 0; u < U; ++u) i[u] = (u < UE) ? __shfl(jc, u * G.G + lp.g, kWave) : -1;
        typename VT::raw dr[U], gr[U];
        float2 stt[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool ok = lp.act && i[u] >= 0;
            dr[u] = ok ? load_vec<T>(P.Q, (int64_t)i[u] * rowlen + lp.col) : VT::zero();
            gr[u] = ok ? load_vec<T>(P.dO, (int64_t)i[u] * rowlen + lp.col) : VT::zero();
            stt[u] = ok ? P.stat[(int64_t)i[u] * G.H + lp.h] : make_float2(0.f, 0.f);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float xd[NV], gf[NV], dph[NV];
            VT::unpack(dr[u], xd);
            VT::unpack(gr[u], gf);
            float ts = 0.f, tp = 0.f;
#pragma unroll
            for (int k = 0; k < NV; ++k) {
                const float z = xs[k] + xd[k];
                ts = fmaf(al[k], z >= 0.f ? z : slope * z, ts);
                dph[k] = z >= 0.f ? an[k] : slope * an[k];
                tp = fmaf(gf[k], vf[k], tp);
            }
            ts = group_sum<LH>(ts);
            tp = group_sum<LH>(tp);
            const float p = (i[u] >= 0) ? fast_exp2(ts - stt[u].x) : 0.f;
            const float ds = p * (tp - stt[u].y);
#pragma unroll
            for (int k = 0; k < NV; ++k) {
                dxs[k] = fmaf(ds, dph[k], dxs[k]);
                dv[k] = fmaf(p, gf[k], dv[k]);
            }
        }
    }
    sum_groups(dxs, G.lr_shift);
    sum_groups(dv, G.lr_shift);
}

template <class T, int NV, bool SEPV>
__device__ __forceinline__ void gat_src_finish(const GatBwdParams &GP, const LanePos &lp, int node, float (&dxs)[NV],
                                               const float (&dv)[NV]) {
    const BwdParams &P = GP.b;
    const int64_t off = (int64_t)node * P.g.H * P.g.D + lp.col;
    if (SEPV) {
        store_scaled<T, NV>(P.dK, off, dxs, 1.f);
        store_scaled<T, NV>(P.dV, off, dv, 1.f);
    } else {
#pragma unroll
        for (int k = 0; k < NV; ++k) dxs[k] += dv[k];
        store_scaled<T, NV>(P.dK, off, dxs, 1.f);
    }
}

template <class T, int LH, bool SEPV, int U>
__global__ __launch_bounds__(512) void k_gat_bwd_src_main(GatBwdParams GP) {
    using VT = Vec<T>;
    constexpr int NV = VT::N;
    extern __shared__ float lds[];
    const BwdParams &P = GP.b;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int heavy_blocks = P.b_n_groups * P.g.NHG;
    const int64_t rowlen = (int64_t)P.g.H * P.g.D;
    if ((int)blockIdx.x < heavy_blocks) {
        const int grp = blockIdx.x / P.g.NHG, hg = blockIdx.x % P.g.NHG;
        const int node = P.b_groups[3 * grp], g0 = P.b_groups[3 * grp + 1], g1 = P.b_groups[3 * grp + 2];
        const int e0 = min(g1, g0 + w * P.C), e1 = min(g1, e0 + P.C);
        const LanePos lp = lane_pos<LH, NV>(P.g, hg);
        float x[2][NV];
        gat_src_stream<T, LH, SEPV, U>(GP, lp, node, e0, e1, x[0], x[1]);
        if (!lds_sum_waves<NV, 2>(lds, w, P.W, lp.lane, 1 << P.g.lr_shift, x) || !lp.act) return;
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            P.ws_b[((int64_t)grp * 2 + 0) * rowlen + lp.col + k] = x[0][k];
            P.ws_b[((int64_t)grp * 2 + 1) * rowlen + lp.col + k] = x[1][k];
        }
        return;
    }
    const int64_t item = (int64_t)(blockIdx.x - heavy_blocks) * P.W + w;
    const int64_t ni = item / P.g.NHG;
    if (ni >= P.b_n_light) return;
    const int hg = (int)(item % P.g.NHG);
    const int node = P.b_light[ni];
    const LanePos lp = lane_pos<LH, NV>(P.g, hg);
    float dxs[NV], dv[NV];
    gat_src_stream<T, LH, SEPV, U>(GP, lp, node, P.cindptr[node], P.cindptr[node + 1], dxs, dv);
    if (lp.g != 0 || !lp.act) return;
    gat_src_finish<T, NV, SEPV>(GP, lp, node, dxs, dv);
}

template <class T, int LH, bool SEPV>
__global__ __launch_bounds__(256) void k_gat_bwd_src_merge(GatBwdParams GP) {
    using VT = Vec<T>;
    constexpr int NV = VT::N;
    const BwdParams &P = GP.b;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t item = (int64_t)blockIdx.x * (blockDim.x / kWave) + w;
    if (item >= (int64_t)P.b_n_heavy * P.g.NHG) return;
    const int k = (int)(item / P.g.NHG), hg = (int)(item % P.g.NHG);
    const int node = P.b_heavy[k];
    const int p0 = P.b_ofs[k], p1 = P.b_ofs[k + 1];
    const LanePos lp = lane_pos<LH, NV>(P.g, hg);
    const int64_t rowlen = (int64_t)P.g.H * P.g.D;
    float dxs[NV], dv[NV];
#pragma unroll
    for (int q = 0; q < NV; ++q) dxs[q] = dv[q] = 0.f;
    if (lp.act) {
        for (int p = p0 + lp.g; p < p1; p += P.g.G) {
#pragma unroll
            for (int q = 0; q < NV; ++q) {
                dxs[q] += P.ws_b[((int64_t)p * 2 + 0) * rowlen + lp.col + q];
                dv[q] += P.ws_b[((int64_t)p * 2 + 1) * rowlen + lp.col + q];
            }
        }
    }
    sum_groups(dxs, P.g.lr_shift);
    sum_groups(dv, P.g.lr_shift);
    if (lp.g != 0 || !lp.act) return;
    gat_src_finish<T, NV, SEPV>(GP, lp, node, dxs, dv);
}

// d_att: fixed-order column sums of da_nodes [N][HD]. Pass 1: each block sums
// a chunk of kColChunk rows for 256 columns (independent loads, unrolled);
// pass 2: one block per column sums the chunk partials with a fixed
// thread-strided order and a fixed LDS tree.
constexpr int kColChunk = 64;

__global__ __launch_bounds__(256) void k_col_partial(const float *x, int64_t n, int64_t cols, float *part) {
    const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t r0 = (int64_t)blockIdx.y * kColChunk, r1 = min(n, r0 + kColChunk);
    if (c >= cols) return;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    int64_t r = r0;
    for (; r + 8 <= r1; r += 8) {
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[k] += x[(r + k) * cols + c];
    }
    for (int k = 0; r < r1; ++r, ++k) acc[k] += x[r * cols + c];
    part[(int64_t)blockIdx.y * cols + c] =
        ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
}

__global__ __launch_bounds__(256) void k_col_final(const float *part, int64_t chunks, int64_t cols, float *out) {
    __shared__ float red[256];
    const int64_t c = blockIdx.x;
    float acc = 0.f;
    for (int64_t k = threadIdx.x; k < chunks; k += blockDim.x) acc += part[k * cols + c];
    red[threadIdx.x] = acc;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) out[c] = red[0];
}

template <class T, int LH, bool SEPV>
static int run_gat_bwd(gnn_plan_t plan, GatBwdParams &GP, hipStream_t s) {
    constexpr int U = 2;
    constexpr int NV = Vec<T>::N;
    BwdParams &P = GP.b;
    const int LR = 1 << P.g.lr_shift;
    {
        const int64_t lb = ((int64_t)P.a_n_light * P.g.NHG + P.W - 1) / P.W;
        const int64_t blocks = gat_dst_heavy_blocks(GP) + lb;
        if (blocks >= (1ll << 31)) return GNN_ERR_INVALID_ARG;
        const size_t lds = P.a_n_groups ? (size_t)P.W * LR * 5 * NV * sizeof(float) : 0;
        GNN_TRY(launch(plan, K_GAT_BWD_DST_MAIN, k_gat_bwd_dst_main<T, LH, SEPV, U>, dim3((unsigned)blocks),
                       dim3(64 * P.W), lds, s, GP));
        const int64_t mb = (int64_t)P.a_n_heavy * P.g.NHG;
        if (mb >= (1ll << 31)) return GNN_ERR_INVALID_ARG;
        if (mb)
            GNN_TRY(launch(plan, K_GAT_BWD_DST_MERGE, k_gat_bwd_dst_merge<T, LH>, dim3((unsigned)mb), dim3(256),
                           (size_t)4 * LR * 5 * NV * sizeof(float), s, GP));
    }
    {
        const int64_t lb = ((int64_t)P.b_n_light * P.g.NHG + P.W - 1) / P.W;
        const int64_t blocks = (int64_t)P.b_n_groups * P.g.NHG + lb;
        if (blocks >= (1ll << 31)) return GNN_ERR_INVALID_ARG;
        const size_t lds = P.b_n_groups ? (size_t)P.W * LR * 2 * NV * sizeof(float) : 0;
        GNN_TRY(launch(plan, K_GAT_BWD_SRC_MAIN, k_gat_bwd_src_main<T, LH, SEPV, U>, dim3((unsigned)blocks),
                       dim3(64 * P.W), lds, s, GP));
        if (P.b_n_heavy)
            GNN_TRY(launch(plan, K_GAT_BWD_SRC_MERGE, k_gat_bwd_src_merge<T, LH, SEPV>,
                           dim3((unsigned)(((int64_t)P.b_n_heavy * P.g.NHG + 3) / 4)), dim3(256), 0, s, GP));
    }
    const int64_t cols = (int64_t)P.g.H * P.g.D;
    const unsigned gx = (unsigned)((cols + 255) / 256);
    GNN_TRY(launch(plan, K_GAT_DATT, k_col_partial, dim3(gx, (unsigned)GP.n_chunks), dim3(256), 0, s,
                   (const float *)GP.da_nodes, (int64_t)P.g.N, cols, GP.da_part));
    GNN_TRY(launch(plan, K_GAT_DATT, k_col_final, dim3((unsigned)cols), dim3(256), 0, s, (const float *)GP.da_part,
                   (int64_t)GP.n_chunks, cols, GP.d_att));
    return GNN_OK;
}

template <bool SEPV>
static int dispatch_gat_bwd(gnn_plan_t plan, GatBwdParams &GP, gnn_dtype_t dt, int D, hipStream_t s) {
    if (dt == GNN_F32) {
        switch (D) {
            case 16: return run_gat_bwd<float, 4, SEPV>(plan, GP, s);
            case 32: return run_gat_bwd<float, 8, SEPV>(plan, GP, s);
            case 64: return run_gat_bwd<float, 16, SEPV>(plan, GP, s);
            case 128: return run_gat_bwd<float, 32, SEPV>(plan, GP, s);
        }
    } else {
        switch (D) {
            case 16: return run_gat_bwd<bf16_tag, 2, SEPV>(plan, GP, s);
            case 32: return run_gat_bwd<bf16_tag, 4, SEPV>(plan, GP, s);
            case 64: return run_gat_bwd<bf16_tag, 8, SEPV>(plan, GP, s);
            case 128: return run_gat_bwd<bf16_tag, 16, SEPV>(plan, GP, s);
        }
    }
    return GNN_ERR_UNSUPPORTED;
}

// this file's kernels' index flag (checked builds)
GNN_INDEX_FAULT_READER(index_fault_gat)

}  // namespace gnn

using namespace gnn;

extern "C" {

static int gat_bwd_impl(gnn_plan_t plan, const int32_t *indptr, const int32_t *indices, int32_t N, int64_t E,
                              int32_t H, int32_t D, const void *Q, const void *K, const void *V, const float *att,
                              float negative_slope, const void *dO, const float *LSE, void *dQ, void *dK, void *dV,
                              float *d_att, gnn_dtype_t dtype, hipStream_t stream) {
    if (!plan) return GNN_ERR_INVALID_ARG;
    GNN_TRY(check_common(plan, indptr, indices, N, E, H, D, dtype));
    if (!plan->has_csc) return GNN_ERR_UNSUPPORTED;
    const bool sepv = V != K;
    if (N > 0 && (!Q || !K || !V || !att || !dO || !LSE || !dQ || !dK || !d_att || (sepv && !dV)))
        return GNN_ERR_INVALID_ARG;
    for (const void *p : {Q, K, V, dO, (const void *)dQ, (const void *)dK})
        if (!aligned16(p)) return GNN_ERR_ALIGNMENT;
    if (sepv && !aligned16(dV)) return GNN_ERR_ALIGNMENT;
    if (N == 0) {
        // no edges: d_att, their sum, is zero (the column sum over no chunks)
        if (d_att)
            GNN_TRY(launch(plan, K_GAT_DATT, k_col_final, dim3((unsigned)((int64_t)H * D)), dim3(256), 0, stream,
                           (const float *)nullptr, (int64_t)0, (int64_t)H * D, d_att));
        return GNN_OK;
    }
    GNN_TRY(checked_graph(indptr, indices, N, E, stream));
    GatBwdParams GP{};
    BwdParams &P = GP.b;
    fill_bwd_params(plan, P, indptr, indices, N, H, D, Q, K, V, dO, LSE, dQ, dK, sepv ? dV : nullptr, 1.f, dtype);
    GP.att = att;
    GP.slope = negative_slope;
    GP.d_att = d_att;
    GP.n_chunks = (int32_t)((N + kColChunk - 1) / kColChunk);
    GP.a_gperm = nullptr;
    GP.a_n_slots = P.a_n_groups;
    // the destination pass takes the forward's source-range groups under the
    // forward's rule (one head group, a range of the gathered tables near an
    // XCD's L2); its partial slots merge in the same fixed order
    const int64_t gathered = (int64_t)N * H * D * (dtype == GNN_BF16 ? 2 : 4) * (sepv ? 2 : 1);
    if (plan->xsplit.n_groups && P.g.NHG == 1 && (gathered + 7) / 8 <= kXsplitMaxRangeBytes) {
        P.a_groups = as<int32_t>(plan->xsplit.groups);
        P.a_ofs = as<int32_t>(plan->xsplit.partial_ofs);
        P.a_n_groups = plan->xsplit.n_groups;
        GP.a_gperm = as<int32_t>(plan->xsplit.order);
        GP.a_n_slots = plan->xsplit.n_slots;
    }
    const size_t rowlen = (size_t)H * D;
    const size_t n_stat = (size_t)N * H * 2;
    const size_t n_a = (size_t)P.a_n_groups * (4 * rowlen + H), n_b = (size_t)P.b_n_groups * 2 * rowlen;
    const size_t n_da = (size_t)N * rowlen, n_part = (size_t)GP.n_chunks * rowlen;
    void *ws = nullptr;
    GNN_TRY(plan_workspace(plan, (n_stat + n_a + n_b + n_da + n_part) * sizeof(float), stream, &ws));
    P.stat = (float2 *)ws;
    P.ws_a = (float *)ws + n_stat;
    P.ws_b = P.ws_a + n_a;
    GP.da_nodes = P.ws_b + n_b;
    GP.da_part = GP.da_nodes + n_da;
    return sepv ? dispatch_gat_bwd<true>(plan, GP, dtype, D, stream)
                : dispatch_gat_bwd<false>(plan, GP, dtype, D, stream);
}

int gatv2_attn_bwd(gnn_plan_t plan, const int32_t *indptr, const int32_t *indices, int32_t N, int64_t E,
                              int32_t H, int32_t D, const void *Q, const void *K, const void *V, const float *att,
                              float negative_slope, const void *dO, const float *LSE, void *dQ, void *dK, void *dV,
                              float *d_att, gnn_dtype_t dtype, hipStream_t stream) {
    return finish_call(gat_bwd_impl(plan, indptr, indices, N, E, H, D, Q, K, V, att, negative_slope, dO, LSE, dQ, dK, dV, d_att, dtype, stream), stream);
}

}  // extern "C"
