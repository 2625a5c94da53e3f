// Fused CSR neighbourhood attention kernels for gfx950.
//
// "On Efficient Scaling of GNNs via IO-Aware Layers Implementations",
// technical summary, Methodology (attention-based layers): one streaming pass
// over each node's neighbours computes the scores, the softmax normalisation
// and the value aggregation; the forward keeps running statistics in
// registers (online softmax) so no edge logit is written; the backward reads
// a cached per-node log-sum-exp and recomputes every weight on the fly.
// Degree-aware tiling (same section): light nodes (in-degree <= T) take one
// wavefront each; heavy nodes are cut into chunk groups whose waves each
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

#include "device.h"
#include "internal.h"

namespace gnn {

constexpr float kNegInf = -INFINITY;

enum Mode { M_GT = 0, M_GAT_ALIAS = 1, M_GAT_SEPV = 2 };

struct Geom {
    int32_t N, H, D;
    int32_t HW;       // heads per wave
    int32_t NHG;      // head groups per node
    int32_t lr_shift; // log2(LR)
    int32_t G;        // edge groups per wave
};

struct FwdParams {
    Geom g;
    const int32_t *indptr, *indices;
    const void *Q, *K, *V;
    void *O;
    float *LSE;
    const float *att;
    float slope, mul;   // mul: score multiplier into log2 units
    const int32_t *light;
    int32_t n_light;
    const int32_t *groups;
    int32_t n_groups, C;
    const int32_t *heavy, *partial_ofs;
    int32_t n_heavy;
    float *ws_acc, *ws_ml;
    int32_t W;
};

// per-lane position inside the wave's (node, head group) slice
struct LanePos {
    int lane, g, r, hh, dv, h;
    bool act;
    int64_t col;   // element offset inside the node's H*D row
};

template <int LH, int NV>
__device__ __forceinline__ LanePos lane_pos(const Geom &G, int hg) {
    LanePos p;
    p.lane = lane_id();
    const int LR = 1 << G.lr_shift;
    p.g = p.lane >> G.lr_shift;
    p.r = p.lane & (LR - 1);
    p.hh = p.r / LH;
    p.dv = p.r % LH;
    p.h = hg * G.HW + p.hh;
    p.act = (p.hh < G.HW) && (p.h < G.H);
    p.col = (int64_t)p.h * G.D + p.dv * NV;
    return p;
}

template <int NV>
struct SoftState {
    float m, l, acc[NV];
};

template <int NV>
__device__ __forceinline__ void merge_state(SoftState<NV> &a, float m2, float l2, const float (&a2)[NV]) {
    const float mn = fmaxf(a.m, m2);
    const float ms = (mn == kNegInf) ? 0.f : mn;
    const float c1 = fast_exp2(a.m - ms), c2 = fast_exp2(m2 - ms);
    a.l = a.l * c1 + l2 * c2;
#pragma unroll
    for (int k = 0; k < NV; ++k) a.acc[k] = a.acc[k] * c1 + a2[k] * c2;
    a.m = mn;
}

template <int NV>
__device__ __forceinline__ void merge_groups(SoftState<NV> &st, int lr_shift) {
    for (int off = 1 << lr_shift; off < kWave; off <<= 1) {
        const float m2 = xor_lane(st.m, off), l2 = xor_lane(st.l, off);
        float a2[NV];
#pragma unroll
        for (int k = 0; k < NV; ++k) a2[k] = xor_lane(st.acc[k], off);
        merge_state(st, m2, l2, a2);
    }
}

// Stream edges [e0, e1) of `node` for this lane's head group; returns the
// wave-merged online-softmax state (valid in every lane).
template <class T, int LH, int MODE, int U>
__device__ __forceinline__ void fwd_stream(const FwdParams &P, const LanePos &lp, int node, int e0, int e1,
                                           SoftState<Vec<T>::N> &st) {
    using VT = Vec<T>;
    constexpr int NV = VT::N;
    const Geom &G = P.g;
    const int64_t rowlen = (int64_t)G.H * G.D;
    float q[NV];
    float a[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) q[k] = a[k] = 0.f;
    if (lp.act) {
        VT::unpack(load_vec<T>(P.Q, (int64_t)node * rowlen + lp.col), q);
        if (MODE != M_GT) {
#pragma unroll
            for (int k = 0; k < NV; ++k) a[k] = P.att[lp.col + k] * kLog2e;
        }
    }
    st.m = kNegInf;
    st.l = 0.f;
#pragma unroll
    for (int k = 0; k < NV; ++k) st.acc[k] = 0.f;

    const int S = min(kWave, G.G * U);   // edges per step
    const int UE = S / G.G;               // steps per group actually used
    int jn = (lp.lane < S && e0 + lp.lane < e1) ? P.indices[e0 + lp.lane] : -1;
    for (int base = e0; base < e1; base += S) {
        const int jc = jn;
        if (base + S < e1) jn = (lp.lane < S && base + S + lp.lane < e1) ? P.indices[base + S + lp.lane] : -1;
        int j[U];
#pragma unroll
        for (int u = 0; u < U; ++u) j[u] = (u < UE) ? __shfl(jc, u * G.G + lp.g, kWave) : -1;
        typename VT::raw kr[U], vr[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            kr[u] = (lp.act && j[u] >= 0) ? load_vec<T>(P.K, (int64_t)j[u] * rowlen + lp.col) : VT::zero();
            if (MODE != M_GAT_ALIAS)
                vr[u] = (lp.act && j[u] >= 0) ? load_vec<T>(P.V, (int64_t)j[u] * rowlen + lp.col) : VT::zero();
        }
        float s[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float kf[NV];
            VT::unpack(kr[u], kf);
            float t = 0.f;
            if (MODE == M_GT) {
#pragma unroll
                for (int k = 0; k < NV; ++k) t = fmaf(q[k], kf[k], t);
            } else {
#pragma unroll
                for (int k = 0; k < NV; ++k) {
                    const float z = kf[k] + q[k];
                    t = fmaf(a[k], z >= 0.f ? z : P.slope * z, t);
                }
            }
            t = group_sum<LH>(t);
            s[u] = (j[u] >= 0) ? t * P.mul : kNegInf;
        }
        float mx = s[0];
#pragma unroll
        for (int u = 1; u < U; ++u) mx = fmaxf(mx, s[u]);
        const float mn = fmaxf(st.m, mx);
        const float ms = (mn == kNegInf) ? 0.f : mn;
        const float c = fast_exp2(st.m - ms);
        st.l *= c;
#pragma unroll
        for (int k = 0; k < NV; ++k) st.acc[k] *= c;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float p = fast_exp2(s[u] - ms);
            st.l += p;
            float vf[NV];
            VT::unpack(MODE == M_GAT_ALIAS ? kr[u] : vr[u], vf);
#pragma unroll
            for (int k = 0; k < NV; ++k) st.acc[k] = fmaf(p, vf[k], st.acc[k]);
        }
        st.m = mn;
    }
    merge_groups(st, G.lr_shift);
}

template <class T, int NV>
__device__ __forceinline__ void write_out(const FwdParams &P, const LanePos &lp, int node, const SoftState<NV> &st) {
    using VT = Vec<T>;
    if (lp.g != 0 || !lp.act) return;
    const int64_t rowlen = (int64_t)P.g.H * P.g.D;
    const float inv = st.l > 0.f ? 1.f / st.l : 0.f;
    float o[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) o[k] = st.acc[k] * inv;
    store_vec<T>(P.O, (int64_t)node * rowlen + lp.col, VT::pack(o));
    if (P.LSE && lp.dv == 0)
        P.LSE[(int64_t)node * P.g.H + lp.h] = st.l > 0.f ? (st.m + fast_log2(st.l)) * kLn2 : kNegInf;
}

// Main forward kernel: blocks [0, n_groups*NHG) are heavy chunk groups,
// the rest hold W light (node, head group) items, one per wave.
template <class T, int LH, int MODE, int U>
__global__ __launch_bounds__(512) void k_fwd_main(FwdParams P) {
    using VT = Vec<T>;
    constexpr int NV = VT::N;
    extern __shared__ float lds[];
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int heavy_blocks = P.n_groups * P.g.NHG;
    if ((int)blockIdx.x < heavy_blocks) {
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
        if (!lp.act) return;
        const int64_t rowlen = (int64_t)P.g.H * P.g.D;
#pragma unroll
        for (int k = 0; k < NV; ++k) P.ws_acc[(int64_t)grp * rowlen + lp.col + k] = st.acc[k];
        if (lp.dv == 0) {
            P.ws_ml[((int64_t)grp * P.g.H + lp.h) * 2 + 0] = st.m;
            P.ws_ml[((int64_t)grp * P.g.H + lp.h) * 2 + 1] = st.l;
        }
        return;
    }
    const int64_t item = (int64_t)(blockIdx.x - heavy_blocks) * P.W + w;
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

// Second pass: one wave per (heavy node, head group) merges the node's
// partials in a fixed order (group-strided, then a fixed xor tree).
template <class T, int LH>
__global__ __launch_bounds__(256) void k_fwd_merge(FwdParams P) {
    using VT = Vec<T>;
    constexpr int NV = VT::N;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t item = (int64_t)blockIdx.x * (blockDim.x / kWave) + w;
    if (item >= (int64_t)P.n_heavy * P.g.NHG) return;
    const int k = (int)(item / P.g.NHG), hg = (int)(item % P.g.NHG);
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
        for (int p = p0 + lp.g; p < p1; p += P.g.G) {
            float a2[NV];
#pragma unroll
            for (int q = 0; q < NV; ++q) a2[q] = P.ws_acc[(int64_t)p * rowlen + lp.col + q];
            merge_state(st, P.ws_ml[((int64_t)p * P.g.H + lp.h) * 2], P.ws_ml[((int64_t)p * P.g.H + lp.h) * 2 + 1], a2);
        }
    }
    merge_groups(st, P.g.lr_shift);
    write_out<T, NV>(P, lp, node, st);
}

// ======================================================================
// backward
// ======================================================================

struct BwdParams {
    Geom g;
    const int32_t *indptr, *indices;     // CSR (destination pass)
    const int32_t *cindptr, *cindices;   // transposed adjacency (source pass)
    const void *Q, *K, *V, *O, *dO;
    const float *LSE;
    void *dQ, *dK, *dV;
    float mul, scale;
    // destination-pass buckets
    const int32_t *a_light, *a_groups, *a_heavy, *a_ofs;
    int32_t a_n_light, a_n_groups, a_n_heavy;
    // source-pass buckets
    const int32_t *b_light, *b_groups, *b_heavy, *b_ofs;
    int32_t b_n_light, b_n_groups, b_n_heavy;
    int32_t C, W;
    float2 *stat;    // [N][H] (LSE * log2 e, Delta)
    float *ws_a;     // [a_n_groups][2*H*D + H]
    float *ws_b;     // [b_n_groups][2][H*D]
};

template <int NV>
__device__ __forceinline__ void sum_groups(float (&x)[NV], int lr_shift) {
    for (int off = 1 << lr_shift; off < kWave; off <<= 1) {
#pragma unroll
        for (int k = 0; k < NV; ++k) x[k] += xor_lane(x[k], off);
    }
}

template <class T, int NV>
__device__ __forceinline__ void store_scaled(void *base, int64_t off, const float (&x)[NV], float sc) {
    float o[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) o[k] = x[k] * sc;
    store_vec<T>(base, off, Vec<T>::pack(o));
}

// Destination side over edges [e0, e1) of `node`. With p = exp(s - LSE) and
// dp = <dO_i, V_j> it accumulates A = sum p*dp*K_j, B = sum p*K_j and
// Delta = sum p*dp, so that dQ_i = scale * (A - Delta * B) in one pass.
// Delta is thus formed from the recomputed weights (its definition), not
// from <dO_i, O_i> with a rounded O. Returns this lane's lse2 = LSE*log2 e.
template <class T, int LH, int U>
__device__ __forceinline__ void bwd_dst_stream(const BwdParams &P, const LanePos &lp, int node, int e0, int e1,
                                               float (&A)[Vec<T>::N], float (&B)[Vec<T>::N], float &dsum,
                                               float &lse2) {
    using VT = Vec<T>;
    constexpr int NV = VT::N;
    const Geom &G = P.g;
    const int64_t rowlen = (int64_t)G.H * G.D;
    float q[NV], dof[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) q[k] = dof[k] = A[k] = B[k] = 0.f;
    dsum = 0.f;
    lse2 = kNegInf;
    if (lp.act) {
        VT::unpack(load_vec<T>(P.Q, (int64_t)node * rowlen + lp.col), q);
        VT::unpack(load_vec<T>(P.dO, (int64_t)node * rowlen + lp.col), dof);
        lse2 = P.LSE[(int64_t)node * G.H + lp.h] * kLog2e;
    }
    const int S = min(kWave, G.G * U);
    const int UE = S / G.G;
    int jn = (lp.lane < S && e0 + lp.lane < e1) ? P.indices[e0 + lp.lane] : -1;
    for (int base = e0; base < e1; base += S) {
        const int jc = jn;
        if (base + S < e1) jn = (lp.lane < S && base + S + lp.lane < e1) ? P.indices[base + S + lp.lane] : -1;
        int j[U];
#pragma unroll
        for (int u = 0; u < U; ++u) j[u] = (u < UE) ? __shfl(jc, u * G.G + lp.g, kWave) : -1;
        typename VT::raw kr[U], vr[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool ok = lp.act && j[u] >= 0;
            kr[u] = ok ? load_vec<T>(P.K, (int64_t)j[u] * rowlen + lp.col) : VT::zero();
            vr[u] = ok ? load_vec<T>(P.V, (int64_t)j[u] * rowlen + lp.col) : VT::zero();
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float kf[NV], vf[NV];
            VT::unpack(kr[u], kf);
            VT::unpack(vr[u], vf);
            float ts = 0.f, tp = 0.f;
#pragma unroll
            for (int k = 0; k < NV; ++k) {
                ts = fmaf(q[k], kf[k], ts);
                tp = fmaf(dof[k], vf[k], tp);
            }
            ts = group_sum<LH>(ts);
            tp = group_sum<LH>(tp);
            const float p = (j[u] >= 0) ? fast_exp2(ts * P.mul - lse2) : 0.f;
            const float pd = p * tp;
            dsum += pd;
#pragma unroll
            for (int k = 0; k < NV; ++k) {
                A[k] = fmaf(pd, kf[k], A[k]);
                B[k] = fmaf(p, kf[k], B[k]);
            }
        }
    }
    sum_groups(A, G.lr_shift);
    sum_groups(B, G.lr_shift);
    for (int off = 1 << G.lr_shift; off < kWave; off <<= 1) dsum += xor_lane(dsum, off);
}

// Source side: dK_j, dV_j partials over transposed edges [e0, e1).
template <class T, int LH, int U>
__device__ __forceinline__ void bwd_src_stream(const BwdParams &P, const LanePos &lp, int node, int e0, int e1,
                                               float (&dk)[Vec<T>::N], float (&dv)[Vec<T>::N]) {
    using VT = Vec<T>;
    constexpr int NV = VT::N;
    const Geom &G = P.g;
    const int64_t rowlen = (int64_t)G.H * G.D;
    float kf[NV], vf[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) kf[k] = vf[k] = dk[k] = dv[k] = 0.f;
    if (lp.act) {
        VT::unpack(load_vec<T>(P.K, (int64_t)node * rowlen + lp.col), kf);
        VT::unpack(load_vec<T>(P.V, (int64_t)node * rowlen + lp.col), vf);
    }
    const int S = min(kWave, G.G * U);
    const int UE = S / G.G;
    int jn = (lp.lane < S && e0 + lp.lane < e1) ? P.cindices[e0 + lp.lane] : -1;
    for (int base = e0; base < e1; base += S) {
        const int jc = jn;
        if (base + S < e1) jn = (lp.lane < S && base + S + lp.lane < e1) ? P.cindices[base + S + lp.lane] : -1;
        int i[U];
#pragma unroll
        for (int u = 0; u < U; ++u) i[u] = (u < UE) ? __shfl(jc, u * G.G + lp.g, kWave) : -1;
        typename VT::raw qr[U], gr[U];
        float2 stt[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool ok = lp.act && i[u] >= 0;
            qr[u] = ok ? load_vec<T>(P.Q, (int64_t)i[u] * rowlen + lp.col) : VT::zero();
            gr[u] = ok ? load_vec<T>(P.dO, (int64_t)i[u] * rowlen + lp.col) : VT::zero();
            stt[u] = ok ? P.stat[(int64_t)i[u] * G.H + lp.h] : make_float2(0.f, 0.f);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float qf[NV], gf[NV];
            VT::unpack(qr[u], qf);
            VT::unpack(gr[u], gf);
            float ts = 0.f, tp = 0.f;
#pragma unroll
            for (int k = 0; k < NV; ++k) {
                ts = fmaf(qf[k], kf[k], ts);
                tp = fmaf(gf[k], vf[k], tp);
            }
            ts = group_sum<LH>(ts);
            tp = group_sum<LH>(tp);
            const float p = (i[u] >= 0) ? fast_exp2(ts * P.mul - stt[u].x) : 0.f;
            const float ds = p * (tp - stt[u].y);
#pragma unroll
            for (int k = 0; k < NV; ++k) {
                dv[k] = fmaf(p, gf[k], dv[k]);
                dk[k] = fmaf(ds, qf[k], dk[k]);
            }
        }
    }
    sum_groups(dk, G.lr_shift);
    sum_groups(dv, G.lr_shift);
}

// LDS sum of W waves' partial vectors (ascending wave order), result in wave 0.
template <int NV, int NA>
__device__ __forceinline__ bool lds_sum_waves(float *lds, int w, int W, int lane, int LR, float (&x)[NA][NV]) {
    float *mine = lds + ((size_t)w * LR + lane) * (NV * NA);
    if (lane < LR) {
#pragma unroll
        for (int a = 0; a < NA; ++a)
#pragma unroll
            for (int k = 0; k < NV; ++k) mine[a * NV + k] = x[a][k];
    }
    __syncthreads();
    if (w != 0 || lane >= LR) return false;
    for (int v = 1; v < W; ++v) {
        const float *o = lds + ((size_t)v * LR + lane) * (NV * NA);
#pragma unroll
        for (int a = 0; a < NA; ++a)
#pragma unroll
            for (int k = 0; k < NV; ++k) x[a][k] += o[a * NV + k];
    }
    return true;
}

template <class T, int NV>
__device__ __forceinline__ void store_dq(const BwdParams &P, const LanePos &lp, int node, const float (&A)[NV],
                                         const float (&B)[NV], float dsum, float lse2) {
    float dq[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) dq[k] = fmaf(-dsum, B[k], A[k]);
    store_scaled<T, NV>(P.dQ, (int64_t)node * P.g.H * P.g.D + lp.col, dq, P.scale);
    if (lp.dv == 0) P.stat[(int64_t)node * P.g.H + lp.h] = make_float2(lse2, dsum);
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
    const int64_t item = (int64_t)(blockIdx.x - heavy_blocks) * P.W + w;
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
    const int64_t item = (int64_t)(blockIdx.x - heavy_blocks) * P.W + w;
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

static int ilog2(int x) {
    int s = 0;
    while ((1 << s) < x) ++s;
    return s;
}

// lanes per head for (dtype, D); 0 if unsupported
static int lanes_per_head(gnn_dtype_t dt, int D) {
    if (!(D == 16 || D == 32 || D == 64 || D == 128)) return 0;
    if (dt == GNN_F32) return D / 4;
    if (dt == GNN_BF16) return D / 8;
    return 0;
}

static Geom make_geom(int N, int H, int D, int LH) {
    Geom g;
    g.N = N;
    g.H = H;
    g.D = D;
    g.HW = std::min(H, kWave / LH);
    g.NHG = (H + g.HW - 1) / g.HW;
    g.lr_shift = ilog2(g.HW * LH);
    g.G = kWave >> g.lr_shift;
    return g;
}

static bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

static int check_common(gnn_plan_t plan, const int32_t *indptr, const int32_t *indices, int32_t N, int64_t E,
                        int32_t H, int32_t D, gnn_dtype_t dtype) {
    if (N < 0 || E < 0 || E >= (1ll << 31) || H < 1 || !indptr) return GNN_ERR_INVALID_ARG;
    if (E > 0 && !indices) return GNN_ERR_INVALID_ARG;
    if (dtype != GNN_F32 && dtype != GNN_BF16) return GNN_ERR_UNSUPPORTED;
    if (!lanes_per_head(dtype, D)) return GNN_ERR_UNSUPPORTED;
    if ((int64_t)N * H * D >= (1ll << 40)) return GNN_ERR_INVALID_ARG;
    if (plan && (plan->n_nodes != N || plan->n_edges != E || plan->indptr != indptr || plan->indices != indices))
        return GNN_ERR_INVALID_ARG;
    return GNN_OK;
}

template <class K, class P>
static int launch(gnn_plan_t plan, int kind, K kernel, dim3 grid, dim3 block, size_t lds, hipStream_t s,
                  const P &params) {
    if (grid.x == 0) return GNN_OK;
    TimingRec rec;
    const bool timed = plan && plan->timer.enabled;
    if (timed) GNN_TRY(plan->timer.begin(kind, s, rec));
    hipLaunchKernelGGL(kernel, grid, block, lds, s, params);
    GNN_HIP(hipGetLastError());
    if (timed) GNN_TRY(plan->timer.end(rec, s));
    return GNN_OK;
}

template <class T, int LH, int MODE>
static int run_fwd(gnn_plan_t plan, FwdParams &P, hipStream_t s) {
    constexpr int U = 4;
    constexpr int NV = Vec<T>::N;
    const int kind_main = MODE == M_GT ? K_FWD_MAIN : K_GAT_MAIN;
    const int kind_merge = MODE == M_GT ? K_FWD_MERGE : K_GAT_MERGE;
    const int64_t light_blocks = ((int64_t)P.n_light * P.g.NHG + P.W - 1) / P.W;
    const int64_t blocks = (int64_t)P.n_groups * P.g.NHG + light_blocks;
    if (blocks >= (1ll << 31)) return GNN_ERR_INVALID_ARG;
    const size_t lds = P.n_groups ? (size_t)P.W * (1 << P.g.lr_shift) * (NV + 2) * sizeof(float) : 0;
    GNN_TRY(launch(plan, kind_main, k_fwd_main<T, LH, MODE, U>, dim3((unsigned)blocks), dim3(64 * P.W), lds, s, P));
    if (P.n_heavy) {
        const int64_t mb = ((int64_t)P.n_heavy * P.g.NHG + 3) / 4;
        GNN_TRY(launch(plan, kind_merge, k_fwd_merge<T, LH>, dim3((unsigned)mb), dim3(256), 0, s, P));
    }
    return GNN_OK;
}

template <int MODE>
static int dispatch_fwd(gnn_plan_t plan, FwdParams &P, gnn_dtype_t dt, int D, hipStream_t s) {
    if (dt == GNN_F32) {
        switch (D) {
            case 16: return run_fwd<float, 4, MODE>(plan, P, s);
            case 32: return run_fwd<float, 8, MODE>(plan, P, s);
            case 64: return run_fwd<float, 16, MODE>(plan, P, s);
            case 128: return run_fwd<float, 32, MODE>(plan, P, s);
        }
    } else {
        switch (D) {
            case 16: return run_fwd<bf16_tag, 2, MODE>(plan, P, s);
            case 32: return run_fwd<bf16_tag, 4, MODE>(plan, P, s);
            case 64: return run_fwd<bf16_tag, 8, MODE>(plan, P, s);
            case 128: return run_fwd<bf16_tag, 16, MODE>(plan, P, s);
        }
    }
    return GNN_ERR_UNSUPPORTED;
}

static int fwd_common(gnn_plan_t plan, const int32_t *indptr, const int32_t *indices, int32_t N, int64_t E,
                      int32_t H, int32_t D, const void *Q, const void *K, const void *V, void *O, float *LSE,
                      const float *att, float slope, float mul, int mode, gnn_dtype_t dtype, hipStream_t s) {
    GNN_TRY(check_common(plan, indptr, indices, N, E, H, D, dtype));
    if (N > 0 && (!Q || !K || !V || !O)) return GNN_ERR_INVALID_ARG;
    if (mode != M_GT && N > 0 && !att) return GNN_ERR_INVALID_ARG;
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O)) return GNN_ERR_ALIGNMENT;
    if (mode != M_GT && !aligned16(att)) return GNN_ERR_ALIGNMENT;
    if (N == 0) return GNN_OK;
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
        P.light = as<int32_t>(plan->fwd.light);
        P.n_light = plan->fwd.n_light;
        P.groups = as<int32_t>(plan->fwd.groups);
        P.n_groups = plan->fwd.n_groups;
        P.heavy = as<int32_t>(plan->fwd.heavy);
        P.partial_ofs = as<int32_t>(plan->fwd.partial_ofs);
        P.n_heavy = plan->fwd.n_heavy;
        P.C = plan->opts.chunk;
        P.W = plan->opts.waves_per_group;
        if (P.n_groups) {
            const size_t rowlen = (size_t)H * D;
            void *ws = nullptr;
            GNN_TRY(plan_workspace(plan, (size_t)P.n_groups * (rowlen + 2 * H) * sizeof(float), s, &ws));
            P.ws_acc = (float *)ws;
            P.ws_ml = P.ws_acc + (size_t)P.n_groups * rowlen;
        }
    } else {
        P.light = nullptr;
        P.n_light = N;
        P.W = 4;
        P.C = 1;
    }
    if (mode == M_GT) return dispatch_fwd<M_GT>(plan, P, dtype, D, s);
    if (mode == M_GAT_ALIAS) return dispatch_fwd<M_GAT_ALIAS>(plan, P, dtype, D, s);
    return dispatch_fwd<M_GAT_SEPV>(plan, P, dtype, D, s);
}

template <class T, int LH>
static int run_bwd(gnn_plan_t plan, BwdParams &P, hipStream_t s) {
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
    }
    return GNN_OK;
}

}  // namespace gnn

using namespace gnn;

extern "C" {

int gnn_attn_fwd(gnn_plan_t plan, const int32_t *indptr, const int32_t *indices, int32_t N, int64_t E, int32_t H,
                 int32_t D, const void *Q, const void *K, const void *V, void *O, float *LSE, float scale,
                 gnn_dtype_t dtype, hipStream_t stream) {
    const float sc = scale > 0.f ? scale : (float)(1.0 / std::sqrt((double)std::max(D, 1)));
    return fwd_common(plan, indptr, indices, N, E, H, D, Q, K, V, O, LSE, nullptr, 0.f, sc * kLog2e, M_GT, dtype,
                      stream);
}

int gatv2_attn_fwd(gnn_plan_t plan, const int32_t *indptr, const int32_t *indices, int32_t N, int64_t E,
                   int32_t H, int32_t D, const void *Q, const void *K, const void *V, const float *att,
                   float negative_slope, void *O, float *LSE, gnn_dtype_t dtype, hipStream_t stream) {
    const int mode = (V == K) ? M_GAT_ALIAS : M_GAT_SEPV;
    return fwd_common(plan, indptr, indices, N, E, H, D, Q, K, V, O, LSE, att, negative_slope, 1.f, mode, dtype,
                      stream);
}

int gnn_attn_bwd(gnn_plan_t plan, const int32_t *indptr, const int32_t *indices, int32_t N, int64_t E, int32_t H,
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
    const float sc = scale > 0.f ? scale : (float)(1.0 / std::sqrt((double)D));
    BwdParams P{};
    const int LH = lanes_per_head(dtype, D);
    P.g = make_geom(N, H, D, LH);
    P.indptr = indptr;
    P.indices = indices;
    P.cindptr = as<int32_t>(plan->cindptr);
    P.cindices = as<int32_t>(plan->cindices);
    P.Q = Q;
    P.K = K;
    P.V = V;
    P.O = O;
    P.dO = dO;
    P.LSE = LSE;
    P.dQ = dQ;
    P.dK = dK;
    P.dV = dV;
    P.mul = sc * kLog2e;
    P.scale = sc;
    P.a_light = as<int32_t>(plan->fwd.light);
    P.a_groups = as<int32_t>(plan->fwd.groups);
    P.a_heavy = as<int32_t>(plan->fwd.heavy);
    P.a_ofs = as<int32_t>(plan->fwd.partial_ofs);
    P.a_n_light = plan->fwd.n_light;
    P.a_n_groups = plan->fwd.n_groups;
    P.a_n_heavy = plan->fwd.n_heavy;
    P.b_light = as<int32_t>(plan->bwd.light);
    P.b_groups = as<int32_t>(plan->bwd.groups);
    P.b_heavy = as<int32_t>(plan->bwd.heavy);
    P.b_ofs = as<int32_t>(plan->bwd.partial_ofs);
    P.b_n_light = plan->bwd.n_light;
    P.b_n_groups = plan->bwd.n_groups;
    P.b_n_heavy = plan->bwd.n_heavy;
    P.C = plan->opts.chunk;
    P.W = plan->opts.waves_per_group;
    const size_t rowlen = (size_t)H * D;
    const size_t n_stat = (size_t)N * H * 2;
    const size_t n_a = (size_t)P.a_n_groups * (2 * rowlen + H), n_b = (size_t)P.b_n_groups * 2 * rowlen;
    void *ws = nullptr;
    GNN_TRY(plan_workspace(plan, (n_stat + n_a + n_b) * sizeof(float), stream, &ws));
    P.stat = (float2 *)ws;
    P.ws_a = (float *)ws + n_stat;
    P.ws_b = P.ws_a + n_a;
    if (dtype == GNN_F32) {
        switch (D) {
            case 16: return run_bwd<float, 4>(plan, P, stream);
            case 32: return run_bwd<float, 8>(plan, P, stream);
            case 64: return run_bwd<float, 16>(plan, P, stream);
            case 128: return run_bwd<float, 32>(plan, P, stream);
        }
    } else {
        switch (D) {
            case 16: return run_bwd<bf16_tag, 2>(plan, P, stream);
            case 32: return run_bwd<bf16_tag, 4>(plan, P, stream);
            case 64: return run_bwd<bf16_tag, 8>(plan, P, stream);
            case 128: return run_bwd<bf16_tag, 16>(plan, P, stream);
        }
    }
    return GNN_ERR_UNSUPPORTED;
}

}  // extern "C"
