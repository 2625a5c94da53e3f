// Device building blocks shared by the CSR attention kernels and the 16x16
// tile kernels: lane geometry, online-softmax state, the per-node edge
// streams of the forward and of both backward passes, and launch helpers.
#pragma once
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
    int32_t n_long;     // packed launches: the first n_long rows of `light` get a wave each
    const int32_t *groups;
    int32_t n_groups, C;
    const int32_t *heavy, *partial_ofs;
    int32_t n_heavy;
    float *ws_acc, *ws_ml;
    int32_t W;
    // XCD-ordered heavy groups: launch slot -> group (-1: an empty slot), and
    // the number of slots (a multiple of 8); null: slot i runs group i
    const int32_t *gperm;
    int32_t n_slots;
};

// per-lane position inside the wave's (node, head group) slice
struct LanePos {
    int lane, g, r, hh, dv, h;
    int rg0;       // first lane of this lane's row group (RPW rows per wave), else 0
    bool act;
    int64_t col;   // element offset inside the node's H*D row
};

// RPW > 1 (rows of at most 64/RPW lanes, one head group): the wave's lanes
// split into RPW row groups of 64/RPW lanes, each streaming its own row with
// the edge groups g = 0 .. G/RPW - 1 inside it.
template <int LH, int NV, int RPW = 1>
__device__ __forceinline__ LanePos lane_pos(const Geom &G, int hg) {
    LanePos p;
    p.lane = lane_id();
    const int LR = 1 << G.lr_shift;
    p.rg0 = p.lane & ~(kWave / RPW - 1);
    p.g = (p.lane - p.rg0) >> G.lr_shift;
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

template <int NV, int RPW = 1>
__device__ __forceinline__ void merge_groups(SoftState<NV> &st, int lr_shift) {
    for (int off = 1 << lr_shift; off < kWave / RPW; off <<= 1) {
        const float m2 = xor_lane(st.m, off), l2 = xor_lane(st.l, off);
        float a2[NV];
#pragma unroll
        for (int k = 0; k < NV; ++k) a2[k] = xor_lane(st.acc[k], off);
        merge_state(st, m2, l2, a2);
    }
}

// Stream edges [e0, e1) of `node` for this lane's head group; returns the
// wave-merged online-softmax state (valid in every lane). With reset false
// the caller's state is continued (only edge group 0 may carry a non-empty
// state, the other groups must start empty). With RPW > 1 each row group of
// the wave streams its own node and range (lane_pos<..., RPW>) and the merge
// stays inside the row group; the wave steps until every row is done.
template <class T, int LH, int MODE, int U, int RPW = 1>
__device__ __forceinline__ void fwd_stream(const FwdParams &P, const LanePos &lp, int node, int e0, int e1,
                                           SoftState<Vec<T>::N> &st, bool reset = true,
                                           const typename Vec<T>::raw *qown_p = nullptr) {
    using VT = Vec<T>;
    constexpr int NV = VT::N;
    const Geom &G = P.g;
    const int64_t rowlen = (int64_t)G.H * G.D;
    float q[NV];
    float a[NV];
    typename VT::raw qraw = VT::zero();       // the GT score takes q packed (dot_vec)
#pragma unroll
    for (int k = 0; k < NV; ++k) q[k] = a[k] = 0.f;
    if (lp.act) {
        qraw = qown_p ? *qown_p : load_vec<T>(P.Q, (int64_t)node * rowlen + lp.col);
        if (MODE != M_GT) {
            VT::unpack(qraw, q);
#pragma unroll
            for (int k = 0; k < NV; ++k) a[k] = P.att[lp.col + k] * kLog2e;
        }
    }
    if (reset) {
        st.m = kNegInf;
        st.l = 0.f;
#pragma unroll
        for (int k = 0; k < NV; ++k) st.acc[k] = 0.f;
    }

    const int GR = G.G / RPW;                       // edge groups of this row
    const int S = min(kWave / RPW, GR * U);         // edges per step of this row
    const int UE = S / GR;                          // steps per group actually used
    const int li = lp.lane - lp.rg0;
    int jn = (li < S && e0 + li < e1) ? checked_index(P.indices[e0 + li], G.N) : -1;
    // steps until every row of the wave has used up its edges (one row: until base >= e1)
    for (int base = e0; RPW == 1 ? base < e1 : __any(base < e1); base += S) {
        const int jc = jn;
        if (RPW == 1) {
            if (base + S < e1) jn = (li < S && base + S + li < e1) ? checked_index(P.indices[base + S + li], G.N) : -1;
        } else {
            jn = (li < S && base + S + li < e1) ? checked_index(P.indices[base + S + li], G.N) : -1;
        }
        int j[U];
#pragma unroll
        for (int u = 0; u < U; ++u) j[u] = (u < UE) ? __shfl(jc, lp.rg0 + u * GR + lp.g, kWave) : -1;
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
            float t = 0.f;
            if (MODE == M_GT) {
                t = dot_vec(qraw, kr[u], 0.f);
            } else {
                float kf[NV];
                VT::unpack(kr[u], kf);
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
    merge_groups<NV, RPW>(st, G.lr_shift);
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
    store_vec_nt<T>(P.O, (int64_t)node * rowlen + lp.col, VT::pack(o));
    if (P.LSE && lp.dv == 0)
        P.LSE[(int64_t)node * P.g.H + lp.h] = st.l > 0.f ? (st.m + fast_log2(st.l)) * kLn2 : kNegInf;
}

// Main forward kernel: blocks [0, n_groups*NHG) are heavy chunk groups,
// the rest hold W light (node, head group) items, one per wave.

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
    store_vec_nt<T>(base, off, Vec<T>::pack(o));
}

// Destination side over edges [e0, e1) of `node`. With p = exp(s - LSE) and
// dp = <dO_i, V_j> it accumulates A = sum p*dp*K_j, B = sum p*K_j and
// Delta = sum p*dp, so that dQ_i = scale * (A - Delta * B) in one pass.
// Delta is thus formed from the recomputed weights (its definition), not
// from <dO_i, O_i> with a rounded O. Returns this lane's lse2 = LSE*log2 e.
template <class T, int LH, int U>
__device__ __forceinline__ void bwd_dst_stream(const BwdParams &P, const LanePos &lp, int node, int e0, int e1,
                                               float (&A)[Vec<T>::N], float (&B)[Vec<T>::N], float &dsum,
                                               float &lse2, bool reset = true,
                                               const typename Vec<T>::raw *qown_p = nullptr,
                                               const typename Vec<T>::raw *down_p = nullptr) {
    using VT = Vec<T>;
    constexpr int NV = VT::N;
    const Geom &G = P.g;
    const int64_t rowlen = (int64_t)G.H * G.D;
    typename VT::raw q = VT::zero(), dof = VT::zero();   // both dot products take packed operands
    if (reset) {
#pragma unroll
        for (int k = 0; k < NV; ++k) A[k] = B[k] = 0.f;
        dsum = 0.f;
    }
    lse2 = kNegInf;
    if (lp.act) {
        if (qown_p) {
            q = *qown_p;
            dof = *down_p;
        } else {
            q = load_vec<T>(P.Q, (int64_t)node * rowlen + lp.col);
            dof = load_vec<T>(P.dO, (int64_t)node * rowlen + lp.col);
        }
        lse2 = P.LSE[(int64_t)node * G.H + lp.h] * kLog2e;
    }
    const int S = min(kWave, G.G * U);
    const int UE = S / G.G;
    int jn = (lp.lane < S && e0 + lp.lane < e1) ? checked_index(P.indices[e0 + lp.lane], G.N) : -1;
    for (int base = e0; base < e1; base += S) {
        const int jc = jn;
        if (base + S < e1) jn = (lp.lane < S && base + S + lp.lane < e1) ? checked_index(P.indices[base + S + lp.lane], G.N) : -1;
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
            float kf[NV];
            VT::unpack(kr[u], kf);
            float ts = dot_vec(q, kr[u], 0.f), tp = dot_vec(dof, vr[u], 0.f);
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
                                               float (&dk)[Vec<T>::N], float (&dv)[Vec<T>::N],
                                               bool reset = true,
                                               const typename Vec<T>::raw *kown_p = nullptr,
                                               const typename Vec<T>::raw *vown_p = nullptr) {
    using VT = Vec<T>;
    constexpr int NV = VT::N;
    const Geom &G = P.g;
    const int64_t rowlen = (int64_t)G.H * G.D;
    typename VT::raw kown = VT::zero(), vown = VT::zero();   // both dot products take packed operands
    if (reset) {
#pragma unroll
        for (int k = 0; k < NV; ++k) dk[k] = dv[k] = 0.f;
    }
    if (lp.act) {
        if (kown_p) {
            kown = *kown_p;
            vown = *vown_p;
        } else {
            kown = load_vec<T>(P.K, (int64_t)node * rowlen + lp.col);
            vown = load_vec<T>(P.V, (int64_t)node * rowlen + lp.col);
        }
    }
    const int S = min(kWave, G.G * U);
    const int UE = S / G.G;
    int jn = (lp.lane < S && e0 + lp.lane < e1) ? checked_index(P.cindices[e0 + lp.lane], G.N) : -1;
    for (int base = e0; base < e1; base += S) {
        const int jc = jn;
        if (base + S < e1) jn = (lp.lane < S && base + S + lp.lane < e1) ? checked_index(P.cindices[base + S + lp.lane], G.N) : -1;
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
            float ts = dot_vec(qr[u], kown, 0.f), tp = dot_vec(gr[u], vown, 0.f);
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


// ------------------------------------------------------------- host helpers

static inline int ilog2(int x) {
    int s = 0;
    while ((1 << s) < x) ++s;
    return s;
}

// lanes per head for (dtype, D); 0 if unsupported
static inline int lanes_per_head(gnn_dtype_t dt, int D) {
    if (!(D == 16 || D == 32 || D == 64 || D == 128)) return 0;
    if (dt == GNN_F32) return D / 4;
    if (dt == GNN_BF16) return D / 8;
    return 0;
}

static inline Geom make_geom(int N, int H, int D, int LH) {
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

static inline bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

static inline int check_common(gnn_plan_t plan, const int32_t *indptr, const int32_t *indices, int32_t N, int64_t E,
                        int32_t H, int32_t D, gnn_dtype_t dtype) {
    if (N < 0 || E < 0 || E > kMaxEdges || H < 1 || !indptr) return GNN_ERR_INVALID_ARG;
    if (E > 0 && !indices) return GNN_ERR_INVALID_ARG;
    if (dtype != GNN_F32 && dtype != GNN_BF16) return GNN_ERR_UNSUPPORTED;
    if (!lanes_per_head(dtype, D)) return GNN_ERR_UNSUPPORTED;
    if ((int64_t)N * H * D >= (1ll << 40)) return GNN_ERR_INVALID_ARG;
    if (plan && (plan->n_nodes != N || plan->n_edges != E || plan->indptr != indptr || plan->indices != indices))
        return GNN_ERR_INVALID_ARG;
    return GNN_OK;
}

// backward parameters from a plan (CSR and transposed-adjacency buckets)
static inline void fill_bwd_params(gnn_plan_t plan, BwdParams &P, const int32_t *indptr, const int32_t *indices,
                                   int32_t N, int32_t H, int32_t D, const void *Q, const void *K, const void *V,
                                   const void *dO, const float *LSE, void *dQ, void *dK, void *dV, float sc,
                                   gnn_dtype_t dtype) {
    P.g = make_geom(N, H, D, lanes_per_head(dtype, D));
    P.indptr = indptr;
    P.indices = indices;
    P.cindptr = as<int32_t>(plan->cindptr);
    P.cindices = as<int32_t>(plan->cindices);
    P.Q = Q;
    P.K = K;
    P.V = V;
    P.O = nullptr;
    P.dO = dO;
    P.LSE = LSE;
    P.dQ = dQ;
    P.dK = dK;
    P.dV = dV;
    P.mul = sc * kLog2e;
    P.scale = sc;
    P.a_light = as<int32_t>(plan->fwd.sched);
    P.a_groups = as<int32_t>(plan->fwd.groups);
    P.a_heavy = as<int32_t>(plan->fwd.heavy);
    P.a_ofs = as<int32_t>(plan->fwd.partial_ofs);
    P.a_n_light = plan->fwd.n_light;
    P.a_n_groups = plan->fwd.n_groups;
    P.a_n_heavy = plan->fwd.n_heavy;
    P.b_light = as<int32_t>(plan->bwd.sched);
    P.b_groups = as<int32_t>(plan->bwd.groups);
    P.b_heavy = as<int32_t>(plan->bwd.heavy);
    P.b_ofs = as<int32_t>(plan->bwd.partial_ofs);
    P.b_n_light = plan->bwd.n_light;
    P.b_n_groups = plan->bwd.n_groups;
    P.b_n_heavy = plan->bwd.n_heavy;
    P.C = plan->opts.chunk;
    P.W = plan->opts.waves_per_group;
}

// kernel launch with optional per-kernel event timing on the plan
template <class K, class... Args>
static int launch(gnn_plan_t plan, int kind, K kernel, dim3 grid, dim3 block, size_t lds, hipStream_t s,
                  const Args &...args) {
    if (grid.x == 0) return GNN_OK;
    TimingRec rec;
    const bool timed = plan && plan->timer.enabled;
    if (timed) GNN_TRY(plan->timer.begin(kind, s, rec));
    hipLaunchKernelGGL(kernel, grid, block, lds, s, args...);
    GNN_HIP(hipGetLastError());
    if (timed) GNN_TRY(plan->timer.end(rec, s));
    return GNN_OK;
}

// 16x16 tile kernels (attn_tile.hip): true when the tile path serves this
// dtype / head size; the launchers run the tiled row (or column) blocks
bool tile_supported(gnn_dtype_t dt, int D);
int launch_tile_fwd(gnn_plan_t plan, const FwdParams &P, int D, hipStream_t s);
int launch_tile_bwd_dst(gnn_plan_t plan, const BwdParams &P, int D, hipStream_t s);
int launch_tile_bwd_src(gnn_plan_t plan, const BwdParams &P, int D, hipStream_t s);

}  // namespace gnn
