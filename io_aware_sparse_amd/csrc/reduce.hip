// Degree-aware neighbourhood max / min reduction with the winning source.
//
// "On Efficient Scaling of GNNs via IO-Aware Layers Implementations",
// technical summary, Methodology (reduction-based aggregations): a per-edge
// computation followed by a neighbourhood min/max; nodes split by a degree
// threshold into light ones, served by a feature-parallel kernel, and heavy
// ones, whose edge lists are cut into chunks reduced in parallel and merged
// with atomic operations on packed (value, index) pairs.
//
// Message of entry (i, j) of row i: m = X[j] (GNN_MSG_SRC) or X[j] - X[i]
// (GNN_MSG_DIFF, one fp32 subtraction). out[i,f] = max (or min) of m[f] over
// the row's entries, arg[i,f] = the smallest j attaining it (values compare
// as floats: -0 == +0); an empty row gives 0 and -1.
//
// Lane geometry: a lane holds one 16-byte slice of a feature row (4 fp32 or
// 8 bf16). A row of L = F*s/16 slices takes LR = next_pow2(L) lanes when
// L <= 64 (64/LR edge groups per wave), else whole waves over NFG = ceil(L/64)
// feature groups. Light rows: one wave per (row, feature group), or on a
// plan with sorted rows 4 or 2 rows per wave for rows of at most 256 or 512
// bytes (see run_red_fwd), the best
// (value, source) pair of each feature kept in registers, edge groups merged
// by a xor tree with the same ordering rule. Heavy rows: the plan's chunk
// groups (C edges per wave, W waves); each wave reduces its chunk and merges
// into a per-heavy-row slot with one 64-bit atomic max / min per feature on
// the key (order-preserving value bits << 32 | source term), whose winner is
// the same pair under any arrival order; a last pass decodes the winner and
// recomputes its message from X, so the stored value is bit for bit the
// winner's (signed zeros included).
//
// Backward (gradient of the max / min through the winners): over the
// transposed adjacency, source j adds dOut[i,f] for every destination i whose
// winner arg[i,f] is j (a source listed several times in row i counts once:
// repeated entries of a transposed row are adjacent and skipped); with
// difference messages row j also loses dOut[j,f] when it is not empty. The
// sum runs in a fixed order (edge groups by a xor tree, heavy-source chunks in
// LDS and then by group in ascending order): no float atomics, bitwise
// reproducible.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "attn_core.h"
#include "gnn_reduce.h"

namespace gnn {

struct RedGeom {
    int32_t N = 0, F = 0;
    int32_t L = 0;          // 16-byte slices per row
    int32_t lr_shift = 0;   // log2 lanes per row slice group (LR)
    int32_t G = 1;          // edge groups per wave
    int32_t NFG = 1;        // feature groups (waves) per row
};

struct RedParams {
    RedGeom g;
    const int32_t *indptr, *indices;   // CSR (forward) or transposed adjacency (backward)
    const int32_t *rowptr;             // backward: CSR indptr (is row j empty?)
    const void *X;                     // forward messages' table; backward: dOut
    void *out;                         // forward out; backward dX
    int32_t *arg;                      // forward arg (nullable)
    const int32_t *arg_in;             // backward: the forward's winners
    const int32_t *light;              // nullable: identity
    int32_t n_light;
    const int32_t *groups;             // (node, e0, e1) per chunk group
    int32_t n_groups;
    const int32_t *heavy;
    const int32_t *partial_ofs;
    int32_t n_heavy;
    int32_t C, W;
    unsigned long long *keys;          // forward: [n_heavy][F] packed winners
    float *part;                       // backward: [n_groups][F] fp32 group partials
};

// With RPW rows per wave the 64 lanes split into RPW row groups of 64/RPW
// lanes, each holding G/RPW edge groups of LR lanes (RPW = 1: one row, G
// edge groups).
struct RLane {
    int lane, g, c;     // lane, edge group within the row group, lane within the edge group
    int rg0;            // first lane of the row group
    int slice;          // 16-byte slice of the row this lane holds
    bool act;           // slice < L
    int64_t col;        // first element of the slice
};

template <int NV, int RPW = 1>
__device__ __forceinline__ RLane rlane(const RedGeom &G, int fg) {
    RLane r;
    r.lane = lane_id();
    const int LR = 1 << G.lr_shift;
    r.rg0 = r.lane & ~(kWave / RPW - 1);
    r.g = (r.lane - r.rg0) >> G.lr_shift;
    r.c = r.lane & (LR - 1);
    r.slice = fg * kWave + r.c;
    r.act = r.slice < G.L;
    r.col = (int64_t)r.slice * NV;
    return r;
}

// Does (v, j) beat the current best (b, bj)? Empty candidates (j < 0) never
// do; any candidate beats an empty best; equal values go to the smaller source.
// (bitwise & and | on purpose: no short-circuit branches, the callers' updates stay selects)
template <int OP>
__device__ __forceinline__ bool better(float v, int j, float b, int bj) {
    const bool strict = OP == GNN_REDUCE_MAX ? (v > b) : (v < b);
    return (j >= 0) & ((bj < 0) | strict | ((v == b) & (j < bj)));
}

__device__ __forceinline__ int xor_int(int x, int off) { return __shfl_xor(x, off, kWave); }

// SORTED: the row lists its sources in non-decreasing order, so a lane meets
// its edges' sources in non-decreasing order and a strict comparison alone
// keeps the smallest source among equal values; the group merge below still
// applies the full rule. Otherwise every step applies the full rule.
template <class T, int OP, int MSG, int U, bool SORTED, int RPW = 1>
__device__ __forceinline__ void red_stream(const RedParams &P, const RLane &lp, int node, int e0, int e1,
                                           float (&best)[Vec<T>::N], int (&bj)[Vec<T>::N]) {
    using VT = Vec<T>;
    constexpr int NV = VT::N;
    constexpr float kWorst = OP == GNN_REDUCE_MAX ? -INFINITY : INFINITY;
    const RedGeom &G = P.g;
    const int64_t F = G.F;
    float xi[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        xi[k] = 0.f;
        best[k] = SORTED ? kWorst : 0.f;
        bj[k] = -1;
    }
    if (MSG == GNN_MSG_DIFF && lp.act && node >= 0) VT::unpack(load_vec<T>(P.X, (int64_t)node * F + lp.col), xi);
    constexpr int kLanesRG = kWave / RPW;
    const int GR = G.G / RPW;                 // edge groups of this row
    const int S = min(kLanesRG, GR * U);      // edges per step of this row
    const int UE = S / GR;
    const int li = lp.lane - lp.rg0;
    int jn = (li < S && e0 + li < e1) ? checked_index(P.indices[e0 + li], G.N) : -1;
    // steps until every row group of the wave has used up its edges (one row: until base >= e1)
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
        // every lane loads (a lane without an edge, or past the row's slices, reads slice 0 of row 0 and
        // ignores it), so the loads need no branch; the updates below are selects
        typename VT::raw r[U];
        bool ok[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            ok[u] = lp.act & (j[u] >= 0);
            const int row = ok[u] ? j[u] : 0;
            const int64_t col = ok[u] ? lp.col : 0;
            r[u] = load_vec<T>(P.X, (int64_t)row * F + col);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float v[NV];
            VT::unpack(r[u], v);
#pragma unroll
            for (int k = 0; k < NV; ++k) {
                const float m = MSG == GNN_MSG_DIFF ? v[k] - xi[k] : v[k];
                const bool take = SORTED ? (ok[u] & (OP == GNN_REDUCE_MAX ? m > best[k] : m < best[k]))
                                         : (ok[u] & better<OP>(m, j[u], best[k], bj[k]));
                best[k] = take ? m : best[k];
                bj[k] = take ? j[u] : bj[k];
            }
        }
    }
    if (SORTED) {
        // a group whose messages all equal the worst value (an infinity) took none of them: its first
        // edge wins; a group without edges stays empty with value 0
        const int e_first = e0 + lp.g;
        const int j_first = e_first < e1 ? checked_index(P.indices[e_first], G.N) : -1;
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            if (bj[k] < 0) {
                bj[k] = j_first;
                if (j_first < 0) best[k] = 0.f;
            }
        }
    }
    // merge the edge groups of the row (lane c of every group ends with the same pair)
    for (int off = 1 << G.lr_shift; off < kLanesRG; off <<= 1) {
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const float ov = xor_lane(best[k], off);
            const int oj = xor_int(bj[k], off);
            const bool take = better<OP>(ov, oj, best[k], bj[k]);
            best[k] = take ? ov : best[k];
            bj[k] = take ? oj : bj[k];
        }
    }
}

// Output row slice: source messages are values of X itself (exact in the
// storage type: bf16 keeps the high half of the fp32 image); difference
// messages are rounded to the storage type (nearest even).
template <class T, int MSG>
__device__ __forceinline__ typename Vec<T>::raw pack_out(const float (&x)[Vec<T>::N]) {
    if constexpr (Vec<T>::bytes == 2 && MSG == GNN_MSG_SRC) {
        uint32_t w[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) w[k] = (__float_as_uint(x[2 * k]) >> 16) | (__float_as_uint(x[2 * k + 1]) & 0xFFFF0000u);
        return make_uint4(w[0], w[1], w[2], w[3]);
    } else {
        return Vec<T>::pack(x);
    }
}

// order-preserving 32-bit image of a float, with -0 mapped onto +0
__device__ __forceinline__ uint32_t ordered_bits(float v) {
    const uint32_t u = __float_as_uint(v == 0.f ? 0.f : v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <int OP>
__device__ __forceinline__ unsigned long long pack_key(float v, int j) {
    const uint32_t lo = OP == GNN_REDUCE_MAX ? 0xFFFFFFFFu - (uint32_t)j : (uint32_t)j;
    return ((unsigned long long)ordered_bits(v) << 32) | lo;
}

template <int OP>
__device__ __forceinline__ unsigned long long key_identity() {
    return OP == GNN_REDUCE_MAX ? 0ull : ~0ull;
}

template <int OP>
__global__ void k_red_init(unsigned long long *keys, int64_t n) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t < n) keys[t] = key_identity<OP>();
}

// heavy index of chunk group grp (partial_ofs[h] <= grp < partial_ofs[h + 1])
__device__ __forceinline__ int heavy_of_group(const int32_t *partial_ofs, int n_heavy, int grp) {
    int lo = 0, hi = n_heavy - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (partial_ofs[mid] <= grp)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

template <class T, int OP, int MSG, int U, bool SORTED, int RPW>
__global__ __launch_bounds__(512) void k_red_main(RedParams P) {
    using VT = Vec<T>;
    constexpr int NV = VT::N;
    const RedGeom &G = P.g;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int heavy_blocks = P.n_groups * G.NFG;
    float best[NV];
    int bj[NV];
    if ((int)blockIdx.x < heavy_blocks) {
        const int grp = blockIdx.x / G.NFG, fg = blockIdx.x % G.NFG;
        const int node = P.groups[3 * grp], g0 = P.groups[3 * grp + 1], g1 = P.groups[3 * grp + 2];
        const int e0 = min(g1, g0 + w * P.C), e1 = min(g1, e0 + P.C);
        const RLane lp = rlane<NV>(G, fg);
        red_stream<T, OP, MSG, U, SORTED, 1>(P, lp, node, e0, e1, best, bj);
        if (lp.g != 0 || !lp.act) return;
        const int h = heavy_of_group(P.partial_ofs, P.n_heavy, grp);
        unsigned long long *slot = P.keys + (int64_t)h * G.F + lp.col;
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            if (bj[k] < 0) continue;
            if (OP == GNN_REDUCE_MAX)
                atomicMax(slot + k, pack_key<OP>(best[k], bj[k]));
            else
                atomicMin(slot + k, pack_key<OP>(best[k], bj[k]));
        }
        return;
    }
    const int64_t item = (int64_t)(blockIdx.x - heavy_blocks) * P.W + w;
    int node;
    int fg = 0;
    const RLane lp = rlane<NV, RPW>(G, 0);
    if (RPW == 1) {
        const int64_t ni = item / G.NFG;
        if (ni >= P.n_light) return;
        fg = (int)(item % G.NFG);
        node = P.light ? P.light[ni] : (int)ni;
    } else {                                  // RPW rows of the light list per wave (NFG == 1)
        const int64_t ni0 = item * RPW;
        if (ni0 >= P.n_light) return;
        const int64_t ni = ni0 + lp.rg0 / (kWave / RPW);
        node = ni < P.n_light ? P.light[ni] : -1;
    }
    const RLane lq = RPW == 1 ? rlane<NV>(G, fg) : lp;
    const int e0 = node >= 0 ? P.indptr[node] : 0, e1 = node >= 0 ? P.indptr[node + 1] : 0;
    red_stream<T, OP, MSG, U, SORTED, RPW>(P, lq, node, e0, e1, best, bj);
    if (lq.g != 0 || !lq.act || node < 0) return;
    const int64_t off = (int64_t)node * G.F + lq.col;
    store_vec<T>(P.out, off, pack_out<T, MSG>(best));
    if (P.arg) {
        int4 *a = reinterpret_cast<int4 *>(P.arg + off);
#pragma unroll
        for (int q = 0; q < NV / 4; ++q) a[q] = make_int4(bj[4 * q], bj[4 * q + 1], bj[4 * q + 2], bj[4 * q + 3]);
    }
}

template <class T>
__device__ __forceinline__ float load_elem(const void *base, int64_t e) {
    if constexpr (Vec<T>::bytes == 4) {
        return reinterpret_cast<const float *>(base)[e];
    } else {
        return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t *>(base)[e] << 16);
    }
}

template <class T>
__device__ __forceinline__ void store_elem(void *base, int64_t e, float v) {
    if constexpr (Vec<T>::bytes == 4)
        reinterpret_cast<float *>(base)[e] = v;
    else
        reinterpret_cast<uint16_t *>(base)[e] = (uint16_t)f32_to_bf16_rne(v);
}

// one thread per (heavy row, feature): decode the winner, recompute its message
template <class T, int OP, int MSG>
__global__ void k_red_final(RedParams P) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t F = P.g.F;
    if (t >= (int64_t)P.n_heavy * F) return;
    const int h = (int)(t / F);
    const int64_t f = t % F;
    const int node = P.heavy[h];
    const unsigned long long key = P.keys[t];
    int j = -1;
    float v = 0.f;
    if (key != key_identity<OP>()) {
        const uint32_t lo = (uint32_t)(key & 0xFFFFFFFFull);
        j = (int)(OP == GNN_REDUCE_MAX ? 0xFFFFFFFFu - lo : lo);
        v = load_elem<T>(P.X, (int64_t)j * F + f);
        if (MSG == GNN_MSG_DIFF) v = v - load_elem<T>(P.X, (int64_t)node * F + f);
    }
    store_elem<T>(P.out, (int64_t)node * F + f, v);
    if (P.arg) P.arg[(int64_t)node * F + f] = j;
}

// ------------------------------------------------------------------ backward

template <class T, int U>
__device__ __forceinline__ void red_bwd_stream(const RedParams &P, const RLane &lp, int src, int row0, int e0, int e1,
                                               float (&acc)[Vec<T>::N]) {
    using VT = Vec<T>;
    constexpr int NV = VT::N;
    const RedGeom &G = P.g;
    const int64_t F = G.F;
#pragma unroll
    for (int k = 0; k < NV; ++k) acc[k] = 0.f;
    const int S = min(kWave, G.G * U);
    const int UE = S / G.G;
    // entry e is skipped when it repeats entry e-1 of the same transposed row
    auto fetch = [&](int e) -> int {
        if (e >= e1) return -1;
        const int i = checked_index(P.indices[e], G.N);
        return (e > row0 && P.indices[e - 1] == i) ? -1 : i;
    };
    int jn = lp.lane < S ? fetch(e0 + lp.lane) : -1;
    for (int base = e0; base < e1; base += S) {
        const int jc = jn;
        if (base + S < e1) jn = lp.lane < S ? fetch(base + S + lp.lane) : -1;
        int i[U];
#pragma unroll
        for (int u = 0; u < U; ++u) i[u] = (u < UE) ? __shfl(jc, u * G.G + lp.g, kWave) : -1;
        typename VT::raw gr[U];
        int4 ar[U][NV / 4];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool ok = lp.act && i[u] >= 0;
            const int64_t off = (int64_t)i[u] * F + lp.col;
            gr[u] = ok ? load_vec<T>(P.X, off) : VT::zero();
#pragma unroll
            for (int q = 0; q < NV / 4; ++q)
                ar[u][q] = ok ? reinterpret_cast<const int4 *>(P.arg_in + off)[q] : make_int4(-1, -1, -1, -1);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float gv[NV];
            VT::unpack(gr[u], gv);
#pragma unroll
            for (int q = 0; q < NV / 4; ++q) {
                const int aq[4] = {ar[u][q].x, ar[u][q].y, ar[u][q].z, ar[u][q].w};
#pragma unroll
                for (int k = 0; k < 4; ++k) acc[4 * q + k] += (aq[k] == src) ? gv[4 * q + k] : 0.f;
            }
        }
    }
    for (int off = 1 << G.lr_shift; off < kWave; off <<= 1) {
#pragma unroll
        for (int k = 0; k < NV; ++k) acc[k] += xor_lane(acc[k], off);
    }
}

template <class T, int MSG>
__device__ __forceinline__ void red_bwd_store(const RedParams &P, const RLane &lp, int src, float (&acc)[Vec<T>::N]) {
    using VT = Vec<T>;
    constexpr int NV = VT::N;
    const int64_t off = (int64_t)src * P.g.F + lp.col;
    if (MSG == GNN_MSG_DIFF && P.rowptr[src + 1] > P.rowptr[src]) {
        float own[NV];
        VT::unpack(load_vec<T>(P.X, off), own);
#pragma unroll
        for (int k = 0; k < NV; ++k) acc[k] -= own[k];
    }
    store_vec<T>(P.out, off, VT::pack(acc));
}

template <class T, int MSG, int U>
__global__ __launch_bounds__(512) void k_red_bwd_main(RedParams P) {
    using VT = Vec<T>;
    constexpr int NV = VT::N;
    extern __shared__ float lds[];
    const RedGeom &G = P.g;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int heavy_blocks = P.n_groups * G.NFG;
    float acc[NV];
    if ((int)blockIdx.x < heavy_blocks) {
        const int grp = blockIdx.x / G.NFG, fg = blockIdx.x % G.NFG;
        const int src = P.groups[3 * grp], g0 = P.groups[3 * grp + 1], g1 = P.groups[3 * grp + 2];
        const int e0 = min(g1, g0 + w * P.C), e1 = min(g1, e0 + P.C);
        const RLane lp = rlane<NV>(G, fg);
        red_bwd_stream<T, U>(P, lp, src, P.indptr[src], e0, e1, acc);
        // waves of the group summed in LDS in ascending wave order
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
    const int64_t ni = item / G.NFG;
    if (ni >= P.n_light) return;
    const int fg = (int)(item % G.NFG);
    const int src = P.light ? P.light[ni] : (int)ni;
    const RLane lp = rlane<NV>(G, fg);
    red_bwd_stream<T, U>(P, lp, src, P.indptr[src], P.indptr[src], P.indptr[src + 1], acc);
    if (lp.g != 0 || !lp.act) return;
    red_bwd_store<T, MSG>(P, lp, src, acc);
}

// heavy sources: their groups' partials summed in ascending group order
template <class T, int MSG>
__global__ void k_red_bwd_merge(RedParams P) {
    using VT = Vec<T>;
    constexpr int NV = VT::N;
    const RedGeom &G = P.g;
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= (int64_t)P.n_heavy * G.L) return;
    const int h = (int)(t / G.L);
    const int slice = (int)(t % G.L);
    const int src = P.heavy[h];
    const int64_t col = (int64_t)slice * NV;
    float acc[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) acc[k] = 0.f;
    for (int grp = P.partial_ofs[h]; grp < P.partial_ofs[h + 1]; ++grp) {
        const float *p = P.part + (int64_t)grp * G.F + col;
#pragma unroll
        for (int k = 0; k < NV; ++k) acc[k] += p[k];
    }
    RLane lp;
    lp.col = col;
    red_bwd_store<T, MSG>(P, lp, src, acc);
}

// ------------------------------------------------------------------ host

static RedGeom red_geom(int32_t N, int32_t F, gnn_dtype_t dt) {
    RedGeom g;
    g.N = N;
    g.F = F;
    const int s = dt == GNN_BF16 ? 2 : 4;
    g.L = (int32_t)(((int64_t)F * s) / 16);
    if (g.L <= kWave) {
        int sh = 0;
        while ((1 << sh) < g.L) ++sh;
        g.lr_shift = sh;
        g.G = kWave >> sh;
        g.NFG = 1;
    } else {
        g.lr_shift = 6;
        g.G = 1;
        g.NFG = (g.L + kWave - 1) / kWave;
    }
    return g;
}

static int red_check(gnn_plan_t plan, const int32_t *indptr, const int32_t *indices, int32_t N, int64_t E, int32_t F,
                     gnn_dtype_t dtype) {
    if (N < 0 || E < 0 || E > kMaxEdges || F < 1 || !indptr) return GNN_ERR_INVALID_ARG;
    if (E > 0 && !indices) return GNN_ERR_INVALID_ARG;
    if (dtype != GNN_F32 && dtype != GNN_BF16) return GNN_ERR_UNSUPPORTED;
    const int s = dtype == GNN_BF16 ? 2 : 4;
    if (((int64_t)F * s) % 16) return GNN_ERR_UNSUPPORTED;
    if ((int64_t)N * F >= (1ll << 40)) return GNN_ERR_INVALID_ARG;
    if (plan && (plan->n_nodes != N || plan->n_edges != E || plan->indptr != indptr || plan->indices != indices))
        return GNN_ERR_INVALID_ARG;
    return GNN_OK;
}

template <class T, int OP, int MSG, bool SORTED, int RPW, int U = 4>
static int launch_red_main(gnn_plan_t plan, const RedParams &P, hipStream_t s) {
    const int64_t light_waves = RPW == 1 ? (int64_t)P.n_light * P.g.NFG : ((int64_t)P.n_light + RPW - 1) / RPW;
    const int64_t blocks = (int64_t)P.n_groups * P.g.NFG + (light_waves + P.W - 1) / P.W;
    if (blocks >= (1ll << 31)) return GNN_ERR_INVALID_ARG;
    return launch(plan, K_RED_MAIN, k_red_main<T, OP, MSG, U, SORTED, RPW>, dim3((unsigned)blocks), dim3(64 * P.W),
                  0, s, P);
}

// Sorted rows on a plan, rows of up to 32 lanes (512 bytes): the light rows
// run from the packed-order list, 4 per wave (rows of up to 256 bytes) or 2
// per wave with 10 edges per step in fp32, 8 in bf16 (up to 512 bytes, so a
// row keeps at least the 8 edges per step it has alone), so rows of similar
// length share a wave and each row merges only its own edge groups.
// Otherwise (wider rows, or unsorted rows) one row per wave.
template <class T, int OP, int MSG>
static int run_red_fwd(gnn_plan_t plan, RedParams &P, hipStream_t s) {
    const int64_t nk = (int64_t)P.n_heavy * P.g.F;
    if (nk) GNN_TRY(launch(plan, K_RED_INIT, k_red_init<OP>, grid1d(nk), dim3(256), 0, s, P.keys, nk));
    if (plan && plan->rows_sorted) {
        if (P.g.NFG == 1 && P.g.G >= 2) {
            RedParams Q = P;
            Q.light = as<int32_t>(plan->fwd.by_degree);
            constexpr int U2 = Vec<T>::bytes == 4 ? 10 : 8;
            if (P.g.G >= 4) GNN_TRY((launch_red_main<T, OP, MSG, true, 4>(plan, Q, s)));
            else GNN_TRY((launch_red_main<T, OP, MSG, true, 2, U2>(plan, Q, s)));
        } else {
            GNN_TRY((launch_red_main<T, OP, MSG, true, 1>(plan, P, s)));
        }
    } else {
        GNN_TRY((launch_red_main<T, OP, MSG, false, 1>(plan, P, s)));
    }
    if (nk) GNN_TRY(launch(plan, K_RED_FINAL, k_red_final<T, OP, MSG>, grid1d(nk), dim3(256), 0, s, P));
    return GNN_OK;
}

template <class T, int MSG>
static int run_red_bwd(gnn_plan_t plan, RedParams &P, hipStream_t s) {
    constexpr int U = 4;
    constexpr int NV = Vec<T>::N;
    const int64_t lb = ((int64_t)P.n_light * P.g.NFG + P.W - 1) / P.W;
    const int64_t blocks = (int64_t)P.n_groups * P.g.NFG + lb;
    if (blocks >= (1ll << 31)) return GNN_ERR_INVALID_ARG;
    const size_t lds = P.n_groups ? (size_t)P.W * (1 << P.g.lr_shift) * NV * sizeof(float) : 0;
    GNN_TRY(launch(plan, K_RED_BWD_MAIN, k_red_bwd_main<T, MSG, U>, dim3((unsigned)blocks), dim3(64 * P.W), lds, s,
                   P));
    const int64_t nm = (int64_t)P.n_heavy * P.g.L;
    if (nm) GNN_TRY(launch(plan, K_RED_BWD_MERGE, k_red_bwd_merge<T, MSG>, grid1d(nm), dim3(256), 0, s, P));
    return GNN_OK;
}

template <class T>
static int dispatch_red_fwd(gnn_plan_t plan, RedParams &P, int op, int msg, hipStream_t s) {
    if (op == GNN_REDUCE_MAX)
        return msg == GNN_MSG_SRC ? run_red_fwd<T, GNN_REDUCE_MAX, GNN_MSG_SRC>(plan, P, s)
                                  : run_red_fwd<T, GNN_REDUCE_MAX, GNN_MSG_DIFF>(plan, P, s);
    return msg == GNN_MSG_SRC ? run_red_fwd<T, GNN_REDUCE_MIN, GNN_MSG_SRC>(plan, P, s)
                              : run_red_fwd<T, GNN_REDUCE_MIN, GNN_MSG_DIFF>(plan, P, s);
}

// this file's kernels' index flag (checked builds)
GNN_INDEX_FAULT_READER(index_fault_reduce)

}  // namespace gnn

using namespace gnn;

extern "C" {

static int reduce_fwd_impl(gnn_plan_t plan, const int32_t *indptr, const int32_t *indices, int32_t N, int64_t E, int32_t F,
                   const void *X, void *out, int32_t *arg, gnn_reduce_op_t op, gnn_msg_t msg, gnn_dtype_t dtype,
                   hipStream_t stream) {
    GNN_TRY(red_check(plan, indptr, indices, N, E, F, dtype));
    if (op != GNN_REDUCE_MAX && op != GNN_REDUCE_MIN) return GNN_ERR_INVALID_ARG;
    if (msg != GNN_MSG_SRC && msg != GNN_MSG_DIFF) return GNN_ERR_INVALID_ARG;
    if (N > 0 && (!X || !out)) return GNN_ERR_INVALID_ARG;
    if (!aligned16(X) || !aligned16(out) || !aligned16(arg)) return GNN_ERR_ALIGNMENT;
    if (N == 0) return GNN_OK;
    GNN_TRY(checked_graph(indptr, indices, N, E, stream));
    RedParams P{};
    P.g = red_geom(N, F, dtype);
    P.indptr = indptr;
    P.indices = indices;
    P.X = X;
    P.out = out;
    P.arg = arg;
    if (plan) {
        P.light = as<int32_t>(plan->fwd.sched);
        P.n_light = plan->fwd.n_light;
        P.groups = as<int32_t>(plan->fwd.groups);
        P.n_groups = plan->fwd.n_groups;
        P.heavy = as<int32_t>(plan->fwd.heavy);
        P.partial_ofs = as<int32_t>(plan->fwd.partial_ofs);
        P.n_heavy = plan->fwd.n_heavy;
        P.C = plan->opts.chunk;
        P.W = plan->opts.waves_per_group;
        if (P.n_heavy) {
            void *ws = nullptr;
            GNN_TRY(plan_workspace(plan, (size_t)P.n_heavy * F * sizeof(unsigned long long), stream, &ws));
            P.keys = (unsigned long long *)ws;
        }
    } else {
        P.light = nullptr;
        P.n_light = N;
        P.W = 4;
        P.C = 1;
    }
    if (dtype == GNN_BF16) return dispatch_red_fwd<bf16_tag>(plan, P, op, msg, stream);
    return dispatch_red_fwd<float>(plan, P, op, msg, stream);
}

int gnn_reduce_fwd(gnn_plan_t plan, const int32_t *indptr, const int32_t *indices, int32_t N, int64_t E, int32_t F,
                   const void *X, void *out, int32_t *arg, gnn_reduce_op_t op, gnn_msg_t msg, gnn_dtype_t dtype,
                   hipStream_t stream) {
    return finish_call(reduce_fwd_impl(plan, indptr, indices, N, E, F, X, out, arg, op, msg, dtype, stream), stream);
}

static int reduce_bwd_impl(gnn_plan_t plan, const int32_t *indptr, const int32_t *indices, int32_t N, int64_t E, int32_t F,
                   const void *dOut, const int32_t *arg, void *dX, gnn_msg_t msg, gnn_dtype_t dtype,
                   hipStream_t stream) {
    if (!plan) return GNN_ERR_INVALID_ARG;
    GNN_TRY(red_check(plan, indptr, indices, N, E, F, dtype));
    if (!plan->has_csc) return GNN_ERR_UNSUPPORTED;
    if (msg != GNN_MSG_SRC && msg != GNN_MSG_DIFF) return GNN_ERR_INVALID_ARG;
    if (N > 0 && (!dOut || !arg || !dX)) return GNN_ERR_INVALID_ARG;
    if (!aligned16(dOut) || !aligned16(arg) || !aligned16(dX)) return GNN_ERR_ALIGNMENT;
    if (N == 0) return GNN_OK;
    GNN_TRY(checked_graph(indptr, indices, N, E, stream));
    RedParams P{};
    P.g = red_geom(N, F, dtype);
    P.indptr = as<int32_t>(plan->cindptr);
    P.indices = as<int32_t>(plan->cindices);
    P.rowptr = indptr;
    P.X = dOut;
    P.out = dX;
    P.arg_in = arg;
    P.light = as<int32_t>(plan->bwd.sched);
    P.n_light = plan->bwd.n_light;
    P.groups = as<int32_t>(plan->bwd.groups);
    P.n_groups = plan->bwd.n_groups;
    P.heavy = as<int32_t>(plan->bwd.heavy);
    P.partial_ofs = as<int32_t>(plan->bwd.partial_ofs);
    P.n_heavy = plan->bwd.n_heavy;
    P.C = plan->opts.chunk;
    P.W = plan->opts.waves_per_group;
    if (P.n_groups) {
        void *ws = nullptr;
        GNN_TRY(plan_workspace(plan, (size_t)P.n_groups * F * sizeof(float), stream, &ws));
        P.part = (float *)ws;
    }
    if (dtype == GNN_BF16)
        return msg == GNN_MSG_SRC ? run_red_bwd<bf16_tag, GNN_MSG_SRC>(plan, P, stream)
                                  : run_red_bwd<bf16_tag, GNN_MSG_DIFF>(plan, P, stream);
    return msg == GNN_MSG_SRC ? run_red_bwd<float, GNN_MSG_SRC>(plan, P, stream)
                              : run_red_bwd<float, GNN_MSG_DIFF>(plan, P, stream);
}

int gnn_reduce_bwd(gnn_plan_t plan, const int32_t *indptr, const int32_t *indices, int32_t N, int64_t E, int32_t F,
                   const void *dOut, const int32_t *arg, void *dX, gnn_msg_t msg, gnn_dtype_t dtype,
                   hipStream_t stream) {
    return finish_call(reduce_bwd_impl(plan, indptr, indices, N, E, F, dOut, arg, dX, msg, dtype, stream), stream);
}

}  // extern "C"
