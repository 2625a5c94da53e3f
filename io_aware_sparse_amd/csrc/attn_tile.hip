// 16x16 block-tile attention on the matrix cores (bf16 inputs, fp32 accumulate).
//
// "On Efficient Scaling of GNNs via IO-Aware Layers Implementations",
// technical summary, Methodology (attention-based layers, Tensor-Core
// optimisation): local neighbourhoods packed into 16x16 tiles so that the
// score and aggregation products of a dense block run on matrix units.
//
// One workgroup (8 waves) owns one aligned block of 16 destination rows (or,
// for the source pass of the backward, 16 source columns) and one head group.
// Phase 1 walks the block's tiles: each wave takes heads of the group and
// runs, per tile,
//   forward:      S^T = K_b Q_b^T                      (v_mfma 16x16x32 bf16)
//                 masked online softmax per row        (registers)
//                 O^T += V_b^T P^T                     (v_mfma 16x16x16 bf16)
//   dst backward: S^T, dP^T = V_b dO_b^T, P = exp(S - LSE), masked
//                 A^T += K_b^T (P*dP)^T, B^T += K_b^T P^T, Delta += rowsum(P*dP)
//   src backward: S = Q_b K_b^T, dP = dO_b V_b^T, dS = P (dP - Delta)
//                 dV^T += dO_b^T P, dK^T += Q_b^T dS
// The transposes are chosen so that every product's output leaves row m of
// the block in lanes l with l % 16 == m, which is the operand layout of the
// next product; K_b / V_b / Q_b / dO_b rows are staged once per tile in LDS
// for all heads of the group. Phase 2 hands the per-row state through LDS to
// the CSR lane geometry and streams the residual (non-tile) edges of the 16
// rows with the same code as the light path, continuing the same state, so
// no cross-kernel merge is needed. The block's own rows that phase 2 needs
// (Q; Q and dO; K and V) are copied to LDS by direct global-to-LDS loads
// issued before the first tile, so phase 2 does not fetch them again. P and
// dS enter the second products as bf16 (rounding 2^-9 relative per term).
//
// Occupancy. The state hand-off buffer overlays the staging rows (it is
// written only after the last tile's products have read them), so a
// workgroup's LDS is the larger of the two, not their sum, plus the own-row
// copy (about 50 KB at most: three workgroups per CU). When the head
// group has fewer heads than the workgroup has waves (the backward passes at
// D = 64 and 128), SPLIT waves share a head, each accumulating its own share
// of the D output columns (the score products are recomputed by each): every
// wave has MFMA work, and each holds 1/SPLIT of the accumulators.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "attn_core.h"

namespace gnn {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

constexpr int kTileWaves = 8;
constexpr int kTileThreads = kTileWaves * kWave;

struct TileArgs {
    const int32_t *blocks;      // tiled row blocks (dst passes) or column blocks (src pass)
    int32_t n_blocks;
    const int32_t *tile_ptr;    // per row block (dst) / column block (src) range
    const int32_t *tile_ids;    // null: identity (dst); ctile (src)
    const int32_t *tile_rc;
    const uint64_t *tile_mask;
    const int32_t *rptr, *ridx; // residual CSR (dst) or transposed residual (src)
};

__device__ __forceinline__ f32x4_t mfma32(const uint4 &a, const uint4 &b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                  c, 0, 0, 0);
}

__device__ __forceinline__ f32x4_t mfma16(const i16x4_t &a, const i16x4_t &b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ i16x4_t pack4(const float (&x)[4]) {
    i16x4_t r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = (short)f32_to_bf16_rne(x[i]);
    return r;
}

__device__ __forceinline__ uint4 ldg16(const void *base, int64_t elem, bool ok) {
    return ok ? *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(base) + elem)
              : make_uint4(0u, 0u, 0u, 0u);
}

// Staged rows are padded by kRowPad elements (16 bytes): consecutive rows then
// start 4 banks apart, so the 16 rows read by a product's 16-byte operand
// loads, and the 4 rows read at once by the strided 16-bit transposed-operand
// reads, fall on different banks (unpadded, 4 rows 8*width bytes apart
// shared their banks); rows stay 16-byte aligned.
constexpr int kRowPad = 8;

// Stage rows r0..r0+15 (head-group columns) of a [N, H*D] bf16 table into
// LDS as [16][stride] (stride = HW*D + kRowPad); rows >= N and heads >= H are zero.
__device__ __forceinline__ void stage_rows(uint16_t *dst, const void *src, int r0, int N, int64_t rowlen, int64_t c0,
                                           int width, int stride, int64_t valid_width) {
    const int nvec = width / 8;
    for (int v = threadIdx.x; v < 16 * nvec; v += kTileThreads) {
        const int r = v / nvec, e = (v % nvec) * 8;
        const bool ok = (r0 + r < N) && (e < valid_width);
        *reinterpret_cast<uint4 *>(dst + r * stride + e) = ldg16(src, (int64_t)(r0 + r) * rowlen + c0 + e, ok);
    }
}

// Copy rows r0..r0+15 (head-group columns) of a [N, H*D] bf16 table into LDS
// as [16][width] (unpadded: only read row-contiguously, one 16-byte slice per
// lane) with direct global-to-LDS loads, which need no registers and complete
// alongside the wave's other loads. Wave w moves the 64-vector chunks w,
// w + 8, ... (16 * width / 8 vectors, a multiple of 64 for width >= 32); lanes
// past the table (rows >= N, heads >= H) load element 0 instead, into slots
// that are never read.
__device__ __forceinline__ void dma_rows(uint16_t *dst, const void *src, int r0, int N, int64_t rowlen, int64_t c0,
                                         int width, int64_t valid_width, int w) {
    const int vpr = width / 8;
    const int nchunk = 16 * vpr / kWave;
    const int lane = lane_id();
    for (int c = w; c < nchunk; c += kTileWaves) {
        const int v = c * kWave + lane;
        const int r = v / vpr, e = (v % vpr) * 8;
        const bool ok = (r0 + r < N) && (e < valid_width);
        const uint16_t *g = reinterpret_cast<const uint16_t *>(src) + (ok ? (int64_t)(r0 + r) * rowlen + c0 + e : 0);
        __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void *)(dst + c * kWave * 8), 16, 0,
                                         0);
    }
}

__device__ __forceinline__ float sum4x(float x) {
    x += xor_lane(x, 16);
    x += xor_lane(x, 32);
    return x;
}

__device__ __forceinline__ float max4x(float x) {
    x = fmaxf(x, xor_lane(x, 16));
    x = fmaxf(x, xor_lane(x, 32));
    return x;
}

// ------------------------------------------------------------------ forward

template <int LH, int D, int HS>
__global__ __launch_bounds__(kTileThreads) void k_tile_fwd(FwdParams P, TileArgs A) {
    constexpr int NV = Vec<bf16_tag>::N;
    constexpr int KC = D / 32, DC = D / 16;
    extern __shared__ float lds[];
    const Geom &G = P.g;
    const int HW = G.HW, N = G.N;
    const int rb = A.blocks[blockIdx.x / G.NHG], hg = blockIdx.x % G.NHG;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), l = lane_id();
    const int64_t rowlen = (int64_t)G.H * D;
    const int width = HW * D, stride = width + kRowPad;
    const int64_t c0 = (int64_t)hg * HW * D;
    const int64_t valid = rowlen - c0;
    // per-row state [16][HW][SW]: acc[D], m, l; SW odd so that the 16 rows a
    // store writes at once fall on different banks (an even SW put HW*SW a
    // multiple of the bank count)
    const int SW = D + 3;
    float *state = lds;                                   // written after the last tile, over the staged rows
    uint16_t *vst = reinterpret_cast<uint16_t *>(lds);   // [16][stride]
    // the block's own Q rows for phase 2, [16][width], past the state / staging
    // region (the staged table takes 8 * stride floats)
    uint16_t *qown = reinterpret_cast<uint16_t *>(lds + std::max(16 * HW * SW, 8 * stride));
    const int row0 = rb * 16;
    const int m = l & 15, q4 = l >> 4;

    float mr[HS], lr[HS];
    f32x4_t acc[HS][DC];
    uint4 qop[HS][KC];
    int hh[HS];
    bool hv[HS];
#pragma unroll
    for (int s = 0; s < HS; ++s) {
        hh[s] = w + kTileWaves * s;
        hv[s] = hh[s] < HW && hg * HW + hh[s] < G.H;
        const int h = hg * HW + hh[s];
#pragma unroll
        for (int kk = 0; kk < KC; ++kk)
            qop[s][kk] = ldg16(P.Q, (int64_t)(row0 + m) * rowlen + (int64_t)h * D + kk * 32 + 8 * q4,
                               hv[s] && row0 + m < N);
        mr[s] = -INFINITY;
        lr[s] = 0.f;
#pragma unroll
        for (int c = 0; c < DC; ++c) acc[s][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    // the tile range is read before the own-row copy is issued, so that waiting
    // for it does not wait for the copy
    const int t0 = A.tile_ptr[rb], t1 = A.tile_ptr[rb + 1];
    dma_rows(qown, P.Q, row0, N, rowlen, c0, width, valid, w);
    for (int t = t0; t < t1; ++t) {
        const int col0 = A.tile_rc[2 * t + 1] * 16;
        stage_rows(vst, P.V, col0, N, rowlen, c0, width, stride, valid);
        __syncthreads();
        const uint64_t word = A.tile_mask[4 * (int64_t)t + (m >> 2)];
#pragma unroll
        for (int s = 0; s < HS; ++s) {
            if (!hv[s]) continue;
            const int h = hg * HW + hh[s];
            f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KC; ++kk) {
                const uint4 kop = ldg16(P.K, (int64_t)(col0 + m) * rowlen + (int64_t)h * D + kk * 32 + 8 * q4,
                                        col0 + m < N);
                sc = mfma32(kop, qop[s][kk], sc);
            }
            // lane l: S[m][n = 4*q4 + i]
            float sv[4];
            float tmax = -INFINITY;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int bit = (m & 3) * 16 + 4 * q4 + i;
                sv[i] = ((word >> bit) & 1ull) ? sc[i] * P.mul : -INFINITY;
                tmax = fmaxf(tmax, sv[i]);
            }
            tmax = max4x(tmax);
            const float mn = fmaxf(mr[s], tmax);
            const float ms = (mn == -INFINITY) ? 0.f : mn;
            const float cf = fast_exp2(mr[s] - ms);
            float p[4], ps = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                p[i] = fast_exp2(sv[i] - ms);
                ps += p[i];
            }
            lr[s] = lr[s] * cf + sum4x(ps);
            mr[s] = mn;
            const i16x4_t pb = pack4(p);
#pragma unroll
            for (int c = 0; c < DC; ++c) {
                i16x4_t va;
#pragma unroll
                for (int i = 0; i < 4; ++i) va[i] = (short)vst[(4 * q4 + i) * stride + hh[s] * D + c * 16 + m];
                acc[s][c] = acc[s][c] * cf;
                acc[s][c] = mfma16(va, pb, acc[s][c]);
            }
        }
        __syncthreads();
    }
#pragma unroll
    for (int s = 0; s < HS; ++s) {
        if (!hv[s]) continue;
        float *row = state + ((int64_t)m * HW + hh[s]) * SW;
#pragma unroll
        for (int c = 0; c < DC; ++c)
#pragma unroll
            for (int i = 0; i < 4; ++i) row[c * 16 + 4 * q4 + i] = acc[s][c][i];
        if (q4 == 0) {
            row[D] = mr[s];
            row[D + 1] = lr[s];
        }
    }
    __syncthreads();
    // phase 2: residual CSR edges of the block's rows, continuing the state
    const LanePos lp = lane_pos<LH, NV>(G, hg);
    FwdParams R = P;
    R.indices = A.ridx;
    for (int r = w; r < 16; r += kTileWaves) {
        const int node = row0 + r;
        if (node >= N) break;
        SoftState<NV> st;
        st.m = -INFINITY;
        st.l = 0.f;
#pragma unroll
        for (int k = 0; k < NV; ++k) st.acc[k] = 0.f;
        if (lp.g == 0 && lp.act) {
            const float *row = state + ((int64_t)r * HW + lp.hh) * SW;
            st.m = row[D];
            st.l = row[D + 1];
#pragma unroll
            for (int k = 0; k < NV; ++k) st.acc[k] = row[lp.dv * NV + k];
        }
        fwd_stream<bf16_tag, LH, M_GT, 4>(R, lp, node, A.rptr[node], A.rptr[node + 1], st, false,
                                          reinterpret_cast<const uint4 *>(qown + r * width + (lp.col - c0)));
        write_out<bf16_tag, NV>(P, lp, node, st);
    }
}

// ----------------------------------------------------- backward, dst pass

// WPE: minimum waves per SIMD the register allocation must allow (1: no constraint)
template <int LH, int D, int HS, int SPLIT, int WPE>
__global__ __launch_bounds__(kTileThreads) __attribute__((amdgpu_waves_per_eu(WPE))) void k_tile_bwd_dst(BwdParams P,
                                                                                                         TileArgs A) {
    constexpr int NV = Vec<bf16_tag>::N;
    constexpr int KC = D / 32, DC = D / 16, DCW = DC / SPLIT;
    extern __shared__ float lds[];
    const Geom &G = P.g;
    const int HW = G.HW, N = G.N;
    const int rb = A.blocks[blockIdx.x / G.NHG], hg = blockIdx.x % G.NHG;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), l = lane_id();
    const int64_t rowlen = (int64_t)G.H * D;
    const int width = HW * D, stride = width + kRowPad;
    const int64_t c0 = (int64_t)hg * HW * D;
    const int64_t valid = rowlen - c0;
    const int SW = 2 * D + 1;
    float *state = lds;                                   // [16][HW][2D+1]: A, B, Delta (after the last tile)
    uint16_t *kst = reinterpret_cast<uint16_t *>(lds);   // [16][stride]
    uint16_t *vst = kst + 16 * stride;
    // the block's own Q and dO rows for phase 2, [16][width] each, past the
    // state / staging region (two staged tables: 16 * stride floats)
    uint16_t *qown = reinterpret_cast<uint16_t *>(lds + std::max(16 * HW * SW, 16 * stride));
    uint16_t *gown = qown + 16 * width;
    const int row0 = rb * 16;
    const int m = l & 15, q4 = l >> 4;
    const int part = w % SPLIT, c0w = part * DCW;        // this wave's output column chunks

    f32x4_t Aa[HS][DCW], Ba[HS][DCW];
    uint4 qop[HS][KC], gop[HS][KC];
    float lse2[HS], dl[HS];
    int hh[HS];
    bool hv[HS];
#pragma unroll
    for (int s = 0; s < HS; ++s) {
        hh[s] = w / SPLIT + (kTileWaves / SPLIT) * s;
        hv[s] = hh[s] < HW && hg * HW + hh[s] < G.H;
        const int h = hg * HW + hh[s];
        const bool ok = hv[s] && row0 + m < N;
#pragma unroll
        for (int kk = 0; kk < KC; ++kk) {
            const int64_t e = (int64_t)(row0 + m) * rowlen + (int64_t)h * D + kk * 32 + 8 * q4;
            qop[s][kk] = ldg16(P.Q, e, ok);
            gop[s][kk] = ldg16(P.dO, e, ok);
        }
        lse2[s] = ok ? P.LSE[(int64_t)(row0 + m) * G.H + h] * kLog2e : 0.f;
        dl[s] = 0.f;
#pragma unroll
        for (int c = 0; c < DCW; ++c) Aa[s][c] = Ba[s][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    const int t0 = A.tile_ptr[rb], t1 = A.tile_ptr[rb + 1];
    dma_rows(qown, P.Q, row0, N, rowlen, c0, width, valid, w);
    dma_rows(gown, P.dO, row0, N, rowlen, c0, width, valid, w);
    for (int t = t0; t < t1; ++t) {
        const int col0 = A.tile_rc[2 * t + 1] * 16;
        stage_rows(kst, P.K, col0, N, rowlen, c0, width, stride, valid);
        stage_rows(vst, P.V, col0, N, rowlen, c0, width, stride, valid);
        __syncthreads();
        const uint64_t word = A.tile_mask[4 * (int64_t)t + (m >> 2)];
#pragma unroll
        for (int s = 0; s < HS; ++s) {
            if (!hv[s]) continue;
            f32x4_t sc = {0.f, 0.f, 0.f, 0.f}, dc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KC; ++kk) {
                const int off = m * stride + hh[s] * D + kk * 32 + 8 * q4;
                sc = mfma32(*reinterpret_cast<const uint4 *>(kst + off), qop[s][kk], sc);
                dc = mfma32(*reinterpret_cast<const uint4 *>(vst + off), gop[s][kk], dc);
            }
            float p[4], pd[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int bit = (m & 3) * 16 + 4 * q4 + i;
                p[i] = ((word >> bit) & 1ull) ? fast_exp2(sc[i] * P.mul - lse2[s]) : 0.f;
                pd[i] = p[i] * dc[i];
                dl[s] += pd[i];
            }
            const i16x4_t pb = pack4(p), pdb = pack4(pd);
#pragma unroll
            for (int c = 0; c < DCW; ++c) {
                i16x4_t ka;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    ka[i] = (short)kst[(4 * q4 + i) * stride + hh[s] * D + (c0w + c) * 16 + m];
                Aa[s][c] = mfma16(ka, pdb, Aa[s][c]);
                Ba[s][c] = mfma16(ka, pb, Ba[s][c]);
            }
        }
        __syncthreads();
    }
#pragma unroll
    for (int s = 0; s < HS; ++s) {
        const float d_row = sum4x(dl[s]);
        if (!hv[s]) continue;
        float *row = state + ((int64_t)m * HW + hh[s]) * SW;
#pragma unroll
        for (int c = 0; c < DCW; ++c)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                row[(c0w + c) * 16 + 4 * q4 + i] = Aa[s][c][i];
                row[D + (c0w + c) * 16 + 4 * q4 + i] = Ba[s][c][i];
            }
        if (q4 == 0 && part == 0) row[2 * D] = d_row;
    }
    __syncthreads();
    const LanePos lp = lane_pos<LH, NV>(G, hg);
    BwdParams R = P;
    R.indices = A.ridx;
    for (int r = w; r < 16; r += kTileWaves) {
        const int node = row0 + r;
        if (node >= N) break;
        float Av[NV], Bv[NV];
        float dsum = 0.f, l2;
#pragma unroll
        for (int k = 0; k < NV; ++k) Av[k] = Bv[k] = 0.f;
        if (lp.g == 0 && lp.act) {
            const float *row = state + ((int64_t)r * HW + lp.hh) * SW;
#pragma unroll
            for (int k = 0; k < NV; ++k) {
                Av[k] = row[lp.dv * NV + k];
                Bv[k] = row[D + lp.dv * NV + k];
            }
            dsum = row[2 * D];
        }
        const int own = r * width + (int)(lp.col - c0);
        bwd_dst_stream<bf16_tag, LH, 2>(R, lp, node, A.rptr[node], A.rptr[node + 1], Av, Bv, dsum, l2, false,
                                        reinterpret_cast<const uint4 *>(qown + own),
                                        reinterpret_cast<const uint4 *>(gown + own));
        if (lp.g == 0 && lp.act) store_dq<bf16_tag, NV>(P, lp, node, Av, Bv, dsum, l2);
    }
}

// ----------------------------------------------------- backward, src pass

template <int LH, int D, int HS, int SPLIT, int WPE>
__global__ __launch_bounds__(kTileThreads) __attribute__((amdgpu_waves_per_eu(WPE))) void k_tile_bwd_src(BwdParams P,
                                                                                                         TileArgs A) {
    constexpr int NV = Vec<bf16_tag>::N;
    constexpr int KC = D / 32, DC = D / 16, DCW = DC / SPLIT;
    extern __shared__ float lds[];
    const Geom &G = P.g;
    const int HW = G.HW, N = G.N;
    const int cb = A.blocks[blockIdx.x / G.NHG], hg = blockIdx.x % G.NHG;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), l = lane_id();
    const int64_t rowlen = (int64_t)G.H * D;
    const int width = HW * D, stride = width + kRowPad;
    const int64_t c0 = (int64_t)hg * HW * D;
    const int64_t valid = rowlen - c0;
    const int SW = 2 * D + 1;                             // odd: see the forward's state
    float *state = lds;                                   // [16][HW][SW]: dK, dV (after the last tile)
    uint16_t *qst = reinterpret_cast<uint16_t *>(lds);   // [16][stride]
    uint16_t *gst = qst + 16 * stride;
    // the block's own K and V rows for phase 2, [16][width] each, past the
    // state / staging region
    uint16_t *kown = reinterpret_cast<uint16_t *>(lds + std::max(16 * HW * SW, 16 * stride));
    uint16_t *vown = kown + 16 * width;
    const int col0 = cb * 16;
    const int n = l & 15, q4 = l >> 4;
    const int part = w % SPLIT, c0w = part * DCW;        // this wave's output column chunks

    f32x4_t dKa[HS][DCW], dVa[HS][DCW];
    uint4 kop[HS][KC], vop[HS][KC];
    int hh[HS];
    bool hv[HS];
#pragma unroll
    for (int s = 0; s < HS; ++s) {
        hh[s] = w / SPLIT + (kTileWaves / SPLIT) * s;
        hv[s] = hh[s] < HW && hg * HW + hh[s] < G.H;
        const int h = hg * HW + hh[s];
        const bool ok = hv[s] && col0 + n < N;
#pragma unroll
        for (int kk = 0; kk < KC; ++kk) {
            const int64_t e = (int64_t)(col0 + n) * rowlen + (int64_t)h * D + kk * 32 + 8 * q4;
            kop[s][kk] = ldg16(P.K, e, ok);
            vop[s][kk] = ldg16(P.V, e, ok);
        }
#pragma unroll
        for (int c = 0; c < DCW; ++c) dKa[s][c] = dVa[s][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    const int x0 = A.tile_ptr[cb], x1 = A.tile_ptr[cb + 1];
    dma_rows(kown, P.K, col0, N, rowlen, c0, width, valid, w);
    dma_rows(vown, P.V, col0, N, rowlen, c0, width, valid, w);
    for (int x = x0; x < x1; ++x) {
        const int t = A.tile_ids[x];
        const int row0 = A.tile_rc[2 * t] * 16;
        stage_rows(qst, P.Q, row0, N, rowlen, c0, width, stride, valid);
        stage_rows(gst, P.dO, row0, N, rowlen, c0, width, stride, valid);
        __syncthreads();
        const uint64_t word = A.tile_mask[4 * (int64_t)t + q4];   // rows 4*q4 .. 4*q4+3
#pragma unroll
        for (int s = 0; s < HS; ++s) {
            if (!hv[s]) continue;
            const int h = hg * HW + hh[s];
            f32x4_t sc = {0.f, 0.f, 0.f, 0.f}, dc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KC; ++kk) {
                const int off = n * stride + hh[s] * D + kk * 32 + 8 * q4;   // row m = l % 16 of Q_b / dO_b
                sc = mfma32(*reinterpret_cast<const uint4 *>(qst + off), kop[s][kk], sc);
                dc = mfma32(*reinterpret_cast<const uint4 *>(gst + off), vop[s][kk], dc);
            }
            // lane l: S[m = 4*q4 + i][n]
            float p[4], ds[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int mrow = 4 * q4 + i;
                const bool on = (word >> (i * 16 + n)) & 1ull;
                float2 stt = make_float2(0.f, 0.f);
                if (on) stt = P.stat[(int64_t)(row0 + mrow) * G.H + h];
                p[i] = on ? fast_exp2(sc[i] * P.mul - stt.x) : 0.f;
                ds[i] = p[i] * (dc[i] - stt.y);
            }
            const i16x4_t pb = pack4(p), dsb = pack4(ds);
#pragma unroll
            for (int c = 0; c < DCW; ++c) {
                i16x4_t ga, qa;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    ga[i] = (short)gst[(4 * q4 + i) * stride + hh[s] * D + (c0w + c) * 16 + n];
                    qa[i] = (short)qst[(4 * q4 + i) * stride + hh[s] * D + (c0w + c) * 16 + n];
                }
                dVa[s][c] = mfma16(ga, pb, dVa[s][c]);
                dKa[s][c] = mfma16(qa, dsb, dKa[s][c]);
            }
        }
        __syncthreads();
    }
#pragma unroll
    for (int s = 0; s < HS; ++s) {
        if (!hv[s]) continue;
        float *row = state + ((int64_t)n * HW + hh[s]) * SW;
#pragma unroll
        for (int c = 0; c < DCW; ++c)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                row[(c0w + c) * 16 + 4 * q4 + i] = dKa[s][c][i];
                row[D + (c0w + c) * 16 + 4 * q4 + i] = dVa[s][c][i];
            }
    }
    __syncthreads();
    const LanePos lp = lane_pos<LH, NV>(G, hg);
    BwdParams R = P;
    R.cindices = A.ridx;
    for (int r = w; r < 16; r += kTileWaves) {
        const int node = col0 + r;
        if (node >= N) break;
        float dk[NV], dv[NV];
#pragma unroll
        for (int k = 0; k < NV; ++k) dk[k] = dv[k] = 0.f;
        if (lp.g == 0 && lp.act) {
            const float *row = state + ((int64_t)r * HW + lp.hh) * SW;
#pragma unroll
            for (int k = 0; k < NV; ++k) {
                dk[k] = row[lp.dv * NV + k];
                dv[k] = row[D + lp.dv * NV + k];
            }
        }
        const int own = r * width + (int)(lp.col - c0);
        bwd_src_stream<bf16_tag, LH, 2>(R, lp, node, A.rptr[node], A.rptr[node + 1], dk, dv, false,
                                        reinterpret_cast<const uint4 *>(kown + own),
                                        reinterpret_cast<const uint4 *>(vown + own));
        if (lp.g != 0 || !lp.act) continue;
        const int64_t off = (int64_t)node * rowlen + lp.col;
        store_scaled<bf16_tag, NV>(P.dK, off, dk, P.scale);
        store_scaled<bf16_tag, NV>(P.dV, off, dv, 1.f);
    }
}

// ------------------------------------------------------------------ host

bool tile_supported(gnn_dtype_t dt, int D) { return dt == GNN_BF16 && (D == 32 || D == 64 || D == 128); }

// LDS of a tile workgroup: the state hand-off buffer overlays the staged rows;
// the own-row copy comes after both
static size_t tile_lds(int kind, int HW, int D) {
    const size_t stage = (size_t)16 * (HW * D + kRowPad) * 2;
    const size_t own = (size_t)16 * HW * D * 2;   // one table of the block's own rows, unpadded
    if (kind == 0) return std::max((size_t)16 * HW * (D + 3) * 4, stage) + own;
    return std::max((size_t)16 * HW * (2 * D + 1) * 4, 2 * stage) + 2 * own;
}

// waves per head in the backward tile kernels: 8 / HW when that divides the
// head's output chunks (D / 16), else 1
static int tile_split(int HW, int D) {
    const int dc = D / 16;
    if (HW * 4 <= kTileWaves && dc % 4 == 0) return 4;
    if (HW * 2 <= kTileWaves && dc % 2 == 0) return 2;
    return 1;
}

// head-group geometry of the tile kernels: as the CSR path, with the head
// group halved until the workgroup's LDS stays within 64 KiB
static Geom tile_geom(const Geom &g0, int kind, int D) {
    Geom g = g0;
    const int LH = D / 8;
    while (g.HW > 1 && tile_lds(kind, g.HW, D) > 65536) g.HW /= 2;
    g.NHG = (g.H + g.HW - 1) / g.HW;
    int sh = 0;
    while ((1 << sh) < g.HW * LH) ++sh;
    g.lr_shift = sh;
    g.G = kWave >> sh;
    return g;
}

template <int D>
static int tile_fwd_d(gnn_plan_t plan, FwdParams P, const TileArgs &A, hipStream_t s) {
    P.g = tile_geom(P.g, 0, D);
    const size_t lds = tile_lds(0, P.g.HW, D);
    const dim3 grid((unsigned)((int64_t)A.n_blocks * P.g.NHG));
    if constexpr (D == 32) {   // only D = 32 allows more heads per group than waves
        if (P.g.HW > kTileWaves)
            return launch(plan, K_TILE_FWD, k_tile_fwd<D / 8, D, 2>, grid, dim3(kTileThreads), lds, s, P, A);
    }
    return launch(plan, K_TILE_FWD, k_tile_fwd<D / 8, D, 1>, grid, dim3(kTileThreads), lds, s, P, A);
}

// Three 8-wave workgroups per CU need 6 waves per SIMD (80 VGPRs). The
// variants that hold at most half a D = 64 head's accumulators per wave fit
// that without spills; the others (two heads per wave at D = 32, a whole
// D = 64 head, D = 128) keep their natural allocation rather than spill.
template <int D, int HS, int SPLIT>
static int launch_tile_bwd(gnn_plan_t plan, const BwdParams &P, const TileArgs &A, int kind, dim3 grid, size_t lds,
                           hipStream_t s) {
    constexpr int WPE = (HS == 1 && D <= 64 && D / SPLIT <= 32) ? 6 : 1;
    if (kind == 1)
        return launch(plan, K_TILE_BWD_DST, k_tile_bwd_dst<D / 8, D, HS, SPLIT, WPE>, grid, dim3(kTileThreads), lds,
                      s, P, A);
    return launch(plan, K_TILE_BWD_SRC, k_tile_bwd_src<D / 8, D, HS, SPLIT, WPE>, grid, dim3(kTileThreads), lds, s,
                  P, A);
}

template <int D>
static int tile_bwd_d(gnn_plan_t plan, BwdParams P, const TileArgs &A, int kind, hipStream_t s) {
    P.g = tile_geom(P.g, kind, D);
    const size_t lds = tile_lds(kind, P.g.HW, D);
    const dim3 grid((unsigned)((int64_t)A.n_blocks * P.g.NHG));
    if constexpr (D == 32) {
        if (P.g.HW > kTileWaves) return launch_tile_bwd<D, 2, 1>(plan, P, A, kind, grid, lds, s);
    }
    const int split = tile_split(P.g.HW, D);
    if constexpr ((D / 16) % 4 == 0) {
        if (split == 4) return launch_tile_bwd<D, 1, 4>(plan, P, A, kind, grid, lds, s);
    }
    if (split == 2) return launch_tile_bwd<D, 1, 2>(plan, P, A, kind, grid, lds, s);
    return launch_tile_bwd<D, 1, 1>(plan, P, A, kind, grid, lds, s);
}

static TileArgs dst_args(gnn_plan_t p) {
    TileArgs A{};
    A.blocks = as<int32_t>(p->trb);
    A.n_blocks = p->n_trb;
    A.tile_ptr = as<int32_t>(p->tile_ptr);
    A.tile_ids = nullptr;
    A.tile_rc = as<int32_t>(p->tile_rc);
    A.tile_mask = as<uint64_t>(p->tile_mask);
    A.rptr = as<int32_t>(p->rindptr);
    A.ridx = as<int32_t>(p->rindices);
    return A;
}

int launch_tile_fwd(gnn_plan_t plan, const FwdParams &P, int D, hipStream_t s) {
    const TileArgs A = dst_args(plan);
    if (A.n_blocks == 0) return GNN_OK;
    switch (D) {
        case 32: return tile_fwd_d<32>(plan, P, A, s);
        case 64: return tile_fwd_d<64>(plan, P, A, s);
        case 128: return tile_fwd_d<128>(plan, P, A, s);
    }
    return GNN_ERR_UNSUPPORTED;
}

int launch_tile_bwd_dst(gnn_plan_t plan, const BwdParams &P, int D, hipStream_t s) {
    const TileArgs A = dst_args(plan);
    if (A.n_blocks == 0) return GNN_OK;
    switch (D) {
        case 32: return tile_bwd_d<32>(plan, P, A, 1, s);
        case 64: return tile_bwd_d<64>(plan, P, A, 1, s);
        case 128: return tile_bwd_d<128>(plan, P, A, 1, s);
    }
    return GNN_ERR_UNSUPPORTED;
}

int launch_tile_bwd_src(gnn_plan_t plan, const BwdParams &P, int D, hipStream_t s) {
    TileArgs A{};
    A.blocks = as<int32_t>(plan->tcb);
    A.n_blocks = plan->n_tcb;
    A.tile_ptr = as<int32_t>(plan->ctile_ptr);
    A.tile_ids = as<int32_t>(plan->ctile);
    A.tile_rc = as<int32_t>(plan->tile_rc);
    A.tile_mask = as<uint64_t>(plan->tile_mask);
    A.rptr = as<int32_t>(plan->rcindptr);
    A.ridx = as<int32_t>(plan->rcindices);
    if (A.n_blocks == 0) return GNN_OK;
    switch (D) {
        case 32: return tile_bwd_d<32>(plan, P, A, 2, s);
        case 64: return tile_bwd_d<64>(plan, P, A, 2, s);
        case 128: return tile_bwd_d<128>(plan, P, A, 2, s);
    }
    return GNN_ERR_UNSUPPORTED;
}

// this file's kernels' index flag (checked builds)
GNN_INDEX_FAULT_READER(index_fault_tile)

}  // namespace gnn
