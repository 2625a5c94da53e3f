// Device-side helpers for gfx950 (CDNA4, 64-lane wavefronts).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gnn {

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ int lane_id() {
    return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

// Cross-lane move through the DPP network (no LDS traffic). CTRL encodings
// (GFX9 DPP): 0xB1 quad_perm[1,0,3,2], 0x4E quad_perm[2,3,0,1],
// 0x141 row_half_mirror, 0x140 row_mirror.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float xor_lane(float x, int off) { return __shfl_xor(x, off, kWave); }

// Sum over aligned groups of G lanes (G a power of two <= 64). Every lane of
// a group receives the same, bitwise identical total (each step adds a
// commutative pair).
template <int G>
__device__ __forceinline__ float group_sum(float x) {
    if constexpr (G >= 2) x += dpp<0xB1>(x);
    if constexpr (G >= 4) x += dpp<0x4E>(x);
    if constexpr (G >= 8) x += dpp<0x141>(x);
    if constexpr (G >= 16) x += dpp<0x140>(x);
    if constexpr (G >= 32) x += xor_lane(x, 16);
    if constexpr (G >= 64) x += xor_lane(x, 32);
    return x;
}

// XCD-aware order of a kernel's row blocks. Workgroups go to the 8 XCDs (each
// with its own L2) round-robin by block id, so consecutive blocks land on
// different L2s. Physical block p (of nb) runs logical block
// ((s / K) * 8 + p % 8) * K + s % K with s = p / 8: each XCD takes runs of
// K = 4 consecutive logical blocks (16 consecutive rows at 4 waves per block),
// so rows that share sources (a community) share one L2, while the runs of
// an XCD stay spread over the whole launch order. Blocks past the last full
// group of 8 K keep their own index; the map is a bijection on [0, nb).
__device__ __forceinline__ int64_t xcd_block(int64_t p, int64_t nb) {
    constexpr int64_t kX = 8, kK = 4;
    const int64_t full = nb / (kX * kK) * (kX * kK);
    if (p >= full) return p;
    const int64_t s = p / kX;
    return ((s / kK) * kX + p % kX) * kK + s % kK;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// --------------------------------------------------------------------------
// 16-byte row vectors: 4 fp32 or 8 bf16 per lane.
// --------------------------------------------------------------------------
struct bf16_tag {};

template <class T>
struct Vec;

template <>
struct Vec<float> {
    static constexpr int N = 4;
    using raw = float4;
    static constexpr int bytes = 4;
    __device__ __forceinline__ static void unpack(const raw &r, float (&o)[N]) {
        o[0] = r.x; o[1] = r.y; o[2] = r.z; o[3] = r.w;
    }
    __device__ __forceinline__ static raw pack(const float (&o)[N]) { return make_float4(o[0], o[1], o[2], o[3]); }
    __device__ __forceinline__ static raw zero() { return make_float4(0.f, 0.f, 0.f, 0.f); }
};

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return 0x7FC0u;  // NaN stays NaN
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

template <>
struct Vec<bf16_tag> {
    static constexpr int N = 8;
    using raw = uint4;
    static constexpr int bytes = 2;
    __device__ __forceinline__ static void unpack(const raw &r, float (&o)[N]) {
        const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            o[2 * k] = __uint_as_float(w[k] << 16);
            o[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
        }
    }
    __device__ __forceinline__ static raw pack(const float (&o)[N]) {
        uint32_t w[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) w[k] = f32_to_bf16_rne(o[2 * k]) | (f32_to_bf16_rne(o[2 * k + 1]) << 16);
        return make_uint4(w[0], w[1], w[2], w[3]);
    }
    __device__ __forceinline__ static raw zero() { return make_uint4(0u, 0u, 0u, 0u); }
};

// acc + <a, b> over one 16-byte vector pair. fp32: four fmas in element
// order. bf16: v_dot2_f32_bf16 on each packed word (the two bf16 products are
// exact in fp32), so the operands are never unpacked.
__device__ __forceinline__ float dot_vec(const float4 &a, const float4 &b, float acc) {
    acc = fmaf(a.x, b.x, acc);
    acc = fmaf(a.y, b.y, acc);
    acc = fmaf(a.z, b.z, acc);
    return fmaf(a.w, b.w, acc);
}

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;

__device__ __forceinline__ float dot_vec(const uint4 &a, const uint4 &b, float acc) {
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.x), __builtin_bit_cast(bf16x2_t, b.x), acc,
                                          false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.y), __builtin_bit_cast(bf16x2_t, b.y), acc,
                                          false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.z), __builtin_bit_cast(bf16x2_t, b.z), acc,
                                          false);
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.w), __builtin_bit_cast(bf16x2_t, b.w), acc,
                                           false);
}

template <class T>
__device__ __forceinline__ typename Vec<T>::raw load_vec(const void *base, int64_t elem_off) {
    using raw = typename Vec<T>::raw;
    return *reinterpret_cast<const raw *>(reinterpret_cast<const char *>(base) + elem_off * Vec<T>::bytes);
}

template <class T>
__device__ __forceinline__ void store_vec(void *base, int64_t elem_off, const typename Vec<T>::raw &v) {
    using raw = typename Vec<T>::raw;
    *reinterpret_cast<raw *>(reinterpret_cast<char *>(base) + elem_off * Vec<T>::bytes) = v;
}

// the same 16-byte store with the non-temporal hint (a streamed output row that
// the kernel does not read back, so it need not displace gathered rows in L2)
template <class T>
__device__ __forceinline__ void store_vec_nt(void *base, int64_t elem_off, const typename Vec<T>::raw &v) {
    typedef unsigned int u4 __attribute__((ext_vector_type(4)));
    static_assert(sizeof(typename Vec<T>::raw) == sizeof(u4), "16-byte vectors");
    u4 x;
    __builtin_memcpy(&x, &v, sizeof(x));
    __builtin_nontemporal_store(x, reinterpret_cast<u4 *>(reinterpret_cast<char *>(base) + elem_off * Vec<T>::bytes));
}

// Checked builds (compiled with GNN_CHECKED): a kernel passes each graph index
// it is about to use as a node-table row through checked_index, which marks an
// index outside [0, n) in this source file's flag and uses row 0 instead, so
// the access stays in bounds; the entry points read and clear the flags and
// return GNN_ERR_BAD_GRAPH. Other builds use the index as it is.
#ifdef GNN_CHECKED
static __device__ int g_index_fault;
#endif

__device__ __forceinline__ int checked_index(int j, int n) {
#ifdef GNN_CHECKED
    if ((unsigned)j >= (unsigned)n) {
        atomicOr(&g_index_fault, 1);
        return 0;
    }
#endif
    return j;
}

// Defines `int NAME(hipStream_t s)` for one source file: in checked builds it
// reads and clears that file's index flag (1: a kernel met a bad index; -1: a
// HIP call failed), in other builds it returns 0.
#ifdef GNN_CHECKED
#define GNN_INDEX_FAULT_READER(NAME)                                                                      \
    int NAME(hipStream_t s) {                                                                             \
        int h = 0;                                                                                        \
        if (hipMemcpyFromSymbolAsync(&h, HIP_SYMBOL(g_index_fault), sizeof(int), 0, hipMemcpyDeviceToHost, \
                                     s) != hipSuccess ||                                                  \
            hipStreamSynchronize(s) != hipSuccess)                                                        \
            return -1;                                                                                    \
        if (h) {                                                                                          \
            const int z = 0;                                                                              \
            if (hipMemcpyToSymbolAsync(HIP_SYMBOL(g_index_fault), &z, sizeof(int), 0, hipMemcpyHostToDevice, \
                                       s) != hipSuccess ||                                                \
                hipStreamSynchronize(s) != hipSuccess)                                                    \
                return -1;                                                                                \
        }                                                                                                 \
        return h;                                                                                         \
    }
#else
#define GNN_INDEX_FAULT_READER(NAME) \
    int NAME(hipStream_t) { return 0; }
#endif

}  // namespace gnn
