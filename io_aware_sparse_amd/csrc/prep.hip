// Graph preprocessing on the device: CSR build, degree bucketing, transposed
// adjacency, and the plan object that caches them.
//
// "On Efficient Scaling of GNNs via IO-Aware Layers Implementations",
// technical summary, Methodology: graph-specific metadata is cached once and
// reused, the transposed adjacency is precomputed for the backward pass, and
// nodes are split into light and heavy sets by a degree threshold, heavy
// neighbour lists being cut into edge chunks.
//
// Everything here is integer work and bit-exact: the LSD radix sort is
// stable, scans are exact, and no result depends on scheduling.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <vector>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "device.h"
#include "internal.h"

namespace gnn {

// ---------------------------------------------------------------- errors

static thread_local char g_hip_msg[256] = "";

void set_hip_error(hipError_t e, const char *what) {
    snprintf(g_hip_msg, sizeof(g_hip_msg), "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

// Test hook: when the environment variable GNN_ALLOC_CAP_BYTES holds a
// non-negative integer, every device allocation of the library larger than it
// fails as out of memory before hipMalloc is called (read at each allocation,
// so a test may set and clear it at run time).
static bool alloc_capped(size_t bytes, long long *cap_out) {
    const char *s = getenv("GNN_ALLOC_CAP_BYTES");
    if (!s || !*s) return false;
    char *end = nullptr;
    const long long cap = strtoll(s, &end, 10);
    if (end == s || *end != '\0' || cap < 0) return false;
    *cap_out = cap;
    return (unsigned long long)bytes > (unsigned long long)cap;
}

int dev_alloc(DevBuf &b, size_t bytes) {
    dev_free(b);
    if (bytes == 0) return GNN_OK;
    long long cap = 0;
    if (alloc_capped(bytes, &cap)) {
        snprintf(g_hip_msg, sizeof(g_hip_msg), "device allocation of %zu bytes refused: above GNN_ALLOC_CAP_BYTES=%lld",
                 bytes, cap);
        return GNN_ERR_OOM;
    }
    void *p = nullptr;
    hipError_t e = hipMalloc(&p, bytes);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        char what[64];
        snprintf(what, sizeof(what), "hipMalloc(%zu bytes)", bytes);
        set_hip_error(e, what);
        return GNN_ERR_OOM;
    }
    b.p = p;
    b.bytes = bytes;
    return GNN_OK;
}

void dev_free(DevBuf &b) {
    if (b.p) (void)hipFree(b.p);
    b.p = nullptr;
    b.bytes = 0;
}

const char *kKernelNames[K_NUM_KINDS] = {
    "gt_fwd_main", "gt_fwd_merge", "gatv2_fwd_main", "gatv2_fwd_merge", "gt_bwd_dst_main",
    "gt_bwd_dst_merge", "gt_bwd_src_main", "gt_bwd_src_merge", "gt_tile_fwd", "gt_tile_bwd_dst", "gt_tile_bwd_src",
    "gatv2_bwd_dst_main", "gatv2_bwd_dst_merge", "gatv2_bwd_src_main", "gatv2_bwd_src_merge", "gatv2_bwd_datt",
    "reduce_fwd_init", "reduce_fwd_main", "reduce_fwd_final", "reduce_bwd_main", "reduce_bwd_merge",
    "spmm_main", "spmm_merge", "spmm_t_main", "spmm_t_merge", "spmm_wsb", "spmm_t_wsb"};

hipEvent_t Timer::get() {
    if (!pool.empty()) {
        hipEvent_t e = pool.back();
        pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

int Timer::begin(int kind, hipStream_t s, TimingRec &r) {
    r.kind = kind;
    r.a = get();
    r.b = get();
    if (!r.a || !r.b) return GNN_ERR_HIP;
    GNN_HIP(hipEventRecord(r.a, s));
    return GNN_OK;
}

int Timer::end(TimingRec &r, hipStream_t s) {
    GNN_HIP(hipEventRecord(r.b, s));
    log.push_back(r);
    return GNN_OK;
}

Timer::~Timer() {
    for (auto &r : log) {
        (void)hipEventDestroy(r.a);
        (void)hipEventDestroy(r.b);
    }
    for (auto e : pool) (void)hipEventDestroy(e);
}

// ---------------------------------------------------------------- scan

constexpr int kScanThreads = 256;
constexpr int kScanItems = 16;
constexpr int kScanTile = kScanThreads * kScanItems;

__device__ __forceinline__ int wave_incl_scan(int v) {
    const int lane = lane_id();
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        int t = __shfl_up(v, off, kWave);
        if (lane >= off) v += t;
    }
    return v;
}

// exclusive scan of one value per thread over the block; *total gets the block sum
__device__ __forceinline__ int block_excl_scan(int v, int *sh, int *total) {
    const int lane = lane_id(), w = threadIdx.x / kWave;
    const int inc = wave_incl_scan(v);
    if (lane == kWave - 1) sh[w] = inc;
    __syncthreads();
    int wofs = 0, tot = 0;
#pragma unroll
    for (int k = 0; k < kScanThreads / kWave; ++k) {
        int c = sh[k];
        wofs += (k < w) ? c : 0;
        tot += c;
    }
    __syncthreads();
    *total = tot;
    return wofs + inc - v;
}

__global__ __launch_bounds__(kScanThreads) void k_scan_tile_sums(const int32_t *in, int64_t n, int32_t *sums) {
    __shared__ int sh[kScanThreads / kWave];
    const int64_t base = (int64_t)blockIdx.x * kScanTile;
    int acc = 0;
#pragma unroll
    for (int k = 0; k < kScanItems; ++k) {
        int64_t i = base + (int64_t)k * kScanThreads + threadIdx.x;
        acc += (i < n) ? in[i] : 0;
    }
    int total;
    (void)block_excl_scan(acc, sh, &total);
    if (threadIdx.x == 0) sums[blockIdx.x] = total;
}

__global__ __launch_bounds__(kScanThreads) void k_scan_apply(const int32_t *in, int32_t *out, int64_t n,
                                                             const int32_t *tile_ofs, int32_t *total_dev) {
    __shared__ int tile[kScanTile];
    __shared__ int sh[kScanThreads / kWave];
    const int64_t base = (int64_t)blockIdx.x * kScanTile;
#pragma unroll
    for (int k = 0; k < kScanItems; ++k) {
        int64_t i = base + (int64_t)k * kScanThreads + threadIdx.x;
        tile[k * kScanThreads + threadIdx.x] = (i < n) ? in[i] : 0;
    }
    __syncthreads();
    int loc[kScanItems];
    int run = 0;
#pragma unroll
    for (int k = 0; k < kScanItems; ++k) {
        loc[k] = run;
        run += tile[threadIdx.x * kScanItems + k];
    }
    int total;
    const int tofs = block_excl_scan(run, sh, &total);
    const int bofs = tile_ofs ? tile_ofs[blockIdx.x] : 0;
#pragma unroll
    for (int k = 0; k < kScanItems; ++k) tile[threadIdx.x * kScanItems + k] = bofs + tofs + loc[k];
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kScanItems; ++k) {
        int64_t i = base + (int64_t)k * kScanThreads + threadIdx.x;
        if (i < n) out[i] = tile[k * kScanThreads + threadIdx.x];
    }
    if (total_dev && !tile_ofs && threadIdx.x == 0) *total_dev = total;
}

__global__ void k_set_i32(int32_t *p, int32_t v) { *p = v; }

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// int32 elements of scratch that scan_exclusive(n) needs
int64_t scan_scratch(int64_t n) {
    int64_t tot = 0;
    while (n > kScanTile) {
        n = cdiv(n, kScanTile);
        tot += n;
    }
    return tot + 1;
}

int scan_rec(const int32_t *in, int32_t *out, int64_t n, int32_t *total_dev, int32_t *scratch,
             hipStream_t s) {
    if (n <= 0) {
        if (total_dev) hipLaunchKernelGGL(k_set_i32, dim3(1), dim3(1), 0, s, total_dev, 0);
        return GNN_OK;
    }
    const int64_t nb = cdiv(n, kScanTile);
    if (nb == 1) {
        hipLaunchKernelGGL(k_scan_apply, dim3(1), dim3(kScanThreads), 0, s, in, out, n, (const int32_t *)nullptr,
                           total_dev);
        return GNN_OK;
    }
    int32_t *sums = scratch;
    hipLaunchKernelGGL(k_scan_tile_sums, dim3((unsigned)nb), dim3(kScanThreads), 0, s, in, n, sums);
    GNN_TRY(scan_rec(sums, sums, nb, total_dev, scratch + nb, s));
    hipLaunchKernelGGL(k_scan_apply, dim3((unsigned)nb), dim3(kScanThreads), 0, s, in, out, n,
                       (const int32_t *)sums, (int32_t *)nullptr);
    return GNN_OK;
}

// ---------------------------------------------------------------- radix sort

constexpr int kSortThreads = 256;
constexpr int kSortItems = 16;
constexpr int kSortTile = kSortThreads * kSortItems;

__global__ __launch_bounds__(kSortThreads) void k_rs_hist(const uint64_t *keys, int64_t n, int shift,
                                                           int32_t *hist, int nblocks) {
    __shared__ int cnt[256];
    cnt[threadIdx.x] = 0;
    __syncthreads();
    const int64_t base = (int64_t)blockIdx.x * kSortTile;
#pragma unroll 4
    for (int k = 0; k < kSortItems; ++k) {
        int64_t i = base + (int64_t)k * kSortThreads + threadIdx.x;
        if (i < n) atomicAdd(&cnt[(int)((keys[i] >> shift) & 0xFF)], 1);
    }
    __syncthreads();
    hist[(int64_t)threadIdx.x * nblocks + blockIdx.x] = cnt[threadIdx.x];
}

// Stable scatter: element order inside a tile is (sub-tile, thread), and the
// ranking below preserves it, so equal digits keep their input order.
__global__ __launch_bounds__(kSortThreads) void k_rs_scatter(const uint64_t *in, uint64_t *out, int64_t n,
                                                              int shift, const int32_t *ofs, int nblocks,
                                                              const int32_t *vin, int32_t *vout) {
    constexpr int NW = kSortThreads / kWave;
    __shared__ int base[256];
    __shared__ int wcnt[NW][256];
    const int t = threadIdx.x, w = t / kWave, lane = lane_id();
    base[t] = ofs[(int64_t)t * nblocks + blockIdx.x];
    const uint64_t lt = (lane == 0) ? 0ull : ((~0ull) >> (64 - lane));
    const int64_t tile0 = (int64_t)blockIdx.x * kSortTile;
    for (int it = 0; it < kSortItems; ++it) {
#pragma unroll
        for (int k = 0; k < NW; ++k) wcnt[k][t] = 0;
        __syncthreads();
        const int64_t i = tile0 + (int64_t)it * kSortThreads + t;
        const bool valid = i < n;
        const uint64_t key = valid ? in[i] : 0ull;
        const int d = (int)((key >> shift) & 0xFF);
        uint64_t m = __ballot(valid);
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            const bool bit = (d >> b) & 1;
            const uint64_t bb = __ballot(bit);
            m &= bit ? bb : ~bb;
        }
        const int rank = __popcll(m & lt);
        if (valid && rank == 0) wcnt[w][d] = __popcll(m);
        __syncthreads();
        int run = 0;
#pragma unroll
        for (int k = 0; k < NW; ++k) {
            int c = wcnt[k][t];
            wcnt[k][t] = run;
            run += c;
        }
        __syncthreads();
        if (valid) {
            const int64_t dst = base[d] + wcnt[w][d] + rank;
            out[dst] = key;
            if (vin) vout[dst] = vin[i];
        }
        __syncthreads();
        base[t] += run;
        __syncthreads();
    }
}

int64_t sort_scratch(int64_t n) {
    const int64_t nb = std::max<int64_t>(1, cdiv(n, kSortTile));
    return 256 * nb + scan_scratch(256 * nb) + 1;
}

// Stable LSD radix sort of keys on bits [0, bits); optional int32 payload
// (vals, with vtmp as its scratch twin) moves with its key.
int radix_sort(uint64_t *keys, uint64_t *tmp, int64_t n, int bits, int32_t *scratch, hipStream_t s,
               int32_t *vals, int32_t *vtmp) {
    if (n <= 1 || bits <= 0) return GNN_OK;
    const int64_t nb = cdiv(n, kSortTile);
    if (nb > 0x7FFFFFFF / 256) return GNN_ERR_INVALID_ARG;
    int32_t *hist = scratch;
    int32_t *tot = scratch + 256 * nb;
    int32_t *sc = tot + 1;
    uint64_t *a = keys, *b = tmp;
    int32_t *va = vals, *vb = vtmp;
    const int passes = (bits + 7) / 8;
    for (int p = 0; p < passes; ++p) {
        hipLaunchKernelGGL(k_rs_hist, dim3((unsigned)nb), dim3(kSortThreads), 0, s, a, n, 8 * p, hist, (int)nb);
        GNN_TRY(scan_rec(hist, hist, 256 * nb, tot, sc, s));
        hipLaunchKernelGGL(k_rs_scatter, dim3((unsigned)nb), dim3(kSortThreads), 0, s, a, b, n, 8 * p,
                           (const int32_t *)hist, (int)nb, (const int32_t *)va, vb);
        std::swap(a, b);
        std::swap(va, vb);
    }
    if (a != keys) {
        GNN_HIP(hipMemcpyAsync(keys, a, (size_t)n * 8, hipMemcpyDeviceToDevice, s));
        if (vals) GNN_HIP(hipMemcpyAsync(vals, va, (size_t)n * 4, hipMemcpyDeviceToDevice, s));
    }
    GNN_HIP(hipGetLastError());
    return GNN_OK;
}

// ---------------------------------------------------------------- CSR / CSC

int bits_for(int64_t n) {
    int b = 1;
    while (b < 31 && (1ll << b) < n) ++b;
    return b;
}

__global__ void k_coo_keys(const int32_t *src, const int32_t *dst, int64_t m, int32_t n_nodes, int nb,
                           int add_self, uint64_t *keys, int32_t *err) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < m) {
        const int32_t a = src[i], b = dst[i];
        if (a < 0 || a >= n_nodes || b < 0 || b >= n_nodes) {
            *err = 1;
            keys[i] = 0;
        } else {
            keys[i] = ((uint64_t)(uint32_t)b << nb) | (uint32_t)a;
        }
    } else if (add_self && i < m + n_nodes) {
        const uint64_t v = (uint64_t)(i - m);
        keys[i] = (v << nb) | v;
    }
}

__global__ void k_flags(const uint64_t *k, int64_t n, int dedupe, int32_t *f) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) f[i] = (!dedupe || i == 0 || k[i] != k[i - 1]) ? 1 : 0;
}

// sorted keys (row << nb | col) -> rowptr/colidx; pos = exclusive scan of flags
__global__ void k_emit(const uint64_t *k, int64_t n, const int32_t *f, const int32_t *pos, int nb,
                       int32_t *rowptr, int32_t *col, int64_t cap, int32_t n_rows) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const uint64_t mask = (1ull << nb) - 1ull;
    const uint64_t key = k[i];
    const int64_t r = (int64_t)(key >> nb);
    const int32_t p = pos[i];
    if (f[i] && p < cap) col[p] = (int32_t)(key & mask);
    const int64_t rprev = (i == 0) ? -1 : (int64_t)(k[i - 1] >> nb);
    for (int64_t q = rprev + 1; q <= r; ++q) rowptr[q] = p;
    if (i == n - 1) {
        const int32_t total = p + f[i];
        for (int64_t q = r + 1; q <= n_rows; ++q) rowptr[q] = total;
    }
}

__global__ void k_fill_i32(int32_t *p, int64_t n, int32_t v) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}

dim3 grid1d(int64_t n, int t) { return dim3((unsigned)std::max<int64_t>(1, cdiv(n, t))); }

// keys must hold the sorted (row << nb | col) keys; writes rowptr [n_rows+1], col [<= cap]
int emit_structure(uint64_t *keys, int64_t n, int nb, int dedupe, int32_t n_rows, int32_t *rowptr,
                          int32_t *col, int64_t cap, int32_t *flags, int32_t *pos, int32_t *total_dev,
                          int32_t *scratch, hipStream_t s) {
    if (n == 0) {
        hipLaunchKernelGGL(k_fill_i32, grid1d(n_rows + 1), dim3(256), 0, s, rowptr, (int64_t)n_rows + 1, 0);
        hipLaunchKernelGGL(k_set_i32, dim3(1), dim3(1), 0, s, total_dev, 0);
        return GNN_OK;
    }
    hipLaunchKernelGGL(k_flags, grid1d(n), dim3(256), 0, s, keys, n, dedupe, flags);
    GNN_TRY(scan_rec(flags, pos, n, total_dev, scratch, s));
    hipLaunchKernelGGL(k_emit, grid1d(n), dim3(256), 0, s, keys, n, flags, pos, nb, rowptr, col, cap, n_rows);
    GNN_HIP(hipGetLastError());
    return GNN_OK;
}

// per-edge keys (col << nb | row) of the transpose, one wave per CSR row
__global__ void k_transpose_keys(const int32_t *indptr, const int32_t *indices, int32_t n, int nb,
                                 uint64_t *keys) {
    const int row = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    if (row >= n) return;
    const int lane = lane_id();
    const int32_t e0 = indptr[row], e1 = indptr[row + 1];
    for (int32_t e = e0 + lane; e < e1; e += kWave)
        keys[e] = ((uint64_t)(uint32_t)indices[e] << nb) | (uint32_t)row;
}

// ---------------------------------------------------------------- buckets

// n_long (zeroed beforehand) counts the light rows of more than kLongRow
// entries: one atomic add per wave
__global__ void k_bucket_flags(const int32_t *indptr, int32_t n, int32_t T, int64_t span, int32_t *fl,
                               int32_t *fh, int32_t *ng, int32_t *n_long) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    bool is_long = false;
    if (i < n) {
        const int64_t deg = (int64_t)indptr[i + 1] - indptr[i];
        const bool heavy = deg > T;
        fl[i] = heavy ? 0 : 1;
        fh[i] = heavy ? 1 : 0;
        ng[i] = heavy ? (int32_t)((deg + span - 1) / span) : 0;
        is_long = !heavy && deg > kLongRow;
    }
    const uint64_t m = __ballot(is_long);
    if (m && lane_id() == 0) atomicAdd(n_long, (int32_t)__popcll(m));
}

__global__ void k_bucket_emit(const int32_t *indptr, int32_t n, int32_t T, int64_t span, const int32_t *lpos,
                              const int32_t *hpos, const int32_t *gofs, int32_t *light, int32_t *heavy,
                              int32_t *partial_ofs, int32_t *groups) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const int32_t e0 = indptr[i], e1 = indptr[i + 1];
    if ((int64_t)e1 - e0 <= T) {
        light[lpos[i]] = (int32_t)i;
        return;
    }
    const int32_t k = hpos[i];
    heavy[k] = (int32_t)i;
    partial_ofs[k] = gofs[i];
    int32_t g = gofs[i];
    for (int64_t e = e0; e < e1; e += span, ++g) {
        groups[3 * (int64_t)g + 0] = (int32_t)i;
        groups[3 * (int64_t)g + 1] = (int32_t)e;
        groups[3 * (int64_t)g + 2] = (int32_t)std::min<int64_t>(e + span, e1);
    }
}

// order 1: descending degree; order 2: nodes of degree > hoist first, by
// descending floor(log2(degree)), everything else after; ties by ascending id
__global__ void k_sched_keys(const int32_t *indptr, const int32_t *light, int32_t n_light, int64_t cap,
                             int32_t order, int64_t hoist, uint64_t *keys) {
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k >= n_light) return;
    const int32_t v = light[k];
    const int64_t deg = (int64_t)indptr[v + 1] - indptr[v];
    uint64_t hi;
    if (order == 1) {
        hi = (uint64_t)(cap - deg);
    } else if (order == 3) {
        hi = (uint64_t)(cap - (deg + 3) / 4);      // descending 4-edge steps
    } else {
        int b = 0;
        while (b < 62 && (2ll << b) <= deg) ++b;   // floor(log2(deg)) for deg >= 1
        hi = deg > hoist ? (uint64_t)(63 - b) : 64ull;
    }
    keys[k] = (hi << 32) | (uint32_t)v;
}

__global__ void k_low32_i32(const uint64_t *keys, int64_t n, int32_t *out) {
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k < n) out[k] = (int32_t)(keys[k] & 0xFFFFFFFFull);
}

// light launch order (see k_sched_keys); order 0 keeps the light list
static int build_sched(const int32_t *indptr, int32_t T, int64_t max_deg, int32_t sched_order, Buckets &b,
                       DevBuf &dst, hipStream_t s) {
    GNN_TRY(dev_alloc(dst, (size_t)std::max(1, b.n_light) * 4));
    if (b.n_light == 0) return GNN_OK;
    if (!sched_order) {
        GNN_HIP(hipMemcpyAsync(dst.p, b.light.p, (size_t)b.n_light * 4, hipMemcpyDeviceToDevice, s));
        return GNN_OK;
    }
    const int64_t cap = std::min<int64_t>(T, max_deg);
    const int64_t m = b.n_light;
    const int64_t ss = sort_scratch(m) + 2;
    DevBuf tmp;
    GNN_TRY(dev_alloc(tmp, (size_t)(16 * m + 4 * ss + 64)));
    uint64_t *keys = as<uint64_t>(tmp), *kt = keys + m;
    int32_t *scr = reinterpret_cast<int32_t *>(kt + m);
    const int64_t hoist = std::max<int64_t>(1, T / 4);
    hipLaunchKernelGGL(k_sched_keys, grid1d(m), dim3(256), 0, s, indptr, as<int32_t>(b.light), b.n_light, cap,
                       sched_order, hoist, keys);
    int rc = radix_sort(keys, kt, m, 32 + (sched_order == 1 || sched_order == 3 ? bits_for(cap + 2) : 7), scr, s);
    if (rc == GNN_OK) {
        hipLaunchKernelGGL(k_low32_i32, grid1d(m), dim3(256), 0, s, keys, m, as<int32_t>(dst));
        if (hipStreamSynchronize(s) != hipSuccess) {
            set_hip_error(hipGetLastError(), "light schedule");
            rc = GNN_ERR_HIP;
        }
    }
    dev_free(tmp);
    return rc;
}

int build_buckets(const int32_t *indptr, int32_t n, int32_t T, int32_t C, int32_t W, int32_t sched_order,
                  Buckets &b, hipStream_t s, bool by_degree) {
    const int64_t span = (int64_t)C * W;
    DevBuf tmp;
    const int64_t sc = scan_scratch(n);
    GNN_TRY(dev_alloc(tmp, (size_t)(6 * (int64_t)n + 4 + sc) * 4));
    int32_t *fl = as<int32_t>(tmp), *fh = fl + n, *ng = fh + n, *lpos = ng + n, *hpos = lpos + n,
            *gofs = hpos + n, *tot = gofs + n, *scr = tot + 4;
    int rc = GNN_OK;
    int32_t h_tot[4] = {0, 0, 0, 0};
    if (n > 0) {
        hipLaunchKernelGGL(k_set_i32, dim3(1), dim3(1), 0, s, tot + 3, 0);
        hipLaunchKernelGGL(k_bucket_flags, grid1d(n), dim3(256), 0, s, indptr, n, T, span, fl, fh, ng, tot + 3);
        if ((rc = scan_rec(fl, lpos, n, tot + 0, scr, s)) != GNN_OK) goto done;
        if ((rc = scan_rec(fh, hpos, n, tot + 1, scr, s)) != GNN_OK) goto done;
        if ((rc = scan_rec(ng, gofs, n, tot + 2, scr, s)) != GNN_OK) goto done;
        if (hipMemcpyAsync(h_tot, tot, sizeof(h_tot), hipMemcpyDeviceToHost, s) != hipSuccess ||
            hipStreamSynchronize(s) != hipSuccess) {
            set_hip_error(hipGetLastError(), "bucket counts");
            rc = GNN_ERR_HIP;
            goto done;
        }
    }
    b.n_light = h_tot[0];
    b.n_heavy = h_tot[1];
    b.n_groups = h_tot[2];
    b.n_long = h_tot[3];
    if ((rc = dev_alloc(b.light, (size_t)std::max(1, b.n_light) * 4)) != GNN_OK) goto done;
    if ((rc = dev_alloc(b.heavy, (size_t)std::max(1, b.n_heavy) * 4)) != GNN_OK) goto done;
    if ((rc = dev_alloc(b.partial_ofs, (size_t)(b.n_heavy + 1) * 4)) != GNN_OK) goto done;
    if ((rc = dev_alloc(b.groups, (size_t)std::max(1, b.n_groups) * 12)) != GNN_OK) goto done;
    if (n > 0)
        hipLaunchKernelGGL(k_bucket_emit, grid1d(n), dim3(256), 0, s, indptr, n, T, span, lpos, hpos, gofs,
                           as<int32_t>(b.light), as<int32_t>(b.heavy), as<int32_t>(b.partial_ofs),
                           as<int32_t>(b.groups));
    hipLaunchKernelGGL(k_set_i32, dim3(1), dim3(1), 0, s, as<int32_t>(b.partial_ofs) + b.n_heavy, b.n_groups);
    if (hipStreamSynchronize(s) != hipSuccess || hipGetLastError() != hipSuccess) {
        set_hip_error(hipErrorUnknown, "bucket emit");
        rc = GNN_ERR_HIP;
        goto done;
    }
    {
        int32_t ends[2] = {0, 0};
        if (n > 0 && (hipMemcpy(&ends[0], indptr, 4, hipMemcpyDeviceToHost) != hipSuccess ||
                      hipMemcpy(&ends[1], indptr + n, 4, hipMemcpyDeviceToHost) != hipSuccess)) {
            set_hip_error(hipGetLastError(), "bucket schedule");
            rc = GNN_ERR_HIP;
            goto done;
        }
        rc = build_sched(indptr, T, (int64_t)ends[1] - ends[0], sched_order, b, b.sched, s);
        // the packed launches' order: descending ceil(degree / 4), ties by ascending id
        // (order 3). Rows packed into one wave then need the same number of
        // 4- (and 8-) edge steps, and rows of one class keep their id order,
        // so rows that share sources (a community) stay next to each other.
        if (rc == GNN_OK && by_degree)
            rc = build_sched(indptr, T, (int64_t)ends[1] - ends[0], 3, b, b.by_degree, s);
    }
done:
    dev_free(tmp);
    return rc;
}

__global__ void k_validate(const int32_t *indptr, const int32_t *indices, int32_t n, int64_t e, int32_t *err) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i == 0 && (indptr[0] != 0 || (int64_t)indptr[n] != e)) *err = 1;
    if (i < n && indptr[i] > indptr[i + 1]) *err = 1;
    if (i < e) {
        const int32_t v = indices[i];
        if (v < 0 || v >= n) *err = 1;
    }
}

// sortedness of the rows: mark row starts, then look for a descending pair inside a row
__global__ void k_row_starts(const int32_t *indptr, int32_t n, uint8_t *start) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n && indptr[i + 1] > indptr[i]) start[indptr[i]] = 1;
}

__global__ void k_fill_u8(uint8_t *p, int64_t n, uint8_t v) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}

__global__ void k_unsorted(const int32_t *indices, int64_t e, const uint8_t *start, int32_t *flag) {
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k > 0 && k < e && !start[k] && indices[k - 1] > indices[k]) *flag = 1;
}

static int check_rows_sorted(const int32_t *indptr, const int32_t *indices, int32_t n, int64_t e, hipStream_t s,
                             bool *sorted) {
    *sorted = true;
    if (e < 2) return GNN_OK;
    DevBuf tmp;
    GNN_TRY(dev_alloc(tmp, (size_t)e + 64));
    int32_t *flag = reinterpret_cast<int32_t *>(tmp.p);
    uint8_t *start = reinterpret_cast<uint8_t *>(tmp.p) + 64;
    hipLaunchKernelGGL(k_set_i32, dim3(1), dim3(1), 0, s, flag, 0);
    hipLaunchKernelGGL(k_fill_u8, grid1d(e), dim3(256), 0, s, start, e, (uint8_t)0);
    hipLaunchKernelGGL(k_row_starts, grid1d(n), dim3(256), 0, s, indptr, n, start);
    hipLaunchKernelGGL(k_unsorted, grid1d(e), dim3(256), 0, s, indices, e, start, flag);
    int32_t h = 0;
    int rc = GNN_OK;
    if (hipMemcpyAsync(&h, flag, 4, hipMemcpyDeviceToHost, s) != hipSuccess || hipStreamSynchronize(s) != hipSuccess) {
        set_hip_error(hipGetLastError(), "gnn_plan_create sortedness");
        rc = GNN_ERR_HIP;
    }
    dev_free(tmp);
    *sorted = h == 0;
    return rc;
}

// pos[9k + b]: the first entry of heavy row k whose source is >= b * R (b = 0..7),
// pos[9k + 8] the row's end (the row's sources ascend)
__global__ void k_range_bounds(const int32_t *indptr, const int32_t *indices, const int32_t *heavy, int32_t n_heavy,
                               int32_t R, int32_t *pos) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= (int64_t)n_heavy * 9) return;
    const int32_t k = (int32_t)(t / 9), b = (int32_t)(t % 9);
    const int32_t node = heavy[k];
    int32_t lo = indptr[node], hi = indptr[node + 1];
    if (b == 8) {
        pos[t] = hi;
        return;
    }
    const int64_t key = (int64_t)b * R;
    while (lo < hi) {
        const int32_t mid = lo + (hi - lo) / 2;
        if (indices[mid] < key) lo = mid + 1;
        else hi = mid;
    }
    pos[t] = lo;
}

// The XSplit structure of a plan (see internal.h); nothing when there are no
// heavy rows or the rows are not sorted.
static int build_xsplit(gnn_plan_s *p, hipStream_t s) {
    const Buckets &b = p->fwd;
    XSplit &x = p->xsplit;
    if (b.n_heavy == 0 || !p->rows_sorted) return GNN_OK;
    const int32_t R = (int32_t)((p->n_nodes + 7) / 8);
    const int64_t span = p->opts.chunk;
    DevBuf pos;
    GNN_TRY(dev_alloc(pos, (size_t)b.n_heavy * 9 * 4));
    hipLaunchKernelGGL(k_range_bounds, grid1d((int64_t)b.n_heavy * 9), dim3(256), 0, s, p->indptr, p->indices,
                       as<int32_t>(b.heavy), b.n_heavy, R, as<int32_t>(pos));
    std::vector<int32_t> hpos((size_t)b.n_heavy * 9), hheavy((size_t)b.n_heavy);
    if (hipMemcpyAsync(hpos.data(), pos.p, hpos.size() * 4, hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipMemcpyAsync(hheavy.data(), b.heavy.p, hheavy.size() * 4, hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess) {
        set_hip_error(hipGetLastError(), "source-range split");
        dev_free(pos);
        return GNN_ERR_HIP;
    }
    dev_free(pos);
    std::vector<int32_t> groups, pofs((size_t)b.n_heavy + 1), lists[8];
    int32_t ng = 0;
    for (int32_t k = 0; k < b.n_heavy; ++k) {
        pofs[k] = ng;
        for (int r = 0; r < 8; ++r) {
            const int64_t a = hpos[(size_t)k * 9 + r], len = hpos[(size_t)k * 9 + r + 1] - a;
            if (len <= 0) continue;
            const int64_t cnt = (len + span - 1) / span;
            for (int64_t j = 0; j < cnt; ++j) {
                groups.push_back(hheavy[k]);
                groups.push_back((int32_t)(a + len * j / cnt));
                groups.push_back((int32_t)(a + len * (j + 1) / cnt));
                lists[r].push_back(ng++);
            }
        }
    }
    pofs[b.n_heavy] = ng;
    size_t most = 0;
    for (const auto &l : lists) most = std::max(most, l.size());
    std::vector<int32_t> order(8 * most, -1);
    for (int r = 0; r < 8; ++r)
        for (size_t i = 0; i < lists[r].size(); ++i) order[i * 8 + r] = lists[r][i];
    GNN_TRY(dev_alloc(x.groups, std::max<size_t>(groups.size(), 1) * 4));
    GNN_TRY(dev_alloc(x.partial_ofs, pofs.size() * 4));
    GNN_TRY(dev_alloc(x.order, std::max<size_t>(order.size(), 1) * 4));
    GNN_HIP(hipMemcpyAsync(x.groups.p, groups.data(), groups.size() * 4, hipMemcpyHostToDevice, s));
    GNN_HIP(hipMemcpyAsync(x.partial_ofs.p, pofs.data(), pofs.size() * 4, hipMemcpyHostToDevice, s));
    GNN_HIP(hipMemcpyAsync(x.order.p, order.data(), order.size() * 4, hipMemcpyHostToDevice, s));
    GNN_HIP(hipStreamSynchronize(s));
    x.n_groups = ng;
    x.n_slots = (int32_t)order.size();
    return GNN_OK;
}

int validate_csr(const int32_t *indptr, const int32_t *indices, int32_t n, int64_t e, hipStream_t s) {
    DevBuf tmp;
    GNN_TRY(dev_alloc(tmp, 64));
    int32_t *err = as<int32_t>(tmp);
    int32_t herr = 0;
    int rc = GNN_OK;
    hipLaunchKernelGGL(k_set_i32, dim3(1), dim3(1), 0, s, err, 0);
    hipLaunchKernelGGL(k_validate, grid1d(std::max<int64_t>(n, e) + 1), dim3(256), 0, s, indptr, indices, n, e, err);
    if (hipMemcpyAsync(&herr, err, 4, hipMemcpyDeviceToHost, s) != hipSuccess || hipStreamSynchronize(s) != hipSuccess) {
        set_hip_error(hipGetLastError(), "graph validation");
        rc = GNN_ERR_HIP;
    } else if (herr) {
        rc = GNN_ERR_BAD_GRAPH;
    }
    dev_free(tmp);
    return rc;
}

int build_transpose(const int32_t *indptr, const int32_t *indices, int32_t n, int64_t m, DevBuf &cindptr,
                    DevBuf &cindices, hipStream_t s) {
    const int nb = bits_for(std::max<int64_t>(2, n));
    const int64_t ss = std::max(sort_scratch(m), scan_scratch(m)) + 2;
    DevBuf tmp;
    int rc = dev_alloc(tmp, (size_t)(24 * std::max<int64_t>(m, 1) + 4 * ss + 64));
    if (rc == GNN_OK) rc = dev_alloc(cindptr, (size_t)(n + 1) * 4);
    if (rc == GNN_OK) rc = dev_alloc(cindices, (size_t)std::max<int64_t>(m, 1) * 4);
    if (rc == GNN_OK) {
        uint64_t *keys = as<uint64_t>(tmp), *kt = keys + std::max<int64_t>(m, 1);
        int32_t *flags = reinterpret_cast<int32_t *>(kt + std::max<int64_t>(m, 1));
        int32_t *pos = flags + std::max<int64_t>(m, 1), *total = pos + std::max<int64_t>(m, 1), *scr = total + 1;
        if (n > 0)
            hipLaunchKernelGGL(k_transpose_keys, dim3((unsigned)cdiv(n, 4)), dim3(256), 0, s, indptr, indices, n, nb,
                               keys);
        rc = radix_sort(keys, kt, m, 2 * nb, scr, s);
        if (rc == GNN_OK)
            rc = emit_structure(keys, m, nb, 0, n, as<int32_t>(cindptr), as<int32_t>(cindices), m, flags, pos, total,
                                scr, s);
        if (rc == GNN_OK && hipStreamSynchronize(s) != hipSuccess) {
            set_hip_error(hipGetLastError(), "transpose");
            rc = GNN_ERR_HIP;
        }
    }
    dev_free(tmp);
    return rc;
}

}  // namespace gnn

using namespace gnn;

std::vector<DevBuf *> gnn_plan_s::structures() {
    return {&fwd.light, &fwd.heavy, &fwd.groups, &fwd.partial_ofs, &fwd.sched, &fwd.by_degree, &xsplit.groups,
            &xsplit.partial_ofs, &xsplit.order, &cindptr, &cindices,
            &bwd.light, &bwd.heavy, &bwd.groups, &bwd.partial_ofs, &bwd.sched, &bwd.by_degree, &tile_rc, &tile_mask,
            &tile_ptr, &trb, &rindptr, &rindices, &light_nt, &ctile, &ctile_ptr, &tcb, &rcindptr, &rcindices,
            &c_light_nt, &spmm_w, &spmm_cw, &spmm_rng, &spmm_crng, &spmm_rw, &spmm_rcw};
}

int64_t gnn_plan_s::structure_bytes() {
    int64_t t = 0;
    for (const DevBuf *b : structures()) t += (int64_t)b->bytes;
    return t;
}

namespace gnn {
int take_index_faults(hipStream_t s) {
    int bad = 0;
    for (auto f : {index_fault_attn, index_fault_gat, index_fault_tile, index_fault_reduce, index_fault_spmm}) {
        const int r = f(s);
        if (r < 0) {
            set_hip_error(hipGetLastError(), "index check");
            return GNN_ERR_HIP;
        }
        bad |= r;
    }
    if (bad) return GNN_ERR_BAD_GRAPH;
    return GNN_OK;
}

int plan_workspace(gnn_plan_s *p, size_t bytes, hipStream_t s, void **out) {
    if (bytes <= p->ws.bytes) {
        *out = p->ws.p;
        return GNN_OK;
    }
    // the old buffer may still be in use by work queued on the stream
    GNN_HIP(hipStreamSynchronize(s));
    GNN_TRY(dev_alloc(p->ws, bytes));
    p->largest_ws = std::max<int64_t>(p->largest_ws, (int64_t)bytes);
    *out = p->ws.p;
    return GNN_OK;
}
}  // namespace gnn

// ======================================================================= ABI

extern "C" {

const char *gnn_status_string(int status) {
    switch (status) {
        case GNN_OK: return "ok";
        case GNN_ERR_INVALID_ARG: return "invalid argument";
        case GNN_ERR_UNSUPPORTED: return "unsupported configuration";
        case GNN_ERR_ALIGNMENT: return "feature pointer not 16-byte aligned";
        case GNN_ERR_OOM: return g_hip_msg[0] ? g_hip_msg : "device allocation failed";
        case GNN_ERR_HIP: return g_hip_msg[0] ? g_hip_msg : "HIP runtime error";
        case GNN_ERR_BAD_GRAPH: return "graph arrays inconsistent or out of range";
        case GNN_ERR_SCRATCH:
            return "the call needs more scratch than the allocation-free entry point's fixed buffer holds";
        default: return "unknown status";
    }
}

int gnn_plan_opts_default(gnn_plan_opts *o) {
    if (!o) return GNN_ERR_INVALID_ARG;
    o->light_threshold = 512;
    o->chunk = 512;
    o->waves_per_group = 4;
    o->tile_density = 0.0f;
    o->want_csc = 0;
    o->sched_order = 2;
    o->xcd_split = 1;
    return GNN_OK;
}

int gnn_csr_build(const int32_t *src, const int32_t *dst, int64_t n_edges_in, int32_t n_nodes,
                  int32_t add_self_loops, int32_t *indptr, int32_t *indices, int64_t cap,
                  int64_t *n_edges_out, hipStream_t stream) {
    if (n_nodes < 0 || n_edges_in < 0 || cap < 0 || !indptr || !n_edges_out) return GNN_ERR_INVALID_ARG;
    if (n_edges_in > 0 && (!src || !dst)) return GNN_ERR_INVALID_ARG;
    if (cap > 0 && !indices) return GNN_ERR_INVALID_ARG;
    const int64_t m = n_edges_in + (add_self_loops ? n_nodes : 0);
    if (m > kMaxEdges) return GNN_ERR_INVALID_ARG;
    if (n_nodes == 0 && n_edges_in > 0) return GNN_ERR_BAD_GRAPH;
    const int nb = bits_for(std::max<int64_t>(2, n_nodes));
    // scratch: keys, tmp keys (8 B each), flags, pos (4 B each), sort/scan scratch
    const int64_t ss = std::max(sort_scratch(m), scan_scratch(m)) + 2;
    DevBuf buf;
    GNN_TRY(dev_alloc(buf, (size_t)(16 * std::max<int64_t>(m, 1) + 8 * std::max<int64_t>(m, 1) + 4 * ss + 64)));
    uint64_t *keys = as<uint64_t>(buf), *tmp = keys + std::max<int64_t>(m, 1);
    int32_t *flags = reinterpret_cast<int32_t *>(tmp + std::max<int64_t>(m, 1));
    int32_t *pos = flags + std::max<int64_t>(m, 1);
    int32_t *err = pos + std::max<int64_t>(m, 1), *total = err + 1, *scr = total + 1;
    int rc = GNN_OK;
    int32_t h[2] = {0, 0};
    hipLaunchKernelGGL(k_set_i32, dim3(1), dim3(1), 0, stream, err, 0);
    if (m > 0)
        hipLaunchKernelGGL(k_coo_keys, grid1d(m), dim3(256), 0, stream, src, dst, n_edges_in, n_nodes, nb,
                           add_self_loops, keys, err);
    if ((rc = radix_sort(keys, tmp, m, 2 * nb, scr, stream)) != GNN_OK) goto done;
    if ((rc = emit_structure(keys, m, nb, 1, n_nodes, indptr, indices, cap, flags, pos, total, scr, stream)) !=
        GNN_OK)
        goto done;
    if (hipMemcpyAsync(h, err, 8, hipMemcpyDeviceToHost, stream) != hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess) {
        set_hip_error(hipGetLastError(), "gnn_csr_build");
        rc = GNN_ERR_HIP;
        goto done;
    }
    if (h[0]) {
        rc = GNN_ERR_BAD_GRAPH;
        goto done;
    }
    *n_edges_out = h[1];
    if (h[1] > cap) rc = GNN_ERR_INVALID_ARG;
done:
    dev_free(buf);
    return rc;
}

int gnn_plan_create(const int32_t *indptr, const int32_t *indices, int32_t n_nodes, int64_t n_edges,
                    const gnn_plan_opts *opts, hipStream_t stream, gnn_plan_t *plan_out) {
    if (!plan_out || !indptr || n_nodes < 0 || n_edges < 0 || n_edges > kMaxEdges) return GNN_ERR_INVALID_ARG;
    if (n_edges > 0 && !indices) return GNN_ERR_INVALID_ARG;
    gnn_plan_opts o;
    gnn_plan_opts_default(&o);
    if (opts) o = *opts;
    if (o.light_threshold < 0 || o.chunk < 1 ||
        !(o.waves_per_group == 1 || o.waves_per_group == 2 || o.waves_per_group == 4 || o.waves_per_group == 8))
        return GNN_ERR_INVALID_ARG;
    if (o.tile_density > 1.0f || o.sched_order < 0 || o.sched_order > 2) return GNN_ERR_INVALID_ARG;
    if (o.xcd_split != 0 && o.xcd_split != 1) return GNN_ERR_INVALID_ARG;
    if ((int64_t)o.chunk * o.waves_per_group > kMaxGroupSpan) return GNN_ERR_INVALID_ARG;

    gnn_plan_s *p = new (std::nothrow) gnn_plan_s();
    if (!p) return GNN_ERR_OOM;
    p->n_nodes = n_nodes;
    p->n_edges = n_edges;
    p->indptr = indptr;
    p->indices = indices;
    p->opts = o;
    int rc = validate_csr(indptr, indices, n_nodes, n_edges, stream);
    if (rc == GNN_OK) rc = check_rows_sorted(indptr, indices, n_nodes, n_edges, stream, &p->rows_sorted);
    if (rc == GNN_OK)
        rc = build_buckets(indptr, n_nodes, o.light_threshold, o.chunk, o.waves_per_group, o.sched_order, p->fwd,
                           stream, true);
    if (rc == GNN_OK && o.xcd_split) rc = build_xsplit(p, stream);
    if (rc == GNN_OK && o.want_csc) {
        rc = build_transpose(indptr, indices, n_nodes, n_edges, p->cindptr, p->cindices, stream);
        if (rc == GNN_OK) {
            p->has_csc = true;
            rc = build_buckets(as<int32_t>(p->cindptr), n_nodes, o.light_threshold, o.chunk, o.waves_per_group,
                               o.sched_order, p->bwd, stream, true);
        }
    }
    if (rc == GNN_OK && o.tile_density > 0.0f) {
        const int32_t min_nnz = std::max(1, (int32_t)std::ceil((double)o.tile_density * 256.0 - 1e-9));
        rc = build_tiles(p, min_nnz, stream);
    }
    if (rc != GNN_OK) {
        gnn_plan_destroy(p);
        return rc;
    }
    *plan_out = p;
    return GNN_OK;
}

int gnn_plan_export(gnn_plan_t p, gnn_plan_info *info) {
    if (!p || !info) return GNN_ERR_INVALID_ARG;
    std::memset(info, 0, sizeof(*info));
    info->n_nodes = p->n_nodes;
    info->n_edges = p->n_edges;
    info->light_threshold = p->opts.light_threshold;
    info->chunk = p->opts.chunk;
    info->waves_per_group = p->opts.waves_per_group;
    info->n_light = p->fwd.n_light;
    info->n_heavy = p->fwd.n_heavy;
    info->n_groups = p->fwd.n_groups;
    info->light_ids = as<int32_t>(p->fwd.light);
    info->heavy_ids = as<int32_t>(p->fwd.heavy);
    info->groups = as<int32_t>(p->fwd.groups);
    info->partial_ofs = as<int32_t>(p->fwd.partial_ofs);
    info->light_sched = as<int32_t>(p->fwd.sched);
    info->c_light_sched = as<int32_t>(p->bwd.sched);
    info->has_csc = p->has_csc;
    info->cindptr = as<int32_t>(p->cindptr);
    info->cindices = as<int32_t>(p->cindices);
    info->c_n_light = p->bwd.n_light;
    info->c_n_heavy = p->bwd.n_heavy;
    info->c_n_groups = p->bwd.n_groups;
    info->c_light_ids = as<int32_t>(p->bwd.light);
    info->c_heavy_ids = as<int32_t>(p->bwd.heavy);
    info->c_groups = as<int32_t>(p->bwd.groups);
    info->c_partial_ofs = as<int32_t>(p->bwd.partial_ofs);
    info->has_tiles = p->has_tiles;
    info->n_tiles = p->n_tiles;
    info->tile_min_nnz = p->tile_min_nnz;
    info->tile_rc = as<int32_t>(p->tile_rc);
    info->tile_mask = as<uint64_t>(p->tile_mask);
    info->tile_ptr = as<int32_t>(p->tile_ptr);
    info->rindptr = as<int32_t>(p->rindptr);
    info->rindices = as<int32_t>(p->rindices);
    info->n_residual = p->n_residual;
    info->n_trb = p->n_trb;
    info->trb = as<int32_t>(p->trb);
    info->n_light_nt = p->n_light_nt;
    info->light_nt = as<int32_t>(p->light_nt);
    info->ctile = as<int32_t>(p->ctile);
    info->ctile_ptr = as<int32_t>(p->ctile_ptr);
    info->n_tcb = p->n_tcb;
    info->tcb = as<int32_t>(p->tcb);
    info->rcindptr = as<int32_t>(p->rcindptr);
    info->rcindices = as<int32_t>(p->rcindices);
    info->n_c_light_nt = p->n_c_light_nt;
    info->c_light_nt = as<int32_t>(p->c_light_nt);
    info->structure_bytes = p->structure_bytes();
    info->workspace_bytes = (int64_t)p->ws.bytes;
    info->largest_workspace_alloc = p->largest_ws;
    info->rows_sorted = p->rows_sorted ? 1 : 0;
    info->light_by_degree = as<int32_t>(p->fwd.by_degree);
    info->c_light_by_degree = as<int32_t>(p->bwd.by_degree);
    info->spmm_norm = p->spmm_norm;
    info->spmm_w = as<float>(p->spmm_w);
    info->spmm_cw = as<float>(p->spmm_cw);
    info->n_long_light = p->fwd.n_long;
    info->c_n_long_light = p->bwd.n_long;
    info->n_xsplit_groups = p->xsplit.n_groups;
    info->n_xsplit_slots = p->xsplit.n_slots;
    info->xsplit_groups = as<int32_t>(p->xsplit.groups);
    info->xsplit_partial_ofs = as<int32_t>(p->xsplit.partial_ofs);
    info->xsplit_order = as<int32_t>(p->xsplit.order);
    return GNN_OK;
}

int gnn_plan_destroy(gnn_plan_t p) {
    if (!p) return GNN_ERR_INVALID_ARG;
    for (DevBuf *b : p->structures()) dev_free(*b);
    dev_free(p->ws);
    delete p;
    return GNN_OK;
}

int gnn_build_checked(void) {
#ifdef GNN_CHECKED
    return 1;
#else
    return 0;
#endif
}

int gnn_plan_set_timing(gnn_plan_t p, int32_t enable) {
    if (!p) return GNN_ERR_INVALID_ARG;
    p->timer.enabled = enable != 0;
    return GNN_OK;
}

int gnn_plan_timing_read(gnn_plan_t p, int32_t cap, const char **names, int32_t *launches, double *total_ms,
                         int32_t *n_out) {
    if (!p || cap < 0 || !n_out || (cap > 0 && (!names || !launches || !total_ms))) return GNN_ERR_INVALID_ARG;
    int32_t cnt[K_NUM_KINDS] = {0};
    double ms[K_NUM_KINDS] = {0};
    int rc = GNN_OK;
    for (auto &r : p->timer.log) {
        float t = 0.f;
        if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&t, r.a, r.b) != hipSuccess) {
            set_hip_error(hipGetLastError(), "timing");
            rc = GNN_ERR_HIP;
        }
        cnt[r.kind] += 1;
        ms[r.kind] += t;
        p->timer.pool.push_back(r.a);
        p->timer.pool.push_back(r.b);
    }
    p->timer.log.clear();
    int32_t n = 0;
    for (int k = 0; k < K_NUM_KINDS; ++k) {
        if (!cnt[k]) continue;
        if (n < cap) {
            names[n] = kKernelNames[k];
            launches[n] = cnt[k];
            total_ms[n] = ms[k];
        }
        ++n;
    }
    *n_out = n;
    return rc;
}

}  // extern "C"
