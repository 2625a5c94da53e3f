// Graph reordering: node orders that improve the locality of the per-edge
// row gathers, and the relabelling of a graph and of its feature rows.
//
// "On Efficient Scaling of GNNs via IO-Aware Layers Implementations",
// technical summary, Methodology (graph reordering revisited: its effect on
// neighbour-parallel and feature-parallel kernels; gather-dominated kernels
// gain on high-degree graphs).
//
// Degree of a node: its row's entries plus the entries naming it (in + out).
//   GNN_ORDER_DEGREE: descending degree, ties by ascending id (one radix sort).
//   GNN_ORDER_RCM: reverse Cuthill-McKee on the symmetrised graph.
//
// Cuthill-McKee visits components one after another, each from its unvisited
// node of smallest (degree, id) rank, breadth first, appending a node's
// unvisited neighbours in ascending rank. Its order is computed here without
// a sequential queue:
//  * the start of a component is its member of smallest rank, and components
//    come in the order of their starts; min-rank labelling over the
//    symmetrised graph labels every node with its start's rank. Each sweep
//    hooks along every entry (the smaller label of its two ends is written to
//    both ends and to the nodes whose ranks their labels are, the roots of
//    their label trees) and then jumps every label one step up its tree
//    (label[v] = label[node of rank label[v]]), so label chains shorten
//    geometrically: about log2(diameter) sweeps instead of one per hop;
//  * one breadth-first search runs from all starts at once, level by level.
//    A node of level L is appended, in the sequential order, by its neighbour
//    of level L-1 that comes first; among the level's new nodes of one
//    component the order is (that parent's place in level L-1, rank). Each
//    level's new nodes are found with an atomic minimum over their parents'
//    within-level indices (order independent), then sorted by (component,
//    parent index, degree, id) with two stable radix passes, which gives
//    their own within-level indices;
//  * the final order sorts all nodes by (component, level, within-level
//    index). Work: O(E) per label sweep, O(E) for the search, sorts of O(N);
//    one host synchronisation per sweep and per level. Both loops are capped
//    (label sweeps: 64 + 8 log2 N; search levels: 65,536); a graph that
//    reaches a cap returns GNN_ERR_UNSUPPORTED (the environment variables
//    GNN_RCM_MAX_SWEEPS and GNN_RCM_MAX_LEVELS override the caps).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cstdlib>
#include <vector>

#include "gnn_reorder.h"
#include "internal.h"

namespace gnn {

__global__ void k_named_count(const int32_t *indices, int64_t e, int32_t *cnt) {
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k < e) atomicAdd(cnt + indices[k], 1);
}

// deg[v] = row entries + entries naming v (cnt holds the latter)
__global__ void k_total_deg(const int32_t *indptr, int32_t n, int32_t *deg) {
    const int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (v < n) deg[v] += indptr[v + 1] - indptr[v];
}

// key (hi << 32 | v): hi = cap - deg (descending degree) or deg (ascending)
__global__ void k_deg_keys(const int32_t *deg, int32_t n, int64_t cap, int descending, uint64_t *keys) {
    const int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (v < n) {
        const uint64_t hi = descending ? (uint64_t)(cap - deg[v]) : (uint64_t)deg[v];
        keys[v] = (hi << 32) | (uint32_t)v;
    }
}

__global__ void k_low32(const uint64_t *keys, int64_t n, int32_t *out) {
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k < n) out[k] = (int32_t)(uint32_t)keys[k];
}

// rank[v] = position of v in the (degree, id) order; label starts as the rank
__global__ void k_rank_of(const int32_t *order, int32_t n, int32_t *rank, int32_t *label) {
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k < n) {
        rank[order[k]] = (int32_t)k;
        label[order[k]] = (int32_t)k;
    }
}

constexpr int kWaveR = 64;

__device__ __forceinline__ int wave_min(int x) {
    for (int off = 32; off > 0; off >>= 1) x = min(x, __shfl_xor(x, off, kWaveR));
    return x;
}

// Labels are ranks of nodes of the same component and only decrease, so the
// node of rank label[v] (node_of[label[v]]) is in v's component and its label
// is a valid label for v.
//
// Hooking sweep along every entry, both directions; one wave per row: the
// smallest label of the row and its sources is written to every larger one
// and to the node owning that larger label (the root of its label tree)
__global__ void k_label_hook(const int32_t *indptr, const int32_t *indices, int32_t n, const int32_t *node_of,
                             int32_t *label, int32_t *changed) {
    const int64_t v = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / kWaveR;
    const int lane = threadIdx.x % kWaveR;
    if (v >= n) return;
    const int32_t e0 = indptr[v], e1 = indptr[v + 1];
    int lv = label[v];
    for (int32_t e = e0 + lane; e < e1; e += kWaveR) lv = min(lv, label[indices[e]]);
    lv = wave_min(lv);
    bool moved = false;
    for (int32_t e = e0 + lane; e < e1; e += kWaveR) {
        const int32_t u = indices[e];
        const int32_t lu = label[u];
        if (lv < lu) {
            atomicMin(label + u, lv);
            atomicMin(label + node_of[lu], lv);
            moved = true;
        }
    }
    if (lane == 0) {
        const int32_t l0 = label[v];
        if (lv < l0) {
            atomicMin(label + v, lv);
            atomicMin(label + node_of[l0], lv);
            moved = true;
        }
    }
    if (moved) *changed = 1;
}

// one pointer-jumping step for every node: label[v] = label[node of rank label[v]]
__global__ void k_label_jump(int32_t n, const int32_t *node_of, int32_t *label, int32_t *changed) {
    const int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (v >= n) return;
    const int32_t l = label[v];
    const int32_t up = label[node_of[l]];
    if (up < l) {
        atomicMin(label + v, up);
        *changed = 1;
    }
}

// starts: nodes whose label is their own rank; level 0, within-level index 0
__global__ void k_starts(const int32_t *rank, const int32_t *label, int32_t n, int32_t *level, int32_t *wr,
                         int32_t *front, int32_t *count) {
    const int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (v < n && label[v] == rank[v]) {
        level[v] = 0;
        wr[v] = 0;
        front[atomicAdd(count, 1)] = (int32_t)v;
    }
}

// frontier expansion over in-lists (CSR) and out-lists (transpose): an
// unvisited neighbour takes the smallest within-level index among its
// frontier neighbours; its first discoverer appends it to the candidates
__global__ void k_expand(const int32_t *front, int32_t nf, const int32_t *indptr, const int32_t *indices,
                         const int32_t *cindptr, const int32_t *cindices, const int32_t *level, const int32_t *wr,
                         int32_t *pmin, int32_t *cand, int32_t *count) {
    const int64_t t = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / kWaveR;   // one wave per frontier node
    const int lane = threadIdx.x % kWaveR;
    if (t >= nf) return;
    const int32_t u = front[t];
    const int32_t w = wr[u];
    for (int side = 0; side < 2; ++side) {
        const int32_t *ip = side ? cindptr : indptr;
        const int32_t *ix = side ? cindices : indices;
        for (int32_t e = ip[u] + lane; e < ip[u + 1]; e += kWaveR) {
            const int32_t v = ix[e];
            if (level[v] >= 0) continue;
            if (atomicMin(pmin + v, w) == INT_MAX) cand[atomicAdd(count, 1)] = v;
        }
    }
}

// keys of the candidates: first pass (degree, id), second pass (component, parent index)
__global__ void k_cand_keys1(const int32_t *cand, int32_t nc, const int32_t *deg, uint64_t *keys, int32_t *vals) {
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k < nc) {
        const int32_t v = cand[k];
        keys[k] = ((uint64_t)(uint32_t)deg[v] << 32) | (uint32_t)v;
        vals[k] = v;
    }
}

__global__ void k_cand_keys2(const int32_t *vals, int32_t nc, const int32_t *label, const int32_t *pmin,
                             uint64_t *keys) {
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k < nc) {
        const int32_t v = vals[k];
        keys[k] = ((uint64_t)(uint32_t)label[v] << 32) | (uint32_t)pmin[v];
    }
}

// sorted candidates: first index of each component's run, then within-level indices
__global__ void k_run_heads(const int32_t *vals, int32_t nc, const int32_t *label, int32_t *head_of) {
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k < nc && (k == 0 || label[vals[k]] != label[vals[k - 1]])) head_of[label[vals[k]]] = (int32_t)k;
}

__global__ void k_assign_level(const int32_t *vals, int32_t nc, const int32_t *label, const int32_t *head_of,
                               int32_t L, int32_t *level, int32_t *wr, int32_t *front) {
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k < nc) {
        const int32_t v = vals[k];
        level[v] = L;
        wr[v] = (int32_t)k - head_of[label[v]];
        front[k] = v;
    }
}

__global__ void k_final_keys1(const int32_t *level, const int32_t *wr, int32_t n, uint64_t *keys, int32_t *vals) {
    const int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (v < n) {
        keys[v] = ((uint64_t)(uint32_t)level[v] << 32) | (uint32_t)wr[v];
        vals[v] = (int32_t)v;
    }
}

__global__ void k_final_keys2(const int32_t *vals, int32_t n, const int32_t *label, uint64_t *keys) {
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k < n) keys[k] = (uint64_t)(uint32_t)label[vals[k]];
}

// perm[new] = cm[n - 1 - new]
__global__ void k_reverse(const int32_t *cm, int32_t n, int32_t *perm) {
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k < n) perm[k] = cm[n - 1 - k];
}

static int read_i32(const int32_t *dev, int32_t *host, hipStream_t s) {
    if (hipMemcpyAsync(host, dev, 4, hipMemcpyDeviceToHost, s) != hipSuccess || hipStreamSynchronize(s) != hipSuccess)
        return GNN_ERR_HIP;
    return GNN_OK;
}

// workspace of the reorder: int32 arrays and 64-bit sort buffers
struct ReorderWs {
    DevBuf buf;
    int32_t *deg, *rank, *label, *level, *wr, *pmin, *front, *cand, *head_of, *vals, *vtmp, *scratch, *flag;
    uint64_t *keys, *tmp;
};

static int reorder_ws(ReorderWs &w, int32_t n) {
    const int64_t m = std::max<int64_t>(n, 1);
    const int64_t ss = sort_scratch(m) + 2;
    const size_t bytes = (size_t)(16 * m) + (size_t)(4 * (11 * m + ss)) + 256;
    GNN_TRY(dev_alloc(w.buf, bytes));
    uint64_t *q = as<uint64_t>(w.buf);
    w.keys = q;
    w.tmp = q + m;
    int32_t *p = reinterpret_cast<int32_t *>(q + 2 * m);
    int32_t **slots[] = {&w.deg, &w.rank, &w.label, &w.level, &w.wr, &w.pmin, &w.front, &w.cand, &w.head_of,
                         &w.vals, &w.vtmp};
    for (int32_t **sl : slots) {
        *sl = p;
        p += m;
    }
    w.flag = p;
    w.scratch = p + 16;
    return GNN_OK;
}

static int degrees(const int32_t *indptr, const int32_t *indices, int32_t n, int64_t e, int32_t *deg, hipStream_t s) {
    hipLaunchKernelGGL(k_fill_i32, grid1d(n), dim3(256), 0, s, deg, (int64_t)n, 0);
    if (e > 0) hipLaunchKernelGGL(k_named_count, grid1d(e), dim3(256), 0, s, indices, e, deg);
    hipLaunchKernelGGL(k_total_deg, grid1d(n), dim3(256), 0, s, indptr, n, deg);
    GNN_HIP(hipGetLastError());
    return GNN_OK;
}

// order by degree into out[n]: descending (perm of GNN_ORDER_DEGREE) or ascending (ranks for RCM)
static int degree_order(ReorderWs &w, int32_t n, int64_t e, int descending, int32_t *out, hipStream_t s) {
    const int64_t cap = 2 * e + 1;
    hipLaunchKernelGGL(k_deg_keys, grid1d(n), dim3(256), 0, s, w.deg, n, cap, descending, w.keys);
    GNN_TRY(radix_sort(w.keys, w.tmp, n, 32 + bits_for(cap + 1), w.scratch, s));
    hipLaunchKernelGGL(k_low32, grid1d(n), dim3(256), 0, s, w.keys, (int64_t)n, out);
    GNN_HIP(hipGetLastError());
    return GNN_OK;
}

// loop cap from the environment variable `name` (a positive integer), else dflt
static int64_t env_cap(const char *name, int64_t dflt) {
    const char *s = getenv(name);
    if (!s || !*s) return dflt;
    char *end = nullptr;
    const long long v = strtoll(s, &end, 10);
    return (end != s && *end == '\0' && v > 0) ? (int64_t)v : dflt;
}

static int rcm(const int32_t *indptr, const int32_t *indices, int32_t n, int64_t e, int32_t *perm, hipStream_t s) {
    const int64_t max_sweeps = env_cap("GNN_RCM_MAX_SWEEPS", 64 + 8 * (int64_t)bits_for((int64_t)n + 1));
    const int64_t max_levels = env_cap("GNN_RCM_MAX_LEVELS", 65536);
    ReorderWs w;
    GNN_TRY(reorder_ws(w, n));
    DevBuf cindptr, cindices;
    int rc = degrees(indptr, indices, n, e, w.deg, s);
    if (rc == GNN_OK) rc = build_transpose(indptr, indices, n, e, cindptr, cindices, s);
    // ranks: position in ascending (degree, id); labels start as ranks
    if (rc == GNN_OK) rc = degree_order(w, n, e, 0, w.front, s);
    if (rc == GNN_OK) {
        hipLaunchKernelGGL(k_rank_of, grid1d(n), dim3(256), 0, s, w.front, n, w.rank, w.label);
        // components: hooking and one jump per sweep until a sweep changes
        // nothing (w.front holds the node of each rank until the search starts)
        for (int64_t sweep = 0;; ++sweep) {
            if (sweep == max_sweeps) {
                rc = GNN_ERR_UNSUPPORTED;
                break;
            }
            int32_t changed = 0;
            hipLaunchKernelGGL(k_set_i32, dim3(1), dim3(1), 0, s, w.flag, 0);
            hipLaunchKernelGGL(k_label_hook, grid1d((int64_t)n * kWaveR), dim3(256), 0, s, indptr, indices, n, w.front,
                               w.label, w.flag);
            hipLaunchKernelGGL(k_label_jump, grid1d(n), dim3(256), 0, s, n, w.front, w.label, w.flag);
            if ((rc = read_i32(w.flag, &changed, s)) != GNN_OK || !changed) break;
        }
    }
    int32_t nf = 0;
    if (rc == GNN_OK) {
        hipLaunchKernelGGL(k_fill_i32, grid1d(n), dim3(256), 0, s, w.level, (int64_t)n, -1);
        hipLaunchKernelGGL(k_fill_i32, grid1d(n), dim3(256), 0, s, w.pmin, (int64_t)n, INT_MAX);
        hipLaunchKernelGGL(k_set_i32, dim3(1), dim3(1), 0, s, w.flag, 0);
        hipLaunchKernelGGL(k_starts, grid1d(n), dim3(256), 0, s, w.rank, w.label, n, w.level, w.wr, w.front,
                           w.flag);
        rc = read_i32(w.flag, &nf, s);
    }
    // level-synchronous search from every start
    for (int32_t L = 1; rc == GNN_OK && nf > 0; ++L) {
        int32_t nc = 0;
        hipLaunchKernelGGL(k_set_i32, dim3(1), dim3(1), 0, s, w.flag, 0);
        hipLaunchKernelGGL(k_expand, grid1d((int64_t)nf * kWaveR), dim3(256), 0, s, w.front, nf, indptr, indices,
                           as<int32_t>(cindptr), as<int32_t>(cindices), w.level, w.wr, w.pmin, w.cand, w.flag);
        if ((rc = read_i32(w.flag, &nc, s)) != GNN_OK || nc == 0) break;
        if (L > max_levels) {      // level L has nodes: the search needs more levels than the cap
            rc = GNN_ERR_UNSUPPORTED;
            break;
        }
        hipLaunchKernelGGL(k_cand_keys1, grid1d(nc), dim3(256), 0, s, w.cand, nc, w.deg, w.keys, w.vals);
        rc = radix_sort(w.keys, w.tmp, nc, 64, w.scratch, s, w.vals, w.vtmp);
        if (rc != GNN_OK) break;
        hipLaunchKernelGGL(k_cand_keys2, grid1d(nc), dim3(256), 0, s, w.vals, nc, w.label, w.pmin, w.keys);
        rc = radix_sort(w.keys, w.tmp, nc, 64, w.scratch, s, w.vals, w.vtmp);
        if (rc != GNN_OK) break;
        hipLaunchKernelGGL(k_run_heads, grid1d(nc), dim3(256), 0, s, w.vals, nc, w.label, w.head_of);
        hipLaunchKernelGGL(k_assign_level, grid1d(nc), dim3(256), 0, s, w.vals, nc, w.label, w.head_of, L, w.level,
                           w.wr, w.front);
        nf = nc;
    }
    // Cuthill-McKee order: by (component, level, within-level index); then reversed
    if (rc == GNN_OK) {
        hipLaunchKernelGGL(k_final_keys1, grid1d(n), dim3(256), 0, s, w.level, w.wr, n, w.keys, w.vals);
        rc = radix_sort(w.keys, w.tmp, n, 64, w.scratch, s, w.vals, w.vtmp);
    }
    if (rc == GNN_OK) {
        hipLaunchKernelGGL(k_final_keys2, grid1d(n), dim3(256), 0, s, w.vals, n, w.label, w.keys);
        rc = radix_sort(w.keys, w.tmp, n, 32, w.scratch, s, w.vals, w.vtmp);
    }
    if (rc == GNN_OK) {
        hipLaunchKernelGGL(k_reverse, grid1d(n), dim3(256), 0, s, w.vals, n, perm);
        if (hipStreamSynchronize(s) != hipSuccess) rc = GNN_ERR_HIP;
    }
    dev_free(cindptr);
    dev_free(cindices);
    dev_free(w.buf);
    return rc;
}

// ---------------------------------------------------------------- relabelling

__global__ void k_perm_check(const int32_t *perm, int32_t n, int32_t *hits, int32_t *bad) {
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k < n) {
        const int32_t v = perm[k];
        if (v < 0 || v >= n || atomicAdd(hits + v, 1) != 0) *bad = 1;
    }
}

__global__ void k_inverse(const int32_t *perm, int32_t n, int32_t *inv) {
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k < n) inv[perm[k]] = (int32_t)k;
}

__global__ void k_new_deg(const int32_t *indptr, const int32_t *perm, int32_t n, int32_t *deg) {
    const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (r < n) deg[r] = indptr[perm[r] + 1] - indptr[perm[r]];
}

// one wave per old row: keys (new row << nb | new source) of its entries
__global__ void k_relabel_keys(const int32_t *indptr, const int32_t *indices, const int32_t *inv, int32_t n, int nb,
                               uint64_t *keys) {
    const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / kWaveR;
    const int lane = threadIdx.x % kWaveR;
    if (i >= n) return;
    const uint64_t r = (uint64_t)(uint32_t)inv[i] << nb;
    for (int32_t e = indptr[i] + lane; e < indptr[i + 1]; e += kWaveR) keys[e] = r | (uint32_t)inv[indices[e]];
}

static inline bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

__global__ void k_low_bits(const uint64_t *keys, int64_t e, int nb, int32_t *out) {
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k < e) out[k] = (int32_t)(keys[k] & ((1ull << nb) - 1));
}

// dst[r] = src[perm[r]] (forward) or dst[perm[r]] = src[r] (back), rows of w 16-byte words
__global__ void k_permute_rows(const uint4 *src, uint4 *dst, const int32_t *perm, int32_t n, int64_t w, int back) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= (int64_t)n * w) return;
    const int64_t r = t / w, c = t % w;
    const int64_t p = perm[r];
    if (back)
        dst[p * w + c] = src[r * w + c];
    else
        dst[r * w + c] = src[p * w + c];
}

// perm must name every node once: GNN_OK or GNN_ERR_INVALID_ARG (synchronises s)
static int check_perm(const int32_t *perm, int32_t n, hipStream_t s) {
    DevBuf tmp;
    GNN_TRY(dev_alloc(tmp, (size_t)std::max(n, 1) * 4 + 64));
    int32_t *bad = as<int32_t>(tmp), *hits = bad + 16;
    hipLaunchKernelGGL(k_set_i32, dim3(1), dim3(1), 0, s, bad, 0);
    hipLaunchKernelGGL(k_fill_i32, grid1d(n), dim3(256), 0, s, hits, (int64_t)n, 0);
    hipLaunchKernelGGL(k_perm_check, grid1d(n), dim3(256), 0, s, perm, n, hits, bad);
    int32_t h = 0;
    int rc = read_i32(bad, &h, s);
    dev_free(tmp);
    if (rc == GNN_OK && h) rc = GNN_ERR_INVALID_ARG;
    return rc;
}

}  // namespace gnn

using namespace gnn;

extern "C" {

int gnn_reorder(const int32_t *indptr, const int32_t *indices, int32_t N, int64_t E, gnn_order_t method,
                int32_t *perm, hipStream_t stream) {
    if (N < 0 || E < 0 || E > kMaxEdges || !indptr || (E > 0 && !indices) || (N > 0 && !perm))
        return GNN_ERR_INVALID_ARG;
    if (method != GNN_ORDER_DEGREE && method != GNN_ORDER_RCM) return GNN_ERR_INVALID_ARG;
    if (N == 0) return GNN_OK;
    GNN_TRY(validate_csr(indptr, indices, N, E, stream));
    if (method == GNN_ORDER_RCM) return rcm(indptr, indices, N, E, perm, stream);
    ReorderWs w;
    GNN_TRY(reorder_ws(w, N));
    int rc = degrees(indptr, indices, N, E, w.deg, stream);
    if (rc == GNN_OK) rc = degree_order(w, N, E, 1, perm, stream);
    if (rc == GNN_OK && hipStreamSynchronize(stream) != hipSuccess) rc = GNN_ERR_HIP;
    dev_free(w.buf);
    return rc;
}

int gnn_permute_graph(const int32_t *indptr, const int32_t *indices, int32_t N, int64_t E, const int32_t *perm,
                      int32_t *new_indptr, int32_t *new_indices, hipStream_t stream) {
    if (N < 0 || E < 0 || E > kMaxEdges || !indptr || !new_indptr || (E > 0 && (!indices || !new_indices)) ||
        (N > 0 && !perm))
        return GNN_ERR_INVALID_ARG;
    if (N == 0) {
        hipLaunchKernelGGL(k_set_i32, dim3(1), dim3(1), 0, stream, new_indptr, 0);
        GNN_HIP(hipGetLastError());
        return GNN_OK;
    }
    GNN_TRY(validate_csr(indptr, indices, N, E, stream));
    GNN_TRY(check_perm(perm, N, stream));
    const int64_t m = std::max<int64_t>(E, 1);
    const int64_t ss = std::max(sort_scratch(m), scan_scratch(N + 1)) + 2;
    DevBuf tmp;
    GNN_TRY(dev_alloc(tmp, (size_t)(16 * m) + (size_t)(4 * (2 * (int64_t)N + 2 + ss)) + 64));
    uint64_t *keys = as<uint64_t>(tmp), *kt = keys + m;
    int32_t *inv = reinterpret_cast<int32_t *>(kt + m), *deg = inv + N, *scr = deg + N + 2;
    const int nb = bits_for(std::max<int64_t>(2, N));
    hipLaunchKernelGGL(k_inverse, grid1d(N), dim3(256), 0, stream, perm, N, inv);
    hipLaunchKernelGGL(k_new_deg, grid1d(N), dim3(256), 0, stream, indptr, perm, N, deg);
    hipLaunchKernelGGL(k_set_i32, dim3(1), dim3(1), 0, stream, deg + N, 0);
    int rc = scan_rec(deg, new_indptr, N + 1, nullptr, scr, stream);
    if (rc == GNN_OK && E > 0) {
        hipLaunchKernelGGL(k_relabel_keys, grid1d((int64_t)N * kWaveR), dim3(256), 0, stream, indptr, indices, inv, N,
                           nb, keys);
        rc = radix_sort(keys, kt, E, 2 * nb, scr, stream);
        if (rc == GNN_OK) hipLaunchKernelGGL(k_low_bits, grid1d(E), dim3(256), 0, stream, keys, E, nb, new_indices);
    }
    if (rc == GNN_OK && hipStreamSynchronize(stream) != hipSuccess) rc = GNN_ERR_HIP;
    dev_free(tmp);
    return rc;
}

int gnn_permute_rows(const void *src, void *dst, int32_t N, int64_t row_bytes, const int32_t *perm, int32_t back,
                     hipStream_t stream) {
    // src == dst is rejected only when there is something to copy: empty
    // tables (N == 0 or row_bytes == 0) may both be null
    if (N < 0 || row_bytes < 0 || (N > 0 && (!src || !dst || !perm))) return GNN_ERR_INVALID_ARG;
    if (N > 0 && row_bytes > 0 && src == dst) return GNN_ERR_INVALID_ARG;
    if (row_bytes % 16) return GNN_ERR_UNSUPPORTED;
    if (!aligned16(src) || !aligned16(dst)) return GNN_ERR_ALIGNMENT;
    if (N == 0 || row_bytes == 0) return GNN_OK;
    GNN_TRY(check_perm(perm, N, stream));
    const int64_t w = row_bytes / 16;
    hipLaunchKernelGGL(k_permute_rows, grid1d((int64_t)N * w), dim3(256), 0, stream, (const uint4 *)src, (uint4 *)dst,
                       perm, N, w, back ? 1 : 0);
    GNN_HIP(hipGetLastError());
    return GNN_OK;
}

}  // extern "C"
