// 16x16 dense-tile census on the device.
//
// "On Efficient Scaling of GNNs via IO-Aware Layers Implementations",
// technical summary, Methodology (attention-based layers, Tensor-Core
// optimisation): local neighbourhoods are packed into 16x16 blocks so that
// matrix units can be used; this pays off only on locally dense graphs.
//
// Definition (bit-exact): aligned 16-node blocks; a pair (row block b,
// column block c) is eligible when no node of b has in-degree > T and no node
// of c has out-degree > T; an eligible pair with >= min_nnz distinct
// (dst, src) positions is a tile with a 256-bit mask (bit (dst%16)*16 +
// src%16). The first copy of each tiled position is covered by the tile;
// every other edge stays in the residual CSR (CSR order). Tiles are listed by
// (b, c). All steps are stable sorts, scans and order-free bit ORs, so the
// result does not depend on scheduling.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "device.h"
#include "internal.h"

namespace gnn {

__global__ void k_fill(int32_t *p, int64_t n, int32_t v) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}

__global__ void k_fill_u64(uint64_t *p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0ull;
}

__global__ void k_outdeg(const int32_t *indices, int64_t e, int32_t *odeg) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < e) atomicAdd(&odeg[indices[i]], 1);
}

__global__ void k_block_heavy(const int32_t *indptr, const int32_t *odeg, int32_t n, int32_t T, int32_t *rb_bad,
                              int32_t *cb_bad) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    if (indptr[i + 1] - indptr[i] > T) rb_bad[i >> 4] = 1;
    if (odeg[i] > T) cb_bad[i >> 4] = 1;
}

// one wave per CSR row: key (rb, cb, position) of each eligible edge, a
// sentinel above every key otherwise; payload = edge position
__global__ void k_tile_keys(const int32_t *indptr, const int32_t *indices, int32_t n, int cbits,
                            const int32_t *rb_bad, const int32_t *cb_bad, uint64_t sentinel, uint64_t *keys,
                            int32_t *vals) {
    const int row = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    if (row >= n) return;
    const int lane = lane_id();
    const uint64_t rb = (uint64_t)(row >> 4);
    const bool row_ok = !rb_bad[row >> 4];
    for (int32_t e = indptr[row] + lane; e < indptr[row + 1]; e += kWave) {
        const int32_t j = indices[e];
        const bool ok = row_ok && !cb_bad[j >> 4];
        keys[e] = ok ? ((((rb << cbits) | (uint64_t)(j >> 4)) << 8) | (uint64_t)(((row & 15) << 4) | (j & 15)))
                     : sentinel;
        vals[e] = e;
    }
}

// over sorted keys: f = first copy of a position, seg = first key of a block pair
__global__ void k_tile_flags(const uint64_t *k, int64_t m, uint64_t sentinel, int32_t *f, int32_t *seg) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= m) return;
    const uint64_t key = k[i];
    const bool valid = key != sentinel;
    const bool first = (i == 0) || key != k[i - 1];
    const bool start = (i == 0) || (key >> 8) != (k[i - 1] >> 8);
    f[i] = (valid && first) ? 1 : 0;
    seg[i] = (valid && start) ? 1 : 0;
}

// per segment: exclusive count of first copies at its start, and its pair
__global__ void k_seg_info(const uint64_t *k, int64_t m, const int32_t *seg, const int32_t *spos,
                           const int32_t *fpos, int32_t *sstart, uint64_t *spair, int32_t n_seg, int32_t n_first) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i == 0) sstart[n_seg] = n_first;
    if (i >= m || !seg[i]) return;
    const int32_t s = spos[i];
    sstart[s] = fpos[i];
    spair[s] = k[i] >> 8;
}

__global__ void k_tile_sel(const int32_t *sstart, int32_t n_seg, int32_t min_nnz, int32_t *tflag) {
    const int64_t s = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (s < n_seg) tflag[s] = (sstart[s + 1] - sstart[s] >= min_nnz) ? 1 : 0;
}

__global__ void k_tile_emit(const uint64_t *spair, const int32_t *tflag, const int32_t *tpos, int32_t n_seg,
                            int cbits, int32_t *tile_rc, int32_t *cnt_rb, int32_t *cnt_cb) {
    const int64_t s = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (s >= n_seg || !tflag[s]) return;
    const int32_t t = tpos[s];
    const int32_t rb = (int32_t)(spair[s] >> cbits);
    const int32_t cb = (int32_t)(spair[s] & ((1ull << cbits) - 1ull));
    tile_rc[2 * (int64_t)t] = rb;
    tile_rc[2 * (int64_t)t + 1] = cb;
    atomicAdd(&cnt_rb[rb], 1);
    atomicAdd(&cnt_cb[cb], 1);
}

// first copies inside tiles: set the mask bit, mark the CSR edge as tiled
__global__ void k_tile_mask(const uint64_t *k, const int32_t *vals, int64_t m, const int32_t *f, const int32_t *seg,
                            const int32_t *spos, const int32_t *tflag, const int32_t *tpos, uint64_t *mask,
                            int32_t *in_tile) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= m || !f[i]) return;
    const int32_t s = spos[i] + seg[i] - 1;
    if (!tflag[s]) return;
    const int32_t t = tpos[s];
    const int pos = (int)(k[i] & 255ull);
    atomicOr((unsigned long long *)&mask[4 * (int64_t)t + (pos >> 6)], 1ull << (pos & 63));
    in_tile[vals[i]] = 1;
}

__global__ void k_not(const int32_t *in, int64_t n, int32_t *out) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) out[i] = in[i] ? 0 : 1;
}

__global__ void k_res_emit(const int32_t *indptr, const int32_t *indices, int32_t n, int64_t e, const int32_t *rflag,
                           const int32_t *rpos, int32_t n_res, int32_t *rindptr, int32_t *rindices) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < e && rflag[i]) rindices[rpos[i]] = indices[i];
    if (i <= n) {
        const int32_t s = indptr[i];
        rindptr[i] = (s < e) ? rpos[s] : n_res;
    }
}

__global__ void k_flag_pos(const int32_t *cnt, int32_t n, int32_t *flag) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) flag[i] = cnt[i] > 0 ? 1 : 0;
}

// nodes of degree <= T (deg from rowptr, or from deg_arr) in blocks without tiles
__global__ void k_flag_light_nt(const int32_t *rowptr, const int32_t *deg_arr, const int32_t *blk_cnt, int32_t n,
                                int32_t T, int32_t *flag) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const int32_t d = rowptr ? rowptr[i + 1] - rowptr[i] : deg_arr[i];
    flag[i] = (d <= T && blk_cnt[i >> 4] == 0) ? 1 : 0;
}

__global__ void k_compact(const int32_t *flag, const int32_t *pos, int64_t n, int32_t *out) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n && flag[i]) out[pos[i]] = (int32_t)i;
}

__global__ void k_ctile_keys(const int32_t *tile_rc, int32_t n_tiles, uint64_t *keys) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t < n_tiles) keys[t] = ((uint64_t)(uint32_t)tile_rc[2 * t + 1] << 32) | (uint64_t)t;
}

__global__ void k_low32(const uint64_t *keys, int32_t n, int32_t *out) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t < n) out[t] = (int32_t)(keys[t] & 0xFFFFFFFFull);
}

namespace {

struct Scratch {
    DevBuf b;
    int32_t *i32(int64_t n) {
        int32_t *p = reinterpret_cast<int32_t *>(cur);
        cur += ((size_t)std::max<int64_t>(n, 1) * 4 + 255) & ~(size_t)255;
        return p;
    }
    uint64_t *u64(int64_t n) {
        uint64_t *p = reinterpret_cast<uint64_t *>(cur);
        cur += ((size_t)std::max<int64_t>(n, 1) * 8 + 255) & ~(size_t)255;
        return p;
    }
    char *cur = nullptr;
};

int read_i32(const int32_t *dev, int32_t *host, int count, hipStream_t s) {
    GNN_HIP(hipMemcpyAsync(host, dev, (size_t)count * 4, hipMemcpyDeviceToHost, s));
    GNN_HIP(hipStreamSynchronize(s));
    return GNN_OK;
}

// out <- ascending indices i < n with flag[i] != 0; count on the host
int compact(const int32_t *flag, int64_t n, DevBuf &out, int32_t &count, int32_t *pos, int32_t *tot,
            int32_t *scr, hipStream_t s) {
    GNN_TRY(scan_rec(flag, pos, n, tot, scr, s));
    GNN_TRY(read_i32(tot, &count, 1, s));
    GNN_TRY(dev_alloc(out, (size_t)std::max(1, count) * 4));
    if (n > 0) hipLaunchKernelGGL(k_compact, grid1d(n), dim3(256), 0, s, flag, pos, n, as<int32_t>(out));
    GNN_HIP(hipGetLastError());
    return GNN_OK;
}

// counts [nb] -> ptr [nb+1] (exclusive scan, total last)
int counts_to_ptr(const int32_t *cnt, int32_t nb, DevBuf &ptr, int32_t *scr, hipStream_t s) {
    GNN_TRY(dev_alloc(ptr, (size_t)(nb + 1) * 4));
    GNN_TRY(scan_rec(cnt, as<int32_t>(ptr), nb, as<int32_t>(ptr) + nb, scr, s));
    return GNN_OK;
}

}  // namespace

int build_tiles(gnn_plan_s *p, int32_t min_nnz, hipStream_t s) {
    const int32_t n = p->n_nodes;
    const int64_t E = p->n_edges;
    const int32_t T = p->opts.light_threshold;
    const int32_t nb = (n + 15) / 16;
    const int cbits = bits_for(std::max<int64_t>(2, nb));
    const int key_bits = 2 * cbits + 8 + 1;
    const uint64_t sentinel = 1ull << (key_bits - 1);
    p->tile_min_nnz = min_nnz;

    const int64_t big = std::max<int64_t>(E, n) + 1;
    const int64_t ss = std::max(sort_scratch(big), scan_scratch(big)) + 8;
    Scratch S;
    // keys x2, vals x2, f, seg, fpos, spos, rflag/rpos, node arrays, scan scratch, headroom
    const size_t bytes = (size_t)(16 * big + 8 * big + 4 * 6 * big + 4 * 8 * (int64_t)(n + 16) + 4 * ss) + 64 * 256;
    GNN_TRY(dev_alloc(S.b, bytes));
    S.cur = reinterpret_cast<char *>(S.b.p);
    uint64_t *keys = S.u64(big), *ktmp = S.u64(big);
    int32_t *vals = S.i32(big), *vtmp = S.i32(big);
    int32_t *f = S.i32(big), *seg = S.i32(big), *fpos = S.i32(big), *spos = S.i32(big);
    int32_t *aux = S.i32(big), *aux2 = S.i32(big);
    int32_t *odeg = S.i32(n), *rb_bad = S.i32(nb), *cb_bad = S.i32(nb), *cnt_rb = S.i32(nb), *cnt_cb = S.i32(nb);
    int32_t *nflag = S.i32(n), *npos = S.i32(n);
    int32_t *tot = S.i32(8);
    int32_t *scr = S.i32(ss);
    int rc = GNN_OK;
    int32_t h[2] = {0, 0};
    int32_t n_seg = 0, n_first = 0;
    DevBuf seginfo, in_tile;

#define TRY(x)                           \
    do {                                 \
        if ((rc = (x)) != GNN_OK) goto done; \
    } while (0)

    for (int32_t *z : {odeg, rb_bad, cb_bad, cnt_rb, cnt_cb})
        hipLaunchKernelGGL(k_fill, grid1d(std::max(n, nb)), dim3(256), 0, s, z, (int64_t)(z == odeg ? n : nb), 0);
    if (E > 0) hipLaunchKernelGGL(k_outdeg, grid1d(E), dim3(256), 0, s, p->indices, E, odeg);
    if (n > 0) {
        hipLaunchKernelGGL(k_block_heavy, grid1d(n), dim3(256), 0, s, p->indptr, odeg, n, T, rb_bad, cb_bad);
        hipLaunchKernelGGL(k_tile_keys, dim3((unsigned)cdiv(n, 4)), dim3(256), 0, s, p->indptr, p->indices, n, cbits,
                           rb_bad, cb_bad, sentinel, keys, vals);
    }
    TRY(radix_sort(keys, ktmp, E, key_bits, scr, s, vals, vtmp));
    if (E > 0) {
        hipLaunchKernelGGL(k_tile_flags, grid1d(E), dim3(256), 0, s, keys, E, sentinel, f, seg);
        TRY(scan_rec(f, fpos, E, tot + 0, scr, s));
        TRY(scan_rec(seg, spos, E, tot + 1, scr, s));
        TRY(read_i32(tot, h, 2, s));
        n_first = h[0];
        n_seg = h[1];
    }
    {
        // per-segment arrays: sstart [n_seg+1], tflag, tpos [n_seg], spair u64 [n_seg]
        TRY(dev_alloc(seginfo, (size_t)(n_seg + 1) * 12 + (size_t)(n_seg + 1) * 8 + 1024));
        int32_t *sstart = as<int32_t>(seginfo), *tflag = sstart + (n_seg + 1), *tpos = tflag + (n_seg + 1);
        uint64_t *spair = reinterpret_cast<uint64_t *>(as<char>(seginfo) + ((((size_t)(n_seg + 1) * 12) + 255) & ~(size_t)255));
        if (E > 0) {
            hipLaunchKernelGGL(k_seg_info, grid1d(E), dim3(256), 0, s, keys, E, seg, spos, fpos, sstart, spair, n_seg,
                               n_first);
            hipLaunchKernelGGL(k_tile_sel, grid1d(n_seg), dim3(256), 0, s, sstart, n_seg, min_nnz, tflag);
        }
        TRY(scan_rec(tflag, tpos, n_seg, tot + 2, scr, s));
        TRY(read_i32(tot + 2, &p->n_tiles, 1, s));
        const int32_t nt = p->n_tiles;
        TRY(dev_alloc(p->tile_rc, (size_t)std::max(1, nt) * 8));
        TRY(dev_alloc(p->tile_mask, (size_t)std::max(1, nt) * 32));
        TRY(dev_alloc(in_tile, (size_t)std::max<int64_t>(E, 1) * 4));
        hipLaunchKernelGGL(k_fill_u64, grid1d(4 * (int64_t)std::max(1, nt)), dim3(256), 0, s, as<uint64_t>(p->tile_mask),
                           4 * (int64_t)std::max(1, nt));
        hipLaunchKernelGGL(k_fill, grid1d(std::max<int64_t>(E, 1)), dim3(256), 0, s, as<int32_t>(in_tile),
                           std::max<int64_t>(E, 1), 0);
        if (n_seg > 0)
            hipLaunchKernelGGL(k_tile_emit, grid1d(n_seg), dim3(256), 0, s, spair, tflag, tpos, n_seg, cbits,
                               as<int32_t>(p->tile_rc), cnt_rb, cnt_cb);
        if (E > 0)
            hipLaunchKernelGGL(k_tile_mask, grid1d(E), dim3(256), 0, s, keys, vals, E, f, seg, spos, tflag, tpos,
                               as<uint64_t>(p->tile_mask), as<int32_t>(in_tile));
    }
    // residual CSR
    {
        int32_t *rflag = aux, *rpos = aux2;
        if (E > 0) hipLaunchKernelGGL(k_not, grid1d(E), dim3(256), 0, s, as<int32_t>(in_tile), E, rflag);
        TRY(scan_rec(rflag, rpos, E, tot + 3, scr, s));
        int32_t n_res = 0;
        TRY(read_i32(tot + 3, &n_res, 1, s));
        p->n_residual = n_res;
        TRY(dev_alloc(p->rindptr, (size_t)(n + 1) * 4));
        TRY(dev_alloc(p->rindices, (size_t)std::max(1, n_res) * 4));
        hipLaunchKernelGGL(k_res_emit, grid1d(std::max<int64_t>(E, n + 1)), dim3(256), 0, s, p->indptr, p->indices, n,
                           E, rflag, rpos, n_res, as<int32_t>(p->rindptr), as<int32_t>(p->rindices));
    }
    // per-block tile ranges and lists
    TRY(counts_to_ptr(cnt_rb, nb, p->tile_ptr, scr, s));
    TRY(counts_to_ptr(cnt_cb, nb, p->ctile_ptr, scr, s));
    if (nb > 0) hipLaunchKernelGGL(k_flag_pos, grid1d(nb), dim3(256), 0, s, cnt_rb, nb, nflag);
    TRY(compact(nflag, nb, p->trb, p->n_trb, npos, tot + 4, scr, s));
    if (n > 0)
        hipLaunchKernelGGL(k_flag_light_nt, grid1d(n), dim3(256), 0, s, p->indptr, (const int32_t *)nullptr, cnt_rb, n,
                           T, nflag);
    TRY(compact(nflag, n, p->light_nt, p->n_light_nt, npos, tot + 4, scr, s));
    // tiles ordered by (column block, row block): stable sort of (cb, tile id)
    {
        const int32_t nt = p->n_tiles;
        TRY(dev_alloc(p->ctile, (size_t)std::max(1, nt) * 4));
        if (nt > 0) {
            hipLaunchKernelGGL(k_ctile_keys, grid1d(nt), dim3(256), 0, s, as<int32_t>(p->tile_rc), nt, keys);
            TRY(radix_sort(keys, ktmp, nt, 32 + cbits, scr, s));
            hipLaunchKernelGGL(k_low32, grid1d(nt), dim3(256), 0, s, keys, nt, as<int32_t>(p->ctile));
        }
    }
    if (p->opts.want_csc) {
        if (nb > 0) hipLaunchKernelGGL(k_flag_pos, grid1d(nb), dim3(256), 0, s, cnt_cb, nb, nflag);
        TRY(compact(nflag, nb, p->tcb, p->n_tcb, npos, tot + 4, scr, s));
        if (n > 0)
            hipLaunchKernelGGL(k_flag_light_nt, grid1d(n), dim3(256), 0, s, (const int32_t *)nullptr, odeg, cnt_cb, n, T,
                               nflag);
        TRY(compact(nflag, n, p->c_light_nt, p->n_c_light_nt, npos, tot + 4, scr, s));
        TRY(build_transpose(as<int32_t>(p->rindptr), as<int32_t>(p->rindices), n, p->n_residual, p->rcindptr,
                            p->rcindices, s));
    }
    if (hipStreamSynchronize(s) != hipSuccess || hipGetLastError() != hipSuccess) {
        set_hip_error(hipErrorUnknown, "tile census");
        rc = GNN_ERR_HIP;
        goto done;
    }
    p->has_tiles = true;
done:
#undef TRY
    dev_free(seginfo);
    dev_free(in_tile);
    dev_free(S.b);
    return rc;
}

}  // namespace gnn
