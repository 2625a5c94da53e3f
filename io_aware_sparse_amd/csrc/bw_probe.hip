// Achievable-bandwidth reference for the roofline of the attention kernels.
//
// Standalone executable, not part of libgnn_attn.so. It times, with HIP
// events over 5 launches each, three access patterns on one GPU:
//   read    a grid-stride 16-byte-per-lane streaming read of 4 GiB, with
//           one load or four independent loads per lane in flight;
//   copy    a grid-stride copy of 2 GiB (read + write bytes counted);
//   gather  one wave per destination gathering 64 rows of R bytes each at
//           seeded random indices from a table of T bytes, R in {1024, 512,
//           256} and T from 64 MiB (held by the 256 MB Infinity Cache after
//           the first launch) to 4 GiB; the bytes counted are the rows and
//           the int32 indices. This is the access pattern of the light-node
//           kernels (a row of H*D elements per edge), without their arithmetic.
// Every index is below the table's row count and every table lies inside the
// 4 GiB buffer; it prints one line per measurement and "done".
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#define CHECK(x)                                                                     \
    do {                                                                             \
        hipError_t e_ = (x);                                                         \
        if (e_ != hipSuccess) {                                                      \
            std::printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
            std::exit(1);                                                            \
        }                                                                            \
    } while (0)

__global__ void k_read(const uint4 *__restrict__ a, int64_t n4, float *out) {
    float s = 0.f;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += (int64_t)gridDim.x * blockDim.x) {
        const uint4 v = a[i];
        s += __uint_as_float(v.x ^ v.y ^ v.z ^ v.w);
    }
    if (s == 12345.678f) out[0] = s;   // keeps the loads; never true for the fill used
}

// four independent loads per lane before any use
__global__ void k_read4(const uint4 *__restrict__ a, int64_t n4, float *out) {
    float s = 0.f;
    const int64_t st = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += 4 * st) {
        uint4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = i + u * st < n4 ? a[i + u * st] : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
        for (int u = 0; u < 4; ++u) s += __uint_as_float(v[u].x ^ v[u].y ^ v[u].z ^ v[u].w);
    }
    if (s == 12345.678f) out[0] = s;
}

__global__ void k_copy(const uint4 *__restrict__ a, uint4 *__restrict__ b, int64_t n4) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += (int64_t)gridDim.x * blockDim.x)
        b[i] = a[i];
}

// one wave per destination; lanes split a row of row4 16-byte words, 64/row4 rows per step, 4 steps in flight
__global__ void k_gather(const uint4 *__restrict__ tab, const int32_t *__restrict__ idx, int32_t nd, int deg,
                         int row4, float *out) {
    const int lane = threadIdx.x & 63;
    const int64_t wv = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    if (wv >= nd) return;
    const int per = 64 / row4;
    const int sub = lane / row4, c = lane % row4;
    float s = 0.f;
    for (int e = 0; e < deg; e += per * 4) {
        uint4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int k = e + u * per + sub;
            const int j = k < deg ? idx[wv * deg + k] : -1;
            v[u] = j >= 0 ? tab[(int64_t)j * row4 + c] : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) s += __uint_as_float(v[u].x ^ v[u].y ^ v[u].z ^ v[u].w);
    }
    if (s == 12345.678f) out[0] = s;
}

int main() {
    const int64_t bytes = 4ll << 30, n4 = bytes / 16;
    uint4 *a = nullptr, *b = nullptr;
    float *out = nullptr;
    CHECK(hipMalloc(&a, bytes));
    CHECK(hipMalloc(&b, bytes));
    CHECK(hipMalloc(&out, 64));
    CHECK(hipMemset(a, 1, bytes));
    CHECK(hipMemset(b, 0, bytes));
    hipEvent_t e0, e1;
    CHECK(hipEventCreate(&e0));
    CHECK(hipEventCreate(&e1));
    float ms = 0.f;
    for (int grid : {2048, 8192, 32768}) {
        for (int r = 0; r < 2; ++r) hipLaunchKernelGGL(k_read, dim3(grid), dim3(256), 0, 0, a, n4, out);
        CHECK(hipEventRecord(e0));
        for (int r = 0; r < 5; ++r) hipLaunchKernelGGL(k_read, dim3(grid), dim3(256), 0, 0, a, n4, out);
        CHECK(hipEventRecord(e1));
        CHECK(hipEventSynchronize(e1));
        CHECK(hipEventElapsedTime(&ms, e0, e1));
        std::printf("read 4 GiB, grid %d x 256: %.1f GB/s\n", grid, 5.0 * bytes / (ms * 1e-3) / 1e9);
        hipLaunchKernelGGL(k_read4, dim3(grid), dim3(256), 0, 0, a, n4, out);
        CHECK(hipEventRecord(e0));
        for (int r = 0; r < 5; ++r) hipLaunchKernelGGL(k_read4, dim3(grid), dim3(256), 0, 0, a, n4, out);
        CHECK(hipEventRecord(e1));
        CHECK(hipEventSynchronize(e1));
        CHECK(hipEventElapsedTime(&ms, e0, e1));
        std::printf("read 4 GiB, 4 loads per lane in flight, grid %d x 256: %.1f GB/s\n", grid,
                    5.0 * bytes / (ms * 1e-3) / 1e9);
        const int64_t h4 = n4 / 2;
        hipLaunchKernelGGL(k_copy, dim3(grid), dim3(256), 0, 0, a, b, h4);
        CHECK(hipEventRecord(e0));
        for (int r = 0; r < 5; ++r) hipLaunchKernelGGL(k_copy, dim3(grid), dim3(256), 0, 0, a, b, h4);
        CHECK(hipEventRecord(e1));
        CHECK(hipEventSynchronize(e1));
        CHECK(hipEventElapsedTime(&ms, e0, e1));
        std::printf("copy 2 GiB, grid %d x 256: %.1f GB/s (read + write)\n", grid,
                    5.0 * 2 * (h4 * 16) / (ms * 1e-3) / 1e9);
    }
    for (int row_bytes : {1024, 512, 256}) {
        const int row4 = row_bytes / 16;
        for (int64_t table_bytes : {64ll << 20, 256ll << 20, 1ll << 30, 4ll << 30}) {
            const int64_t n_rows = table_bytes / row_bytes;
            const int deg = 64;
            const int32_t nd = (int32_t)std::min<int64_t>(1 << 20, (3ll << 30) / row_bytes / deg);
            std::vector<int32_t> h((size_t)nd * deg);
            uint64_t x = 88172645463325252ull;   // xorshift64
            for (auto &v : h) {
                x ^= x << 13;
                x ^= x >> 7;
                x ^= x << 17;
                v = (int32_t)(x % (uint64_t)n_rows);
            }
            int32_t *idx = nullptr;
            CHECK(hipMalloc(&idx, h.size() * sizeof(int32_t)));
            CHECK(hipMemcpy(idx, h.data(), h.size() * sizeof(int32_t), hipMemcpyHostToDevice));
            const dim3 grid((unsigned)(((int64_t)nd * 64 + 255) / 256));
            hipLaunchKernelGGL(k_gather, grid, dim3(256), 0, 0, a, idx, nd, deg, row4, out);
            CHECK(hipEventRecord(e0));
            for (int r = 0; r < 5; ++r) hipLaunchKernelGGL(k_gather, grid, dim3(256), 0, 0, a, idx, nd, deg, row4, out);
            CHECK(hipEventRecord(e1));
            CHECK(hipEventSynchronize(e1));
            CHECK(hipEventElapsedTime(&ms, e0, e1));
            const double gb = 5.0 * ((double)nd * deg * (row_bytes + 4)) / 1e9;
            std::printf("gather %d-byte rows from a %lld MiB table, %d destinations x 64: %.1f GB/s\n", row_bytes,
                        (long long)(table_bytes >> 20), nd, gb / (ms * 1e-3));
            CHECK(hipFree(idx));
        }
    }
    CHECK(hipDeviceSynchronize());
    CHECK(hipFree(a));
    CHECK(hipFree(b));
    CHECK(hipFree(out));
    std::printf("done\n");
    return 0;
}
