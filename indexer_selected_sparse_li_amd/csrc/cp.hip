// Context-parallel helpers: the Zigzag partition of a sequence and the
// restoration of the original row order after the shards' results are
// gathered ("Day0 Inference Adaptation and Performance Optimization for a New
// Model", section 5.2; "Day0 Inference Adaptation and Performance
// Optimization for Kimi K3.1 Pro", section 5: GPU g of G takes the g-th
// segment from the head and the g-th from the tail of the sequence, so a
// short-history and a long-history segment share a GPU and the causal index
// work balances; the original order is restored afterwards).
//
// Segments: the sequence of n rows is cut into 2G segments, segment i =
// [start(i), start(i+1)) with start(i) = floor(i * n / 2G).  GPU g holds
// segment g followed by segment 2G-1-g; a gather of the shares in rank order
// therefore holds GPU 0's two segments, then GPU 1's, and so on.
#include "common.hpp"

namespace lisfa {

__host__ __device__ inline int64_t zz_start(int64_t i, int64_t n, int G) { return i * n / (2 * G); }

// Gathered index of original row t.  Rank g's block starts after ranks 0..g-1,
// whose segments are [start(0), start(g)) and [start(2G-g), n):
// base(g) = start(g) + n - start(2G - g).
__device__ inline int64_t zz_gathered_index(int64_t t, int64_t n, int G) {
    int64_t i = t * 2 * G / n;                       // segment guess, off by at most one
    if (i > 2 * G - 1) i = 2 * G - 1;
    while (i > 0 && zz_start(i, n, G) > t) --i;
    while (i < 2 * G - 1 && zz_start(i + 1, n, G) <= t) ++i;
    const int g = i < G ? (int)i : (int)(2 * G - 1 - i);
    const int64_t base = zz_start(g, n, G) + n - zz_start(2 * G - g, n, G);
    const int64_t s = zz_start(i, n, G);
    if (i < G) return base + (t - s);
    return base + (zz_start(g + 1, n, G) - zz_start(g, n, G)) + (t - s);
}

// dst row t = src row zz_gathered_index(t); rows of row_bytes bytes copied
// in units of U bytes (16, 4 or 1).  Block b handles rows b, b + gridDim.x, ...
template <int U>
__global__ __launch_bounds__(256) void zigzag_restore_kernel(const uint8_t* __restrict__ src,
                                                             uint8_t* __restrict__ dst, int64_t n, int G,
                                                             int64_t row_bytes) {
    typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
    const int64_t units = row_bytes / U;
    for (int64_t t = blockIdx.x; t < n; t += gridDim.x) {
        const int64_t gi = zz_gathered_index(t, n, G);
        const uint8_t* s = src + gi * row_bytes;
        uint8_t* d = dst + t * row_bytes;
        for (int64_t u = threadIdx.x; u < units; u += 256) {
            if constexpr (U == 16) ((u32x4v*)d)[u] = ((const u32x4v*)s)[u];
            else if constexpr (U == 4) ((uint32_t*)d)[u] = ((const uint32_t*)s)[u];
            else d[u] = s[u];
        }
    }
}

hipError_t zigzag_restore_dispatch(const void* src, void* dst, int64_t n, int G, int64_t row_bytes,
                                   hipStream_t stream) {
    if (n <= 0 || row_bytes <= 0) return hipSuccess;
    const unsigned grid = (unsigned)(n < 65536 ? n : 65536);
    const uintptr_t al = (uintptr_t)src | (uintptr_t)dst | (uintptr_t)row_bytes;
    if ((al & 15) == 0)
        hipLaunchKernelGGL(zigzag_restore_kernel<16>, dim3(grid), dim3(256), 0, stream, (const uint8_t*)src,
                           (uint8_t*)dst, n, G, row_bytes);
    else if ((al & 3) == 0)
        hipLaunchKernelGGL(zigzag_restore_kernel<4>, dim3(grid), dim3(256), 0, stream, (const uint8_t*)src,
                           (uint8_t*)dst, n, G, row_bytes);
    else
        hipLaunchKernelGGL(zigzag_restore_kernel<1>, dim3(grid), dim3(256), 0, stream, (const uint8_t*)src,
                           (uint8_t*)dst, n, G, row_bytes);
    return hipGetLastError();
}

void zigzag_share_ranges(int64_t n, int G, int g, int64_t* r4) {
    r4[0] = zz_start(g, n, G);
    r4[1] = zz_start(g + 1, n, G);
    r4[2] = zz_start(2 * G - 1 - g, n, G);
    r4[3] = zz_start(2 * G - g, n, G);
}

}  // namespace lisfa
