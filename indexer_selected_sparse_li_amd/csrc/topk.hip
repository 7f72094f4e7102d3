// Per-row Top-K selection by radix select ("Kimi New Model Open Source ...",
// section 3: Top-K position selection whose only output is the list of
// selected indices; "Large Language Model Inference Acceleration in
// Practice", section 3.1: Top-K on chip generating index pointers).
//
// One workgroup of 1024 threads (16 wavefronts) per query row.
//  1. Scores map to order-preserving uint32 keys (-0.0 folded onto +0.0).
//  2. A min/max reduction finds the highest bit on which the row's keys differ;
//     bits above it are common to every key and are skipped.
//  3. Radix select from that bit down in digits of at most 11 bits: an LDS
//     histogram of the keys that match the prefix chosen so far, then a
//     block-wide suffix scan locates the digit holding the K-th largest key.
//     At the end T is the K-th largest key and `need` is how many keys equal
//     to T are taken (the rest of the K are strictly greater than T).
//  4. Ordered emission: per 1024-position chunk, each wavefront's ballots of
//     "key > T" and "key == T" give counts; a block scan over (chunk, wave)
//     in position order gives every selected position its output slot, so
//     the list comes out ascending and ties at T go to the lowest positions.
// Every step is integer counting, so the result is deterministic.
#include "common.hpp"

namespace lisfa {

constexpr int kTkThreads = 1024;
constexpr int kTkWaves = kTkThreads / kWave;
constexpr int kTkSegChunks = kTkThreads / kTkWaves;  // chunks per emission segment (64)

// Exclusive block-wide scan of one value per thread; also returns the total.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* wsum, uint32_t& total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        uint32_t y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    if (wave == 0) {
        uint32_t t = lane < kTkWaves ? wsum[lane] : 0u;
#pragma unroll
        for (int o = 1; o < kTkWaves; o <<= 1) {
            uint32_t y = __shfl_up(t, o);
            if (lane >= o) t += y;
        }
        if (lane < kTkWaves) wsum[lane] = t;
    }
    __syncthreads();
    const uint32_t before = wave ? wsum[wave - 1] : 0u;
    total = wsum[kTkWaves - 1];
    __syncthreads();
    return before + x - v;
}

__global__ __launch_bounds__(kTkThreads) void topk_kernel(const float* __restrict__ scores, int64_t ld,
                                                          const int32_t* __restrict__ row_pos, int K,
                                                          int32_t* __restrict__ idx) {
    __shared__ uint32_t hist[2048];
    __shared__ uint32_t cnt_gt[kTkSegChunks * kTkWaves];
    __shared__ uint32_t cnt_eq[kTkSegChunks * kTkWaves];
    __shared__ uint32_t wsum[kTkWaves];
    __shared__ uint32_t red[2 * kTkWaves];
    __shared__ uint32_t sh_digit, sh_above;

    const int r = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int32_t* out = idx + (int64_t)r * K;
    int64_t n = (int64_t)row_pos[r] + 1;
    if (n < 0) n = 0;
    if (n > ld) n = ld;
    if (n <= K) {
        for (int64_t i = tid; i < K; i += kTkThreads) out[i] = i < n ? (int32_t)i : -1;
        return;
    }
    const float* s = scores + (int64_t)r * ld;

    // 2. min / max key
    uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
    for (int64_t i = tid; i < n; i += kTkThreads) {
        const uint32_t k = float_key(s[i]);
        kmin = k < kmin ? k : kmin;
        kmax = k > kmax ? k : kmax;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        uint32_t a = __shfl_xor(kmin, o), b = __shfl_xor(kmax, o);
        kmin = a < kmin ? a : kmin;
        kmax = b > kmax ? b : kmax;
    }
    if (lane == 0) {
        red[wave] = kmin;
        red[kTkWaves + wave] = kmax;
    }
    __syncthreads();
    kmin = red[0];
    kmax = red[kTkWaves];
#pragma unroll
    for (int w = 1; w < kTkWaves; ++w) {
        kmin = red[w] < kmin ? red[w] : kmin;
        kmax = red[kTkWaves + w] > kmax ? red[kTkWaves + w] : kmax;
    }

    // 3. radix select
    uint32_t need = (uint32_t)K;
    uint32_t T;
    const uint32_t diff = kmin ^ kmax;
    if (diff == 0u) {
        T = kmin;
    } else {
        int hi = 31 - __clz(diff);
        uint32_t prefix = hi == 31 ? 0u : (kmax & ~((2u << hi) - 1u));
        while (true) {
            const int lo = hi - 10 > 0 ? hi - 10 : 0;
            const uint32_t mask = (1u << (hi - lo + 1)) - 1u;
            hist[tid] = 0u;
            hist[tid + kTkThreads] = 0u;
            __syncthreads();
            for (int64_t i = tid; i < n; i += kTkThreads) {
                const uint32_t k = float_key(s[i]);
                const bool match = hi == 31 ? true : ((k ^ prefix) >> (hi + 1)) == 0u;
                if (match) atomicAdd(&hist[(k >> lo) & mask], 1u);
            }
            __syncthreads();
            // thread t owns bins 2047-2t (c1) and 2046-2t (c0), i.e. descending order
            const uint32_t c1 = hist[2047 - 2 * tid], c0 = hist[2046 - 2 * tid];
            uint32_t tot;
            const uint32_t E = block_excl_scan(c1 + c0, wsum, tot);
            if (E < need && need <= E + c1) {
                sh_digit = 2047u - 2u * tid;
                sh_above = E;
            } else if (E + c1 < need && need <= E + c1 + c0) {
                sh_digit = 2046u - 2u * tid;
                sh_above = E + c1;
            }
            __syncthreads();
            const uint32_t d = sh_digit;
            need -= sh_above;
            prefix |= d << lo;
            __syncthreads();
            if (lo == 0) break;
            hi = lo - 1;
        }
        T = prefix;
    }
    const uint32_t need_eq = need;

    // 4. ordered emission
    uint32_t base_gt = 0u, base_eq = 0u;
    const int64_t nch = (n + kTkThreads - 1) / kTkThreads;
    for (int64_t seg0 = 0; seg0 < nch; seg0 += kTkSegChunks) {
        const int segn = (int)((nch - seg0) < kTkSegChunks ? (nch - seg0) : kTkSegChunks);
        for (int c = 0; c < segn; ++c) {
            const int64_t i = (seg0 + c) * kTkThreads + tid;
            const bool v = i < n;
            const uint32_t k = v ? float_key(s[i]) : 0u;
            const uint64_t bg = __ballot(v && k > T);
            const uint64_t be = __ballot(v && k == T);
            if (lane == 0) {
                cnt_gt[c * kTkWaves + wave] = (uint32_t)__popcll(bg);
                cnt_eq[c * kTkWaves + wave] = (uint32_t)__popcll(be);
            }
        }
        __syncthreads();
        const bool own = tid < segn * kTkWaves;
        const uint32_t g = own ? cnt_gt[tid] : 0u, e = own ? cnt_eq[tid] : 0u;
        uint32_t tg, te;
        const uint32_t eg = block_excl_scan(g, wsum, tg);
        const uint32_t ee = block_excl_scan(e, wsum, te);
        if (own) {
            cnt_gt[tid] = eg + base_gt;
            cnt_eq[tid] = ee + base_eq;
        }
        base_gt += tg;
        base_eq += te;
        __syncthreads();
        for (int c = 0; c < segn; ++c) {
            const int64_t i = (seg0 + c) * kTkThreads + tid;
            const bool v = i < n;
            const uint32_t k = v ? float_key(s[i]) : 0u;
            const bool gt = v && k > T, eq = v && k == T;
            const uint64_t bg = __ballot(gt), be = __ballot(eq);
            const uint32_t rg = cnt_gt[c * kTkWaves + wave] + lanemask_count(bg);
            const uint32_t re = cnt_eq[c * kTkWaves + wave] + lanemask_count(be);
            if (gt) out[rg + (re < need_eq ? re : need_eq)] = (int32_t)i;
            else if (eq && re < need_eq) out[rg + re] = (int32_t)i;
        }
        __syncthreads();
    }
}

hipError_t topk_dispatch(const float* scores, int64_t ld, const int32_t* row_pos, int R, int K,
                         int32_t* idx, hipStream_t stream) {
    if (R <= 0) return hipSuccess;
    hipLaunchKernelGGL(topk_kernel, dim3((unsigned)R), dim3(kTkThreads), 0, stream, scores, ld, row_pos,
                       K, idx);
    return hipGetLastError();
}

}  // namespace lisfa
