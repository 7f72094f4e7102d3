// Per-row Top-K selection by radix select ("Kimi New Model Open Source ...",
// section 3: Top-K position selection whose only output is the list of
// selected indices; "Large Language Model Inference Acceleration in
// Practice", section 3.1: Top-K on chip generating index pointers).
//
// One workgroup of 1024 threads (16 wavefronts) per query row.
//  1. Scores map to order-preserving uint32 keys (-0.0 folded onto +0.0).
//  2. A min/max reduction gives the key range; selection then works on
//     d = key - kmin, whose top bit is that of the range.
//  3. Radix select on d from its top bit down in digits of at most 13 bits:
//     an LDS histogram of the values that match the prefix chosen so far,
//     then a block-wide suffix scan locates the digit holding the K-th
//     largest value (usually two levels for fp32 scores).
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
constexpr int kTkDigitBits = 13;                      // radix digit width
constexpr int kTkBins = 1 << kTkDigitBits;

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

// Keys come from registers (EPT > 0: element i = c * 1024 + tid lives in
// register c of thread tid, all loads issued up front) or are re-read from
// global memory on every pass (EPT == 0, rows longer than 64K positions).
template <int EPT>
__global__ __launch_bounds__(kTkThreads) void topk_kernel(const float* __restrict__ scores, int64_t ld,
                                                          const int32_t* __restrict__ row_pos, int K,
                                                          int32_t* __restrict__ idx) {
    __shared__ uint32_t hist[kTkBins];
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
    const int64_t nch = (n + kTkThreads - 1) / kTkThreads;

    // 1. keys (registers when they fit)
    constexpr int NR = EPT > 0 ? EPT : 1;
    uint32_t kr[NR];
    if constexpr (EPT > 0) {
#pragma unroll
        for (int c = 0; c < EPT; ++c) {
            const int64_t i = (int64_t)c * kTkThreads + tid;
            kr[c] = (c < nch && i < n) ? float_key(s[i]) : 0u;
        }
    }
    static_assert(EPT <= kTkSegChunks, "register rows must fit one emission segment");
    auto key_at = [&](int c, int64_t i) -> uint32_t {
        if constexpr (EPT > 0) return kr[c];
        else return float_key(s[i]);
    };
    auto for_each = [&](auto&& fn) {   // fn(c, i, key) over this thread's valid positions
        if constexpr (EPT > 0) {
#pragma unroll
            for (int c = 0; c < EPT; ++c) {
                const int64_t i = (int64_t)c * kTkThreads + tid;
                if (c < nch && i < n) fn(c, i, kr[c]);
            }
        } else {
            for (int64_t c = 0; c < nch; ++c) {
                const int64_t i = c * kTkThreads + tid;
                if (i < n) fn((int)c, i, float_key(s[i]));
            }
        }
    };

    // 2. min / max key
    uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
    for_each([&](int, int64_t, uint32_t k) {
        kmin = k < kmin ? k : kmin;
        kmax = k > kmax ? k : kmax;
    });
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

    // 3. radix select on d = key - kmin (a monotone map onto [0, kmax - kmin]):
    // starting the digits at the top bit of the range spreads the bulk of the
    // row over many bins (the top bits of the keys themselves may only split
    // the range into a handful of exponent bins).
    uint32_t need = (uint32_t)K;
    uint32_t T;
    const uint32_t range = kmax - kmin;
    if (range == 0u) {
        T = kmin;
    } else {
        int hi = 31 - __clz(range);
        uint32_t prefix = 0u;   // chosen high digits of d
        while (true) {
            const int lo = hi - (kTkDigitBits - 1) > 0 ? hi - (kTkDigitBits - 1) : 0;
            const uint32_t mask = (1u << (hi - lo + 1)) - 1u;
#pragma unroll
            for (int j = 0; j < kTkBins / kTkThreads; ++j) hist[tid + j * kTkThreads] = 0u;
            __syncthreads();
            for_each([&](int, int64_t, uint32_t k) {
                const uint32_t d = k - kmin;
                const bool match = hi == 31 ? true : ((d ^ prefix) >> (hi + 1)) == 0u;
                if (match) atomicAdd(&hist[(d >> lo) & mask], 1u);
            });
            __syncthreads();
            // thread t owns the kTkBins / 1024 consecutive bins counted from the top
            constexpr int PB = kTkBins / kTkThreads;
            uint32_t c[PB], loc = 0u;
#pragma unroll
            for (int j = 0; j < PB; ++j) {
                c[j] = hist[kTkBins - 1 - (tid * PB + j)];
                loc += c[j];
            }
            uint32_t tot;
            uint32_t E = block_excl_scan(loc, wsum, tot);
            if (E < need && need <= E + loc) {
#pragma unroll
                for (int j = 0; j < PB; ++j) {
                    if (E < need && need <= E + c[j]) {
                        sh_digit = (uint32_t)(kTkBins - 1 - (tid * PB + j));
                        sh_above = E;
                    }
                    E += c[j];
                }
            }
            __syncthreads();
            const uint32_t dg = sh_digit;
            need -= sh_above;
            prefix |= dg << lo;
            __syncthreads();
            if (lo == 0) break;
            hi = lo - 1;
        }
        T = kmin + prefix;
    }
    const uint32_t need_eq = need;

    // 4. ordered emission
    uint32_t base_gt = 0u, base_eq = 0u;
    for (int64_t seg0 = 0; seg0 < nch; seg0 += kTkSegChunks) {
        const int segn = (int)((nch - seg0) < kTkSegChunks ? (nch - seg0) : kTkSegChunks);
#pragma unroll
        for (int c = 0; c < (EPT > 0 ? (EPT < kTkSegChunks ? EPT : kTkSegChunks) : kTkSegChunks); ++c) {
            if (c >= segn) break;
            const int64_t i = (seg0 + c) * kTkThreads + tid;
            const bool v = i < n;
            const uint32_t k = v ? key_at(c, i) : 0u;  // EPT > 0: seg0 == 0 (one segment)
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
#pragma unroll
        for (int c = 0; c < (EPT > 0 ? (EPT < kTkSegChunks ? EPT : kTkSegChunks) : kTkSegChunks); ++c) {
            if (c >= segn) break;
            const int64_t i = (seg0 + c) * kTkThreads + tid;
            const bool v = i < n;
            const uint32_t k = v ? key_at(c, i) : 0u;  // EPT > 0: seg0 == 0 (one segment)
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
    // registers per thread needed for the longest possible row (ld)
    const int64_t ept = (ld + kTkThreads - 1) / kTkThreads;
#define LISFA_TK(E_)                                                                               \
    hipLaunchKernelGGL((topk_kernel<E_>), dim3((unsigned)R), dim3(kTkThreads), 0, stream, scores, ld, \
                       row_pos, K, idx)
    if (ept <= 8) LISFA_TK(8);
    else if (ept <= 16) LISFA_TK(16);
    else if (ept <= 32) LISFA_TK(32);
    else if (ept <= 64) LISFA_TK(64);
    else LISFA_TK(0);
#undef LISFA_TK
    return hipGetLastError();
}

}  // namespace lisfa
