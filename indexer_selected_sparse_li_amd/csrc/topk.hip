// Per-row Top-K selection by radix select ("Kimi New Model Open Source ...",
// section 3: Top-K position selection whose only output is the list of
// selected indices; "Large Language Model Inference Acceleration in
// Practice", section 3.1: Top-K on chip generating index pointers).
//
// Scores map to order-preserving uint32 keys (-0.0 folded onto +0.0; NaN
// above +inf).  The K largest keys of a row are selected; equal keys at the
// K-th place go to the lowest positions; the positions are written in
// ascending order.  Every step is integer counting, so the result is
// deterministic and the same on every path.
//  * topk_row_kernel (topk_select): one 1024-thread workgroup per row.  The
//    keys stay in registers (rows up to 64K positions; longer rows re-read
//    them from global memory).  One histogram of the first 12 bits of the
//    keys finds the bin holding the K-th largest key; only the keys in that
//    bin or above (a few thousand for K = 2048) move on, to LDS in position
//    order, where two 10-bit levels over that bin's keys fix the threshold
//    and one block scan orders the output.  A row with more candidates than
//    LDS holds (few distinct first digits near the K-th value) takes the
//    general selection: radix select from the top bit of the row's key range
//    (tk_select on registers, tk_row_global on global memory).
//  * topk_cand_kernel + topk_merge_kernel (context-parallel shards): slices of
//    a row keep their own Top-K as (position, score) pairs, a merge selects
//    the K best of the gathered pairs.  Every globally selected position is
//    among its own slice's Top-K, so the result is the same.
#include <type_traits>

#include "common.hpp"

namespace lisfa {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

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

// Inclusive scan / minimum / maximum within each row of 16 lanes (DPP row shifts).
__device__ __forceinline__ uint32_t row16_incl_sum(uint32_t x) {
    x += dpp<0x111, 0xF>(0u, x);
    x += dpp<0x112, 0xF>(0u, x);
    x += dpp<0x114, 0xF>(0u, x);
    x += dpp<0x118, 0xF>(0u, x);
    return x;
}

// Exclusive block-wide scans of two values per thread with one barrier: wave
// totals go to wsum[0 .. 15] and wsum[16 .. 31]; each wave then scans the 16
// totals across a row of its lanes and reads its own prefix from lane
// wave - 1.  The caller keeps wsum unwritten until a later barrier.
__device__ __forceinline__ void block_excl_scan2(uint32_t& a, uint32_t& b, uint32_t* wsum, uint32_t& ta, uint32_t& tb) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t xa = wave_incl_sum(a), xb = wave_incl_sum(b);
    if (lane == 63) {
        wsum[wave] = xa;
        wsum[kTkWaves + wave] = xb;
    }
    __syncthreads();
    const uint32_t sa = row16_incl_sum(wsum[lane & 15]), sb = row16_incl_sum(wsum[kTkWaves + (lane & 15)]);
    ta = (uint32_t)__builtin_amdgcn_readlane((int)sa, 15);
    tb = (uint32_t)__builtin_amdgcn_readlane((int)sb, 15);
    const uint32_t ba = wave > 0 ? (uint32_t)__builtin_amdgcn_readlane((int)sa, wave - 1) : 0u;
    const uint32_t bb = wave > 0 ? (uint32_t)__builtin_amdgcn_readlane((int)sb, wave - 1) : 0u;
    a = ba + xa - a;
    b = bb + xb - b;
}

// Exclusive block-wide scan of one 64-bit value per thread; also returns the total.
__device__ __forceinline__ uint64_t block_excl_scan64(uint64_t v, uint64_t* wsum, uint64_t& total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint64_t x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint64_t y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    if (wave == 0) {
        uint64_t t = lane < kTkWaves ? wsum[lane] : 0ull;
#pragma unroll
        for (int o = 1; o < kTkWaves; o <<= 1) {
            const uint64_t y = __shfl_up(t, o);
            if (lane >= o) t += y;
        }
        if (lane < kTkWaves) wsum[lane] = t;
    }
    __syncthreads();
    const uint64_t before = wave ? wsum[wave - 1] : 0ull;
    total = wsum[kTkWaves - 1];
    __syncthreads();
    return before + x - v;
}

constexpr int kTkCandMax = 2048;   // threshold-bin candidates kept in LDS

struct TkShared {
    uint32_t hist[kTkBins];
    uint32_t cand[kTkCandMax];
    uint64_t wsum64[kTkWaves];
    uint32_t wsum[kTkWaves];
    uint32_t red[2 * kTkWaves];
    uint32_t digit, above, ncand;
};

// Threshold of the selection core shared by the Top-K kernels.  The block
// holds keys kr[c] of thread t (list index t * EPT + c); valid(c) marks the
// valid ones (a prefix of the thread's keys, or a bit mask).  Finds T, the K-th largest valid key, and `need`, how many
// keys equal to T belong to the K largest (K < number of valid keys).
//  * min / max key, then radix select on d = key - kmin from the top bit of
//    the range in digits of at most 13 bits (LDS histogram + block scan).
//    The first level runs over all keys; once the bin holding the K-th value
//    has at most kTkCandMax keys, their d values move to LDS and the remaining
//    levels histogram only them.
template <int EPT, typename Valid>
__device__ __forceinline__ void tk_threshold(TkShared& sh, const uint32_t (&kr)[EPT], Valid&& valid, uint32_t K,
                                             uint32_t& T_out, uint32_t& need_out) {
    static_assert(EPT <= 64, "keys per thread");
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
    for (int c = 0; c < EPT; ++c) {
        if (valid(c)) {
            kmin = kr[c] < kmin ? kr[c] : kmin;
            kmax = kr[c] > kmax ? kr[c] : kmax;
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const uint32_t x = __shfl_xor(kmin, o), y = __shfl_xor(kmax, o);
        kmin = x < kmin ? x : kmin;
        kmax = y > kmax ? y : kmax;
    }
    if (lane == 0) {
        sh.red[wave] = kmin;
        sh.red[kTkWaves + wave] = kmax;
    }
    if (tid == 0) sh.ncand = 0u;
    __syncthreads();
    kmin = sh.red[0];
    kmax = sh.red[kTkWaves];
#pragma unroll
    for (int w = 1; w < kTkWaves; ++w) {
        kmin = sh.red[w] < kmin ? sh.red[w] : kmin;
        kmax = sh.red[kTkWaves + w] > kmax ? sh.red[kTkWaves + w] : kmax;
    }

    uint32_t need = K;
    uint32_t T;
    const uint32_t range = kmax - kmin;
    if (range == 0u) {
        T = kmin;
    } else {
        int hi = 31 - __clz(range);
        uint32_t prefix = 0u;       // chosen high digits of d
        bool compact = false;       // the remaining candidates are in sh.cand
        uint32_t ncand = 0u;
        while (true) {
            const int lo = hi - (kTkDigitBits - 1) > 0 ? hi - (kTkDigitBits - 1) : 0;
            const uint32_t mask = (1u << (hi - lo + 1)) - 1u;
#pragma unroll
            for (int j = 0; j < kTkBins / kTkThreads; ++j) sh.hist[tid + j * kTkThreads] = 0u;
            __syncthreads();
            if (!compact) {
#pragma unroll
                for (int c = 0; c < EPT; ++c) {
                    const uint32_t d = kr[c] - kmin;
                    const bool match = hi == 31 ? true : ((d ^ prefix) >> (hi + 1)) == 0u;
                    if (valid(c) && match) atomicAdd(&sh.hist[(d >> lo) & mask], 1u);
                }
            } else {
                for (uint32_t i = tid; i < ncand; i += kTkThreads) {
                    const uint32_t d = sh.cand[i];
                    if (((d ^ prefix) >> (hi + 1)) == 0u) atomicAdd(&sh.hist[(d >> lo) & mask], 1u);
                }
            }
            __syncthreads();
            // thread t owns the kTkBins / 1024 consecutive bins counted from the top
            constexpr int PB = kTkBins / kTkThreads;
            uint32_t cb[PB], loc = 0u;
#pragma unroll
            for (int j = 0; j < PB; ++j) {
                cb[j] = sh.hist[kTkBins - 1 - (tid * PB + j)];
                loc += cb[j];
            }
            uint32_t tot;
            uint32_t E = block_excl_scan(loc, sh.wsum, tot);
            if (E < need && need <= E + loc) {
#pragma unroll
                for (int j = 0; j < PB; ++j) {
                    if (E < need && need <= E + cb[j]) {
                        sh.digit = (uint32_t)(kTkBins - 1 - (tid * PB + j));
                        sh.above = E;
                    }
                    E += cb[j];
                }
            }
            __syncthreads();
            const uint32_t dg = sh.digit;
            const uint32_t inbin = sh.hist[dg];
            need -= sh.above;
            prefix |= dg << lo;
            if (lo == 0) break;
            // keys sharing all digits chosen so far: move them to LDS once few enough
            if (!compact && inbin <= (uint32_t)kTkCandMax) {
#pragma unroll
                for (int c = 0; c < EPT; ++c) {
                    const uint32_t d = kr[c] - kmin;
                    if (valid(c) && ((d ^ prefix) >> lo) == 0u) sh.cand[atomicAdd(&sh.ncand, 1u)] = d;
                }
                compact = true;
                ncand = inbin;
            }
            __syncthreads();
            if (compact && ncand <= 64u) {
                // at most 64 candidates left: one wavefront sorts them (bitonic,
                // descending, in registers) instead of further block-wide levels.
                // The need-th largest d is the threshold; the candidates strictly
                // above it are taken whole.
                if (wave == 0) {
                    const uint32_t d = (uint32_t)lane < ncand ? sh.cand[lane] : 0u;
                    const bool ok = (uint32_t)lane < ncand && ((d ^ prefix) >> lo) == 0u;
                    uint64_t x = ok ? ((1ull << 32) | d) : 0ull;
#pragma unroll
                    for (int k = 2; k <= 64; k <<= 1)
#pragma unroll
                        for (int j = k >> 1; j > 0; j >>= 1) {
                            const uint64_t y = ((uint64_t)(uint32_t)__shfl_xor((int)(x >> 32), j) << 32) |
                                               (uint32_t)__shfl_xor((int)(uint32_t)x, j);
                            const bool keep_max = ((lane & j) == 0) == ((lane & k) == 0);
                            x = keep_max ? (x > y ? x : y) : (x < y ? x : y);
                        }
                    const uint32_t v = (uint32_t)__shfl((int)(uint32_t)x, (int)need - 1);
                    const uint64_t gt = __ballot(ok && d > v);
                    if (lane == 0) {
                        sh.digit = v;
                        sh.above = (uint32_t)__popcll(gt);
                    }
                }
                __syncthreads();
                prefix = sh.digit;   // the full d of the threshold
                need -= sh.above;
                break;
            }
            hi = lo - 1;
        }
        T = kmin + prefix;
    }
    T_out = T;
    need_out = need;
}

// validity functors: the first nv keys of the thread, or the bits of a mask
struct TkPrefix {
    int nv;
    __device__ __forceinline__ bool operator()(int c) const { return c < nv; }
};
struct TkMask {
    uint64_t m;
    __device__ __forceinline__ bool operator()(int c) const { return (m >> c) & 1ull; }
};

// Selection core: the K largest valid keys, ties to the lower list index;
// calls emit(c, slot) for every selected key with its output slot (list
// order), for K < number of valid keys.  Emission: one block scan of each
// thread's (greater than T, equal to T) counts gives its first slot; equal
// keys are taken while their rank among equals is below `need`.
template <int EPT, typename Valid, typename Emit>
__device__ __forceinline__ void tk_select(TkShared& sh, const uint32_t (&kr)[EPT], Valid&& valid, uint32_t K,
                                          Emit&& emit) {
    uint32_t T, need_eq;
    tk_threshold<EPT>(sh, kr, valid, K, T, need_eq);
    uint64_t gtm = 0ull, eqm = 0ull;
#pragma unroll
    for (int c = 0; c < EPT; ++c) {
        if (valid(c)) {
            gtm |= (uint64_t)(kr[c] > T) << c;
            eqm |= (uint64_t)(kr[c] == T) << c;
        }
    }
    const uint64_t cnt = ((uint64_t)__popcll(eqm) << 32) | (uint64_t)__popcll(gtm);
    uint64_t total;
    const uint64_t ex = block_excl_scan64(cnt, sh.wsum64, total);
    uint32_t rg = (uint32_t)ex, re = (uint32_t)(ex >> 32);
#pragma unroll
    for (int c = 0; c < EPT; ++c) {
        const bool gt = (gtm >> c) & 1ull, eq = (eqm >> c) & 1ull;
        if (gt) {
            emit(c, rg + (re < need_eq ? re : need_eq));
            ++rg;
        } else if (eq) {
            if (re < need_eq) emit(c, rg + re);
            ++re;
        }
    }
}

// keys of positions [base, base + EPT) of row s (n valid positions in total)
template <int EPT>
__device__ __forceinline__ int tk_load(const float* s, bool vec, int64_t base, int64_t n, uint32_t (&kr)[EPT]) {
    const int nv = n - base >= EPT ? EPT : (n > base ? (int)(n - base) : 0);
    if (EPT % 4 == 0 && vec && nv == EPT) {
#pragma unroll
        for (int c = 0; c + 3 < EPT; c += 4) {
            const f32x4 v = *(const f32x4*)(s + base + c);
            kr[c] = float_key(v.x);
            kr[c + 1] = float_key(v.y);
            kr[c + 2] = float_key(v.z);
            kr[c + 3] = float_key(v.w);
        }
    } else {
#pragma unroll
        for (int c = 0; c < EPT; ++c) kr[c] = c < nv ? float_key(s[base + c]) : 0u;
    }
    return nv;
}

// visible positions of a row: row_pos + 1, clamped to [0, ld]
__device__ __forceinline__ int64_t tk_row_len(int32_t row_pos, int64_t ld) {
    int64_t n = (int64_t)row_pos + 1;
    if (n < 0) n = 0;
    if (n > ld) n = ld;
    return n;
}

__device__ __forceinline__ void tk_write_all(int32_t* out, int64_t n, int K) {
    for (int64_t i = threadIdx.x; i < K; i += kTkThreads) out[i] = i < n ? (int32_t)i : -1;
}

// The K largest of the n > K keys of one row by one workgroup, with the keys
// re-read from global memory on every pass (no workspace): min / max key, a
// radix select on d = key - kmin from the top bit of the range (digits of at
// most 13 bits; starting at the range's top bit spreads the row over many
// bins even when the keys share their exponent), then the ordered emission:
// per 1024-position chunk, wavefront ballots count the keys above and equal
// to the threshold, a block scan turns the counts into output slots.
__device__ void tk_row_global(TkShared& sh, const float* __restrict__ s, int64_t n, int K,
                              int32_t* __restrict__ out) {
    static_assert(2 * kTkSegChunks * kTkWaves <= kTkCandMax, "emission counts fit the candidate buffer");
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint32_t* cnt_gt = sh.cand;
    uint32_t* cnt_eq = sh.cand + kTkSegChunks * kTkWaves;
    const int64_t nch = (n + kTkThreads - 1) / kTkThreads;

    uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
    for (int64_t i = tid; i < n; i += kTkThreads) {
        const uint32_t k = float_key(s[i]);
        kmin = k < kmin ? k : kmin;
        kmax = k > kmax ? k : kmax;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const uint32_t a = __shfl_xor(kmin, o), b = __shfl_xor(kmax, o);
        kmin = a < kmin ? a : kmin;
        kmax = b > kmax ? b : kmax;
    }
    if (lane == 0) {
        sh.red[wave] = kmin;
        sh.red[kTkWaves + wave] = kmax;
    }
    __syncthreads();
    kmin = sh.red[0];
    kmax = sh.red[kTkWaves];
#pragma unroll
    for (int w = 1; w < kTkWaves; ++w) {
        kmin = sh.red[w] < kmin ? sh.red[w] : kmin;
        kmax = sh.red[kTkWaves + w] > kmax ? sh.red[kTkWaves + w] : kmax;
    }

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
            for (int j = 0; j < kTkBins / kTkThreads; ++j) sh.hist[tid + j * kTkThreads] = 0u;
            __syncthreads();
            for (int64_t i = tid; i < n; i += kTkThreads) {
                const uint32_t d = float_key(s[i]) - kmin;
                const bool match = hi == 31 ? true : ((d ^ prefix) >> (hi + 1)) == 0u;
                if (match) atomicAdd(&sh.hist[(d >> lo) & mask], 1u);
            }
            __syncthreads();
            // thread t owns the kTkBins / 1024 consecutive bins counted from the top
            constexpr int PB = kTkBins / kTkThreads;
            uint32_t c[PB], loc = 0u;
#pragma unroll
            for (int j = 0; j < PB; ++j) {
                c[j] = sh.hist[kTkBins - 1 - (tid * PB + j)];
                loc += c[j];
            }
            uint32_t tot;
            uint32_t E = block_excl_scan(loc, sh.wsum, tot);
            if (E < need && need <= E + loc) {
#pragma unroll
                for (int j = 0; j < PB; ++j) {
                    if (E < need && need <= E + c[j]) {
                        sh.digit = (uint32_t)(kTkBins - 1 - (tid * PB + j));
                        sh.above = E;
                    }
                    E += c[j];
                }
            }
            __syncthreads();
            const uint32_t dg = sh.digit;
            need -= sh.above;
            prefix |= dg << lo;
            __syncthreads();
            if (lo == 0) break;
            hi = lo - 1;
        }
        T = kmin + prefix;
    }
    const uint32_t need_eq = need;

    uint32_t base_gt = 0u, base_eq = 0u;
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
        const uint32_t eg = block_excl_scan(g, sh.wsum, tg);
        const uint32_t ee = block_excl_scan(e, sh.wsum, te);
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

// ------------------------------------------------- one workgroup per row ---

constexpr int kTkD1Bins = 4096;                         // first-digit bins
constexpr int kTkCandCap = 8192;                        // candidates kept in LDS
static_assert(kTkD1Bins == 4 * kTkThreads, "four first-digit bins per thread");

constexpr int kTkStageChunks = 8192;   // 16-byte chunks of a row staged in LDS at once (128 KB)

struct TkRowShared {
    uint32_t hist[kTkD1Bins];
    union {
        f32x4 stage[kTkStageChunks];   // the row on its way to the registers (kept until the bin keys are read)
        struct {
            int32_t pos[kTkCandCap];
            uint32_t key[kTkCandCap];
        } c;
        TkShared tk;   // the general selection, for rows with too many candidates
    } u;
    uint64_t wsum64[kTkWaves];
    uint32_t wsum[kTkWaves];
    alignas(16) uint32_t wsum2[2 * kTkWaves];
    uint32_t red[2 * kTkWaves];
    alignas(16) uint32_t binkey[kWave];   // d of the threshold bin's keys, when it holds at most 64
    uint32_t binown[kWave];               // their owners: thread * 32 + key index
    uint32_t own_gt[kTkThreads], own_eq[kTkThreads];   // per thread: its bin keys above / at the threshold
    uint32_t bin, above, nbin;
};

// m * 2 + (key > thr): the compare's lane mask is the add's carry-in, so a
// per-thread bit mask grows by one bit in two instructions (keys taken from the
// last to the first leave key c's bit at position c)
__device__ __forceinline__ uint32_t tk_push_gt(uint32_t m, uint32_t key, uint32_t thr) {
    asm volatile("v_cmp_gt_u32 vcc, %1, %2\n\tv_addc_co_u32 %0, vcc, %0, %0, vcc" : "+v"(m) : "v"(key), "v"(thr)
                 : "vcc");
    return m;
}

// x * 4 + c in one instruction (an LDS word address from an index)
__device__ __forceinline__ uint32_t tk_lshl2_add(uint32_t x, uint32_t c) {
    uint32_t r;
    asm("v_lshl_add_u32 %0, %1, 2, %2" : "=v"(r) : "v"(x), "v"(c));
    return r;
}

// LDS slot of staged chunk k, for runs of S = 2^L chunks a thread: the low 4
// bits of k are XORed with the 4 bits above the run index (bits L .. L+3), a
// GF(2)-linear bijection that keeps each group of 16 chunks in place.  The 16
// threads t0 .. t0+15 that read chunk t * S + j (fixed j) then hit 16 distinct
// 16-byte bank groups, and any 8 aligned ones of them 8 distinct 32-byte
// halves, where plain runs would be S-strided.
template <int S>
__device__ __forceinline__ int tk_slot(int k) {
    constexpr int L = S == 2 ? 1 : S == 4 ? 2 : S == 8 ? 3 : 4;
    return k ^ ((k >> L) & 15);
}
// inverse of tk_slot: y ^ N(y) ^ N(N(y)) ^ ... with N(y) = (y >> L) & 15,
// which vanishes after at most 4 steps
template <int S>
__device__ __forceinline__ int tk_chunk(int y) {
    constexpr int L = S == 2 ? 1 : S == 4 ? 2 : S == 8 ? 3 : 4;
    int k = y, x = y;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x = (x >> L) & 15;
        k ^= x;
    }
    return k;
}

// Keys of positions base .. base + EPT - 1 (base = tid * EPT) of a row whose
// floats are 16-byte aligned: the row's 16-byte chunks come in whole cache lines
// per wave instruction (direct-to-LDS loads; a thread-contiguous load from
// global memory touches 64 lines per instruction), up to 8192 chunks at a time,
// and each thread then reads its own run from LDS.  Chunks past the last valid
// position are not read from global memory (their lanes fetch chunk 0); keys
// past n are zero.  The caller's next barrier precedes any reuse of the stage.
template <int EPT>
__device__ __forceinline__ int tk_load_staged(const float* s, int64_t n, f32x4* stage, uint32_t (&kr)[EPT]) {
    constexpr int S = EPT / 4;
    constexpr int ROWCH = kTkThreads * S;
    constexpr int CH = ROWCH < kTkStageChunks ? ROWCH : kTkStageChunks;
    constexpr int NPH = ROWCH / CH;   // 1, or 2 for 64 keys a thread
    constexpr int TPP = CH / S;       // threads whose runs one phase holds
    static_assert(EPT % 4 == 0 && S <= 16 && ROWCH % CH == 0, "runs of 2..16 chunks");
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t base = (int64_t)tid * EPT;
    const int nv = n - base >= EPT ? EPT : (n > base ? (int)(n - base) : 0);
    const int nch = (int)((n + 3) >> 2), nch16 = (nch + 15) & ~15;
    const uint32_t lds_w = (uint32_t)(uintptr_t)stage + (uint32_t)(wave * kWave * 16);
#pragma unroll
    for (int ph = 0; ph < NPH; ++ph) {
        if (ph > 0) __syncthreads();   // the previous phase's runs are read
        const int c0 = ph * CH;
#pragma unroll
        for (int i = 0; i < CH / kTkThreads; ++i) {
            const int p0 = i * kTkThreads + wave * kWave;
            if (c0 + p0 < nch16) {   // wave-uniform: a group of 16 chunks maps onto itself
                const int k = c0 + tk_chunk<S>(p0 + lane);
                lds_dma<16, 0>(s + 4 * (int64_t)(k < nch ? k : 0), lds_w + (uint32_t)(i * kTkThreads * 16));
            }
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (NPH == 1 || tid / TPP == ph) {
            const int tl = tid - ph * TPP;
#pragma unroll
            for (int j = 0; j < S; ++j) {
                const f32x4 v = stage[tk_slot<S>(tl * S + j)];
                kr[4 * j] = float_key(v.x);
                kr[4 * j + 1] = float_key(v.y);
                kr[4 * j + 2] = float_key(v.z);
                kr[4 * j + 3] = float_key(v.w);
            }
        }
    }
#pragma unroll
    for (int c = 0; c < EPT; ++c) kr[c] = c < nv ? kr[c] : 0u;
    return nv;
}

template <int EPT>
using TkBits = typename std::conditional<(EPT <= 32), uint32_t, uint64_t>::type;

// Ordered emission from per-thread masks: every key in gtm, and of the keys in
// eqm the first need_eq in list order (thread t's keys c are list entries
// t * EPT + c).  One block scan of the per-thread counts; the stores are
// bounded by K.
template <int EPT, class Emit>
__device__ __forceinline__ void tk_emit_masks(TkRowShared& sh, TkBits<EPT> gtm, TkBits<EPT> eqm, uint32_t need_eq,
                                              uint32_t K, Emit& emit) {
    using M = TkBits<EPT>;
    uint32_t rg = (uint32_t)__builtin_popcountll(gtm), re = (uint32_t)__builtin_popcountll(eqm), tg, te;
    block_excl_scan2(rg, re, sh.wsum2, tg, te);
    // a loop over set bits: only the list index is needed
    M m = gtm | eqm;
    while (m != (M)0) {
        const int c = (int)__builtin_ctzll((uint64_t)m);
        m &= m - (M)1;
        if ((gtm >> c) & (M)1) {
            const uint32_t o = rg + (re < need_eq ? re : need_eq);
            if (o < K) emit(c, o);   // always true; bounds the store
            ++rg;
        } else {
            if (re < need_eq && rg + re < K) emit(c, rg + re);
            ++re;
        }
    }
}

// The K largest of the valid keys held by a workgroup, in registers: thread t
// holds list entries t * EPT + c as keys kr[c] (float_key order; invalid
// entries are 0, below every key of a float), valid(c) tells them apart and
// `full` says that all EPT are valid (the passes then skip the test).  More
// than K entries are valid.  Larger keys win, equal keys go to the lower list
// index; the selected entries come out in list order through
// emit(c, slot) (by the owning thread) or emit_list(slot, list index) (any
// thread), and `fallback` takes over when bin B holds too many candidates.
// stf: the workgroup's floats staged in LDS (tk_load_staged layout), or null.
//  1. min and max key;
//  2. a histogram of the first digit (key >> s) - (kmin >> s), with s the
//     smallest shift that keeps the row below 4096 bins, and the bin B
//     holding the K-th largest key: the keys with a larger digit are selected;
//  3'. bin B with at most 64 keys (or one value): its keys go to LDS with
//     their owners, one wavefront ranks them, finds the threshold and sets
//     the owners' bits; then the emission straight from the registers;
//  3. otherwise the C keys with digit >= B move to LDS in list order, 10-bit
//     digits of their remaining bits fix the threshold, and the emission
//     walks the list.
template <int EPT, class Valid, class Emit, class EmitList, class Fallback>
__device__ __forceinline__ void tk_block_topk(TkRowShared& sh, const uint32_t (&kr)[EPT], Valid valid, bool full,
                                              const float* stf, uint32_t K, Emit emit, EmitList emit_list,
                                              Fallback fallback) {
    using M = TkBits<EPT>;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    // 1. min and max.  Every pass over the keys has a copy without the per-key
    // validity test for the threads whose keys are all valid.
    uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
    if (full) {
#pragma unroll
        for (int c = 0; c < EPT; ++c) {
            kmin = kr[c] < kmin ? kr[c] : kmin;
            kmax = kr[c] > kmax ? kr[c] : kmax;
        }
    } else {
#pragma unroll
        for (int c = 0; c < EPT; ++c) {
            if (valid(c)) {
                kmin = kr[c] < kmin ? kr[c] : kmin;
                kmax = kr[c] > kmax ? kr[c] : kmax;
            }
        }
    }
    kmin = wave_incl_min(kmin);
    kmax = wave_incl_max(kmax);
    if (lane == 63) {
        sh.red[wave] = kmin;
        sh.red[kTkWaves + wave] = kmax;
    }
    *(u32x4*)&sh.hist[4 * tid] = u32x4{0u, 0u, 0u, 0u};
    if (tid == 0) sh.nbin = 0u;
    __syncthreads();
    if constexpr (EPT == 64) {   // (fewer live registers)
        const u32x4* rm = (const u32x4*)sh.red;
#pragma unroll
        for (int q = 0; q < kTkWaves / 4; ++q) {
            const u32x4 a = rm[q], b = rm[kTkWaves / 4 + q];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                kmin = a[e] < kmin ? a[e] : kmin;
                kmax = b[e] > kmax ? b[e] : kmax;
            }
        }
    } else {
        // the 16 wave results across a row of lanes, reduced by DPP; lane 15 has the block's
        uint32_t vmin = sh.red[lane & 15], vmax = sh.red[kTkWaves + (lane & 15)];
        vmin = min(vmin, dpp<0x111, 0xF>(~0u, vmin));
        vmax = max(vmax, dpp<0x111, 0xF>(0u, vmax));
        vmin = min(vmin, dpp<0x112, 0xF>(~0u, vmin));
        vmax = max(vmax, dpp<0x112, 0xF>(0u, vmax));
        vmin = min(vmin, dpp<0x114, 0xF>(~0u, vmin));
        vmax = max(vmax, dpp<0x114, 0xF>(0u, vmax));
        vmin = min(vmin, dpp<0x118, 0xF>(~0u, vmin));
        vmax = max(vmax, dpp<0x118, 0xF>(0u, vmax));
        kmin = (uint32_t)__builtin_amdgcn_readlane((int)vmin, 15);
        kmax = (uint32_t)__builtin_amdgcn_readlane((int)vmax, 15);
    }
    const uint32_t range = kmax - kmin;
    if (range == 0u) {   // every valid key equal: the first K valid entries
        M vm = (M)0;
#pragma unroll
        for (int c = 0; c < EPT; ++c) vm |= (M)valid(c) << c;
        tk_emit_masks<EPT>(sh, (M)0, vm, K, K, emit);
        return;
    }
    // first digit of a key: (key >> sh1) - (kmin >> sh1) = d >> sh1 with
    // d = key - kb, kb = kmin with its low sh1 bits cleared; sh1 is the
    // smallest shift that keeps the digit below 4096
    const int top = 31 - __clz(range);
    int sh1 = top >= 11 ? top - 11 : 0;
    if ((kmax >> sh1) - (kmin >> sh1) >= (uint32_t)kTkD1Bins) ++sh1;
    const uint32_t kb = (kmin >> sh1) << sh1;

    // 2. first-digit histogram; thread t owns bins 4095 - 4t - j (j < 4), top first
    if (full) {
        const uint32_t hb = (uint32_t)(uintptr_t)sh.hist - ((kb >> sh1) << 2);
#pragma unroll
        for (int c = 0; c < EPT; ++c)
            __hip_atomic_fetch_add((lds_u32*)(uintptr_t)tk_lshl2_add(kr[c] >> sh1, hb), 1u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_WORKGROUP);
    } else {
#pragma unroll
        for (int c = 0; c < EPT; ++c)
            if (valid(c)) atomicAdd(&sh.hist[(kr[c] - kb) >> sh1], 1u);
    }
    __syncthreads();
    {
        uint32_t cb[4], loc = 0u;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            cb[j] = sh.hist[kTkD1Bins - 1 - (4 * tid + j)];
            loc += cb[j];
        }
        uint32_t E = loc, dummy = 0u, tot, tot2;
        block_excl_scan2(E, dummy, sh.wsum2, tot, tot2);
        if (E < K && K <= E + loc) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (E < K && K <= E + cb[j]) {
                    sh.bin = (uint32_t)(kTkD1Bins - 1 - (4 * tid + j));
                    sh.above = E;
                }
                E += cb[j];
            }
        }
        __syncthreads();
    }
    const uint32_t bin = sh.bin, above = sh.above;
    const uint32_t inbin = sh.hist[bin];
    const uint32_t C = above + inbin;
    uint32_t need = K - above;   // taken from bin B, >= 1

    if (sh1 == 0 || inbin <= (uint32_t)kWave) {
        // 3'. small threshold bin (at most 64 keys, or one value when sh1 = 0)
        if constexpr (EPT <= 32) {
            // one pass marks the keys above bin B (above_m) and in it (bin_m)
            // bin B's valid keys lie in [max(Kb, kmin), Khi]; the invalid keys (0) below kmin
            const uint32_t Kb = kb + (bin << sh1);
            const uint32_t Klo = Kb > kmin ? Kb : kmin;
            const uint64_t hi = (uint64_t)Kb + ((uint64_t)1 << sh1) - 1u;
            const uint32_t Khi = hi > 0xFFFFFFFFull ? 0xFFFFFFFFu : (uint32_t)hi;
            uint32_t above_m = 0u, bin_m = 0u;
#pragma unroll
            for (int c = EPT - 1; c >= 0; --c) {
                above_m = tk_push_gt(above_m, kr[c], Khi);
                bin_m = tk_push_gt(bin_m, kr[c], Klo - 1u);
            }
            bin_m &= ~above_m;
            if (sh1 > 0) {
                if (bin_m != 0u) {
                    sh.own_gt[tid] = 0u;
                    sh.own_eq[tid] = 0u;
                    // the few bin keys with their owners to LDS: from the staged
                    // floats when there are some (registers cannot be indexed at run time)
                    for (uint32_t m = bin_m; m != 0u; m &= m - 1u) {
                        const int c = __builtin_ctz(m);
                        uint32_t key = 0u;
                        if (stf) {
                            key = float_key(stf[tk_slot<EPT / 4>(tid * (EPT / 4) + (c >> 2)) * 4 + (c & 3)]);
                        } else {
#pragma unroll
                            for (int cc = 0; cc < EPT; ++cc) key = cc == c ? kr[cc] : key;
                        }
                        const uint32_t slot = atomicAdd(&sh.nbin, 1u);
                        sh.binkey[slot] = key;
                        sh.binown[slot] = ((uint32_t)tid << 5) | (uint32_t)c;
                    }
                }
                __syncthreads();
                if (wave == 0) {
                    // the need-th largest key of the bin is every key with
                    // #greater < need <= #greater-or-equal
                    const bool ok = (uint32_t)lane < inbin;
                    const uint32_t d = ok ? sh.binkey[lane] : 0u;
                    uint32_t gt = 0u, ge = 0u;
#pragma unroll 1
                    for (uint32_t j = 0; j < inbin; j += 4) {
                        const uint4 o = *reinterpret_cast<const uint4*>(&sh.binkey[j]);
                        gt += (o.x > d) + (j + 1 < inbin && o.y > d) + (j + 2 < inbin && o.z > d) +
                              (j + 3 < inbin && o.w > d);
                        ge += (o.x >= d) + (j + 1 < inbin && o.y >= d) + (j + 2 < inbin && o.z >= d) +
                              (j + 3 < inbin && o.w >= d);
                    }
                    const uint64_t hit = __ballot(ok && gt < need && need <= ge);
                    const uint32_t dT = (uint32_t)__shfl((int)d, (int)__builtin_ctzll(hit));
                    const uint64_t gtb = __ballot(ok && d > dT);
                    if (ok && d >= dT) {
                        const uint32_t ow = sh.binown[lane];
                        atomicOr(d > dT ? &sh.own_gt[ow >> 5] : &sh.own_eq[ow >> 5], 1u << (ow & 31u));
                    }
                    if (lane == 0) sh.above = (uint32_t)__popcll(gtb);
                }
                __syncthreads();
                need -= sh.above;
                above_m |= sh.own_gt[tid] & bin_m;
                bin_m &= sh.own_eq[tid];
            }
            tk_emit_masks<EPT>(sh, above_m, bin_m, need, K, emit);
        } else {
            // 64 keys a thread: bin B's keys go to LDS, one wavefront ranks them,
            // a second pass takes the masks (fewer live registers)
            uint32_t T = kb + bin;   // sh1 = 0: every key of bin B is kb + B
            if (sh1 > 0) {
#pragma unroll
                for (int c = 0; c < EPT; ++c)
                    if (valid(c) && ((kr[c] - kb) >> sh1) == bin) sh.binkey[atomicAdd(&sh.nbin, 1u)] = kr[c];
                __syncthreads();
                if (wave == 0) {
                    const bool ok = (uint32_t)lane < inbin;
                    const uint32_t d = ok ? sh.binkey[lane] : 0u;
                    uint32_t gt = 0u, ge = 0u;
#pragma unroll 1
                    for (uint32_t j = 0; j < inbin; j += 4) {
                        const uint4 o = *reinterpret_cast<const uint4*>(&sh.binkey[j]);
                        gt += (o.x > d) + (j + 1 < inbin && o.y > d) + (j + 2 < inbin && o.z > d) +
                              (j + 3 < inbin && o.w > d);
                        ge += (o.x >= d) + (j + 1 < inbin && o.y >= d) + (j + 2 < inbin && o.z >= d) +
                              (j + 3 < inbin && o.w >= d);
                    }
                    const uint64_t hit = __ballot(ok && gt < need && need <= ge);
                    const uint32_t v = (uint32_t)__shfl((int)d, (int)__builtin_ctzll(hit));
                    const uint64_t gtb = __ballot(ok && d > v);
                    if (lane == 0) {
                        sh.bin = v;
                        sh.above = (uint32_t)__popcll(gtb);
                    }
                }
                __syncthreads();
                T = sh.bin;
                need -= sh.above;
            }
            // invalid keys (0) lie below kmin <= T
            uint32_t g0 = 0u, g1 = 0u, e0 = 0u, e1 = 0u;
#pragma unroll
            for (int c = EPT / 2 - 1; c >= 0; --c) {
                g0 = tk_push_gt(g0, kr[c], T);
                e0 = tk_push_gt(e0, kr[c], T - 1u);
                g1 = tk_push_gt(g1, kr[c + EPT / 2], T);
                e1 = tk_push_gt(e1, kr[c + EPT / 2], T - 1u);
            }
            const uint64_t gtm = ((uint64_t)g1 << 32) | g0;
            const uint64_t eqm = (((uint64_t)e1 << 32) | e0) & ~gtm;
            tk_emit_masks<EPT>(sh, gtm, eqm, need, K, emit);
        }
        return;
    }
    if (C > (uint32_t)kTkCandCap) {
        fallback();
        return;
    }

    // 3. candidates (list index, d) to LDS in list order
    {
        uint64_t fm = 0ull;
#pragma unroll
        for (int c = 0; c < EPT; ++c) fm |= (uint64_t)(valid(c) && ((kr[c] - kb) >> sh1) >= bin) << c;
        uint32_t at = (uint32_t)__popcll(fm), dummy = 0u, tot, tot2;
        block_excl_scan2(at, dummy, sh.wsum2, tot, tot2);
#pragma unroll
        for (int c = 0; c < EPT; ++c) {
            if ((fm >> c) & 1ull) {
                sh.u.c.pos[at] = (int32_t)(tid * EPT + c);
                sh.u.c.key[at] = kr[c] - kb;
                ++at;
            }
        }
    }
    __syncthreads();

    // 4. the remaining sh1 bits of d, 10 at a time, over bin B's candidates
    uint32_t prefix = bin;
    for (int hi = sh1; hi > 0;) {
        const int w = hi < 10 ? hi : 10, lo = hi - w;
        const uint32_t nb = 1u << w;
        sh.hist[tid] = 0u;
        __syncthreads();
        for (uint32_t i = tid; i < C; i += kTkThreads) {
            const uint32_t d = sh.u.c.key[i];
            if ((d >> hi) == prefix) atomicAdd(&sh.hist[(d >> lo) & (nb - 1u)], 1u);
        }
        __syncthreads();
        const uint32_t cb = (uint32_t)tid < nb ? sh.hist[nb - 1u - tid] : 0u;
        uint32_t E = cb, dummy = 0u, tot, tot2;
        block_excl_scan2(E, dummy, sh.wsum2, tot, tot2);
        if (E < need && need <= E + cb) {
            sh.bin = nb - 1u - (uint32_t)tid;
            sh.above = E;
        }
        __syncthreads();
        prefix = (prefix << w) | sh.bin;
        need -= sh.above;
        __syncthreads();
        hi = lo;
    }
    const uint32_t T = prefix, need_eq = need;   // threshold d

    // 5. ordered emission: thread t takes list entries [t * E2, t * E2 + E2)
    const uint32_t E2 = (C + kTkThreads - 1) / kTkThreads;   // <= 8
    const uint32_t b0 = (uint32_t)tid * E2;
    uint32_t rg = 0u, re = 0u;
    for (uint32_t j = 0; j < E2; ++j) {
        const uint32_t i = b0 + j;
        if (i < C) {
            const uint32_t d = sh.u.c.key[i];
            rg += d > T;
            re += d == T;
        }
    }
    uint32_t tg, te;
    block_excl_scan2(rg, re, sh.wsum2, tg, te);
    for (uint32_t j = 0; j < E2; ++j) {
        const uint32_t i = b0 + j;
        if (i < C) {
            const uint32_t d = sh.u.c.key[i];
            if (d > T) {
                const uint32_t o = rg + (re < need_eq ? re : need_eq);
                if (o < K) emit_list(o, (uint32_t)sh.u.c.pos[i]);
                ++rg;
            } else if (d == T) {
                if (re < need_eq && rg + re < K) emit_list(rg + re, (uint32_t)sh.u.c.pos[i]);
                ++re;
            }
        }
    }
}

// Top-K of one row per workgroup (n > K visible positions), the row's keys in
// registers (16-byte aligned rows come through the LDS stage); rows whose
// threshold bin holds more than kTkCandCap candidates take the general
// selection on global memory.
template <int EPT>
__global__ __launch_bounds__(kTkThreads) void topk_row_kernel(const float* __restrict__ scores, int64_t ld,
                                                              const int32_t* __restrict__ row_pos, int K,
                                                              int32_t* __restrict__ idx) {
    __shared__ TkRowShared sh;
    const int r = blockIdx.x, tid = threadIdx.x;
    const int64_t n = tk_row_len(row_pos[r], ld);
    int32_t* out = idx + (int64_t)r * K;
    if (n <= K) {
        tk_write_all(out, n, K);
        return;
    }
    const float* s = scores + (int64_t)r * ld;
    uint32_t kr[EPT];
    const int64_t base = (int64_t)tid * EPT;
    const bool vec = ((ld & 3) == 0) && ((((uintptr_t)scores) & 15) == 0);
    const int nv = vec ? tk_load_staged<EPT>(s, n, sh.u.stage, kr) : tk_load<EPT>(s, false, base, n, kr);
    tk_block_topk<EPT>(
        sh, kr, TkPrefix{nv}, nv == EPT, (vec && EPT <= 32) ? (const float*)sh.u.stage : nullptr, (uint32_t)K,
        [&](int c, uint32_t o) { out[o] = (int32_t)(base + c); },
        [&](uint32_t o, uint32_t li) { out[o] = (int32_t)li; },
        [&]() { tk_row_global(sh.u.tk, s, n, K, out); });
}

// One workgroup per row with the keys re-read from global memory: rows
// longer than 64K positions when no workspace is given.
__global__ __launch_bounds__(kTkThreads) void topk_stream_kernel(const float* __restrict__ scores, int64_t ld,
                                                                 const int32_t* __restrict__ row_pos, int K,
                                                                 int32_t* __restrict__ idx) {
    __shared__ TkShared sh;
    const int r = blockIdx.x;
    const int64_t n = tk_row_len(row_pos[r], ld);
    int32_t* out = idx + (int64_t)r * K;
    if (n <= K) {
        tk_write_all(out, n, K);
        return;
    }
    tk_row_global(sh, scores + (int64_t)r * ld, n, K, out);
}

// Local Top-K of slices: workgroup (s, r) selects among positions
// [s * SL, s * SL + SL) of row r's visible range (SL = 1024 * EPT) and writes
// min(K, count) (position + pos_offset[r], score) pairs, positions ascending,
// padded with (-1, -inf), to candidate block (r, s) of S per row.  With one
// slice per row this is the local Top-K of a context shard; with several it
// is the first pass of the selection of rows too long for one workgroup.
template <int EPT>
__global__ __launch_bounds__(kTkThreads) void topk_cand_kernel(const float* __restrict__ scores, int64_t ld,
                                                               const int32_t* __restrict__ row_pos, int K, int S,
                                                               const int32_t* __restrict__ pos_offset,
                                                               int32_t* __restrict__ cand_pos,
                                                               float* __restrict__ cand_score) {
    __shared__ TkRowShared sh;
    const int sl = blockIdx.x, r = blockIdx.y, tid = threadIdx.x;
    int64_t n = (int64_t)row_pos[r] + 1;
    if (n < 0) n = 0;
    if (n > ld) n = ld;
    const int64_t lo = (int64_t)sl * kTkThreads * EPT;
    int64_t cnt = n - lo;
    if (cnt < 0) cnt = 0;
    if (cnt > (int64_t)kTkThreads * EPT) cnt = (int64_t)kTkThreads * EPT;
    const int32_t off = pos_offset ? pos_offset[r] : 0;
    int32_t* op = cand_pos + ((int64_t)r * S + sl) * K;
    float* os = cand_score + ((int64_t)r * S + sl) * K;
    const float* s = scores + (int64_t)r * ld + lo;   // the slice
    if (cnt <= K) {
        for (int64_t i = tid; i < K; i += kTkThreads) {
            const bool v = i < cnt;
            op[i] = v ? (int32_t)(lo + i + off) : -1;
            os[i] = v ? s[i] : -__builtin_inff();
        }
        return;
    }
    const bool vec = ((ld & 3) == 0) && ((((uintptr_t)scores) & 15) == 0);   // lo is a multiple of 4
    const int64_t base = (int64_t)tid * EPT;
    uint32_t kr[EPT];
    const int nv = vec ? tk_load_staged<EPT>(s, cnt, sh.u.stage, kr) : tk_load<EPT>(s, false, base, cnt, kr);
    auto put = [&](int64_t li, uint32_t o) {
        op[o] = (int32_t)(lo + li + off);
        os[o] = s[li];
    };
    tk_block_topk<EPT>(
        sh, kr, TkPrefix{nv}, nv == EPT, (vec && EPT <= 32) ? (const float*)sh.u.stage : nullptr, (uint32_t)K,
        [&](int c, uint32_t o) { put(base + c, o); }, [&](uint32_t o, uint32_t li) { put(li, o); },
        [&]() { tk_select<EPT>(sh.u.tk, kr, TkPrefix{nv}, (uint32_t)K, [&](int c, uint32_t o) { put(base + c, o); }); });
}

// Ordered merge (the valid candidates of a row in ascending position order,
// so list order settles ties): the K best of n (position, score) pairs,
// position < 0 = none, out in list order, -1 padded.
template <int EPT>
__global__ __launch_bounds__(kTkThreads) void topk_merge_ordered_kernel(const float* __restrict__ cand_score,
                                                                        const int32_t* __restrict__ cand_pos,
                                                                        int64_t ldc, int n, int K,
                                                                        int32_t* __restrict__ idx,
                                                                        float* __restrict__ idx_score) {
    __shared__ TkRowShared sh;
    const int r = blockIdx.x, tid = threadIdx.x;
    const float* cs = cand_score + (int64_t)r * ldc;
    const int32_t* cp = cand_pos + (int64_t)r * ldc;
    int32_t* out = idx + (int64_t)r * K;
    float* outs = idx_score ? idx_score + (int64_t)r * K : nullptr;
    const int base = tid * EPT;
    uint32_t kr[EPT];
    int32_t pr[EPT];
    uint64_t vm = 0ull;
    // 16-byte loads when this thread's candidates are whole and aligned
    const bool vec = EPT % 4 == 0 && (ldc & 3) == 0 && base + EPT <= n &&
                     ((((uintptr_t)cand_score) | ((uintptr_t)cand_pos)) & 15) == 0;
    if (vec) {
#pragma unroll
        for (int c = 0; c < EPT; c += 4) {
            const i32x4 p4 = *(const i32x4*)(cp + base + c);
            const f32x4 s4 = *(const f32x4*)(cs + base + c);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                pr[c + e] = p4[e];
                kr[c + e] = p4[e] >= 0 ? float_key(s4[e]) : 0u;
                vm |= (uint64_t)(p4[e] >= 0) << (c + e);
            }
        }
    } else {
#pragma unroll
        for (int c = 0; c < EPT; ++c) {
            const int i = base + c;
            const int32_t p = i < n ? cp[i] : -1;
            pr[c] = p;
            kr[c] = p >= 0 ? float_key(cs[i]) : 0u;
            vm |= (uint64_t)(p >= 0) << c;
        }
    }
    uint32_t first = (uint32_t)__popcll(vm), dummy = 0u, nvalid, tot2;
    block_excl_scan2(first, dummy, sh.wsum2, nvalid, tot2);
    if (nvalid <= (uint32_t)K) {
#pragma unroll
        for (int c = 0; c < EPT; ++c) {
            if ((vm >> c) & 1ull) {
                out[first] = pr[c];
                if (outs) outs[first] = cs[base + c];
                ++first;
            }
        }
        for (int i = (int)nvalid + tid; i < K; i += kTkThreads) {
            out[i] = -1;
            if (outs) outs[i] = -__builtin_inff();
        }
        return;
    }
    __syncthreads();   // wsum2 is read above and written again below
    constexpr uint64_t all = EPT == 64 ? ~0ull : ((1ull << EPT) - 1ull);
    tk_block_topk<EPT>(
        sh, kr, TkMask{vm}, vm == all, nullptr, (uint32_t)K,
        [&](int c, uint32_t o) {
            out[o] = pr[c];
            if (outs) outs[o] = cs[base + c];
        },
        [&](uint32_t o, uint32_t li) {
            out[o] = cp[li];
            if (outs) outs[o] = cs[li];
        },
        [&]() {
            tk_select<EPT>(sh.u.tk, kr, TkMask{vm}, (uint32_t)K, [&](int c, uint32_t o) {
                out[o] = pr[c];
                if (outs) outs[o] = cs[base + c];
            });
        });
}

constexpr int kTkMergeMaxK = 4096;   // unordered merge: selected pairs sorted in LDS

struct TkMergeShared {
    TkShared tk;
    int32_t pos[kTkMergeMaxK];
    float sc[kTkMergeMaxK];
};

// Writes the pairs of this thread marked in selm (list order) to out[0..m)
// sorted by position (bitonic sort in LDS), then pads with -1 to K.  m =
// number of marked pairs in the block, at most min(K, kTkMergeMaxK) for valid
// input (unique positions); anything beyond is dropped, never written.
template <int EPT>
__device__ __forceinline__ void tk_emit_sorted(TkMergeShared& sh, const int32_t (&pr)[EPT], const float* cs,
                                               int base, uint64_t selm, int K, int32_t* out, float* out_score) {
    const int tid = threadIdx.x;
    uint32_t m;
    uint32_t at = block_excl_scan((uint32_t)__popcll(selm), sh.tk.wsum, m);
    const uint32_t cap = (uint32_t)(K < kTkMergeMaxK ? K : kTkMergeMaxK);
    if (m > cap) m = cap;
#pragma unroll
    for (int c = 0; c < EPT; ++c) {
        if ((selm >> c) & 1ull) {
            if (at < cap) {
                sh.pos[at] = pr[c];
                sh.sc[at] = cs[base + c];
            }
            ++at;
        }
    }
    uint32_t P = 1;
    while (P < m) P <<= 1;
    for (uint32_t i = m + tid; i < P; i += kTkThreads) {
        sh.pos[i] = 0x7FFFFFFF;
        sh.sc[i] = 0.0f;
    }
    __syncthreads();
    for (uint32_t k = 2; k <= P; k <<= 1) {
        for (uint32_t j = k >> 1; j > 0; j >>= 1) {
            for (uint32_t i = tid; i < P; i += kTkThreads) {
                const uint32_t ij = i ^ j;
                if (ij > i) {
                    const int32_t a = sh.pos[i], b = sh.pos[ij];
                    const bool up = (i & k) == 0;
                    if ((a > b) == up) {
                        const float fa = sh.sc[i];
                        sh.pos[i] = b;
                        sh.pos[ij] = a;
                        sh.sc[i] = sh.sc[ij];
                        sh.sc[ij] = fa;
                    }
                }
            }
            __syncthreads();
        }
    }
    for (int i = tid; i < K; i += kTkThreads) {
        const bool v = (uint32_t)i < m;
        out[i] = v ? sh.pos[i] : -1;
        if (out_score) out_score[i] = v ? sh.sc[i] : -__builtin_inff();
    }
}

// The K best of n (position, score) candidates per row (position < 0 = none):
// larger score first, equal scores toward the lower position; ascending
// positions, -1 padded.  `ordered`: the valid candidates of a row come in
// ascending position order (slices of one row, or the shards of a contiguous
// context split gathered in rank order); then list order settles ties and the
// output needs no sort.  Otherwise ties at the K-th score are settled by a
// second selection on the positions and the selected pairs are sorted in LDS
// (K <= kTkMergeMaxK).
template <int EPT>
__global__ __launch_bounds__(kTkThreads) void topk_merge_kernel(const float* __restrict__ cand_score,
                                                                const int32_t* __restrict__ cand_pos, int64_t ldc,
                                                                int n, int K, int ordered, int32_t* __restrict__ idx,
                                                                float* __restrict__ idx_score) {
    __shared__ TkMergeShared sh;
    const int r = blockIdx.x, tid = threadIdx.x;
    const float* cs = cand_score + (int64_t)r * ldc;
    const int32_t* cp = cand_pos + (int64_t)r * ldc;
    int32_t* out = idx + (int64_t)r * K;
    float* outs = idx_score ? idx_score + (int64_t)r * K : nullptr;
    const int base = tid * EPT;
    uint32_t kr[EPT];
    int32_t pr[EPT];
    uint64_t vm = 0ull;
    // 16-byte loads when this thread's candidates are whole and aligned
    const bool vec = EPT % 4 == 0 && (ldc & 3) == 0 && base + EPT <= n &&
                     ((((uintptr_t)cand_score) | ((uintptr_t)cand_pos)) & 15) == 0;
    if (vec) {
#pragma unroll
        for (int c = 0; c < EPT; c += 4) {
            const i32x4 p4 = *(const i32x4*)(cp + base + c);
            const f32x4 s4 = *(const f32x4*)(cs + base + c);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                pr[c + e] = p4[e];
                kr[c + e] = float_key(p4[e] >= 0 ? s4[e] : 0.0f);
                vm |= (uint64_t)(p4[e] >= 0) << (c + e);
            }
        }
    } else {
#pragma unroll
        for (int c = 0; c < EPT; ++c) {
            const int i = base + c;
            const int32_t p = i < n ? cp[i] : -1;
            pr[c] = p;
            kr[c] = float_key(p >= 0 ? cs[i] : 0.0f);
            vm |= (uint64_t)(p >= 0) << c;
        }
    }
    uint32_t nvalid;
    uint32_t first = block_excl_scan((uint32_t)__popcll(vm), sh.tk.wsum, nvalid);
    if (nvalid <= (uint32_t)K) {
        if (ordered) {
#pragma unroll
            for (int c = 0; c < EPT; ++c) {
                if ((vm >> c) & 1ull) {
                    out[first] = pr[c];
                    if (outs) outs[first] = cs[base + c];
                    ++first;
                }
            }
            for (int i = (int)nvalid + tid; i < K; i += kTkThreads) {
                out[i] = -1;
                if (outs) outs[i] = -__builtin_inff();
            }
        } else {
            tk_emit_sorted<EPT>(sh, pr, cs, base, vm, K, out, outs);
        }
        return;
    }
    if (ordered) {
        tk_select<EPT>(sh.tk, kr, TkMask{vm}, (uint32_t)K, [&](int c, uint32_t slot) {
            out[slot] = pr[c];
            if (outs) outs[slot] = cs[base + c];
        });
        return;
    }
    uint32_t T, need_eq;
    tk_threshold<EPT>(sh.tk, kr, TkMask{vm}, (uint32_t)K, T, need_eq);
    uint64_t gtm = 0ull, eqm = 0ull;
#pragma unroll
    for (int c = 0; c < EPT; ++c) {
        if ((vm >> c) & 1ull) {
            gtm |= (uint64_t)(kr[c] > T) << c;
            eqm |= (uint64_t)(kr[c] == T) << c;
        }
    }
    uint32_t neq;
    (void)block_excl_scan((uint32_t)__popcll(eqm), sh.tk.wsum, neq);
    uint64_t selm = gtm | eqm;
    if (need_eq < neq) {
        // the need_eq lowest positions among the tied keys = the largest ~position
#pragma unroll
        for (int c = 0; c < EPT; ++c) kr[c] = ~(uint32_t)pr[c];
        uint32_t T2, need2;
        tk_threshold<EPT>(sh.tk, kr, TkMask{eqm}, need_eq, T2, need2);
        uint64_t tie = 0ull;
#pragma unroll
        for (int c = 0; c < EPT; ++c) tie |= (uint64_t)(((eqm >> c) & 1ull) && kr[c] >= T2) << c;
        selm = gtm | tie;
    }
    tk_emit_sorted<EPT>(sh, pr, cs, base, selm, K, out, outs);
}

// ------------------------------------------------------------------ host ---

constexpr int kTkSliceEPT = 16;                            // shard candidates: slices of 16384 positions
constexpr int64_t kTkSliceLen = (int64_t)kTkThreads * kTkSliceEPT;
constexpr int kTkMergeMaxN = kTkThreads * 16;            // candidates one merge workgroup holds

// Slices a long shard row is cut into for topk_candidates, or 0 when its
// two-pass selection does not apply.
int topk_slices(int64_t ld, int K) {
    if (ld <= (int64_t)kTkThreads * 64) return 0;
    const int64_t S = (ld + kTkSliceLen - 1) / kTkSliceLen;
    if (S * K > kTkMergeMaxN) return 0;
    return (int)S;
}

size_t topk_workspace_bytes(int R, int64_t ld, int K) {
    const int S = topk_slices(ld, K);
    if (S == 0 || R <= 0) return 0;
    return (size_t)R * S * K * (sizeof(int32_t) + sizeof(float));
}

static hipError_t launch_merge(const float* cs, const int32_t* cp, int64_t ldc, int n, int R, int K, int ordered,
                               int32_t* idx, float* idx_score, hipStream_t stream) {
    const int ept = (n + kTkThreads - 1) / kTkThreads;
#define LISFA_TKM(E_)                                                                                    \
    hipLaunchKernelGGL((topk_merge_kernel<E_>), dim3((unsigned)R), dim3(kTkThreads), 0, stream, cs, cp, ldc, n, \
                       K, ordered, idx, idx_score)
#define LISFA_TKMO(E_)                                                                                       \
    hipLaunchKernelGGL((topk_merge_ordered_kernel<E_>), dim3((unsigned)R), dim3(kTkThreads), 0, stream, cs, cp, \
                       ldc, n, K, idx, idx_score)
    if (ordered) {
        if (ept <= 8) LISFA_TKMO(8);
        else LISFA_TKMO(16);
    } else {
        if (ept <= 8) LISFA_TKM(8);
        else LISFA_TKM(16);
    }
#undef LISFA_TKMO
#undef LISFA_TKM
    return hipGetLastError();
}

hipError_t topk_merge_dispatch(const float* cand_score, const int32_t* cand_pos, int64_t ldc, int R, int n, int K,
                               int ordered, int32_t* idx, float* idx_score, hipStream_t stream) {
    if (R <= 0) return hipSuccess;
    return launch_merge(cand_score, cand_pos, ldc, n, R, K, ordered, idx, idx_score, stream);
}

static hipError_t launch_cand(const float* scores, int64_t ld, const int32_t* row_pos, int R, int K, int S, int ept,
                              const int32_t* pos_offset, int32_t* cp, float* cs, hipStream_t stream) {
#define LISFA_TKC(E_)                                                                                    \
    hipLaunchKernelGGL((topk_cand_kernel<E_>), dim3((unsigned)S, (unsigned)R), dim3(kTkThreads), 0, stream, \
                       scores, ld, row_pos, K, S, pos_offset, cp, cs)
    if (ept <= 8) LISFA_TKC(8);
    else if (ept <= 16) LISFA_TKC(16);
    else if (ept <= 32) LISFA_TKC(32);
    else LISFA_TKC(64);
#undef LISFA_TKC
    return hipGetLastError();
}

// Local Top-K candidates of a context shard.  Rows up to 64K positions: one
// slice per row straight into the outputs; longer rows: slices into ws, then
// an ordered merge that also carries the scores.
hipError_t topk_candidates_dispatch(const float* scores, int64_t ld, const int32_t* row_pos, int R, int K,
                                    const int32_t* pos_offset, int32_t* cand_pos, float* cand_score, void* ws,
                                    hipStream_t stream) {
    if (R <= 0) return hipSuccess;
    if (ld <= (int64_t)kTkThreads * 64) {
        const int ept = (int)((ld + kTkThreads - 1) / kTkThreads);
        return launch_cand(scores, ld, row_pos, R, K, 1, ept, pos_offset, cand_pos, cand_score, stream);
    }
    const int S = topk_slices(ld, K);
    int32_t* cp = (int32_t*)ws;
    float* cs = (float*)((uint8_t*)ws + (size_t)R * S * K * sizeof(int32_t));
    hipError_t e = launch_cand(scores, ld, row_pos, R, K, S, kTkSliceEPT, pos_offset, cp, cs, stream);
    if (e != hipSuccess) return e;
    return launch_merge(cs, cp, (int64_t)S * K, S * K, R, K, 1, cand_pos, cand_score, stream);
}

// Rows up to 64K positions: one workgroup per row, keys in registers.
// Longer rows: with ws, slices of 16384 positions keep their own Top-K and
// an ordered merge selects (topk_workspace_bytes); without, one
// workgroup per row re-reads the keys from global memory.
hipError_t topk_dispatch(const float* scores, int64_t ld, const int32_t* row_pos, int R, int K,
                         int32_t* idx, void* ws, hipStream_t stream) {
    if (R <= 0) return hipSuccess;
    const int64_t ept = (ld + kTkThreads - 1) / kTkThreads;
    if (ept > 64) {
        const int S = topk_slices(ld, K);
        if (S > 0 && ws) {
            int32_t* cp = (int32_t*)ws;
            float* cs = (float*)((uint8_t*)ws + (size_t)R * S * K * sizeof(int32_t));
            hipError_t e = launch_cand(scores, ld, row_pos, R, K, S, kTkSliceEPT, nullptr, cp, cs, stream);
            if (e != hipSuccess) return e;
            return launch_merge(cs, cp, (int64_t)S * K, S * K, R, K, 1, idx, nullptr, stream);
        }
        hipLaunchKernelGGL(topk_stream_kernel, dim3((unsigned)R), dim3(kTkThreads), 0, stream, scores, ld, row_pos,
                           K, idx);
        return hipGetLastError();
    }
#define LISFA_TK(E_)                                                                                       \
    hipLaunchKernelGGL((topk_row_kernel<E_>), dim3((unsigned)R), dim3(kTkThreads), 0, stream, scores, ld, \
                       row_pos, K, idx)
    if (ept <= 8) LISFA_TK(8);
    else if (ept <= 16) LISFA_TK(16);
    else if (ept <= 32) LISFA_TK(32);
    else LISFA_TK(64);
#undef LISFA_TK
    return hipGetLastError();
}

}  // namespace lisfa
