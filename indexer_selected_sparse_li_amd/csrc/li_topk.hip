// Fused indexer scores + Top-K for decode rows: the scores never leave the chip.
//
// "Kimi New Model Open Source ... on Ascend", section 3: one operator reads the
// paged indexer key cache and returns only the list of selected positions;
// "Large Language Model Inference Acceleration in Practice", section 3.1: the
// head-weight weighting and the Top-K run on chip and the index list is handed
// to the attention step.  The result is the one li_score followed by
// topk_select gives, bit for bit: the scores come from the same scoring loops
// (li_dec.hpp) and the selection orders the same keys (float_key: larger
// first, equal keys toward the lower position; ascending positions out).
//
// Work decomposition.  The positions of a row are split into n <= 64 chunks of
// kpw positions; workgroup (m, r) scores chunk m of row r exactly as the score
// kernel does, but keeps the chunk's order keys in LDS.  The n workgroups of a
// row then select the row's K best together, exchanging only small summaries
// through a per-row area of the workspace:
//   1. key range: every member publishes its minimum and maximum key;
//   2. up to three histogram levels: 4096 bins over the current key range,
//      each member publishes the suffix sums S_m(b) = #{its keys in bins >= b}
//      of its local histogram; the boundary bin b* (the highest bin with
//      sum_m S_m(b) >= the number still needed) is found by reading the sums at
//      64 evenly spaced bins, then at the 64 bins of the chosen segment;
//   3. finish, from the counts of the boundary bin:
//        - it is needed whole: every key at or above its low edge is selected;
//        - it holds one key value (ties): the lowest positions of that value,
//          member by member, since chunks are position-ordered;
//        - it holds <= 256 keys: the members publish those (key, position)
//          pairs and every member ranks them to find the K-th element;
//        - otherwise the next level refines the bin.
//   Each member knows from the published suffix sums how many keys every lower
//   member selects, so it writes its selected positions, ascending, straight to
//   their final slots: no score, candidate or partial list is written to HBM.
//
// Cross-workgroup exchange.  Exchanged words are written and read with
// device-scope (sc1) accesses only, so a barrier is: wait until this wave's
// stores are acknowledged, workgroup barrier, one atomic add on the row's
// counter, poll it.  No cache-wide writeback or invalidate is issued (an
// agent-scope fence costs ~15 us per barrier when 256 workgroups sync at once;
// this form ~1.2 us, measured in-bounds).  Every member of a row must be
// resident at once: launches with more than one member per row are limited to
// kLtMaxWg workgroups (one per CU).  The polls are bounded; a bound that runs
// out (it cannot while the members are co-resident) sets the row's flag in the
// control area and the kernel still ends.
#include "li_dec.hpp"

namespace lisfa {

constexpr int kLtThreads = 64 * kLiDecWaves;   // 256
constexpr int kLtEpt = 64;                     // keys per thread at most
constexpr int kLtMaxKeys = kLtThreads * kLtEpt;   // positions of one workgroup (16384)
constexpr int kLtMaxMembers = 64;              // workgroups per row
constexpr int kLtMaxWg = 256;                  // workgroups of a launch that exchanges
constexpr int kLtBins = 4096;
constexpr int kLtLevels = 3;                   // 12 + 12 + 8 key bits
constexpr int kLtListMax = 256;                // boundary bins ranked directly up to this size
constexpr int kLtCtlWords = 16;                // per row: counter, time-out flag (own 64 bytes)
constexpr uint32_t kLtSpinCap = 1u << 21;      // polls (each >= ~0.1 us) before giving up
// Per-row exchange area (bytes): member key ranges, the boundary list, then
// for every level and member 64 coarse and 4096 fine suffix sums, 16-bit
// (a member holds at most 16384 keys).
constexpr int64_t kLtListOff = 512;
constexpr int64_t kLtLevelOff = kLtListOff + kLtListMax * 8;
constexpr int64_t kLtCoarseBytes = 64 * 2;
constexpr int64_t kLtMemberBytes = kLtCoarseBytes + kLtBins * 2;
constexpr int kLtDevScope = 16;                // buffer cache policy: device scope (sc1)

inline int64_t lt_row_bytes(int nchunk) { return kLtLevelOff + (int64_t)kLtLevels * nchunk * kLtMemberBytes; }

struct LtArgs {
    int32_t* idx;        // [R, K] out
    uint32_t* ctl;       // [R, kLtCtlWords], zero at launch
    uint8_t* xch;        // [R, row_bytes]
    int64_t row_bytes;
    int64_t ld;          // visible positions of a row: row_pos + 1 clamped to [0, ld]
    int32_t K;
    int32_t kpw;         // positions per workgroup: 256 << lg_ept
    int32_t lg_ept;      // log2 of the keys per thread
    int32_t nchunk;      // workgroups per row (grid x)
};

// Exchange accesses: buffer loads and stores at device scope through a
// descriptor that covers the row's area (the hardware drops accesses past it).
__device__ __forceinline__ void xst4(__amdgpu_buffer_rsrc_t b, uint32_t off, u32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(v, b, off, 0, kLtDevScope);
}
__device__ __forceinline__ void xst2(__amdgpu_buffer_rsrc_t b, uint32_t off, u32x2 v) {
    __builtin_amdgcn_raw_buffer_store_b64(v, b, off, 0, kLtDevScope);
}
__device__ __forceinline__ u32x4 xld4(__amdgpu_buffer_rsrc_t b, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(b, off, 0, kLtDevScope);
}
__device__ __forceinline__ u32x2 xld2(__amdgpu_buffer_rsrc_t b, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b64(b, off, 0, kLtDevScope);
}

// Row barrier: returns once `target` arrivals are counted in ctl[0].
__device__ __forceinline__ void lt_barrier(uint32_t* ctl, uint32_t target) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's stores acknowledged
    __syncthreads();
    if (threadIdx.x == 0) {
        __hip_atomic_fetch_add(ctl, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        uint32_t it = 0;
        while (__hip_atomic_load(ctl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
            __builtin_amdgcn_s_sleep(2);
            if (++it == kLtSpinCap) {
                __hip_atomic_store(ctl + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
        }
    }
    __syncthreads();
}

// wave-wide results through the DPP scans (lane 63 holds the total)
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_min(v), 63);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_max(v), 63);
}
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_sum(v), 63);
}

// m = 2 m + (key > thr) / (key == thr) / (key - lo <= span): the compare goes
// to VCC and into the mask through the carry, so a mask over a thread's keys
// costs two instructions per key and holds no per-key condition registers.
// After 32 pushes key e of the group sits at bit 31 - e.
__device__ __forceinline__ void push_gt(uint32_t& m, uint32_t key, uint32_t thr) {
    asm volatile("v_cmp_gt_u32 vcc, %1, %2\n\tv_addc_co_u32 %0, vcc, %0, %0, vcc"
                 : "+v"(m) : "v"(key), "v"(thr) : "vcc");
}
__device__ __forceinline__ void push_eq(uint32_t& m, uint32_t key, uint32_t thr) {
    asm volatile("v_cmp_eq_u32 vcc, %1, %2\n\tv_addc_co_u32 %0, vcc, %0, %0, vcc"
                 : "+v"(m) : "v"(key), "v"(thr) : "vcc");
}
__device__ __forceinline__ void push_le(uint32_t& m, uint32_t d, uint32_t span) {
    asm volatile("v_cmp_le_u32 vcc, %1, %2\n\tv_addc_co_u32 %0, vcc, %0, %0, vcc"
                 : "+v"(m) : "v"(d), "v"(span) : "vcc");
}

// 8 16-bit suffix sums of a 16-byte load into sv[i0 .. i0 + 7]
__device__ __forceinline__ void unpack16(uint32_t* dst, u32x4 v) {
    dst[0] = v.x & 0xFFFFu;
    dst[1] = v.x >> 16;
    dst[2] = v.y & 0xFFFFu;
    dst[3] = v.y >> 16;
    dst[4] = v.z & 0xFFFFu;
    dst[5] = v.z >> 16;
    dst[6] = v.w & 0xFFFFu;
    dst[7] = v.w >> 16;
}

enum { kLtAll = 0, kLtTie = 1, kLtList = 2 };

// FMT 0: bf16 keys (D_I = DI); 1: MXFP8 keys; 2: per-token fp8 keys (D_I = 128).
template <int FMT, int DI, int MT>
__global__ __launch_bounds__(kLtThreads) void li_topk_kernel(IndexerDev a, LtArgs t) {
    // order keys of the chunk: position p at word (p % E) * 256 + p / E,
    // E = kpw / 256, so thread i reads its run p = E i .. E i + E - 1 without
    // bank conflicts; words no position fills stay 0 (no key)
    __shared__ __attribute__((aligned(16))) uint32_t keys[kLtMaxKeys];
    __shared__ int64_t blk_slot0[kLiMaxBlocks];
    __shared__ int32_t blk_lim[kLiMaxBlocks];
    // level histogram (then its suffix sums) and a spill bin per lane for the
    // keys outside the level's range
    __shared__ __attribute__((aligned(16))) uint32_t hist[kLtBins + 64];
    __shared__ __attribute__((aligned(16))) uint16_t coarse[64];      // suffix sums at bins 64 i
    __shared__ uint32_t sv[kLtMaxMembers][65];   // members' suffix sums at the 64 (+1) search points
    __shared__ uint32_t above[kLtMaxMembers];    // members' keys above the current bin
    __shared__ uint32_t inb[kLtMaxMembers];      // members' keys in the boundary bin
    __shared__ uint32_t gtl[kLtMaxMembers];      // members' selected bin keys above the threshold key
    __shared__ uint32_t xs[kLtMaxMembers];       // members' selected keys equal to the threshold key
    __shared__ u32x2 lst[kLtListMax];            // boundary bin: (key, position)
    __shared__ uint32_t red[8];
    __shared__ uint32_t bc[8];                   // broadcast scalars

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = blockIdx.y, m = blockIdx.x;
    const int K = t.K;
    const int64_t vis = li_visible(a, r, t.ld);
    int32_t* out = t.idx + (int64_t)r * K;
    const int64_t c0 = (int64_t)m * t.kpw;
    if (vis <= K) {   // every visible position is selected, in order; member 0 pads
        const int64_t e = c0 + t.kpw < vis ? c0 + t.kpw : vis;
        for (int64_t j = c0 + tid; j < e; j += kLtThreads) out[j] = (int32_t)j;
        if (m == 0)
            for (int64_t j = vis + tid; j < K; j += kLtThreads) out[j] = -1;
        return;
    }
    if (c0 >= vis) return;   // uniform: not a member of this row
    const int64_t kend = c0 + t.kpw < vis ? c0 + t.kpw : vis;
    const int cnt = (int)(kend - c0);
    const int n = (int)((vis + t.kpw - 1) / t.kpw);
    const int le = t.lg_ept, E = 1 << le;

    auto sink = [&](int64_t key, float v) {
        const uint32_t p = (uint32_t)(key - c0);
        keys[((p & (uint32_t)(E - 1)) << 8) + (p >> le)] = float_key(v);
    };
#pragma unroll
    for (int q = 0; q < kLtEpt / 4; ++q) *(u32x4*)&keys[4 * (tid + kLtThreads * q)] = u32x4{0u, 0u, 0u, 0u};
    // (the scoring loop's first barrier orders these before the scores)
    if constexpr (FMT == 0)
        li_dec_chunk<DI, MT>(a, r, c0, kend, blk_slot0, blk_lim, sink);
    else
        li_mx_chunk<MT, FMT == 2>(a, r, c0, kend, blk_slot0, blk_lim, sink);

    uint32_t* ctl = t.ctl + (int64_t)r * kLtCtlWords;
    const __amdgpu_buffer_rsrc_t xb =
        __builtin_amdgcn_make_buffer_rsrc(t.xch + (int64_t)r * t.row_bytes, (short)0, (int)t.row_bytes, 0x00020000);
    uint32_t nbar = 0;
    __syncthreads();   // keys complete

    // this thread's keys, positions c0 + E tid + e (0: no key)
    uint32_t kr[kLtEpt];
#pragma unroll
    for (int e = 0; e < kLtEpt; ++e) kr[e] = keys[(e << 8) + tid];

    // 1. key range of the row
    uint32_t kmn = 0xFFFFFFFFu, kmx = 0u;
#pragma unroll
    for (int e = 0; e < kLtEpt; ++e) {
        kmn = min(kmn, kr[e] ? kr[e] : 0xFFFFFFFFu);
        kmx = max(kmx, kr[e]);
    }
    kmn = wave_min_u32(kmn);
    kmx = wave_max_u32(kmx);
    if (lane == 0) {
        red[wave] = kmn;
        red[4 + wave] = kmx;
    }
    for (int i = tid; i < n; i += kLtThreads) above[i] = 0;
    __syncthreads();
    uint32_t slo = min(min(red[0], red[1]), min(red[2], red[3]));
    uint32_t shi = max(max(red[4], red[5]), max(red[6], red[7]));
    if (n > 1) {
        if (tid == 0) xst2(xb, 8 * m, u32x2{slo, shi});
        lt_barrier(ctl, ++nbar * (uint32_t)n);
        if (wave == 0) {
            uint32_t v0 = 0xFFFFFFFFu, v1 = 0u;
            if (lane < n) {
                const u32x2 v = xld2(xb, 8 * lane);
                v0 = v.x;
                v1 = v.y;
            }
            v0 = wave_min_u32(v0);
            v1 = wave_max_u32(v1);
            if (lane == 0) {
                bc[0] = v0;
                bc[1] = v1;
            }
        }
        __syncthreads();
        slo = bc[0];
        shi = bc[1];
    }

    // 2. histogram levels over the keys in [lo, hi] (first the row's exact
    // key range); need = how many of those are selected.  Bin b holds
    // [lo + b 2^s, lo + (b + 1) 2^s); each level refines one bin.
    uint32_t lo = slo, hi = shi, base = slo, need = (uint32_t)K;
    int s = shi - slo < (uint32_t)kLtBins ? 0 : 20 - __builtin_clz(shi - slo);
    uint32_t Kt = 0, blo = 0, bhi = 0;
    int mode = kLtTie;
    for (int lev = 0; lev < kLtLevels; ++lev) {
        if (lev > 0) {
            base = lo;
            s = hi - lo < (uint32_t)kLtBins ? 0 : 20 - __builtin_clz(hi - lo);   // ((hi - lo) >> s) < 4096
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) *(u32x4*)&hist[16 * tid + 4 * q] = u32x4{0u, 0u, 0u, 0u};
        if (tid < 16) *(u32x4*)&hist[kLtBins + 4 * tid] = u32x4{0u, 0u, 0u, 0u};
        __syncthreads();
#pragma unroll
        for (int e = 0; e < kLtEpt; ++e) {
            const uint32_t k = kr[e];   // lo >= 1 leaves out the empty slots
            const uint32_t d = k < base ? 0u : (k - base) >> s;
            const uint32_t b = d < (uint32_t)kLtBins ? d : (uint32_t)(kLtBins - 1);
            atomicAdd(&hist[(k >= lo && k <= hi) ? b : (uint32_t)(kLtBins + lane)], 1u);
        }
        __syncthreads();
        // suffix sums; thread tid owns bins [16 tid, 16 tid + 16)
        uint32_t hv[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const u32x4 v = *(const u32x4*)&hist[16 * tid + 4 * q];
            hv[4 * q] = v.x;
            hv[4 * q + 1] = v.y;
            hv[4 * q + 2] = v.z;
            hv[4 * q + 3] = v.w;
        }
        uint32_t acc = 0;
#pragma unroll
        for (int i = 15; i >= 0; --i) {
            acc += hv[i];
            hv[i] = acc;
        }
        const uint32_t incl = wave_incl_sum(acc);
        if (lane == 63) red[wave] = incl;
        __syncthreads();
        uint32_t before = 0, total = 0;
#pragma unroll
        for (int w = 0; w < kLiDecWaves; ++w) {
            total += red[w];
            if (w < wave) before += red[w];
        }
        const uint32_t higher = total - before - incl;   // keys in bins of higher threads
#pragma unroll
        for (int i = 0; i < 16; ++i) hv[i] += higher;
        const uint32_t lev_off = (uint32_t)(kLtLevelOff + (int64_t)lev * t.nchunk * kLtMemberBytes);
        if (n > 1) {
            const uint32_t mo = lev_off + (uint32_t)(m * kLtMemberBytes);
            xst4(xb, mo + kLtCoarseBytes + 32 * tid,
                 u32x4{hv[0] | hv[1] << 16, hv[2] | hv[3] << 16, hv[4] | hv[5] << 16, hv[6] | hv[7] << 16});
            xst4(xb, mo + kLtCoarseBytes + 32 * tid + 16,
                 u32x4{hv[8] | hv[9] << 16, hv[10] | hv[11] << 16, hv[12] | hv[13] << 16, hv[14] | hv[15] << 16});
            if ((tid & 3) == 0) coarse[tid >> 2] = (uint16_t)hv[0];
            __syncthreads();
            if (tid < 8) xst4(xb, mo + 16 * tid, *(const u32x4*)&coarse[8 * tid]);
            lt_barrier(ctl, ++nbar * (uint32_t)n);
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q)
                *(u32x4*)&hist[16 * tid + 4 * q] = u32x4{hv[4 * q], hv[4 * q + 1], hv[4 * q + 2], hv[4 * q + 3]};
            __syncthreads();
        }
        // search: the suffix sums at bins 64 i, then at the 64 bins of the chosen segment
        if (n > 1) {
            for (int e = tid; e < n * 8; e += kLtThreads)
                unpack16(&sv[e >> 3][8 * (e & 7)], xld4(xb, lev_off + (uint32_t)((e >> 3) * kLtMemberBytes) + 16 * (e & 7)));
        } else if (tid < 64) {
            sv[0][tid] = hist[64 * tid];
        }
        __syncthreads();
        if (wave == 0) {
            uint32_t G = 0;
            for (int mm = 0; mm < n; ++mm) G += sv[mm][lane];
            const int i1 = (int)__popcll(__ballot(G >= need)) - 1;
            if (lane == 0) bc[2] = (uint32_t)(i1 > 0 ? i1 : 0);
        }
        __syncthreads();
        const int i1 = (int)bc[2];
        for (int mm = tid; mm < n; mm += kLtThreads) sv[mm][64] = i1 < 63 ? sv[mm][i1 + 1] : 0u;
        __syncthreads();
        if (n > 1) {
            for (int e = tid; e < n * 8; e += kLtThreads)
                unpack16(&sv[e >> 3][8 * (e & 7)],
                         xld4(xb, lev_off + (uint32_t)((e >> 3) * kLtMemberBytes) + kLtCoarseBytes + 128 * i1 +
                                      16 * (e & 7)));
        } else if (tid < 64) {
            sv[0][tid] = hist[64 * i1 + tid];
        }
        __syncthreads();
        if (wave == 0) {
            uint32_t G = 0, G64 = 0;
            for (int mm = 0; mm < n; ++mm) {
                G += sv[mm][lane];
                G64 += sv[mm][64];
            }
            int js = (int)__popcll(__ballot(G >= need)) - 1;
            js = js > 0 ? js : 0;
            const uint32_t Gj = (uint32_t)__shfl((int)G, js);
            const uint32_t Gj1 = js < 63 ? (uint32_t)__shfl((int)G, js + 1) : G64;
            if (lane == 0) {
                bc[3] = (uint32_t)js;
                bc[4] = Gj;
                bc[5] = Gj1;
            }
        }
        __syncthreads();
        const int js = (int)bc[3];
        const uint32_t Gj = bc[4], Gj1 = bc[5];
        for (int mm = tid; mm < n; mm += kLtThreads) {
            const uint32_t h1 = sv[mm][js + 1];
            above[mm] += h1;
            inb[mm] = sv[mm][js] - h1;
        }
        __syncthreads();
        const uint32_t bstar = (uint32_t)(64 * i1 + js);
        const uint32_t C = Gj - Gj1;   // keys of the row in bin b*
        need -= Gj1;                   // 1 <= need <= C
        // the bin's key interval (it holds keys, so its low edge is a key value)
        const uint64_t b0 = (uint64_t)base + ((uint64_t)bstar << s);
        blo = bstar == 0 ? lo : (uint32_t)(b0 < hi ? b0 : hi);
        const uint64_t b1 = b0 + (((uint64_t)1 << s) - 1);
        bhi = (bstar == (uint32_t)(kLtBins - 1) || b1 >= hi) ? hi : (uint32_t)b1;
        if (C == need) {
            mode = kLtAll;
            Kt = blo - 1;   // blo >= 1: no float has key 0
            break;
        }
        if (blo == bhi) {   // one key value: ties
            mode = kLtTie;
            Kt = blo;
            break;
        }
        if (C <= (uint32_t)kLtListMax) {
            mode = kLtList;
            break;
        }
        lo = blo;
        hi = bhi;
    }

    // 3. finish: per member, keys above Kt (above + gtl) and equal keys taken (xs)
    for (int mm = tid; mm < n; mm += kLtThreads) {
        gtl[mm] = 0;
        xs[mm] = 0;
    }
    if (mode == kLtList) {
        uint32_t base = 0;   // this member's first list slot
        for (int mm = 0; mm < m; ++mm) base += inb[mm];
        if (tid == 0) bc[6] = 0;
        __syncthreads();
        // this thread's keys in the bin (empty slots are 0 < blo)
        uint32_t bl = 0u, bh = 0u;
#pragma unroll
        for (int e = 0; e < 32; ++e) push_le(bl, kr[e] - blo, bhi - blo);
#pragma unroll
        for (int e = 32; e < kLtEpt; ++e) push_le(bh, kr[e] - blo, bhi - blo);
        uint64_t bm = ((uint64_t)bl << 32) | bh;   // key e at bit 63 - e
        while (bm) {
            const int bit = 63 - __builtin_clzll(bm);
            bm &= ~(1ull << bit);
            const int e = 63 - bit;
            const uint32_t k = keys[(e << 8) + tid];
            const uint32_t p = atomicAdd(&bc[6], 1u);
            const u32x2 item = u32x2{k, (uint32_t)(c0 + tid * E + e)};
            if (n > 1) {
                if (base + p < (uint32_t)kLtListMax) xst2(xb, (uint32_t)kLtListOff + 8 * (base + p), item);
            } else if (p < (uint32_t)kLtListMax) {
                lst[p] = item;
            }
        }
        uint32_t C = 0;
        for (int mm = 0; mm < n; ++mm) C += inb[mm];
        C = C < (uint32_t)kLtListMax ? C : (uint32_t)kLtListMax;
        if (n > 1) {
            lt_barrier(ctl, ++nbar * (uint32_t)n);
            for (int e = tid; e < (int)C; e += kLtThreads) lst[e] = xld2(xb, (uint32_t)kLtListOff + 8 * e);
        }
        __syncthreads();
        // the need-th largest (key descending, position ascending)
        for (int e = tid; e < (int)C; e += kLtThreads) {
            const u32x2 me = lst[e];
            uint32_t rk = 0;
#pragma unroll 8
            for (int u = 0; u < (int)C; ++u) {
                const u32x2 o = lst[u];
                rk += (o.x > me.x || (o.x == me.x && o.y < me.y)) ? 1u : 0u;
            }
            if (rk == need - 1) {
                bc[6] = me.x;
                bc[7] = me.y;
            }
        }
        __syncthreads();
        Kt = bc[6];
        const uint32_t Pt = bc[7];
        for (int e = tid; e < (int)C; e += kLtThreads) {
            const u32x2 o = lst[e];
            int mm = (int)((o.y - (uint32_t)0) / (uint32_t)t.kpw);
            mm = mm < n ? mm : n - 1;
            if (o.x > Kt)
                atomicAdd(&gtl[mm], 1u);
            else if (o.x == Kt && o.y <= Pt)
                atomicAdd(&xs[mm], 1u);
        }
        __syncthreads();
    } else if (mode == kLtTie) {
        __syncthreads();
        for (int mm = tid; mm < n; mm += kLtThreads) {
            uint32_t pre = 0;
            for (int q = 0; q < mm; ++q) pre += inb[q];
            const uint32_t left = need > pre ? need - pre : 0u;
            xs[mm] = left < inb[mm] ? left : inb[mm];
        }
        __syncthreads();
    } else {
        __syncthreads();
        for (int mm = tid; mm < n; mm += kLtThreads) gtl[mm] = inb[mm];
        __syncthreads();
    }
    // selected keys of the lower members: this member's first output slot
    if (wave == 0) {
        const uint32_t sel = lane < m ? above[lane] + gtl[lane] + xs[lane] : 0u;
        const uint32_t off = wave_sum_u32(sel);
        if (lane == 0) bc[5] = off;
    }
    __syncthreads();
    const uint32_t offset = bc[5];
    const uint32_t xm = xs[m];

    // 4. emission: threads own position-ordered runs; masks of the keys above
    // and equal to Kt, a block scan of their counts, then each thread writes
    // the positions it selects (an equal key is taken while the row's equal
    // keys before it number fewer than xm; Kt is 0 only when xm is 0)
    uint32_t gl = 0u, gh = 0u, el = 0u, eh = 0u;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
        push_gt(gl, kr[e], Kt);
        push_eq(el, kr[e], Kt);
    }
#pragma unroll
    for (int e = 32; e < kLtEpt; ++e) {
        push_gt(gh, kr[e], Kt);
        push_eq(eh, kr[e], Kt);
    }
    const uint64_t gm = ((uint64_t)gl << 32) | gh;   // key e at bit 63 - e
    uint64_t em = ((uint64_t)el << 32) | eh;
    const uint32_t g = (uint32_t)__popcll(gm), q = (uint32_t)__popcll(em);
    const uint32_t gi = wave_incl_sum(g), qi = wave_incl_sum(q);
    if (lane == 63) {
        red[wave] = gi;
        red[4 + wave] = qi;
    }
    __syncthreads();
    uint32_t gb = gi - g, qb = qi - q;
    for (int w = 0; w < wave; ++w) {
        gb += red[w];
        qb += red[4 + w];
    }
    const uint32_t take = qb < xm ? (xm - qb < q ? xm - qb : q) : 0u;   // equal keys this thread takes
    if (take == 0u) em = 0u;
    while ((uint32_t)__popcll(em) > take) em &= em - 1u;   // keep the first `take` (highest bits)
    uint64_t sm = gm | em;
    uint32_t pos = offset + gb + (qb < xm ? qb : xm);
    const int32_t p0 = (int32_t)(c0 + tid * E);
    while (sm && pos < (uint32_t)K) {
        const int bit = 63 - __builtin_clzll(sm);
        sm &= ~(1ull << bit);
        out[pos++] = p0 + (63 - bit);
    }
}

__global__ void lt_clear_kernel(uint32_t* p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

namespace {

struct LtPlan {
    int64_t kpw;
    int lg_ept;
    int nchunk;
};

// Chunking of the fused launch (256 << k positions per workgroup), or false
// when the shape is left to the separate score and Top-K kernels: more than
// kLtMaxMembers chunks per row, a chunk whose block map would not fit, or an
// exchanging launch of more than kLtMaxWg workgroups.
bool lt_plan(int R, int64_t ld, const CacheDev& c, LtPlan& p) {
    const int sh = c.paged ? c.bs_shift : 6;
    const int64_t bsz = (int64_t)1 << sh;
    int64_t nchunk = (kLtMaxWg + R - 1) / R;
    if (nchunk > kLtMaxMembers) nchunk = kLtMaxMembers;
    const int64_t want = (ld + nchunk - 1) / nchunk;
    int64_t kpw = 1024;
    while (kpw < want && kpw < kLtMaxKeys) kpw *= 2;
    while (kpw < bsz && kpw < kLtMaxKeys) kpw *= 2;   // chunks start on block boundaries
    while (kpw > 1024 && kpw / bsz > kLiMaxBlocks - 1) kpw /= 2;
    if (kpw < bsz || kpw / bsz > kLiMaxBlocks - 1) return false;
    nchunk = (ld + kpw - 1) / kpw;
    if (nchunk > kLtMaxMembers) return false;
    if (nchunk > 1 && nchunk * R > kLtMaxWg) return false;
    p.kpw = kpw;
    p.nchunk = (int)nchunk;
    p.lg_ept = 0;
    while ((kLtThreads << p.lg_ept) < kpw) ++p.lg_ept;
    return true;
}

template <int FMT, int DI, int MT>
hipError_t launch_lt(const IndexerDev& a, const LtArgs& t, hipStream_t st) {
    hipLaunchKernelGGL((li_topk_kernel<FMT, DI, MT>), dim3((unsigned)t.nchunk, (unsigned)a.R), dim3(kLtThreads), 0,
                       st, a, t);
    return hipGetLastError();
}

}  // namespace

// Workspace bound of the fused launch for R rows: rows that span several
// workgroups (only launches of at most kLtMaxWg / 2 rows have them) need
// control words and exchange areas; single-workgroup rows need nothing.
size_t li_topk_workspace_bytes(int R) {
    if (R < 1 || R > kLtMaxWg / 2) return 0;
    const size_t ctl = ((size_t)R * kLtCtlWords * 4 + 255) / 256 * 256;
    return ctl + (size_t)R * kLtLevelOff + (size_t)kLtLevels * kLtMaxWg * kLtMemberBytes;
}

// Workgroups per row of the fused launch for these arguments, or 0 when the
// separate score and Top-K kernels take them.  layer != 0: the rule of the
// layer call, which takes the fused launch only where it measured faster
// than the separate kernels: bf16 keys and at most 4 workgroups per row (each
// exchange between the workgroups of a row costs ~1.5 us, so rows split over
// many workgroups, and the MXFP8 / per-token fp8 scoring, which runs twice as
// many workgroups on its own, stay with the separate kernels).
int li_topk_fused_chunks(const IndexerDev& a, int D_I, int dtype, int qg, int64_t ld, int K, int layer) {
    const bool bf16 = dtype == LISFA_BF16 && qg == 1;
    const bool mx = dtype == LISFA_MXFP8 && D_I == 128;
    const bool tok = dtype == LISFA_FP8_E4M3 && qg == 1 && D_I == 128;
    if (!bf16 && !mx && !tok) return 0;
    if (a.R < 1 || ld < 1 || K < 1) return 0;
    LtPlan p;
    if (!lt_plan(a.R, ld, a.k, p)) return 0;
    if (layer && (!bf16 || p.nchunk > 4)) return 0;
    return p.nchunk;
}

// Scores and selects rows of decode indexer formats in one launch (plus a
// clear of the control words when rows span several workgroups).  Returns
// hipErrorNotSupported, launching nothing, for shapes and formats it does not
// take (then li_score + topk_select do the same work).
hipError_t li_topk_dispatch(const IndexerDev& a, int D_I, int dtype, int qg, int64_t ld, int K, int32_t* idx,
                            void* ws, size_t ws_bytes, int layer, hipStream_t st) {
    if (li_topk_fused_chunks(a, D_I, dtype, qg, ld, K, layer) == 0) return hipErrorNotSupported;
    const bool bf16 = dtype == LISFA_BF16 && qg == 1;
    const bool mx = dtype == LISFA_MXFP8 && D_I == 128;
    LtPlan p;
    lt_plan(a.R, ld, a.k, p);
    const size_t ctl_bytes = p.nchunk > 1 ? ((size_t)a.R * kLtCtlWords * 4 + 255) / 256 * 256 : 0;
    const int64_t row_bytes = p.nchunk > 1 ? lt_row_bytes(p.nchunk) : 0;
    const size_t need = ctl_bytes + (size_t)a.R * row_bytes;
    if (need > 0 && (!ws || ws_bytes < need || ((uintptr_t)ws & 255))) return hipErrorInvalidValue;
    LtArgs t;
    t.idx = idx;
    t.ctl = (uint32_t*)ws;
    t.xch = (uint8_t*)ws + ctl_bytes;
    t.row_bytes = row_bytes;
    t.ld = ld;
    t.K = K;
    t.kpw = (int32_t)p.kpw;
    t.lg_ept = p.lg_ept;
    t.nchunk = p.nchunk;
    if (p.nchunk > 1) {
        const int64_t words = (int64_t)a.R * kLtCtlWords;
        hipLaunchKernelGGL(lt_clear_kernel, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, st, t.ctl, words);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int mt = a.H_I <= 16 ? 1 : (a.H_I <= 32 ? 2 : 4);
#define LISFA_LT_CASE(F_, DI_, MT_) \
    if (mt == MT_) return launch_lt<F_, DI_, MT_>(a, t, st);
    if (bf16 && D_I == 128) {
        LISFA_LT_CASE(0, 128, 4) LISFA_LT_CASE(0, 128, 2) LISFA_LT_CASE(0, 128, 1)
    } else if (bf16 && D_I == 32) {
        LISFA_LT_CASE(0, 32, 4) LISFA_LT_CASE(0, 32, 2) LISFA_LT_CASE(0, 32, 1)
    } else if (mx) {
        LISFA_LT_CASE(1, 128, 4) LISFA_LT_CASE(1, 128, 2) LISFA_LT_CASE(1, 128, 1)
    } else {
        LISFA_LT_CASE(2, 128, 4) LISFA_LT_CASE(2, 128, 2) LISFA_LT_CASE(2, 128, 1)
    }
#undef LISFA_LT_CASE
    return hipErrorNotSupported;
}

}  // namespace lisfa
