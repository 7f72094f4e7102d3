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
constexpr int kLtMaxKeys = 16384;              // positions of one workgroup (LDS keys)
constexpr int kLtMaxMembers = 64;              // workgroups per row
constexpr int kLtMaxWg = 256;                  // workgroups of a launch that exchanges
constexpr int kLtBins = 4096;
constexpr int kLtLevels = 3;                   // 12 + 12 + 8 key bits
constexpr int kLtListMax = 256;                // boundary bins ranked directly up to this size
constexpr int kLtCtlWords = 16;                // per row: counter, time-out flag (own 64 bytes)
constexpr uint32_t kLtSpinCap = 1u << 21;      // polls (each >= ~0.1 us) before giving up
// per-row exchange area: member ranges, boundary list, suffix-sum histograms
constexpr int64_t kLtListOff = 512;
constexpr int64_t kLtHistOff = kLtListOff + kLtListMax * 8;

inline int64_t lt_row_bytes(int nchunk) { return kLtHistOff + (int64_t)kLtLevels * nchunk * kLtBins * 4; }

struct LtArgs {
    int32_t* idx;        // [R, K] out
    uint32_t* ctl;       // [R, kLtCtlWords], zero at launch
    uint8_t* xch;        // [R, row_bytes]
    int64_t row_bytes;
    int64_t ld;          // visible positions of a row: row_pos + 1 clamped to [0, ld]
    int32_t K;
    int32_t kpw;         // positions per workgroup
    int32_t nchunk;      // workgroups per row (grid x)
};

__device__ __forceinline__ void st_dev(uint32_t* p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_dev(const uint32_t* p) {
    return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Four words at device scope.  Compiler-generated stores: a 16-byte store
// issued from inline assembly reads its data registers after the next
// instructions may have rewritten them (the compiler cannot guard a store it
// does not see), which corrupted the first word of such stores here.
__device__ __forceinline__ void st_dev4(uint32_t* p, u32x4 v) {
    st_dev(p, v.x);
    st_dev(p + 1, v.y);
    st_dev(p + 2, v.z);
    st_dev(p + 3, v.w);
}

// Row barrier: returns once `target` arrivals are counted in ctl[0].
__device__ __forceinline__ void lt_barrier(uint32_t* ctl, uint32_t target) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's stores acknowledged
    __syncthreads();
    if (threadIdx.x == 0) {
        __hip_atomic_fetch_add(ctl, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        uint32_t it = 0;
        while (ld_dev(ctl) < target) {
            __builtin_amdgcn_s_sleep(2);
            if (++it == kLtSpinCap) {
                st_dev(ctl + 1, 1u);
                break;
            }
        }
    }
    __syncthreads();
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, o));
    return v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o));
    return v;
}
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += (uint32_t)__shfl_xor((int)v, o);
    return v;
}
__device__ __forceinline__ uint32_t wave_incl_prefix_u32(uint32_t v, int lane) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t u = (uint32_t)__shfl_up((int)v, o);
        if (lane >= o) v += u;
    }
    return v;
}

enum { kLtAll = 0, kLtTie = 1, kLtList = 2 };

// FMT 0: bf16 keys (D_I = DI); 1: MXFP8 keys; 2: per-token fp8 keys (D_I = 128).
template <int FMT, int DI, int MT>
__global__ __launch_bounds__(kLtThreads) void li_topk_kernel(IndexerDev a, LtArgs t) {
    extern __shared__ uint32_t keys[];   // [kpw] order keys of the chunk
    __shared__ int64_t blk_slot0[kLiMaxBlocks];
    __shared__ int32_t blk_lim[kLiMaxBlocks];
    __shared__ __attribute__((aligned(16))) uint32_t hist[kLtBins];   // level histogram, then suffix sums
    __shared__ uint32_t sv[kLtMaxMembers][65];   // members' suffix sums at the 64 (+1) search points
    __shared__ uint32_t above[kLtMaxMembers];    // members' keys above the current bin
    __shared__ uint32_t inb[kLtMaxMembers];      // members' keys in the boundary bin
    __shared__ uint32_t gtl[kLtMaxMembers];      // list finish: members' bin keys above the K-th key
    __shared__ uint32_t xs[kLtMaxMembers];       // members' selected keys equal to the threshold key
    __shared__ uint32_t lkey[kLtListMax];
    __shared__ int32_t lpos[kLtListMax];
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

    auto sink = [&](int64_t key, float v) { keys[key - c0] = float_key(v); };
    if constexpr (FMT == 0)
        li_dec_chunk<DI, MT>(a, r, c0, kend, blk_slot0, blk_lim, sink);
    else
        li_mx_chunk<MT, FMT == 2>(a, r, c0, kend, blk_slot0, blk_lim, sink);

    uint32_t* ctl = t.ctl + (int64_t)r * kLtCtlWords;
    uint8_t* xr = t.xch + (int64_t)r * t.row_bytes;
    uint32_t* xrange = (uint32_t*)xr;
    uint32_t* xlist = (uint32_t*)(xr + kLtListOff);
    uint32_t nbar = 0;
    __syncthreads();   // keys complete

    // 1. key range of the row
    uint32_t kmn = 0xFFFFFFFFu, kmx = 0u;
    for (int j = tid; j < cnt; j += kLtThreads) {
        const uint32_t k = keys[j];
        kmn = min(kmn, k);
        kmx = max(kmx, k);
    }
    kmn = wave_min_u32(kmn);
    kmx = wave_max_u32(kmx);
    if (lane == 0) {
        red[wave] = kmn;
        red[4 + wave] = kmx;
    }
    for (int i = tid; i < n; i += kLtThreads) above[i] = 0;
    __syncthreads();
    kmn = min(min(red[0], red[1]), min(red[2], red[3]));
    kmx = max(max(red[4], red[5]), max(red[6], red[7]));
    if (n > 1) {
        if (tid == 0) {
            st_dev(xrange + 2 * m, kmn);
            st_dev(xrange + 2 * m + 1, kmx);
        }
        lt_barrier(ctl, ++nbar * (uint32_t)n);
        if (wave == 0) {
            uint32_t v0 = 0xFFFFFFFFu, v1 = 0u;
            if (lane < n) {
                v0 = ld_dev(xrange + 2 * lane);
                v1 = ld_dev(xrange + 2 * lane + 1);
            }
            v0 = wave_min_u32(v0);
            v1 = wave_max_u32(v1);
            if (lane == 0) {
                bc[0] = v0;
                bc[1] = v1;
            }
        }
        __syncthreads();
        kmn = bc[0];
        kmx = bc[1];
    }

    // 2. histogram levels over [lo, hi]; need = how many of those are selected
    uint32_t lo = kmn, hi = kmx, need = (uint32_t)K;
    uint32_t Kt = 0, blo = 0, bhi = 0;
    int mode = kLtTie;
    for (int lev = 0; lev < kLtLevels; ++lev) {
        const uint32_t range = hi - lo;
        const int s = range < (uint32_t)kLtBins ? 0 : 20 - __builtin_clz(range);   // (range >> s) < 4096
        for (int b = tid; b < kLtBins; b += kLtThreads) hist[b] = 0;
        __syncthreads();
        for (int j = tid; j < cnt; j += kLtThreads) {
            const uint32_t k = keys[j];
            if (k >= lo && k <= hi) atomicAdd(&hist[(k - lo) >> s], 1u);
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
        const uint32_t incl = wave_incl_prefix_u32(acc, lane);
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
        const uint32_t* hg0 = (const uint32_t*)(xr + kLtHistOff) + (int64_t)lev * t.nchunk * kLtBins;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const u32x4 v = u32x4{hv[4 * q], hv[4 * q + 1], hv[4 * q + 2], hv[4 * q + 3]};
            *(u32x4*)&hist[16 * tid + 4 * q] = v;
            if (n > 1) st_dev4(const_cast<uint32_t*>(hg0) + (int64_t)m * kLtBins + 16 * tid + 4 * q, v);
        }
        if (n > 1)
            lt_barrier(ctl, ++nbar * (uint32_t)n);
        else
            __syncthreads();
        auto S = [&](int mm, int b) -> uint32_t {
            return n > 1 ? ld_dev(hg0 + (int64_t)mm * kLtBins + b) : hist[b];
        };
        // search: 64 points 64 i, then the 64 bins of the chosen segment
        for (int e = tid; e < n * 64; e += kLtThreads) sv[e >> 6][e & 63] = S(e >> 6, 64 * (e & 63));
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
        for (int e = tid; e < n * 64; e += kLtThreads) sv[e >> 6][e & 63] = S(e >> 6, 64 * i1 + (e & 63));
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
        blo = lo + (bstar << s);
        const uint64_t bh = (uint64_t)blo + (((uint64_t)1 << s) - 1);
        bhi = bh < hi ? (uint32_t)bh : hi;
        if (C == need) {
            mode = kLtAll;
            Kt = blo - 1;   // blo >= 1: no float has key 0
            break;
        }
        if (s == 0) {
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

    // 3. finish: per member, keys above Kt (gtl + above) and equal keys taken (xs)
    for (int mm = tid; mm < n; mm += kLtThreads) {
        gtl[mm] = 0;
        xs[mm] = 0;
    }
    if (mode == kLtList) {
        uint32_t base = 0;   // this member's first list slot
        for (int mm = 0; mm < m; ++mm) base += inb[mm];
        if (tid == 0) bc[6] = 0;
        __syncthreads();
        for (int j = tid; j < cnt; j += kLtThreads) {
            const uint32_t k = keys[j];
            if (k >= blo && k <= bhi) {
                const uint32_t p = atomicAdd(&bc[6], 1u);
                if (n > 1) {
                    if (base + p < (uint32_t)kLtListMax) {
                        st_dev(xlist + 2 * (base + p), k);
                        st_dev(xlist + 2 * (base + p) + 1, (uint32_t)(c0 + j));
                    }
                } else if (p < (uint32_t)kLtListMax) {
                    lkey[p] = k;
                    lpos[p] = (int32_t)(c0 + j);
                }
            }
        }
        uint32_t C = 0;
        for (int mm = 0; mm < n; ++mm) C += inb[mm];
        C = C < (uint32_t)kLtListMax ? C : (uint32_t)kLtListMax;
        if (n > 1) {
            lt_barrier(ctl, ++nbar * (uint32_t)n);
            for (int e = tid; e < (int)C; e += kLtThreads) {
                lkey[e] = ld_dev(xlist + 2 * e);
                lpos[e] = (int32_t)ld_dev(xlist + 2 * e + 1);
            }
        }
        __syncthreads();
        // the need-th largest (key descending, position ascending)
        for (int e = tid; e < (int)C; e += kLtThreads) {
            const uint32_t ke = lkey[e];
            const int32_t pe = lpos[e];
            uint32_t rk = 0;
            for (int u = 0; u < (int)C; ++u) {
                const uint32_t ku = lkey[u];
                rk += (ku > ke || (ku == ke && lpos[u] < pe)) ? 1u : 0u;
            }
            if (rk == need - 1) {
                bc[6] = ke;
                bc[7] = (uint32_t)pe;
            }
        }
        __syncthreads();
        Kt = bc[6];
        const int32_t Pt = (int32_t)bc[7];
        for (int e = tid; e < (int)C; e += kLtThreads) {
            int mm = lpos[e] / t.kpw;
            mm = mm < 0 ? 0 : (mm < n ? mm : n - 1);
            if (lkey[e] > Kt)
                atomicAdd(&gtl[mm], 1u);
            else if (lkey[e] == Kt && lpos[e] <= Pt)
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

    // 4. emission in position order: waves take contiguous runs of 64 keys
    const int nb = (cnt + 63) >> 6;
    const int b0 = wave * nb / kLiDecWaves, b1 = (wave + 1) * nb / kLiDecWaves;
    uint32_t g = 0, e = 0;
    for (int b = b0; b < b1; ++b) {
        const int j = 64 * b + lane;
        const bool v = j < cnt;
        const uint32_t k = v ? keys[j] : 0u;
        g += (uint32_t)__popcll(__ballot(v && k > Kt));
        e += (uint32_t)__popcll(__ballot(v && k == Kt));
    }
    if (lane == 0) {
        red[wave] = g;
        red[4 + wave] = e;
    }
    __syncthreads();
    uint32_t gw = 0, ew = 0;
    for (int w = 0; w < wave; ++w) {
        gw += red[w];
        ew += red[4 + w];
    }
    uint32_t pos = offset + gw + (ew < xm ? ew : xm);
    uint32_t eseen = ew;
    for (int b = b0; b < b1; ++b) {
        const int j = 64 * b + lane;
        const bool v = j < cnt;
        const uint32_t k = v ? keys[j] : 0u;
        const uint64_t eqm = __ballot(v && k == Kt);
        const uint32_t eq_before = eseen + lanemask_count(eqm);
        const bool sel = v && (k > Kt || (k == Kt && eq_before < xm));
        const uint64_t sm = __ballot(sel);
        if (sel) {
            const uint32_t slot = pos + lanemask_count(sm);
            if (slot < (uint32_t)K) out[slot] = (int32_t)(c0 + j);
        }
        pos += (uint32_t)__popcll(sm);
        eseen += (uint32_t)__popcll(eqm);
    }
}

__global__ void lt_clear_kernel(uint32_t* p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

namespace {

struct LtPlan {
    int64_t kpw;
    int nchunk;
};

// Chunking of the fused launch, or false when the shape is left to the
// separate score and Top-K kernels: more than kLtMaxMembers chunks per row,
// more than kLtMaxKeys positions per workgroup, or an exchanging launch of
// more than kLtMaxWg workgroups.
bool lt_plan(int R, int64_t ld, const CacheDev& c, LtPlan& p) {
    const int sh = c.paged ? c.bs_shift : 6;
    const int64_t bsz = (int64_t)1 << sh;
    const int64_t align = bsz > 64 ? bsz : 64;   // chunks start on block boundaries
    if (align > kLtMaxKeys) return false;
    int64_t nchunk = (kLtMaxWg + R - 1) / R;
    if (nchunk > kLtMaxMembers) nchunk = kLtMaxMembers;
    int64_t kpw = (ld + nchunk - 1) / nchunk;
    if (kpw < 1024) kpw = 1024;
    kpw = (kpw + align - 1) / align * align;
    if (kpw > kLtMaxKeys) kpw = kLtMaxKeys / align * align;
    const int64_t cap = (int64_t)(kLiMaxBlocks - 1) * bsz / align * align;   // the block map of a chunk
    if (kpw > cap) kpw = cap;
    if (kpw < 1) return false;
    nchunk = (ld + kpw - 1) / kpw;
    if (nchunk < 1) nchunk = 1;
    if (nchunk > kLtMaxMembers) return false;
    if (nchunk > 1 && nchunk * R > kLtMaxWg) return false;
    p.kpw = kpw;
    p.nchunk = (int)nchunk;
    return true;
}

template <int FMT, int DI, int MT>
hipError_t launch_lt(const IndexerDev& a, const LtArgs& t, hipStream_t st) {
    const size_t lds = (size_t)t.kpw * sizeof(uint32_t);
    hipLaunchKernelGGL((li_topk_kernel<FMT, DI, MT>), dim3((unsigned)t.nchunk, (unsigned)a.R), dim3(kLtThreads), lds,
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
    return ctl + (size_t)R * kLtHistOff + (size_t)kLtLevels * kLtMaxWg * kLtBins * 4;
}

// Scores and selects rows of decode indexer formats in one launch (plus a
// clear of the control words when rows span several workgroups).  Returns
// hipErrorNotSupported, launching nothing, for shapes and formats it does not
// take (then li_score + topk_select do the same work).
hipError_t li_topk_dispatch(const IndexerDev& a, int D_I, int dtype, int qg, int64_t ld, int K, int32_t* idx,
                            void* ws, size_t ws_bytes, hipStream_t st) {
    const bool bf16 = dtype == LISFA_BF16 && qg == 1;
    const bool mx = dtype == LISFA_MXFP8 && D_I == 128;
    const bool tok = dtype == LISFA_FP8_E4M3 && qg == 1 && D_I == 128;
    if (!bf16 && !mx && !tok) return hipErrorNotSupported;
    if (a.R < 1 || ld < 1 || K < 1) return hipErrorNotSupported;
    LtPlan p;
    if (!lt_plan(a.R, ld, a.k, p)) return hipErrorNotSupported;
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
