// Lightning indexer scores on gfx950 MFMA.
//
// score[r, s] = sum_j w[r, j] * ReLU(q_idx[r, j, :] . k_idx[slot(s), :]) for
// s <= row_pos[r] ("Large Language Model Inference Acceleration in Practice",
// section 1.2 Lightning Indexer and section 3.1: relevance scores followed by
// head-weight weighting).
//
// Work decomposition.  A workgroup of 8 wavefronts owns QG query rows of one
// sequence and a contiguous chunk of key positions, streamed in tiles of TK
// keys through a 4-deep LDS ring:
//   * tiles are gathered with direct global->LDS 16-byte loads (no VGPR
//     staging), three tiles in flight while one is consumed, with exact
//     vmcnt waits; rows are stored unpadded with their 16-byte chunks
//     XOR-swizzled by row so operand reads are bank-conflict free;
//   * one fp32 factor per key rides along in the same ring (fp8: the key's
//     scale; bf16: 1; NaN for a position the cache cannot address);
//   * wave w scores query row (w % QG) against 16-key subtiles of the tile:
//     decode (QG = 1) splits each tile over the 8 waves, prefill (QG = 8)
//     gives every wave its own query and all subtiles.
// Per 16-key subtile a wave computes S[heads, keys] with v_mfma_f32_16x16x32
// (A = the query's heads, held in VGPRs; B = K^T from LDS).  In the 16x16
// accumulator lane l holds key l%16 and 4 heads per M-tile, so the weighted
// ReLU sum over heads is 4*MT fused multiply-adds plus two lane exchanges.
// Scores are fp32 end to end.  MXFP8 keys (one E8M0 scale per 32 elements)
// use the block-scaled MFMA decode kernel further down.
#include "li_dec.hpp"

namespace lisfa {

constexpr int kLiNbuf = 4;         // tiles in the LDS ring
constexpr int64_t kLiL2Bytes = 4 << 20;   // L2 of one XCD

__device__ __attribute__((aligned(16))) uint8_t g_li_zero16[16];
__device__ float g_li_one = 1.0f;
__device__ float g_li_nan = __builtin_nanf("");

__device__ __forceinline__ f32x4 mfma16x16x32_fp8(int64_t a, int64_t b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a, b, c, 0, 0, 0);
}

template <int DI, int MT, int QG, bool FP8>
struct LiCfg {
    static constexpr int ELT = FP8 ? 1 : 2;
    static constexpr int RB = DI * ELT;                    // bytes of one key row
    static constexpr int CPK = RB / 16;                    // 16-byte chunks per row
    static constexpr int TK0 = 128;
    static constexpr int TK = (TK0 * CPK >= 512) ? TK0 : 512 / CPK;  // >= one chunk per thread
    static constexpr int LPT = TK * CPK / 512;             // chunk loads per thread per tile
    static constexpr int TILE = TK * RB;                   // bytes per tile
    static constexpr int NSUB = TK / 16;                   // 16-key subtiles per tile
    static constexpr int KS = DI / 32;                     // MFMA K-steps
    static_assert(TK * CPK % 512 == 0 && TK <= 512, "tile shape");
};

template <int DI, int MT, int QG, bool FP8>
__global__ __launch_bounds__(512) void li_score_kernel(IndexerDev a, float* __restrict__ scores,
                                                       int64_t ld, int keys_per_wg) {
    using C = LiCfg<DI, MT, QG, FP8>;
    constexpr int ELT = C::ELT, RB = C::RB, CPK = C::CPK, TK = C::TK, LPT = C::LPT;
    constexpr int TILE = C::TILE, NSUB = C::NSUB, KS = C::KS, NBUF = kLiNbuf;

    __shared__ __attribute__((aligned(16))) uint8_t ring[NBUF][TILE];
    __shared__ float kmul[NBUF][512];
    __shared__ int64_t blk_slot0[kLiMaxBlocks];
    __shared__ int32_t blk_lim[kLiMaxBlocks];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    // rows of this wave: QG <= 8: row wave % QG of the group; QG = 16: rows
    // wave and wave + 8 (each operand read then feeds both rows' products)
    constexpr int RPW = QG > 8 ? QG / 8 : 1;
    static_assert(QG <= 8 || QG % 8 == 0, "groups of up to 8 rows, or whole multiples of 8");
    const int r0 = blockIdx.y * QG;
    const int rw0 = r0 + wave % (QG < 8 ? QG : 8);
    const int64_t c0 = (int64_t)blockIdx.x * keys_per_wg;

    const int seq0 = a.row_seq[r0];
    int64_t gvis = 0;
#pragma unroll
    for (int i = 0; i < QG; ++i) {
        if (r0 + i < a.R) {
            int64_t v = (int64_t)a.row_pos[r0 + i] + 1;
            v = v < ld ? v : ld;
            gvis = v > gvis ? v : gvis;
        }
    }
    const int64_t kend = (c0 + keys_per_wg < gvis) ? c0 + keys_per_wg : gvis;
    if (c0 >= kend) return;  // uniform across the workgroup

    int64_t vis[RPW];
    bool row_ok[RPW], row_bad[RPW];
    int64_t vis_any = 0;
    bool live = false;
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        const int r = rw0 + 8 * i;
        vis[i] = 0;
        row_ok[i] = row_bad[i] = false;
        if (r < a.R) {
            vis[i] = (int64_t)a.row_pos[r] + 1;
            if (vis[i] < 0) vis[i] = 0;
            if (vis[i] > ld) vis[i] = ld;
            row_ok[i] = a.row_seq[r] == seq0;
            row_bad[i] = !row_ok[i];
            live = true;
            vis_any = vis[i] > vis_any ? vis[i] : vis_any;
        }
    }

    // Block map of [c0, kend): first slot and addressable length of each block.
    // Contiguous caches use virtual 64-token blocks.
    const bool seq_ok = seq0 >= 0 && seq0 < a.k.num_seqs;
    const int sh = a.k.paged ? a.k.bs_shift : 6;
    const int64_t bsz = (int64_t)1 << sh;
    const int64_t b0 = c0 >> sh;
    {
        const int nb = (int)(((kend - 1) >> sh) - b0 + 1);
        for (int i = tid; i < nb; i += 512) {
            const int64_t blk = b0 + i;
            int64_t s0 = -1;
            if (seq_ok) {
                if (a.k.paged) {
                    if (blk < a.k.bt_stride) {
                        const int32_t b = a.k.block_table[(int64_t)seq0 * a.k.bt_stride + blk];
                        if (b >= 0) s0 = (int64_t)b << sh;
                    }
                } else {
                    s0 = a.k.seq_base[seq0] + blk * bsz;
                }
            }
            int64_t lim = 0;
            if (s0 >= 0 && s0 < a.k.num_slots) {
                lim = a.k.num_slots - s0;
                lim = lim < bsz ? lim : bsz;
            }
            blk_slot0[i] = s0;
            blk_lim[i] = (int32_t)lim;
        }
    }

    // query heads of this wave's row in A-operand layout (row = head l%16, 8 d)
    // and weights in the accumulator's head layout (4 heads per M-tile)
    typedef typename std::conditional<FP8, int64_t, bf16x8>::type OpT;
    OpT qa[RPW][MT][KS];
    float wv[RPW][MT][4];
#pragma unroll
    for (int q = 0; q < RPW; ++q) {
        const int r = rw0 + 8 * q;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int head = mt * 16 + (lane & 15);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                if (row_ok[q] && head < a.H_I) {
                    const uint8_t* p = a.q + (((int64_t)r * a.H_I + head) * DI + ks * 32 + (lane >> 4) * 8) * ELT;
                    if constexpr (FP8) qa[q][mt][ks] = *(const int64_t*)p;
                    else qa[q][mt][ks] = *(const bf16x8*)p;
                } else {
                    if constexpr (FP8) qa[q][mt][ks] = 0;
                    else qa[q][mt][ks] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int h = mt * 16 + 4 * (lane >> 4) + i;
                float wvv = 0.f;
                if (row_ok[q] && h < a.H_I) {
                    wvv = a.w[(int64_t)r * a.H_I + h];
                    if constexpr (FP8)
                        wvv *= a.q_scale_per_head ? a.q_scale[(int64_t)r * a.H_I + h] : a.q_scale[r];
                }
                wv[q][mt][i] = wvv;
            }
        }
    }
    __syncthreads();  // block map ready

    // Tile loads.  Thread tid, load j: chunk position P = j * 512 + tid of the
    // tile, i.e. row P / CPK, stored position P % CPK, holding global chunk
    // (P % CPK) ^ (row % CPK).  Every wave issues exactly LPT + 1 loads per
    // tile (the extra one: 64 key factors), so vmcnt counts are uniform.
    const uint32_t ring0 = (uint32_t)(uintptr_t)(&ring[0][0]);
    const uint32_t kmul0 = (uint32_t)(uintptr_t)(&kmul[0][0]);
    // Every source address of a tile is computed (block-map reads from LDS)
    // before the first load goes out: the loads are opaque to the compiler,
    // which would otherwise wait for each lookup separately.
    auto issue_tile = [&](int64_t t0, int buf) {
        const uint8_t* src[LPT];
#pragma unroll
        for (int j = 0; j < LPT; ++j) {
            const int P = j * 512 + tid;
            const int row = P / CPK, pos = P % CPK;
            const int part = pos ^ (row % CPK);
            const int64_t kp = t0 + row;
            const bool inr = kp < kend;
            const int bi = inr ? (int)((kp >> sh) - b0) : 0;   // tiles may run past kend
            const int off = (int)(kp & (bsz - 1));
            const int lim = blk_lim[bi];                       // entry 0 always exists: read unconditionally
            const int64_t s0 = blk_slot0[bi];
            src[j] = (inr && off < lim) ? a.k.data + (s0 + off) * a.k.row_stride + part * 16 : g_li_zero16;
        }
        const float* fsrc = &g_li_nan;   // waves whose keys lie past the tile load a dummy
        {
            const int key = tid;
            if (key < TK) {
                const int64_t kp = t0 + key;
                const bool inr = kp < kend;
                const int bi = inr ? (int)((kp >> sh) - b0) : 0;
                const int off = (int)(kp & (bsz - 1));
                const int lim = blk_lim[bi];
                const int64_t s0 = blk_slot0[bi];
                if (inr && off < lim) {
                    if constexpr (FP8) fsrc = a.k.scale + (s0 + off) / a.k.scale_group;
                    else fsrc = &g_li_one;
                }
            }
        }
#pragma unroll
        for (int j = 0; j < LPT; ++j)
            lds_dma<16, 0>(src[j], ring0 + (uint32_t)(buf * TILE + (j * 512 + (tid & ~63)) * 16));
        lds_dma<4, 0>(fsrc, kmul0 + (uint32_t)((buf * 512 + (tid & ~63)) * 4));
    };

    // per-lane LDS byte offset of the B operand of subtile sub, K-step ks
    // (row = key l%16, 8 elements starting at ks*32 + (l/16)*8)
    const int krow = lane & 15;
    auto b_off = [&](int sub, int ks) -> uint32_t {
        const int rowi = sub * 16 + krow;
        const int byte = (ks * 32 + (lane >> 4) * 8) * ELT;
        const int chunk = (byte >> 4) ^ (rowi % CPK);
        return (uint32_t)(rowi * RB + chunk * 16 + (byte & 15));
    };

    const int ntiles = (int)((kend - c0 + TK - 1) / TK);
    // prologue: tiles 0 .. NBUF-2 in flight
#pragma unroll
    for (int p = 0; p < NBUF - 1; ++p)
        if (p < ntiles) issue_tile(c0 + (int64_t)p * TK, p);

    for (int t = 0; t < ntiles; ++t) {
        const int buf = t % NBUF;
        // wait for this wave's loads of tile t: tiles t+1 .. t+NBUF-2 may still fly
        const int later = (ntiles - 1 - t) < (NBUF - 2) ? (ntiles - 1 - t) : (NBUF - 2);
        if (later >= 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * (LPT + 1)) : "memory");
        else if (later == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LPT + 1) : "memory");
        else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();  // everyone's part of tile t landed; tile t-1 fully consumed
        if (t + NBUF - 1 < ntiles) issue_tile(c0 + (int64_t)(t + NBUF - 1) * TK, (t + NBUF - 1) % NBUF);

        const int64_t t0 = c0 + (int64_t)t * TK;
        const lds_u8* T = (const lds_u8*)&ring[buf][0];
        // subtiles of this wave: decode splits the tile over the 8 waves.  The
        // products and head sums of all of them come first, in one branch-free
        // block the compiler can software-pipeline (operand reads of subtile
        // u + 1 under the products of u); the stores follow.
        constexpr int SUBW = QG == 1 ? NSUB / 8 : NSUB;
        const int64_t tfirst = t0 + (QG == 1 ? wave * 16 : 0);
        if (live && tfirst < vis_any) {                  // wave-uniform
            // in batches of SB subtiles (fewer scores held at once with two rows)
            constexpr int SB = (RPW > 1 && SUBW > 4) ? 4 : SUBW;
            static_assert(SUBW % SB == 0, "whole batches");
#pragma unroll
            for (int u0 = 0; u0 < SUBW; u0 += SB) {
                float sc[RPW][SB];
#pragma unroll
                for (int uu = 0; uu < SB; ++uu) {
                    const int u = u0 + uu;
                    const int sub = QG == 1 ? (u * 8 + wave) : u;
                    f32x4 acc[RPW][MT];
#pragma unroll
                    for (int q = 0; q < RPW; ++q)
#pragma unroll
                        for (int mt = 0; mt < MT; ++mt) acc[q][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) {
                        const uint32_t bo = b_off(sub, ks);
                        if constexpr (FP8) {
                            const int64_t b = *(const __attribute__((address_space(3))) int64_t*)(T + bo);
#pragma unroll
                            for (int q = 0; q < RPW; ++q)
#pragma unroll
                                for (int mt = 0; mt < MT; ++mt)
                                    acc[q][mt] = mfma16x16x32_fp8(qa[q][mt][ks], b, acc[q][mt]);
                        } else {
                            const bf16x8 b = *(const lds_bf16x8*)(T + bo);
#pragma unroll
                            for (int q = 0; q < RPW; ++q)
#pragma unroll
                                for (int mt = 0; mt < MT; ++mt)
                                    acc[q][mt] = mfma16x16x32_bf16(qa[q][mt][ks], b, acc[q][mt]);
                        }
                    }
#pragma unroll
                    for (int q = 0; q < RPW; ++q) {
                        float part = 0.f;
#pragma unroll
                        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                // ReLU as an integer max on the bit pattern (negative
                                // floats, -0.0 included, are negative integers)
                                const int bits = __float_as_int(acc[q][mt][i]);
                                part = fmaf(wv[q][mt][i], __int_as_float(bits > 0 ? bits : 0), part);
                            }
                        {   // sum over the four 16-lane groups (lanes l ^ 16, l ^ 32) without LDS
                            const auto w16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(part), __float_as_uint(part), false, false);
                            part = __uint_as_float(w16[0]) + __uint_as_float(w16[1]);
                            const auto w32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(part), __float_as_uint(part), false, false);
                            part = __uint_as_float(w32[0]) + __uint_as_float(w32[1]);
                        }
                        sc[q][uu] = part;
                    }
                }
#pragma unroll
                for (int q = 0; q < RPW; ++q) {
                    const int r = rw0 + 8 * q;
#pragma unroll
                    for (int uu = 0; uu < SB; ++uu) {
                        const int sub = QG == 1 ? ((u0 + uu) * 8 + wave) : u0 + uu;
                        const int64_t key = t0 + sub * 16 + (lane & 15);
                        if (lane < 16 && key < vis[q] && (row_ok[q] || row_bad[q]))
                            scores[(int64_t)r * ld + key] =
                                row_ok[q] ? sc[q][uu] * kmul[buf][sub * 16 + lane] : __builtin_nanf("");
                    }
                }
            }
        }
    }
}

// Decode kernels (one query row per sequence): the scoring loops live in
// li_dec.hpp, shared with the fused score + Top-K kernels.
template <int DI, int MT>
__global__ __launch_bounds__(64 * kLiDecWaves) void li_score_dec_kernel(IndexerDev a, float* __restrict__ scores,
                                                                     int64_t ld, int keys_per_wg) {
    __shared__ int64_t blk_slot0[kLiMaxBlocks];
    __shared__ int32_t blk_lim[kLiMaxBlocks];
    const int r = blockIdx.y;
    const int64_t c0 = (int64_t)blockIdx.x * keys_per_wg;
    const int64_t vis = li_visible(a, r, ld);
    const int64_t kend = (c0 + keys_per_wg < vis) ? c0 + keys_per_wg : vis;
    if (c0 >= kend) return;  // uniform across the workgroup
    float* srow = scores + (int64_t)r * ld;
    li_dec_chunk<DI, MT>(a, r, c0, kend, blk_slot0, blk_lim, [&](int64_t key, float v) { srow[key] = v; });
}

template <int MT, bool TOK = false>
__global__ __launch_bounds__(64 * kLiDecWaves) void li_score_mx_kernel(IndexerDev a, float* __restrict__ scores,
                                                                    int64_t ld, int keys_per_wg) {
    __shared__ int64_t blk_slot0[kLiMaxBlocks];
    __shared__ int32_t blk_lim[kLiMaxBlocks];
    const int r = blockIdx.y;
    const int64_t c0 = (int64_t)blockIdx.x * keys_per_wg;
    const int64_t vis = li_visible(a, r, ld);
    const int64_t kend = (c0 + keys_per_wg < vis) ? c0 + keys_per_wg : vis;
    if (c0 >= kend) return;  // uniform across the workgroup
    float* srow = scores + (int64_t)r * ld;
    li_mx_chunk<MT, TOK>(a, r, c0, kend, blk_slot0, blk_lim, [&](int64_t key, float v) { srow[key] = v; });
}

// host-side launcher ---------------------------------------------------------

template <int DI, int MT, int QG, bool FP8>
static hipError_t launch_li(const IndexerDev& a, float* scores, int64_t ld, int64_t max_visible,
                            hipStream_t stream) {
    constexpr int TK = LiCfg<DI, MT, QG, FP8>::TK;
    const int sh = a.k.paged ? a.k.bs_shift : 6;
    const int64_t bsz = (int64_t)1 << sh;
    // keys per workgroup: enough workgroups to fill 256 CUs a few times over
    const int64_t groups = (a.R + QG - 1) / QG;
    const int64_t want_wg = 256;   // about one long-running workgroup per CU
    int64_t nchunk = (want_wg + groups - 1) / groups;
    int64_t kpw = (max_visible + nchunk - 1) / nchunk;
    const int64_t min_kpw = QG == 1 ? 4 * TK : 2048;
    if (kpw < min_kpw) kpw = min_kpw;
    // chunks start on tile and block boundaries
    const int64_t align = bsz > TK ? bsz : TK;
    kpw = (kpw + align - 1) / align * align;
    const int64_t cap = (int64_t)(kLiMaxBlocks - 1) * bsz / align * align;
    if (kpw > cap) kpw = cap;
    if (kpw > (1 << 30)) kpw = (int64_t)(1 << 30) / align * align;
    nchunk = (max_visible + kpw - 1) / kpw;
    if (nchunk < 1) nchunk = 1;
    if (QG > 1) {
        // Grouped rows of one sequence all stream the same keys.  Workgroup
        // ids go round-robin over the 8 XCDs, so with a power-of-two number
        // of key chunks (<= 8) every XCD streams one fixed chunk; keeping a
        // chunk's keys within the XCD's L2 lets all groups on it share them
        // (a 1024-row prefill chunk at 65536 keys: 2000 -> 1100 us per call
        // with 8 MB -> 4 MB chunks).
        const int64_t l2_keys = kLiL2Bytes / LiCfg<DI, MT, QG, FP8>::RB;
        int64_t nc = 1;
        while (nc < 8 && (max_visible + nc - 1) / nc > l2_keys) nc *= 2;
        if (nc > nchunk) {
            int64_t k2 = (max_visible + nc - 1) / nc;
            k2 = (k2 + align - 1) / align * align;
            if (k2 < kpw) {
                kpw = k2;
                nchunk = (max_visible + kpw - 1) / kpw;
            }
        }
    }
    dim3 grid((unsigned)nchunk, (unsigned)groups);
    hipLaunchKernelGGL((li_score_kernel<DI, MT, QG, FP8>), grid, dim3(512), 0, stream, a, scores, ld, (int)kpw);
    return hipGetLastError();
}

template <int DI, int MT>
static hipError_t launch_li_dec(const IndexerDev& a, float* scores, int64_t ld, int64_t max_visible,
                                hipStream_t stream) {
    const int sh = a.k.paged ? a.k.bs_shift : 6;
    const int64_t bsz = (int64_t)1 << sh;
    // one four-wave workgroup per CU (measured against two per CU: 2 % faster
    // on uniform and on mixed-length batches; finer chunks are slower).  Few
    // rows still get about 256 workgroups, down to two blocks of 64 keys each:
    // one row of 32768 keys takes 5.6 us so against 11.1 us with 1024-key chunks
    const int64_t want_wg = 256;
    int64_t nchunk = (want_wg + a.R - 1) / a.R;
    int64_t kpw = (max_visible + nchunk - 1) / nchunk;
    if (kpw < 128) kpw = 128;
    const int64_t align = bsz > 64 ? bsz : 64;   // chunks start on block boundaries
    kpw = (kpw + align - 1) / align * align;
    const int64_t cap = (int64_t)(kLiMaxBlocks - 1) * bsz / align * align;
    if (kpw > cap) kpw = cap;
    if (kpw > (1 << 30)) kpw = (int64_t)(1 << 30) / align * align;
    nchunk = (max_visible + kpw - 1) / kpw;
    if (nchunk < 1) nchunk = 1;
    dim3 grid((unsigned)nchunk, (unsigned)a.R);
    hipLaunchKernelGGL((li_score_dec_kernel<DI, MT>), grid, dim3(64 * kLiDecWaves), 0, stream, a, scores, ld,
                       (int)kpw);
    return hipGetLastError();
}

template <int MT, bool TOK>
static hipError_t launch_li_mx(const IndexerDev& a, float* scores, int64_t ld, int64_t max_visible,
                               hipStream_t stream) {
    const int sh = a.k.paged ? a.k.bs_shift : 6;
    const int64_t bsz = (int64_t)1 << sh;
    const int64_t want_wg = 512;
    int64_t nchunk = (want_wg + a.R - 1) / a.R;
    int64_t kpw = (max_visible + nchunk - 1) / nchunk;
    // few rows: chunks down to 512 keys (one MXFP8 row of 32768 keys: 6.9 us
    // against 9.8 us with 1024-key chunks; 256 and 128 measured no better)
    if (kpw < 512) kpw = 512;
    const int64_t align = bsz > 64 ? bsz : 64;
    kpw = (kpw + align - 1) / align * align;
    const int64_t cap = (int64_t)(kLiMaxBlocks - 1) * bsz / align * align;
    if (kpw > cap) kpw = cap;
    if (kpw > (1 << 30)) kpw = (int64_t)(1 << 30) / align * align;
    nchunk = (max_visible + kpw - 1) / kpw;
    if (nchunk < 1) nchunk = 1;
    dim3 grid((unsigned)nchunk, (unsigned)a.R);
    hipLaunchKernelGGL((li_score_mx_kernel<MT, TOK>), grid, dim3(64 * kLiDecWaves), 0, stream, a, scores, ld,
                       (int)kpw);
    return hipGetLastError();
}

hipError_t li_score_dispatch(const IndexerDev& a, int D_I, int dtype, int qg, float* scores, int64_t ld,
                             int64_t max_visible, hipStream_t stream) {
    const int mt = a.H_I <= 16 ? 1 : (a.H_I <= 32 ? 2 : 4);
    if (dtype == LISFA_MXFP8) {   // one row at a time whatever the grouping
        if (D_I != 128) return hipErrorInvalidValue;
        if (mt == 4) return launch_li_mx<4, false>(a, scores, ld, max_visible, stream);
        if (mt == 2) return launch_li_mx<2, false>(a, scores, ld, max_visible, stream);
        return launch_li_mx<1, false>(a, scores, ld, max_visible, stream);
    }
    const int fp8 = dtype == LISFA_FP8_E4M3;
    if (qg == 1 && fp8 != 0 && D_I == 128) {   // one row at a time: stream the keys
        if (mt == 4) return launch_li_mx<4, true>(a, scores, ld, max_visible, stream);
        if (mt == 2) return launch_li_mx<2, true>(a, scores, ld, max_visible, stream);
        return launch_li_mx<1, true>(a, scores, ld, max_visible, stream);
    }
    if (qg == 1 && fp8 == 0) {
        if (D_I == 128 && mt == 4) return launch_li_dec<128, 4>(a, scores, ld, max_visible, stream);
        if (D_I == 128 && mt == 2) return launch_li_dec<128, 2>(a, scores, ld, max_visible, stream);
        if (D_I == 128 && mt == 1) return launch_li_dec<128, 1>(a, scores, ld, max_visible, stream);
        if (D_I == 32 && mt == 4) return launch_li_dec<32, 4>(a, scores, ld, max_visible, stream);
        if (D_I == 32 && mt == 2) return launch_li_dec<32, 2>(a, scores, ld, max_visible, stream);
        if (D_I == 32 && mt == 1) return launch_li_dec<32, 1>(a, scores, ld, max_visible, stream);
    }
    // 16-row groups are built for the 64 x 128 indexer; other shapes take the
    // 16-aligned group as two 8-row groups.  What reaches the grouped kernel:
    // bf16 keys with 8- or 16-row groups, per-token fp8 keys with 8- or 16-row
    // groups, and per-token fp8 keys with D_I = 32 one row at a time.
    if (qg == 16 && !(D_I == 128 && mt == 4)) qg = 8;
#define LISFA_LI_CASE(DI_, MT_, QG_, F8_)                                                    \
    if (D_I == DI_ && mt == MT_ && qg == QG_ && (fp8 != 0) == F8_)                            \
        return launch_li<DI_, MT_, QG_, F8_>(a, scores, ld, max_visible, stream);
    LISFA_LI_CASE(128, 4, 16, false)
    LISFA_LI_CASE(128, 4, 16, true)
    LISFA_LI_CASE(128, 4, 8, false)
    LISFA_LI_CASE(128, 4, 8, true)
    LISFA_LI_CASE(128, 2, 8, false)
    LISFA_LI_CASE(128, 2, 8, true)
    LISFA_LI_CASE(128, 1, 8, false)
    LISFA_LI_CASE(128, 1, 8, true)
    LISFA_LI_CASE(32, 4, 8, false)
    LISFA_LI_CASE(32, 4, 1, true)
    LISFA_LI_CASE(32, 4, 8, true)
    LISFA_LI_CASE(32, 2, 8, false)
    LISFA_LI_CASE(32, 2, 1, true)
    LISFA_LI_CASE(32, 2, 8, true)
    LISFA_LI_CASE(32, 1, 8, false)
    LISFA_LI_CASE(32, 1, 1, true)
    LISFA_LI_CASE(32, 1, 8, true)
#undef LISFA_LI_CASE
    return hipErrorInvalidValue;
}

}  // namespace lisfa
