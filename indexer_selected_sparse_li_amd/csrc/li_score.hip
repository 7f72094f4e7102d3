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
#include "common.hpp"

namespace lisfa {

constexpr int kLiMaxBlocks = 512;  // block-table entries one workgroup may touch
constexpr int kLiNbuf = 4;         // tiles in the LDS ring
constexpr int64_t kLiL2Bytes = 4 << 20;   // L2 of one XCD

__device__ __attribute__((aligned(16))) uint8_t g_li_zero16[16];
__device__ __attribute__((aligned(16))) uint8_t g_li_zero_row[256];   // stands in for unaddressable key rows
__device__ float g_li_one = 1.0f;
__device__ float g_li_nan = __builtin_nanf("");

__device__ __forceinline__ f32x4 mfma16x16x32_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
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

// Decode (one query row per sequence, bf16 keys) -------------------------------
//
// Each key row is scored against a single query, so nothing is gained by
// staging tiles in LDS: every wavefront streams its own 16-key subtiles from
// HBM straight into MFMA B-operand registers, kLiPrefetch subtiles ahead, and
// the workgroup shares only the block map.  Lane l of a subtile loads, for
// K-step ks, the 16 bytes of key row l % 16 holding elements ks * 32 + 8 (l / 16)
// .. + 8, the same layout the query operand uses, so S[heads, keys] comes out
// of v_mfma_f32_16x16x32_bf16 exactly as in li_score_kernel.  Key rows are
// read once, with non-temporal loads.
constexpr int kLiDecWaves = 4;      // wavefronts per workgroup
constexpr int kLiPrefetch = 4;      // subtiles in flight per wavefront

template <int DI, int MT>
__global__ __launch_bounds__(64 * kLiDecWaves) void li_score_dec_kernel(IndexerDev a, float* __restrict__ scores,
                                                                     int64_t ld, int keys_per_wg) {
    constexpr int KS = DI / 32;
    constexpr int NT = 64 * kLiDecWaves;
    constexpr int P = kLiPrefetch;
    __shared__ int64_t blk_slot0[kLiMaxBlocks];
    __shared__ int32_t blk_lim[kLiMaxBlocks];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = blockIdx.y;
    const int64_t c0 = (int64_t)blockIdx.x * keys_per_wg;
    int64_t vis = (int64_t)a.row_pos[r] + 1;
    if (vis < 0) vis = 0;
    if (vis > ld) vis = ld;
    const int64_t kend = (c0 + keys_per_wg < vis) ? c0 + keys_per_wg : vis;
    if (c0 >= kend) return;  // uniform across the workgroup
    const int seq = a.row_seq[r];

    // block map of [c0, kend) (contiguous caches: virtual 64-token blocks)
    const bool seq_ok = seq >= 0 && seq < a.k.num_seqs;
    const int sh = a.k.paged ? a.k.bs_shift : 6;
    const int64_t bsz = (int64_t)1 << sh;
    const int64_t b0 = c0 >> sh;
    {
        const int nb = (int)(((kend - 1) >> sh) - b0 + 1);
        for (int i = tid; i < nb; i += NT) {
            const int64_t blk = b0 + i;
            int64_t s0 = -1;
            if (seq_ok) {
                if (a.k.paged) {
                    if (blk < a.k.bt_stride) {
                        const int32_t b = a.k.block_table[(int64_t)seq * a.k.bt_stride + blk];
                        if (b >= 0) s0 = (int64_t)b << sh;
                    }
                } else {
                    s0 = a.k.seq_base[seq] + blk * bsz;
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

    // query operand (row = head l % 16 of M-tile mt, 8 elements of K-step ks)
    // and head weights in the accumulator layout (4 heads per M-tile)
    const int g = lane >> 4;
    bf16x8 qa[MT][KS];
    float wv[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int head = mt * 16 + (lane & 15);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (head < a.H_I)
                qa[mt][ks] = *(const bf16x8*)(a.q + (((int64_t)r * a.H_I + head) * DI + ks * 32 + g * 8) * 2);
            else
                qa[mt][ks] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int h = mt * 16 + 4 * g + i;
            wv[mt][i] = h < a.H_I ? a.w[(int64_t)r * a.H_I + h] : 0.f;
        }
    }
    __syncthreads();  // block map ready

    // subtiles of this wave: u = wave, wave + W, ... over [c0, kend)
    const int nsub = (int)((kend - c0 + 15) / 16);
    const int mine = nsub > wave ? (nsub - wave + kLiDecWaves - 1) / kLiDecWaves : 0;
    // address of lane's key row in subtile i of this wave (zero row if the
    // position is past the row or not addressable) and its score factor
    auto locate = [&](int i, const uint8_t*& gp, float& fac) {
        const int64_t key = c0 + (int64_t)(wave + i * kLiDecWaves) * 16 + (lane & 15);
        gp = g_li_zero_row + g * 16;
        fac = __builtin_nanf("");
        if (i < mine && key < kend) {
            const int bi = (int)((key >> sh) - b0);
            const int off = (int)(key & (bsz - 1));
            if (off < blk_lim[bi]) {
                gp = a.k.data + (blk_slot0[bi] + off) * a.k.row_stride + g * 16;
                fac = 1.f;
            }
        }
    };
    static_assert(DI * 2 <= 256, "zero row covers one key row");
    auto fetch = [&](const uint8_t* gp, bf16x8 (&kb)[KS]) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kb[ks] = __builtin_nontemporal_load((const bf16x8*)(gp + ks * 64));
    };

    bf16x8 kbuf[P][KS];
    float fac[P];
#pragma unroll
    for (int j = 0; j < P; ++j) {
        const uint8_t* gp;
        locate(j, gp, fac[j]);
        fetch(gp, kbuf[j]);
    }
    // whole groups of P subtiles: those past this wave's share score the
    // zero row and their stores are masked
    for (int i0 = 0; i0 < mine; i0 += P) {
#pragma unroll
        for (int j = 0; j < P; ++j) {
            const int i = i0 + j;
            f32x4 acc[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) acc[mt] = mfma16x16x32_bf16(qa[mt][ks], kbuf[j][ks], acc[mt]);
            const float f = fac[j];
            // refill this slot with subtile i + P
            {
                const uint8_t* gp;
                locate(i + P, gp, fac[j]);
                fetch(gp, kbuf[j]);
            }
            // ReLU as an integer max on the bit pattern (negative floats,
            // -0.0 included, are negative integers; +0.0 is 0)
            float part = 0.f;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int bits = __float_as_int(acc[mt][q]);
                    part = fmaf(wv[mt][q], __int_as_float(bits > 0 ? bits : 0), part);
                }
            {
                const auto w16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(part), __float_as_uint(part), false, false);
                part = __uint_as_float(w16[0]) + __uint_as_float(w16[1]);
                const auto w32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(part), __float_as_uint(part), false, false);
                part = __uint_as_float(w32[0]) + __uint_as_float(w32[1]);
            }
            const int64_t key = c0 + (int64_t)(wave + i * kLiDecWaves) * 16 + lane;
            if (lane < 16 && key < kend) scores[(int64_t)r * ld + key] = part * f;
        }
    }
}

// Decode with MXFP8 queries and keys -------------------------------------------
//
// The pages' indexer format ("Day0 Inference Adaptation and Performance
// Optimization for Kimi K3.1 Pro", section 4; "... for a New Model", section
// 4): e4m3 elements with one power-of-two (E8M0) scale per 32 consecutive
// elements, here D_I = 128 = four blocks per row.  gfx950's block-scaled MFMA
// v_mfma_scale_f32_16x16x128_f8f6f4 multiplies a 16 x 128 e4m3 block of
// queries (heads) by a 128 x 16 block of keys and applies both operands' E8M0
// scales per 32-element block, so one instruction per (16-head tile, 16-key
// subtile) yields the exact scaled dot products.  Operand layout (checked
// bit-exactly on the GPU): lane l holds row l % 16, bytes [16 g, 16 g + 16)
// and [64 + 16 g, 64 + 16 g + 16) of it (g = l / 16), and supplies the scale
// of row l % 16, block g in byte 0 of its scale operand.  The accumulator
// layout is that of the other 16x16 MFMAs (lane = key l % 16, 4 heads per
// tile).
// Work: each wave streams whole groups of 64 keys (4 subtiles), kLiMxGroups
// groups ahead.  The keys' scale bytes are fetched with one coalesced dword
// per lane per group (lane l: the 4 scales of key l of the group) and handed
// to the lanes that need them with ds_bpermute: a per-lane byte gather per
// subtile, or a dword read by 4 lanes at once, costs much more.  ReLU is an
// integer max, the head sum two permlane swaps.  132 bytes per key instead
// of 256.
constexpr int kLiMxGroups = 2;

typedef int i32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ i32x8 mx_operand(const uint8_t* row, int g) {
    const u32x4 lo = __builtin_nontemporal_load((const u32x4*)(row + 16 * g));
    const u32x4 hi = __builtin_nontemporal_load((const u32x4*)(row + 64 + 16 * g));
    return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// TOK: e4m3 queries and keys with per-token fp32 scales instead (config-4
// style): the same instruction with unit E8M0 scales (127 = 2^0) gives the
// exact e4m3 dot products, the query scale is folded into the head weights
// and the key's scale is the score factor, in the order of the LDS-ring fp8
// kernel (w * s_q, then the weighted ReLU sum, then * s_k).
template <int MT, bool TOK = false>
__global__ __launch_bounds__(64 * kLiDecWaves) void li_score_mx_kernel(IndexerDev a, float* __restrict__ scores,
                                                                    int64_t ld, int keys_per_wg) {
    constexpr int DI = 128;
    constexpr int NB = DI / 32;          // scale blocks per row
    constexpr int NT = 64 * kLiDecWaves;
    constexpr int PG = kLiMxGroups;
    __shared__ int64_t blk_slot0[kLiMaxBlocks];
    __shared__ int32_t blk_lim[kLiMaxBlocks];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = blockIdx.y;
    const int64_t c0 = (int64_t)blockIdx.x * keys_per_wg;
    int64_t vis = (int64_t)a.row_pos[r] + 1;
    if (vis < 0) vis = 0;
    if (vis > ld) vis = ld;
    const int64_t kend = (c0 + keys_per_wg < vis) ? c0 + keys_per_wg : vis;
    if (c0 >= kend) return;  // uniform across the workgroup
    const int seq = a.row_seq[r];

    // block map of [c0, kend) (contiguous caches: virtual 64-token blocks)
    const bool seq_ok = seq >= 0 && seq < a.k.num_seqs;
    const int sh = a.k.paged ? a.k.bs_shift : 6;
    const int64_t bsz = (int64_t)1 << sh;
    const int64_t b0 = c0 >> sh;
    {
        const int nb = (int)(((kend - 1) >> sh) - b0 + 1);
        for (int i = tid; i < nb; i += NT) {
            const int64_t blk = b0 + i;
            int64_t s0 = -1;
            if (seq_ok) {
                if (a.k.paged) {
                    if (blk < a.k.bt_stride) {
                        const int32_t b = a.k.block_table[(int64_t)seq * a.k.bt_stride + blk];
                        if (b >= 0) s0 = (int64_t)b << sh;
                    }
                } else {
                    s0 = a.k.seq_base[seq] + blk * bsz;
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

    // query operand of head tile mt (row = head mt * 16 + l % 16) with its
    // E8M0 scale (block g), and head weights in the accumulator layout
    const int g = lane >> 4;
    i32x8 qa[MT];
    int qs[MT];
    float wv[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int head = mt * 16 + (lane & 15);
        if (head < a.H_I) {
            const int64_t hr = (int64_t)r * a.H_I + head;
            qa[mt] = mx_operand(a.q + hr * DI, g);
            qs[mt] = TOK ? 127 : a.q_mx_scale[hr * NB + g];
        } else {
            qa[mt] = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
            qs[mt] = 127;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int h = mt * 16 + 4 * g + i;
            float wvv = 0.f;
            if (h < a.H_I) {
                wvv = a.w[(int64_t)r * a.H_I + h];
                if constexpr (TOK) wvv *= a.q_scale_per_head ? a.q_scale[(int64_t)r * a.H_I + h] : a.q_scale[r];
            }
            wv[mt][i] = wvv;
        }
    }
    __syncthreads();  // block map ready

    // 64-key groups of this wave: u = wave, wave + W, ... over [c0, kend)
    const int ngrp = (int)((kend - c0 + 63) / 64);
    const int mine = ngrp > wave ? (ngrp - wave + kLiDecWaves - 1) / kLiDecWaves : 0;
    auto slot_of_key = [&](int64_t key) -> int64_t {   // -1: past the row or not addressable
        if (key >= kend) return -1;
        const int bi = (int)((key >> sh) - b0);
        const int off = (int)(key & (bsz - 1));
        return off < blk_lim[bi] ? blk_slot0[bi] + off : -1;
    };
    // subtile s4 of group i: operand of key 16 s4 + l % 16 of the group (the
    // zero row and factor NaN where there is no key); the group's scale dword:
    // the 4 scales of key l of the group (2^0 where there is none)
    auto fetch_sub = [&](int i, int s4, i32x8& kb, float& fac) {
        const int64_t base = c0 + (int64_t)(wave + i * kLiDecWaves) * 64;
        const int64_t slot = i < mine ? slot_of_key(base + 16 * s4 + (lane & 15)) : -1;
        kb = mx_operand(slot >= 0 ? a.k.data + slot * a.k.row_stride : g_li_zero_row, g);
        if constexpr (TOK) fac = slot >= 0 ? a.k.scale[slot / a.k.scale_group] : __builtin_nanf("");
        else fac = slot >= 0 ? 1.f : __builtin_nanf("");
    };
    auto fetch_scales = [&](int i) -> uint32_t {
        if constexpr (TOK) return 0x7F7F7F7Fu;
        const int64_t base = c0 + (int64_t)(wave + i * kLiDecWaves) * 64;
        const int64_t ks = i < mine ? slot_of_key(base + lane) : -1;
        return ks >= 0 ? __builtin_nontemporal_load((const uint32_t*)(a.k.mx_scale + ks * NB)) : 0x7F7F7F7Fu;
    };
    static_assert(DI <= 256, "zero row covers one key row");

    i32x8 kbuf[PG][4];
    uint32_t sbuf[PG];
    float fac[PG][4];
#pragma unroll
    for (int j = 0; j < PG; ++j) {
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) fetch_sub(j, s4, kbuf[j][s4], fac[j][s4]);
        sbuf[j] = fetch_scales(j);
    }
    for (int i0 = 0; i0 < mine; i0 += PG) {
#pragma unroll
        for (int j = 0; j < PG; ++j) {
            const int i = i0 + j;
            const int64_t base = c0 + (int64_t)(wave + i * kLiDecWaves) * 64;
            uint32_t sw = sbuf[j];
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) {
                // byte g of the scale dword held by the lane of this lane's key
                const uint32_t w = (uint32_t)__builtin_amdgcn_ds_bpermute((16 * s4 + (lane & 15)) * 4, (int)sw);
                const int ksc = (int)((w >> (8 * g)) & 255u);
                f32x4 acc[MT];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    acc[mt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        qa[mt], kbuf[j][s4], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, qs[mt], 0, ksc);
                const float f = fac[j][s4];
                fetch_sub(i + PG, s4, kbuf[j][s4], fac[j][s4]);   // same subtile of the group PG ahead
                if (s4 == 3) sbuf[j] = fetch_scales(i + PG);
                float part = 0.f;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int bits = __float_as_int(acc[mt][q]);
                        part = fmaf(wv[mt][q], __int_as_float(bits > 0 ? bits : 0), part);
                    }
                const auto w16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(part), __float_as_uint(part), false, false);
                part = __uint_as_float(w16[0]) + __uint_as_float(w16[1]);
                const auto w32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(part), __float_as_uint(part), false, false);
                part = __uint_as_float(w32[0]) + __uint_as_float(w32[1]);
                const int64_t key = base + 16 * s4 + lane;
                if (lane < 16 && key < kend) scores[(int64_t)r * ld + key] = part * f;
            }
        }
    }
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
    // on uniform and on mixed-length batches; finer chunks are slower)
    const int64_t want_wg = 256;
    int64_t nchunk = (want_wg + a.R - 1) / a.R;
    int64_t kpw = (max_visible + nchunk - 1) / nchunk;
    if (kpw < 1024) kpw = 1024;
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
    if (kpw < 1024) kpw = 1024;
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
