// Decode-row indexer scoring shared by the score kernels and the fused
// score + Top-K kernels: one query row per sequence, the keys of a chunk of
// positions streamed from HBM into MFMA operand registers.
//
// score[r, s] = sum_j w[r, j] * ReLU(q_idx[r, j, :] . k_idx[slot(s), :]) for
// s <= row_pos[r] ("Large Language Model Inference Acceleration in Practice",
// section 1.2 Lightning Indexer and section 3.1: relevance scores followed by
// head-weight weighting).
#pragma once
#include "common.hpp"

namespace lisfa {

constexpr int kLiMaxBlocks = 512;  // block-table entries one workgroup may touch

// stands in for unaddressable key rows (one copy per code object)
static __device__ __attribute__((aligned(16))) uint8_t g_li_zero_row[256];

__device__ __forceinline__ f32x4 mfma16x16x32_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Positions row r sees: row_pos[r] + 1 clamped to [0, ld].
__device__ __forceinline__ int64_t li_visible(const IndexerDev& a, int r, int64_t ld) {
    int64_t vis = (int64_t)a.row_pos[r] + 1;
    if (vis < 0) vis = 0;
    if (vis > ld) vis = ld;
    return vis;
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

// Scores of keys [c0, kend) of row r (kend > c0, uniform across the
// workgroup); sink(key, score) receives each one once, from lanes 0..15.
template <int DI, int MT, class Sink>
__device__ __forceinline__ void li_dec_chunk(const IndexerDev& a, int r, int64_t c0, int64_t kend,
                                             int64_t* blk_slot0, int32_t* blk_lim, Sink&& sink) {
    constexpr int KS = DI / 32;
    constexpr int NT = 64 * kLiDecWaves;
    constexpr int P = kLiPrefetch;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
            if (lane < 16 && key < kend) sink(key, part * f);
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
// Scores of keys [c0, kend) of row r, as li_dec_chunk.
template <int MT, bool TOK, class Sink>
__device__ __forceinline__ void li_mx_chunk(const IndexerDev& a, int r, int64_t c0, int64_t kend,
                                            int64_t* blk_slot0, int32_t* blk_lim, Sink&& sink) {
    constexpr int DI = 128;
    constexpr int NB = DI / 32;          // scale blocks per row
    constexpr int NT = 64 * kLiDecWaves;
    constexpr int PG = kLiMxGroups;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
                if (lane < 16 && key < kend) sink(key, part * f);
            }
        }
    }
}

}  // namespace lisfa
