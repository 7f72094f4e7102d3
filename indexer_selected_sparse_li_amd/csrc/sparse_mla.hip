// Sparse MLA flash attention on gfx950 MFMA ("Large Language Model Inference
// Acceleration in Practice", section 1.2 SFA and section 3.1: the index
// pointers address the paged KV cache and feed the sparse attention
// directly; "Day0 Inference Adaptation and Performance Optimization for a New
// Model", section 3.1: the sparse module reads the main KV by the selected
// indices).
//
// For row r, head h and selected positions idx_k:
//   z_k = scale * q[r,h,:] . row_k      (row = [latent | rope], D_qk wide)
//   out[r,h,:] = sum_k softmax(z)_k * row_k[:D_latent],  lse = log sum_k e^{z_k}
//
// Work decomposition.  A workgroup owns one query row, 32*NHG heads and a
// contiguous range of the row's index list (split-K over the list when one
// row alone cannot fill the chip).  Every gathered latent row is therefore
// read from HBM once per (row, split) and shared by all heads of the
// workgroup through LDS.  Rows are gathered 32 at a time with direct
// global->LDS 16-byte loads (no VGPR staging) into a double-buffered, padded
// LDS tile, driven by the slot list computed once per workgroup.
//
// Wave pairs: wave (hg, dh) owns heads [32hg, 32hg+32) of the workgroup and
// the dh-th half of the QK^T reduction and of the value columns.
//   QK:  S^T[32 keys, 32 heads] += K_tile[32 x 16] * Q^T[16 x 32] per K-step
//        (v_mfma_f32_32x32x16_bf16; the query half stays in VGPRs), then the
//        two halves' partial logits are summed through LDS.
//   softmax: in the S^T accumulator layout lane l holds head l%32 and 16 of
//        the 32 keys, so max/sum need only one cross-half exchange and the
//        running (max, sum) of a head lives in one lane.
//   PV:  O^T[32 cols, 32 heads] += V^T[32 x 16 keys] * P^T[16 keys x 32 heads].
//        P^T's operand layout is exactly the S^T accumulator layout (keys of
//        the K-step permuted identically on both operands), so probabilities
//        go from accumulator to operand without any data movement.
// Online softmax in base 2 with fp32 statistics; probabilities are rounded to
// bf16 for the PV product, the normaliser is accumulated from the unrounded
// fp32 values.  fp8 rows are converted exactly to bf16 and their per-group
// fp32 factor is folded into the logit and into the probability.
#include "common.hpp"

namespace lisfa {

__device__ __attribute__((aligned(16))) uint8_t g_zero16[64];

constexpr int kSfaMaxKeys = 2048;  // index entries one workgroup handles

// XOR swizzle of the 16-byte chunks of LDS row r (values < 8, so a chunk stays
// inside its aligned group of 8).  With it, 16 consecutive rows read at one
// chunk (QK operand) hit 16 distinct bank groups, and the transpose reads of
// the PV operand (8 consecutive rows x 4 chunks) are at the 2-way minimum.
__device__ __forceinline__ int sfa_swz(int r) { return (((r >> 1) & 1) << 2) | ((r >> 2) & 3); }

template <int DLAT, int DROPE, bool FP8, int NHG, bool TSC = false>
__global__ __launch_bounds__(128 * NHG) void sfa_kernel(MlaDev a, int kps, int nsplit, int nhb,
                                                        __bf16* __restrict__ out, float* __restrict__ lse,
                                                        float* __restrict__ part_o,
                                                        float* __restrict__ part_lse) {
    constexpr int DQK = DLAT + DROPE;
    constexpr int ELT = FP8 ? 1 : 2;
    constexpr int RB = DQK * ELT;           // bytes per cached row
    constexpr int CPK = RB / 16;            // 16-byte chunks per row
    // bf16 rows whose chunk count is a multiple of 8: swizzled, unpadded rows
    // and transpose reads (ds_read_b64_tr_b16) for the value operand.
    // Otherwise: one pad chunk per row and gathered value reads.
    constexpr bool SWZ = !FP8 && (CPK % 8 == 0);
    constexpr int CPKP = SWZ ? CPK : CPK + 1;
    constexpr int RBP = CPKP * 16;          // LDS row stride
    constexpr int TROWS = 32;               // rows per tile
    constexpr int NBUF = 3;                 // tile ring: PV(t) | QK(t+1) | loading t+2
    constexpr int TCH = TROWS * CPKP;       // chunk positions per tile
    constexpr int NT = 128 * NHG;           // threads
    constexpr int NLD = (TCH + NT - 1) / NT;
    constexpr int KS = DQK / 16;            // QK K-steps
    constexpr int KS0 = (KS + 1) / 2;       // K-steps of the dh = 0 wave
    constexpr int DVH = DLAT / 2;           // value columns per wave
    constexpr int MTV = DVH / 32;           // PV M-tiles per wave
    constexpr bool ILV = !SWZ && (MTV % 4 == 0);  // interleaved value columns (gathered path)
    static_assert(DQK % 16 == 0 && DVH % 32 == 0, "shape");
    // TSC: fp8 rows with one fp32 scale per 128-column tile.  QK^T sums each
    // tile's K-steps apart and adds them with the key's tile scale; PV takes
    // the probabilities times the key's scale of the value tile.
    constexpr int NTL = TSC ? (DQK + 127) / 128 : 1;
    static_assert(!TSC || FP8, "tile scales come with fp8 rows");
    static_assert(!TSC || (ILV && DVH % 128 == 0) || NTL == 1, "value tiles: whole 128-column groups per wave");

    __shared__ __attribute__((aligned(16))) uint8_t tile[NBUF][TROWS * RBP];
    __shared__ int64_t roff[kSfaMaxKeys];              // byte offset of each selected row, -1 = skip
    __shared__ __attribute__((aligned(16))) float kvs[FP8 ? NTL * kSfaMaxKeys : 1];   // fp8 factors [tile][row]
                                                                                       // (0 for skipped rows)
    __shared__ uint32_t vmask[kSfaMaxKeys / 32];        // valid-row bits of each 32-row tile
    __shared__ __attribute__((aligned(16))) float xbuf[2][NHG * 2 * 4 * 64 * 4];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hg = wave >> 1, dh = wave & 1;
    // 1-D grid, XCD-aware: workgroups are dealt round-robin to the 8 XCDs, so
    // the nhb head blocks of one (row, split) get ids 8 apart and share the
    // XCD's L2 (and run at about the same time).
    const int bid = blockIdx.x;
    const int hb = (bid >> 3) % nhb;
    const int u = ((bid >> 3) / nhb) * 8 + (bid & 7);
    if (u >= a.R * nsplit) return;
    const int r = u / nsplit, sp = u % nsplit;
    const int k0 = sp * kps;
    const int k1 = (k0 + kps < a.K) ? k0 + kps : a.K;
    const int nk = k1 - k0;
    const int seq = a.row_seq[r];
    const int nt_fill = (nk + TROWS - 1) / TROWS;
    __shared__ int s_ntiles;
    if (tid == 0) s_ntiles = 1;

    // query half of this wave in B-operand layout (col = head, 8 consecutive d)
    const int head = hb * 32 * NHG + hg * 32 + (lane & 31);
    const int ksb = dh ? KS0 : 0;
    const int nks = dh ? KS - KS0 : KS0;
    bf16x8 qb[KS0];
#pragma unroll
    for (int j = 0; j < KS0; ++j) {
        if (j < nks && head < a.H)
            qb[j] = *(const bf16x8*)(a.q + (((int64_t)r * a.H + head) * DQK + (ksb + j) * 16 + (lane >> 5) * 8) * 2);
        else
            qb[j] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
    }

    // selected rows -> byte offsets, and one validity bit per row via ballots
    for (int i0 = 0; i0 < nt_fill * TROWS; i0 += NT) {
        const int i = i0 + tid;
        int64_t s = -1;
        if (i < nk) {
            const int p = a.idx[(int64_t)r * a.K + k0 + i];
            s = p >= 0 ? slot_of(a.kv, seq, p) : -1;
        }
        if (i < nt_fill * TROWS) {
            roff[i] = s >= 0 ? s * a.kv.row_stride : -1;
            if constexpr (TSC) {
#pragma unroll
                for (int j = 0; j < NTL; ++j) kvs[j * kSfaMaxKeys + i] = s >= 0 ? a.kv.scale[s * NTL + j] : 0.f;
            } else if constexpr (FP8) {
                kvs[i] = s >= 0 ? a.kv.scale[s / a.kv.scale_group] : 0.f;
            }
        }
        const uint64_t bal = __ballot(s >= 0);
        if (lane == 0 && i < nt_fill * TROWS) {
            vmask[i / 32] = (uint32_t)bal;
            if (i + 32 < nt_fill * TROWS) vmask[i / 32 + 1] = (uint32_t)(bal >> 32);
        }
    }
    __syncthreads();
    // trailing tiles without a valid row are skipped; at least one tile is
    // always processed (an empty tile contributes nothing)
    for (int t = tid; t < nt_fill; t += NT)
        if (vmask[t] != 0u) atomicMax(&s_ntiles, t + 1);
    __syncthreads();
    const int ntiles = s_ntiles;

    // per-lane constants of the LDS addressing
    const int krow = lane & 31;                 // QK: cached row = key of this lane
    const int kswz = SWZ ? sfa_swz(krow) : 0;
    const int g16 = lane >> 4, i16 = lane & 15; // PV transpose reads: 16-lane group, lane in group
    const int trow = 4 * (g16 >> 1) + (i16 >> 2);          // + 16 kk + 8 j
    const int tcol = 16 * (g16 & 1) + 4 * (i16 & 3);       // + value column base
    // transpose-read byte offsets of rows 8 j + trow at value column
    // dh * DVH + tcol + 32 (mt % 2); other (kk, mt) add immediates
    uint32_t pvb[2][2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int par = 0; par < 2; ++par) {
            const int rr = 8 * j + trow;
            const int byte = (dh * DVH + tcol + 32 * par) * 2;
            pvb[j][par] = (uint32_t)(rr * RBP + (((byte >> 4) ^ (SWZ ? sfa_swz(rr) : 0)) << 4) + (byte & 15));
        }

    // tile loads: chunk position P = j * NT + tid of the tile (row P / CPKP,
    // position P % CPKP) receives global chunk (position ^ swizzle(row)) of
    // that row; row offsets come from roff.  The LDS destination of a wave's
    // instruction is contiguous (lane * 16 bytes from a wave-uniform base).
    auto issue_tile = [&](int t, int buf) {
        const uint32_t lds0 = (uint32_t)(uintptr_t)(tile[buf]) + (uint32_t)((tid & ~63) * 16);
#pragma unroll
        for (int j = 0; j < NLD; ++j) {
            const int P = j * NT + tid;           // chunk position in the tile
            if (TCH % NT == 0 || P < TCH) {
                const int row = P / CPKP, pos = P - row * CPKP;
                const int part = SWZ ? (pos ^ sfa_swz(row)) : pos;
                const int64_t off = roff[t * TROWS + row];
                const uint8_t* g = (off >= 0 && part < CPK) ? a.kv.data + off + part * 16 : g_zero16;
                lds_dma<16, 0>(g, lds0 + (uint32_t)(j * NT * 16));
            }
        }
    };

    // partial S^T[32 keys x 32 heads] over this wave's K-steps of tile buffer T.
    // The K-steps of each half are compile-time constants, so every operand
    // read is one of four per-lane base addresses plus an immediate offset
    // (the swizzle only permutes chunks inside aligned groups of 8).
    uint32_t qkb[4];                              // SWZ: byte offset of chunk (8q + 2m + h) ^ swz
#pragma unroll
    for (int m = 0; m < 4; ++m)
        qkb[m] = (uint32_t)(krow * RBP + ((((2 * m) + (lane >> 5)) ^ kswz) << 4));
    auto qk_half = [&](const lds_u8* T, int kbase, auto ksb_c) {
        constexpr int KSB = decltype(ksb_c)::value;
        constexpr int NKS = KSB == 0 ? KS0 : KS - KS0;
        auto operand = [&](int ks) -> bf16x8 {
            if constexpr (FP8) {
                return fp8x8_to_bf16x8(*(const lds_u32x2*)(T + krow * RBP + ks * 16 + (lane >> 5) * 8));
            } else if constexpr (SWZ) {
                // chunk 2 ks + h = 8 (ks / 4) + 2 (ks % 4) + h
                return *(const lds_bf16x8*)(T + qkb[ks & 3] + 128 * (ks >> 2));
            } else {
                return *(const lds_bf16x8*)(T + krow * RBP + (2 * ks + (lane >> 5)) * 16);
            }
        };
        constexpr int PF = 3;  // operands in flight ahead of the MFMA that uses them
        f32x16 s, seg;
#pragma unroll
        for (int i = 0; i < 16; ++i) s[i] = seg[i] = 0.f;
        bf16x8 buf[PF];
#pragma unroll
        for (int j = 0; j < PF && j < NKS; ++j) buf[j] = operand(KSB + j);
#pragma unroll
        for (int j = 0; j < NKS; ++j) {
            const bf16x8 av = buf[j % PF];
            if (j + PF < NKS) buf[j % PF] = operand(KSB + j + PF);
            if constexpr (TSC) {
                seg = mfma32x32x16_bf16(av, qb[j], seg);
                const int ks = KSB + j;
                if ((ks + 1) % 8 == 0 || j + 1 == NKS) {   // last K-step of a 128-column tile
                    // accumulator i holds key 8 (i / 4) + 4 (lane / 32) + i % 4
                    const float* f0 = &kvs[(ks / 8) * kSfaMaxKeys + kbase + 4 * (lane >> 5)];
#pragma unroll
                    for (int j4 = 0; j4 < 4; ++j4) {
                        const f32x4 f = *(const f32x4*)(f0 + 8 * j4);
                        s[4 * j4] = fmaf(seg[4 * j4], f.x, s[4 * j4]);
                        s[4 * j4 + 1] = fmaf(seg[4 * j4 + 1], f.y, s[4 * j4 + 1]);
                        s[4 * j4 + 2] = fmaf(seg[4 * j4 + 2], f.z, s[4 * j4 + 2]);
                        s[4 * j4 + 3] = fmaf(seg[4 * j4 + 3], f.w, s[4 * j4 + 3]);
                    }
#pragma unroll
                    for (int i = 0; i < 16; ++i) seg[i] = 0.f;
                }
            } else {
                s = mfma32x32x16_bf16(av, qb[j], s);
            }
        }
        return s;
    };
    auto qk = [&](const lds_u8* T, int kbase) {
        if (dh == 0) return qk_half(T, kbase, std::integral_constant<int, 0>{});
        return qk_half(T, kbase, std::integral_constant<int, KS0>{});
    };
    // the two waves of a pair exchange partial logits through LDS;
    // layout [pair][i/4][lane][4]: consecutive lanes write consecutive 16 bytes
    auto put_partial = [&](const f32x16& s, int xb) {
        float* xs = xbuf[xb] + (hg * 2 + dh) * 1024 + lane * 4;
#pragma unroll
        for (int i = 0; i < 16; i += 4) *(f32x4*)(xs + i * 64) = f32x4{s[i], s[i + 1], s[i + 2], s[i + 3]};
    };

    f32x16 o[MTV];
#pragma unroll
    for (int mt = 0; mt < MTV; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[mt][i] = 0.f;
    float m2 = -__builtin_inff(), lsum = 0.f;
    f32x16 s_cur;
#pragma unroll
    for (int i = 0; i < 16; ++i) s_cur[i] = 0.f;

    if (ntiles > 0) issue_tile(0, 0);
    if (ntiles > 1) issue_tile(1, 1);
    if (ntiles > 0) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        s_cur = qk((const lds_u8*)tile[0], 0);
        put_partial(s_cur, 0);
    }

    const lds_u8* tile0 = (const lds_u8*)tile[0];
    int bcur = 0;                               // ring index of tile t
    for (int t = 0; t < ntiles; ++t) {
        const int bnext = bcur == NBUF - 1 ? 0 : bcur + 1;
        const int bnext2 = bnext == NBUF - 1 ? 0 : bnext + 1;
        // tile t+1 landed; everyone is done with tile t-1 (its buffer is free)
        // and has published the partial logits of tile t
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (t + 2 < ntiles) issue_tile(t + 2, bnext2);
        const lds_u8* T = tile0 + bcur * (TROWS * RBP);
        const uint32_t vm = vmask[t];

        // full logits of tile t = own partial + partner's partial
        f32x16 s = s_cur;
        {
            const float* xp = xbuf[t & 1] + (hg * 2 + (dh ^ 1)) * 1024 + lane * 4;
#pragma unroll
            for (int i = 0; i < 16; i += 4) {
                const f32x4 v = *(const f32x4*)(xp + i * 64);
                s[i] += v.x;
                s[i + 1] += v.y;
                s[i + 2] += v.z;
                s[i + 3] += v.w;
            }
        }
        bf16x8 pb[2];
        bf16x8 pbv[TSC && ILV ? MTV / 4 : 1][2];   // TSC: probabilities times each value tile's scale
        {
            // logits (base 2), masking, online softmax in place on s.  The
            // reference maximum m2 of a head is raised only when a tile's maximum
            // exceeds it by more than kLazy (log2 units); otherwise probabilities
            // are formed against the stale maximum (at most 2^kLazy) and the
            // accumulator is not rescaled.  Same softmax; only rounding differs.
            constexpr float kLazy = 8.0f;
            float tmax = -__builtin_inff();
            if constexpr (FP8 && !TSC) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
                    const float f = a.scale_log2 * kvs[t * TROWS + key];
                    s[i] = ((vm >> key) & 1u) ? s[i] * f : -__builtin_inff();
                    tmax = fmaxf(tmax, s[i]);
                }
            } else if (vm == 0xFFFFFFFFu) {     // every row of the tile selected (common case)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    s[i] *= a.scale_log2;
                    tmax = fmaxf(tmax, s[i]);
                }
            } else {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
                    s[i] = ((vm >> key) & 1u) ? s[i] * a.scale_log2 : -__builtin_inff();
                    tmax = fmaxf(tmax, s[i]);
                }
            }
            tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
            const bool raise = tmax > m2 + kLazy;   // also true on the first valid tile
            if (__ballot(raise) != 0ull) {
                const float mnew = raise ? tmax : m2;
                const float alpha = __builtin_amdgcn_exp2f(m2 - mnew);  // m2 = -inf -> 0
                lsum *= alpha;
#pragma unroll
                for (int mt = 0; mt < MTV; ++mt)
#pragma unroll
                    for (int i = 0; i < 16; ++i) o[mt][i] *= alpha;
                m2 = mnew;
            }
            // a head with no valid row so far keeps m2 = -inf; its probabilities
            // (all of masked rows) must come out 0, not NaN
            const float mref = m2 == -__builtin_inff() ? 0.f : m2;
            float rs = 0.f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                s[i] = __builtin_amdgcn_exp2f(s[i] - mref);
                rs += s[i];
            }
            rs += __shfl_xor(rs, 32);
            lsum += rs;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    float p = s[8 * kk + e];
                    const int key = t * TROWS + 8 * (2 * kk + (e >> 2)) + 4 * (lane >> 5) + (e & 3);
                    if constexpr (TSC && ILV) {
#pragma unroll
                        for (int gv = 0; gv < MTV / 4; ++gv)
                            pbv[gv][kk][e] = (__bf16)(p * kvs[((dh * DVH) / 128 + gv) * kSfaMaxKeys + key]);
                    } else if constexpr (FP8) {
                        p *= kvs[key];   // TSC with one tile: that tile's scale
                    }
                    pb[kk][e] = (__bf16)p;
                }
        }
        // QK^T of the next tile: independent of this tile's PV, so the two MFMA
        // streams interleave (same basic block, no branch in between)
        if (t + 1 < ntiles) s_cur = qk(tile0 + bnext * (TROWS * RBP), (t + 1) * TROWS);
        {

            // PV: O^T[32 value columns x 32 heads] += V^T[32 x 16 keys] * P^T.
            // Keys of K-step kk for lane half h are 16 kk + 4 h + {0..3} (operand
            // elements 0..3) and 16 kk + 8 + 4 h + {0..3} (elements 4..7), the
            // same keys the S^T accumulator registers 8 kk .. 8 kk + 7 hold.
            if constexpr (SWZ) {
                // Two transpose reads per operand: the 16 lanes of group g16 read
                // rows 16 kk + 8 j + 4 (g16 / 2) + i16 / 4 at columns
                // base + 16 (g16 % 2) + 4 (i16 % 4); lane l then holds column
                // base + l % 32 of four consecutive keys.
                typedef short s16x4 __attribute__((ext_vector_type(4)));
                typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
                // row 16 kk + 8 j + trow; chunk (4 (mt % 2) + c0) ^ swz + 8 (mt / 2)
                auto trd = [&](int mt, int kk, int j) -> s16x4 {
                    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_s16x4*)(T + pvb[j][mt & 1] + 16 * kk * RBP + 128 * (mt >> 1)));
                };
                s16x4 cur[4], nxt[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) cur[q] = trd(0, q >> 1, q & 1);
#pragma unroll
                for (int mt = 0; mt < MTV; ++mt) {
                    if (mt + 1 < MTV) {
#pragma unroll
                        for (int q = 0; q < 4; ++q) nxt[q] = trd(mt + 1, q >> 1, q & 1);
                    }
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk) {
                        const u32x2 lo = __builtin_bit_cast(u32x2, cur[2 * kk]);
                        const u32x2 hi = __builtin_bit_cast(u32x2, cur[2 * kk + 1]);
                        const u32x4 w = {lo.x, lo.y, hi.x, hi.y};
                        o[mt] = mfma32x32x16_bf16(__builtin_bit_cast(bf16x8, w), pb[kk], o[mt]);
                    }
#pragma unroll
                    for (int q = 0; q < 4; ++q) cur[q] = nxt[q];
                }
            } else if constexpr (ILV) {
                // Interleaved columns over groups of 4 M-tiles: in group g, M-tile
                // j holds columns base + 128 g + 4 c + j (c = lane % 32); one read
                // of 4 consecutive columns per key feeds all 4 M-tiles after a
                // 16-bit transpose with v_perm.
#pragma unroll
                for (int g = 0; g < MTV / 4; ++g) {
                    const int col = dh * DVH + 128 * g + 4 * (lane & 31);
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk) {
                        u32x2 x[8];
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const int key = 16 * kk + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                            if constexpr (FP8) {
                                const uint32_t c4 = *(const lds_u32*)(T + key * RBP + col);
                                const f32x2 f0 = fp8x2_to_f32<false>(c4), f1 = fp8x2_to_f32<true>(c4);
                                x[e] = u32x2{pack_hi16(f0.x, f0.y), pack_hi16(f1.x, f1.y)};
                            } else {
                                x[e] = *(const lds_u32x2*)(T + key * RBP + col * 2);
                            }
                        }
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            u32x4 w;
                            const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
                            for (int m = 0; m < 4; ++m) {
                                const uint32_t a0 = (j < 2) ? x[2 * m].x : x[2 * m].y;
                                const uint32_t a1 = (j < 2) ? x[2 * m + 1].x : x[2 * m + 1].y;
                                w[m] = __builtin_amdgcn_perm(a1, a0, sel);
                            }
                            if constexpr (TSC)
                                o[4 * g + j] = mfma32x32x16_bf16(__builtin_bit_cast(bf16x8, w), pbv[g][kk], o[4 * g + j]);
                            else
                                o[4 * g + j] = mfma32x32x16_bf16(__builtin_bit_cast(bf16x8, w), pb[kk], o[4 * g + j]);
                        }
                    }
                }
            } else {
#pragma unroll
                for (int mt = 0; mt < MTV; ++mt) {
                    const int col = dh * DVH + mt * 32 + (lane & 31);
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk) {
                        bf16x8 av;
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const int key = 16 * kk + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                            if constexpr (FP8) {
                                const uint32_t code = T[key * RBP + col];
                                const f32x2 f = fp8x2_to_f32<false>(code);
                                av[e] = __builtin_bit_cast(__bf16, (uint16_t)(__float_as_uint(f.x) >> 16));
                            } else {
                                av[e] = *(const lds_bf16*)(T + key * RBP + col * 2);
                            }
                        }
                        o[mt] = mfma32x32x16_bf16(av, pb[kk], o[mt]);
                    }
                }
            }
        }
        if constexpr (SWZ) {
            // interleave the QK^T(t+1) and PV(t) streams: operand reads run ahead
            // of the MFMAs that consume them
#pragma unroll
            for (int i = 0; i < KS0 + 2 * MTV; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // LDS reads
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
            }
        }
        if (t + 1 < ntiles) put_partial(s_cur, (t + 1) & 1);
        bcur = bnext;
    }

    // epilogue: normalise and store.  O^T layout: lane = head; accumulator
    // register i of M-tile m is value row rho = 8 (i / 4) + 4 h + i % 4.
    auto store_rows = [&](auto* dst, float inv) {
        typedef typename std::remove_pointer<decltype(dst)>::type E;
        if constexpr (ILV) {
            // interleaved M-tiles: column = base + 128 g + 4 rho + j
#pragma unroll
            for (int g = 0; g < MTV / 4; ++g)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int rho = 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
                    const int col = dh * DVH + 128 * g + 4 * rho;
                    if constexpr (std::is_same<E, float>::value) {
                        *(f32x4*)(dst + col) = f32x4{o[4 * g][i] * inv, o[4 * g + 1][i] * inv,
                                                     o[4 * g + 2][i] * inv, o[4 * g + 3][i] * inv};
                    } else {
                        bf16x4 v;
#pragma unroll
                        for (int j = 0; j < 4; ++j) v[j] = (__bf16)(o[4 * g + j][i] * inv);
                        *(bf16x4*)(dst + col) = v;
                    }
                }
        } else {
#pragma unroll
            for (int mt = 0; mt < MTV; ++mt)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const int col = dh * DVH + mt * 32 + 8 * q4 + 4 * (lane >> 5);
                    if constexpr (std::is_same<E, float>::value) {
                        *(f32x4*)(dst + col) = f32x4{o[mt][4 * q4] * inv, o[mt][4 * q4 + 1] * inv,
                                                     o[mt][4 * q4 + 2] * inv, o[mt][4 * q4 + 3] * inv};
                    } else {
                        bf16x4 v;
#pragma unroll
                        for (int j = 0; j < 4; ++j) v[j] = (__bf16)(o[mt][4 * q4 + j] * inv);
                        *(bf16x4*)(dst + col) = v;
                    }
                }
        }
    };
    if (head < a.H) {
        const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
        const float l_nat = lsum > 0.f ? (m2 + log2f(lsum)) * kLn2 : -__builtin_inff();
        if (nsplit == 1 && out != nullptr) {
            __bf16* orow = out + ((int64_t)r * a.H + head) * DLAT;
            store_rows(orow, inv);
            if (lse != nullptr && dh == 0 && lane < 32) lse[(int64_t)r * a.H + head] = l_nat;
        } else {
            float* prow = part_o + (((int64_t)r * nsplit + sp) * a.H + head) * DLAT;
            store_rows(prow, inv);
            if (dh == 0 && lane < 32) part_lse[((int64_t)r * nsplit + sp) * a.H + head] = l_nat;
        }
    }
}

// Wide bf16 rows (a whole number of 128-byte groups, e.g. 512 + 64) -----------
//
// Same decomposition, softmax and MFMA layouts as sfa_kernel; what differs is
// how the tile is brought in and how each wave's stream is laid out.
//
// Blocked tile layout: the 32 rows of a tile form 4 groups of 8 rows; group g
// holds NJ = CPK / 8 blocks of 1 KB, block j = chunks [8j, 8j + 8) of the
// group's rows (128 B per row), chunk slots of row r permuted by XOR
// sfa_swz(r).  Chunk c of tile row r sits at
//   (r / 8) * NJ KB + (c / 8) KB + (r % 8) * 128 + ((c % 8) ^ swz(r)) * 16.
// A wave's load instruction j fills exactly one block: lane l brings chunk
// 8j + ((l % 8) ^ swz(row)) of row 8 w + l / 8 to block + 16 l.  A thread
// therefore looks up one cache slot per tile and issues NJ loads that differ
// only in their immediate offsets.
//
// Each wave runs a loop specialised for its half of the QK^T reduction (no
// divergent branch inside), and the exponentials of tile t are computed
// between the QK^T MFMAs of tile t + 1, which do not depend on them.
__device__ __attribute__((aligned(16))) uint8_t g_zero_row[2048];

// fn(std::integral_constant<int, i>) for i = 0 .. N-1 (immediate operands)
template <int I = 0, int N, typename F>
__device__ __forceinline__ void static_for_impl(F&& fn) {
    if constexpr (I < N) {
        fn(std::integral_constant<int, I>{});
        static_for_impl<I + 1, N>(fn);
    }
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& fn) { static_for_impl<0, N>(fn); }

template <int DLAT, int DROPE, int NHG>
__global__ __launch_bounds__(128 * NHG) void sfa_bf16_kernel(MlaDev a, int kps, int nsplit, int nhb,
                                                             __bf16* __restrict__ out, float* __restrict__ lse,
                                                             float* __restrict__ part_o,
                                                             float* __restrict__ part_lse) {
    constexpr int DQK = DLAT + DROPE;
    constexpr int CPK = DQK * 2 / 16;       // 16-byte chunks per row
    static_assert((DQK * 2) % 128 == 0 && CPK * 16 <= 2048, "rows must be whole 128-byte groups");
    constexpr int NJ = CPK / 8;             // 1 KB blocks per 8-row group
    constexpr int GB = NJ * 1024;           // bytes per 8-row group
    constexpr int TROWS = 32;
    constexpr int TB = (TROWS / 8) * GB;    // bytes per tile
    constexpr int NBUF = 3;                 // tile ring: PV(t) | QK(t+1) | loading t+2
    constexpr int NT = 128 * NHG;
    constexpr int RPP = NT / 8;             // tile rows loaded per pass
    constexpr int NPASS = TROWS / RPP;
    constexpr int KS = DQK / 16;            // QK K-steps
    static_assert(KS % 2 == 0, "even K-step count");
    constexpr int NKS = KS / 2;             // K-steps per wave
    constexpr int DVH = DLAT / 2;           // value columns per wave
    constexpr int MTV = DVH / 32;           // PV M-tiles per wave
    static_assert(DVH % 64 == 0, "shape");

    __shared__ __attribute__((aligned(1024))) uint8_t tile[NBUF * TB];
    __shared__ uint32_t rslot[kSfaMaxKeys];            // cache slot of each selected row, ~0 = skip
    __shared__ uint32_t vmask[kSfaMaxKeys / 32];       // valid-row bits of each 32-row tile
    __shared__ __attribute__((aligned(16))) float xbuf[2][NHG * 2 * 1024];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hg = wave >> 1;
    const int bid = blockIdx.x;
    const int hb = (bid >> 3) % nhb;
    const int u = ((bid >> 3) / nhb) * 8 + (bid & 7);
    if (u >= a.R * nsplit) return;
    const int r = u / nsplit, sp = u % nsplit;
    const int k0 = sp * kps;
    const int k1 = (k0 + kps < a.K) ? k0 + kps : a.K;
    const int nk = k1 - k0;
    const int seq = a.row_seq[r];
    const int nt_fill = (nk + TROWS - 1) / TROWS;
    __shared__ int s_ntiles;
    if (tid == 0) s_ntiles = 1;

    for (int i0 = 0; i0 < nt_fill * TROWS; i0 += NT) {
        const int i = i0 + tid;
        int64_t s = -1;
        if (i < nk) {
            const int p = a.idx[(int64_t)r * a.K + k0 + i];
            s = p >= 0 ? slot_of(a.kv, seq, p) : -1;
        }
        if (i < nt_fill * TROWS) rslot[i] = s >= 0 ? (uint32_t)s : 0xFFFFFFFFu;
        const uint64_t bal = __ballot(s >= 0);
        if (lane == 0 && i < nt_fill * TROWS) {
            vmask[i / 32] = (uint32_t)bal;
            if (i + 32 < nt_fill * TROWS) vmask[i / 32 + 1] = (uint32_t)(bal >> 32);
        }
    }
    __syncthreads();
    // trailing tiles without a valid row are skipped; at least one tile is
    // always processed (an empty tile contributes nothing)
    for (int t = tid; t < nt_fill; t += NT)
        if (vmask[t] != 0u) atomicMax(&s_ntiles, t + 1);
    __syncthreads();
    const int ntiles = s_ntiles;

    const lds_u8* tile0 = (const lds_u8*)tile;
    const uint32_t tile_lds = (uint32_t)(uintptr_t)tile;
    // loads: this thread's row within a pass and its chunk permutation
    const int lrow = tid >> 3;
    const uint32_t goff = (uint32_t)(((tid & 7) ^ sfa_swz(lrow)) << 4);  // swz(lrow) == swz(lrow + 16)
    // slots of this thread's rows of tile t (read one iteration ahead of use)
    auto read_slots = [&](int t, uint32_t (&sl)[NPASS]) {
#pragma unroll
        for (int p = 0; p < NPASS; ++p) sl[p] = rslot[(t < ntiles ? t : 0) * TROWS + p * RPP + lrow];
    };
    auto issue_tile = [&](const uint32_t (&sl)[NPASS], int buf) {
#pragma unroll
        for (int p = 0; p < NPASS; ++p) {
            const uint32_t s = sl[p];
            const uint8_t* g = (s != 0xFFFFFFFFu ? a.kv.data + (uint64_t)s * (uint32_t)a.kv.row_stride : g_zero_row) + goff;
            const uint32_t blk = tile_lds + (uint32_t)(buf * TB + (p * (RPP / 8) + wave) * GB);
            static_for<NJ>([&](auto jc) {
                constexpr int j = decltype(jc)::value;
                // the immediate offset moves both the global and the LDS address;
                // block j lands at blk + j KB
                lds_dma<16, j * 128>(g, blk + (uint32_t)(j * (1024 - 128)));
            });
        }
    };
    auto body = [&](auto dh_c) {
        constexpr int DH = decltype(dh_c)::value;
        constexpr int KSB = DH * NKS;
        const int head = hb * 32 * NHG + hg * 32 + (lane & 31);
        bf16x8 qb[NKS];
#pragma unroll
        for (int j = 0; j < NKS; ++j) {
            if (head < a.H)
                qb[j] = *(const bf16x8*)(a.q + (((int64_t)r * a.H + head) * DQK + (KSB + j) * 16 + (lane >> 5) * 8) * 2);
            else
                qb[j] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
        }
        // QK operand: lane = key row krow, 8 values of chunk 2 ks + lane / 32
        const int krow = lane & 31;
        uint32_t qkb[4];
#pragma unroll
        for (int m = 0; m < 4; ++m)
            qkb[m] = (uint32_t)((krow >> 3) * GB + (krow & 7) * 128 + ((((2 * m) + (lane >> 5)) ^ sfa_swz(krow)) << 4));
        auto qk_op = [&](const lds_u8* T, int ks) -> bf16x8 {   // ks: compile-time after unrolling
            return *(const lds_bf16x8*)(T + qkb[ks & 3] + (ks >> 2) * 1024);
        };
        // PV operand (transpose reads): 16-lane group g16 reads rows 8 j + trow
        // of each 16-key half, at 4 consecutive value columns per lane
        const int g16 = lane >> 4, i16 = lane & 15;
        const int trow = 4 * (g16 >> 1) + (i16 >> 2);
        uint32_t pvb[2][2];
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int par = 0; par < 2; ++par) {
                const int cc = 4 * par + 2 * (g16 & 1) + ((i16 & 3) >> 1);
                pvb[j][par] = (uint32_t)(j * GB + trow * 128 + ((cc ^ sfa_swz(8 * j + trow)) << 4) + 8 * (i16 & 1));
            }
        typedef short s16x4 __attribute__((ext_vector_type(4)));
        typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
        auto trd = [&](const lds_u8* T, int mt, int kk, int j) -> s16x4 {
            return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4*)(T + pvb[j][mt & 1] + kk * 2 * GB + (4 * DH + (mt >> 1)) * 1024));
        };
        auto qk = [&](const lds_u8* T) {
            f32x16 s;
#pragma unroll
            for (int i = 0; i < 16; ++i) s[i] = 0.f;
            constexpr int PF = 4;
            bf16x8 buf[PF];
#pragma unroll
            for (int j = 0; j < PF; ++j) buf[j] = qk_op(T, KSB + j);
#pragma unroll
            for (int j = 0; j < NKS; ++j) {
                const bf16x8 av = buf[j % PF];
                if (j + PF < NKS) buf[j % PF] = qk_op(T, KSB + j + PF);
                s = mfma32x32x16_bf16(av, qb[j], s);
            }
            return s;
        };
        auto put_partial = [&](const f32x16& s, int xb) {
            float* xs = xbuf[xb] + (hg * 2 + DH) * 1024 + lane * 4;
#pragma unroll
            for (int i = 0; i < 16; i += 4) *(f32x4*)(xs + i * 64) = f32x4{s[i], s[i + 1], s[i + 2], s[i + 3]};
        };

        f32x16 o[MTV];
#pragma unroll
        for (int mt = 0; mt < MTV; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[mt][i] = 0.f;
        float m2 = -__builtin_inff(), lsum = 0.f;
        const float c = a.scale_log2;
        f32x16 s_cur;
#pragma unroll
        for (int i = 0; i < 16; ++i) s_cur[i] = 0.f;

        uint32_t sl[NPASS];
        if (ntiles > 0) {
            read_slots(0, sl);
            issue_tile(sl, 0);
        }
        if (ntiles > 1) {
            read_slots(1, sl);
            issue_tile(sl, 1);
        }
        read_slots(2, sl);
        if (ntiles > 0) {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            s_cur = qk(tile0);
            put_partial(s_cur, 0);
        }

        int bcur = 0;
        for (int t = 0; t < ntiles; ++t) {
            const int bnext = bcur == NBUF - 1 ? 0 : bcur + 1;
            const int bnext2 = bnext == NBUF - 1 ? 0 : bnext + 1;
            // tile t+1 landed; tile t-1's buffer is free; partials of tile t published
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            const lds_u8* T = tile0 + bcur * TB;
            const lds_u8* Tn = tile0 + bnext * TB;
            constexpr int PF = 4;   // QK^T operand reads in flight
            constexpr int PD = 2;   // PV: M-tiles of operands in flight

            // every LDS read this step needs first is issued here, ahead of
            // the loads of tile t+2, so a single wait covers them
            f32x4 xr[4];
            {
                const float* xp = xbuf[t & 1] + (hg * 2 + (DH ^ 1)) * 1024 + lane * 4;
#pragma unroll
                for (int i = 0; i < 4; ++i) xr[i] = *(const f32x4*)(xp + i * 256);
            }
            const uint32_t vmr = vmask[t];
            bf16x8 buf[PF];
#pragma unroll
            for (int j = 0; j < PF; ++j) buf[j] = qk_op(Tn, KSB + j);
            if (t + 2 < ntiles) issue_tile(sl, bnext2);
            read_slots(t + 3, sl);
            __builtin_amdgcn_sched_barrier(0);

            // raw logits of tile t = own partial + partner's partial
            f32x16 s = s_cur;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                s[4 * i] += xr[i].x;
                s[4 * i + 1] += xr[i].y;
                s[4 * i + 2] += xr[i].z;
                s[4 * i + 3] += xr[i].w;
            }
            const uint32_t vm = __builtin_amdgcn_readfirstlane(vmr);
            if (vm != 0xFFFFFFFFu) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
                    if (!((vm >> key) & 1u)) s[i] = -__builtin_inff();
                }
            }
            // tile maximum of each head (both lane halves), in log2 units
            float tmax = fmaxf(fmaxf(s[0], s[1]), s[2]);
#pragma unroll
            for (int i = 3; i < 15; i += 2) tmax = fmaxf(fmaxf(tmax, s[i]), s[i + 1]);
            tmax = fmaxf(tmax, s[15]);
            {
                const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax), __float_as_uint(tmax), false, false);
                tmax = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
            }
            tmax *= c;   // c > 0
            // lazy reference maximum (raised only past kLazy log2 units)
            constexpr float kLazy = 8.0f;
            const bool raise = tmax > m2 + kLazy;   // also true on the first valid tile
            if (__ballot(raise) != 0ull) {
                const float mnew = raise ? tmax : m2;
                const float alpha = __builtin_amdgcn_exp2f(m2 - mnew);  // m2 = -inf -> 0
                lsum *= alpha;
#pragma unroll
                for (int mt = 0; mt < MTV; ++mt)
#pragma unroll
                    for (int i = 0; i < 16; ++i) o[mt][i] *= alpha;
                m2 = mnew;
            }
            // a head with no valid row so far keeps m2 = -inf: its (masked)
            // probabilities must come out 0, not NaN
            const float negm = m2 == -__builtin_inff() ? 0.f : -m2;

            // Phase 1: QK^T of tile t+1 (independent of this tile's softmax)
            // with the exponentials of tile t between its MFMAs; operand reads
            // run PF K-steps ahead.
            s16x4 rb[PD + 1][4];
            f32x16 s_next;
#pragma unroll
            for (int i = 0; i < 16; ++i) s_next[i] = 0.f;
            float pe[16];
            {
#pragma unroll
                for (int j = 0; j < NKS; ++j) {
                    const bf16x8 av = buf[j % PF];
                    if (j + PF < NKS) buf[j % PF] = qk_op(Tn, KSB + j + PF);
                    s_next = mfma32x32x16_bf16(av, qb[j], s_next);
                    if (j < 16) pe[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[j], c, negm));
                }
            }
            float rs = 0.f;
#pragma unroll
            for (int i = 0; i < 16; ++i) rs += pe[i];
            {
                const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(rs), __float_as_uint(rs), false, false);
                rs = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
            }
            lsum += rs;
            bf16x8 pb[2];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int e = 0; e < 8; ++e) pb[kk][e] = (__bf16)pe[8 * kk + e];
#pragma unroll
            for (int j = 0; j < NKS; ++j) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (j + PF < NKS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int m = 0; m < PD; ++m)
#pragma unroll
                for (int q = 0; q < 4; ++q) rb[m][q] = trd(T, m, q >> 1, q & 1);

            // Phase 2, PV(t): O^T[32 value columns x 32 heads] += V^T[32 x 16
            // keys] * P^T.  Keys of K-step kk for lane half h: 16 kk + 4 h +
            // {0..3} (operand elements 0..3) and 16 kk + 8 + 4 h + {0..3}
            // (elements 4..7): the keys of S^T accumulator registers 8 kk ..
            // 8 kk + 7.  Transpose reads run PD M-tiles ahead.
#pragma unroll
            for (int mt = 0; mt < MTV; ++mt) {
                if (mt + PD < MTV) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) rb[(mt + PD) % (PD + 1)][q] = trd(T, mt + PD, q >> 1, q & 1);
                }
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    const u32x2 lo = __builtin_bit_cast(u32x2, rb[mt % (PD + 1)][2 * kk]);
                    const u32x2 hi = __builtin_bit_cast(u32x2, rb[mt % (PD + 1)][2 * kk + 1]);
                    const u32x4 w = {lo.x, lo.y, hi.x, hi.y};
                    o[mt] = mfma32x32x16_bf16(__builtin_bit_cast(bf16x8, w), pb[kk], o[mt]);
                }
            }
            put_partial(s_next, (t + 1) & 1);
            __builtin_amdgcn_sched_group_barrier(0x100, 4 * PD, 0);
#pragma unroll
            for (int mt = 0; mt < MTV; ++mt) {
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                if (mt + PD < MTV) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x200, 4, 0);
            __builtin_amdgcn_sched_barrier(0);
            s_cur = s_next;
            bcur = bnext;
        }

        // epilogue: normalise and store.  O^T layout: lane = head; accumulator
        // register i of M-tile m is value column 32 m + 8 (i / 4) + 4 h + i % 4.
        if (head < a.H) {
            const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
            const float l_nat = lsum > 0.f ? (m2 + log2f(lsum)) * kLn2 : -__builtin_inff();
            if (nsplit == 1 && out != nullptr) {
                __bf16* orow = out + ((int64_t)r * a.H + head) * DLAT;
#pragma unroll
                for (int mt = 0; mt < MTV; ++mt)
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) {
                        const int col = DH * DVH + mt * 32 + 8 * q4 + 4 * (lane >> 5);
                        bf16x4 v;
#pragma unroll
                        for (int j = 0; j < 4; ++j) v[j] = (__bf16)(o[mt][4 * q4 + j] * inv);
                        *(bf16x4*)(orow + col) = v;
                    }
                if (lse != nullptr && DH == 0 && lane < 32) lse[(int64_t)r * a.H + head] = l_nat;
            } else {
                float* prow = part_o + (((int64_t)r * nsplit + sp) * a.H + head) * DLAT;
#pragma unroll
                for (int mt = 0; mt < MTV; ++mt)
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) {
                        const int col = DH * DVH + mt * 32 + 8 * q4 + 4 * (lane >> 5);
                        *(f32x4*)(prow + col) = f32x4{o[mt][4 * q4] * inv, o[mt][4 * q4 + 1] * inv,
                                                      o[mt][4 * q4 + 2] * inv, o[mt][4 * q4 + 3] * inv};
                    }
                if (DH == 0 && lane < 32) part_lse[((int64_t)r * nsplit + sp) * a.H + head] = l_nat;
            }
        }
    };
    if (wave & 1) body(std::integral_constant<int, 1>{});
    else body(std::integral_constant<int, 0>{});
}

// Chunk permutation of the warp-specialised kernel: for rows of one parity,
// swz8 maps (r / 2) % 8 = m to 2 (m % 4) + m / 4, a bijection (16 consecutive
// rows read at one chunk hit 16 distinct 16-byte bank groups) whose halves
// m < 4 and m >= 4 give distinct chunk pairs (8 consecutive rows read at two
// adjacent chunks by a transpose read hit 16 distinct bank groups).
__device__ __forceinline__ int sfa_swz8(int r) { return (((r >> 1) & 3) << 1) | ((r >> 3) & 1); }

// Warp-specialised eight-wave kernel for 64 heads of 512 + 64 bf16 rows ---------
//
// Tiles of 32 gathered rows in 8-row groups of 1 KB blocks (chunk permutation
// sfa_swz8), a lazy online softmax (the reference maximum is raised only when a
// tile exceeds it by 2^8), and the waves split the work by kind:
//  * q-waves 0..3: wave w owns heads 16 w .. 16 w + 15 of the block over all
//    576 QK columns (query in 72 VGPRs): S^T of tile t+1 (36 MFMAs), masking,
//    tile maximum, lazy reference raise and exponentials; it writes P^T to an
//    LDS ring in the PV B-operand's lane layout (lane = head, K-slots 8 g ..
//    8 g + 7 = keys 16 kb + 4 g + i), with a per-tile raise flag and factors.
//  * p-waves 4..7: wave 4 + c owns value columns 128 c .. 128 c + 127 of all
//    64 heads (O^T in 128 accumulator VGPRs): applies the raise factors of the
//    flagged head tiles and runs PV of tile t (32 MFMAs), the value operand
//    from transpose reads of 4 consecutive rows at 4 value columns per lane
//    (the P^T operand's key order).  The p-waves also issue the
//    direct-to-LDS tile loads, NBUF - 2 tiles ahead, from inline assembly
//    (lds_dma): hidden from the compiler's wait-count model, they no longer
//    turn every LDS operand wait of the issuing wave into a full drain; explicit
//    vmcnt waits and the per-tile barrier order them instead.
// Waves w and w + 4 share a SIMD, so QK^T + softmax of tile t+1 and PV of tile
// t overlap; one barrier per tile hands P over.  The two roles run separate
// loops with the same number of barriers, so their registers do not add up.
template <int DLAT, int DROPE, int NBUF, int MAXK, int KVF = 0>
__global__ __launch_bounds__(512) void sfa_ws_kernel(MlaDev a, int kps, int nsplit, int nhb,
                                                      __bf16* __restrict__ out, float* __restrict__ lse,
                                                      float* __restrict__ part_o, float* __restrict__ part_lse) {
    constexpr int DQK = DLAT + DROPE;
    constexpr int CPK = DQK * 2 / 16;       // 16-byte chunks per row
    static_assert((DQK * 2) % 128 == 0 && CPK * 16 <= 2048, "rows must be whole 128-byte groups");
    constexpr int NJ = CPK / 8;             // 1 KB blocks per 8-row group
    constexpr int GB = NJ * 1024;           // bytes per 8-row group
    constexpr int TROWS = 32;
    constexpr int TB = (TROWS / 8) * GB;    // bytes per tile
    static_assert(NBUF >= 3, "PV(t) | QK(t+1) | tiles t+2 .. in flight");
    constexpr int NT = 512;
    constexpr int KS = DQK / 32;            // 16x16x32 K-steps of a row
    constexpr int DVP = DLAT / 4;           // value columns per p-wave
    constexpr int MTP = DVP / 16;           // PV M-tiles per p-wave
    static_assert(DVP % 64 == 0, "whole 1 KB blocks per p-wave");
    typedef float f32x4v __attribute__((ext_vector_type(4)));

    // KVF (cached rows): 0 bf16; 1 e4m3 with one factor per row (group); 2 e4m3
    // with one factor per 128-column tile.  fp8 rows are turned into bf16 rows
    // of the same tile layout by the loading waves, so the QK and PV code is the
    // same for every format.
    constexpr int NTL = KVF == 2 ? (DQK + 127) / 128 : 1;     // factors per row
    static_assert(KVF == 0 || (DQK % 128 == 0 || (DQK - DQK / 128 * 128) % 64 == 0),
                  "fp8 rows: 1 KB blocks never straddle a factor tile");
    __shared__ __attribute__((aligned(1024))) uint8_t tile[NBUF * TB];
    __shared__ uint32_t rslot[MAXK];                   // cache slot of each selected row, ~0 = skip
    __shared__ float kvf[KVF ? NTL * MAXK : 1];        // fp8 factors [tile][row] (0 for skipped rows)
    __shared__ uint32_t vmask[MAXK / 32];              // valid-row bits of each 32-row tile
    __shared__ __attribute__((aligned(16))) uint8_t pbuf[2][4][64 * 16];   // P^T operands [slot][head tile][lane]
    __shared__ float alph[2][64];                      // raise factors [slot][head]
    __shared__ int rflag[2][4];                        // raised head tiles [slot][head tile]
    float* const fin_l = (float*)&pbuf[0][0][0];       // softmax totals after the last tile (the P ring is
                                                       // free by then)

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int bid = blockIdx.x;
    const int hb = (bid >> 3) % nhb;
    const int u = ((bid >> 3) / nhb) * 8 + (bid & 7);
    if (u >= a.R * nsplit) return;
    const int r = u / nsplit, sp = u % nsplit;
    const int k0 = sp * kps;
    const int k1 = (k0 + kps < a.K) ? k0 + kps : a.K;
    const int nk = k1 - k0;
    const int seq = a.row_seq[r];
    const int nt_fill = (nk + TROWS - 1) / TROWS;
    __shared__ int s_ntiles;
    if (tid == 0) s_ntiles = 1;

    // every index load of the thread first, then every block-table lookup, so
    // the slots cost two dependent global round trips in all
    constexpr int EPT = MAXK / NT;          // index entries per thread
    static_assert(MAXK % NT == 0, "whole rounds");
    int pidx[EPT];
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        const int i = j * NT + tid;
        pidx[j] = i < nk ? a.idx[(int64_t)r * a.K + k0 + i] : -1;
    }
    int64_t sv[EPT];
#pragma unroll
    for (int j = 0; j < EPT; ++j) sv[j] = pidx[j] >= 0 ? slot_of(a.kv, seq, pidx[j]) : -1;
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        const int i = j * NT + tid;
        if (i < nt_fill * TROWS) rslot[i] = sv[j] >= 0 ? (uint32_t)sv[j] : 0xFFFFFFFFu;
        if constexpr (KVF == 1) {
            if (i < nt_fill * TROWS) kvf[i] = sv[j] >= 0 ? a.kv.scale[sv[j] / a.kv.scale_group] : 0.f;
        } else if constexpr (KVF == 2) {
            if (i < nt_fill * TROWS) {
#pragma unroll
                for (int q = 0; q < NTL; ++q) kvf[q * MAXK + i] = sv[j] >= 0 ? a.kv.scale[sv[j] * NTL + q] : 0.f;
            }
        }
        const uint64_t bal = __ballot(sv[j] >= 0);
        if (lane == 0 && i < nt_fill * TROWS) {
            vmask[i / 32] = (uint32_t)bal;
            if (i + 32 < nt_fill * TROWS) vmask[i / 32 + 1] = (uint32_t)(bal >> 32);
        }
    }
    __syncthreads();
    // trailing tiles without a valid row are skipped; at least one tile is
    // always processed (an empty tile contributes nothing)
    for (int t = tid; t < nt_fill; t += NT)
        if (vmask[t] != 0u) atomicMax(&s_ntiles, t + 1);
    __syncthreads();
    const int ntiles = s_ntiles;

    const lds_u8* tile0 = (const lds_u8*)tile;
    const int g = lane >> 4, l16 = lane & 15;
    const float kLazy = 8.0f;

    if (wave < 4) {
        // ---------------------------------------------------------------- q-wave
        const int hq = wave;
        const int head = hb * 64 + hq * 16 + l16;
        // the query in B-operand layout: lane = head, 8 consecutive d of K-step ks
        bf16x8 qb[KS];
#pragma unroll
        for (int j = 0; j < KS; ++j) {
            if (head < a.H)
                qb[j] = *(const bf16x8*)(a.q + (((int64_t)r * a.H + head) * DQK + j * 32 + g * 8) * 2);
            else
                qb[j] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
        }
        // QK operand of key block kb, K-step ks: row 16 kb + l16, chunk 4 ks + g
        uint32_t qa[2];
#pragma unroll
        for (int par = 0; par < 2; ++par)
            qa[par] = (uint32_t)((l16 >> 3) * GB + (l16 & 7) * 128 + (((4 * par + g) ^ sfa_swz8(l16)) << 4));
        auto qk_op = [&](const lds_u8* T, int kb, int ks) -> bf16x8 {   // compile-time kb, ks
            return *(const lds_bf16x8*)(T + qa[ks & 1] + kb * 2 * GB + (ks >> 1) * 1024);
        };
        float m2 = -__builtin_inff(), lsum = 0.f;
        const float c = a.scale_log2;

        // S^T of one tile, softmax statistics, P^T to LDS slot ps
        auto q_tile = [&](const lds_u8* T, uint32_t vm, int ps) {
            f32x4v s[2] = {f32x4v{0.f, 0.f, 0.f, 0.f}, f32x4v{0.f, 0.f, 0.f, 0.f}};
            // operand reads in batches of PB, software-pipelined: the reads of
            // batch b + 1 go out before the MFMAs of batch b, so 6 .. 12 reads
            // are in flight while the MFMAs run (the scheduling barriers keep the
            // compiler from pairing each read with its MFMA)
            constexpr int PB = 6;
            constexpr int NB = (2 * KS) / PB;
            static_assert((2 * KS) % PB == 0, "whole batches");
            bf16x8 av[2][PB];
#pragma unroll
            for (int j = 0; j < PB; ++j) av[0][j] = qk_op(T, j & 1, j >> 1);
            static_for<NB>([&](auto bc) {
                constexpr int b = decltype(bc)::value;
                if constexpr (b + 1 < NB) {
#pragma unroll
                    for (int j = 0; j < PB; ++j)
                        av[(b + 1) & 1][j] = qk_op(T, ((b + 1) * PB + j) & 1, ((b + 1) * PB + j) >> 1);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int j = 0; j < PB; ++j)
                    s[(b * PB + j) & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        av[b & 1][j], qb[(b * PB + j) >> 1], s[(b * PB + j) & 1], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            });
            if (vm != 0xFFFFFFFFu) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (!((vm >> (16 * kb + 4 * g + i)) & 1u)) s[kb][i] = -__builtin_inff();
            }
            float tmax = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                               fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
            {
                const auto w16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(tmax), __float_as_uint(tmax), false, false);
                tmax = fmaxf(__uint_as_float(w16[0]), __uint_as_float(w16[1]));
                const auto w32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax), __float_as_uint(tmax), false, false);
                tmax = fmaxf(__uint_as_float(w32[0]), __uint_as_float(w32[1]));
            }
            tmax *= c;   // c > 0
            const bool raise = tmax > m2 + kLazy;   // also true on the first valid tile
            const bool any = __ballot(raise) != 0ull;
            if (any) {
                const float mnew = raise ? tmax : m2;
                const float alpha = __builtin_amdgcn_exp2f(m2 - mnew);  // m2 = -inf -> 0
                lsum *= alpha;
                m2 = mnew;
                if (g == 0) alph[ps][hq * 16 + l16] = alpha;
            }
            if (lane == 0) rflag[ps][hq] = any ? 1 : 0;
            const float negm = m2 == -__builtin_inff() ? 0.f : -m2;
            float pe[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) pe[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[e >> 2][e & 3], c, negm));
            float rs = ((pe[0] + pe[1]) + (pe[2] + pe[3])) + ((pe[4] + pe[5]) + (pe[6] + pe[7]));
            {
                const auto w16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(rs), __float_as_uint(rs), false, false);
                rs = __uint_as_float(w16[0]) + __uint_as_float(w16[1]);
                const auto w32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(rs), __float_as_uint(rs), false, false);
                rs = __uint_as_float(w32[0]) + __uint_as_float(w32[1]);
            }
            lsum += rs;
            bf16x8 pb;
#pragma unroll
            for (int e = 0; e < 8; ++e) pb[e] = (__bf16)pe[e];
            *(__attribute__((address_space(3))) bf16x8*)((lds_u8*)pbuf[ps][hq] + lane * 16) = pb;
        };

        __syncthreads();                                   // barrier P: tile 0 landed
        q_tile(tile0, vmask[0], 0);
        int bq = 1;                                        // buffer of tile t+1
        for (int t = 0; t < ntiles; ++t) {
            __syncthreads();                               // barrier t: P(t) published, tile t+1 landed
            if (t + 1 < ntiles) {
                const uint32_t vmn = __builtin_amdgcn_readfirstlane(vmask[t + 1]);
                q_tile(tile0 + bq * TB, vmn, (t + 1) & 1);
            }
            bq = bq == NBUF - 1 ? 0 : bq + 1;
        }
        // softmax totals for the p-waves, and the normaliser
        __syncthreads();                                   // barrier F: the P ring is no longer read
        if (g == 0) {
            fin_l[hq * 16 + l16] = lsum;
            if (head < a.H) {
                const float l_nat = lsum > 0.f ? (m2 + log2f(lsum)) * kLn2 : -__builtin_inff();
                if (nsplit == 1 && out != nullptr) {
                    if (lse != nullptr) lse[(int64_t)r * a.H + head] = l_nat;
                } else {
                    part_lse[((int64_t)r * nsplit + sp) * a.H + head] = l_nat;
                }
            }
        }
        __syncthreads();                                   // barrier E
    } else {
        // ---------------------------------------------------------------- p-wave
        // The p-waves also load the tiles (see the kernel comment).
        const int pc = wave - 4;
        const uint32_t tile_lds = (uint32_t)(uintptr_t)tile;
        const int lrow = (tid >> 3) & 31;
        const uint32_t goff = (uint32_t)(((tid & 7) ^ sfa_swz8(lrow)) << 4);
        auto read_slot = [&](int t) -> uint32_t { return rslot[(t < ntiles ? t : 0) * TROWS + lrow]; };
        auto issue_tile = [&](uint32_t s, int buf) {
            const uint8_t* gp = (s != 0xFFFFFFFFu ? a.kv.data + (uint64_t)s * (uint32_t)a.kv.row_stride : g_zero_row) + goff;
            const uint32_t blk = tile_lds + (uint32_t)(buf * TB + pc * GB);
            static_for<NJ>([&](auto jc) {
                constexpr int j = decltype(jc)::value;
                // the immediate offset moves both the global and the LDS address;
                // block j lands at blk + j KB
                lds_dma<16, j * 128>(gp, blk + (uint32_t)(j * (1024 - 128)));
            });
        };
        // tiles 0 .. LA up front; tile t + 1 + LA goes out in iteration t into the
        // buffer PV(t-1) has released.  Each thread issues NJ loads per tile, so
        // "tile j landed" = at most NJ * (tiles issued after j) loads pending.
        constexpr int LA = NBUF - 2;
        static_assert(LA <= 2, "wait counts cover two tiles in flight");
        auto wait_tile = [&](int j, int last) {            // tile j landed; tiles up to `last` issued
            const int after = (ntiles - 1 < last ? ntiles - 1 : last) - j;
            if (after >= 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * NJ) : "memory");
            else if (after == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NJ) : "memory");
            else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        };
        // fp8 rows: wave pc fills rows 8 pc .. 8 pc + 7 of each tile.  In 1 KB block
        // j, lane l owns position l % 8 of row 8 pc + l / 8, i.e. bf16 chunk c = 8 j
        // + ((l % 8) ^ swz8(row)) = columns 8 c .. 8 c + 7: it loads their 8 e4m3
        // codes, multiplies by the row's factor of that column tile (block j lies in
        // tile j / 2) and writes the 16 bytes, one contiguous 1 KB per instruction.
        // Codes are fetched two tiles ahead into registers.
        const int frow = 8 * pc + (lane >> 3);
        const int fsw = (lane & 7) ^ sfa_swz8(frow);
        auto fetch = [&](int t, u32x2 (&v)[NJ]) {
            const uint32_t s = t < ntiles ? rslot[t * TROWS + frow] : 0xFFFFFFFFu;
            const uint8_t* gp = s != 0xFFFFFFFFu ? a.kv.data + (uint64_t)s * (uint32_t)a.kv.row_stride : g_zero_row;
#pragma unroll
            for (int j = 0; j < NJ; ++j) v[j] = __builtin_nontemporal_load((const u32x2*)(gp + (8 * j + fsw) * 8));
        };
        auto put = [&](int t, const u32x2 (&v)[NJ], int buf) {
            lds_u8* dst = (lds_u8*)tile + buf * TB + pc * GB + lane * 16;
            float fr[NTL];                                 // the row's factors, read once
#pragma unroll
            for (int q = 0; q < NTL; ++q) fr[q] = kvf[q * MAXK + t * TROWS + frow];
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const float f = fr[KVF == 1 ? 0 : j / 2];
                const f32x2 x0 = fp8x2_to_f32<false>(v[j].x), x1 = fp8x2_to_f32<true>(v[j].x);
                const f32x2 x2 = fp8x2_to_f32<false>(v[j].y), x3 = fp8x2_to_f32<true>(v[j].y);
                bf16x8 b;
                b[0] = (__bf16)(x0.x * f);
                b[1] = (__bf16)(x0.y * f);
                b[2] = (__bf16)(x1.x * f);
                b[3] = (__bf16)(x1.y * f);
                b[4] = (__bf16)(x2.x * f);
                b[5] = (__bf16)(x2.y * f);
                b[6] = (__bf16)(x3.x * f);
                b[7] = (__bf16)(x3.y * f);
                *(__attribute__((address_space(3))) bf16x8*)(dst + j * 1024) = b;
            }
        };
        static_assert(KVF == 0 || NBUF == 3, "fp8 rows: PV(t) | QK(t+1) | tile t+2 being written");
        u32x2 fv[KVF ? 2 : 1][NJ];
        uint32_t sl = 0;
        if constexpr (KVF == 0) {
            for (int j = 0; j <= LA; ++j)
                if (j < ntiles) issue_tile(read_slot(j), j);
            sl = read_slot(LA + 1);
        } else {
            fetch(0, fv[0]);
            fetch(1, fv[1]);
            put(0, fv[0], 0);
            put(1, fv[1], 1);
            fetch(2, fv[0]);
            fetch(3, fv[1]);
        }
        // PV operand of M-tile mt: transpose reads of rows 4 g + l16 / 4 (keys of
        // K-slots 0..3) and 16 + 4 g + l16 / 4 (K-slots 4..7), 4 value columns each
        uint32_t pva[4];
#pragma unroll
        for (int m4 = 0; m4 < 4; ++m4) {
            const int rr = 4 * g + (l16 >> 2);
            const int cc = 2 * m4 + ((l16 & 3) >> 1);
            pva[m4] = (uint32_t)((rr >> 3) * GB + (rr & 7) * 128 + ((cc ^ sfa_swz8(rr)) << 4) + 8 * (l16 & 1));
        }
        typedef short s16x4 __attribute__((ext_vector_type(4)));
        typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
        auto trd = [&](const lds_u8* T, int mt, int half) -> s16x4 {   // compile-time mt, half
            return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4*)(T + pva[mt & 3] + half * 2 * GB + (2 * pc + (mt >> 2)) * 1024));
        };
        f32x4v o[4][MTP];
#pragma unroll
        for (int ht = 0; ht < 4; ++ht)
#pragma unroll
            for (int mt = 0; mt < MTP; ++mt) o[ht][mt] = f32x4v{0.f, 0.f, 0.f, 0.f};

        if constexpr (KVF == 0) wait_tile(0, LA);
        __syncthreads();                                   // barrier P: tile 0 landed
        int bc = 0;                                        // buffer of tile t
        for (int t = 0; t < ntiles; ++t) {
            if constexpr (KVF == 0) wait_tile(t + 1, t + LA);
            __syncthreads();                               // barrier t: tile t+1 landed
            if constexpr (KVF == 0) {
                const int bn = bc + LA + 1 >= NBUF ? bc + LA + 1 - NBUF : bc + LA + 1;   // = buffer of tile t-1
                if (t + 1 + LA < ntiles) issue_tile(sl, bn);
                sl = read_slot(t + 2 + LA);
            } else {
                // tile t+2 into the buffer tile t-1 has released; codes of tile t+4 out.
                // Constant register-set indices in each branch keep fv in registers (an
                // index of t & 1 would put the array in scratch memory).
                const int bw = bc == 0 ? 2 : bc - 1;
                if (t & 1) {
                    if (t + 2 < ntiles) put(t + 2, fv[1], bw);
                    if (t + 4 < ntiles) fetch(t + 4, fv[1]);
                } else {
                    if (t + 2 < ntiles) put(t + 2, fv[0], bw);
                    if (t + 4 < ntiles) fetch(t + 4, fv[0]);
                }
            }
            const int ps = t & 1;
            const lds_u8* T = tile0 + bc * TB;
            s16x4 va[MTP][2];
#pragma unroll
            for (int mt = 0; mt < MTP; ++mt) {
                va[mt][0] = trd(T, mt, 0);
                va[mt][1] = trd(T, mt, 1);
            }
            bf16x8 pbt[4];
#pragma unroll
            for (int ht = 0; ht < 4; ++ht)
                pbt[ht] = *(const __attribute__((address_space(3))) bf16x8*)((const lds_u8*)pbuf[ps][ht] + lane * 16);
            const int fl = rflag[ps][0] | (rflag[ps][1] << 1) | (rflag[ps][2] << 2) | (rflag[ps][3] << 3);
            if (fl != 0) {
#pragma unroll
                for (int ht = 0; ht < 4; ++ht) {
                    if ((fl >> ht) & 1) {
                        const float al = alph[ps][ht * 16 + l16];
#pragma unroll
                        for (int mt = 0; mt < MTP; ++mt) o[ht][mt] *= al;
                    }
                }
            }
#pragma unroll
            for (int mt = 0; mt < MTP; ++mt) {
                const u32x2 lo = __builtin_bit_cast(u32x2, va[mt][0]);
                const u32x2 hi = __builtin_bit_cast(u32x2, va[mt][1]);
                const bf16x8 v = __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
#pragma unroll
                for (int ht = 0; ht < 4; ++ht)
                    o[ht][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v, pbt[ht], o[ht][mt], 0, 0, 0);
            }
            bc = bc == NBUF - 1 ? 0 : bc + 1;
        }
        __syncthreads();                                   // barrier F
        __syncthreads();                                   // barrier E
        // normalise and store.  O^T accumulator of head tile ht, M-tile mt: lane =
        // head l16, register i = value column 128 pc + 16 mt + 4 g + i.
#pragma unroll
        for (int ht = 0; ht < 4; ++ht) {
            const int head = hb * 64 + ht * 16 + l16;
            if (head >= a.H) continue;
            const float ls = fin_l[ht * 16 + l16];
            const float inv = ls > 0.f ? 1.f / ls : 0.f;
            if (nsplit == 1 && out != nullptr) {
                __bf16* orow = out + ((int64_t)r * a.H + head) * DLAT + pc * DVP + 4 * g;
#pragma unroll
                for (int mt = 0; mt < MTP; ++mt) {
                    bf16x4 v;
#pragma unroll
                    for (int i = 0; i < 4; ++i) v[i] = (__bf16)(o[ht][mt][i] * inv);
                    *(bf16x4*)(orow + 16 * mt) = v;
                }
            } else {
                float* prow = part_o + (((int64_t)r * nsplit + sp) * a.H + head) * DLAT + pc * DVP + 4 * g;
#pragma unroll
                for (int mt = 0; mt < MTP; ++mt) *(f32x4v*)(prow + 16 * mt) = o[ht][mt] * inv;
            }
        }
    }
}

// Merge partial results: out = sum_i e^{lse_i - M} O_i / sum_i e^{lse_i - M},
// lse = M + log sum_i e^{lse_i - M} (M = max_i lse_i; a part with lse = -inf
// holds no row).  Partial i of row r lives at entry (r * row_str + i *
// split_str) * H + h: split-K partials [R, nsplit, H] use (nsplit, 1), the
// gathered shards of a context split [G, R, H] use (1, R).  8 consecutive
// value columns per thread (two 16-byte loads per part), DLAT / 8 threads per
// (row, head), 256 threads per block; bf16 or fp32 output.
template <int DLAT, bool F32OUT>
__global__ __launch_bounds__(256) void sfa_combine_kernel(const float* __restrict__ part_o,
                                                          const float* __restrict__ part_lse, int nsplit,
                                                          int64_t row_str, int64_t split_str, int H, int RH,
                                                          void* __restrict__ out, float* __restrict__ lse) {
    constexpr int TPH = DLAT / 8;            // threads per (row, head)
    static_assert(DLAT % 8 == 0 && 256 % TPH == 0, "shape");
    constexpr int HPB = 256 / TPH;
    const int rh = blockIdx.x * HPB + threadIdx.x / TPH;   // r * H + h
    if (rh >= RH) return;
    const int r = rh / H, h = rh % H;
    const int c = (threadIdx.x % TPH) * 8;
    float M = -__builtin_inff();
    float acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = 0.f;
    float W = 0.f;
    if (nsplit == 2) {
        // both parts' loads in one round trip; the same arithmetic in the same order
        // as the general loop below
        const int64_t e0 = (int64_t)r * row_str * H + h, e1 = ((int64_t)r * row_str + split_str) * H + h;
        const float l0 = part_lse[e0], l1 = part_lse[e1];
        const f32x4* p0 = (const f32x4*)(part_o + e0 * DLAT + c);
        const f32x4* p1 = (const f32x4*)(part_o + e1 * DLAT + c);
        const f32x4 a0 = p0[0], a1 = p0[1], b0 = p1[0], b1 = p1[1];
        M = fmaxf(fmaxf(M, l0), l1);
        if (M != -__builtin_inff()) {
            const float w0 = __expf(l0 - M), w1 = __expf(l1 - M);
            W = w0 + w1;
            const float x0[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
            const float x1[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[j] = fmaf(w1, x1[j], fmaf(w0, x0[j], 0.f));
        }
    } else {
        for (int i = 0; i < nsplit; ++i) M = fmaxf(M, part_lse[((int64_t)r * row_str + i * split_str) * H + h]);
    }
    if (nsplit != 2 && M != -__builtin_inff()) {
        for (int i = 0; i < nsplit; ++i) {
            const int64_t e = ((int64_t)r * row_str + i * split_str) * H + h;
            const float wi = __expf(part_lse[e] - M);
            W += wi;
            const f32x4* po = (const f32x4*)(part_o + e * DLAT + c);
            const f32x4 v0 = po[0], v1 = po[1];
            acc[0] = fmaf(wi, v0.x, acc[0]);
            acc[1] = fmaf(wi, v0.y, acc[1]);
            acc[2] = fmaf(wi, v0.z, acc[2]);
            acc[3] = fmaf(wi, v0.w, acc[3]);
            acc[4] = fmaf(wi, v1.x, acc[4]);
            acc[5] = fmaf(wi, v1.y, acc[5]);
            acc[6] = fmaf(wi, v1.z, acc[6]);
            acc[7] = fmaf(wi, v1.w, acc[7]);
        }
    }
    const float inv = W > 0.f ? 1.f / W : 0.f;
    if constexpr (F32OUT) {
        f32x4* o = (f32x4*)((float*)out + (int64_t)rh * DLAT + c);
        o[0] = f32x4{acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
        o[1] = f32x4{acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv};
    } else {
        bf16x8 v;
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = (__bf16)(acc[j] * inv);
        *(bf16x8*)((__bf16*)out + (int64_t)rh * DLAT + c) = v;
    }
    if (lse != nullptr && c == 0) lse[rh] = W > 0.f ? M + __logf(W) : -__builtin_inff();
}

// Entries of each row's index list inside the row's range [lo, hi) (range[r]
// = {lo, hi}), as positions relative to lo, compacted in list order and
// padded with -1: the part of a gathered index list that one context shard
// holds.  One workgroup of 256 threads per row.
__global__ __launch_bounds__(256) void sfa_localize_kernel(const int32_t* __restrict__ idx, int K,
                                                           const int32_t* __restrict__ range,
                                                           int32_t* __restrict__ out) {
    __shared__ uint32_t wsum[4];
    const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int32_t lo = range[2 * r], hi = range[2 * r + 1];
    const int32_t* in = idx + (int64_t)r * K;
    int32_t* o = out + (int64_t)r * K;
    uint32_t base = 0;
    for (int k0 = 0; k0 < K; k0 += 256) {
        const int i = k0 + tid;
        const int32_t e = i < K ? in[i] : -1;
        const bool take = e >= 0 && e >= lo && e < hi;
        const uint64_t bal = __ballot(take);
        if (lane == 0) wsum[wave] = (uint32_t)__popcll(bal);
        __syncthreads();
        uint32_t before = 0, total = 0;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            before += w < wave ? wsum[w] : 0u;
            total += wsum[w];
        }
        if (take) o[base + before + lanemask_count(bal)] = e - lo;
        base += total;
        __syncthreads();
    }
    for (int i = (int)base + tid; i < K; i += 256) o[i] = -1;
}

// split heuristic shared with the workspace query ------------------------------

struct SfaPlan {
    int nhg;      // 32-head groups per workgroup
    int nhb;      // head blocks
    int nsplit;   // splits of the index list
    int kps;      // index entries per split
};

SfaPlan sfa_plan(int R, int K, int H) {
    SfaPlan p;
    p.nhg = H <= 32 ? 1 : 2;  // 4 waves (64 heads) per workgroup, 1 per SIMD
    p.nhb = (H + 32 * p.nhg - 1) / (32 * p.nhg);
    const int64_t wgs = (int64_t)(R > 0 ? R : 1) * p.nhb;
    int64_t ns = (256 + wgs - 1) / wgs;
    const int64_t max_by_len = (K + 127) / 128;  // keep >= 4 tiles per split
    if (ns > max_by_len) ns = max_by_len;
    const int64_t min_by_lds = (K + kSfaMaxKeys - 1) / kSfaMaxKeys;
    if (ns < min_by_lds) ns = min_by_lds;
    if (ns < 1) ns = 1;
    int kps = (int)((K + ns - 1) / ns);
    kps = (kps + 31) / 32 * 32;
    if (kps > kSfaMaxKeys) kps = kSfaMaxKeys;
    p.kps = kps;
    p.nsplit = (K + kps - 1) / kps;
    return p;
}

// out != nullptr: bf16 output; out == nullptr: fp32 normalised output in
// out_f32 (partial results of one context shard) and lse required.
template <int DLAT, int DROPE, bool FP8, int NHG, bool TSC>
static hipError_t launch_sfa_t(const MlaDev& a, const SfaPlan& p, __bf16* out, float* out_f32, float* lse,
                               float* part_o, float* part_lse, hipStream_t stream) {
    const int64_t units = (int64_t)a.R * p.nsplit;
    const int64_t nwg = (units + 7) / 8 * 8 * p.nhb;
    if (out == nullptr && p.nsplit == 1) {   // one split writes the fp32 result directly
        part_o = out_f32;
        part_lse = lse;
    }
    if (!FP8 && DLAT == 512 && DROPE == 64 && NHG == 2 && p.kps <= 1024)
        hipLaunchKernelGGL((sfa_ws_kernel<512, 64, 4, 1024>), dim3((unsigned)nwg), dim3(512), 0, stream, a, p.kps,
                           p.nsplit, p.nhb, out, lse, part_o, part_lse);
    else if (!FP8 && DLAT == 512 && DROPE == 64 && NHG == 2)
        hipLaunchKernelGGL((sfa_ws_kernel<512, 64, 3, kSfaMaxKeys>), dim3((unsigned)nwg), dim3(512), 0, stream, a,
                           p.kps, p.nsplit, p.nhb, out, lse, part_o, part_lse);
    else if (FP8 && DLAT == 512 && DROPE == 64 && NHG == 2 && p.kps <= 1024)
        // fp8 rows turned into bf16 tiles by the loading waves (factor per row or per 128-column tile)
        hipLaunchKernelGGL((sfa_ws_kernel<512, 64, 3, 1024, TSC ? 2 : 1>), dim3((unsigned)nwg), dim3(512), 0, stream,
                           a, p.kps, p.nsplit, p.nhb, out, lse, part_o, part_lse);
    else if constexpr (!FP8 && ((DLAT + DROPE) * 2) % 128 == 0)
        hipLaunchKernelGGL((sfa_bf16_kernel<DLAT, DROPE, NHG>), dim3((unsigned)nwg), dim3(128 * NHG), 0, stream,
                           a, p.kps, p.nsplit, p.nhb, out, lse, part_o, part_lse);
    else
        hipLaunchKernelGGL((sfa_kernel<DLAT, DROPE, FP8, NHG, TSC>), dim3((unsigned)nwg), dim3(128 * NHG), 0, stream, a,
                           p.kps, p.nsplit, p.nhb, out, lse, part_o, part_lse);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.nsplit == 1) return e;
    constexpr int HPB = 256 / (DLAT / 8);
    const int RH = a.R * a.H;
    if (out != nullptr)
        hipLaunchKernelGGL((sfa_combine_kernel<DLAT, false>), dim3((unsigned)((RH + HPB - 1) / HPB)), dim3(256), 0,
                           stream, part_o, part_lse, p.nsplit, (int64_t)p.nsplit, (int64_t)1, a.H, RH, (void*)out,
                           lse);
    else
        hipLaunchKernelGGL((sfa_combine_kernel<DLAT, true>), dim3((unsigned)((RH + HPB - 1) / HPB)), dim3(256), 0,
                           stream, part_o, part_lse, p.nsplit, (int64_t)p.nsplit, (int64_t)1, a.H, RH,
                           (void*)out_f32, lse);
    return hipGetLastError();
}

hipError_t sfa_dispatch(const MlaDev& a, int D_latent, int kv_mode, __bf16* out, float* out_f32, float* lse, void* ws,
                        hipStream_t stream) {
    // kv_mode: 0 bf16 rows, 1 fp8 rows with per-group factors, 2 fp8 rows with
    // one factor per 128-column tile
    const SfaPlan p = sfa_plan(a.R, a.K, a.H);
    float* part_o = (float*)ws;
    float* part_lse = part_o + (size_t)a.R * p.nsplit * a.H * D_latent;
#define LISFA_SFA_CASE(DL_, DR_, F8_, TS_, G_)                                                         \
    if (D_latent == DL_ && kv_mode == (TS_ ? 2 : F8_ ? 1 : 0) && p.nhg == G_)                          \
        return launch_sfa_t<DL_, DR_, F8_, G_, TS_>(a, p, out, out_f32, lse, part_o, part_lse, stream);
    LISFA_SFA_CASE(512, 64, false, false, 2)
    LISFA_SFA_CASE(512, 64, true, false, 2)
    LISFA_SFA_CASE(512, 64, true, true, 2)
    LISFA_SFA_CASE(512, 64, false, false, 1)
    LISFA_SFA_CASE(512, 64, true, false, 1)
    LISFA_SFA_CASE(512, 64, true, true, 1)
    LISFA_SFA_CASE(64, 16, false, false, 1)
    LISFA_SFA_CASE(64, 16, true, false, 1)
    LISFA_SFA_CASE(64, 16, true, true, 1)
    LISFA_SFA_CASE(64, 16, false, false, 2)
    LISFA_SFA_CASE(64, 16, true, false, 2)
    LISFA_SFA_CASE(64, 16, true, true, 2)
#undef LISFA_SFA_CASE
    return hipErrorInvalidValue;
}

static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Attention of one context shard over the rows of a gathered index list that
// it holds: range[r] = {lo, hi} are the logical positions of row r's
// sequence in this shard (its cache addresses them as 0..hi-lo-1); NULL =
// the list already holds local positions.  fp32 normalised output + lse.
hipError_t sfa_partial_dispatch(const MlaDev& a, const int32_t* range, int D_latent, int kv_mode, float* out_f32,
                                float* lse, void* ws, hipStream_t stream) {
    MlaDev d = a;
    uint8_t* w = (uint8_t*)ws;
    if (range != nullptr) {
        int32_t* li = (int32_t*)w;
        hipLaunchKernelGGL(sfa_localize_kernel, dim3((unsigned)a.R), dim3(256), 0, stream, a.idx, a.K, range, li);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        d.idx = li;
        w += align256((size_t)a.R * a.K * sizeof(int32_t));
    }
    return sfa_dispatch(d, D_latent, kv_mode, nullptr, out_f32, lse, w, stream);
}

// LSE combine of G gathered partial results [G, R, H, D] -> [R, H, D] bf16.
hipError_t lse_combine_dispatch(const float* part_o, const float* part_lse, int G, int R, int H, int D, __bf16* out,
                                float* lse, hipStream_t stream) {
    const int RH = R * H;
    if (RH == 0) return hipSuccess;
#define LISFA_COMB(D_)                                                                                   \
    if (D == D_) {                                                                                       \
        constexpr int HPB = 256 / (D_ / 8);                                                              \
        hipLaunchKernelGGL((sfa_combine_kernel<D_, false>), dim3((unsigned)((RH + HPB - 1) / HPB)), dim3(256), 0, \
                           stream, part_o, part_lse, G, (int64_t)1, (int64_t)R, H, RH, (void*)out, lse);  \
        return hipGetLastError();                                                                        \
    }
    LISFA_COMB(512)
    LISFA_COMB(64)
#undef LISFA_COMB
    return hipErrorInvalidValue;
}

size_t sfa_workspace_bytes(int R, int K, int H, int D_latent) {
    const SfaPlan p = sfa_plan(R, K, H);
    if (p.nsplit <= 1) return 0;
    return (size_t)R * p.nsplit * H * ((size_t)D_latent + 1) * sizeof(float);
}

size_t sfa_partial_workspace_bytes(int R, int K, int H, int D_latent, int with_range) {
    return (with_range ? align256((size_t)R * K * sizeof(int32_t)) : 0) + sfa_workspace_bytes(R, K, H, D_latent);
}

}  // namespace lisfa
