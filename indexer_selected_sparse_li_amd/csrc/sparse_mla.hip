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
// Two kernels compute it:
//  * sfa_mla_kernel, for 512 + 64 rows (the MLA shape of the layer): 64 heads
//    per workgroup, eight waves split by role (scores, value products), bf16
//    MFMA on tiles of 32 gathered rows staged in LDS; fp8 rows are converted
//    to bf16 exactly and their fp32 factors applied to the logits and
//    probabilities (see the kernel's comment);
//  * sfa_kernel, for 64 + 16 rows (the small shape): the four-wave design
//    below.
// Split-K over the index list when rows alone cannot fill the chip, with an
// LSE merge of the parts (sfa_combine_kernel).
//
// sfa_kernel.  A workgroup owns one query row, 32*NHG heads and a
// contiguous range of the row's index list.  Every gathered latent row is
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
                if (a.gather_nt) lds_dma<16, 0, true>(g, lds0 + (uint32_t)(j * NT * 16));
                else lds_dma<16, 0>(g, lds0 + (uint32_t)(j * NT * 16));
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

// Rows that a tile leaves empty (an index of -1, or a position the cache cannot
// address) are loaded from here.
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
// Chunk permutation of the 512 + 64 tiles: for rows of one parity, swz8 maps
// (r / 2) % 8 = m to 2 (m % 4) + m / 4, a bijection (16 consecutive rows read
// at one chunk hit 16 distinct 16-byte bank groups) whose halves m < 4 and
// m >= 4 give distinct chunk pairs (8 consecutive rows read at two adjacent
// chunks by a transpose read hit 16 distinct bank groups).
__device__ __forceinline__ int sfa_swz8(int r) { return (((r >> 1) & 3) << 1) | ((r >> 3) & 1); }

// Sparse MLA attention over 512 + 64 latent rows ---------------------------------
//
// A workgroup owns one query row, a block of 64 heads and a range of the row's
// index list.  Tiles of 32 gathered rows sit in LDS as 8-row groups of 1 KB
// blocks (chunk c of tile row r at (r / 8) * 9 KB + (c / 8) KB + (r % 8) * 128
// + ((c % 8) ^ swz8(r)) * 16), and the eight waves split the work by role; wave
// w runs on SIMD w % 4, so the score work sits on SIMDs 0 and 1 and the value
// products on SIMDs 2 and 3:
//  * q-waves 0, 1 (SIMDs 0, 1): q-wave h owns heads 32 h .. 32 h + 31 of the
//    block (the query as 36 B operands of v_mfma_f32_32x32x16_bf16, 144 VGPRs)
//    and all 32 keys of every tile.  For tile t + 1 it computes
//    S^T[32 keys, 32 heads] (36 MFMAs; every 1 KB key operand read from LDS
//    feeds 32 heads), masks, takes the per-head maxima inside the wave (one
//    permlane swap), raises the base-2 reference lazily (only when the tile's
//    maximum exceeds it by 2^8), and writes P^T into a two-slot LDS ring in the
//    16-head PV B-operand layout (lane = head, K-slots 8 g .. 8 g + 7 = keys
//    4 g + i and 16 + 4 g + i) with a raise flag and factors per head tile.
//  * p-waves 2, 3, 6, 7 (two on each of SIMDs 2, 3): p-wave c (0..3) owns value
//    columns 128 c .. 128 c + 127 of the 64 heads (O^T in 128 VGPRs): it applies
//    the raise factors of flagged head tiles and runs PV of tile t (32 MFMAs of
//    16x16x32), the value operand from transposed LDS reads in the P^T
//    operand's key order, read for tile t + 1 in period t into the registers
//    PV(t) has just taken its operands from, so after the barrier only the P^T
//    operand stands between it and its MFMAs.  bf16 rows: the p-waves also bring
//    the tiles (p-wave c rows 8 c .. 8 c + 7) by direct global->LDS loads
//    NBUF - 2 tiles ahead, issued from inline assembly (lds_dma) and ordered by
//    explicit vmcnt waits and the tile barrier; the first tiles go out before
//    the slot table is complete.
//  * helper waves 4, 5 (SIMDs 0, 1, beside the q-waves' matrix work): the slot
//    table; fp8 rows: the tiles, e4m3 codes two tiles ahead into registers,
//    converted exactly to bf16 (v_cvt_scalef32_pk_bf16_fp8 with scale 1) into
//    the tile one tile ahead, the rows' fp32 factors beside it (NBUF = 3).
// MFMA cycles per tile: 1152 on SIMDs 0 and 1 (QK^T), 1024 on SIMDs 2 and 3
// (PV).  One barrier per tile hands P over; the roles run separate loops with
// the same number of barriers.
//
// fp8 factors are applied exactly, never folded into the bf16 rows:
//  KVF 1 (one factor f per row):  z = scale * f * (q . code), and the P^T
//        operand is p * f (the normaliser sums p);
//  KVF 2 (one factor per 128-column tile j of the row): the QK^T K-steps of
//        each column tile accumulate apart (two alternating accumulators) and
//        are added with the row's f_j two K-steps into the next column tile;
//        p-wave c, whose value columns are column tile c, multiplies its P^T
//        operand by f_c.
//
// Outputs: nsplit == 1: bf16 out (+ lse) or, with out == nullptr, normalised
// fp32 out_f32 + lse; nsplit > 1: normalised bf16 partials part_o [R, nsplit,
// H, 512] + part_lse [R, nsplit, H] for the combine kernel, the 512 columns of
// a part in the store order of the p-waves (value column 32 b + 16 h + 4 g + i
// at 32 b + 8 g + 4 h + i: each lane stores 16 contiguous bytes).
template <int NBUF, int MAXK, int KVF, bool GNT = false>
__global__ __launch_bounds__(512) void sfa_mla_kernel(MlaDev a, int kps, int nsplit, int nhb,
                                                       __bf16* __restrict__ out, float* __restrict__ lse,
                                                       float* __restrict__ out_f32, __bf16* __restrict__ part_o,
                                                       float* __restrict__ part_lse) {
    constexpr int DLAT = 512, DQK = 576;
    constexpr int CPK = DQK * 2 / 16;       // 16-byte chunks per row (72)
    constexpr int NJ = CPK / 8;             // 1 KB blocks per 8-row group (9)
    constexpr int GB = NJ * 1024;           // bytes per 8-row group
    constexpr int TROWS = 32;
    constexpr int TB = (TROWS / 8) * GB;    // bytes per tile
    constexpr int KS = DQK / 32;            // 16x16x32 K-steps of a row (18)
    constexpr int DVP = DLAT / 4;           // value columns per p-wave
    constexpr int MTP = DVP / 16;           // PV M-tiles per p-wave
    constexpr int NTL = KVF == 2 ? (DQK + 127) / 128 : 1;   // fp8 factors per row
    constexpr int LA = NBUF - 2;            // tiles in flight ahead of QK^T
    constexpr int HT = 2;                   // bf16 rows: tiles the helper waves bring (the p-waves the rest)
    static_assert(NBUF >= 3 && (KVF == 0 || NBUF == 3), "PV(t) | QK(t+1) | tiles t+2 ..");
    typedef float f32x4v __attribute__((ext_vector_type(4)));
    typedef __bf16 bf16x4v __attribute__((ext_vector_type(4)));

    __shared__ __attribute__((aligned(1024))) uint8_t tile[NBUF * TB];
    __shared__ uint32_t rslot[MAXK];                    // cache slot of each selected row, ~0 = skip
    __shared__ uint32_t vmask[MAXK / 32];               // valid-row bits of each 32-row tile
    __shared__ __attribute__((aligned(16))) float kvf[KVF ? NBUF * NTL * TROWS : 4];   // [buf][tile j][row]
    __shared__ __attribute__((aligned(16))) uint8_t pbuf[2][4][64 * 16];   // P^T [slot][head tile][lane]
    __shared__ float alph[2][64];                       // raise factors [slot][head]
    __shared__ int rflag[2][4];                         // raised head tiles [slot][head tile]
    __shared__ int s_ntw[2];                            // tiles up to the last valid row, per table-building wave
    // after the last tile the P ring is free: partial row sums [key block][head]
    // (one block for bf16 rows) and the references [head]
    float* const fin_l = (float*)&pbuf[0][0][0];
    float* const fin_m = fin_l + 128;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int bid = blockIdx.x;
    // the head blocks of one (row, split) get workgroup ids 8 apart: they run on
    // one XCD and share its L2 for the rows they both gather (grouping the splits
    // of a row on one XCD as well measured slower)
    const int hb = (bid >> 3) % nhb;
    const int u = ((bid >> 3) / nhb) * 8 + (bid & 7);
    if (u >= a.R * nsplit) return;
    const int r = u / nsplit, sp = u % nsplit;
    const int k0 = sp * kps;
    const int k1 = (k0 + kps < a.K) ? k0 + kps : a.K;
    const int nk = k1 - k0;
    const int seq = a.row_seq[r];
    const int nt_fill = (nk + TROWS - 1) / TROWS;
    // roles: q-waves 0, 1 (32 heads each, SIMDs 0 and 1), p-waves 2, 3, 6, 7
    // (SIMDs 2 and 3), helper waves 4 and 5 (the slot table, the first tiles;
    // fp8 rows: every tile)
    const bool is_q = wave < 2;
    const bool is_p = (wave & 3) >= 2;

    const lds_u8* tile0 = (const lds_u8*)tile;
    const uint32_t tile_lds = (uint32_t)(uintptr_t)tile;
    const int g = lane >> 4, l16 = lane & 15;
    // value column block of a p-wave
    const int pc = (wave & 3) - 2 + 2 * (wave >> 2);
    // bf16 tile loads: lane l brings chunk 8 j + ((l % 8) ^ swz8(row)) of row
    // 8 grp + l / 8 into block j of row group grp, at block + 16 l
    auto row_goff = [&](int grp) { return (uint32_t)(((lane & 7) ^ sfa_swz8(8 * grp + (lane >> 3))) << 4); };
    // one tile's row of this lane in 8-row group grp (row 8 grp + lane / 8);
    // go = the lane's chunk offset for that row
    auto issue_rows = [&](uint32_t s, int buf, int grp, uint32_t go) {
        const uint8_t* gp = (s != 0xFFFFFFFFu ? a.kv.data + (uint64_t)s * (uint32_t)a.kv.row_stride : g_zero_row) + go;
        const uint32_t blk = tile_lds + (uint32_t)(buf * TB + grp * GB);
        // the immediate offset moves both the global and the LDS address; block j
        // lands at blk + j KB.  GNT: non-temporal gathers (the launch's gather_nt)
        static_for<NJ>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            lds_dma<16, j * 128, GNT>(gp, blk + (uint32_t)(j * (1024 - 128)));
        });
    };

    const float kLazy = 8.0f;
    // the last tile with a valid row (trailing tiles without one are skipped; at
    // least one tile is always processed): the q-waves, which build the slot
    // table, count between the two prologue barriers
    // The slot table, built by the helper waves: helper hw owns rows
    // 16 hw .. 16 hw + 15 of every tile (the rows it also brings), lane l entry
    // j = row 16 hw + l % 16 of tile 4 j + l / 16.  Paged caches: the sequence's
    // block-table row is staged in the tile buffer the prologue leaves free (one
    // copy per helper wave) while the index loads are in flight, so a slot costs
    // one LDS read instead of a second dependent global round trip.  Returns the
    // slots in sv; publishes rslot, this helper's 16-bit halves of vmask and, in
    // s_ntw[hw], the number of tiles up to its last valid row.
    constexpr int EPT = MAXK / 128;
    constexpr int kBtStage = (TB / 2) / 4;              // block-table entries one staged copy holds
    auto build_slots = [&](int hw, int64_t (&sv)[EPT]) {
        int pidx[EPT];
#pragma unroll
        for (int j = 0; j < EPT; ++j) {
            const int i = (4 * j + (lane >> 4)) * TROWS + 16 * hw + (lane & 15);
            pidx[j] = i < nk ? a.idx[(int64_t)r * a.K + k0 + i] : -1;
        }
        const int nbt = a.kv.bt_stride;
        const bool staged = a.kv.paged && seq >= 0 && seq < a.kv.num_seqs && (nbt & 3) == 0 && nbt <= kBtStage &&
                            ((uintptr_t)a.kv.block_table & 15) == 0;
        if (staged) {
            const u32x4* src = (const u32x4*)(a.kv.block_table + (int64_t)seq * nbt);
            uint32_t* bt = (uint32_t*)(tile + (NBUF - 1) * TB) + hw * kBtStage;
            const int n4 = nbt >> 2;
            for (int c0 = 0; c0 < n4; c0 += 8 * 64) {
                u32x4 v[8];
#pragma unroll
                for (int m = 0; m < 8; ++m) {
                    const int c = c0 + m * 64 + lane;
                    if (c < n4) v[m] = src[c];
                }
#pragma unroll
                for (int m = 0; m < 8; ++m) {
                    const int c = c0 + m * 64 + lane;
                    if (c < n4) *(__attribute__((address_space(3))) u32x4*)(bt + 4 * c) = v[m];
                }
            }
            const int sh = a.kv.bs_shift;
#pragma unroll
            for (int j = 0; j < EPT; ++j) {
                const int p = pidx[j];
                int64_t sl = -1;
                if (p >= 0 && (p >> sh) < nbt) {
                    const int32_t blk = (int32_t)bt[p >> sh];
                    if (blk >= 0) {
                        sl = ((int64_t)blk << sh) + (p & ((1 << sh) - 1));
                        if (sl >= a.kv.num_slots) sl = -1;
                    }
                }
                sv[j] = sl;
            }
        } else {
#pragma unroll
            for (int j = 0; j < EPT; ++j) sv[j] = pidx[j] >= 0 ? slot_of(a.kv, seq, pidx[j]) : -1;
        }
        int nt_mine = 0;
        uint16_t* vm16 = (uint16_t*)vmask;
#pragma unroll
        for (int j = 0; j < EPT; ++j) {
            const int t = 4 * j + (lane >> 4);
            const int i = t * TROWS + 16 * hw + (lane & 15);
            if (t < nt_fill) rslot[i] = sv[j] >= 0 ? (uint32_t)sv[j] : 0xFFFFFFFFu;
            if (sv[j] >= 0) nt_mine = t + 1;
            const uint64_t bal = __ballot(sv[j] >= 0);
            if (lane < 4 && 4 * j + lane < nt_fill) vm16[(4 * j + lane) * 2 + hw] = (uint16_t)(bal >> (16 * lane));
        }
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) nt_mine = max(nt_mine, __shfl_xor(nt_mine, d));
        if (lane == 0) s_ntw[hw] = nt_mine;
    };
    // after barrier P
    auto read_ntiles = [&]() { return max(1, max(s_ntw[0], s_ntw[1])); };

    if (is_q) {
        // ---------------------------------------------------------------- q-wave
        {
            // q-wave qh owns heads 32 qh .. 32 qh + 31 of the block and all
            // 32 keys of every tile: S^T[32 keys, 32 heads] from 36 K-steps of
            // v_mfma_f32_32x32x16_bf16, every key operand read from LDS feeding 32
            // heads; the per-head maxima need no exchange between waves.  The query
            // as B operand: lane = head l % 32, columns 16 ks + 8 (l / 32) .. + 8.
            constexpr int KS2 = DQK / 16;                  // 36
            const int qh = wave, hq = lane & 31, kh = lane >> 5;
            bf16x8 qb[KS2];
            {
                const int head = hb * 64 + qh * 32 + hq;
#pragma unroll
                for (int j = 0; j < KS2; ++j) {
                    if (head < a.H)
                        qb[j] = *(const bf16x8*)(a.q + (((int64_t)r * a.H + head) * DQK + j * 16 + kh * 8) * 2);
                    else
                        qb[j] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
                }
            }
            // key operand of K-step ks: row hq, chunk 2 ks + kh = block ks / 4,
            // chunk 2 (ks % 4) + kh inside it
            uint32_t qa[4];
#pragma unroll
            for (int m = 0; m < 4; ++m)
                qa[m] = (uint32_t)((hq >> 3) * GB + (hq & 7) * 128 + (((2 * m + kh) ^ sfa_swz8(hq)) << 4));
            auto qk_op = [&](const lds_u8* T, int ks) -> bf16x8 {   // compile-time ks
                return *(const lds_bf16x8*)(T + qa[ks & 3] + (ks >> 2) * 1024);
            };
            float m2 = -__builtin_inff(), lsum = 0.f;
            const float c = a.scale_log2;
            // accumulator register i of lane l: key 8 (i / 4) + 4 (l / 32) + i % 4
            // of head l % 32.  The P^T ring keeps the 16-head operand layout of the
            // p-waves (lane (g, head), K-slots 0..3 = keys 4 g + i, 4..7 = keys
            // 16 + 4 g + i): registers 0..3 and 8..11 of this lane are K-slots of
            // group g = kh, registers 4..7 and 12..15 of group g = 2 + kh.
            const int pt = 2 * qh + (hq >> 4), phl = hq & 15;
            // the fp32 factors of this lane's 16 keys from row table tb of buffer buf
            // (keys 8 k + 4 kh .. + 3 are contiguous)
            auto key_factors = [&](int buf, int tb, float (&f)[16]) {
                const float* kf = kvf + (buf * NTL + tb) * TROWS + 4 * kh;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const f32x4v v = *(const f32x4v*)(kf + 8 * k);
#pragma unroll
                    for (int i = 0; i < 4; ++i) f[4 * k + i] = v[i];
                }
            };
            auto q_tile = [&](const lds_u8* T, int buf, uint32_t vm, int ps) {
                // operand reads in batches of KPB K-steps, software-pipelined: the reads
                // of batch b + 1 go out before the MFMAs of batch b (the scheduling
                // barriers keep the compiler from pairing each read with its MFMA)
                constexpr int KPB = KVF == 2 ? 2 : 6;
                constexpr int NB = KS2 / KPB;
                static_assert(KS2 % KPB == 0, "whole batches");
                f32x16 s;
#pragma unroll
                for (int i = 0; i < 16; ++i) s[i] = 0.f;
                // KVF 2: column tile j (K-steps 8 j .. 8 j + 7; the rope tile 4: 32 .. 35)
                // accumulates into sc[j & 1] and is added, times the keys' f_j, two
                // K-steps into the next column tile
                f32x16 sc[KVF == 2 ? 2 : 1];
                if constexpr (KVF == 2) {
#pragma unroll
                    for (int u = 0; u < 2; ++u)
#pragma unroll
                        for (int i = 0; i < 16; ++i) sc[u][i] = 0.f;
                }
                auto fold = [&](int j) {   // compile-time j: s += f_j(key) * sc[j & 1]
                    const float* kf = kvf + (buf * NTL + j) * TROWS + 4 * kh;
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const f32x4v f = *(const f32x4v*)(kf + 8 * k);
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            s[4 * k + i] = __builtin_fmaf(f[i], sc[j & 1][4 * k + i], s[4 * k + i]);
                            sc[j & 1][4 * k + i] = 0.f;
                        }
                    }
                };
                bf16x8 av[2][KPB];
#pragma unroll
                for (int j = 0; j < KPB; ++j) av[0][j] = qk_op(T, j);
                static_for<NB>([&](auto bc) {
                    constexpr int b = decltype(bc)::value;
                    if constexpr (b + 1 < NB) {
#pragma unroll
                        for (int j = 0; j < KPB; ++j) av[(b + 1) & 1][j] = qk_op(T, (b + 1) * KPB + j);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    static_for<KPB>([&](auto jc) {
                        constexpr int j = decltype(jc)::value;
                        constexpr int ks = b * KPB + j;
                        if constexpr (KVF == 2) {
                            sc[(ks / 8) & 1] = mfma32x32x16_bf16(av[b & 1][j], qb[ks], sc[(ks / 8) & 1]);
                            if constexpr (ks >= 9 && ks % 8 == 1) fold(ks / 8 - 1);
                        } else {
                            s = mfma32x32x16_bf16(av[b & 1][j], qb[ks], s);
                        }
                    });
                    __builtin_amdgcn_sched_barrier(0);
                });
                if constexpr (KVF == 2) fold(NTL - 1);
                float fk[16];   // KVF 1: the factor of each of this lane's keys
                if constexpr (KVF == 1) {
                    key_factors(buf, 0, fk);
                    // one factor per row: the logit is scale * f * (q . code)
#pragma unroll
                    for (int i = 0; i < 16; ++i) s[i] *= fk[i];
                }
                if (vm != 0xFFFFFFFFu) {
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        if (!((vm >> (8 * (i >> 2) + 4 * kh + (i & 3))) & 1u)) s[i] = -__builtin_inff();
                }
                // per-head maximum over the 32 keys: this lane's 16, then the other half
                float tm = s[0];
#pragma unroll
                for (int i = 1; i < 16; ++i) tm = fmaxf(tm, s[i]);
                {
                    const auto w32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(tm), __float_as_uint(tm), false, false);
                    tm = fmaxf(__uint_as_float(w32[0]), __uint_as_float(w32[1]));
                }
                const float tmax = tm * c;   // c > 0
                const bool raise = tmax > m2 + kLazy;   // also true on the first valid tile
                const uint64_t rb = __ballot(raise);
                const float mnew = raise ? tmax : m2;
                const float alpha = raise ? __builtin_amdgcn_exp2f(m2 - mnew) : 1.f;   // m2 = -inf -> 0
                lsum *= alpha;
                m2 = mnew;
                const float negm = mnew == -__builtin_inff() ? 0.f : -mnew;
                float pe[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) pe[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], c, negm));
                float rs = (((pe[0] + pe[1]) + (pe[2] + pe[3])) + ((pe[4] + pe[5]) + (pe[6] + pe[7]))) +
                           (((pe[8] + pe[9]) + (pe[10] + pe[11])) + ((pe[12] + pe[13]) + (pe[14] + pe[15])));
                {
                    const auto w32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(rs), __float_as_uint(rs), false, false);
                    lsum += __uint_as_float(w32[0]) + __uint_as_float(w32[1]);
                }
                if (kh == 0) alph[ps][qh * 32 + hq] = alpha;
                if (lane == 0) {
                    rflag[ps][2 * qh] = (rb & 0x0000FFFF0000FFFFull) != 0ull ? 1 : 0;
                    rflag[ps][2 * qh + 1] = (rb & 0xFFFF0000FFFF0000ull) != 0ull ? 1 : 0;
                }
                // KVF 1: the P^T operand is p * f (the normaliser sums p)
                float pf[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) pf[i] = KVF == 1 ? pe[i] * fk[i] : pe[i];
                bf16x8 p0, p1;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    p0[i] = (__bf16)pf[i];
                    p0[4 + i] = (__bf16)pf[8 + i];
                    p1[i] = (__bf16)pf[4 + i];
                    p1[4 + i] = (__bf16)pf[12 + i];
                }
                lds_u8* pp = (lds_u8*)pbuf[ps][pt];
                *(__attribute__((address_space(3))) bf16x8*)(pp + (kh * 16 + phl) * 16) = p0;
                *(__attribute__((address_space(3))) bf16x8*)(pp + ((2 + kh) * 16 + phl) * 16) = p1;
            };

            __syncthreads();                                   // barrier P: the slot table is complete, tile 0 landed
            const int ntiles = read_ntiles();
            q_tile(tile0, 0, vmask[0], 0);
            int bq = 1;                                        // buffer of tile t+1
            for (int t = 0; t < ntiles; ++t) {
                __syncthreads();                               // barrier t: P(t) published, tile t+1 landed
                if (t + 1 < ntiles) {
                    const uint32_t vmn = __builtin_amdgcn_readfirstlane(vmask[t + 1]);
                    q_tile(tile0 + bq * TB, bq, vmn, (t + 1) & 1);
                }
                bq = bq == NBUF - 1 ? 0 : bq + 1;
            }
            __syncthreads();                                   // barrier F: the P ring is no longer read
            if (kh == 0) {
                fin_l[qh * 32 + hq] = lsum;
                fin_m[qh * 32 + hq] = m2;
            }
            __syncthreads();                                   // barrier E
        }
    } else if (!is_p) {
        // ------------------------------------------------------ helper waves 4, 5
        // The slot table, then the first tiles, helper hw rows 16 hw .. 16 hw + 15
        // of each.  bf16 rows: tiles 0 .. HT - 1 by direct global->LDS loads from
        // the slots still in registers (the p-waves bring the later tiles); the
        // helper waits for tile t + 1 (< HT) before barrier t.  fp8 rows: every tile: in
        // 1 KB block j, lane l owns position l % 8 of row 16 hw + 8 rr + l / 8,
        // i.e. bf16 chunk 8 j + ((l % 8) ^ swz8(row)) = 8 columns: it loads their 8
        // e4m3 codes, converts them exactly and writes the 16 bytes (one
        // contiguous 1 KB per instruction).  Codes go out two tiles ahead,
        // converted tiles one tile ahead (tile t + 2 into the buffer tile t - 1 has
        // released, in period t).
        const int hw = wave - 4;
        int64_t sv[EPT];
        build_slots(hw, sv);
        // helper tile j landed (j < HT); later helper tiles may still be in flight
        static_assert(HT == 2 && HT <= LA + 1 && 2 * NJ < 64, "vmcnt covers the helper tiles in flight");
        auto hwait = [&](int j) {
            if (j == 0 && 1 < nt_fill) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * NJ) : "memory");
            else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        };
        if constexpr (KVF == 0) {
            // tile t row 16 hw + 8 rr + l / 8 = entry 0 of lane 16 t + 8 rr + l / 8
#pragma unroll
            for (int t = 0; t < HT; ++t) {
#pragma unroll
                for (int rr = 0; rr < 2; ++rr) {
                    const int64_t sl = __shfl(sv[0], 16 * t + 8 * rr + (lane >> 3));
                    if (t < nt_fill) issue_rows(sl >= 0 ? (uint32_t)sl : 0xFFFFFFFFu, t, 2 * hw + rr, row_goff(2 * hw + rr));
                }
            }
        }
        // KVF 2: lane q (q < NTL) of a row's 8 lanes holds the row's factor of
        // column tile q (one load per row group instead of NTL); KVF 1: every lane
        // holds the row's factor
        // codes of the 512 latent columns as 16-byte loads (lane: pair
        // p = 8 k + l % 8 of 16 columns, bf16 chunks 2 p and 2 p + 1), the 64 rope
        // columns as one 8-byte load (chunk 64 + ((l % 8) ^ swz8(row)))
        struct Codes {
            u32x4 v[2][4];
            u32x2 rope[2];
            float f[2];
        };
        int frow[2], fsw[2];
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
            frow[rr] = 16 * hw + 8 * rr + (lane >> 3);
            fsw[rr] = (lane & 7) ^ sfa_swz8(frow[rr]);
        }
        auto fetch = [&](int t, Codes& cd) {
#pragma unroll
            for (int rr = 0; rr < 2; ++rr) {
                const uint32_t sl = t < nt_fill ? rslot[t * TROWS + frow[rr]] : 0xFFFFFFFFu;
                const bool ok = sl != 0xFFFFFFFFu;
                const uint8_t* gp = ok ? a.kv.data + (uint64_t)sl * (uint32_t)a.kv.row_stride : g_zero_row;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const u32x4* src = (const u32x4*)(gp + (8 * k + (lane & 7)) * 16);
                    cd.v[rr][k] = a.gather_nt ? __builtin_nontemporal_load(src) : *src;
                }
                {
                    const u32x2* src = (const u32x2*)(gp + (64 + fsw[rr]) * 8);
                    cd.rope[rr] = a.gather_nt ? __builtin_nontemporal_load(src) : *src;
                }
                if constexpr (KVF == 1) {
                    cd.f[rr] = ok ? a.kv.scale[(int64_t)sl / a.kv.scale_group] : 0.f;
                } else if constexpr (KVF == 2) {
                    const int q = lane & 7;
                    cd.f[rr] = ok && q < NTL ? a.kv.scale[(int64_t)sl * NTL + q] : 0.f;
                }
            }
        };
        auto put = [&](const Codes& cd, int buf) {
            auto cvt8 = [](u32x2 c) {   // 8 e4m3 codes -> 8 bf16, exact
                u32x4 b;
                b.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.x, 1.0f, false));
                b.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.x, 1.0f, true));
                b.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.y, 1.0f, false));
                b.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.y, 1.0f, true));
                return b;
            };
#pragma unroll
            for (int rr = 0; rr < 2; ++rr) {
                lds_u8* grp = (lds_u8*)tile + buf * TB + (2 * hw + rr) * GB;
                lds_u8* rowp = grp + (lane >> 3) * 128;
                const int sw = sfa_swz8(frow[rr]);
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int pp = 8 * k + (lane & 7);            // chunks 2 pp, 2 pp + 1 of block pp / 4
                    lds_u8* blk = rowp + (pp >> 2) * 1024;
                    const int c0 = (2 * pp) & 7;
                    *(__attribute__((address_space(3))) u32x4*)(blk + ((c0 ^ sw) << 4)) = cvt8(u32x2{cd.v[rr][k].x, cd.v[rr][k].y});
                    *(__attribute__((address_space(3))) u32x4*)(blk + (((c0 + 1) ^ sw) << 4)) =
                        cvt8(u32x2{cd.v[rr][k].z, cd.v[rr][k].w});
                }
                *(__attribute__((address_space(3))) u32x4*)(grp + lane * 16 + 8 * 1024) = cvt8(cd.rope[rr]);
                if constexpr (KVF == 1) {
                    if ((lane & 7) == 0) kvf[buf * TROWS + frow[rr]] = cd.f[rr];
                } else if constexpr (KVF == 2) {
                    const int q = lane & 7;
                    if (q < NTL) kvf[(buf * NTL + q) * TROWS + frow[rr]] = cd.f[rr];
                }
            }
        };
        Codes c0, c1;
        if constexpr (KVF != 0) {
            fetch(0, c0);
            fetch(1, c1);
            put(c0, 0);
            put(c1, 1);
            fetch(2, c0);
            fetch(3, c1);
        } else {
            hwait(0);
        }
        __syncthreads();                                   // barrier P: the slot table is complete, tile 0 landed
        const int ntiles = read_ntiles();
        int bc = 0;                                        // buffer of tile t
        for (int t = 0; t < ntiles; ++t) {
            if constexpr (KVF == 0)
                if (t + 1 < HT) hwait(t + 1);
            __syncthreads();                               // barrier t
            if constexpr (KVF != 0) {
                // tile t+2 into the buffer tile t-1 has released; codes of tile t+4 out.
                // Constant register-set names in each branch keep the codes in registers.
                const int bw = bc == 0 ? 2 : bc - 1;
                if (t & 1) {
                    if (t + 2 < ntiles) put(c1, bw);
                    if (t + 4 < ntiles) fetch(t + 4, c1);
                } else {
                    if (t + 2 < ntiles) put(c0, bw);
                    if (t + 4 < ntiles) fetch(t + 4, c0);
                }
            }
            bc = bc == NBUF - 1 ? 0 : bc + 1;
        }
        __syncthreads();                                   // barrier F
        __syncthreads();                                   // barrier E
    } else {
        // ---------------------------------------------------------------- p-wave
        // bf16 rows: the helpers bring tiles 0 .. HT - 1; tiles HT .. LA go out
        // after barrier P, tile t + 1 + LA in iteration t, each into the buffer
        // tile t - 1 has released.  Every tile is NJ loads per thread: "tile j
        // landed" = at most NJ * (tiles issued after j) loads still pending.
        static_assert(LA <= 2 && NJ * LA < 64, "vmcnt covers the tiles in flight");
        int ntiles = 1;
        auto issued = [&](int i) { return i >= HT && i < ntiles; };
        auto wait_tile = [&](int j, int last) {            // tile j landed; tiles up to `last` issued
            if (j < HT) return;                            // a helper tile: waited for by the helpers
            int after = 0;
#pragma unroll
            for (int d = 1; d <= LA; ++d) after += (j + d <= last && issued(j + d)) ? 1 : 0;
            if (after >= 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * NJ) : "memory");
            else if (after == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NJ) : "memory");
            else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        };
        const int prow = 8 * pc + (lane >> 3);            // bf16 rows: this lane's row of every tile
        const uint32_t pgo = row_goff(pc);
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

        // the V operands of tile t + 1 are read in period t, into the registers the
        // PV products of tile t have just taken theirs from, so after barrier t + 1
        // only the P^T operand stands between the p-wave and its MFMAs
        auto read_v = [&](const lds_u8* T, s16x4 (&va)[MTP][2]) {
#pragma unroll
            for (int mt = 0; mt < MTP; ++mt) {
                va[mt][0] = trd(T, mt, 0);
                va[mt][1] = trd(T, mt, 1);
            }
        };
        s16x4 va[MTP][2];
        __syncthreads();                                   // barrier P: the slot table is complete, tile 0 landed
        ntiles = read_ntiles();
        if constexpr (KVF == 0) {
#pragma unroll
            for (int t = HT; t <= LA; ++t)
                if (t < ntiles) issue_rows(rslot[t * TROWS + prow], t, pc, pgo);
        }
        read_v(tile0, va);
        int bc = 0;                                        // buffer of tile t
        for (int t = 0; t < ntiles; ++t) {
            if constexpr (KVF == 0) wait_tile(t + 1, t + LA);
            __syncthreads();                               // barrier t: P(t) published, tile t+1 landed
            if constexpr (KVF == 0) {
                const int bn = bc + LA + 1 >= NBUF ? bc + LA + 1 - NBUF : bc + LA + 1;   // = buffer of tile t-1
                if (t + 1 + LA < ntiles) issue_rows(rslot[(t + 1 + LA) * TROWS + prow], bn, pc, pgo);
            }
            const int ps = t & 1;
            bf16x8 pbt[4];
#pragma unroll
            for (int ht = 0; ht < 4; ++ht)
                pbt[ht] = *(const __attribute__((address_space(3))) bf16x8*)((const lds_u8*)pbuf[ps][ht] + lane * 16);
            if constexpr (KVF == 2) {
                // value columns of column tile pc: the P^T operand times the keys' f_pc
                const float* kf = kvf + (bc * NTL + pc) * TROWS;
                const f32x4v f0 = *(const f32x4v*)(kf + 4 * g);
                const f32x4v f1 = *(const f32x4v*)(kf + 16 + 4 * g);
#pragma unroll
                for (int ht = 0; ht < 4; ++ht) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) pbt[ht][e] = (__bf16)((float)pbt[ht][e] * (e < 4 ? f0[e] : f1[e - 4]));
                }
            }
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
            if (t + 1 < ntiles) read_v(tile0 + (bc == NBUF - 1 ? 0 : bc + 1) * TB, va);
            bc = bc == NBUF - 1 ? 0 : bc + 1;
        }
        __syncthreads();                                   // barrier F
        __syncthreads();                                   // barrier E
        // normalise and store.  O^T accumulator of head tile ht, M-tile mt: lane =
        // head l16, register i = value column 128 pc + 16 mt + 4 g + i.
#pragma unroll
        for (int ht = 0; ht < 4; ++ht) {
            const int head = hb * 64 + ht * 16 + l16;
            const float ls = fin_l[ht * 16 + l16];
            const float mref = fin_m[ht * 16 + l16];
            if (head >= a.H) continue;
            const float inv = ls > 0.f ? 1.f / ls : 0.f;
            if (pc == 0 && g == 0) {
                const float l_nat = ls > 0.f ? (mref + log2f(ls)) * kLn2 : -__builtin_inff();
                if (nsplit == 1) {
                    if (lse != nullptr) lse[(int64_t)r * a.H + head] = l_nat;
                } else {
                    part_lse[((int64_t)r * nsplit + sp) * a.H + head] = l_nat;
                }
            }
            const int64_t col0 = pc * DVP + 4 * g;
            if (nsplit > 1) {
                // split-K part in store order: of the head's 128 columns of this
                // p-wave, M-tiles 2s and 2s + 1 of lane group g go to the 16 bytes
                // at 32 s + 8 g (each store writes 64 contiguous bytes per head);
                // the combine kernel reads this order back
                __bf16* prow = part_o + (((int64_t)r * nsplit + sp) * a.H + head) * DLAT + pc * DVP + 8 * g;
#pragma unroll
                for (int s2 = 0; s2 < MTP / 2; ++s2) {
                    bf16x8 v;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        v[i] = (__bf16)(o[ht][2 * s2][i] * inv);
                        v[4 + i] = (__bf16)(o[ht][2 * s2 + 1][i] * inv);
                    }
                    *(bf16x8*)(prow + 32 * s2) = v;
                }
            } else if (out_f32 != nullptr) {
                float* orow = out_f32 + ((int64_t)r * a.H + head) * DLAT + col0;
#pragma unroll
                for (int mt = 0; mt < MTP; ++mt) *(f32x4v*)(orow + 16 * mt) = o[ht][mt] * inv;
            } else {
                __bf16* orow = out + ((int64_t)r * a.H + head) * DLAT + col0;
#pragma unroll
                for (int mt = 0; mt < MTP; ++mt) {
                    bf16x4 v;
#pragma unroll
                    for (int i = 0; i < 4; ++i) v[i] = (__bf16)(o[ht][mt][i] * inv);
                    *(bf16x4*)(orow + 16 * mt) = v;
                }
            }
        }
    }
}

// Merge partial results: out = sum_i e^{lse_i - M} O_i / sum_i e^{lse_i - M},
// lse = M + log sum_i e^{lse_i - M} (M = max_i lse_i; a part with lse = -inf
// holds no row).  Partial i of row r lives at entry (r * row_str + i *
// split_str) * H + h: split-K partials [R, nsplit, H] use (nsplit, 1), the
// gathered shards of a context split [G, R, H] use (1, R).  Partials are bf16
// (the 512 + 64 attention's split-K parts) or fp32; 8 consecutive value
// columns per thread, DLAT / 8 threads per (row, head), 256 threads per
// block; bf16 or fp32 output.  SORD: the parts hold their columns in the
// 512 + 64 kernel's store order (of each 32 columns, 4-column groups 0 and 4,
// 1 and 5, 2 and 6, 3 and 7 side by side); the output is in value order.
template <int DLAT, typename PT, bool F32OUT, bool SORD = false>
__global__ __launch_bounds__(256) void sfa_combine_kernel(const PT* __restrict__ part_o,
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
    auto load8 = [&](int64_t e, float (&x)[8]) {   // 8 values of part entry e from column c
        if constexpr (std::is_same<PT, float>::value) {
            const f32x4* po = (const f32x4*)(part_o + e * DLAT + c);
            const f32x4 v0 = po[0], v1 = po[1];
            x[0] = v0.x; x[1] = v0.y; x[2] = v0.z; x[3] = v0.w;
            x[4] = v1.x; x[5] = v1.y; x[6] = v1.z; x[7] = v1.w;
        } else {
            const bf16x8 v = *(const bf16x8*)(part_o + e * DLAT + c);
#pragma unroll
            for (int j = 0; j < 8; ++j) x[j] = (float)v[j];
        }
    };
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
        float x0[8], x1[8];
        load8(e0, x0);
        load8(e1, x1);
        M = fmaxf(fmaxf(M, l0), l1);
        if (M != -__builtin_inff()) {
            const float w0 = __expf(l0 - M), w1 = __expf(l1 - M);
            W = w0 + w1;
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[j] = fmaf(w1, x1[j], fmaf(w0, x0[j], 0.f));
        }
    } else {
        // the parts' lse values 16 at a time, all in flight together (a loop of
        // single loads waits one round trip per part)
        for (int i0 = 0; i0 < nsplit; i0 += 16) {
            float l[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int i = i0 + j < nsplit ? i0 + j : nsplit - 1;
                l[j] = part_lse[((int64_t)r * row_str + i * split_str) * H + h];
            }
#pragma unroll
            for (int j = 0; j < 16; ++j) M = fmaxf(M, l[j]);
        }
    }
    if (nsplit != 2 && M != -__builtin_inff()) {
        // CH parts' loads issued together, then their terms added in part order
        constexpr int CH = std::is_same<PT, float>::value ? 8 : 16;
        for (int i0 = 0; i0 < nsplit; i0 += CH) {
            float l[CH], x[CH][8];
#pragma unroll
            for (int j = 0; j < CH; ++j) {
                const int i = i0 + j < nsplit ? i0 + j : nsplit - 1;
                const int64_t e = ((int64_t)r * row_str + i * split_str) * H + h;
                l[j] = part_lse[e];
                load8(e, x[j]);
            }
#pragma unroll
            for (int j = 0; j < CH; ++j) {
                if (i0 + j < nsplit) {
                    const float wi = __expf(l[j] - M);
                    W += wi;
#pragma unroll
                    for (int c8 = 0; c8 < 8; ++c8) acc[c8] = fmaf(wi, x[j][c8], acc[c8]);
                }
            }
        }
    }
    const float inv = W > 0.f ? 1.f / W : 0.f;
    if constexpr (SORD) {
        // lane q of each quad holds 4-column groups q and q + 4 of a 32-column
        // block; two quad permutations give it groups 2 q and 2 q + 1, the 8
        // value columns from c (every lane of a quad works on the same head)
        const bool lowq = (threadIdx.x & 2) == 0;
        float y[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t a = __float_as_uint(acc[j]), b = __float_as_uint(acc[4 + j]);
            const uint32_t a0 = dpp<0x88, 0xF>(0u, a), b0 = dpp<0x88, 0xF>(0u, b);   // from quad lanes 0 2 0 2
            const uint32_t a1 = dpp<0xDD, 0xF>(0u, a), b1 = dpp<0xDD, 0xF>(0u, b);   // from quad lanes 1 3 1 3
            y[j] = __uint_as_float(lowq ? a0 : b0);
            y[4 + j] = __uint_as_float(lowq ? a1 : b1);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = y[j];
    }
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
    int hpb;      // heads per workgroup
    int nhb;      // head blocks
    int nsplit;   // splits of the index list
    int kps;      // index entries per split
};

// 512 + 64 rows: 64-head workgroups (sfa_mla_kernel); 64 + 16 rows: 32 or 64
// heads (sfa_kernel).  The index list of a row is split only as far as needed
// to give the chip about 256 workgroups, keeping >= 4 tiles per split.
SfaPlan sfa_plan(int R, int K, int H, int D_latent) {
    SfaPlan p;
    p.hpb = D_latent == 512 ? 64 : (H <= 32 ? 32 : 64);
    p.nhb = (H + p.hpb - 1) / p.hpb;
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

// bytes of split-K partials: bf16 outputs for 512 + 64 rows, fp32 otherwise,
// then the fp32 lse of every part
static size_t sfa_part_elt(int D_latent) { return D_latent == 512 ? 2 : 4; }

// kv_mode: 0 bf16 rows, 1 fp8 rows with per-group factors, 2 fp8 rows with one
// factor per 128-column tile.  out != nullptr: bf16 output; out == nullptr:
// fp32 normalised output in out_f32 (partial results of one context shard),
// lse required.
static hipError_t launch_sfa512(const MlaDev& a, const SfaPlan& p, int kv_mode, __bf16* out, float* out_f32,
                                float* lse, __bf16* part_o, float* part_lse, hipStream_t stream) {
    const int64_t units = (int64_t)a.R * p.nsplit;
    const dim3 grid((unsigned)((units + 7) / 8 * 8 * p.nhb)), block(512);
#define LISFA_MLA4(NB_, MK_, KVF_, GNT_)                                                                     \
    hipLaunchKernelGGL((sfa_mla_kernel<NB_, MK_, KVF_, GNT_>), grid, block, 0, stream, a, p.kps, p.nsplit, p.nhb, \
                       out, lse, out_f32, part_o, part_lse)
#define LISFA_MLA(NB_, MK_, KVF_) LISFA_MLA4(NB_, MK_, KVF_, false)
    const bool short_list = p.kps <= 1024;
    // bf16 rows: the gather policy is a template argument (fp8 rows read a.gather_nt)
    if (kv_mode == 0 && short_list) {
        if (a.gather_nt) LISFA_MLA4(4, 1024, 0, true);
        else LISFA_MLA4(4, 1024, 0, false);
    } else if (kv_mode == 0) {
        if (a.gather_nt) LISFA_MLA4(3, kSfaMaxKeys, 0, true);
        else LISFA_MLA4(3, kSfaMaxKeys, 0, false);
    } else if (kv_mode == 1 && short_list) {
        LISFA_MLA(3, 1024, 1);
    } else if (kv_mode == 1) {
        LISFA_MLA(3, kSfaMaxKeys, 1);
    } else if (short_list) {
        LISFA_MLA(3, 1024, 2);
    } else {
        LISFA_MLA(3, kSfaMaxKeys, 2);
    }
#undef LISFA_MLA
#undef LISFA_MLA4
    return hipGetLastError();
}

template <bool FP8, int NHG, bool TSC>
static hipError_t launch_sfa64(const MlaDev& a, const SfaPlan& p, __bf16* out, float* out_f32, float* lse,
                               float* part_o, float* part_lse, hipStream_t stream) {
    const int64_t units = (int64_t)a.R * p.nsplit;
    const int64_t nwg = (units + 7) / 8 * 8 * p.nhb;
    if (out == nullptr && p.nsplit == 1) {   // one split writes the fp32 result directly
        part_o = out_f32;
        part_lse = lse;
    }
    hipLaunchKernelGGL((sfa_kernel<64, 16, FP8, NHG, TSC>), dim3((unsigned)nwg), dim3(128 * NHG), 0, stream, a,
                       p.kps, p.nsplit, p.nhb, out, lse, part_o, part_lse);
    return hipGetLastError();
}

// SORD: the parts are in the 512 + 64 kernel's store order
template <int DLAT, typename PT, bool SORD>
static hipError_t launch_combine(const MlaDev& a, const SfaPlan& p, const PT* part_o, const float* part_lse,
                                 __bf16* out, float* out_f32, float* lse, hipStream_t stream) {
    constexpr int HPB = 256 / (DLAT / 8);
    const int RH = a.R * a.H;
    const dim3 grid((unsigned)((RH + HPB - 1) / HPB));
    if (out != nullptr)
        hipLaunchKernelGGL((sfa_combine_kernel<DLAT, PT, false, SORD>), grid, dim3(256), 0, stream, part_o, part_lse,
                           p.nsplit, (int64_t)p.nsplit, (int64_t)1, a.H, RH, (void*)out, lse);
    else
        hipLaunchKernelGGL((sfa_combine_kernel<DLAT, PT, true, SORD>), grid, dim3(256), 0, stream, part_o, part_lse,
                           p.nsplit, (int64_t)p.nsplit, (int64_t)1, a.H, RH, (void*)out_f32, lse);
    return hipGetLastError();
}

hipError_t sfa_dispatch(const MlaDev& a, int D_latent, int kv_mode, __bf16* out, float* out_f32, float* lse, void* ws,
                        hipStream_t stream) {
    const SfaPlan p = sfa_plan(a.R, a.K, a.H, D_latent);
    const size_t npart = (size_t)a.R * p.nsplit * a.H;
    float* part_lse = (float*)((uint8_t*)ws + npart * D_latent * sfa_part_elt(D_latent));
    hipError_t e;
    if (D_latent == 512) {
        __bf16* part_o = (__bf16*)ws;
        e = launch_sfa512(a, p, kv_mode, out, out_f32, lse, part_o, part_lse, stream);
        if (e != hipSuccess || p.nsplit == 1) return e;
        return launch_combine<512, __bf16, true>(a, p, part_o, part_lse, out, out_f32, lse, stream);
    }
    if (D_latent != 64) return hipErrorInvalidValue;
    float* part_o = (float*)ws;
    const bool g2 = p.hpb == 64;
    if (kv_mode == 0) e = g2 ? launch_sfa64<false, 2, false>(a, p, out, out_f32, lse, part_o, part_lse, stream)
                             : launch_sfa64<false, 1, false>(a, p, out, out_f32, lse, part_o, part_lse, stream);
    else if (kv_mode == 1) e = g2 ? launch_sfa64<true, 2, false>(a, p, out, out_f32, lse, part_o, part_lse, stream)
                                  : launch_sfa64<true, 1, false>(a, p, out, out_f32, lse, part_o, part_lse, stream);
    else e = g2 ? launch_sfa64<true, 2, true>(a, p, out, out_f32, lse, part_o, part_lse, stream)
                : launch_sfa64<true, 1, true>(a, p, out, out_f32, lse, part_o, part_lse, stream);
    if (e != hipSuccess || p.nsplit == 1) return e;
    return launch_combine<64, float, false>(a, p, part_o, part_lse, out, out_f32, lse, stream);
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
        hipLaunchKernelGGL((sfa_combine_kernel<D_, float, false>), dim3((unsigned)((RH + HPB - 1) / HPB)), dim3(256), 0, \
                           stream, part_o, part_lse, G, (int64_t)1, (int64_t)R, H, RH, (void*)out, lse);  \
        return hipGetLastError();                                                                        \
    }
    LISFA_COMB(512)
    LISFA_COMB(64)
#undef LISFA_COMB
    return hipErrorInvalidValue;
}

size_t sfa_workspace_bytes(int R, int K, int H, int D_latent) {
    const SfaPlan p = sfa_plan(R, K, H, D_latent);
    if (p.nsplit <= 1) return 0;
    const size_t npart = (size_t)R * p.nsplit * H;
    return npart * D_latent * sfa_part_elt(D_latent) + npart * sizeof(float);
}

size_t sfa_partial_workspace_bytes(int R, int K, int H, int D_latent, int with_range) {
    return (with_range ? align256((size_t)R * K * sizeof(int32_t)) : 0) + sfa_workspace_bytes(R, K, H, D_latent);
}

}  // namespace lisfa
