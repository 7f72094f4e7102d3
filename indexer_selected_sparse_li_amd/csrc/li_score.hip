// Lightning indexer scores on gfx950 MFMA.
//
// score[r, s] = sum_j w[r, j] * ReLU(q_idx[r, j, :] . k_idx[slot(s), :]) for
// s <= row_pos[r] ("Large Language Model Inference Acceleration in Practice",
// section 1.2 Lightning Indexer and section 3.1: relevance scores followed by
// head-weight weighting).
//
// Work decomposition.  A workgroup of 8 wavefronts owns QG query rows of one
// sequence and a contiguous chunk of key positions.  Key tiles of TK keys are
// gathered from the (paged or contiguous) key cache with coalesced 16-byte
// loads into registers one tile ahead, then written to a padded LDS tile.
// Wave w handles query row (w % QG) and the 32-key subtile (w / QG):
//   decode  (QG = 1): the 8 waves split a 256-key tile, one query row;
//   prefill (QG = 8): the 8 waves share a 32-key tile, eight query rows.
// Per wave the head x key product S[32 heads, 32 keys] is one
// v_mfma_f32_32x32x16 per 16-element K-step and 32-head M-tile: A = the
// query's heads (held in VGPRs for the whole kernel), B = K^T read from LDS.
// In the 32x32 accumulator layout lane l holds key l%32 and 16 heads, so the
// weighted ReLU sum over heads is 16*MT fused multiply-adds per lane plus one
// cross-half exchange (lane l ^ 32).  Scores are fp32 end to end.
#include "common.hpp"

namespace lisfa {

constexpr int kLiMaxBlocks = 512;  // block-table entries one workgroup may touch

template <int DI, int MT, int QG, bool FP8>
__global__ __launch_bounds__(512) void li_score_kernel(IndexerDev a, float* __restrict__ scores,
                                                       int64_t ld, int keys_per_wg) {
    constexpr int ELT = FP8 ? 1 : 2;
    constexpr int RB = DI * ELT;            // bytes of one key row
    constexpr int CPK = RB / 16;            // 16-byte chunks per key row
    constexpr int RBP = RB + 16;            // padded LDS row stride (bank spread)
    constexpr int NST = 8 / QG;             // 32-key subtiles per tile
    constexpr int TK = 32 * NST;            // keys per tile
    constexpr int TCH = TK * CPK;           // chunks per tile
    constexpr int NPRE = (TCH + 511) / 512; // chunks per thread
    constexpr int KS = DI / 16;             // MFMA K-steps

    __shared__ __attribute__((aligned(16))) uint8_t tile[TK * RBP];
    __shared__ float kmul[TK];
    __shared__ int32_t blk_id[kLiMaxBlocks];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int qi = wave % QG;
    const int st = wave / QG;
    const int r0 = blockIdx.y * QG;
    const int r = r0 + qi;
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

    int64_t vis = 0;
    bool row_ok = false, row_bad = false;
    if (r < a.R) {
        vis = (int64_t)a.row_pos[r] + 1;
        if (vis < 0) vis = 0;
        if (vis > ld) vis = ld;
        row_ok = a.row_seq[r] == seq0;
        row_bad = !row_ok;
    }

    // block-table entries for [c0, kend)
    const int sh = a.k.bs_shift;
    const int64_t b0 = a.k.paged ? (c0 >> sh) : 0;
    if (a.k.paged) {
        const int nb = (int)(((kend - 1) >> sh) - b0 + 1);
        for (int i = tid; i < nb; i += 512) {
            int64_t blk = b0 + i;
            int32_t v = -1;
            if (seq0 >= 0 && seq0 < a.k.num_seqs && blk < a.k.bt_stride)
                v = a.k.block_table[(int64_t)seq0 * a.k.bt_stride + blk];
            blk_id[i] = v;
        }
    }
    const int64_t cbase = (!a.k.paged && seq0 >= 0 && seq0 < a.k.num_seqs) ? a.k.seq_base[seq0] : -1;
    __syncthreads();

    auto slot_at = [&](int64_t pos) -> int64_t {
        int64_t s;
        if (a.k.paged) {
            int32_t b = blk_id[(pos >> sh) - b0];
            if (b < 0) return -1;
            s = ((int64_t)b << sh) + (pos & ((1 << sh) - 1));
        } else {
            if (cbase < 0) return -1;
            s = cbase + pos;
        }
        return (s >= 0 && s < a.k.num_slots) ? s : -1;
    };

    // query heads of this wave's row in MFMA A-operand layout, and weights in
    // the accumulator's head layout
    typedef typename std::conditional<FP8, int64_t, bf16x8>::type OpT;
    OpT qa[MT][KS];
    float wv[MT][16];
    {
        const bool have = row_ok;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int head = mt * 32 + (lane & 31);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                if (have && head < a.H_I) {
                    const uint8_t* p = a.q + (((int64_t)r * a.H_I + head) * DI + ks * 16 + (lane >> 5) * 8) * ELT;
                    if constexpr (FP8) qa[mt][ks] = *(const int64_t*)p;
                    else qa[mt][ks] = *(const bf16x8*)p;
                } else {
                    if constexpr (FP8) qa[mt][ks] = 0;
                    else qa[mt][ks] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
                }
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int h = mt * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
                float wvv = 0.f;
                if (have && h < a.H_I) {
                    wvv = a.w[(int64_t)r * a.H_I + h];
                    if constexpr (FP8)
                        wvv *= a.q_scale_per_head ? a.q_scale[(int64_t)r * a.H_I + h] : a.q_scale[r];
                }
                wv[mt][i] = wvv;
            }
        }
    }

    u32x4 pre[NPRE];
    float pre_mul = 0.f;
    auto prefetch = [&](int64_t t0) {
#pragma unroll
        for (int j = 0; j < NPRE; ++j) {
            const int c = tid + j * 512;
            u32x4 v = {0u, 0u, 0u, 0u};
            if (c < TCH) {
                const int key = c / CPK, part = c % CPK;
                const int64_t pos = t0 + key;
                if (pos < kend) {
                    const int64_t s = slot_at(pos);
                    if (s >= 0) v = *(const u32x4*)(a.k.data + s * a.k.row_stride + part * 16);
                }
            }
            pre[j] = v;
        }
        if (tid < TK) {
            const int64_t pos = t0 + tid;
            float m = __builtin_nanf("");
            if (pos < kend) {
                const int64_t s = slot_at(pos);
                if (s >= 0) m = FP8 ? a.k.scale[s / a.k.scale_group] : 1.0f;
            }
            pre_mul = m;
        }
    };

    prefetch(c0);
    for (int64_t t0 = c0; t0 < kend; t0 += TK) {
        __syncthreads();  // previous tile fully consumed
#pragma unroll
        for (int j = 0; j < NPRE; ++j) {
            const int c = tid + j * 512;
            if (c < TCH) {
                const int key = c / CPK, part = c % CPK;
                *(u32x4*)(tile + key * RBP + part * 16) = pre[j];
            }
        }
        if (tid < TK) kmul[tid] = pre_mul;
        __syncthreads();
        if (t0 + TK < kend) prefetch(t0 + TK);

        const int64_t kb = t0 + st * 32;  // first key of this wave's subtile
        if (row_ok && kb < vis) {
            f32x16 acc[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[mt][i] = 0.f;
            const uint8_t* brow = tile + (st * 32 + (lane & 31)) * RBP + (lane >> 5) * 8 * ELT;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                if constexpr (FP8) {
                    const int64_t b = *(const int64_t*)(brow + ks * 16);
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) acc[mt] = mfma32x32x16_fp8(qa[mt][ks], b, acc[mt]);
                } else {
                    const bf16x8 b = *(const bf16x8*)(brow + ks * 32);
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) acc[mt] = mfma32x32x16_bf16(qa[mt][ks], b, acc[mt]);
                }
            }
            float part = 0.f;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int i = 0; i < 16; ++i) part = fmaf(wv[mt][i], fmaxf(acc[mt][i], 0.f), part);
            const float tot = part + __shfl_xor(part, 32);
            const int64_t key = kb + (lane & 31);
            if (lane < 32 && key < vis) scores[(int64_t)r * ld + key] = tot * kmul[st * 32 + lane];
        } else if (row_bad && kb < vis) {
            const int64_t key = kb + (lane & 31);
            if (lane < 32 && key < vis) scores[(int64_t)r * ld + key] = __builtin_nanf("");
        }
    }
}

// host-side launcher ---------------------------------------------------------

template <int DI, int MT, int QG, bool FP8>
static hipError_t launch_li(const IndexerDev& a, float* scores, int64_t ld, int64_t max_visible,
                            hipStream_t stream) {
    constexpr int TK = 32 * (8 / QG);
    const int bsz = a.k.paged ? (1 << a.k.bs_shift) : (1 << 30);
    // keys per workgroup: enough workgroups to fill 256 CUs a few times over
    const int64_t groups = (a.R + QG - 1) / QG;
    int64_t want_wg = 1024;
    int64_t nchunk = (want_wg + groups - 1) / groups;
    int64_t kpw = (max_visible + nchunk - 1) / nchunk;
    int64_t min_kpw = QG == 1 ? TK : 2048;
    if (kpw < min_kpw) kpw = min_kpw;
    kpw = (kpw + TK - 1) / TK * TK;
    if (a.k.paged) {
        int64_t cap = (int64_t)(kLiMaxBlocks - 1) * bsz / TK * TK;
        if (kpw > cap) kpw = cap;
    }
    if (kpw > (1 << 30)) kpw = (1 << 30) / TK * TK;
    nchunk = (max_visible + kpw - 1) / kpw;
    if (nchunk < 1) nchunk = 1;
    dim3 grid((unsigned)nchunk, (unsigned)groups);
    hipLaunchKernelGGL((li_score_kernel<DI, MT, QG, FP8>), grid, dim3(512), 0, stream, a, scores, ld,
                       (int)kpw);
    return hipGetLastError();
}

hipError_t li_score_dispatch(const IndexerDev& a, int D_I, int fp8, int qg, float* scores, int64_t ld,
                             int64_t max_visible, hipStream_t stream) {
    const int mt = a.H_I <= 32 ? 1 : 2;
#define LISFA_LI_CASE(DI_, MT_, QG_, F8_)                                                    \
    if (D_I == DI_ && mt == MT_ && qg == QG_ && (fp8 != 0) == F8_)                            \
        return launch_li<DI_, MT_, QG_, F8_>(a, scores, ld, max_visible, stream);
    LISFA_LI_CASE(128, 2, 1, false)
    LISFA_LI_CASE(128, 2, 8, false)
    LISFA_LI_CASE(128, 2, 1, true)
    LISFA_LI_CASE(128, 2, 8, true)
    LISFA_LI_CASE(128, 1, 1, false)
    LISFA_LI_CASE(128, 1, 8, false)
    LISFA_LI_CASE(128, 1, 1, true)
    LISFA_LI_CASE(128, 1, 8, true)
    LISFA_LI_CASE(32, 1, 1, false)
    LISFA_LI_CASE(32, 1, 8, false)
    LISFA_LI_CASE(32, 1, 1, true)
    LISFA_LI_CASE(32, 1, 8, true)
    LISFA_LI_CASE(32, 2, 1, false)
    LISFA_LI_CASE(32, 2, 8, false)
    LISFA_LI_CASE(32, 2, 1, true)
    LISFA_LI_CASE(32, 2, 8, true)
#undef LISFA_LI_CASE
    return hipErrorInvalidValue;
}

}  // namespace lisfa
