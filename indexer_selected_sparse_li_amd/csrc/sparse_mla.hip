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

template <int DLAT, int DROPE, bool FP8, int NHG>
__global__ __launch_bounds__(128 * NHG) void sfa_kernel(MlaDev a, int kps, int nsplit,
                                                        __bf16* __restrict__ out, float* __restrict__ lse,
                                                        float* __restrict__ part_o,
                                                        float* __restrict__ part_lse) {
    constexpr int DQK = DLAT + DROPE;
    constexpr int ELT = FP8 ? 1 : 2;
    constexpr int RB = DQK * ELT;           // bytes per cached row
    constexpr int CPK = RB / 16;            // 16-byte chunks per row
    constexpr int CPKP = CPK + 1;           // + 1 pad chunk (bank spread)
    constexpr int RBP = CPKP * 16;          // LDS row stride
    constexpr int TROWS = 32;               // rows per tile
    constexpr int TCH = TROWS * CPKP;       // chunks per tile (with pads)
    constexpr int NT = 128 * NHG;           // threads
    constexpr int NLD = (TCH + NT - 1) / NT;
    constexpr int KS = DQK / 16;            // QK K-steps
    constexpr int KS0 = (KS + 1) / 2;       // K-steps of the dh = 0 wave
    constexpr int DVH = DLAT / 2;           // value columns per wave
    constexpr int MTV = DVH / 32;           // PV M-tiles per wave
    static_assert(DQK % 16 == 0 && DVH % 32 == 0, "shape");

    __shared__ __attribute__((aligned(16))) uint8_t tile[2][TROWS * RBP];
    __shared__ int64_t slots[kSfaMaxKeys];
    __shared__ float kvs[FP8 ? kSfaMaxKeys : 1];
    __shared__ __attribute__((aligned(16))) float xbuf[NHG * 2 * 64 * 16];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hg = wave >> 1, dh = wave & 1;
    const int sp = blockIdx.x, hb = blockIdx.y, r = blockIdx.z;
    const int k0 = sp * kps;
    const int k1 = (k0 + kps < a.K) ? k0 + kps : a.K;
    const int nk = k1 - k0;
    const int seq = a.row_seq[r];

    for (int i = tid; i < nk; i += NT) {
        const int p = a.idx[(int64_t)r * a.K + k0 + i];
        const int64_t s = p >= 0 ? slot_of(a.kv, seq, p) : -1;
        slots[i] = s;
        if constexpr (FP8) kvs[i] = s >= 0 ? a.kv.scale[s / a.kv.scale_group] : 0.f;
    }

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
    __syncthreads();  // slots ready

    const int ntiles = (nk + TROWS - 1) / TROWS;
    auto issue_tile = [&](int t, int buf) {
#pragma unroll
        for (int j = 0; j < NLD; ++j) {
            const int P = j * NT + tid;          // chunk position in the tile
            if (P < TCH) {
                const int row = P / CPKP, part = P % CPKP;
                const int kk = t * TROWS + row;
                const int64_t s = kk < nk ? slots[kk] : -1;
                const uint8_t* g = (s >= 0 && part < CPK) ? a.kv.data + s * a.kv.row_stride + part * 16
                                                          : g_zero16;
                __builtin_amdgcn_global_load_lds(
                    g, (__attribute__((address_space(3))) void*)(tile[buf] + (j * NT + wave * 64) * 16), 16, 0, 0);
            }
        }
    };

    f32x16 o[MTV];
#pragma unroll
    for (int mt = 0; mt < MTV; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[mt][i] = 0.f;
    float m2 = -__builtin_inff(), lsum = 0.f;

    if (ntiles > 0) issue_tile(0, 0);
    for (int t = 0; t < ntiles; ++t) {
        const int buf = t & 1;
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (t + 1 < ntiles) issue_tile(t + 1, buf ^ 1);
        const uint8_t* T = tile[buf];

        // QK^T partial over this wave's K-steps: A = cached rows (key = lane%32)
        f32x16 s;
#pragma unroll
        for (int i = 0; i < 16; ++i) s[i] = 0.f;
        const uint8_t* arow = T + (lane & 31) * RBP;
#pragma unroll
        for (int j = 0; j < KS0; ++j) {
            if (j < nks) {
                const int ks = ksb + j;
                bf16x8 av;
                if constexpr (FP8) av = fp8x8_to_bf16x8(*(const u32x2*)(arow + ks * 16 + (lane >> 5) * 8));
                else av = *(const bf16x8*)(arow + (ks * 16 + (lane >> 5) * 8) * 2);
                s = mfma32x32x16_bf16(av, qb[j], s);
            }
        }
        // sum the two halves' partial logits through LDS
        float* xs = xbuf + ((hg * 2 + dh) * 64 + lane) * 16;
#pragma unroll
        for (int i = 0; i < 16; i += 4) *(f32x4*)(xs + i) = f32x4{s[i], s[i + 1], s[i + 2], s[i + 3]};
        __syncthreads();
        const float* xp = xbuf + ((hg * 2 + (dh ^ 1)) * 64 + lane) * 16;
#pragma unroll
        for (int i = 0; i < 16; i += 4) {
            const f32x4 v = *(const f32x4*)(xp + i);
            s[i] += v.x;
            s[i + 1] += v.y;
            s[i + 2] += v.z;
            s[i + 3] += v.w;
        }

        // logits (base 2), masking, online softmax -- in place on s
        float tmax = -__builtin_inff();
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int kk = t * TROWS + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
            const bool valid = kk < nk && slots[kk] >= 0;
            float f = a.scale_log2;
            if constexpr (FP8) f *= valid ? kvs[kk] : 0.f;
            s[i] = valid ? s[i] * f : -__builtin_inff();
            tmax = fmaxf(tmax, s[i]);
        }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        const float mnew = fmaxf(m2, tmax);
        if (mnew == -__builtin_inff()) continue;  // nothing valid yet (same in both waves)
        const float alpha = exp2f(m2 - mnew);     // m2 = -inf -> 0
        float rs = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            s[i] = exp2f(s[i] - mnew);
            rs += s[i];
        }
        rs += __shfl_xor(rs, 32);
        lsum = lsum * alpha + rs;
        m2 = mnew;
#pragma unroll
        for (int mt = 0; mt < MTV; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[mt][i] *= alpha;
        bf16x8 pb[2];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float p = s[8 * kk + e];
                if constexpr (FP8) {
                    const int key = t * TROWS + 8 * (2 * kk + (e >> 2)) + 4 * (lane >> 5) + (e & 3);
                    p = key < nk ? p * kvs[key] : 0.f;
                }
                pb[kk][e] = (__bf16)p;
            }

        // PV: A = V^T (row = value column lane%32, 8 keys of the K-step)
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
                        av[e] = *(const __bf16*)(T + key * RBP + col * 2);
                    }
                }
                o[mt] = mfma32x32x16_bf16(av, pb[kk], o[mt]);
            }
        }
    }

    // epilogue: normalise and store (O^T layout: lane = head, 4 runs of 4 columns)
    if (head < a.H) {
        const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
        const float l_nat = lsum > 0.f ? (m2 + log2f(lsum)) * kLn2 : -__builtin_inff();
        if (nsplit == 1) {
            __bf16* orow = out + ((int64_t)r * a.H + head) * DLAT;
#pragma unroll
            for (int mt = 0; mt < MTV; ++mt)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int col = dh * DVH + mt * 32 + 8 * g + 4 * (lane >> 5);
                    bf16x4 v;
#pragma unroll
                    for (int j = 0; j < 4; ++j) v[j] = (__bf16)(o[mt][4 * g + j] * inv);
                    *(bf16x4*)(orow + col) = v;
                }
            if (lse != nullptr && dh == 0 && lane < 32) lse[(int64_t)r * a.H + head] = l_nat;
        } else {
            float* prow = part_o + (((int64_t)r * nsplit + sp) * a.H + head) * DLAT;
#pragma unroll
            for (int mt = 0; mt < MTV; ++mt)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int col = dh * DVH + mt * 32 + 8 * g + 4 * (lane >> 5);
                    *(f32x4*)(prow + col) = f32x4{o[mt][4 * g] * inv, o[mt][4 * g + 1] * inv,
                                                  o[mt][4 * g + 2] * inv, o[mt][4 * g + 3] * inv};
                }
            if (dh == 0 && lane < 32) part_lse[((int64_t)r * nsplit + sp) * a.H + head] = l_nat;
        }
    }
}

// Merge split-K partials: out = sum_i e^{lse_i - M} O_i / sum_i e^{lse_i - M}.
template <int DLAT>
__global__ __launch_bounds__(128) void sfa_combine_kernel(const float* __restrict__ part_o,
                                                          const float* __restrict__ part_lse, int nsplit,
                                                          int H, __bf16* __restrict__ out,
                                                          float* __restrict__ lse) {
    const int rh = blockIdx.x;           // r * H + h
    const int r = rh / H, h = rh % H;
    float M = -__builtin_inff();
    for (int i = 0; i < nsplit; ++i) M = fmaxf(M, part_lse[((int64_t)r * nsplit + i) * H + h]);
    float W = 0.f;
    constexpr int PER = (DLAT + 127) / 128;
    float acc[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) acc[j] = 0.f;
    if (M != -__builtin_inff()) {
        for (int i = 0; i < nsplit; ++i) {
            const float li = part_lse[((int64_t)r * nsplit + i) * H + h];
            const float wi = __expf(li - M);
            W += wi;
            const float* po = part_o + (((int64_t)r * nsplit + i) * H + h) * DLAT;
#pragma unroll
            for (int j = 0; j < PER; ++j) {
                const int c = threadIdx.x + 128 * j;
                if (c < DLAT) acc[j] = fmaf(wi, po[c], acc[j]);
            }
        }
    }
    const float inv = W > 0.f ? 1.f / W : 0.f;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int c = threadIdx.x + 128 * j;
        if (c < DLAT) out[(int64_t)rh * DLAT + c] = (__bf16)(acc[j] * inv);
    }
    if (lse != nullptr && threadIdx.x == 0) lse[rh] = W > 0.f ? M + __logf(W) : -__builtin_inff();
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
    p.nhg = H <= 32 ? 1 : (H <= 64 ? 2 : 4);
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

template <int DLAT, int DROPE, bool FP8, int NHG>
static hipError_t launch_sfa_t(const MlaDev& a, const SfaPlan& p, __bf16* out, float* lse, float* part_o,
                               float* part_lse, hipStream_t stream) {
    dim3 grid((unsigned)p.nsplit, (unsigned)p.nhb, (unsigned)a.R);
    hipLaunchKernelGGL((sfa_kernel<DLAT, DROPE, FP8, NHG>), grid, dim3(128 * NHG), 0, stream, a, p.kps,
                       p.nsplit, out, lse, part_o, part_lse);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.nsplit == 1) return e;
    hipLaunchKernelGGL((sfa_combine_kernel<DLAT>), dim3((unsigned)(a.R * a.H)), dim3(128), 0, stream, part_o,
                       part_lse, p.nsplit, a.H, out, lse);
    return hipGetLastError();
}

hipError_t sfa_dispatch(const MlaDev& a, int D_latent, int fp8, __bf16* out, float* lse, void* ws,
                        hipStream_t stream) {
    const SfaPlan p = sfa_plan(a.R, a.K, a.H);
    float* part_o = (float*)ws;
    float* part_lse = part_o + (size_t)a.R * p.nsplit * a.H * D_latent;
#define LISFA_SFA_CASE(DL_, DR_, F8_, G_)                                                     \
    if (D_latent == DL_ && (fp8 != 0) == F8_ && p.nhg == G_)                                   \
        return launch_sfa_t<DL_, DR_, F8_, G_>(a, p, out, lse, part_o, part_lse, stream);
    LISFA_SFA_CASE(512, 64, false, 4)
    LISFA_SFA_CASE(512, 64, true, 4)
    LISFA_SFA_CASE(512, 64, false, 2)
    LISFA_SFA_CASE(512, 64, true, 2)
    LISFA_SFA_CASE(512, 64, false, 1)
    LISFA_SFA_CASE(512, 64, true, 1)
    LISFA_SFA_CASE(64, 16, false, 1)
    LISFA_SFA_CASE(64, 16, true, 1)
    LISFA_SFA_CASE(64, 16, false, 2)
    LISFA_SFA_CASE(64, 16, true, 2)
    LISFA_SFA_CASE(64, 16, false, 4)
    LISFA_SFA_CASE(64, 16, true, 4)
#undef LISFA_SFA_CASE
    return hipErrorInvalidValue;
}

size_t sfa_workspace_bytes(int R, int K, int H, int D_latent) {
    const SfaPlan p = sfa_plan(R, K, H);
    if (p.nsplit <= 1) return 0;
    return (size_t)R * p.nsplit * H * ((size_t)D_latent + 1) * sizeof(float);
}

}  // namespace lisfa
