// Indexer prolog: dynamic quantisation of the indexer queries, and
// normalisation of the new keys with their store into the key cache.
//
// The pages put these steps in front of the index computation and run them on
// separate streams ("Day0 Inference Adaptation and Performance Optimization
// for Kimi K3.1 Pro", section 3; "Large Language Model Inference Acceleration
// in Practice", section 3.2; "... for a New Model", section 3.2): K
// normalisation with the cache update on one stream, Q quantisation on
// another.  The projections that produce q and k need trained weights and are
// not part of this library; these kernels start from their bf16 outputs.
//  * indexer_q_quant: one workgroup per query row, read once into registers
//    (16-byte loads; a row holds at most 64 x 128 elements).  fp8: one scale per row
//    over all heads, scale = amax / 448 (1 if amax = 0), element = x / scale
//    (IEEE division) rounded to e4m3; MXFP8: per 32-element block the shared
//    exponent floor(log2 amax) - 8 (clamped to [-127, 127], 0 for a zero
//    block), element = x * 2^-shared rounded to e4m3 (exact scaling).
//  * indexer_prolog: both in one launch, the workgroups split between the
//    query rows and the keys (the overlap of the two parts without a second
//    stream).
//  * indexer_k_store: one wavefront per new key.  Optional LayerNorm in fp32
//    (y = (x - mean) / sqrt(var + eps) * gamma + beta, biased variance), then
//    the cache's format: bf16, fp8 with a per-token scale, or MXFP8, written
//    at the key's slot (paged or contiguous).
// e4m3 rounding is round to nearest even with saturation to +-448, computed
// from the float's bits (no conversion instruction), so it is exact.
#include "common.hpp"

namespace lisfa {

// e4m3 code of v, round to nearest even, saturating at +-448 (OCP e4m3: bias
// 7, largest normal 1.75 * 2^8, subnormals multiples of 2^-9).
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
    const uint32_t sgn = (__float_as_uint(v) >> 31) << 7;
    const float a = fminf(fabsf(v), 448.f);
    uint32_t code;
    if (a < 0.015625f) {                                   // below 2^-6: subnormal grid 2^-9
        code = (uint32_t)__builtin_rintf(a * 512.f);        // 8 lands on the first normal code
    } else {
        int e = (int)((__float_as_uint(a) >> 23) & 0xFFu) - 127;              // -6 .. 8
        const float m = __uint_as_float((__float_as_uint(a) & 0x007FFFFFu) | 0x3F800000u);  // [1, 2)
        uint32_t m3 = (uint32_t)__builtin_rintf((m - 1.f) * 8.f);             // 0 .. 8
        if (m3 == 8u) {
            m3 = 0u;
            ++e;
        }
        code = ((uint32_t)(e + 7) << 3) | m3;
    }
    return code | sgn;
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t b16) { return __uint_as_float(b16 << 16); }

// shared exponent of an MX block with maximum magnitude amax
__device__ __forceinline__ int mx_shared_exp(float amax) {
    if (!(amax > 0.f)) return 0;
    int e = __builtin_amdgcn_frexp_expf(amax) - 1 - 8;    // amax = m 2^exp, m in [0.5, 1)
    return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// queries -------------------------------------------------------------------

// One workgroup per query row of n = H_I * D_I <= 8192 elements: thread t
// holds the 32-element block t (four 16-byte loads) in registers, so the row
// is read once whichever the format.
template <bool MX>
__device__ __forceinline__ void q_quant_row(const uint16_t* __restrict__ q, int n, uint8_t* __restrict__ out,
                                            void* __restrict__ scale_out, int r, float* red) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const bool on = tid < n / 32;
    float v[32];
    float amax = 0.f;
    {
        const u32x4* x = (const u32x4*)(q + (int64_t)r * n + tid * 32);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const u32x4 w = on ? x[c] : u32x4{0u, 0u, 0u, 0u};
            const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[8 * c + 2 * i] = bf16_bits_to_float(ws[i] & 0xFFFFu);
                v[8 * c + 2 * i + 1] = bf16_bits_to_float(ws[i] >> 16);
            }
        }
#pragma unroll
        for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
    }
    uint32_t w[8];
    if constexpr (MX) {
        const int se = mx_shared_exp(amax);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            w[i] = 0u;
#pragma unroll
            for (int k = 0; k < 4; ++k) w[i] |= e4m3_encode(__builtin_ldexpf(v[4 * i + k], -se)) << (8 * k);
        }
        if (on) ((uint8_t*)scale_out)[(int64_t)r * (n / 32) + tid] = (uint8_t)(se + 127);
    } else {
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
        if (lane == 0) red[wave] = amax;
        __syncthreads();
        amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
        const float sc = amax > 0.f ? amax / 448.f : 1.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            w[i] = 0u;
#pragma unroll
            for (int k = 0; k < 4; ++k) w[i] |= e4m3_encode(v[4 * i + k] / sc) << (8 * k);
        }
        if (tid == 0) ((float*)scale_out)[r] = sc;
    }
    if (on) {
        u32x4* d = (u32x4*)(out + (int64_t)r * n + tid * 32);
        d[0] = u32x4{w[0], w[1], w[2], w[3]};
        d[1] = u32x4{w[4], w[5], w[6], w[7]};
    }
}

template <bool MX>
__global__ __launch_bounds__(256) void q_quant_kernel(const uint16_t* __restrict__ q, int n, uint8_t* __restrict__ out,
                                                      void* __restrict__ scale_out) {
    __shared__ float red[4];
    q_quant_row<MX>(q, n, out, scale_out, blockIdx.x, red);
}

hipError_t q_quant_dispatch(const void* q, int R, int n, int mx, void* out, void* scale_out, hipStream_t stream) {
    if (R <= 0) return hipSuccess;
    if (n > 256 * 32 || n % 32 != 0) return hipErrorInvalidValue;
    if (mx)
        hipLaunchKernelGGL(q_quant_kernel<true>, dim3((unsigned)R), dim3(256), 0, stream, (const uint16_t*)q, n,
                           (uint8_t*)out, scale_out);
    else
        hipLaunchKernelGGL(q_quant_kernel<false>, dim3((unsigned)R), dim3(256), 0, stream, (const uint16_t*)q, n,
                           (uint8_t*)out, scale_out);
    return hipGetLastError();
}

// keys ----------------------------------------------------------------------

// One wavefront per key: lane l holds elements 2l, 2l + 1 (D_I = 128) or,
// for D_I = 32, lanes 0..15 hold them.  FMT: 0 bf16, 1 fp8 per token, 2 MXFP8.
template <int DI, int FMT>
__device__ __forceinline__ void k_store_key(const uint32_t* __restrict__ k, const float* __restrict__ gamma,
                                            const float* __restrict__ beta, float eps, int normalize,
                                            const int32_t* __restrict__ tok_seq, const int32_t* __restrict__ tok_pos,
                                            const CacheDev& c, int t) {
    static_assert(DI == 32 || DI == 128, "indexer key width");
    constexpr int ACT = DI / 2;          // active lanes
    const int lane = threadIdx.x & 63;
    // destination slot; keys the cache cannot address are skipped
    const int seq = tok_seq[t], pos = tok_pos[t];
    int64_t slot = -1;
    if (seq >= 0 && seq < c.num_seqs && pos >= 0) {
        if (c.paged) {
            const int64_t blk = (int64_t)pos >> c.bs_shift;
            if (blk < c.bt_stride) {
                const int32_t b = c.block_table[(int64_t)seq * c.bt_stride + blk];
                if (b >= 0) slot = ((int64_t)b << c.bs_shift) + (pos & ((1 << c.bs_shift) - 1));
            }
        } else {
            slot = c.seq_base[seq] + pos;
        }
    }
    if (slot < 0 || slot >= c.num_slots) return;   // uniform across the wavefront

    const bool on = lane < ACT;
    const uint32_t pair = on ? k[(int64_t)t * ACT + lane] : 0u;
    float y0 = bf16_bits_to_float(pair & 0xFFFFu), y1 = bf16_bits_to_float(pair >> 16);
    if (normalize) {
        float s = y0 + y1;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
        const float mean = s / (float)DI;
        const float d0 = on ? y0 - mean : 0.f, d1 = on ? y1 - mean : 0.f;
        float q = d0 * d0 + d1 * d1;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) q += __shfl_xor(q, off);
        const float inv = 1.f / sqrtf(q / (float)DI + eps);
        y0 = d0 * inv;
        y1 = d1 * inv;
        if (gamma) {
            y0 *= on ? gamma[2 * lane] : 1.f;
            y1 *= on ? gamma[2 * lane + 1] : 1.f;
        }
        if (beta) {
            y0 += on ? beta[2 * lane] : 0.f;
            y1 += on ? beta[2 * lane + 1] : 0.f;
        }
    }
    uint8_t* row = (uint8_t*)c.data + slot * c.row_stride;
    if constexpr (FMT == 0) {
        const __bf16 b0 = (__bf16)y0, b1 = (__bf16)y1;
        const uint32_t w = (uint32_t)__builtin_bit_cast(uint16_t, b0) | ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
        if (on) ((uint32_t*)row)[lane] = w;
    } else if constexpr (FMT == 1) {
        float amax = on ? fmaxf(fabsf(y0), fabsf(y1)) : 0.f;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
        const float s = amax > 0.f ? amax / 448.f : 1.f;
        const uint32_t w = e4m3_encode(y0 / s) | (e4m3_encode(y1 / s) << 8);
        if (on) ((uint16_t*)row)[lane] = (uint16_t)w;
        if (lane == 0) ((float*)c.scale)[slot] = s;
    } else {
        // 32-element block = 16 lanes
        float amax = on ? fmaxf(fabsf(y0), fabsf(y1)) : 0.f;
#pragma unroll
        for (int off = 8; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
        const int se = mx_shared_exp(amax);
        const uint32_t w = e4m3_encode(__builtin_ldexpf(y0, -se)) | (e4m3_encode(__builtin_ldexpf(y1, -se)) << 8);
        if (on) ((uint16_t*)row)[lane] = (uint16_t)w;
        if (on && (lane & 15) == 0) ((uint8_t*)c.mx_scale)[slot * (DI / 32) + lane / 16] = (uint8_t)(se + 127);
    }
}

template <int DI, int FMT>
__global__ __launch_bounds__(64) void k_store_kernel(const uint32_t* __restrict__ k, const float* __restrict__ gamma,
                                                     const float* __restrict__ beta, float eps, int normalize,
                                                     const int32_t* __restrict__ tok_seq,
                                                     const int32_t* __restrict__ tok_pos, CacheDev c) {
    k_store_key<DI, FMT>(k, gamma, beta, eps, normalize, tok_seq, tok_pos, c, blockIdx.x);
}

// both ----------------------------------------------------------------------

// The two parts of the prolog in one launch: workgroups 0..R-1 quantise a
// query row each, the others store four keys each (one per wavefront), so
// the two independent parts run side by side without a second launch or a
// dependency between streams.
constexpr int kKeysPerGroup = 4;

template <bool MX, int DI, int FMT>
__global__ __launch_bounds__(256) void prolog_kernel(const uint16_t* __restrict__ q, int R, int n,
                                                     uint8_t* __restrict__ q_out, void* __restrict__ q_scale_out,
                                                     const uint32_t* __restrict__ k, int T,
                                                     const float* __restrict__ gamma, const float* __restrict__ beta,
                                                     float eps, int normalize, const int32_t* __restrict__ tok_seq,
                                                     const int32_t* __restrict__ tok_pos, CacheDev c) {
    __shared__ float red[4];
    const int b = blockIdx.x;
    if (b < R) {
        q_quant_row<MX>(q, n, q_out, q_scale_out, b, red);
        return;
    }
    const int t = (b - R) * kKeysPerGroup + (threadIdx.x >> 6);
    if (t < T) k_store_key<DI, FMT>(k, gamma, beta, eps, normalize, tok_seq, tok_pos, c, t);
}

hipError_t prolog_dispatch(const void* q, int R, int n, int mx, void* q_out, void* q_scale_out, const void* k, int T,
                           int D_I, const float* gamma, const float* beta, float eps, int normalize,
                           const int32_t* tok_seq, const int32_t* tok_pos, const CacheDev& c, int dtype,
                           hipStream_t stream) {
    if (n > 256 * 32 || n % 32 != 0) return hipErrorInvalidValue;
    const int groups = R + (T + kKeysPerGroup - 1) / kKeysPerGroup;
    if (groups <= 0) return hipSuccess;
    const int fmt = dtype == LISFA_MXFP8 ? 2 : (dtype == LISFA_FP8_E4M3 ? 1 : 0);
#define LISFA_PL(MX_, DI_, F_)                                                                                  \
    if ((mx != 0) == MX_ && D_I == DI_ && fmt == F_) {                                                          \
        hipLaunchKernelGGL((prolog_kernel<MX_, DI_, F_>), dim3((unsigned)groups), dim3(256), 0, stream,        \
                           (const uint16_t*)q, R, n, (uint8_t*)q_out, q_scale_out, (const uint32_t*)k, T, gamma, \
                           beta, eps, normalize, tok_seq, tok_pos, c);                                          \
        return hipGetLastError();                                                                               \
    }
    LISFA_PL(false, 128, 0)
    LISFA_PL(false, 128, 1)
    LISFA_PL(false, 128, 2)
    LISFA_PL(false, 32, 0)
    LISFA_PL(false, 32, 1)
    LISFA_PL(false, 32, 2)
    LISFA_PL(true, 128, 0)
    LISFA_PL(true, 128, 1)
    LISFA_PL(true, 128, 2)
    LISFA_PL(true, 32, 0)
    LISFA_PL(true, 32, 1)
    LISFA_PL(true, 32, 2)
#undef LISFA_PL
    return hipErrorInvalidValue;
}

hipError_t k_store_dispatch(const void* k, int T, int D_I, const float* gamma, const float* beta, float eps,
                            int normalize, const int32_t* tok_seq, const int32_t* tok_pos, const CacheDev& c,
                            int dtype, hipStream_t stream) {
    if (T <= 0) return hipSuccess;
#define LISFA_KS(DI_, F_)                                                                                    \
    if (D_I == DI_ && fmt == F_) {                                                                           \
        hipLaunchKernelGGL((k_store_kernel<DI_, F_>), dim3((unsigned)T), dim3(64), 0, stream, (const uint32_t*)k,    \
                           gamma, beta, eps, normalize, tok_seq, tok_pos, c);                              \
        return hipGetLastError();                                                                            \
    }
    const int fmt = dtype == LISFA_MXFP8 ? 2 : (dtype == LISFA_FP8_E4M3 ? 1 : 0);
    LISFA_KS(128, 0)
    LISFA_KS(128, 1)
    LISFA_KS(128, 2)
    LISFA_KS(32, 0)
    LISFA_KS(32, 1)
    LISFA_KS(32, 2)
#undef LISFA_KS
    return hipErrorInvalidValue;
}

}  // namespace lisfa
