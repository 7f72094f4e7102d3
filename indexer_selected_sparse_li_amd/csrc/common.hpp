// Device-side helpers shared by the lisfa kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "lisfa.h"

namespace lisfa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// LDS-qualified element types (keep LDS addressing 32-bit so constant offsets
// fold into the DS instruction's offset field)
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) uint32_t lds_u32;
typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) __bf16 lds_bf16;

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Kernel-side view of a cache (passed by value).
struct CacheDev {
    const uint8_t* data;
    int64_t num_slots;
    const float* scale;          // fp8: fp32 factor per scale group
    const uint8_t* mx_scale;     // mxfp8: E8M0 byte per 32 elements, [num_slots, width / 32]
    const int32_t* block_table;
    const int64_t* seq_base;
    int32_t row_stride;      // bytes
    int32_t scale_group;     // fp8 scale group (slots)
    int32_t bs_shift;        // log2(block_size) (paged)
    int32_t bt_stride;
    int32_t num_seqs;
    int32_t paged;
};

struct IndexerDev {
    const uint8_t* q;
    const float* q_scale;        // fp8: [R] or [R, H_I]
    const uint8_t* q_mx_scale;   // mxfp8: E8M0 [R, H_I, D_I / 32]
    const float* w;
    const int32_t* row_seq;
    const int32_t* row_pos;
    CacheDev k;
    int32_t q_scale_per_head;
    int32_t R;
    int32_t H_I;
};

struct MlaDev {
    const uint8_t* q;        // bf16 [R, H, DQK]
    const int32_t* row_seq;
    const int32_t* idx;      // [R, K]
    CacheDev kv;
    int32_t R, H, K;
    float scale_log2;        // softmax_scale * log2(e)
    int32_t gather_nt;       // latent rows gathered with non-temporal loads (no row shared by two query rows)
};

// Physical slot of (sequence, logical position), or -1 when the position is
// outside what the block table / pool can address.
__device__ __forceinline__ int64_t slot_of(const CacheDev& c, int seq, int64_t pos) {
    if (seq < 0 || seq >= c.num_seqs || pos < 0) return -1;
    int64_t s;
    if (c.paged) {
        int64_t blk = pos >> c.bs_shift;
        if (blk >= c.bt_stride) return -1;
        int32_t b = c.block_table[(int64_t)seq * c.bt_stride + blk];
        if (b < 0) return -1;
        s = ((int64_t)b << c.bs_shift) + (pos & ((1 << c.bs_shift) - 1));
    } else {
        s = c.seq_base[seq] + pos;
    }
    return (s >= 0 && s < c.num_slots) ? s : -1;
}

// Exact e4m3 (OCP) pair -> fp32 pair via the hardware converter.
template <bool HI>
__device__ __forceinline__ f32x2 fp8x2_to_f32(uint32_t word) {
    return __builtin_amdgcn_cvt_pk_f32_fp8((int)word, HI);
}

// fp32 whose low 16 bits are zero -> bf16 bits (exact truncation).
__device__ __forceinline__ uint32_t pack_hi16(float lo, float hi) {
    return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);
}

// 8 e4m3 codes (two dwords) -> 8 bf16 (exact: every e4m3 value is a bf16 value).
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(u32x2 v) {
    f32x2 a = fp8x2_to_f32<false>(v.x), b = fp8x2_to_f32<true>(v.x);
    f32x2 c = fp8x2_to_f32<false>(v.y), d = fp8x2_to_f32<true>(v.y);
    u32x4 r;
    r.x = pack_hi16(a.x, a.y);
    r.y = pack_hi16(b.x, b.y);
    r.z = pack_hi16(c.x, c.y);
    r.w = pack_hi16(d.x, d.y);
    return __builtin_bit_cast(bf16x8, r);
}

__device__ __forceinline__ f32x16 mfma32x32x16_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma32x32x16_fp8(int64_t a, int64_t b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(a, b, c, 0, 0, 0);
}

// Order-preserving map fp32 -> uint32 with -0.0 and +0.0 on one key: sign
// clear: b + 2^31; sign set: 2^31 - |b| (b's two's complement), so no float
// maps to 0, which marks an invalid entry below every key.  NaN (sign clear)
// orders above +inf.  Both Top-K paths select on these keys.
__device__ __forceinline__ uint32_t float_key(float f) {
    const uint32_t b = __float_as_uint(f);
    const uint32_t s = (uint32_t)((int32_t)b >> 31);
    return (b ^ (s | 0x80000000u)) - s;
}

// Wave-wide inclusive scans through DPP (row shifts by 1, 2, 4, 8 within
// each row of 16 lanes, then row 0/2's last lane to rows 1/3 and lane 31 to
// rows 2 and 3); lanes without a source keep the identity.  Lane 63 ends
// with the wave's total.
template <int CTRL, int ROWM>
__device__ __forceinline__ uint32_t dpp(uint32_t old, uint32_t x) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)x, CTRL, ROWM, 0xF, false);
}
__device__ __forceinline__ uint32_t wave_incl_sum(uint32_t x) {
    x += dpp<0x111, 0xF>(0u, x);
    x += dpp<0x112, 0xF>(0u, x);
    x += dpp<0x114, 0xF>(0u, x);
    x += dpp<0x118, 0xF>(0u, x);
    x += dpp<0x142, 0xA>(0u, x);
    x += dpp<0x143, 0xC>(0u, x);
    return x;
}
__device__ __forceinline__ uint32_t wave_incl_min(uint32_t x) {
    x = min(x, dpp<0x111, 0xF>(~0u, x));
    x = min(x, dpp<0x112, 0xF>(~0u, x));
    x = min(x, dpp<0x114, 0xF>(~0u, x));
    x = min(x, dpp<0x118, 0xF>(~0u, x));
    x = min(x, dpp<0x142, 0xA>(~0u, x));
    x = min(x, dpp<0x143, 0xC>(~0u, x));
    return x;
}
__device__ __forceinline__ uint32_t wave_incl_max(uint32_t x) {
    x = max(x, dpp<0x111, 0xF>(0u, x));
    x = max(x, dpp<0x112, 0xF>(0u, x));
    x = max(x, dpp<0x114, 0xF>(0u, x));
    x = max(x, dpp<0x118, 0xF>(0u, x));
    x = max(x, dpp<0x142, 0xA>(0u, x));
    x = max(x, dpp<0x143, 0xC>(0u, x));
    return x;
}

__device__ __forceinline__ uint32_t lanemask_count(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

// Direct-to-LDS load of SIZE (4 or 16) bytes per lane: global gp + OFF lands at
// LDS byte lds + OFF + SIZE * lane, with lds wave-uniform.  It is issued from
// inline assembly, so the compiler's wait-count model does not see it and does
// not make the wave's own LDS reads wait for it; the caller orders it with
// explicit vmcnt waits and a barrier before the destination is read, and only
// reuses a destination that every wave has finished reading.  m0 (the LDS base
// register of the instruction) is saved and restored around the load.  NT sets
// the non-temporal bit: scattered row gathers from HBM measured 5.3 TB/s with it
// against 2.8 TB/s without (data already in the MALL: 5.7 against 6.1 TB/s).
template <int SIZE, int OFF, bool NT = false>
__device__ __forceinline__ void lds_dma(const void* gp, uint32_t lds) {
    static_assert(SIZE == 4 || SIZE == 16, "dword or dwordx4");
    static_assert(OFF >= 0 && OFF < 4096, "13-bit signed immediate, kept non-negative");
    static_assert(!NT || SIZE == 16, "non-temporal form for dwordx4 only");
    const uint32_t base = __builtin_amdgcn_readfirstlane(lds);
    uint32_t m0s;
    if constexpr (SIZE == 16 && NT)
        asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\t"
                     "global_load_lds_dwordx4 %1, off offset:%3 nt\n\ts_mov_b32 m0, %0"
                     : "=&s"(m0s) : "v"(gp), "s"(base), "n"(OFF) : "memory");
    else if constexpr (SIZE == 16)
        asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\t"
                     "global_load_lds_dwordx4 %1, off offset:%3\n\ts_mov_b32 m0, %0"
                     : "=&s"(m0s) : "v"(gp), "s"(base), "n"(OFF) : "memory");
    else
        asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\t"
                     "global_load_lds_dword %1, off offset:%3\n\ts_mov_b32 m0, %0"
                     : "=&s"(m0s) : "v"(gp), "s"(base), "n"(OFF) : "memory");
}

}  // namespace lisfa
