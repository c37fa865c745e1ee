// pa_device.h -- device helpers shared by the gfx950 attention kernels:
// vector types, the hardware exp2, reductions over the four lanes that hold
// one query row in the 16x16 matrix-core layouts, bf16 packing, the e4m3
// to bf16 conversion, the fp32 to e4m3 encoding of the append and
// cache-line loads with or without the nontemporal hint. Not part of the
// public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_internal.h"

namespace pa {
namespace dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;

enum KvKind { KV_F32 = PA_F32, KV_BF16 = PA_BF16, KV_FP8 = PA_FP8_E4M3FN, KV_FP8Q = KIND_FP8_QK };

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

// fp32 -> OCP e4m3fn by bit manipulation: round to nearest, ties to even;
// magnitudes at or above 448 saturate to 448 (0x7E); NaN -> 0x7F.
__device__ __forceinline__ uint32_t encode_e4m3fn(float x) {
    const uint32_t u = __float_as_uint(x);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7fffffffu;
    if (a > 0x7f800000u) return 0x7fu;            // NaN
    if (a >= 0x43e00000u) return sign | 0x7eu;    // >= 448 (and inf)
    if (a >= 0x3c800000u) {                       // >= 2^-6: normal in e4m3
        // keep 3 of 23 mantissa bits, rounding the dropped 20 to even
        uint32_t r = (a + 0x7ffffu + ((a >> 20) & 1u)) >> 20;
        return sign | (r - (120u << 3));          // rebias exponent 127 -> 7
    }
    // subnormal grid: multiples of 2^-9; the result 8 is 2^-6, code 0x08
    const float q = __uint_as_float(a) * 512.0f;
    return sign | (uint32_t)__builtin_rintf(q);
}

// Reductions over the four lanes n, n + 16, n + 32, n + 48 that hold one
// query row, with the gfx950 row swaps: permlane16_swap exchanges 16-lane
// rows 1 <-> 0 and 3 <-> 2 between its two operands, permlane32_swap rows
// 2, 3 <-> 0, 1; given the same value twice, the two results hold a lane's
// own value and its partner's, in some order, so any symmetric op of them
// reduces over the pair.
__device__ __forceinline__ float pair16_max(float v) {
    const auto w = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                    false);
    return fmaxf(__uint_as_float(w[0]), __uint_as_float(w[1]));
}
__device__ __forceinline__ float pair32_max(float v) {
    const auto w = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                    false);
    return fmaxf(__uint_as_float(w[0]), __uint_as_float(w[1]));
}
__device__ __forceinline__ float row_max(float v) { return pair32_max(pair16_max(v)); }
__device__ __forceinline__ float row_sum(float v) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                    false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                    false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Two floats -> two bf16 (round to nearest even) packed low, high: one
// v_cvt_pk_bf16_f32.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2_t f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// Two e4m3fn bytes (the low or the high half of a dword, b0 low) -> two
// bf16 packed in a dword, with one gfx950 conversion (scale 1). Every e4m3
// value is exact in bf16, so the conversion rounds nothing.
template <bool hi>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t word) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(word, 1.0f, hi));
}

// K/V loads. A block that one wave reads once per call (a decode's context)
// is streamed with nontemporal loads, so it does not evict the block tables,
// queries and partials from the caches; blocks that several query tiles read
// (a chunked-prefill span's context) use ordinary loads, so the tiles after
// the first find them in L2.
#ifndef PA_NT_LOADS
#define PA_NT_LOADS 1
#endif
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

template <bool nt>
__device__ __forceinline__ uint4 ld_kv(const uint4* p) {
    if constexpr (nt) {
        const u32x4_t v = __builtin_nontemporal_load((const u32x4_t*)p);
        return make_uint4(v.x, v.y, v.z, v.w);
    } else {
        return *p;
    }
}
template <bool nt>
__device__ __forceinline__ uint2 ld_kv(const uint2* p) {
    if constexpr (nt) {
        const u32x2_t v = __builtin_nontemporal_load((const u32x2_t*)p);
        return make_uint2(v.x, v.y);
    } else {
        return *p;
    }
}
template <bool nt>
__device__ __forceinline__ uint32_t ld_kv(const uint32_t* p) {
    if constexpr (nt) {
        return __builtin_nontemporal_load(p);
    } else {
        return *p;
    }
}
template <bool nt>
__device__ __forceinline__ float4 ld_kv(const float4* p) {
    const uint4 v = ld_kv<nt>((const uint4*)p);
    return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z),
                       __uint_as_float(v.w));
}

// An empty use of a register: the wait for the load that wrote it is
// placed here, in straight-line code where the count of loads issued after
// it is known, rather than at a later use (a loop's head, or the join of
// paths of which only some read it), where the compiler, unable to count,
// waits for every load in flight.
__device__ __forceinline__ void take_reg(float x) { asm volatile("" ::"v"(x)); }

}  // namespace dev
}  // namespace pa
