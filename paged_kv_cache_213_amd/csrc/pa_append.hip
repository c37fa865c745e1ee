// pa_append.hip -- write this step's new K/V rows into their physical slots.
//
// Slot s addresses block s / 16, offset s % 16: the block table's
// logical-to-physical mapping ("03 -- Engines Papers", section 2). K rows
// are contiguous in the cache ([block][head][16][D]); V is stored
// [block][head][D][16], so one token's V row lands as D values 16 apart.
// An FP8 cache gets e4m3fn(fp32(x) / scale[block][head]) ("The LLM inference
// engine playbook", Themes 3 and 6: FP8 E4M3 KV with a scale).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

using dev::encode_e4m3fn;


__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float((uint32_t)b << 16);
}

// One thread per (token, head, element).
template <int newd, int kvd>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
    const int64_t D = a.head_dim, H = a.num_kv_heads;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (int64_t)a.num_tokens * H * D) return;
    const int64_t d = idx % D;
    const int64_t g = (idx / D) % H;
    const int64_t t = idx / (D * H);
    const int32_t s = a.slot_mapping[t];
    if (s < 0 || s / 16 >= a.num_blocks) return;  // skipped, or outside the pool
    const int64_t b = s / 16, o = s % 16;
    const int64_t kdst = ((b * H + g) * 16 + o) * D + d;
    const int64_t vdst = ((b * H + g) * D + d) * 16 + o;
    if constexpr (kvd == newd && kvd == PA_F32) {
        ((float*)a.k_cache)[kdst] = ((const float*)a.k_new)[idx];
        ((float*)a.v_cache)[vdst] = ((const float*)a.v_new)[idx];
    } else if constexpr (kvd == newd && kvd == PA_BF16) {
        ((uint16_t*)a.k_cache)[kdst] = ((const uint16_t*)a.k_new)[idx];
        ((uint16_t*)a.v_cache)[vdst] = ((const uint16_t*)a.v_new)[idx];
    } else {
        static_assert(kvd == PA_FP8_E4M3FN, "unsupported combination");
        static_assert(newd == PA_BF16, "fp8 caches take bf16 rows");
        const float kx = bf16_to_f32(((const uint16_t*)a.k_new)[idx]);
        const float vx = bf16_to_f32(((const uint16_t*)a.v_new)[idx]);
        const float ks = a.k_scale[b * H + g], vs = a.v_scale[b * H + g];
        ((uint8_t*)a.k_cache)[kdst] = (uint8_t)encode_e4m3fn(__fdiv_rn(kx, ks));
        ((uint8_t*)a.v_cache)[vdst] = (uint8_t)encode_e4m3fn(__fdiv_rn(vx, vs));
    }
}

// Copy-on-write copies: one workgroup per (source, destination) pair moves
// the whole block, K and V of every KV head (16-byte words), and its scales.
__global__ __launch_bounds__(256) void copy_blocks_kernel(CopyArgs a) {
    const int32_t src = a.pairs[2 * blockIdx.x], dst = a.pairs[2 * blockIdx.x + 1];
    if (src < 0 || src >= a.num_blocks || dst < 0 || dst >= a.num_blocks) return;
    const int64_t words = a.block_bytes / 16;  // per cache
    const uint4* ks = (const uint4*)a.k_cache + src * words;
    const uint4* vs = (const uint4*)a.v_cache + src * words;
    uint4* kd = (uint4*)a.k_cache + dst * words;
    uint4* vd = (uint4*)a.v_cache + dst * words;
    for (int64_t i = threadIdx.x; i < words; i += blockDim.x) {
        kd[i] = ks[i];
        vd[i] = vs[i];
    }
    if (a.k_scale && (int)threadIdx.x < a.num_kv_heads) {
        a.k_scale[(int64_t)dst * a.num_kv_heads + threadIdx.x] =
            a.k_scale[(int64_t)src * a.num_kv_heads + threadIdx.x];
        a.v_scale[(int64_t)dst * a.num_kv_heads + threadIdx.x] =
            a.v_scale[(int64_t)src * a.num_kv_heads + threadIdx.x];
    }
}

}  // namespace

hipError_t launch_copy_blocks(const CopyArgs& a, int num_pairs, hipStream_t s) {
    if (num_pairs <= 0) return hipSuccess;
    hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)num_pairs), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_append(int new_dtype, int kv_dtype, const AppendArgs& a, hipStream_t s) {
    const int64_t total = (int64_t)a.num_tokens * a.num_kv_heads * a.head_dim;
    if (total == 0) return hipSuccess;
    const dim3 grid((unsigned)((total + 255) / 256)), block(256);
    if (new_dtype == PA_F32 && kv_dtype == PA_F32)
        hipLaunchKernelGGL((append_kernel<PA_F32, PA_F32>), grid, block, 0, s, a);
    else if (new_dtype == PA_BF16 && kv_dtype == PA_BF16)
        hipLaunchKernelGGL((append_kernel<PA_BF16, PA_BF16>), grid, block, 0, s, a);
    else if (new_dtype == PA_BF16 && kv_dtype == PA_FP8_E4M3FN)
        hipLaunchKernelGGL((append_kernel<PA_BF16, PA_FP8_E4M3FN>), grid, block, 0, s, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace pa
