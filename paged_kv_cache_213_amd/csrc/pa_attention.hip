// pa_attention.hip -- paged attention kernels for gfx950 (MI355X).
//
// Three kernels run in order on the caller's stream:
//
//   plan       one workgroup turns (query spans, context lengths) into a list
//              of work items -- (sequence, query tile, key partition) -- in
//              device memory, so the host never reads lengths back. This is
//              the per-step "plan" of the request trace on "03 -- Engines
//              Papers" (whiteboard test), done on the device.
//   attention  a persistent grid; each workgroup takes (item, KV head) units
//              from an atomic counter. Its four waves split the partition's
//              16-token blocks, gather them through the block table
//              ("03 -- Engines Papers", section 2), and keep an online
//              softmax (running max and sum, Milakov & Gimelshein on the
//              "References" page) in registers; the waves' states are then
//              combined through LDS. A unit covering a whole context writes
//              the output; otherwise it writes a partial (lse, o) per row.
//   merge      combines the partials of split rows by log-sum-exp (split-K
//              decode, playbook Theme 4; LSE merge, first page section 12).
//
// Matrix cores: with K stored [block][head][16 tokens][D] and V stored
// [block][head][D][16 tokens], both contractions read K-contiguous operands
// straight from HBM:
//   S[t][n]  = sum_d K[t][d] q[n][d]       A = K tile, B = q rows
//   O[d][n] += sum_t V^T[d][t] P[t][n]     A = V^T tile, B = P
// The 16x16 MFMA result layout puts S[4g+r][n] in lane (n + 16g), register r,
// which is exactly the B-operand layout the P.V product needs: no shuffles
// between the two products. Query rows n (up to 16: G heads x tile tokens)
// share every K/V byte a wave loads, so GQA reads the cache once.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "pa_internal.h"

namespace pa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;

enum KvKind { KV_F32 = PA_F32, KV_BF16 = PA_BF16, KV_FP8 = PA_FP8_E4M3FN };

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float wave_max_xor_16_32(float v) {
    v = fmaxf(v, __shfl_xor(v, 16));
    v = fmaxf(v, __shfl_xor(v, 32));
    return v;
}

__device__ __forceinline__ float wave_sum_xor_16_32(float v) {
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    return v;
}

// Round-to-nearest-even float -> bf16 bits.
__device__ __forceinline__ uint32_t bf16_bits_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;  // NaN stays NaN
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Two e4m3fn bytes (b0 low) -> two bf16 packed in a dword. Every e4m3 value
// is exact in fp32 and in bf16, so the fp32 -> bf16 step drops zero bits.
template <bool hi>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t word) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    f32x2 f = __builtin_amdgcn_cvt_pk_f32_fp8(word, hi);
    return (__float_as_uint(f.x) >> 16) | (__float_as_uint(f.y) & 0xffff0000u);
}

// ---- per-dtype register images of one 16-token block ---------------------

template <int kv, int D>
struct Tile;

// fp32: QK with 16x16x4 f32 MFMA (D/4 steps), PV with 4 steps per 16 dims.
template <int D>
struct Tile<KV_F32, D> {
    float4 k[D / 16];  // K[t][(D/4)g + j], j < D/4
    float4 v[D / 16];  // V^T[16dt + d][4g .. 4g+3]
    using QReg = float[D / 4];

    __device__ __forceinline__ void load(const void* kc, const void* vc, int64_t blk_head,
                                         int lane) {
        const int t = lane & 15, g = lane >> 4;
        const float4* kp =
            (const float4*)((const float*)kc + blk_head * 16 * D + t * D + (D / 4) * g);
#pragma unroll
        for (int j = 0; j < D / 16; ++j) k[j] = kp[j];
        const float* vb = (const float*)vc + blk_head * 16 * D;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt)
            v[dt] = *(const float4*)(vb + (16 * dt + t) * 16 + 4 * g);
    }
    __device__ __forceinline__ f32x4 qk(const float* q) const {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < D / 16; ++j) {
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(k[j].x, q[4 * j + 0], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(k[j].y, q[4 * j + 1], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(k[j].z, q[4 * j + 2], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(k[j].w, q[4 * j + 3], acc, 0, 0, 0);
        }
        return acc;
    }
    __device__ __forceinline__ void mask_v(int nvalid) {
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
            v[dt].x = nvalid > 0 ? v[dt].x : 0.f;
            v[dt].y = nvalid > 1 ? v[dt].y : 0.f;
            v[dt].z = nvalid > 2 ? v[dt].z : 0.f;
            v[dt].w = nvalid > 3 ? v[dt].w : 0.f;
        }
    }
    __device__ __forceinline__ void pv(const float p[4], f32x4* o) const {
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
            o[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(v[dt].x, p[0], o[dt], 0, 0, 0);
            o[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(v[dt].y, p[1], o[dt], 0, 0, 0);
            o[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(v[dt].z, p[2], o[dt], 0, 0, 0);
            o[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(v[dt].w, p[3], o[dt], 0, 0, 0);
        }
    }
};

// bf16 (and fp8 after conversion): QK with 16x16x32 bf16 MFMA, PV with
// 16x16x16 bf16 MFMA (one per 16 output dims).
template <int D>
struct Tile<KV_BF16, D> {
    uint4 k[D / 32];  // 8 bf16 each: K[t][(D/4)g + 8j .. +8]
    uint2 v[D / 16];  // 4 bf16 each: V^T[16dt + d][4g .. 4g+3]

    __device__ __forceinline__ void load(const void* kc, const void* vc, int64_t blk_head,
                                         int lane) {
        const int t = lane & 15, g = lane >> 4;
        const uint4* kp = (const uint4*)((const uint16_t*)kc + blk_head * 16 * D + t * D +
                                         (D / 4) * g);
#pragma unroll
        for (int j = 0; j < D / 32; ++j) k[j] = kp[j];
        const uint16_t* vb = (const uint16_t*)vc + blk_head * 16 * D;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt)
            v[dt] = *(const uint2*)(vb + (16 * dt + t) * 16 + 4 * g);
    }
    __device__ __forceinline__ f32x4 qk(const uint4* q) const {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < D / 32; ++j)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k[j]),
                                                          __builtin_bit_cast(bf16x8, q[j]), acc,
                                                          0, 0, 0);
        return acc;
    }
    __device__ __forceinline__ void mask_v(int nvalid) {
        const uint32_t mx = nvalid >= 2 ? 0xffffffffu : (nvalid == 1 ? 0x0000ffffu : 0u);
        const uint32_t my = nvalid >= 4 ? 0xffffffffu : (nvalid == 3 ? 0x0000ffffu : 0u);
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
            v[dt].x &= mx;
            v[dt].y &= my;
        }
    }
    __device__ __forceinline__ void pv(s16x4 p, f32x4* o) const {
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt)
            o[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, v[dt]), p,
                                                              o[dt], 0, 0, 0);
    }
};

template <int D>
struct Tile<KV_FP8, D> {
    uint4 k[D / 64];     // 16 e4m3 bytes each: K[t][(D/4)g + 16j .. +16]
    uint32_t v[D / 16];  // 4 e4m3 bytes each: V^T[16dt + d][4g .. 4g+3]

    __device__ __forceinline__ void load(const void* kc, const void* vc, int64_t blk_head,
                                         int lane) {
        const int t = lane & 15, g = lane >> 4;
        const uint4* kp =
            (const uint4*)((const uint8_t*)kc + blk_head * 16 * D + t * D + (D / 4) * g);
#pragma unroll
        for (int j = 0; j < D / 64; ++j) k[j] = kp[j];
        const uint8_t* vb = (const uint8_t*)vc + blk_head * 16 * D;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt)
            v[dt] = *(const uint32_t*)(vb + (16 * dt + t) * 16 + 4 * g);
    }
    __device__ __forceinline__ f32x4 qk(const uint4* q) const {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < D / 64; ++j) {
            const uint32_t w[4] = {k[j].x, k[j].y, k[j].z, k[j].w};
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                uint4 kb;
                kb.x = fp8x2_to_bf16x2<false>(w[2 * h]);
                kb.y = fp8x2_to_bf16x2<true>(w[2 * h]);
                kb.z = fp8x2_to_bf16x2<false>(w[2 * h + 1]);
                kb.w = fp8x2_to_bf16x2<true>(w[2 * h + 1]);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8, kb), __builtin_bit_cast(bf16x8, q[2 * j + h]), acc,
                    0, 0, 0);
            }
        }
        return acc;
    }
    __device__ __forceinline__ void mask_v(int nvalid) {
        const uint32_t m =
            nvalid >= 4 ? 0xffffffffu : (nvalid <= 0 ? 0u : ((1u << (8 * nvalid)) - 1u));
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) v[dt] &= m;
    }
    __device__ __forceinline__ void pv(s16x4 p, f32x4* o) const {
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
            uint2 vb;
            vb.x = fp8x2_to_bf16x2<false>(v[dt]);
            vb.y = fp8x2_to_bf16x2<true>(v[dt]);
            o[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, vb), p,
                                                              o[dt], 0, 0, 0);
        }
    }
};

// ---- plan ------------------------------------------------------------------

constexpr int kPlanThreads = 1024;

__device__ __forceinline__ int tile_parts(int L, int n, int k0, int ntok, int P) {
    const int maxpos = L - n + k0 + ntok - 1;  // last query position of the tile
    const int parts = (maxpos + 1 + P - 1) / P;
    return parts > 1 ? parts : 1;
}

// Block-wide exclusive scan of one int per thread (1024 threads).
__device__ int block_exclusive_scan(int v, int* total) {
    __shared__ int s_wave[kPlanThreads / 64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        int y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    if (lane == 63) s_wave[wave] = x;
    __syncthreads();
    if (wave == 0) {
        int w = lane < kPlanThreads / 64 ? s_wave[lane] : 0;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            int y = __shfl_up(w, off);
            if (lane >= off) w += y;
        }
        if (lane < kPlanThreads / 64) s_wave[lane] = w;
    }
    __syncthreads();
    const int before = (wave > 0 ? s_wave[wave - 1] : 0) + x - v;
    *total = s_wave[kPlanThreads / 64 - 1];
    __syncthreads();
    return before;
}

// Items of multi-token spans (heavier, chunked prefill) come first, then
// decodes; within a class sequences keep their order.
__global__ __launch_bounds__(kPlanThreads) void plan_kernel(PlanArgs a) {
    int base = 0;
    for (int phase = 0; phase < 2; ++phase) {
        for (int c0 = 0; c0 < a.num_seqs; c0 += kPlanThreads) {
            const int i = c0 + (int)threadIdx.x;
            int n = 0, L = 0, qs = 0, cnt = 0;
            bool mine = false;
            if (i < a.num_seqs) {
                qs = a.qsl ? a.qsl[i] : i;
                n = a.qsl ? a.qsl[i + 1] - qs : 1;
                L = min(a.context_lens[i], a.max_context_len);
                if (qs < 0 || n < 0 || qs + n > a.num_tokens) n = 0;  // malformed span
                mine = n > 0 && ((n > 1) == (phase == 0));
                if (mine)
                    for (int k0 = 0; k0 < n; k0 += a.tile_tokens) {
                        const int nt = min(a.tile_tokens, n - k0);
                        cnt += tile_parts(L, n, k0, nt, a.part_size);
                    }
            }
            int total;
            int off = base + block_exclusive_scan(cnt, &total);
            if (mine) {
                for (int k0 = 0; k0 < n; k0 += a.tile_tokens) {
                    const int nt = min(a.tile_tokens, n - k0);
                    const int np = tile_parts(L, n, k0, nt, a.part_size);
                    for (int p = 0; p < np; ++p, ++off)
                        if (off < a.max_items) a.items[off] = WorkItem{i, k0, p, nt};
                    for (int j = 0; j < nt; ++j) a.tok_np[qs + k0 + j] = np;
                }
            }
            base += total;
        }
    }
    if (threadIdx.x == 0) {
        a.hdr[HDR_NITEMS] = (int)min((int64_t)base, a.max_items);
        a.hdr[HDR_COUNTER] = 0;
    }
}

// ---- attention ---------------------------------------------------------------

constexpr int kWaves = 4;

template <int kv, int D>
__global__ __launch_bounds__(64 * kWaves) void attention_kernel(AttnArgs a) {
    using T = Tile<kv, D>;
    constexpr int NW = kWaves;
    constexpr int TPR = 4 * NW;      // merge threads per row
    constexpr int DPT = D / TPR;     // merge dims per thread
    constexpr int LDSW = D + 4;      // padded LDS row

    __shared__ int s_unit;
    __shared__ float s_m[NW][16];
    __shared__ float s_l[NW][16];
    __shared__ __attribute__((aligned(16))) float s_o[NW][16][LDSW];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15;  // query row owned in MFMA layouts
    const int g = lane >> 4;  // lane group
    const int Hkv = a.num_kv_heads, G = a.group, Hq = a.num_q_heads;
    const int total = a.hdr[HDR_NITEMS] * Hkv;

    for (;;) {
        if (threadIdx.x == 0) s_unit = atomicAdd(&a.hdr[HDR_COUNTER], 1);
        __syncthreads();
        const int u = __builtin_amdgcn_readfirstlane(s_unit);
        if (u >= total) break;
        const int item_idx = u / Hkv;
        const int kvh = u - item_idx * Hkv;
        const WorkItem it = a.items[item_idx];
        const int seq = it.seq;
        const int L = min(a.context_lens[seq], a.max_context_len);
        const int qs = a.qsl ? a.qsl[seq] : seq;
        const int nspan = a.qsl ? a.qsl[seq + 1] - qs : 1;
        const int nrows = it.ntok * G;
        const int tile_maxpos = L - nspan + it.qtok0 + it.ntok - 1;
        const int kbeg = it.part * a.part_size;
        const int kend = min(kbeg + a.part_size, tile_maxpos + 1);
        const int nblk = kend > kbeg ? (kend - kbeg + 15) >> 4 : 0;
        const int nparts = max(1, (tile_maxpos + 1 + a.part_size - 1) / a.part_size);

        // this lane's query row: token j = n / G, head kvh*G + n % G
        const int qj = n / G;
        const int qrow = qs + it.qtok0 + qj;
        const int qhead = kvh * G + (n - qj * G);
        const bool row_ok = n < nrows;
        const int pos = row_ok ? L - nspan + it.qtok0 + qj : -1;

        // q operand (B of S = K q^T): dims (D/4)g + j of row n
        typename std::conditional<kv == KV_F32, float[D / 4], uint4[D / 32]>::type qreg;
        if constexpr (kv == KV_F32) {
            const float* qp = (const float*)a.q + ((int64_t)qrow * Hq + qhead) * D + (D / 4) * g;
#pragma unroll
            for (int j = 0; j < D / 16; ++j) {
                float4 x = row_ok ? ((const float4*)qp)[j] : make_float4(0.f, 0.f, 0.f, 0.f);
                qreg[4 * j] = x.x;
                qreg[4 * j + 1] = x.y;
                qreg[4 * j + 2] = x.z;
                qreg[4 * j + 3] = x.w;
            }
        } else {
            const uint4* qp = (const uint4*)((const uint16_t*)a.q +
                                             ((int64_t)qrow * Hq + qhead) * D + (D / 4) * g);
#pragma unroll
            for (int j = 0; j < D / 32; ++j) qreg[j] = row_ok ? qp[j] : make_uint4(0, 0, 0, 0);
        }

        f32x4 o[D / 16];
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        float m_run = -INFINITY, l_run = 0.f;

        const int32_t* bt_row = a.block_tables + (int64_t)seq * a.max_blocks_per_seq;
        const int kb0 = kbeg >> 4;
        const int nbw = nblk > wave ? (nblk - wave + NW - 1) / NW : 0;  // my blocks

        for (int c0 = 0; c0 < nbw; c0 += 64) {
            const int cnt = min(64, nbw - c0);
            // block ids (and fp8 scales) of up to 64 of my blocks, one per lane
            int my_phys = 0;
            float my_ks = 1.f, my_vs = 1.f;
            if (lane < cnt) {
                // ids outside the pool are clamped into it: wrong tables give
                // undefined results, never an out-of-bounds access
                my_phys = min(max(bt_row[kb0 + wave + NW * (c0 + lane)], 0), a.num_blocks - 1);
                if constexpr (kv == KV_FP8) {
                    my_ks = a.k_scale[(int64_t)my_phys * Hkv + kvh];
                    my_vs = a.v_scale[(int64_t)my_phys * Hkv + kvh];
                }
            }
            T cur, nxt;
            {
                const int ph = __builtin_amdgcn_readlane(my_phys, 0);
                cur.load(a.k_cache, a.v_cache, (int64_t)ph * Hkv + kvh, lane);
            }
            for (int j = 0; j < cnt; ++j) {
                if (j + 1 < cnt) {
                    const int ph = __builtin_amdgcn_readlane(my_phys, j + 1);
                    nxt.load(a.k_cache, a.v_cache, (int64_t)ph * Hkv + kvh, lane);
                }
                const int jb = kb0 + wave + NW * (c0 + j);  // logical block
                const int t0 = jb * 16 + 4 * g;             // my first token in it
                float c = a.scale_log2;
                float vsc = 1.f;
                if constexpr (kv == KV_FP8) {
                    c *= __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                                       __builtin_bit_cast(int, my_ks), j));
                    vsc = __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                                        __builtin_bit_cast(int, my_vs), j));
                }
                f32x4 s = cur.qk(qreg);
                float sv[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) sv[r] = (t0 + r <= pos) ? s[r] * c : -INFINITY;
                float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
                mx = wave_max_xor_16_32(mx);
                const float m_new = fmaxf(m_run, mx);
                const float m_use = m_new == -INFINITY ? 0.f : m_new;
                const float alpha = fexp2(m_run - m_use);
                float p[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) p[r] = fexp2(sv[r] - m_use);
                l_run = l_run * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
                m_run = m_new;
#pragma unroll
                for (int dt = 0; dt < D / 16; ++dt) o[dt] *= alpha;
                if (jb * 16 + 16 > L) cur.mask_v(L - t0);  // slots past the context
                if constexpr (kv == KV_F32) {
                    cur.pv(p, o);
                } else {
                    s16x4 pb;
                    pb[0] = (short)bf16_bits_rne(p[0] * vsc);
                    pb[1] = (short)bf16_bits_rne(p[1] * vsc);
                    pb[2] = (short)bf16_bits_rne(p[2] * vsc);
                    pb[3] = (short)bf16_bits_rne(p[3] * vsc);
                    cur.pv(pb, o);
                }
                cur = nxt;
            }
        }

        // combine the waves' states through LDS
        l_run = wave_sum_xor_16_32(l_run);
        if (g == 0) {
            s_m[wave][n] = m_run;
            s_l[wave][n] = l_run;
        }
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt)
            *(f32x4*)&s_o[wave][n][16 * dt + 4 * g] = o[dt];
        __syncthreads();

        const int rn = threadIdx.x / TPR, rc = threadIdx.x % TPR;
        if (rn < nrows) {
            float M = -INFINITY;
#pragma unroll
            for (int w = 0; w < NW; ++w) M = fmaxf(M, s_m[w][rn]);
            float wt[NW], l = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                wt[w] = s_m[w][rn] == -INFINITY ? 0.f : fexp2(s_m[w][rn] - M);
                l += wt[w] * s_l[w][rn];
            }
            float acc[DPT];
#pragma unroll
            for (int e = 0; e < DPT; ++e) acc[e] = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w)
#pragma unroll
                for (int e = 0; e < DPT; ++e) acc[e] += wt[w] * s_o[w][rn][rc * DPT + e];
            const float inv = l > 0.f ? 1.0f / l : 0.f;
            const int oj = rn / G;
            const int orow = qs + it.qtok0 + oj;
            const int ohead = kvh * G + (rn - oj * G);
            const int64_t rowid = (int64_t)orow * Hq + ohead;
            if (nparts == 1) {
                if constexpr (kv == KV_F32) {
                    float* op = (float*)a.out + rowid * D + rc * DPT;
#pragma unroll
                    for (int e = 0; e < DPT; ++e) op[e] = acc[e] * inv;
                } else {
                    uint16_t* op = (uint16_t*)a.out + rowid * D + rc * DPT;
#pragma unroll
                    for (int e = 0; e < DPT; ++e) op[e] = (uint16_t)bf16_bits_rne(acc[e] * inv);
                }
                if (a.lse && rc == 0)
                    a.lse[rowid] = l > 0.f ? (M + __log2f(l)) * kLn2 : -INFINITY;
            } else {
                float* pp = a.part_o + (rowid * a.max_parts + it.part) * D + rc * DPT;
#pragma unroll
                for (int e = 0; e < DPT; ++e) pp[e] = acc[e] * inv;
                if (rc == 0)
                    a.part_lse[rowid * a.max_parts + it.part] =
                        l > 0.f ? M + __log2f(l) : -INFINITY;
            }
        }
        __syncthreads();
    }
}

// ---- merge -------------------------------------------------------------------

template <int qd, int D>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t rowid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (rowid >= (int64_t)a.num_tokens * a.num_q_heads) return;
    const int tok = (int)(rowid / a.num_q_heads);
    const int np = a.tok_np[tok];
    if (np <= 1) return;  // written directly by the attention kernel
    const float* lp = a.part_lse + rowid * a.max_parts;
    float M = -INFINITY;
    for (int p = lane; p < np; p += 64) M = fmaxf(M, lp[p]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    constexpr int DPL = D / 64;  // dims per lane
    float acc[DPL];
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[e] = 0.f;
    float W = 0.f;
    const float* po = a.part_o + rowid * a.max_parts * D + lane * DPL;
    for (int p = 0; p < np; ++p) {
        const float lv = lp[p];
        const float w = (lv == -INFINITY) ? 0.f : fexp2(lv - M);
        W += w;
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[e] += w * po[(int64_t)p * D + e];
    }
    const float inv = W > 0.f ? 1.0f / W : 0.f;
    if constexpr (qd == PA_F32) {
        float* op = (float*)a.out + rowid * D + lane * DPL;
#pragma unroll
        for (int e = 0; e < DPL; ++e) op[e] = acc[e] * inv;
    } else {
        uint16_t* op = (uint16_t*)a.out + rowid * D + lane * DPL;
#pragma unroll
        for (int e = 0; e < DPL; ++e) op[e] = (uint16_t)bf16_bits_rne(acc[e] * inv);
    }
    if (a.lse && lane == 0) a.lse[rowid] = W > 0.f ? (M + __log2f(W)) * kLn2 : -INFINITY;
}

__global__ void fp8_decode_kernel(const uint8_t* in, float* out, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    f32x2 f = __builtin_amdgcn_cvt_pk_f32_fp8((uint32_t)in[i], false);
    out[i] = f.x;
}

// ---- occupancy-sized persistent grid ----------------------------------------

template <int kv, int D>
hipError_t launch_attention_t(const AttnArgs& a, int64_t max_units, hipStream_t s) {
    static int per_cu = -1, num_cu = 0;
    if (per_cu < 0) {
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return e;
        e = hipDeviceGetAttribute(&num_cu, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        int occ = 0;
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, attention_kernel<kv, D>,
                                                         64 * kWaves, 0);
        if (e != hipSuccess) return e;
        per_cu = occ > 0 ? occ : 1;
    }
    int64_t grid = (int64_t)per_cu * num_cu;
    if (max_units < grid) grid = max_units;
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL((attention_kernel<kv, D>), dim3((unsigned)grid), dim3(64 * kWaves), 0, s,
                       a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_plan(const PlanArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_attention(int kv_dtype, int head_dim, const AttnArgs& a, int64_t max_units,
                            hipStream_t s) {
    switch (kv_dtype * 1000 + head_dim) {
    case PA_F32 * 1000 + 64: return launch_attention_t<KV_F32, 64>(a, max_units, s);
    case PA_F32 * 1000 + 128: return launch_attention_t<KV_F32, 128>(a, max_units, s);
    case PA_BF16 * 1000 + 64: return launch_attention_t<KV_BF16, 64>(a, max_units, s);
    case PA_BF16 * 1000 + 128: return launch_attention_t<KV_BF16, 128>(a, max_units, s);
    case PA_FP8_E4M3FN * 1000 + 64: return launch_attention_t<KV_FP8, 64>(a, max_units, s);
    case PA_FP8_E4M3FN * 1000 + 128: return launch_attention_t<KV_FP8, 128>(a, max_units, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_merge(int q_dtype, int head_dim, const MergeArgs& a, hipStream_t s) {
    const int64_t rows = (int64_t)a.num_tokens * a.num_q_heads;
    const dim3 grid((unsigned)((rows + 3) / 4));
    if (rows == 0) return hipSuccess;
    if (q_dtype == PA_F32 && head_dim == 64)
        hipLaunchKernelGGL((merge_kernel<PA_F32, 64>), grid, dim3(256), 0, s, a);
    else if (q_dtype == PA_F32 && head_dim == 128)
        hipLaunchKernelGGL((merge_kernel<PA_F32, 128>), grid, dim3(256), 0, s, a);
    else if (q_dtype == PA_BF16 && head_dim == 64)
        hipLaunchKernelGGL((merge_kernel<PA_BF16, 64>), grid, dim3(256), 0, s, a);
    else if (q_dtype == PA_BF16 && head_dim == 128)
        hipLaunchKernelGGL((merge_kernel<PA_BF16, 128>), grid, dim3(256), 0, s, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_fp8_decode(const uint8_t* in, float* out, int n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(fp8_decode_kernel, dim3((n + 255) / 256), dim3(256), 0, s, in, out, n);
    return hipGetLastError();
}

}  // namespace pa
