// pa_attention.hip -- paged attention kernels for gfx950 (MI355X).
//
// Three kernels run in order on the caller's stream:
//
//   plan       one workgroup turns (query spans, context lengths) into the
//              work of the call, in device memory, so the host never reads
//              lengths back. This is the per-step "plan" of the request
//              trace on "03 -- Engines Papers" (whiteboard test), done on
//              the device. Query rows are grouped into tiles: a narrow tile
//              holds up to 16 rows (G query heads x 16/G tokens of one
//              span); a wide tile holds 2 x 16 rows of a
//              chunked-prefill span. Every (tile, KV head) pair is a segment
//              of 16-token key blocks; the segments of each tile class form
//              one stream of blocks, cut into pieces of equal size (one per
//              resident wave, or partition_size tokens each).
//   attention  a persistent grid of one-wave workgroups per tile class; wave
//              v walks pieces v, v + grid, ... Inside a piece it gathers the
//              blocks through the block table ("03 -- Engines Papers",
//              section 2), one block ahead in a register ring, and keeps an
//              online softmax (running max and sum, Milakov & Gimelshein on
//              the "References" page) in registers. A segment the piece saw
//              whole writes its output rows; a segment cut by a piece
//              boundary writes a partial (lse, normalized o) per row.
//   merge      one wave per cut segment combines its partials by
//              log-sum-exp (split-K decode, playbook Theme 4; LSE merge,
//              first page section 12).
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

#include <atomic>
#include <type_traits>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

using namespace dev;

// ---- per-dtype register images of one 16-token block ---------------------

template <int kv, int D>
struct Tile;

// fp32: QK with 16x16x4 f32 MFMA (D/4 steps), PV with 4 steps per 16 dims.
template <int D>
struct Tile<KV_F32, D> {
    float4 k[D / 16];  // load j, element e: K[t][16j + 4g + e]
    float4 v[D / 16];  // V^T[16dt + d][4g .. 4g+3]
    using QReg = float[D / 4];

    template <bool nt>
    __device__ __forceinline__ void load(const void* kc, const void* vc, int64_t blk_head,
                                         int lane) {
        const int t = lane & 15, g = lane >> 4;
        // load j reads 64 contiguous bytes of row t across the 4 lane groups
        const float* kp = (const float*)kc + blk_head * 16 * D + t * D + 4 * g;
#pragma unroll
        for (int j = 0; j < D / 16; ++j) k[j] = ld_kv<nt>((const float4*)(kp + 16 * j));
        const float* vb = (const float*)vc + blk_head * 16 * D;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt)
            v[dt] = ld_kv<nt>((const float4*)(vb + (16 * dt + t) * 16 + 4 * g));
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
    uint4 k[D / 32];  // 8 bf16 each: K[t][32j + 8g .. +8]
    uint2 v[D / 16];  // 4 bf16 each: V^T[16dt + d][4g .. 4g+3]

    template <bool nt>
    __device__ __forceinline__ void load(const void* kc, const void* vc, int64_t blk_head,
                                         int lane) {
        const int t = lane & 15, g = lane >> 4;
        // load j reads 64 contiguous bytes of row t across the 4 lane groups
        const uint16_t* kp = (const uint16_t*)kc + blk_head * 16 * D + t * D + 8 * g;
#pragma unroll
        for (int j = 0; j < D / 32; ++j) k[j] = ld_kv<nt>((const uint4*)(kp + 32 * j));
        const uint16_t* vb = (const uint16_t*)vc + blk_head * 16 * D;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt)
            v[dt] = ld_kv<nt>((const uint2*)(vb + (16 * dt + t) * 16 + 4 * g));
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
    uint4 k[D / 64];     // 16 e4m3 bytes each: K[t][64j + 16g .. +16]
    uint32_t v[D / 16];  // 4 e4m3 bytes each: V^T[16dt + d][4g .. 4g+3]

    template <bool nt>
    __device__ __forceinline__ void load(const void* kc, const void* vc, int64_t blk_head,
                                         int lane) {
        const int t = lane & 15, g = lane >> 4;
        // load j reads 64 contiguous bytes of row t across the 4 lane groups
        const uint8_t* kp = (const uint8_t*)kc + blk_head * 16 * D + t * D + 16 * g;
#pragma unroll
        for (int j = 0; j < D / 64; ++j) k[j] = ld_kv<nt>((const uint4*)(kp + 64 * j));
        const uint8_t* vb = (const uint8_t*)vc + blk_head * 16 * D;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt)
            v[dt] = ld_kv<nt>((const uint32_t*)(vb + (16 * dt + t) * 16 + 4 * g));
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

// fp8 cache with S = K q^T on the fp8 matrix cores. The query row arrives as
// two e4m3 terms over the lane's dims in the K tile's byte order: the row
// scaled to the e4m3 range (hi) and 16 times what that rounding left
// (lo), so q / sq = hi + lo / 16 to about 2^-8 of each value. One
// v_mfma_scale_f32_16x16x128_f8f6f4 per term takes the lo term with an
// E8M0 block scale of 2^-4 into the same accumulator. P V is unchanged.
typedef int i32x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ i32x8 join8(uint4 a, uint4 b) {
    return i32x8{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
}
constexpr int kE8M0One = 127;          // E8M0 code of 2^0
constexpr int kE8M0Sixteenth = 123;    // 2^-4
template <int D>
__device__ __forceinline__ f32x4 qk_fp8(const uint4 (&k)[D / 64], const uint4* q) {
    // q[0], q[1]: hi term; q[2], q[3]: lo term (D = 64 fills only q[0], q[2])
    i32x8 a;
    if constexpr (D == 128) {
        a = join8(k[0], k[1]);
    } else {
        a = join8(k[0], make_uint4(0, 0, 0, 0));
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, join8(q[0], q[1]), acc, 0, 0, 0,
                                                           kE8M0One, 0, kE8M0One);
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, join8(q[2], q[3]), acc, 0, 0, 0,
                                                           kE8M0One, 0, kE8M0Sixteenth);
    return acc;
}

template <int D>
struct Tile<KV_FP8Q, D> : Tile<KV_FP8, D> {
    __device__ __forceinline__ f32x4 qk(const uint4* q) const { return qk_fp8<D>(this->k, q); }
    // O += V^T P on the fp8 matrix cores, one v_mfma_f32_16x16x32_fp8_fp8
    // per 16 output dims: the 32-long contraction holds the block's 16 keys
    // twice, once against P's e4m3 term and once against what that term's
    // rounding left (p8 from p_fp8_two_term), so the e4m3 V bytes are used
    // as stored and P keeps about 2^-8 of its value.
    __device__ __forceinline__ void pv8(uint64_t p8, f32x4* o) const {
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
            const uint64_t a = (uint64_t)this->v[dt] | ((uint64_t)this->v[dt] << 32);
            o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8((long)a, (long)p8, o[dt], 0, 0, 0);
        }
    }
};

// Decode with this step's tokens appended in the same pass: the wave that
// reads a sequence's last block for KV head h puts the new token's K row and
// V column (key o = (L - 1) % 16 of that block) into the tile it loaded, in
// place of what the cache held there, and writes them to the cache as the
// append does (an fp8 cache gets e4m3fn(fp32(x) / scale) of the block).
// NewRow holds a lane's share of the new row as given: dims lane + 64 m.
template <int kv, int D>
struct NewRow {
    using Src = typename std::conditional<kv == KV_F32, float, uint16_t>::type;
    static constexpr int kPer = (D + 63) / 64;
    Src k[kPer], v[kPer];
    __device__ __forceinline__ void load(const void* kn, const void* vn, int lane) {
#pragma unroll
        for (int m = 0; m < kPer; ++m) {
            const int d = min(lane + 64 * m, D - 1);
            k[m] = ((const Src*)kn)[d];
            v[m] = ((const Src*)vn)[d];
        }
    }
};

// Replace 16-bit element e (0..3) of four packed in a uint2.
__device__ __forceinline__ uint2 put16(uint2 w, int e, uint16_t x) {
    const uint32_t sh = 16u * (e & 1);
    const uint32_t m = 0xffffu << sh;
    if (e < 2)
        w.x = (w.x & ~m) | ((uint32_t)x << sh);
    else
        w.y = (w.y & ~m) | ((uint32_t)x << sh);
    return w;
}

// Row q (bf16) -> the two e4m3 terms of qk_fp8 for this lane's dims 16g +
// [0, 16) and, for D = 128, 64 + 16g + [0, 16); returns the row's scale sq
// (amax / 448; every lane of the row gets the same one). Rows of zeros get
// sq = 0 and zero terms.
__device__ __forceinline__ uint32_t pk_fp8(float a, float b, float c, float d) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
template <int D>
__device__ __forceinline__ float quantize_q_fp8(const uint16_t* qrow, bool ok, int g,
                                                uint4 (&out)[4]) {
    constexpr int P = D / 64;  // 16-dim parts per lane
    float x[P][16];
#pragma unroll
    for (int p = 0; p < P; ++p) {
        const uint4* src = (const uint4*)(qrow + 64 * p + 16 * g);
        const uint4 a = ok ? src[0] : make_uint4(0, 0, 0, 0);
        const uint4 b = ok ? src[1] : make_uint4(0, 0, 0, 0);
        const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            x[p][2 * i] = bf16_lo(w[i]);
            x[p][2 * i + 1] = bf16_hi(w[i]);
        }
    }
    float amax = 0.f;
#pragma unroll
    for (int p = 0; p < P; ++p)
#pragma unroll
        for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(x[p][i]));
    amax = row_max(amax);
    const float inv = amax > 0.f ? 448.f / amax : 0.f;
    uint32_t hi[8] = {0, 0, 0, 0, 0, 0, 0, 0}, lo[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int p = 0; p < P; ++p) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float u[4], r[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) u[e] = fminf(fmaxf(x[p][4 * i + e] * inv, -448.f), 448.f);
            const uint32_t h = pk_fp8(u[0], u[1], u[2], u[3]);
            const f32x2_t h01 = __builtin_amdgcn_cvt_pk_f32_fp8((int)h, false);
            const f32x2_t h23 = __builtin_amdgcn_cvt_pk_f32_fp8((int)h, true);
            r[0] = 16.f * (u[0] - h01.x);
            r[1] = 16.f * (u[1] - h01.y);
            r[2] = 16.f * (u[2] - h23.x);
            r[3] = 16.f * (u[3] - h23.y);
            hi[4 * p + i] = h;
            lo[4 * p + i] = pk_fp8(r[0], r[1], r[2], r[3]);
        }
    }
    out[0] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
    out[1] = make_uint4(hi[4], hi[5], hi[6], hi[7]);
    out[2] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
    out[3] = make_uint4(lo[4], lo[5], lo[6], lo[7]);
    return amax * (1.f / 448.f);
}

// Four probabilities (already scaled into the e4m3 range) -> the B operand
// of Tile<KV_FP8Q>::pv8: bytes 0-3 their e4m3 roundings, bytes 4-7 the
// e4m3 roundings of the remainders, so hi + lo matches each value to about
// 2^-8 of it (remainders below the e4m3 normal range keep an absolute error
// under 2^-10).
__device__ __forceinline__ uint64_t p_fp8_two_term(const float (&p)[4], float s) {
    float u[4], r[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) u[e] = fminf(p[e] * s, 448.f);
    const uint32_t h = pk_fp8(u[0], u[1], u[2], u[3]);
    const f32x2_t h01 = __builtin_amdgcn_cvt_pk_f32_fp8((int)h, false);
    const f32x2_t h23 = __builtin_amdgcn_cvt_pk_f32_fp8((int)h, true);
    r[0] = u[0] - h01.x;
    r[1] = u[1] - h01.y;
    r[2] = u[2] - h23.x;
    r[3] = u[3] - h23.y;
    const uint32_t l = pk_fp8(r[0], r[1], r[2], r[3]);
    return (uint64_t)h | ((uint64_t)l << 32);
}

// ---- plan ------------------------------------------------------------------
//
// The work of each tile class is a stream of 16-token key blocks: segment
// (tile t, KV head h) contributes the nb[t] blocks its rows read. The stream
// is laid out KV-head-major: one substream per KV head, holding that head's
// segments in tile order. Each substream is cut into pieces of R
// consecutive blocks, and piece k of head h gets number k * Hkv + h, so the
// pieces of one head interleave with period Hkv. Each wave of the attention
// grid streams whole pieces: wave w takes pieces w, w + grid, ... With a
// grid that is a multiple of Hkv, every piece a wave takes belongs to head
// w mod Hkv; since workgroups are dealt to the XCDs in turn, the waves of
// one XCD then serve one KV head (or a few), and tiles that read the same
// blocks (the query tiles of a chunked-prefill span) find them in that
// XCD's L2. With R chosen as Hkv * substream / resident waves, every wave
// gets the same number of blocks, so all finish together whatever the
// spread of context lengths (the split-KV decode of the playbook's Theme 4,
// balanced by block count). A segment cut by a piece boundary leaves
// partial results that the merge pass combines.

constexpr int kPlanThreads = 1024;

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

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(PlanArgs a) {
    __shared__ int s_tp[kMaxTiles + 1];  // nb per tile, then its exclusive prefix
    __shared__ int s_nsplit;
    const int cap = min(a.max_tiles, kMaxTiles);
    const int H = a.num_kv_heads;
    const int S = a.num_seqs;
    auto span_of = [&](int i, int& qs, int& n, int& L) {
        qs = a.qsl ? a.qsl[i] : i;
        n = a.qsl ? a.qsl[i + 1] - qs : 1;
        L = min(max(a.context_lens[i], 0), a.max_context_len);
        if (qs < 0 || n < 0 || qs + n > a.num_tokens) n = 0;  // malformed span
    };

    // 0. shared-prefix groups: a single-token member whose context extends
    //    past the group's prefix reads the prefix through its group's tiles
    //    and only the rest itself (cascade attention)
    // member entries and the group of an entry (the last group whose first
    // entry is at or before it)
    const int num_entries =
        a.num_groups > 0 ? min(max(a.group_offsets[a.num_groups], 0), S) : 0;
    auto group_of = [&](int e) {
        int lo = 0, hi = a.num_groups - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (a.group_offsets[mid] <= e) lo = mid; else hi = mid - 1;
        }
        return lo;
    };
    if (a.num_groups > 0) {
        for (int i = threadIdx.x; i < S; i += kPlanThreads) {
            a.cas_prefix[i] = 0;
            a.cas_tile[i] = -1;
            a.cas_gtile[i] = -1;
            a.cas_pos[i] = 0;
            // the attention pass reads the members from the workspace (the
            // host guarantees at most num_seqs of them)
            a.cas_members[i] = i < a.group_offsets[a.num_groups] ? a.group_members[i] : -1;
        }
        __syncthreads();
        // one thread per member entry (the groups of a batch can be large)
        for (int e = threadIdx.x; e < num_entries; e += kPlanThreads) {
            const int g = group_of(e);
            const int pb = a.group_prefix_blocks[g];
            const int lead = a.group_members[a.group_offsets[g]];  // its table is read
            const int i = a.group_members[e];
            if (pb < 1 || lead < 0 || lead >= S || i < 0 || i >= S) continue;
            int qs, n, L;
            span_of(i, qs, n, L);
            if (n == 1 && L > 16 * pb) a.cas_prefix[i] = pb;
        }
        __syncthreads();
    }

    // 1. tiles: spans longer than one narrow tile get wide tiles (stream 0);
    //    everything else narrow ones (stream 1); the groups' tiles form
    //    stream 2; sequence order within each. Stream st holds tiles
    //    [t_first[st], t_first[st + 1]).
    int tile_base = 0;
    __shared__ int t_first[NUM_STREAMS + 1];
    for (int st = 0; st < NUM_STREAMS; ++st) {
        if (threadIdx.x == 0) t_first[st] = min(tile_base, cap);
        if (st != STREAM_GROUP) {
        for (int c0 = 0; c0 < S; c0 += kPlanThreads) {
            const int i = c0 + (int)threadIdx.x;
            int n = 0, L = 0, ntl = 0, qs = 0, tt = 1;
            if (i < S) {
                span_of(i, qs, n, L);
                const bool wide = a.wide_tokens > 0 && n > a.narrow_tokens;
                tt = wide ? a.wide_tokens : a.narrow_tokens;
                ntl = (n > 0 && wide == (st == STREAM_WIDE)) ? (n + tt - 1) / tt : 0;
            }
            int total;
            const int off = tile_base + block_exclusive_scan(ntl, &total);
            const int pre = (st == STREAM_NARROW && a.num_groups > 0 && i < S) ? a.cas_prefix[i]
                                                                               : 0;
            for (int k = 0; k < ntl; ++k) {
                const int t = off + k;
                if (t >= cap) break;
                const int k0 = k * tt;
                const int nt = min(tt, n - k0);
                const int maxpos = L - n + k0 + nt - 1;  // last query position of the tile
                int nb = max(1, maxpos >= 0 ? (min(maxpos + 1, L) + 15) >> 4 : 0);
                TileDesc td{i, k0, nt, nb, L, qs, n, 0, 0, {0, 0, 0}};
                if (pre > 0) {  // a cascade member's suffix: blocks pre .. of its context
                    td.flags = TILE_SUFFIX;
                    td.b0 = pre;
                    td.nb = nb - pre;
                    a.cas_tile[i] = t;
                }
                a.tiles[t] = td;
                s_tp[t] = td.nb;
            }
            tile_base += total;
        }
        }
        if (st == STREAM_GROUP && a.num_groups > 0) {
            const int mpt = a.members_per_tile;
            for (int c0 = 0; c0 < a.num_groups; c0 += kPlanThreads) {
                const int g = c0 + (int)threadIdx.x;
                int ntl = 0, e0 = 0, cnt = 0, pb = 0, lead = -1;
                if (g < a.num_groups) {
                    pb = a.group_prefix_blocks[g];
                    e0 = a.group_offsets[g];
                    cnt = a.group_offsets[g + 1] - e0;
                    lead = cnt > 0 ? a.group_members[e0] : -1;
                    if (pb >= 1 && cnt > 0 && lead >= 0 && lead < S) ntl = (cnt + mpt - 1) / mpt;
                }
                int total;
                const int off = tile_base + block_exclusive_scan(ntl, &total);
                if (g < a.num_groups) a.cas_gbase[g] = ntl > 0 ? off : -1;
                for (int k = 0; k < ntl; ++k) {
                    const int t = off + k;
                    if (t >= cap) break;
                    const int m0 = k * mpt, mn = min(mpt, cnt - m0);
                    a.tiles[t] = TileDesc{lead, e0 + m0, mn, pb, 16 * pb, 0, 1, TILE_GROUP, 0,
                                          {0, 0, 0}};
                    s_tp[t] = pb;
                }
                tile_base += total;
            }
            __syncthreads();
            // each qualifying member's group tile and place in it
            for (int e = threadIdx.x; e < num_entries; e += kPlanThreads) {
                const int g = group_of(e);
                const int base = a.cas_gbase[g];
                const int i = a.group_members[e];
                if (base < 0 || i < 0 || i >= S ||
                    a.cas_prefix[i] != a.group_prefix_blocks[g])
                    continue;
                const int m = e - a.group_offsets[g];
                const int t = base + m / mpt;
                if (t < cap) {
                    a.cas_gtile[i] = t;
                    a.cas_pos[i] = m % mpt;
                }
            }
        }
    }
    const int ntiles = min(tile_base, cap);
    if (threadIdx.x == 0) t_first[NUM_STREAMS] = ntiles;
    __syncthreads();

    // 2. exclusive prefix of blocks over tiles (in LDS)
    int carry = 0;
    for (int c0 = 0; c0 < ntiles; c0 += kPlanThreads) {
        const int t = c0 + (int)threadIdx.x;
        const int nb = t < ntiles ? s_tp[t] : 0;
        int total;
        const int before = block_exclusive_scan(nb, &total);
        if (t < ntiles) s_tp[t] = carry + before;
        carry += total;
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        s_tp[ntiles] = carry;
        s_nsplit = 0;
    }
    __syncthreads();

    // 3. per stream: piece size, piece starts (all KV heads' substreams
    //    hold the same blocks, B = the stream's tiles' nb summed). When
    //    balancing, pieces are cut at equal cost, where a segment costs its
    //    blocks plus c blocks for its start (row setup, the first block's
    //    latency, the epilogue): a piece that starts more segments gets
    //    fewer blocks, so waves finish together. In the cost coordinate the
    //    c units of a tile come before its blocks; a piece that starts
    //    inside them starts at the tile's first block. With at least c + 1
    //    units per piece no piece is empty. A fixed partition size uses c =
    //    0, pieces of exactly P / 16 blocks.
    //    The span stream is cut for a.span_shared workgroups (one per
    //    compute unit, running beside the narrow launches) when the other
    //    streams' cost is at least kSpanShareRatio times its own.
    int Rs[NUM_STREAMS], Cs[NUM_STREAMS];
    int64_t cost_of[NUM_STREAMS];
    for (int st = 0; st < NUM_STREAMS; ++st) {
        const int t_lo = t_first[st], t_hi = t_first[st + 1];
        const int c = a.part_blocks > 0 ? 0 : max(a.part_cost[st], 0);
        cost_of[st] = (int64_t)(s_tp[t_hi] - s_tp[t_lo]) + (int64_t)c * (t_hi - t_lo);
    }
    const bool share = a.span_shared > 0 && a.part_blocks <= 0 && cost_of[STREAM_WIDE] > 0 &&
                       cost_of[STREAM_NARROW] + cost_of[STREAM_GROUP] >=
                           (int64_t)kSpanShareRatio * cost_of[STREAM_WIDE];
    for (int st = 0; st < NUM_STREAMS; ++st) {
        const int t_lo = t_first[st], t_hi = t_first[st + 1];
        const int64_t B = s_tp[t_hi] - s_tp[t_lo];
        const int c = a.part_blocks > 0 ? 0 : max(a.part_cost[st], 0);
        const int64_t Bc = cost_of[st];  // cost of the substream
        const int waves = share && st == STREAM_WIDE ? a.span_shared : a.waves[st];
        int64_t R = a.part_blocks;
        if (R <= 0) {
            R = ((int64_t)H * Bc + waves - 1) / max(waves, 1);
            R = max(R, (int64_t)a.min_blocks[st] + c);
        }
        int64_t K = (Bc + R - 1) / R;  // pieces per substream
        const int64_t kmax = a.max_pieces[st] / H;
        if (kmax == 0) {  // no room: the caller understated max_query_len
            K = 0;
        } else if (K > kmax) {  // never for sizes the host planned for
            R = max((Bc + kmax - 1) / kmax, (int64_t)c + 1);
            K = (Bc + R - 1) / R;
        }
        R = max(R, (int64_t)1);
        Rs[st] = (int)R;
        Cs[st] = c;
        // the stream position (blocks) of cost coordinate x
        auto position = [&](int64_t x, int& tile, int& jj) {
            int lo = t_lo, hi = t_hi - 1;  // last tile whose cost prefix is <= x
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                const int64_t cp = (int64_t)(s_tp[mid] - s_tp[t_lo]) + (int64_t)c * (mid - t_lo);
                if (cp <= x) lo = mid; else hi = mid - 1;
            }
            const int64_t cp = (int64_t)(s_tp[lo] - s_tp[t_lo]) + (int64_t)c * (lo - t_lo);
            tile = lo;
            jj = (int)max((int64_t)0, x - cp - c);
        };
        const int64_t V = K * H;
        for (int64_t v = threadIdx.x; v < V; v += kPlanThreads) {
            const int h = (int)(v % H);
            const int64_t k = v / H;
            int t0, j0, t1 = t_hi, j1 = 0;
            position(k * R, t0, j0);
            if (k + 1 < K) position((k + 1) * R, t1, j1);
            PieceStart ps{};
            ps.tile = t0;
            ps.kvh = h;
            ps.j = j0;
            ps.nblocks = (s_tp[t1] + j1) - (s_tp[t0] + j0);
            ps.td = a.tiles[t0];
            a.pieces[st][v] = ps;
        }
        if (threadIdx.x == 0) {
            a.hdr[HDR_STREAM + 4 * st + HDR_TOTAL] = (int)B;
            a.hdr[HDR_STREAM + 4 * st + HDR_R] = (int)R;
            a.hdr[HDR_STREAM + 4 * st + HDR_NPIECES] = (int)V;
        }
    }
    auto stream_of = [&](int t) {
        return t < t_first[STREAM_NARROW] ? STREAM_WIDE
               : t < t_first[STREAM_GROUP] ? STREAM_NARROW
                                           : STREAM_GROUP;
    };
    // pieces of substream h holding a segment's first and last blocks: the
    // block at stream offset b of tile t sits at cost b + c (t - t_lo + 1)
    auto cut = [&](int t, int& k0, int& k1) {
        const int st = stream_of(t);
        const int t_lo = t_first[st];
        const int64_t x0 =
            (int64_t)(s_tp[t] - s_tp[t_lo]) + (int64_t)Cs[st] * (t - t_lo + 1);
        k0 = (int)(x0 / Rs[st]);
        k1 = (int)((x0 + s_tp[t + 1] - s_tp[t] - 1) / Rs[st]);
    };

    // 4. segments cut by a piece boundary, for the merge pass (a segment is
    //    cut iff its first and last blocks fall in different pieces of its
    //    KV head's substream); cascade parts are combined per member (5.)
    const int64_t max_splits = a.max_splits;
    for (int sg = threadIdx.x; sg < ntiles * H; sg += kPlanThreads) {
        const int t = sg / H, h = sg % H;
        const TileDesc td = a.tiles[t];
        if (td.flags != 0) continue;
        int k0, k1;
        cut(t, k0, k1);
        if (k0 != k1) {
            const int k = atomicAdd(&s_nsplit, 1);  // list order is irrelevant
            if (k < max_splits)
                a.splits[k] = SplitSeg{td.qs + td.qtok0, td.ntok, h, k0, k1,
                                       stream_of(t), {0, 0}};
        }
    }
    __syncthreads();
    // records past the list are marked empty, so a merge wave needs one load
    const int nsplit = (int)min((int64_t)s_nsplit, max_splits);
    for (int64_t k = nsplit + threadIdx.x; k < max_splits; k += kPlanThreads)
        a.splits[k] = SplitSeg{0, 0, 0, -1, -1, 0, {0, 0}};

    // 5. one record per (cascade member, KV head): its prefix and suffix
    int ncas = 0;
    if (a.num_groups > 0) {
        for (int c0 = 0; c0 < S; c0 += kPlanThreads) {
            const int i = c0 + (int)threadIdx.x;
            const bool mem = i < S && a.cas_prefix[i] > 0 && a.cas_tile[i] >= 0 &&
                             a.cas_gtile[i] >= 0 && a.cas_tile[i] < ntiles &&
                             a.cas_gtile[i] < ntiles;
            int total;
            const int rank = ncas + block_exclusive_scan(mem ? 1 : 0, &total);
            if (mem && (int64_t)(rank + 1) * H <= a.max_cas_recs) {
                const TileDesc td = a.tiles[a.cas_tile[i]];
                int sk0, sk1, pk0, pk1;
                cut(a.cas_tile[i], sk0, sk1);
                cut(a.cas_gtile[i], pk0, pk1);
                for (int h = 0; h < H; ++h)
                    a.cas_recs[(int64_t)rank * H + h] =
                        CascadeRec{td.qs, h, sk0, sk1, pk0, pk1, a.cas_pos[i], 0};
            }
            ncas += total;
        }
        ncas = (int)min((int64_t)ncas * H, (int64_t)a.max_cas_recs);
    }
    // 6. tree verification masks travel with the plan
    if (a.tree_mask)
        for (int r = threadIdx.x; r < a.num_tokens; r += kPlanThreads) a.tree_ws[r] = a.tree_mask[r];
    if (threadIdx.x == 0) {
        a.hdr[HDR_NTILES] = ntiles;
        a.hdr[HDR_NSPLIT] = nsplit;
        a.hdr[HDR_NCAS] = ncas;
        a.hdr[HDR_TREE] = a.tree_mask ? 1 : 0;
    }
}

// ---- attention ---------------------------------------------------------------

// K/V blocks in flight per wave beyond the one in use (one wave per SIMD).
// An fp8 block is half the bytes of a bf16 one, so fp8 caches keep more
// blocks in flight for the same bytes.
#ifndef PA_PREFETCH
#define PA_PREFETCH 2
#endif
// Registers of block ids per lane: a chunk of the narrow kernel holds up to
// 64 times this many blocks. For bf16 caches 2 left the Llama-3-8B-shaped
// and the long-context passes within 1 us of 1 (alternating runs, each
// after a pause). An fp8 chunk carries half the bytes of a bf16 one for the
// same drain and refill of the ring at its end: with 2, the fp8
// parallel-sampling pass went from 114.9-118.1 to 112.1-112.9 us (the same
// batch without its groups 369 -> 368 us); 4 gave no more.
#ifndef PA_ID_WINDOWS
#define PA_ID_WINDOWS 1
#endif
#ifndef PA_ID_WINDOWS_FP8
#define PA_ID_WINDOWS_FP8 2
#endif
#ifndef PA_PREFETCH_FP8
#define PA_PREFETCH_FP8 2
#endif
// Group tiles (a shared prefix read for several members) load through L2
// (1) or stream past it like the other narrow tiles (0).
#ifndef PA_GROUP_L2
#define PA_GROUP_L2 0
#endif

// New keys staged in LDS (the workgroup is one wave) in the cache's
// encoding: each lane encodes its share of the row, and the lanes that hold
// key o of the tile read their elements back from the staged row. The
// cache write of a new key is a partial-line store (its V column is one
// element in each 32-byte row of the block), and on gfx9 a wave's later
// loads wait for its earlier stores: written where the wave goes on to read
// blocks, it would hold the next block's wait until the line has been
// filled and written. The attention pass never reads a new key from the
// cache (it takes it from the tile), so the writes wait for the end of the
// wave's work, where nothing waits for them. A wave that stages more than
// kMax keys writes them out early.
template <int kv, int D>
struct NewStage {
    using E = typename std::conditional<kv == KV_F32, float,
                                        typename std::conditional<kv == KV_BF16, uint16_t,
                                                                  uint8_t>::type>::type;
    static constexpr int kMax = 16;
    E* k;         // [kMax][D]: K rows in the cache's encoding
    E* v;         // [kMax][D]: V columns
    int64_t* bh;  // [kMax] block-head
    int* o;       // [kMax] key in the block
    int count = 0;

    __device__ __forceinline__ static E enc(typename NewRow<kv, D>::Src x, float scale) {
        if constexpr (kv == KV_F32 || kv == KV_BF16)
            return x;
        else
            return (E)encode_e4m3fn(__fdiv_rn(__uint_as_float((uint32_t)x << 16), scale));
    }

    // Stage the new row nr (key o of block-head blk_head; ks, vs: the
    // block's fp8 scales) and put it into tile cur.
    __device__ __forceinline__ void add(const AttnArgs& a, Tile<kv, D>& cur,
                                        const NewRow<kv, D>& nr, const int key,
                                        const int64_t blk_head, const float ks, const float vs,
                                        const int lane) {
        if (count == kMax) flush(a, lane);
        E* kr = k + count * D;
        E* vr = v + count * D;
#pragma unroll
        for (int m = 0; m < NewRow<kv, D>::kPer; ++m) {
            const int d = lane + 64 * m;
            if (d < D) {
                kr[d] = enc(nr.k[m], ks);
                vr[d] = enc(nr.v[m], vs);
            }
        }
        if (lane == 0) {
            bh[count] = blk_head;
            o[count] = key;
        }
        ++count;
        const int t = lane & 15, g = lane >> 4, e = key & 3;
        if (t == key) {
            if constexpr (kv == KV_F32) {
#pragma unroll
                for (int j = 0; j < D / 16; ++j) cur.k[j] = *(const float4*)(kr + 16 * j + 4 * g);
            } else if constexpr (kv == KV_BF16) {
#pragma unroll
                for (int j = 0; j < D / 32; ++j) cur.k[j] = *(const uint4*)(kr + 32 * j + 8 * g);
            } else {
#pragma unroll
                for (int j = 0; j < D / 64; ++j) cur.k[j] = *(const uint4*)(kr + 64 * j + 16 * g);
            }
        }
        if (g == (key >> 2)) {
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt) {
                const E x = vr[16 * dt + t];
                if constexpr (kv == KV_F32) {
                    if (e == 0) cur.v[dt].x = x;
                    if (e == 1) cur.v[dt].y = x;
                    if (e == 2) cur.v[dt].z = x;
                    if (e == 3) cur.v[dt].w = x;
                } else if constexpr (kv == KV_BF16) {
                    cur.v[dt] = put16(cur.v[dt], e, x);
                } else {
                    cur.v[dt] = (cur.v[dt] & ~(0xffu << (8 * e))) | ((uint32_t)x << (8 * e));
                }
            }
        }
    }

    // Write the staged keys to the cache: K rows whole, V columns element
    // by element.
    __device__ __forceinline__ void flush(const AttnArgs& a, const int lane) {
        for (int n = 0; n < count; ++n) {
            const int64_t b = bh[n];
            const int key = o[n];
            E* kd = (E*)a.k_cache + (b * 16 + key) * D;
            E* vd = (E*)a.v_cache + b * D * 16 + key;
#pragma unroll
            for (int d = lane; d < D; d += 64) {
                kd[d] = k[n * D + d];
                vd[d * 16] = v[n * D + d];
            }
        }
        count = 0;
    }
};

// Blocks [j, j + take) of segment (tile td, KV head kvh), by one wave: gather
// each block through the block table, S = K q^T on the matrix cores, online
// softmax in registers, O += V^T P, for NR 16-row tiles of query rows (the
// G heads of up to 16 NR / G query tokens, or of a group tile's members)
// that share every K/V block the wave loads. Then either write the rows'
// output (the wave saw the whole segment) or write a partial result into
// the piece's slot (NR row tiles) for the merge pass.
template <int kv, int D, bool kStreamLoads, int NR>
__device__ __forceinline__ void run_segment(const AttnArgs& a, const TileDesc td, const int kvh,
                                            const int j, const int take, const int piece,
                                            NewStage<kv, D>& stage) {
    using T = Tile<kv, D>;
    constexpr int NT = NR;  // row tiles of a slot: those the wave holds
    constexpr bool kFp8Cache = kv == KV_FP8 || kv == KV_FP8Q;
    using QReg = typename std::conditional<
        kv == KV_F32, float[D / 4],
        typename std::conditional<kv == KV_FP8Q, uint4[4], uint4[D / 32]>::type>::type;
    const int lane = threadIdx.x & 63;
    const int n = lane & 15;  // query row owned in MFMA layouts (within a row tile)
    const int g = lane >> 4;  // lane group
    const int Hkv = a.num_kv_heads, G = a.group, Hq = a.num_q_heads;
    const int seq = td.seq;
    const int L = td.L, qs = td.qs, nspan = td.nspan;
    const int nrows = td.ntok * G;
    // decode with append: the segment that holds its sequence's last block
    // puts the step's new token (key L - 1) into the tile of that block in
    // place of what the cache held there, and stages its cache write
    const bool app = a.k_new != nullptr && td.flags != TILE_GROUP && td.ntok == 1 &&
                     nspan == 1 && L >= 1 && j + take == td.nb;

    // this lane's query row in row tile r: tile row 16 r + n = token qj,
    // head kvh*G + (row % G)
    QReg qreg[NR];
    float qscale[NR];  // fp8 q: the row's scale times the score scale (log2 units)
    // output row index of row tile r (token row * Hq + head; the output of a
    // call is far below 2^31 rows, so 32 bits)
    int rowid[NR];
    bool row_ok[NR];
    // tree verification masks: span token k is visible to a row only where
    // bit k of its token's mask is set (spans of at most 64 tokens)
    const int span_start = L - nspan;
    const bool tree = td.flags == 0 && nspan <= 64 && a.hdr[HDR_TREE] != 0;
    uint64_t tbits[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const int rr = 16 * r + n;
        const int qj = rr / G;  // token of the span (group tile: member)
        row_ok[r] = rr < nrows;
        if (td.flags == TILE_GROUP) {
            // the single query token of member qj sees every prefix key; a
            // member that reads its whole context itself has no row here
            int i = -1;
            if (row_ok[r]) i = a.group_members[td.qtok0 + qj];
            row_ok[r] = i >= 0 && i < a.num_seqs && a.cas_prefix[i] == td.nb;
            const int qrow = row_ok[r] ? (a.qsl ? a.qsl[i] : i) : 0;
            rowid[r] = qrow * Hq + kvh * G + (rr - qj * G);
        } else {
            rowid[r] = (qs + td.qtok0 + qj) * Hq + kvh * G + (rr - qj * G);
        }
        tbits[r] = (tree && row_ok[r]) ? a.tree[qs + td.qtok0 + qj] : ~0ull;
        // q operand (B of S = K q^T), holding the row's dims in the same order
        // as the K tile: f32 16m + 4g + e; bf16 32m + 8g + e; fp8
        // 64(m/2) + 16g + 8(m%2) + e for MFMA step m
        qscale[r] = 1.f;
        if constexpr (kv == KV_FP8Q) {
            const uint16_t* qp = (const uint16_t*)a.q + (int64_t)(row_ok[r] ? rowid[r] : 0) * D;
            qscale[r] = a.scale_log2 * quantize_q_fp8<D>(qp, row_ok[r], g, qreg[r]);
        } else if constexpr (kv == KV_F32) {
            const float* qp = (const float*)a.q + (int64_t)rowid[r] * D + 4 * g;
#pragma unroll
            for (int m = 0; m < D / 16; ++m) {
                float4 x = row_ok[r] ? *(const float4*)(qp + 16 * m)
                                     : make_float4(0.f, 0.f, 0.f, 0.f);
                qreg[r][4 * m] = x.x;
                qreg[r][4 * m + 1] = x.y;
                qreg[r][4 * m + 2] = x.z;
                qreg[r][4 * m + 3] = x.w;
            }
        } else {
            const uint16_t* qp = (const uint16_t*)a.q + (int64_t)rowid[r] * D;
#pragma unroll
            for (int m = 0; m < D / 32; ++m) {
                const int d0 =
                    kv == KV_FP8 ? 64 * (m / 2) + 16 * g + 8 * (m % 2) : 32 * m + 8 * g;
                qreg[r][m] = row_ok[r] ? *(const uint4*)(qp + d0) : make_uint4(0, 0, 0, 0);
            }
        }
    }

    // the last key position row tile r's row of this lane sees (-1: no row);
    // recomputed where a mask needs it rather than held through the loop
    auto pos_of = [&](int r) {
        const int qj = (16 * r + n) / G;
        return !row_ok[r] ? -1 : td.flags == TILE_GROUP ? L - 1 : L - nspan + td.qtok0 + qj;
    };

    // Online softmax with a lazily moved reference (log2 units): scores are
    // taken relative to m_use, the row maximum when the reference was last
    // moved, and p = 2^(s - m_use). The reference moves (rescaling o and l)
    // only when some score exceeds it by more than kLazy, so p <= 2^kLazy and
    // most blocks need neither a row reduction nor a rescale. thr is kLazy
    // once a row has a reference and -inf before its first visible key.
    constexpr float kLazy = 8.f;
    f32x4 o[NR][D / 16];
    float m_use[NR], thr[NR], l_run[NR];
    // fp8 P.V: o holds the output times osc, a power of two that keeps
    // p * v_scale * osc in the e4m3 range for p <= 2^kLazy; it follows the
    // blocks' V scales, and o is rescaled when it moves
    float osc[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) o[r][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        m_use[r] = 0.f;
        thr[r] = -INFINITY;
        l_run[r] = 0.f;
        osc[r] = 1.f;
    }
    // blocks ending at or before the tile's first query position are visible
    // to every row and lie inside the context: no masks
    const int pos_first = td.flags == TILE_GROUP ? L - 1
                          : tree                 ? span_start - 1
                                                 : L - nspan + td.qtok0;

    NewRow<kv, D> nrow;
    if (app) {
        constexpr int kEl = kv == KV_F32 ? 4 : 2;  // bytes of a new row's element
        const int64_t off = ((int64_t)(qs + td.qtok0) * Hkv + kvh) * D * kEl;
        nrow.load((const char*)a.k_new + off, (const char*)a.v_new + off, lane);
    }

    const int32_t* bt_row = a.block_tables + (int64_t)seq * a.max_blocks_per_seq;
    // blocks are taken in chunks of up to 64 NW, their ids (and fp8 scales)
    // held one per lane in NW registers; the ring drains at a chunk's end
    // and refills after the next chunk's ids arrive
    constexpr int NW = kFp8Cache ? PA_ID_WINDOWS_FP8 : PA_ID_WINDOWS;
    for (int c0 = 0; c0 < take; c0 += 64 * NW) {
        const int cnt = min(64 * NW, take - c0);
        // ids outside the pool are clamped into it: a wrong table gives
        // undefined results, never an out-of-bounds access
        int my_phys_w[NW];
        float my_ks_w[NW], my_vs_w[NW];
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            my_phys_w[w] = 0;
            my_ks_w[w] = my_vs_w[w] = 1.f;
            if (64 * w + lane < cnt)
                my_phys_w[w] =
                    min(max(bt_row[td.b0 + j + c0 + 64 * w + lane], 0), a.num_blocks - 1);
        }
        if constexpr (kFp8Cache) {
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                if (64 * w + lane < cnt) {
                    my_ks_w[w] = a.k_scale[(int64_t)my_phys_w[w] * Hkv + kvh];
                    my_vs_w[w] = a.v_scale[(int64_t)my_phys_w[w] * Hkv + kvh];
                }
            }
        }
        // the values of block i of the chunk (wave-uniform)
        // (each register read out, the scalar results selected: no register
        // is indexed by a runtime value)
        auto phys_of = [&](int i) {
            int x = __builtin_amdgcn_readlane(my_phys_w[0], i & 63);
#pragma unroll
            for (int w = 1; w < NW; ++w) {
                const int y = __builtin_amdgcn_readlane(my_phys_w[w], i & 63);
                x = (i >> 6) == w ? y : x;
            }
            return x;
        };
        auto scale_of = [&](const float (&arr)[NW], int i) {
            int x = __builtin_amdgcn_readlane(__builtin_bit_cast(int, arr[0]), i & 63);
#pragma unroll
            for (int w = 1; w < NW; ++w) {
                const int y = __builtin_amdgcn_readlane(__builtin_bit_cast(int, arr[w]), i & 63);
                x = (i >> 6) == w ? y : x;
            }
            return __builtin_bit_cast(float, x);
        };
        // per-block work on block i of the chunk
        auto consume_tile = [&](auto& cur, int i) {
            const int jb = td.b0 + j + c0 + i;  // logical block
            const int t0 = jb * 16 + 4 * g;  // my first token in it
            const bool full = jb * 16 + 15 <= pos_first;  // wave-uniform
            float c = kv == KV_FP8Q ? 1.f : a.scale_log2;
            float vsc = 1.f;
            if constexpr (kFp8Cache) {
                c *= scale_of(my_ks_w, i);
                vsc = scale_of(my_vs_w, i);
            }
            // The row tiles' steps are laid out phase by phase (all
            // products, all scores, one shared test for a reference move,
            // all weights, all P.V products), so the scheduler can overlap
            // one tile's matrix-core work with another's vector work.
            f32x4 sc[NR];
#pragma unroll
            for (int r = 0; r < NR; ++r) sc[r] = cur.qk(qreg[r]);
            float x[NR][4];  // scores relative to the reference
            float mx[NR];
            bool up = false;
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                const float cr = kv == KV_FP8Q ? c * qscale[r] : c;
#pragma unroll
                for (int e = 0; e < 4; ++e) x[r][e] = fmaf(sc[r][e], cr, -m_use[r]);
                if (!full) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int t = t0 + e, k = t - span_start;
                        const bool vis = t <= pos_of(r) && (k < 0 || ((tbits[r] >> (k & 63)) & 1u));
                        x[r][e] = vis ? x[r][e] : -INFINITY;
                    }
                }
                mx[r] = fmaxf(fmaxf(x[r][0], x[r][1]), fmaxf(x[r][2], x[r][3]));
                up |= mx[r] > thr[r];
            }
            if (__builtin_amdgcn_ballot_w64(up) != 0) {
#pragma unroll
                for (int r = 0; r < NR; ++r) {
                    if (__builtin_amdgcn_ballot_w64(mx[r] > thr[r]) == 0) continue;
                    // move the reference of the tile's rows up to their maxima
                    const float rm = row_max(mx[r]);
                    const bool had = thr[r] != -INFINITY;
                    const float delta = had ? fmaxf(rm, 0.f) : (rm == -INFINITY ? 0.f : rm);
                    const float alpha = had ? fexp2(-delta) : 1.f;  // o, l are 0 before
#pragma unroll
                    for (int e = 0; e < 4; ++e) x[r][e] -= delta;
                    m_use[r] += delta;
                    if (rm != -INFINITY) thr[r] = kLazy;
                    l_run[r] *= alpha;
#pragma unroll
                    for (int dt = 0; dt < D / 16; ++dt) o[r][dt] *= alpha;
                }
            }
            typename std::conditional<kv == KV_F32, float[NR][4],
                                      typename std::conditional<kv == KV_FP8Q, uint64_t[NR],
                                                                s16x4[NR]>::type>::type pk;
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                float p[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) p[e] = fexp2(x[r][e]);
                l_run[r] += (p[0] + p[1]) + (p[2] + p[3]);
                if constexpr (kv == KV_F32) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) pk[r][e] = p[e];
                } else if constexpr (kv == KV_FP8Q) {
                    // p <= 2^kLazy, so p * v_scale * osc <= 384 while
                    // v_scale * osc stays in [1/2, 3/2]; a block whose scale
                    // leaves that range moves osc to the nearest power of two
                    // of 1 / v_scale (wave-uniform)
                    float xs = vsc * osc[r];
                    if (vsc > 0.f && (xs > 1.5f || xs < 0.5f)) {
                        const float nsc = ldexpf(1.f, -(int)rintf(__log2f(vsc)));
                        const float ratio = nsc / osc[r];
#pragma unroll
                        for (int dt = 0; dt < D / 16; ++dt) o[r][dt] *= ratio;
                        osc[r] = nsc;
                        xs = vsc * nsc;
                    }
                    pk[r] = p_fp8_two_term(p, xs);
                } else {
                    const uint32_t lo = pack_bf16x2(p[0] * vsc, p[1] * vsc);
                    const uint32_t hi = pack_bf16x2(p[2] * vsc, p[3] * vsc);
                    pk[r] = __builtin_bit_cast(s16x4, make_uint2(lo, hi));
                }
            }
            // zero V slots past the context (NaN there must not reach P.V)
            if (!full) cur.mask_v(L - t0);
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                if constexpr (kv == KV_FP8Q)
                    cur.pv8(pk[r], o[r]);
                else
                    cur.pv(pk[r], o[r]);
            }
        };
        auto consume = [&](T& cur, int i) { consume_tile(cur, i); };
        // the chunk's last blocks: the segment's last block takes the step's
        // new token first
        auto consume_tail = [&](T& cur, int i) {
            if (app && c0 + i == take - 1) {
                float ks = 1.f, vs = 1.f;
                if constexpr (kFp8Cache) {
                    ks = scale_of(my_ks_w, i);
                    vs = scale_of(my_vs_w, i);
                }
                stage.add(a, cur, nrow, (L - 1) & 15, (int64_t)phys_of(i) * Hkv + kvh, ks, vs,
                          lane);
            }
            consume_tile(cur, i);
        };
        auto fetch = [&](T& dst, int i) {
            const int ph = phys_of(i);
            dst.template load<kStreamLoads>(a.k_cache, a.v_cache, (int64_t)ph * Hkv + kvh, lane);
        };
        constexpr int PF = kFp8Cache ? PA_PREFETCH_FP8 : PA_PREFETCH;
        // ring of PF + 1 register tiles: PF blocks stay in flight while one is
        // consumed. In the steady-state loop every refill is in range, so it
        // is straight-line code in which each wait covers exactly one block;
        // the last (at most 2 PF) blocks of the chunk are finished by a short
        // tail that refills only while blocks remain.
        T ring[PF + 1];
        // The chunk's fp8 block scales, loaded before the ring's first
        // blocks, are taken here, once. Left pending into the loop, their
        // read in every block step waited for all the loads in flight behind
        // them (the loop's entry and back edge disagree on how many follow
        // them), draining the ring once per block. (The query operands,
        // loaded at the segment's start, are older than every block of the
        // ring: the first step's wait covers them.)
        auto take_scales = [&]() {
            if constexpr (kFp8Cache) {
#pragma unroll
                for (int w = 0; w < NW; ++w) {
                    take_reg(my_ks_w[w]);
                    take_reg(my_vs_w[w]);
                }
            }
        };
        int i0 = 0;
        auto steady = [&]() {
            for (; i0 + 2 * PF < cnt; i0 += PF + 1) {
#pragma unroll
                for (int r = 0; r <= PF; ++r) {
                    fetch(ring[(r + PF) % (PF + 1)], i0 + r + PF);
                    // fp8: the refill is issued before the step waits for
                    // its block (the scheduler otherwise placed it after the
                    // wait for the block's K, so a wave stalled there had one
                    // block fewer in flight); the parallel-sampling pass
                    // measured 113-114 -> 111.7 us
                    if constexpr (kFp8Cache) __builtin_amdgcn_sched_barrier(0);
                    consume(ring[r], i0 + r);
                    // keep the steps in order: the scheduler would otherwise
                    // hoist later steps' products above their loads' waits
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        };
        // bf16 and f32: a chunk long enough for the steady loop fetches its
        // first PF blocks unconditionally and in order, and runs the loop
        // inside that branch. Entered after the conditional fetches (or with
        // the first block's loads scheduled after the second's), the loop's
        // head took the first block for the newest in flight and waited
        // for every load but the step's refill, draining the ring once per
        // loop step; with exact waits C2's pass went from 84.2 to 83.8 us
        // and C3's from 677 to 675 (alternating runs, each after a pause).
        // The fp8 loop's waits were already exact, and it measured slower.
        constexpr bool kOrdered = !kFp8Cache;
        if (kOrdered && cnt > 2 * PF) {
#pragma unroll
            for (int r = 0; r < PF; ++r) {
                fetch(ring[r], r);
                __builtin_amdgcn_sched_barrier(0);
            }
            take_scales();
            steady();
        } else {
#pragma unroll
            for (int r = 0; r < PF; ++r)
                if (r < cnt) fetch(ring[r], r);
            take_scales();
            if constexpr (!kOrdered) steady();
        }
#pragma unroll
        for (int r = 0; r <= 2 * PF; ++r) {
            const int i = i0 + r;
            if (i < cnt) {
                if (i + PF < cnt) fetch(ring[(r + PF) % (PF + 1)], i + PF);
                consume_tail(ring[r % (PF + 1)], i);
            }
        }
    }

    const bool whole = j == 0 && take == td.nb;
    const int64_t slot = (int64_t)piece * 2 + (j > 0 ? SLOT_HEAD : SLOT_TAIL);
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        // row totals: l summed over the four lane groups that share a row
        const float l = row_sum(l_run[r]);
        const float inv = l > 0.f ? (1.0f / l) * (1.0f / osc[r]) : 0.f;
        if (!row_ok[r]) continue;
        if (whole && td.flags != 0) {
            // a whole cascade part: normalized output and lse per row
            const int kind = td.flags == TILE_GROUP ? CAS_PRE : CAS_SUF;
            float* bo = a.cas_o[kind] + (int64_t)rowid[r] * D;
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt)
                *(float4*)(bo + 16 * dt + 4 * g) =
                    make_float4(o[r][dt][0] * inv, o[r][dt][1] * inv, o[r][dt][2] * inv,
                                o[r][dt][3] * inv);
            if (g == 0) a.cas_lse[kind][rowid[r]] = l > 0.f ? m_use[r] + __log2f(l) : -INFINITY;
        } else if (whole) {
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt) {
                const int d = 16 * dt + 4 * g;
                if constexpr (kv == KV_F32) {
                    *(float4*)((float*)a.out + (int64_t)rowid[r] * D + d) =
                        make_float4(o[r][dt][0] * inv, o[r][dt][1] * inv, o[r][dt][2] * inv,
                                    o[r][dt][3] * inv);
                } else {
                    uint2 w;
                    w.x = pack_bf16x2(o[r][dt][0] * inv, o[r][dt][1] * inv);
                    w.y = pack_bf16x2(o[r][dt][2] * inv, o[r][dt][3] * inv);
                    *(uint2*)((uint16_t*)a.out + (int64_t)rowid[r] * D + d) = w;
                }
            }
            if (a.lse && g == 0)
                a.lse[rowid[r]] = l > 0.f ? (m_use[r] + __log2f(l)) * kLn2 : -INFINITY;
        } else {
            // partials keep the accumulator's register layout:
            // [slot][r][dt][lane] float4, one contiguous kilobyte per store
            float4* po = (float4*)a.part_o + ((slot * NT + r) * (D / 16)) * 64 + lane;
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt)
                po[dt * 64] = make_float4(o[r][dt][0] * inv, o[r][dt][1] * inv,
                                          o[r][dt][2] * inv, o[r][dt][3] * inv);
            if (g == 0)
                a.part_lse[slot * (16 * NT) + 16 * r + n] =
                    l > 0.f ? m_use[r] + __log2f(l) : -INFINITY;
        }
    }
}

// One wave per workgroup; wave w streams pieces w, w + grid, ... of the
// narrow stream (NR = 1) or of the group stream (NR = kGroupRowTiles).
template <int kv, int D, int NR>
__device__ __forceinline__ void narrow_pieces(const AttnArgs& a, NewStage<kv, D>& stage) {
    const int* h = a.hdr + HDR_STREAM + 4 * a.stream;
    const int V = h[HDR_NPIECES];
    for (int v = blockIdx.x; v < V; v += gridDim.x) {
        const PieceStart ps = a.pieces[v];
        int t = ps.tile, j = ps.j;
        const int kvh = ps.kvh;
        TileDesc td = ps.td;
        int left = ps.nblocks;  // the piece's blocks, within its KV head's substream
        while (left > 0) {
            const int take = min(left, td.nb - j);
            // a decode's context and a cascade member's suffix are read by no
            // other tile of the call, so they are streamed past the caches
            if (PA_GROUP_L2 && td.flags == TILE_GROUP)
                run_segment<kv, D, false, NR>(a, td, kvh, j, take, v, stage);
            else
                run_segment<kv, D, PA_NT_LOADS != 0, NR>(a, td, kvh, j, take, v, stage);
            left -= take;
            j = 0;
            ++t;
            if (left > 0) td = a.tiles[t];
        }
    }
}

// LDS stage of the new keys a wave appends (decode with append).
#define PA_NEW_STAGE(kv, D, stage)                                       \
    using E_ = typename NewStage<kv, D>::E;                              \
    constexpr int kMax_ = NewStage<kv, D>::kMax;                         \
    __shared__ __align__(16) E_ s_new_k[kMax_ * D];                      \
    __shared__ __align__(16) E_ s_new_v[kMax_ * D];                      \
    __shared__ int64_t s_new_bh[kMax_];                                  \
    __shared__ int s_new_o[kMax_];                                       \
    NewStage<kv, D> stage;                                               \
    stage.k = s_new_k;                                                   \
    stage.v = s_new_v;                                                   \
    stage.bh = s_new_bh;                                                 \
    stage.o = s_new_o

// Single-token tiles: bound by HBM. PA_NARROW_MIN_WAVES > 0 would make the
// compiler budget registers for that many waves per SIMD.
#ifndef PA_NARROW_MIN_WAVES
#define PA_NARROW_MIN_WAVES 0
#endif
#if PA_NARROW_MIN_WAVES > 0
#define PA_NARROW_OCCUPANCY __attribute__((amdgpu_waves_per_eu(PA_NARROW_MIN_WAVES, 8)))
#else
#define PA_NARROW_OCCUPANCY
#endif

// One wave per workgroup; wave w takes pieces w, w + grid, ... of a.stream:
// the narrow stream (NR = 1) or the group stream (NR = kGroupRowTiles).
template <int kv, int D, int NR>
__global__ __launch_bounds__(64) PA_NARROW_OCCUPANCY void attention_narrow(AttnArgs a) {
    PA_NEW_STAGE(kv, D, stage);
    narrow_pieces<kv, D, NR>(a, stage);
    stage.flush(a, threadIdx.x & 63);  // decode with append: the staged cache writes
}

// A decode batch with shared-prefix groups: one launch in which each wave
// takes its pieces of the group stream, then its pieces of the narrow
// stream (the members' suffixes and the other decodes), rather than a
// launch per stream. Both streams are cut for the same waves.
template <int kv, int D>
__global__ __launch_bounds__(64) PA_NARROW_OCCUPANCY void attention_narrow_pair(AttnArgs g,
                                                                               AttnArgs n) {
    PA_NEW_STAGE(kv, D, stage);
    narrow_pieces<kv, D, kGroupRowTiles>(g, stage);
    narrow_pieces<kv, D, 1>(n, stage);
    stage.flush(n, threadIdx.x & 63);
}

// ---- merge -------------------------------------------------------------------

// Second pass: one wave per cut segment combines its pieces' partial results
// by log-sum-exp: M = max_p lse_p, out = sum_p 2^(lse_p - M) o_p / sum_p
// 2^(lse_p - M) ("03 -- Engines Papers", section 12; playbook Theme 4),
// taken four pieces at a time with a running rescale so that one round trip
// of loads covers the usual two to four pieces. Lanes keep the attention
// kernel's accumulator layout (row lane % 16, dims 16dt + 4(lane / 16) + i).
// Log-sum-exp combination of partial results for one query row, fed one
// part at a time: (lse in log2 units, normalized output dims of this lane).
template <int D>
struct LseAcc {
    float M = -INFINITY, W = 0.f;
    float4 acc[D / 16];
    __device__ LseAcc() {
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) acc[dt] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    __device__ __forceinline__ void add(float l, const float4* x) {
        if (l == -INFINITY) return;
        const float m = fmaxf(M, l);
        const float r = M == -INFINITY ? 0.f : fexp2(M - m);
        const float w = fexp2(l - m);
        W = W * r + w;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
            acc[dt].x = acc[dt].x * r + w * x[dt].x;
            acc[dt].y = acc[dt].y * r + w * x[dt].y;
            acc[dt].z = acc[dt].z * r + w * x[dt].z;
            acc[dt].w = acc[dt].w * r + w * x[dt].w;
        }
        M = m;
    }
};

// Writes a merged row: out (the q dtype) and lse (natural log).
template <int qd, int D>
__device__ __forceinline__ void write_row(const MergeArgs& a, int64_t row, int g, float M,
                                          float W, const float4* acc) {
    const float inv = W > 0.f ? 1.0f / W : 0.f;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
        const int d = 16 * dt + 4 * g;
        if constexpr (qd == PA_F32) {
            *(float4*)((float*)a.out + row * D + d) =
                make_float4(acc[dt].x * inv, acc[dt].y * inv, acc[dt].z * inv, acc[dt].w * inv);
        } else {
            uint2 w;
            w.x = pack_bf16x2(acc[dt].x * inv, acc[dt].y * inv);
            w.y = pack_bf16x2(acc[dt].z * inv, acc[dt].w * inv);
            *(uint2*)((uint16_t*)a.out + row * D + d) = w;
        }
    }
    if (a.lse && g == 0) a.lse[row] = W > 0.f ? (M + __log2f(W)) * kLn2 : -INFINITY;
}

// A cascade member's rows (G, one per query head of its KV head): the
// prefix part and the suffix part, each either one whole part in the
// per-row buffers or the slots of the pieces that cut it.
template <int qd, int D>
__device__ __forceinline__ void merge_cascade(const MergeArgs& a, const CascadeRec rc) {
    const int lane = threadIdx.x & 63;
    const int n = lane & 15, g = lane >> 4;
    const int G = a.group, Hkv = a.num_kv_heads;
    if (n >= G) return;
    const int64_t row = (int64_t)rc.row * a.num_q_heads + rc.kvh * G + n;
    LseAcc<D> acc;
    float4 x[D / 16];
    for (int kind = CAS_PRE; kind <= CAS_SUF; ++kind) {
        const int k0 = kind == CAS_PRE ? rc.pre_k0 : rc.suf_k0;
        const int k1 = kind == CAS_PRE ? rc.pre_k1 : rc.suf_k1;
        if (k0 == k1) {  // read whole by one piece
            const float* bo = a.cas_o[kind] + row * D;
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt) x[dt] = *(const float4*)(bo + 16 * dt + 4 * g);
            acc.add(a.cas_lse[kind][row], x);
            continue;
        }
        // group tiles hold kGroupRowTiles 16-row tiles per slot, suffix
        // tiles one
        const int st = kind == CAS_PRE ? STREAM_GROUP : STREAM_NARROW;
        const int nt = slot_row_tiles(st);
        const int rr = (kind == CAS_PRE ? rc.pre_pos * G : 0) + n;  // row in the slot
        const float4* po = (const float4*)a.part_o[st];
        // four pieces per round trip: all their loads are issued first
        for (int kb = k0; kb <= k1; kb += 4) {
            float l4[4];
            float4 x4[4][D / 16];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int k = min(kb + u, k1);
                const int64_t sl =
                    ((int64_t)k * Hkv + rc.kvh) * 2 + (k == k0 ? SLOT_TAIL : SLOT_HEAD);
                const float4* p = po + ((sl * nt + rr / 16) * (D / 16)) * 64 + (rr % 16) + 16 * g;
#pragma unroll
                for (int dt = 0; dt < D / 16; ++dt) x4[u][dt] = p[dt * 64];
                l4[u] = kb + u <= k1 ? a.part_lse[st][sl * (16 * nt) + rr] : -INFINITY;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) acc.add(l4[u], x4[u]);
        }
    }
    write_row<qd, D>(a, row, g, acc.M, acc.W, acc.acc);
}

// One workgroup per record; a wide segment's row tiles are shared among the
// workgroup's waves (one wave for the others).
template <int qd, int D>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
    const int wave = (int)threadIdx.x >> 6, nwaves = (int)blockDim.x >> 6;
    if ((int)blockIdx.x >= a.max_splits) {
        const int c = (int)blockIdx.x - a.max_splits;
        if (wave == 0 && c < a.hdr[HDR_NCAS]) merge_cascade<qd, D>(a, a.cas_recs[c]);
        return;
    }
    const SplitSeg sp = a.splits[blockIdx.x];
    if (sp.k0 < 0) return;  // past the list of cut segments
    const int lane = threadIdx.x & 63;
    const int n = lane & 15, g = lane >> 4;  // the attention kernel's layout
    const int G = a.group;
    const int nt = slot_row_tiles(sp.stream);  // row tiles per slot
    const float* part_lse = a.part_lse[sp.stream];
    const float4* part_o = (const float4*)a.part_o[sp.stream];
    const int Hkv = a.num_kv_heads;
    // slot of the segment's k-th piece (k0: the tail it left unfinished)
    auto slot_of = [&](int k) {
        return ((int64_t)k * Hkv + sp.kvh) * 2 + (k == sp.k0 ? SLOT_TAIL : SLOT_HEAD);
    };
    for (int r = wave; r < nt; r += nwaves) {
        const int rr = 16 * r + n;
        if (rr >= sp.ntok * G) break;  // rows past the tile hold no partials
        float M = -INFINITY, W = 0.f;
        float4 acc[D / 16];
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) acc[dt] = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int k = sp.k0; k <= sp.k1; k += 4) {
            // all four pieces' values are requested before any is used
            float l4[4];
            float4 x[4][D / 16];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const bool ok = k + u <= sp.k1;
                const int64_t sl = slot_of(ok ? k + u : sp.k1);
                l4[u] = ok ? part_lse[sl * (16 * nt) + rr] : -INFINITY;
                const float4* po = part_o + ((sl * nt + r) * (D / 16)) * 64 + lane;
#pragma unroll
                for (int dt = 0; dt < D / 16; ++dt) x[u][dt] = po[dt * 64];
            }
            // fold the group into the running (M, W, acc) with one rescale
            float m4 = M;
#pragma unroll
            for (int u = 0; u < 4; ++u) m4 = fmaxf(m4, l4[u]);
            const float rescale = M == -INFINITY ? 0.f : fexp2(M - m4);
            W *= rescale;
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt) {
                acc[dt].x *= rescale;
                acc[dt].y *= rescale;
                acc[dt].z *= rescale;
                acc[dt].w *= rescale;
            }
            M = m4;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float w = l4[u] == -INFINITY ? 0.f : fexp2(l4[u] - M);
                W += w;
#pragma unroll
                for (int dt = 0; dt < D / 16; ++dt) {
                    acc[dt].x += w * x[u][dt].x;
                    acc[dt].y += w * x[u][dt].y;
                    acc[dt].z += w * x[u][dt].z;
                    acc[dt].w += w * x[u][dt].w;
                }
            }
        }
        const float inv = W > 0.f ? 1.0f / W : 0.f;
        const int mj = rr / G;
        const int64_t row = (int64_t)(sp.row0 + mj) * a.num_q_heads + sp.kvh * G + (rr - mj * G);
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
            const int d = 16 * dt + 4 * g;
            if constexpr (qd == PA_F32) {
                *(float4*)((float*)a.out + row * D + d) = make_float4(
                    acc[dt].x * inv, acc[dt].y * inv, acc[dt].z * inv, acc[dt].w * inv);
            } else {
                uint2 w;
                w.x = pack_bf16x2(acc[dt].x * inv, acc[dt].y * inv);
                w.y = pack_bf16x2(acc[dt].z * inv, acc[dt].w * inv);
                *(uint2*)((uint16_t*)a.out + row * D + d) = w;
            }
        }
        if (a.lse && g == 0) a.lse[row] = W > 0.f ? (M + __log2f(W)) * kLn2 : -INFINITY;
    }
}

// The attention kernels' e4m3 conversion, one byte per thread, widened to
// float32 (exact: bf16 is a prefix of float32).
__global__ void fp8_decode_kernel(const uint8_t* in, float* out, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    out[i] = __uint_as_float(fp8x2_to_bf16x2<false>((uint32_t)in[i]) << 16);
}

// ---- launch configuration ----------------------------------------------------

// Waves per SIMD of the persistent narrow grid (0: as many as fit). Its
// registers would allow two or three. One wave per SIMD with two blocks in
// flight beyond the one in use measured fastest: half the pieces of two
// waves per SIMD, so fewer segments are cut (a cheaper merge) and fewer
// waves restart their block ring at a segment boundary. With registers
// budgeted for two waves per SIMD and twice the grid (alternating runs, each
// after a pause): Llama-3-8B-shaped decode 83.5 -> 97.6 us, long-context
// 675 -> 725 us, fp8 parallel sampling 110.5 -> 113.6 us.
#ifndef PA_NARROW_MAX_WAVES
#define PA_NARROW_MAX_WAVES 1
#endif

template <typename K>
int resident_waves_of(K kernel, int cap_per_simd) {
    int dev = 0, num_cu = 0, occ = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&num_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, 64, 0) != hipSuccess)
        return 0;
    if (cap_per_simd > 0 && occ > 4 * cap_per_simd) occ = 4 * cap_per_simd;
    return (occ > 0 ? occ : 1) * num_cu;
}

// Resident waves per (kernel instance, device), queried once per
// device and kept for the life of the process. The value depends only on
// the kernel's resources and the device's compute-unit count, so threads
// that race on a first query compute the same number; the table is atomic
// so that such a race is well defined, and the first value stored is the
// one every later call sees. Devices past kMaxDevices are queried each call.
constexpr int kMaxDevices = 64;
template <int kv, int D>
int resident_waves_d() {
    static std::atomic<int> cached[kMaxDevices];  // 0: not yet queried
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
    std::atomic<int>* slot = dev < kMaxDevices ? &cached[dev] : nullptr;
    if (slot) {
        const int c = slot->load(std::memory_order_acquire);
        if (c > 0) return c;
    }
    const int w = resident_waves_of(attention_narrow<kv, D, 1>, PA_NARROW_MAX_WAVES);
    if (w <= 0) return 0;
    if (!slot) return w;
    int expected = 0;
    slot->compare_exchange_strong(expected, w, std::memory_order_acq_rel);
    return slot->load(std::memory_order_acquire);
}

template <int kv, int D>
hipError_t launch_narrow_d(const AttnArgs& a, int64_t max_pieces, hipStream_t s) {
    int64_t grid = resident_waves_d<kv, D>();
    if (grid <= 0) return hipErrorInvalidDevice;
    if (max_pieces < grid) grid = max_pieces;
    if (grid < 1) grid = 1;
    if (a.stream == STREAM_GROUP)
        hipLaunchKernelGGL((attention_narrow<kv, D, kGroupRowTiles>), dim3((unsigned)grid),
                           dim3(64), 0, s, a);
    else
        hipLaunchKernelGGL((attention_narrow<kv, D, 1>), dim3((unsigned)grid), dim3(64), 0, s, a);
    return hipGetLastError();
}

template <int kv, int D>
hipError_t launch_narrow_pair_d(const AttnArgs& g, const AttnArgs& n, int64_t max_pieces,
                                hipStream_t s) {
    int64_t grid = resident_waves_d<kv, D>();
    if (grid <= 0) return hipErrorInvalidDevice;
    if (max_pieces < grid) grid = max_pieces;
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL((attention_narrow_pair<kv, D>), dim3((unsigned)grid), dim3(64), 0, s, g, n);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_narrow_pair(int kind, int head_dim, const AttnArgs& g, const AttnArgs& n,
                              int64_t max_pieces, hipStream_t s) {
    switch (kind * 1000 + head_dim) {
    case PA_F32 * 1000 + 64: return launch_narrow_pair_d<KV_F32, 64>(g, n, max_pieces, s);
    case PA_F32 * 1000 + 128: return launch_narrow_pair_d<KV_F32, 128>(g, n, max_pieces, s);
    case PA_BF16 * 1000 + 64: return launch_narrow_pair_d<KV_BF16, 64>(g, n, max_pieces, s);
    case PA_BF16 * 1000 + 128: return launch_narrow_pair_d<KV_BF16, 128>(g, n, max_pieces, s);
    case PA_FP8_E4M3FN * 1000 + 64: return launch_narrow_pair_d<KV_FP8, 64>(g, n, max_pieces, s);
    case PA_FP8_E4M3FN * 1000 + 128: return launch_narrow_pair_d<KV_FP8, 128>(g, n, max_pieces, s);
    case KIND_FP8_QK * 1000 + 64: return launch_narrow_pair_d<KV_FP8Q, 64>(g, n, max_pieces, s);
    case KIND_FP8_QK * 1000 + 128: return launch_narrow_pair_d<KV_FP8Q, 128>(g, n, max_pieces, s);
    default: return hipErrorInvalidValue;
    }
}

int resident_waves(int kind, int head_dim, int stream) {
    if (stream == STREAM_WIDE) return span_resident_groups(kind, head_dim);
    switch (kind * 1000 + head_dim) {
    case PA_F32 * 1000 + 64: return resident_waves_d<KV_F32, 64>();
    case PA_F32 * 1000 + 128: return resident_waves_d<KV_F32, 128>();
    case PA_BF16 * 1000 + 64: return resident_waves_d<KV_BF16, 64>();
    case PA_BF16 * 1000 + 128: return resident_waves_d<KV_BF16, 128>();
    case PA_FP8_E4M3FN * 1000 + 64: return resident_waves_d<KV_FP8, 64>();
    case PA_FP8_E4M3FN * 1000 + 128: return resident_waves_d<KV_FP8, 128>();
    case KIND_FP8_QK * 1000 + 64: return resident_waves_d<KV_FP8Q, 64>();
    case KIND_FP8_QK * 1000 + 128: return resident_waves_d<KV_FP8Q, 128>();
    default: return 0;
    }
}

hipError_t launch_plan(const PlanArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_attention(int kind, int head_dim, const AttnArgs& a, int64_t max_pieces,
                            hipStream_t s) {
    if (a.stream == STREAM_WIDE) return launch_span(kind, head_dim, a, max_pieces, s);
    switch (kind * 1000 + head_dim) {
    case PA_F32 * 1000 + 64: return launch_narrow_d<KV_F32, 64>(a, max_pieces, s);
    case PA_F32 * 1000 + 128: return launch_narrow_d<KV_F32, 128>(a, max_pieces, s);
    case PA_BF16 * 1000 + 64: return launch_narrow_d<KV_BF16, 64>(a, max_pieces, s);
    case PA_BF16 * 1000 + 128: return launch_narrow_d<KV_BF16, 128>(a, max_pieces, s);
    case PA_FP8_E4M3FN * 1000 + 64: return launch_narrow_d<KV_FP8, 64>(a, max_pieces, s);
    case PA_FP8_E4M3FN * 1000 + 128: return launch_narrow_d<KV_FP8, 128>(a, max_pieces, s);
    case KIND_FP8_QK * 1000 + 64: return launch_narrow_d<KV_FP8Q, 64>(a, max_pieces, s);
    case KIND_FP8_QK * 1000 + 128: return launch_narrow_d<KV_FP8Q, 128>(a, max_pieces, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_merge(int q_dtype, int head_dim, const MergeArgs& a, int64_t records,
                        bool wide, hipStream_t s) {
    if (records <= 0) return hipSuccess;
    // a wide segment's eight row tiles go to four waves
    const dim3 grid((unsigned)records), block(wide ? 256 : 64);
    if (q_dtype == PA_F32 && head_dim == 64)
        hipLaunchKernelGGL((merge_kernel<PA_F32, 64>), grid, block, 0, s, a);
    else if (q_dtype == PA_F32 && head_dim == 128)
        hipLaunchKernelGGL((merge_kernel<PA_F32, 128>), grid, block, 0, s, a);
    else if (q_dtype == PA_BF16 && head_dim == 64)
        hipLaunchKernelGGL((merge_kernel<PA_BF16, 64>), grid, block, 0, s, a);
    else if (q_dtype == PA_BF16 && head_dim == 128)
        hipLaunchKernelGGL((merge_kernel<PA_BF16, 128>), grid, block, 0, s, a);
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
