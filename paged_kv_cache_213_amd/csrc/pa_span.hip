// pa_span.hip -- the chunked-prefill span kernel for gfx950 (MI355X).
//
// A chunked-prefill span is a dense contraction: every query row of a tile
// meets every key block before it (causally), so unlike a decode the K/V
// bytes a tile reads can serve many rows at once ("03 -- Engines Papers",
// section 3: chunks co-scheduled with decodes in one hybrid batch; the
// FlashAttention entry of "References": tiling through on-chip memory with
// an online softmax; playbook Theme 4: the work partition of FlashAttention-2
// across warps and thread blocks).
//
// One workgroup of kSpanWaves waves owns a tile of up to kSpanRows query
// rows (the G heads of kSpanRows / G consecutive tokens of one span, one KV
// head); each wave owns RT of its 16-row matrix-core tiles. The
// workgroup walks the tile's key blocks KB at a time: all of its threads
// gather the KB blocks' K and V through the block table (ordinary loads, so
// the tiles of one span also share blocks through L2), convert them to
// bf16, and store them in LDS; every wave then computes
//   S^T = K Q^T   on v_mfma_f32_16x16x32_bf16 (K from LDS, Q in registers)
//   online softmax of its rows (lazily moved reference, as the narrow kernel)
//   O^T += V^T P^T on v_mfma_f32_16x16x32_bf16 (V from LDS, P from S)
// The S^T result layout of two 16-key tiles (keys 4g + i and 16 + 4g + i in
// lane n + 16g) is the B-operand layout of a 32-key contraction once the V
// operand is read with the same key order, so P never leaves registers. The
// next step's K/V are loaded into registers while the current step
// computes, and written to the other LDS buffer after it: one barrier per
// step. Causal masks apply only on steps that reach past a wave's first
// query position; waves whose rows all lie before a step skip it.
//
// Pieces, partial slots and the merge are those of the narrow kernel (the
// plan cuts each stream of key blocks into balanced pieces; a cut segment's
// pieces write (lse, normalized o) per row and the merge pass combines
// them), with kSpanRowTiles 16-row tiles per slot.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <atomic>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

using namespace dev;

// 16-token blocks per LDS step (a step holds 16 * KB keys).
#ifndef PA_SPAN_BLOCKS
#define PA_SPAN_BLOCKS 2
#endif
constexpr int KB = PA_SPAN_BLOCKS;
static_assert(KB == 2 || KB == 4, "steps hold pairs of blocks");
// Steps whose global loads are in flight while a step computes (register
// sets of loaded K/V; the LDS stays double-buffered).
#ifndef PA_SPAN_PREFETCH
#define PA_SPAN_PREFETCH 2
#endif
constexpr int PF = PA_SPAN_PREFETCH;
static_assert(PF == 1 || PF == 2, "one or two steps ahead");
constexpr int kThreads = 64 * kSpanWaves;
constexpr int RT = kSpanRowTiles / kSpanWaves;  // 16-row tiles per wave
constexpr int kWaveRows = 16 * RT;

// LDS image of one step (bf16), per buffer:
//   K  [16 KB rows][D / 8 units of 16 bytes]: unit u of row t is stored at
//      position u ^ (t mod D/8), so the 16 rows one matrix-core read touches
//      fall in different banks
//   V  [KB / 2 block pairs][D rows][4 units]: unit g of row d holds keys
//      4g .. 4g+3 of the pair's first block (low 8 bytes) and of its second
//      block (high 8 bytes), the key order of the P operand; stored at
//      position g ^ ((d / 4) mod 4)
//   per-block fp8 scales: k_scale[KB], v_scale[KB]
template <int D>
struct SpanLds {
    static constexpr int kUnitsPerRow = D / 8;
    static constexpr int kKBytes = KB * 16 * D * 2;
    static constexpr int kVBytes = KB * 16 * D * 2;
    static constexpr int kScaleOff = kKBytes + kVBytes;
    static constexpr int kBufBytes = kScaleOff + 2 * KB * 4 + (16 - (2 * KB * 4) % 16) % 16;
    __device__ static int k_unit(int row, int u) {
        return (row * kUnitsPerRow + (u ^ (row & (kUnitsPerRow - 1)))) * 16;
    }
    __device__ static int v_unit(int pair, int d, int g) {
        return kKBytes + ((pair * D + d) * 4 + (g ^ ((d >> 2) & 3))) * 16;
    }
};

// Global loads of one step, held in registers until the LDS write. For a
// bf16 cache a thread moves 16-byte units of K rows and of V rows (8 keys);
// for an fp8 cache, 16-byte units of 16 dims of a K row and whole V rows
// (16 keys), converted to bf16 when written.
template <int kv, int D>
struct StepRegs {
    static constexpr bool kFp8 = kv == KV_FP8 || kv == KV_FP8Q;
    static constexpr int kKUnits = kFp8 ? KB * D : KB * 16 * (D / 8);
    static constexpr int kVUnits = kFp8 ? KB * D : KB * D * 2;
    static constexpr int kKPer = (kKUnits + kThreads - 1) / kThreads;
    static constexpr int kVPer = (kVUnits + kThreads - 1) / kThreads;
    uint4 k[kKPer];
    uint4 v[kVPer];
    float ks, vs;  // this thread's block scale (threads < KB, fp8)
};

template <int kv, int D>
struct SpanStep {
    using L = SpanLds<D>;
    using Regs = StepRegs<kv, D>;
    static constexpr bool kFp8 = Regs::kFp8;
    // units of one block in each region: a multiple of 64, so the block of a
    // unit is the same for every lane of a wave
    static constexpr int kKPerBlock = Regs::kKUnits / KB;
    static constexpr int kVPerBlock = Regs::kVUnits / KB;
    static_assert(kKPerBlock % 64 == 0 && kVPerBlock % 64 == 0, "wave-uniform blocks");

    // Issue the loads of the step's blocks (nblk of KB present); ids: the
    // physical block of chunk block `lane`, with `base` the step's first
    // block within the chunk. Every call issues the same loads, in range:
    // units of absent blocks (and of a step past the segment, nblk <= 0)
    // re-read a present block or the chunk's first, and a wave past the
    // last unit re-reads one; their data is never written to LDS. With a
    // fixed number of loads per step the compiler's wait counts can let
    // the next steps' loads stay in flight while a step computes.
    __device__ static void issue(Regs& r, const AttnArgs& a, int kvh, int ids, int base,
                                 int nblk, int tid, int wave) {
        const int Hkv = a.num_kv_heads;
        const int last = nblk > 0 ? nblk - 1 : 0;
        constexpr int kBlockBytes = 16 * D * (kFp8 ? 1 : 2);
#pragma unroll
        for (int i = 0; i < Regs::kKPer; ++i) {
            const int ku0 = (wave * 64 + kThreads * i) % Regs::kKUnits;  // the wave's first unit
            const int ku = (tid + kThreads * i) % Regs::kKUnits;
            const int b = min(ku0 / kKPerBlock, last);  // wave-uniform
            const int64_t bh = (int64_t)__builtin_amdgcn_readlane(ids, base + b) * Hkv + kvh;
            r.k[i] = *(const uint4*)((const uint8_t*)a.k_cache + bh * kBlockBytes +
                                     (int64_t)(ku % kKPerBlock) * 16);
        }
#pragma unroll
        for (int i = 0; i < Regs::kVPer; ++i) {
            const int vu0 = (wave * 64 + kThreads * i) % Regs::kVUnits;
            const int vu = (tid + kThreads * i) % Regs::kVUnits;
            const int b = min(vu0 / kVPerBlock, last);
            const int64_t bh = (int64_t)__builtin_amdgcn_readlane(ids, base + b) * Hkv + kvh;
            r.v[i] = *(const uint4*)((const uint8_t*)a.v_cache + bh * kBlockBytes +
                                     (int64_t)(vu % kVPerBlock) * 16);
        }
        if constexpr (kFp8) {
            // every lane reads the scales of step block lane % KB (lanes
            // 0 .. KB-1 of wave 0 write them)
            const int lb = min((tid & 63) % KB, last);
            const int64_t bh = (int64_t)__shfl(ids, base + lb) * Hkv + kvh;
            r.ks = a.k_scale[bh];
            r.vs = a.v_scale[bh];
        }
    }

    // Write the loaded step into an LDS buffer: V values of keys at or past
    // the context length L, and every value of absent blocks, become zero
    // (a NaN left in an unused slot must not reach P.V).
    __device__ static void commit(uint8_t* buf, const Regs& r, int jb0, int L, int nblk, int tid,
                                  int wave) {
#pragma unroll
        for (int i = 0; i < Regs::kKPer; ++i) {
            const int ku0 = wave * 64 + kThreads * i;
            const int ku = tid + kThreads * i;
            const int b = ku0 / kKPerBlock;
            if (ku0 >= Regs::kKUnits) continue;
            const int w = ku % kKPerBlock;
            if constexpr (!kFp8) {
                const int t = w / (D / 8), u = w % (D / 8);
                const uint4 x = b < nblk ? r.k[i] : make_uint4(0, 0, 0, 0);
                *(uint4*)(buf + L::k_unit(b * 16 + t, u)) = x;
            } else {
                const int t = w / (D / 16), u16 = w % (D / 16);
                const uint4 x = b < nblk ? r.k[i] : make_uint4(0, 0, 0, 0);
                uint4 lo, hi;
                lo.x = fp8x2_to_bf16x2<false>(x.x);
                lo.y = fp8x2_to_bf16x2<true>(x.x);
                lo.z = fp8x2_to_bf16x2<false>(x.y);
                lo.w = fp8x2_to_bf16x2<true>(x.y);
                hi.x = fp8x2_to_bf16x2<false>(x.z);
                hi.y = fp8x2_to_bf16x2<true>(x.z);
                hi.z = fp8x2_to_bf16x2<false>(x.w);
                hi.w = fp8x2_to_bf16x2<true>(x.w);
                *(uint4*)(buf + L::k_unit(b * 16 + t, 2 * u16)) = lo;
                *(uint4*)(buf + L::k_unit(b * 16 + t, 2 * u16 + 1)) = hi;
            }
        }
#pragma unroll
        for (int i = 0; i < Regs::kVPer; ++i) {
            const int vu0 = wave * 64 + kThreads * i;
            const int vu = tid + kThreads * i;
            const int b = vu0 / kVPerBlock;
            if (vu0 >= Regs::kVUnits) continue;
            const int w = vu % kVPerBlock;
            const int pair = b >> 1, half = b & 1;
            const int key0 = (jb0 + b) * 16;  // the block's first key
            if constexpr (!kFp8) {
                // keys 8h .. 8h+7 of dim row d
                const int d = w >> 1, h = w & 1;
                uint4 x = b < nblk ? r.v[i] : make_uint4(0, 0, 0, 0);
                const int nvalid = L - (key0 + 8 * h);  // keys of the 8 still in the context
                if (nvalid < 8) {
                    uint32_t e[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const uint32_t lo = 2 * q < nvalid ? 0x0000ffffu : 0u;
                        const uint32_t hi = 2 * q + 1 < nvalid ? 0xffff0000u : 0u;
                        e[q] &= lo | hi;
                    }
                    x = make_uint4(e[0], e[1], e[2], e[3]);
                }
                *(uint2*)(buf + L::v_unit(pair, d, 2 * h) + 8 * half) = make_uint2(x.x, x.y);
                *(uint2*)(buf + L::v_unit(pair, d, 2 * h + 1) + 8 * half) = make_uint2(x.z, x.w);
            } else {
                // all 16 keys of dim row d
                const int d = w;
                uint4 x = b < nblk ? r.v[i] : make_uint4(0, 0, 0, 0);
                const int nvalid = L - key0;
                if (nvalid < 16) {
                    uint32_t e[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int nv = nvalid - 4 * q;
                        e[q] &= nv >= 4 ? 0xffffffffu : (nv <= 0 ? 0u : ((1u << (8 * nv)) - 1u));
                    }
                    x = make_uint4(e[0], e[1], e[2], e[3]);
                }
                const uint32_t e[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    *(uint2*)(buf + L::v_unit(pair, d, g) + 8 * half) =
                        make_uint2(fp8x2_to_bf16x2<false>(e[g]), fp8x2_to_bf16x2<true>(e[g]));
            }
        }
        if constexpr (kFp8) {
            if (tid < KB) {
                float* sc = (float*)(buf + L::kScaleOff);
                sc[tid] = tid < nblk ? r.ks : 1.f;
                sc[KB + tid] = tid < nblk ? r.vs : 1.f;
            }
        }
    }
};

// Blocks [j, j + take) of span segment (tile td, KV head kvh), by the whole
// workgroup. Then each wave writes its rows' output (the workgroup saw the
// whole segment) or a partial result into the piece's slot.
template <int kv, int D>
__device__ __forceinline__ void span_segment(const AttnArgs& a, uint8_t* smem, const TileDesc td,
                                             const int kvh, const int j, const int take,
                                             const int piece) {
    using L = SpanLds<D>;
    using Step = SpanStep<kv, D>;
    constexpr bool kFp8 = Step::kFp8;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15, g = lane >> 4;
    const int G = a.group, Hq = a.num_q_heads;
    const int L_ = td.L, qs = td.qs, nspan = td.nspan;
    const int nrows = td.ntok * G;
    const int span_start = L_ - nspan;
    const bool tree = nspan <= 64 && a.hdr[HDR_TREE] != 0;

    // this wave's rows: kWaveRows wave + 16 r + n
    uint4 qreg[RT][D / 32];
    int rowid[RT];
    bool row_ok[RT];
    uint64_t tbits[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r) {
        const int rr = kWaveRows * wave + 16 * r + n;
        const int qj = rr / G;
        row_ok[r] = rr < nrows;
        rowid[r] = (qs + td.qtok0 + qj) * Hq + kvh * G + (rr - qj * G);
        tbits[r] = (tree && row_ok[r]) ? a.tree[qs + td.qtok0 + qj] : ~0ull;
        const uint16_t* qp = (const uint16_t*)a.q + (int64_t)(row_ok[r] ? rowid[r] : 0) * D;
#pragma unroll
        for (int m = 0; m < D / 32; ++m)
            qreg[r][m] = row_ok[r] ? *(const uint4*)(qp + 32 * m + 8 * g) : make_uint4(0, 0, 0, 0);
    }
    auto pos_of = [&](int r) {
        const int qj = (kWaveRows * wave + 16 * r + n) / G;
        return row_ok[r] ? span_start + td.qtok0 + qj : -1;
    };
    // the wave's rows, in positions: first and last (wave-uniform)
    const int wrows = min(max(nrows - kWaveRows * wave, 0), kWaveRows);
    const int wfirst = span_start + td.qtok0 + (kWaveRows * wave) / G;
    const int wlast = wrows > 0 ? span_start + td.qtok0 + (kWaveRows * wave + wrows - 1) / G : -1;
    // steps ending at or before this key are visible to every row of the
    // wave and lie inside the context: no masks
    const int full_until = tree ? span_start - 1 : wfirst;

    constexpr float kLazy = 8.f;
    f32x4 o[RT][D / 16];
    float m_use[RT], thr[RT], l_run[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r) {
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) o[r][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        m_use[r] = 0.f;
        thr[r] = -INFINITY;
        l_run[r] = 0.f;
    }

    const int32_t* bt_row = a.block_tables + (int64_t)td.seq * a.max_blocks_per_seq + td.b0 + j;
    const int nsteps = (take + KB - 1) / KB;
    // physical ids of 64 blocks at a time, one per lane (clamped into the
    // pool: a wrong table gives undefined results, never an access outside)
    int cbase = 0;
    auto load_ids = [&](int c0) {
        const int cnt = min(64, take - c0);
        const int id = lane < cnt ? min(max(bt_row[c0 + lane], 0), a.num_blocks - 1) : 0;
        // used at once (no load of ids stays in flight past this point)
        return __builtin_amdgcn_readfirstlane(0) + id;
    };
    int ids = load_ids(0);

    // regs[x % PF] holds the loads of step x from their issue until the
    // LDS write; step x is issued PF steps before it computes
    typename Step::Regs regs[PF];
    auto issue_step = [&](typename Step::Regs& r, int x) {
        const int rel = x * KB;
        if (rel - cbase >= 64) {  // the next 64 blocks' ids
            cbase += 64;
            ids = load_ids(cbase);
        }
        Step::issue(r, a, kvh, ids, rel - cbase, min(KB, take - rel), tid, wave);
    };
    auto commit_step = [&](const typename Step::Regs& r, int x) {
        const int rel = x * KB;
        Step::commit(smem + (x & 1) * L::kBufBytes, r, td.b0 + j + rel, L_, min(KB, take - rel),
                     tid, wave);
    };
#pragma unroll
    for (int x = 0; x < PF; ++x) issue_step(regs[x], x);
    commit_step(regs[0], 0);
    __syncthreads();

    // steps s0 + u, u < PF: the register set of step x is regs[x % PF], a
    // compile-time index here
    for (int s0 = 0; s0 < nsteps; s0 += PF) {
#pragma unroll
    for (int u = 0; u < PF; ++u) {
        const int s = s0 + u;
        if (s >= nsteps) break;
        uint8_t* cur = smem + (s & 1) * L::kBufBytes;
        const int rel0 = s * KB;                 // first block of the step, in the part
        const int nblk = min(KB, take - rel0);   // blocks present
        const int jb0 = td.b0 + j + rel0;        // its logical block
        issue_step(regs[u], s + PF);  // past the segment: in-range loads, never used
        const int key_first = jb0 * 16, key_last = (jb0 + KB) * 16 - 1;
        if (wrows > 0 && key_first <= wlast) {
            const bool full = nblk == KB && key_last <= full_until;  // wave-uniform
            float cks[KB], vsc[KB];
#pragma unroll
            for (int kt = 0; kt < KB; ++kt) {
                cks[kt] = a.scale_log2;
                vsc[kt] = 1.f;
                if constexpr (kFp8) {
                    const float* sc = (const float*)(cur + L::kScaleOff);
                    cks[kt] *= sc[kt];
                    vsc[kt] = sc[KB + kt];
                }
            }
            // S^T = K Q^T for the step's KB key tiles and the wave's RT row tiles
            f32x4 sc[KB][RT];
#pragma unroll
            for (int kt = 0; kt < KB; ++kt)
#pragma unroll
                for (int r = 0; r < RT; ++r) sc[kt][r] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int m = 0; m < D / 32; ++m) {
#pragma unroll
                for (int kt = 0; kt < KB; ++kt) {
                    const uint4 ka = *(const uint4*)(cur + L::k_unit(kt * 16 + n, 4 * m + g));
#pragma unroll
                    for (int r = 0; r < RT; ++r)
                        sc[kt][r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8, ka), __builtin_bit_cast(bf16x8, qreg[r][m]),
                            sc[kt][r], 0, 0, 0);
                }
            }
            // scores relative to the reference; on boundary steps keys past
            // a row's position, outside the tree mask or in absent blocks are
            // selected to -inf (branch-free: one wave-uniform test per step)
            float x[RT][KB][4];
            if (full) {
#pragma unroll
                for (int r = 0; r < RT; ++r)
#pragma unroll
                    for (int kt = 0; kt < KB; ++kt)
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            x[r][kt][e] = fmaf(sc[kt][r][e], cks[kt], -m_use[r]);
            } else {
#pragma unroll
                for (int r = 0; r < RT; ++r) {
                    const int pr = pos_of(r);
#pragma unroll
                    for (int kt = 0; kt < KB; ++kt) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int t = key_first + 16 * kt + 4 * g + e, k = t - span_start;
                            const bool in_tree =
                                (k < 0) | (((uint32_t)(tbits[r] >> (k & 63)) & 1u) != 0u);
                            const bool vis = (kt < nblk) & (t <= pr) & in_tree;
                            const float xv = fmaf(sc[kt][r][e], cks[kt], -m_use[r]);
                            x[r][kt][e] = vis ? xv : -INFINITY;
                        }
                    }
                }
            }
            float mx[RT];
            bool up = false;
#pragma unroll
            for (int r = 0; r < RT; ++r) {
                mx[r] = fmaxf(fmaxf(fmaxf(x[r][0][0], x[r][0][1]), fmaxf(x[r][0][2], x[r][0][3])),
                              fmaxf(fmaxf(x[r][1][0], x[r][1][1]), fmaxf(x[r][1][2], x[r][1][3])));
#pragma unroll
                for (int kt = 2; kt < KB; ++kt)
                    mx[r] = fmaxf(mx[r], fmaxf(fmaxf(x[r][kt][0], x[r][kt][1]),
                                               fmaxf(x[r][kt][2], x[r][kt][3])));
                up |= mx[r] > thr[r];
            }
            if (__builtin_amdgcn_ballot_w64(up) != 0) {
#pragma unroll
                for (int r = 0; r < RT; ++r) {
                    if (__builtin_amdgcn_ballot_w64(mx[r] > thr[r]) == 0) continue;
                    const float rm = row_max(mx[r]);
                    const bool had = thr[r] != -INFINITY;
                    const float delta = had ? fmaxf(rm, 0.f) : (rm == -INFINITY ? 0.f : rm);
                    const float alpha = had ? fexp2(-delta) : 1.f;
#pragma unroll
                    for (int kt = 0; kt < KB; ++kt)
#pragma unroll
                        for (int e = 0; e < 4; ++e) x[r][kt][e] -= delta;
                    m_use[r] += delta;
                    if (rm != -INFINITY) thr[r] = kLazy;
                    l_run[r] *= alpha;
#pragma unroll
                    for (int dt = 0; dt < D / 16; ++dt) o[r][dt] *= alpha;
                }
            }
            // weights, P operands (8 bf16: keys 4g+e of the pair's two
            // blocks) and O^T += V^T P^T per block pair
#pragma unroll
            for (int pr = 0; pr < KB / 2; ++pr) {
                uint4 pk[RT];
#pragma unroll
                for (int r = 0; r < RT; ++r) {
                    float p0[4], p1[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        p0[e] = fexp2(x[r][2 * pr][e]);
                        p1[e] = fexp2(x[r][2 * pr + 1][e]);
                    }
                    l_run[r] += ((p0[0] + p0[1]) + (p0[2] + p0[3])) +
                                ((p1[0] + p1[1]) + (p1[2] + p1[3]));
                    const float v0 = vsc[2 * pr], v1 = vsc[2 * pr + 1];
                    pk[r] = make_uint4(pack_bf16x2(p0[0] * v0, p0[1] * v0),
                                       pack_bf16x2(p0[2] * v0, p0[3] * v0),
                                       pack_bf16x2(p1[0] * v1, p1[1] * v1),
                                       pack_bf16x2(p1[2] * v1, p1[3] * v1));
                }
#pragma unroll
                for (int dt = 0; dt < D / 16; ++dt) {
                    const uint4 va = *(const uint4*)(cur + L::v_unit(pr, 16 * dt + n, g));
#pragma unroll
                    for (int r = 0; r < RT; ++r)
                        o[r][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8, va), __builtin_bit_cast(bf16x8, pk[r]),
                            o[r][dt], 0, 0, 0);
                }
            }
        }
        if (s + 1 < nsteps) commit_step(regs[(u + 1) % PF], s + 1);
        __syncthreads();
    }
    }

    // epilogue (per wave, no LDS)
    const bool whole = j == 0 && take == td.nb;
    const int64_t slot = (int64_t)piece * 2 + (j > 0 ? SLOT_HEAD : SLOT_TAIL);
#pragma unroll
    for (int r = 0; r < RT; ++r) {
        const float l = row_sum(l_run[r]);
        const float inv = l > 0.f ? 1.0f / l : 0.f;
        if (!row_ok[r]) continue;
        if (whole) {
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt) {
                uint2 w;
                w.x = pack_bf16x2(o[r][dt][0] * inv, o[r][dt][1] * inv);
                w.y = pack_bf16x2(o[r][dt][2] * inv, o[r][dt][3] * inv);
                *(uint2*)((uint16_t*)a.out + (int64_t)rowid[r] * D + 16 * dt + 4 * g) = w;
            }
            if (a.lse && g == 0)
                a.lse[rowid[r]] = l > 0.f ? (m_use[r] + __log2f(l)) * kLn2 : -INFINITY;
        } else {
            const int rt = RT * wave + r;  // row tile within the slot
            float4* po = (float4*)a.part_o + ((slot * kSpanRowTiles + rt) * (D / 16)) * 64 + lane;
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt)
                po[dt * 64] = make_float4(o[r][dt][0] * inv, o[r][dt][1] * inv,
                                          o[r][dt][2] * inv, o[r][dt][3] * inv);
            if (g == 0)
                a.part_lse[slot * kSpanRows + 16 * rt + n] =
                    l > 0.f ? m_use[r] + __log2f(l) : -INFINITY;
        }
    }
}

// Persistent grid: workgroup w takes pieces w, w + grid, ... of the wide
// stream. Two workgroups per compute unit.
template <int kv, int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kSpanWaves / 2,
                                                                          kSpanWaves / 2))) void
attention_span(AttnArgs a) {
    __shared__ __align__(16) uint8_t smem[2 * SpanLds<D>::kBufBytes];
    const int* h = a.hdr + HDR_STREAM + 4 * a.stream;
    const int V = h[HDR_NPIECES];
    for (int v = blockIdx.x; v < V; v += gridDim.x) {
        const PieceStart ps = a.pieces[v];
        int t = ps.tile, j = ps.j;
        const int kvh = ps.kvh;
        TileDesc td = ps.td;
        int left = ps.nblocks;
        while (left > 0) {
            const int take = min(left, td.nb - j);
            span_segment<kv, D>(a, smem, td, kvh, j, take, v);
            left -= take;
            j = 0;
            ++t;
            if (left > 0) td = a.tiles[t];
        }
    }
}

constexpr int kMaxDevices = 64;

// Resident workgroups per (kernel instance, device), queried once per
// device and kept for the process (threads that race on a first query
// compute the same number; the first stored is the one every call sees).
template <int kv, int D>
int span_resident_d() {
    static std::atomic<int> cached[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
    std::atomic<int>* slot = dev < kMaxDevices ? &cached[dev] : nullptr;
    if (slot) {
        const int c = slot->load(std::memory_order_acquire);
        if (c > 0) return c;
    }
    int num_cu = 0, occ = 0;
    if (hipDeviceGetAttribute(&num_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, attention_span<kv, D>, kThreads, 0) !=
            hipSuccess)
        return 0;
    const int w = (occ > 0 ? occ : 1) * num_cu;
    if (!slot) return w;
    int expected = 0;
    slot->compare_exchange_strong(expected, w, std::memory_order_acq_rel);
    return slot->load(std::memory_order_acquire);
}

// Span workgroups that leave a narrow wave room on every SIMD: one per
// compute unit when the span kernel's resources allow two (its four waves
// then hold one wave slot of each SIMD), else 0.
template <int kv, int D>
int span_shared_d() {
    const int w = span_resident_d<kv, D>();
    int dev = 0, num_cu = 0;
    if (w <= 0 || hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&num_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        num_cu <= 0)
        return 0;
    return w >= 2 * num_cu ? num_cu : 0;
}

template <int kv, int D>
hipError_t launch_span_d(const AttnArgs& a, int64_t max_pieces, hipStream_t s) {
    int64_t grid = span_resident_d<kv, D>();
    if (grid <= 0) return hipErrorInvalidDevice;
    if (max_pieces < grid) grid = max_pieces;
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL((attention_span<kv, D>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace

// fp8 caches with fp8_qk take the same span kernel: the span's products run
// on the bf16 matrix cores after the exact e4m3 -> bf16 conversion.
int span_resident_groups(int kind, int head_dim) {
    switch ((kind == KIND_FP8_QK ? PA_FP8_E4M3FN : kind) * 1000 + head_dim) {
    case PA_BF16 * 1000 + 64: return span_resident_d<KV_BF16, 64>();
    case PA_BF16 * 1000 + 128: return span_resident_d<KV_BF16, 128>();
    case PA_FP8_E4M3FN * 1000 + 64: return span_resident_d<KV_FP8, 64>();
    case PA_FP8_E4M3FN * 1000 + 128: return span_resident_d<KV_FP8, 128>();
    default: return 0;
    }
}

int span_shared_groups(int kind, int head_dim) {
    switch ((kind == KIND_FP8_QK ? PA_FP8_E4M3FN : kind) * 1000 + head_dim) {
    case PA_BF16 * 1000 + 64: return span_shared_d<KV_BF16, 64>();
    case PA_BF16 * 1000 + 128: return span_shared_d<KV_BF16, 128>();
    case PA_FP8_E4M3FN * 1000 + 64: return span_shared_d<KV_FP8, 64>();
    case PA_FP8_E4M3FN * 1000 + 128: return span_shared_d<KV_FP8, 128>();
    default: return 0;
    }
}

hipError_t launch_span(int kind, int head_dim, const AttnArgs& a, int64_t max_pieces,
                       hipStream_t s) {
    switch ((kind == KIND_FP8_QK ? PA_FP8_E4M3FN : kind) * 1000 + head_dim) {
    case PA_BF16 * 1000 + 64: return launch_span_d<KV_BF16, 64>(a, max_pieces, s);
    case PA_BF16 * 1000 + 128: return launch_span_d<KV_BF16, 128>(a, max_pieces, s);
    case PA_FP8_E4M3FN * 1000 + 64: return launch_span_d<KV_FP8, 64>(a, max_pieces, s);
    case PA_FP8_E4M3FN * 1000 + 128: return launch_span_d<KV_FP8, 128>(a, max_pieces, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace pa
