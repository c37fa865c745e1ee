/*
 * oracle.c -- CPU float64 reference for paged attention.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may call this: only
 * the tests, the smoke check and the CPU-baseline leg of the benchmark load
 * it. It shares no code, header or table with the HIP library.
 *
 * What it computes is the plain definition of attention over a paged KV
 * cache, written out directly ("gather, then softmax"):
 *
 *   - KV storage in fixed 16-token physical blocks reached through a
 *     per-sequence block table ("03 -- Engines Papers", section 2, key trick;
 *     "The LLM inference engine playbook", Theme 3). Attention must gather
 *     K/V rows from those non-contiguous blocks (section 2, "What to
 *     extract", the PagedAttention kernel bullet).
 *   - Attention is per sequence (section 1, selective batching), over that
 *     sequence's own context length.
 *   - GQA: several query heads share one KV head ("References", GQA entry);
 *     query head h reads KV head h / G, G = Hq / Hkv.
 *   - A chunked-prefill span attends causally to the K/V already present:
 *     its tokens are the last n positions of the context, and a query at
 *     position p sees keys 0..p ("03 -- Engines Papers", section 3).
 *   - The online softmax normalizer (Milakov & Gimelshein, "References")
 *     reaches exactly this softmax; the oracle does not use it: it takes
 *     the max, the exponentials and their sum in separate passes.
 *   - Tree verification of speculative candidates ("03 -- Engines Papers",
 *     sections 5 to 7: the draft tokens of a span are nodes of a candidate
 *     tree verified in one pass under a tree attention mask): with a tree
 *     mask, span token j of a span of at most 64 tokens sees every key
 *     before the span and span token k <= j only where bit k of its mask
 *     word is set. Spans of more than 64 tokens stay causal.
 *   - FP8 E4M3 KV with a scale ("The LLM inference engine playbook",
 *     Themes 3 and 6): a stored byte means e4m3fn(byte) * scale, with one
 *     fp32 scale per (block, KV head).
 *
 * Layouts (the library's contract):
 *   q, out      [T][Hq][D]
 *   K cache     [NB][Hkv][16][D]   V cache [NB][Hkv][D][16]
 *   k/v scale   [NB][Hkv] float32 (fp8 only)
 *   block table [S][max_blocks] int32; context_lens [S];
 *   query_start_loc [S+1] (NULL: one query token per sequence, T = S)
 */
#include <fenv.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_BLOCK 16

enum { OR_F32 = 0, OR_BF16 = 1, OR_FP8 = 2 };

/* ---- element decoding ------------------------------------------------- */

/* bf16 is the top half of an IEEE binary32; widening is exact. */
static double or_bf16_bits_to_double(uint16_t bits) {
    uint32_t w = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &w, 4);
    return (double)f;
}

/* OCP FP8 E4M3FN ("the FP8 formats paper" of the playbook's Theme 6):
 * 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits. Exponent field 0
 * holds subnormals (m/8)*2^-6; exponent 15 with mantissa 7 is NaN; there is
 * no infinity. */
double or_fp8_e4m3fn_decode(uint8_t code) {
    int s = code >> 7, e = (code >> 3) & 0xF, m = code & 7;
    double mag;
    if (e == 15 && m == 7) return NAN;
    if (e == 0)
        mag = ldexp((double)m / 8.0, -6);
    else
        mag = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -mag : mag;
}

/* Encode a float to E4M3FN: round to nearest, ties to even, saturate to
 * +-448 (the largest finite value), NaN to 0x7F. The grid spacing is
 * 2^(E-3) for a value in [2^E, 2^(E+1)), E >= -6, and 2^-9 below 2^-6. */
uint8_t or_fp8_e4m3fn_encode(float x) {
    if (isnan(x)) return 0x7F;
    int neg = signbit(x) ? 1 : 0;
    double a = fabs((double)x);
    uint8_t code;
    if (a >= 448.0) {
        code = 0x7E;
    } else if (a == 0.0) {
        code = 0;
    } else {
        int k;
        frexp(a, &k); /* a = f * 2^k, f in [0.5, 1) -> a in [2^(k-1), 2^k) */
        int E = k - 1;
        if (E < -6) E = -6;
        double quantum = ldexp(1.0, E - 3);
        double r = nearbyint(a / quantum); /* exact division; RNE rounding */
        double val = r * quantum;
        if (val < ldexp(1.0, -6)) {
            code = (uint8_t)r; /* subnormal: mantissa = r (r == 8 is 2^-6) */
        } else {
            int k2;
            double f2 = frexp(val, &k2);
            int E2 = k2 - 1;
            int m = (int)((f2 * 2.0 - 1.0) * 8.0);
            code = (uint8_t)(((E2 + 7) << 3) | m);
        }
    }
    return (uint8_t)(code | (neg << 7));
}

void or_fp8_decode_array(const uint8_t* codes, double* out, long n) {
    for (long i = 0; i < n; ++i) out[i] = or_fp8_e4m3fn_decode(codes[i]);
}

void or_fp8_encode_array(const float* x, uint8_t* out, long n) {
    for (long i = 0; i < n; ++i) out[i] = or_fp8_e4m3fn_encode(x[i]);
}

/* Quantize whole block-heads: every group of `elems` source values shares
 * one scale; byte = e4m3fn(fp32(src) / scale) with IEEE fp32 division. */
void or_fp8_encode_blocks(const float* src, const float* scales, long groups, long elems,
                          uint8_t* dst) {
    long g;
#pragma omp parallel for schedule(static)
    for (g = 0; g < groups; ++g) {
        float s = scales[g];
        for (long e = 0; e < elems; ++e) {
            float y = src[g * elems + e] / s;
            dst[g * elems + e] = or_fp8_e4m3fn_encode(y);
        }
    }
}

/* ---- KV append ---------------------------------------------------------- */

/* Write new K/V rows into their physical slots: slot s lives in block
 * s / 16 at offset s % 16 (the block table's logical-to-physical mapping,
 * "03 -- Engines Papers" section 2). A negative slot is skipped. Same-dtype
 * caches receive the bits unchanged; fp8 caches receive
 * e4m3fn(fp32(new) / scale[block][head]). */
int or_kv_append(int num_kv_heads, int head_dim, int kv_dtype, int new_dtype, void* k_cache,
                 void* v_cache, const float* k_scale, const float* v_scale, const void* k_new,
                 const void* v_new, const int32_t* slot_mapping, int num_tokens) {
    const int H = num_kv_heads, D = head_dim;
    for (int t = 0; t < num_tokens; ++t) {
        int s = slot_mapping[t];
        if (s < 0) continue;
        long b = s / OR_BLOCK, o = s % OR_BLOCK;
        for (int g = 0; g < H; ++g) {
            for (int d = 0; d < D; ++d) {
                long src = ((long)t * H + g) * D + d;
                long kdst = ((b * H + g) * OR_BLOCK + o) * D + d;
                long vdst = ((b * H + g) * D + d) * OR_BLOCK + o;
                if (kv_dtype == new_dtype && kv_dtype == OR_F32) {
                    ((float*)k_cache)[kdst] = ((const float*)k_new)[src];
                    ((float*)v_cache)[vdst] = ((const float*)v_new)[src];
                } else if (kv_dtype == new_dtype && kv_dtype == OR_BF16) {
                    ((uint16_t*)k_cache)[kdst] = ((const uint16_t*)k_new)[src];
                    ((uint16_t*)v_cache)[vdst] = ((const uint16_t*)v_new)[src];
                } else if (kv_dtype == OR_FP8) {
                    float kx, vx;
                    if (new_dtype == OR_F32) {
                        kx = ((const float*)k_new)[src];
                        vx = ((const float*)v_new)[src];
                    } else if (new_dtype == OR_BF16) {
                        kx = (float)or_bf16_bits_to_double(((const uint16_t*)k_new)[src]);
                        vx = (float)or_bf16_bits_to_double(((const uint16_t*)v_new)[src]);
                    } else {
                        return -1;
                    }
                    float ks = k_scale[b * H + g], vs = v_scale[b * H + g];
                    ((uint8_t*)k_cache)[kdst] = or_fp8_e4m3fn_encode(kx / ks);
                    ((uint8_t*)v_cache)[vdst] = or_fp8_e4m3fn_encode(vx / vs);
                } else {
                    return -1;
                }
            }
        }
    }
    return 0;
}

/* ---- attention ----------------------------------------------------------- */

typedef struct {
    int num_seqs, num_q_heads, num_kv_heads, head_dim;
    const void* q;
    int q_dtype;
    const void* k_cache;
    const void* v_cache;
    int kv_dtype;
    const float* k_scale;
    const float* v_scale;
    const int32_t* block_tables;
    int max_blocks_per_seq;
    const int32_t* context_lens;
    const int32_t* query_start_loc;
    float scale;
    const uint64_t* tree_mask; /* [T] or NULL: causal spans */
} or_args;

static double or_q_at(const or_args* a, long idx) {
    if (a->q_dtype == OR_F32) return (double)((const float*)a->q)[idx];
    return or_bf16_bits_to_double(((const uint16_t*)a->q)[idx]);
}

/* One stored cache element, dequantized to float64. */
static double or_kv_at(const or_args* a, const void* cache, const float* scales, long idx,
                       long scale_idx) {
    switch (a->kv_dtype) {
    case OR_F32: return (double)((const float*)cache)[idx];
    case OR_BF16: return or_bf16_bits_to_double(((const uint16_t*)cache)[idx]);
    default:
        return or_fp8_e4m3fn_decode(((const uint8_t*)cache)[idx]) * (double)scales[scale_idx];
    }
}

/* Gather the first L keys and values of sequence i, KV head g, into
 * contiguous [L][D] float64 arrays, following the block table. */
static void or_gather(const or_args* a, int i, int g, int L, double* K, double* V) {
    const int H = a->num_kv_heads, D = a->head_dim;
    for (int t = 0; t < L; ++t) {
        long b = a->block_tables[(long)i * a->max_blocks_per_seq + t / OR_BLOCK];
        long o = t % OR_BLOCK;
        long sidx = b * H + g;
        for (int d = 0; d < D; ++d) {
            K[(long)t * D + d] = or_kv_at(a, a->k_cache, a->k_scale, ((sidx)*OR_BLOCK + o) * D + d, sidx);
            V[(long)t * D + d] = or_kv_at(a, a->v_cache, a->v_scale, ((sidx)*D + d) * OR_BLOCK + o, sidx);
        }
    }
}

/* Softmax attention of one query row over the keys 0..nk-1 of gathered
 * K/V for which vis[t] is nonzero (vis NULL: all of them). */
static void or_attend_row(const or_args* a, long qrow, int h, const double* K, const double* V,
                          int nk, const unsigned char* vis, double* s, double* out,
                          double* lse) {
    const int D = a->head_dim;
    const double scale = (double)a->scale;
    int any = 0;
    for (int t = 0; t < nk; ++t) any |= vis ? vis[t] : 1;
    if (!any) {
        for (int d = 0; d < D; ++d) out[d] = 0.0;
        *lse = -INFINITY;
        return;
    }
    double M = -INFINITY;
    for (int t = 0; t < nk; ++t) {
        if (vis && !vis[t]) continue;
        double acc = 0.0;
        for (int d = 0; d < D; ++d)
            acc += or_q_at(a, (qrow * a->num_q_heads + h) * D + d) * K[(long)t * D + d];
        s[t] = scale * acc;
        if (s[t] > M) M = s[t];
    }
    double Z = 0.0;
    for (int t = 0; t < nk; ++t) {
        s[t] = (vis && !vis[t]) ? 0.0 : exp(s[t] - M);
        Z += s[t];
    }
    for (int d = 0; d < D; ++d) {
        double acc = 0.0;
        for (int t = 0; t < nk; ++t) acc += s[t] * V[(long)t * D + d];
        out[d] = acc / Z;
    }
    *lse = M + log(Z);
}

/* Attention of one KV-head group of one sequence, all its query tokens. */
static void or_seq_group(const or_args* a, int i, int g, double* out, double* lse) {
    const int G = a->num_q_heads / a->num_kv_heads, D = a->head_dim, Hq = a->num_q_heads;
    const int L = a->context_lens[i];
    long q0, n;
    if (a->query_start_loc) {
        q0 = a->query_start_loc[i];
        n = a->query_start_loc[i + 1] - q0;
    } else {
        q0 = i;
        n = 1;
    }
    double* K = (double*)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1) * D);
    double* V = (double*)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1) * D);
    double* s = (double*)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
    unsigned char* vis = (unsigned char*)malloc((size_t)(L > 0 ? L : 1));
    if (L > 0) or_gather(a, i, g, L, K, V);
    const int tree = a->tree_mask != NULL && n <= 64;
    for (long j = 0; j < n; ++j) {
        long pos = (long)L - n + j; /* the span is the last n positions */
        int nk = (int)(pos + 1);    /* causal: keys 0..pos inclusive */
        if (nk > L) nk = L;
        if (tree) { /* keys before the span, and the marked span tokens k <= j */
            const uint64_t bits = a->tree_mask[q0 + j];
            for (int t = 0; t < nk; ++t) {
                const long k = t - ((long)L - n);
                vis[t] = k < 0 || ((bits >> k) & 1u);
            }
        }
        for (int hh = 0; hh < G; ++hh) {
            int h = g * G + hh;
            long r = q0 + j;
            or_attend_row(a, r, h, K, V, nk, tree ? vis : NULL, s, out + (r * Hq + h) * D,
                          lse + r * Hq + h);
        }
    }
    free(K);
    free(V);
    free(s);
    free(vis);
}

/* Compute out [T][Hq][D] and lse [T][Hq] (natural log) in float64.
 * seq_subset (optional, n_subset entries) restricts the work to those
 * sequences; rows of other sequences are left untouched. */
int or_paged_attention(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                       const void* q, int q_dtype, const void* k_cache, const void* v_cache,
                       int kv_dtype, const float* k_scale, const float* v_scale,
                       const int32_t* block_tables, int max_blocks_per_seq,
                       const int32_t* context_lens, const int32_t* query_start_loc, float scale,
                       const uint64_t* tree_mask, const int32_t* seq_subset, int n_subset,
                       double* out, double* lse, int num_threads) {
    if (num_kv_heads <= 0 || num_q_heads % num_kv_heads) return -1;
    if (fegetround() != FE_TONEAREST) return -2;
    or_args a = {num_seqs, num_q_heads, num_kv_heads, head_dim, q, q_dtype, k_cache, v_cache,
                 kv_dtype, k_scale, v_scale, block_tables, max_blocks_per_seq, context_lens,
                 query_start_loc, scale, tree_mask};
    const int H = num_kv_heads;
    const long nseq = seq_subset ? n_subset : num_seqs;
    const long ntask = nseq * H;
    long task;
#ifdef _OPENMP
    if (num_threads > 0) omp_set_num_threads(num_threads);
#endif
#pragma omp parallel for schedule(dynamic, 1)
    for (task = 0; task < ntask; ++task) {
        long si = task / H;
        int i = seq_subset ? seq_subset[si] : (int)si;
        int g = (int)(task % H);
        or_seq_group(&a, i, g, out, lse);
    }
    return 0;
}

/* Partial result over keys [t0, t1) of one row: m = max score,
 * l = sum exp(s - m), o = sum exp(s - m) v / l. */
static void or_partial(const or_args* a, long qrow, int h, const double* K, const double* V,
                       int t0, int t1, double* s, double* m, double* l, double* o) {
    const int D = a->head_dim;
    const double scale = (double)a->scale;
    double M = -INFINITY;
    for (int t = t0; t < t1; ++t) {
        double acc = 0.0;
        for (int d = 0; d < D; ++d)
            acc += or_q_at(a, (qrow * a->num_q_heads + h) * D + d) * K[(long)t * D + d];
        s[t - t0] = scale * acc;
        if (s[t - t0] > M) M = s[t - t0];
    }
    double Z = 0.0;
    for (int t = t0; t < t1; ++t) Z += exp(s[t - t0] - M);
    for (int d = 0; d < D; ++d) {
        double acc = 0.0;
        for (int t = t0; t < t1; ++t) acc += exp(s[t - t0] - M) * V[(long)t * D + d];
        o[d] = acc / Z;
    }
    *m = M;
    *l = Z;
}

/* Test-only: the same rows computed as partial results (m_p, l_p, o_p)
 * over key ranges and merged by log-sum-exp ("03 -- Engines Papers",
 * section 12; "The LLM inference engine playbook", Theme 4, split-K
 * decode):
 *   M = max_p m_p,  w_p = l_p exp(m_p - M),
 *   out = sum_p w_p o_p / sum_p w_p,  lse = M + ln sum_p w_p.
 * The ranges of sequence i are [0, f_i), [f_i, f_i + P), ... with f_i =
 * first_len[i] (first_len NULL: f_i = P), so the cuts can sit anywhere in
 * a context, as where a stream of blocks cut into equal pieces meets a
 * sequence's blocks at an arbitrary offset. Used only to pin that
 * splitting reaches the unsplit result. */
int or_paged_attention_split(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                             const void* q, int q_dtype, const void* k_cache,
                             const void* v_cache, int kv_dtype, const float* k_scale,
                             const float* v_scale, const int32_t* block_tables,
                             int max_blocks_per_seq, const int32_t* context_lens,
                             const int32_t* query_start_loc, float scale, int partition_size,
                             const int32_t* first_len, double* out, double* lse) {
    if (partition_size <= 0 || num_q_heads % num_kv_heads) return -1;
    if (first_len)
        for (int i = 0; i < num_seqs; ++i)
            if (first_len[i] <= 0 || first_len[i] > partition_size) return -1;
    or_args a = {num_seqs, num_q_heads, num_kv_heads, head_dim, q, q_dtype, k_cache, v_cache,
                 kv_dtype, k_scale, v_scale, block_tables, max_blocks_per_seq, context_lens,
                 query_start_loc, scale};
    const int H = num_kv_heads, G = num_q_heads / num_kv_heads, D = head_dim, Hq = num_q_heads;
    int maxL = 1;
    for (int i = 0; i < num_seqs; ++i)
        if (context_lens[i] > maxL) maxL = context_lens[i];
    const int maxP = (maxL + partition_size - 1) / partition_size + 1;
    double* K = (double*)malloc(sizeof(double) * (size_t)maxL * D);
    double* V = (double*)malloc(sizeof(double) * (size_t)maxL * D);
    double* s = (double*)malloc(sizeof(double) * (size_t)partition_size);
    double* mp = (double*)malloc(sizeof(double) * (size_t)maxP);
    double* lp = (double*)malloc(sizeof(double) * (size_t)maxP);
    double* op = (double*)malloc(sizeof(double) * (size_t)maxP * D);
    for (int i = 0; i < num_seqs; ++i) {
        const int L = context_lens[i];
        long q0 = query_start_loc ? query_start_loc[i] : i;
        long n = query_start_loc ? query_start_loc[i + 1] - q0 : 1;
        for (int g = 0; g < H; ++g) {
            if (L > 0) or_gather(&a, i, g, L, K, V);
            for (long j = 0; j < n; ++j) {
                long pos = (long)L - n + j;
                int nk = (int)(pos + 1);
                if (nk > L) nk = L;
                const int f = first_len ? first_len[i] : partition_size;
                const int np = nk <= 0 ? 0
                               : nk <= f ? 1
                                         : 1 + (nk - f + partition_size - 1) / partition_size;
                for (int hh = 0; hh < G; ++hh) {
                    const int h = g * G + hh;
                    const long r = q0 + j;
                    double* o = out + (r * Hq + h) * D;
                    for (int p = 0; p < np; ++p) {
                        int t0 = p == 0 ? 0 : f + (p - 1) * partition_size;
                        int t1 = p == 0 ? f : t0 + partition_size;
                        if (t1 > nk) t1 = nk;
                        or_partial(&a, r, h, K, V, t0, t1, s, &mp[p], &lp[p], op + (long)p * D);
                    }
                    if (np == 0) {
                        for (int d = 0; d < D; ++d) o[d] = 0.0;
                        lse[r * Hq + h] = -INFINITY;
                        continue;
                    }
                    double M = -INFINITY;
                    for (int p = 0; p < np; ++p)
                        if (mp[p] > M) M = mp[p];
                    double W = 0.0;
                    for (int d = 0; d < D; ++d) o[d] = 0.0;
                    for (int p = 0; p < np; ++p) {
                        double w = lp[p] * exp(mp[p] - M);
                        W += w;
                        for (int d = 0; d < D; ++d) o[d] += w * op[(long)p * D + d];
                    }
                    for (int d = 0; d < D; ++d) o[d] /= W;
                    lse[r * Hq + h] = M + log(W);
                }
            }
        }
    }
    free(K);
    free(V);
    free(s);
    free(mp);
    free(lp);
    free(op);
    return 0;
}
