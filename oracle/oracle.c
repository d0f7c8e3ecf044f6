/*
 * Plain fp64 CPU oracle for single-token decode attention over a KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no source with the HIP library: it has its
 * own dtype codes, its own number conversions and its own FP8 codec.
 *
 * Pages cited (by address; section names as printed on each page):
 *   [mlqm]  www.mlqm.cn/news/394450          (KV Cache explainer, sections 一..十)
 *   [cf1]   www.cf-1.com/news/5824798        (KV Cache memory + PagedAttention, §1..§5)
 *   [lqnn]  m.lqnn.cn/news/219451            (capacity planning to strategy, §1..§13)
 *   [xph]   inference.xph.ink kp-013          ("KV Cache：原理与显存占比")
 *   [moo]   www.mooersco.com/news/1484987    (practitioner guide, §1..§5)
 *
 * Everything here is deliberately slow and literal: values are widened to
 * double exactly, the softmax is two-pass (max, then exponentials), sums run
 * in ascending token order.  The only parallelism is one OpenMP task per
 * (sequence, kv-head), which does not change any arithmetic.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Storage type codes of this oracle (numerically equal to the library's by
 * convention, so the harness can pass one integer; defined independently). */
enum { OR_F32 = 0, OR_F16 = 1, OR_BF16 = 2, OR_E4M3 = 3, OR_F64 = 5 };   /* OR_F64: values already
                                                                           dequantised by the caller */

/* ------------------------------------------------------------------------
 * KV size formula.  [cf1] §1.2: per token, 2 (K and V) x layers x KV heads x
 * head dim x element bytes.  [lqnn] §1 and [xph] "公式与模型" multiply by the
 * cached tokens and the batch.  Invalid structure (any of layers, kv_heads,
 * head_dim, elem_bytes <= 0) or negative tokens/seqs gives 0, mirroring the
 * ValueError of the budget script in [lqnn] §2.
 * ------------------------------------------------------------------------ */
uint64_t oracle_kv_cache_bytes(int64_t layers, int64_t kv_heads, int64_t head_dim,
                               int64_t elem_bytes, int64_t tokens, int64_t seqs) {
    if (layers <= 0 || kv_heads <= 0 || head_dim <= 0 || elem_bytes <= 0) return 0;
    if (tokens < 0 || seqs < 0) return 0;
    return (uint64_t)2 * (uint64_t)layers * (uint64_t)kv_heads * (uint64_t)head_dim *
           (uint64_t)elem_bytes * (uint64_t)tokens * (uint64_t)seqs;
}

/* ------------------------------------------------------------------------
 * Exact widening of stored values to double.
 * ------------------------------------------------------------------------ */

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double oracle_f16_to_f64(uint16_t h) {
    int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 31) v = m ? NAN : INFINITY;
    else if (e == 0) v = ldexp((double)m, -24);           /* subnormal: m * 2^-24 */
    else v = ldexp((double)(1024 + m), e - 25);           /* (1 + m/1024) * 2^(e-15) */
    return s ? -v : v;
}

/* bfloat16 is the upper half of an IEEE binary32. */
double oracle_bf16_to_f64(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* OCP 8-bit floating point, E4M3 ("FN") encoding, the specification the
 * [lqnn] reference list names: 1 sign bit, 4 exponent bits with bias 7,
 * 3 mantissa bits; exponent field 0 is subnormal (m/8 * 2^-6); the pattern
 * S.1111.111 is NaN; there are no infinities; the largest finite is
 * 1.75 * 2^8 = 448.  [moo] §3.3 names the format (4-bit exponent, 3-bit
 * mantissa). */
double oracle_e4m3_to_f64(uint8_t c) {
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7) v = NAN;
    else if (e == 0) v = ldexp((double)m, -9);            /* m/8 * 2^-6 */
    else v = ldexp((double)(8 + m), e - 10);              /* (1 + m/8) * 2^(e-7) */
    return s ? -v : v;
}

/* Encode a float to E4M3: round to the nearest representable magnitude,
 * ties to the even code, and saturate anything beyond the largest finite
 * value (448) to 448, as the "saturate outliers" reading of [lqnn] §4 and the
 * OCP saturating conversion require.  NaN becomes 0x7F.  Written as a search
 * over the 127 non-negative finite codes, which are increasing in value. */
uint8_t oracle_e4m3_from_f32(float x) {
    if (isnan(x)) return 0x7F;
    uint8_t sign = signbit(x) ? 0x80 : 0x00;
    double a = fabs((double)x);
    if (a >= 448.0) return (uint8_t)(sign | 0x7E);
    /* No table and no static state: the search decodes the codes it visits, so
     * the function is safe to call from any number of threads at once. */
    int lo = 0, hi = 126;    /* invariant: value(lo) <= a < value(hi) */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (oracle_e4m3_to_f64((uint8_t)mid) <= a) lo = mid; else hi = mid;
    }
    double dlo = a - oracle_e4m3_to_f64((uint8_t)lo);      /* both exact in double */
    double dhi = oracle_e4m3_to_f64((uint8_t)hi) - a;
    int c;
    if (dlo < dhi) c = lo;
    else if (dhi < dlo) c = hi;
    else c = (lo % 2 == 0) ? lo : hi;                      /* tie: even mantissa */
    return (uint8_t)(sign | c);
}

/* Array forms, so the harness does not loop in Python. */
void oracle_e4m3_encode_f32_array(const float* x, int64_t n, uint8_t* out, int32_t nthreads) {
#ifdef _OPENMP
#pragma omp parallel for schedule(static) num_threads(nthreads > 0 ? nthreads : omp_get_max_threads())
#endif
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_from_f32(x[i]);
    (void)nthreads;
}

void oracle_widen_array(const void* src, int32_t dtype, int64_t n, double* out) {
    for (int64_t i = 0; i < n; ++i) {
        switch (dtype) {
            case OR_F32: out[i] = (double)((const float*)src)[i]; break;
            case OR_F16: out[i] = oracle_f16_to_f64(((const uint16_t*)src)[i]); break;
            case OR_BF16: out[i] = oracle_bf16_to_f64(((const uint16_t*)src)[i]); break;
            case OR_E4M3: out[i] = oracle_e4m3_to_f64(((const uint8_t*)src)[i]); break;
            case OR_F64: out[i] = ((const double*)src)[i]; break;
            default: out[i] = NAN;
        }
    }
}

static double widen(const void* base, int32_t dtype, int64_t i) {
    switch (dtype) {
        case OR_F32: return (double)((const float*)base)[i];
        case OR_F16: return oracle_f16_to_f64(((const uint16_t*)base)[i]);
        case OR_BF16: return oracle_bf16_to_f64(((const uint16_t*)base)[i]);
        case OR_E4M3: return oracle_e4m3_to_f64(((const uint8_t*)base)[i]);
        case OR_F64: return ((const double*)base)[i];
        default: return NAN;
    }
}

/* ------------------------------------------------------------------------
 * Decode attention over de-paged (logical order) K/V.
 *
 * For sequence b the cached keys and values are K_b[j][g][i], V_b[j][g][i],
 * j = 0..n_b-1 oldest first; the newest token (appended before attending, as
 * in [cf1] §1.1 and the forward_new_token walk-through of [mlqm] 四) is the
 * last one.  Query head h reads kv head g = floor(h / G), G = H_q / H_kv
 * (several query heads share one KV head, [mlqm] 六 GQA/MQA).
 *
 *   z_j  = scale * sum_i q[b][h][i] * K_b[j][g][i]
 *   w_j  = exp(z_j - max_k z_k) / sum_k exp(z_k - max_k z_k)
 *   out  = sum_j w_j * V_b[j][g][:]            (n_b <= 0 gives out = 0)
 *
 * This is softmax(Q K^T / sqrt(d)) V from [mlqm] 二 for one query row, with the
 * max subtracted before exp as in [mlqm] 四; the caller supplies scale.
 *
 * Layout: K and V hold all sequences back to back, [total_tokens][H_kv][D];
 * sequence b starts at token tok_off[b].  q is [B][H_q][D] in q_dtype, out is
 * [B][H_q][D] double.  For OR_E4M3 storage the stored value is
 * decode(code) * k_scale[g] (resp. v_scale[g]), per KV head, separately for
 * K and V ([lqnn] §4 per-attention-head scales); the product is exact in
 * double.  Returns 0, or -1 on bad arguments.
 * ------------------------------------------------------------------------ */
int oracle_decode_attention(int32_t B, int32_t H_q, int32_t H_kv, int32_t D,
                            const void* q, int32_t q_dtype,
                            const void* K, const void* V, int32_t kv_dtype,
                            const int64_t* tok_off, const int32_t* lens,
                            const float* k_scale, const float* v_scale,
                            float scale, int32_t nthreads, double* out) {
    if (B < 0 || H_q <= 0 || H_kv <= 0 || D <= 0 || H_q % H_kv != 0) return -1;
    if (kv_dtype == OR_E4M3 && (!k_scale || !v_scale)) return -1;
    const int32_t G = H_q / H_kv;
    const double s = (double)scale;
    int bad = 0;
#ifdef _OPENMP
#pragma omp parallel for collapse(2) schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : omp_get_max_threads()) reduction(|| : bad)
#endif
    for (int32_t b = 0; b < B; ++b) {
        for (int32_t g = 0; g < H_kv; ++g) {
            const int32_t n = lens[b];
            for (int32_t hh = 0; hh < G; ++hh) {
                const int32_t h = g * G + hh;
                double* o = out + ((int64_t)b * H_q + h) * D;
                for (int32_t i = 0; i < D; ++i) o[i] = 0.0;
            }
            if (n <= 0) continue;
            double* z = (double*)malloc(sizeof(double) * (size_t)n);
            if (!z) { bad = 1; continue; }
            const double ks = (kv_dtype == OR_E4M3) ? (double)k_scale[g] : 1.0;
            const double vs = (kv_dtype == OR_E4M3) ? (double)v_scale[g] : 1.0;
            for (int32_t hh = 0; hh < G; ++hh) {
                const int32_t h = g * G + hh;
                const int64_t qbase = ((int64_t)b * H_q + h) * D;
                /* logits */
                for (int32_t j = 0; j < n; ++j) {
                    const int64_t kbase = ((tok_off[b] + j) * H_kv + g) * (int64_t)D;
                    double dot = 0.0;
                    for (int32_t i = 0; i < D; ++i)
                        dot += widen(q, q_dtype, qbase + i) * (widen(K, kv_dtype, kbase + i) * ks);
                    z[j] = s * dot;
                }
                /* pass 1: max */
                double m = z[0];
                for (int32_t j = 1; j < n; ++j) if (z[j] > m) m = z[j];
                /* pass 2: exponentials, their sum, and the weighted sum of V */
                double l = 0.0;
                double* o = out + qbase;
                for (int32_t j = 0; j < n; ++j) {
                    const double e = exp(z[j] - m);
                    l += e;
                    const int64_t vbase = ((tok_off[b] + j) * H_kv + g) * (int64_t)D;
                    for (int32_t i = 0; i < D; ++i) o[i] += e * (widen(V, kv_dtype, vbase + i) * vs);
                }
                for (int32_t i = 0; i < D; ++i) o[i] /= l;
            }
            free(z);
        }
    }
    (void)nthreads;
    return bad ? -1 : 0;
}

/* ------------------------------------------------------------------------
 * Multi-query attention over de-paged K/V (a prompt chunk, or a whole
 * prompt, attending through the cache).
 *
 * [mlqm] 三 describes the prefill stage: every prompt token's Q, K and V are
 * computed at once, all K/V are written to the cache, and the queries attend
 * in parallel; [mlqm] 七 turns on chunked prefill, where a long prompt goes in
 * pieces.  Sequence s holds n_s = lens[s] tokens in total (its K/V appended
 * before the call) and brings q_len_s = q_start[s+1] - q_start[s] query
 * tokens: the last q_len_s positions.  Query token i of s sits at position
 * p = n_s - q_len_s + i and reads the positions j it may see:
 *   causal != 0:  j = 0 .. p      (a chunk of one token is exactly decode)
 *   causal == 0:  j = 0 .. n_s-1  (every token sees the whole context, as the
 *                                  prefill listing of [mlqm] 四 computes)
 *   z_j = scale * <q[t][h], K_s[j][g]>,  out[t][h] = sum_j softmax(z)_j V_s[j][g]
 * with t = q_start[s] + i and g = floor(h / G).  FP8 values are
 * decode(code) * scale of their head, as for decode.
 * ---------------------------------------------------------------------- */
int oracle_prefill_attention(int32_t S, int32_t H_q, int32_t H_kv, int32_t D,
                             const void* q, int32_t q_dtype, const int64_t* q_start,
                             const void* K, const void* V, int32_t kv_dtype,
                             const int64_t* tok_off, const int32_t* lens,
                             const float* k_scale, const float* v_scale,
                             float scale, int32_t causal, int32_t nthreads, double* out) {
    if (S < 0 || H_q <= 0 || H_kv <= 0 || D <= 0 || H_q % H_kv != 0) return -1;
    if (kv_dtype == OR_E4M3 && (!k_scale || !v_scale)) return -1;
    for (int32_t s = 0; s < S; ++s)
        if (q_start[s + 1] < q_start[s] || q_start[s + 1] - q_start[s] > lens[s]) return -1;
    const int32_t G = H_q / H_kv;
    const double sc = (double)scale;
    const int64_t T = q_start[S];
    int bad = 0;
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : omp_get_max_threads()) reduction(|| : bad)
#endif
    for (int64_t t = 0; t < T; ++t) {
        int32_t s = 0;                                  /* the sequence of query token t */
        while (q_start[s + 1] <= t) ++s;
        const int32_t n = lens[s];
        const int64_t q_len = q_start[s + 1] - q_start[s];
        const int64_t p = n - q_len + (t - q_start[s]);
        const int64_t last = causal ? p : n - 1;        /* newest position this token sees */
        double* z = (double*)malloc(sizeof(double) * (size_t)(last + 1));
        if (!z) { bad = 1; continue; }
        for (int32_t h = 0; h < H_q; ++h) {
            const int32_t g = h / G;
            const double ks = (kv_dtype == OR_E4M3) ? (double)k_scale[g] : 1.0;
            const double vs = (kv_dtype == OR_E4M3) ? (double)v_scale[g] : 1.0;
            const int64_t qbase = (t * H_q + h) * D;
            double* o = out + qbase;
            for (int32_t i = 0; i < D; ++i) o[i] = 0.0;
            for (int64_t j = 0; j <= last; ++j) {
                const int64_t kbase = ((tok_off[s] + j) * H_kv + g) * (int64_t)D;
                double dot = 0.0;
                for (int32_t i = 0; i < D; ++i)
                    dot += widen(q, q_dtype, qbase + i) * (widen(K, kv_dtype, kbase + i) * ks);
                z[j] = sc * dot;
            }
            double m = z[0];
            for (int64_t j = 1; j <= last; ++j) if (z[j] > m) m = z[j];
            double l = 0.0;
            for (int64_t j = 0; j <= last; ++j) {
                const double e = exp(z[j] - m);
                l += e;
                const int64_t vbase = ((tok_off[s] + j) * H_kv + g) * (int64_t)D;
                for (int32_t i = 0; i < D; ++i) o[i] += e * (widen(V, kv_dtype, vbase + i) * vs);
            }
            for (int32_t i = 0; i < D; ++i) o[i] /= l;
        }
        free(z);
    }
    return bad ? -1 : 0;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
