/*
 * oracle.c -- plain, slow fp64 CPU oracle for masked softmax attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the GPU library, and it never calls it.
 *
 * What it computes is the plain definition of attention, with no tiling,
 * blocking, online softmax or reordering:
 *
 *     s_j = scale * sum_d Q[i,d] K[j,d]          (fp64, d ascending)
 *     m   = max_j s_j,  w_j = exp(s_j - m),  Z = sum_j w_j   (j ascending)
 *     O[i,:] = sum_j (w_j / Z) V[j,:]                        (j ascending)
 *     lse = m + log(Z)
 *
 * over the allowed key set of each query row.  Sources:
 *  - "RFC: Gemma-4-31B-it train/rollout consistency" (RL-Kernel issue 415),
 *    section 3 "Architecture map": sliding and global layers are distinct
 *    attention cores with different head geometry and mask semantics;
 *    section 1 "Motivation", Phase B: vision tokens carry a bidirectional
 *    mask.
 *  - "Gemma-4-E4B-it multimodal baseline" (vllm.cpp PR 3476), commit log:
 *    an image expands into one contiguous run of soft tokens, which is the
 *    span that is bidirectional.
 *  - "Vime ROCm Attention operator ablation", section "Prerequisites": strict
 *    decode reads the paged KV cache directly through the block table.
 *
 * Readings taken where the pages are silent (every one is a reading, not a
 * page fact): the window W admits key j for query i when 0 <= i - j < W
 * (W keys including the query itself), W < 0 means no window (global
 * causal); a key j is also admitted, whatever the window, when i and j lie
 * in the same bidirectional span [s, e); GQA groups are contiguous, so query
 * head h reads KV head h / (Hq / Hkv); decode's query is the last token of
 * its sequence and its own key is already in the cache.
 *
 * Inputs may be bf16 bit patterns (converted exactly), fp32 or fp64.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_BF16 = 0, ORACLE_F32 = 1, ORACLE_F64 = 2 };

/* Exact widening of one stored element to fp64. */
static double load_elem(const void* base, int dtype, int64_t idx) {
    if (dtype == ORACLE_BF16) {
        uint32_t bits = ((uint32_t)((const uint16_t*)base)[idx]) << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return (double)f;
    }
    if (dtype == ORACLE_F32) return (double)((const float*)base)[idx];
    return ((const double*)base)[idx];
}

/* Is key j admitted for query i of a sequence?  i, j are positions within
 * the sequence; span_lo/span_hi are the sequence-relative bounds of the
 * span holding i, or -1 when i is in no span. */
static int allowed(int64_t i, int64_t j, int32_t window,
                   int64_t span_lo, int64_t span_hi) {
    int causal_ok = (j <= i) && (window < 0 || i - j < (int64_t)window);
    int span_ok = span_lo >= 0 && j >= span_lo && j < span_hi;
    return causal_ok || span_ok;
}

/* One query row against an explicit list of key rows.
 * q: pointer/offset of the query vector; key_off[n]: element offsets of the
 * key rows (same offsets serve V).  out: D doubles.  s: scratch, n doubles. */
static void attend_row(const void* q, int qt, int64_t q_off,
                       const void* k, const void* v, int kvt,
                       const int64_t* key_off, int64_t n, int32_t d,
                       double scale, double* s, double* out, double* lse) {
    double m = -INFINITY;
    for (int64_t a = 0; a < n; ++a) {
        double dot = 0.0;
        for (int32_t c = 0; c < d; ++c)
            dot += load_elem(q, qt, q_off + c) * load_elem(k, kvt, key_off[a] + c);
        s[a] = scale * dot;
        if (s[a] > m) m = s[a];
    }
    double z = 0.0;
    for (int64_t a = 0; a < n; ++a) {
        s[a] = exp(s[a] - m);
        z += s[a];
    }
    for (int32_t c = 0; c < d; ++c) out[c] = 0.0;
    for (int64_t a = 0; a < n; ++a) {
        double p = s[a] / z;
        for (int32_t c = 0; c < d; ++c) out[c] += p * load_elem(v, kvt, key_off[a] + c);
    }
    if (lse) *lse = m + log(z);
}

/*
 * Prefill over packed variable-length sequences.
 *   q   [T, hq, d], k/v [T, hkv, d]  (dtype codes above)
 *   o   [T, hq, d] fp64 out; lse [T, hq] fp64 out or NULL
 *   cu_seqlens[batch+1]: sequence b holds packed tokens [cu[b], cu[b+1])
 *   spans[num_spans][2]: packed [start, end) ranges, each inside one sequence
 *   rows: optional list of n_rows (token, head) pairs to compute; NULL = all.
 *     With a row list, o and lse are indexed by list position: o[n_rows, d],
 *     lse[n_rows].
 * Returns 0, or -1 on bad arguments.
 */
int oracle_prefill(const void* q, int qdtype, const void* k, const void* v,
                   int kvdtype, double* o, double* lse,
                   const int32_t* cu_seqlens, int32_t batch, int32_t hq,
                   int32_t hkv, int32_t d, int32_t window, double scale,
                   const int32_t* spans, int32_t num_spans,
                   const int64_t* rows, int64_t n_rows, int32_t threads) {
    if (batch < 0 || hq <= 0 || hkv <= 0 || d <= 0 || hq % hkv) return -1;
    const int64_t total = cu_seqlens[batch];
    const int32_t group = hq / hkv;
    int64_t max_len = 0;
    for (int32_t b = 0; b < batch; ++b) {
        int64_t len = cu_seqlens[b + 1] - cu_seqlens[b];
        if (len < 0) return -1;
        if (len > max_len) max_len = len;
    }
    /* Sequence id of every packed token. */
    int32_t* seq_of = (int32_t*)malloc(sizeof(int32_t) * (size_t)(total > 0 ? total : 1));
    for (int32_t b = 0; b < batch; ++b)
        for (int64_t t = cu_seqlens[b]; t < cu_seqlens[b + 1]; ++t) seq_of[t] = b;
    const int64_t n_work = rows ? n_rows : total * hq;
#ifdef _OPENMP
    if (threads > 0) omp_set_num_threads(threads);
#endif
    int bad = 0;
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)(max_len > 0 ? max_len : 1));
        int64_t* key_off = (int64_t*)malloc(sizeof(int64_t) * (size_t)(max_len > 0 ? max_len : 1));
#pragma omp for schedule(dynamic, 16)
        for (int64_t w = 0; w < n_work; ++w) {
            int64_t t = rows ? rows[2 * w] : w / hq;
            int32_t h = (int32_t)(rows ? rows[2 * w + 1] : w % hq);
            if (t < 0 || t >= total || h < 0 || h >= hq) {
#pragma omp atomic write
                bad = 1;
                continue;
            }
            int32_t b = seq_of[t];
            int64_t start = cu_seqlens[b], len = cu_seqlens[b + 1] - start;
            int64_t i = t - start;
            int64_t span_lo = -1, span_hi = -1;
            for (int32_t sp = 0; sp < num_spans; ++sp) {
                if (t >= spans[2 * sp] && t < spans[2 * sp + 1]) {
                    span_lo = spans[2 * sp] - start;
                    span_hi = spans[2 * sp + 1] - start;
                }
            }
            int32_t g = h / group;
            int64_t n = 0;
            for (int64_t j = 0; j < len; ++j)
                if (allowed(i, j, window, span_lo, span_hi))
                    key_off[n++] = ((start + j) * hkv + g) * (int64_t)d;
            double* out = o + (rows ? w : t * hq + h) * (int64_t)d;
            double* l = lse ? lse + (rows ? w : t * hq + h) : NULL;
            attend_row(q, qdtype, (t * hq + h) * (int64_t)d, k, v, kvdtype,
                       key_off, n, d, scale, s, out, l);
        }
        free(s);
        free(key_off);
    }
    free(seq_of);
    return bad ? -1 : 0;
}

/*
 * Single-token decode against a paged KV cache.
 *   q [batch, hq, d]; k_cache/v_cache [num_blocks, block_size, hkv, d]
 *   block_table [batch, max_blocks]; seq_lens[batch] counts the current token
 *   o [batch, hq, d] fp64 out; lse [batch, hq] fp64 out or NULL.
 * Key j of sequence b sits in physical block block_table[b][j / block_size],
 * slot j % block_size.  The query is position seq_lens[b] - 1.
 */
int oracle_decode(const void* q, int qdtype, const void* k_cache,
                  const void* v_cache, int kvdtype,
                  const int32_t* block_table, int32_t max_blocks,
                  const int32_t* seq_lens, int32_t batch, int32_t hq,
                  int32_t hkv, int32_t d, int32_t block_size, int32_t window,
                  double scale, double* o, double* lse, int32_t threads) {
    if (batch < 0 || hq <= 0 || hkv <= 0 || d <= 0 || hq % hkv || block_size <= 0)
        return -1;
    const int32_t group = hq / hkv;
    int64_t max_len = 1;
    for (int32_t b = 0; b < batch; ++b) {
        if (seq_lens[b] < 1 || seq_lens[b] > (int64_t)max_blocks * block_size) return -1;
        if (seq_lens[b] > max_len) max_len = seq_lens[b];
    }
#ifdef _OPENMP
    if (threads > 0) omp_set_num_threads(threads);
#endif
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)max_len);
        int64_t* key_off = (int64_t*)malloc(sizeof(int64_t) * (size_t)max_len);
#pragma omp for schedule(dynamic, 1)
        for (int64_t w = 0; w < (int64_t)batch * hq; ++w) {
            int32_t b = (int32_t)(w / hq), h = (int32_t)(w % hq), g = h / group;
            int64_t len = seq_lens[b], i = len - 1, n = 0;
            for (int64_t j = 0; j < len; ++j) {
                if (!allowed(i, j, window, -1, -1)) continue;
                int64_t blk = block_table[(int64_t)b * max_blocks + j / block_size];
                int64_t slot = j % block_size;
                key_off[n++] = ((blk * block_size + slot) * hkv + g) * (int64_t)d;
            }
            attend_row(q, qdtype, w * (int64_t)d, k_cache, v_cache, kvdtype,
                       key_off, n, d, scale, s, o + w * (int64_t)d,
                       lse ? lse + w : NULL);
        }
        free(s);
        free(key_off);
    }
    return 0;
}

/*
 * Gradient of prefill attention with respect to q, k and v for an upstream
 * gradient dout = dL/dO, by the chain rule applied to the definition above
 * (the derivative of softmax: dL/ds_j = p_j (dL/dp_j - sum_a p_a dL/dp_a)):
 *
 *     p_j    = exp(s_j - lse)                         (the row's softmax)
 *     o      = sum_j p_j V[j,:]
 *     delta  = sum_c dout[i,c] o[c]                   (= sum_j p_j dp_j)
 *     dp_j   = sum_c dout[i,c] V[j,c]
 *     ds_j   = p_j (dp_j - delta)
 *     dQ[i,:]  = scale * sum_j ds_j K[j,:]            (j ascending)
 *     dK[j,:] += scale * ds_j Q[i,:]                  (rows i ascending, then
 *     dV[j,:] += p_j dout[i,:]                         the group's heads)
 *
 * Same mask, GQA map and layouts as oracle_prefill.  Three passes: the
 * softmax statistics (lse, delta) of every (row, query head) needed, then
 * dq per (row, query head), then dk and dv per (key row, KV head), summed
 * over every row and query head that admits the key.
 *
 * dq_units / kv_units: optional lists of n_dq (token * hq + head) and n_kv
 * (token * hkv + kv head) indices; NULL means every one.  With a list, dq
 * (or dk and dv) is indexed by list position: dq [n_dq, d], dk / dv
 * [n_kv, d]; without, dq [T, hq, d] and dk / dv [T, hkv, d].  Statistics
 * are formed only for the rows the listed units read, so a few units of a
 * long sequence cost a few rows.  Outputs are fp64.  Returns 0, or -1 on bad
 * arguments.
 */
int oracle_prefill_backward_units(const void* q, int qdtype, const void* k, const void* v,
                                  int kvdtype, const void* dout, int dodtype,
                                  double* dq, double* dk, double* dv,
                                  const int32_t* cu_seqlens, int32_t batch, int32_t hq,
                                  int32_t hkv, int32_t d, int32_t window, double scale,
                                  const int32_t* spans, int32_t num_spans,
                                  const int64_t* dq_units, int64_t n_dq,
                                  const int64_t* kv_units, int64_t n_kv, int32_t threads) {
    if (batch < 0 || hq <= 0 || hkv <= 0 || d <= 0 || hq % hkv || n_dq < 0 || n_kv < 0)
        return -1;
    const int64_t total = cu_seqlens[batch];
    const int32_t group = hq / hkv;
    int64_t max_len = 1;
    for (int32_t b = 0; b < batch; ++b) {
        int64_t len = cu_seqlens[b + 1] - cu_seqlens[b];
        if (len < 0) return -1;
        if (len > max_len) max_len = len;
    }
    if (!dq_units) n_dq = total * hq;
    if (!kv_units) n_kv = total * hkv;
    for (int64_t u = 0; dq_units && u < n_dq; ++u)
        if (dq_units[u] < 0 || dq_units[u] >= total * hq) return -1;
    for (int64_t u = 0; kv_units && u < n_kv; ++u)
        if (kv_units[u] < 0 || kv_units[u] >= total * hkv) return -1;
    const int64_t nt = total > 0 ? total : 1;
    int32_t* seq_of = (int32_t*)malloc(sizeof(int32_t) * (size_t)nt);
    int64_t* span_lo = (int64_t*)malloc(sizeof(int64_t) * (size_t)nt);
    int64_t* span_hi = (int64_t*)malloc(sizeof(int64_t) * (size_t)nt);
    double* lse = (double*)malloc(sizeof(double) * (size_t)(nt * hq));
    double* delta = (double*)malloc(sizeof(double) * (size_t)(nt * hq));
    char* need = (char*)calloc((size_t)(nt * hq), 1);
    int64_t* rows = (int64_t*)malloc(sizeof(int64_t) * (size_t)(nt * hq));
    for (int32_t b = 0; b < batch; ++b)
        for (int64_t t = cu_seqlens[b]; t < cu_seqlens[b + 1]; ++t) {
            seq_of[t] = b;
            span_lo[t] = span_hi[t] = -1;
            for (int32_t sp = 0; sp < num_spans; ++sp)
                if (t >= spans[2 * sp] && t < spans[2 * sp + 1]) {
                    span_lo[t] = spans[2 * sp] - cu_seqlens[b];
                    span_hi[t] = spans[2 * sp + 1] - cu_seqlens[b];
                }
        }
    /* Which (row, query head) statistics the listed units read. */
    for (int64_t u = 0; u < n_dq; ++u) need[dq_units ? dq_units[u] : u] = 1;
    for (int64_t u = 0; u < n_kv; ++u) {
        int64_t w = kv_units ? kv_units[u] : u, tj = w / hkv;
        int32_t g = (int32_t)(w % hkv), b = seq_of[tj];
        int64_t start = cu_seqlens[b], len = cu_seqlens[b + 1] - start, j = tj - start;
        for (int64_t i = 0; i < len; ++i)
            if (allowed(i, j, window, span_lo[start + i], span_hi[start + i]))
                for (int32_t h = g * group; h < (g + 1) * group; ++h)
                    need[(start + i) * hq + h] = 1;
    }
    int64_t n_rows = 0;
    for (int64_t w = 0; w < total * hq; ++w)
        if (need[w]) rows[n_rows++] = w;
#ifdef _OPENMP
    if (threads > 0) omp_set_num_threads(threads);
#endif
    /* Pass 1: softmax statistics per needed (row, query head). */
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)max_len);
        int64_t* key_off = (int64_t*)malloc(sizeof(int64_t) * (size_t)max_len);
        double* o = (double*)malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(dynamic, 16)
        for (int64_t r = 0; r < n_rows; ++r) {
            int64_t w = rows[r], t = w / hq;
            int32_t h = (int32_t)(w % hq), g = h / group, b = seq_of[t];
            int64_t start = cu_seqlens[b], len = cu_seqlens[b + 1] - start, i = t - start;
            int64_t n = 0;
            for (int64_t j = 0; j < len; ++j)
                if (allowed(i, j, window, span_lo[t], span_hi[t]))
                    key_off[n++] = ((start + j) * hkv + g) * (int64_t)d;
            double l;
            attend_row(q, qdtype, w * (int64_t)d, k, v, kvdtype, key_off, n, d, scale, s, o, &l);
            lse[w] = l;
            double del = 0.0;
            for (int32_t c = 0; c < d; ++c) del += load_elem(dout, dodtype, w * (int64_t)d + c) * o[c];
            delta[w] = del;
        }
        free(s);
        free(key_off);
        free(o);
    }
    /* Pass 2: dq per listed (row, query head). */
#pragma omp parallel
    {
        int64_t* key_off = (int64_t*)malloc(sizeof(int64_t) * (size_t)max_len);
#pragma omp for schedule(dynamic, 16)
        for (int64_t u = 0; u < n_dq; ++u) {
            int64_t w = dq_units ? dq_units[u] : u, t = w / hq;
            int32_t h = (int32_t)(w % hq), g = h / group, b = seq_of[t];
            int64_t start = cu_seqlens[b], len = cu_seqlens[b + 1] - start, i = t - start;
            int64_t n = 0;
            for (int64_t j = 0; j < len; ++j)
                if (allowed(i, j, window, span_lo[t], span_hi[t]))
                    key_off[n++] = ((start + j) * hkv + g) * (int64_t)d;
            double del = delta[w];
            double* dqi = dq + u * (int64_t)d;
            for (int32_t c = 0; c < d; ++c) dqi[c] = 0.0;
            for (int64_t a = 0; a < n; ++a) {
                double dot = 0.0, dp = 0.0;
                for (int32_t c = 0; c < d; ++c) {
                    dot += load_elem(q, qdtype, w * (int64_t)d + c) * load_elem(k, kvdtype, key_off[a] + c);
                    dp += load_elem(dout, dodtype, w * (int64_t)d + c) * load_elem(v, kvdtype, key_off[a] + c);
                }
                double p = exp(scale * dot - lse[w]);
                double ds = p * (dp - del);
                for (int32_t c = 0; c < d; ++c) dqi[c] += scale * ds * load_elem(k, kvdtype, key_off[a] + c);
            }
        }
        free(key_off);
    }
    /* Pass 3: dk, dv per listed (key row, KV head). */
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t u = 0; u < n_kv; ++u) {
        int64_t w = kv_units ? kv_units[u] : u, tj = w / hkv;
        int32_t g = (int32_t)(w % hkv), b = seq_of[tj];
        int64_t start = cu_seqlens[b], len = cu_seqlens[b + 1] - start, j = tj - start;
        double* dkj = dk + u * (int64_t)d;
        double* dvj = dv + u * (int64_t)d;
        for (int32_t c = 0; c < d; ++c) dkj[c] = dvj[c] = 0.0;
        for (int64_t i = 0; i < len; ++i) {
            int64_t ti = start + i;
            if (!allowed(i, j, window, span_lo[ti], span_hi[ti])) continue;
            for (int32_t h = g * group; h < (g + 1) * group; ++h) {
                int64_t qo = (ti * hq + h) * (int64_t)d, ko = w * (int64_t)d;
                double dot = 0.0, dp = 0.0;
                for (int32_t c = 0; c < d; ++c) {
                    dot += load_elem(q, qdtype, qo + c) * load_elem(k, kvdtype, ko + c);
                    dp += load_elem(dout, dodtype, qo + c) * load_elem(v, kvdtype, ko + c);
                }
                double p = exp(scale * dot - lse[ti * hq + h]);
                double ds = p * (dp - delta[ti * hq + h]);
                for (int32_t c = 0; c < d; ++c) {
                    dkj[c] += scale * ds * load_elem(q, qdtype, qo + c);
                    dvj[c] += p * load_elem(dout, dodtype, qo + c);
                }
            }
        }
    }
    free(seq_of);
    free(span_lo);
    free(span_hi);
    free(lse);
    free(delta);
    free(need);
    free(rows);
    return 0;
}

/* Every dq, dk and dv: dq [T, hq, d], dk / dv [T, hkv, d]. */
int oracle_prefill_backward(const void* q, int qdtype, const void* k, const void* v,
                            int kvdtype, const void* dout, int dodtype,
                            double* dq, double* dk, double* dv,
                            const int32_t* cu_seqlens, int32_t batch, int32_t hq,
                            int32_t hkv, int32_t d, int32_t window, double scale,
                            const int32_t* spans, int32_t num_spans, int32_t threads) {
    return oracle_prefill_backward_units(q, qdtype, k, v, kvdtype, dout, dodtype, dq, dk, dv,
                                         cu_seqlens, batch, hq, hkv, d, window, scale, spans,
                                         num_spans, NULL, 0, NULL, 0, threads);
}

/*
 * The attention prologue of a layer: RMSNorm over the head dim of every
 * (row, head) vector of Q or K, then rotary position embedding (RoPE).
 * Sources: the layer's prologue names a Q/K RMSNorm for head dims 256 and
 * 512, a RoPE on the sliding layers and a proportional ("p") RoPE on the
 * global layers ("RFC: Gemma-4-31B-it train/rollout consistency", section 6,
 * items 4 and 6); the RMSNorm formula with an additive weight offset and
 * fp32 math is the one of "Gated RMSNorm CUDA kernel for the GDN block"
 * (Summary), without its gate.  The pages give no epsilon, offset, rotary
 * width, frequency base or pairing; they are arguments here.  Readings
 * (every one a reading, not a page fact):
 *
 *   norm:  r = 1 / sqrt(mean_d x_d^2 + eps),  y_d = x_d * r * (offset + w_d)
 *          (skipped when weight is NULL: y = x);
 *   rope:  for i < R/2 the pair (y_i, y_{i+R/2}) turns by the angle
 *          pos * theta^(-2i/F):  (a, b) -> (a cos - b sin, a sin + b cos);
 *          dims R .. D-1 pass through.  R = D is the full RoPE; R < D with
 *          F = D is the proportional reading (the turned dims keep the
 *          frequencies of a full RoPE over D), F = R the plain partial one.
 *
 * x [rows, heads, d] (bf16 bits, fp32 or fp64), positions [rows], weight
 * [d] or NULL, out [rows, heads, d] fp64.
 */
int oracle_qk_prologue(const void* x, int xdtype, int64_t rows, int32_t heads, int32_t d,
                       const int32_t* positions, const void* weight, int wdtype, double eps,
                       double offset, int32_t rotary_dims, int32_t freq_dims, double theta,
                       double* out, int32_t threads) {
    if (rows < 0 || heads <= 0 || d <= 0 || rotary_dims < 0 || rotary_dims > d ||
        rotary_dims % 2 != 0 || (rotary_dims > 0 && (freq_dims <= 0 || !(theta > 0))) ||
        !(eps >= 0) || (rows > 0 && positions == NULL))
        return -1;
#ifdef _OPENMP
    if (threads > 0) omp_set_num_threads(threads);
#pragma omp parallel for schedule(dynamic, 16)
#else
    (void)threads;
#endif
    for (int64_t rh = 0; rh < rows * heads; ++rh) {
        const int64_t base = rh * d;
        const int64_t row = rh / heads;
        double* y = out + base;
        if (weight != NULL) {
            double ss = 0.0;
            for (int32_t j = 0; j < d; ++j) {
                const double v = load_elem(x, xdtype, base + j);
                ss += v * v;
            }
            const double r = 1.0 / sqrt(ss / d + eps);
            for (int32_t j = 0; j < d; ++j)
                y[j] = load_elem(x, xdtype, base + j) * r * (offset + load_elem(weight, wdtype, j));
        } else {
            for (int32_t j = 0; j < d; ++j) y[j] = load_elem(x, xdtype, base + j);
        }
        const int32_t half = rotary_dims / 2;
        const double pos = (double)positions[row];
        for (int32_t i = 0; i < half; ++i) {
            const double ang = pos * pow(theta, -2.0 * i / freq_dims);
            const double c = cos(ang), s = sin(ang);
            const double a = y[i], b = y[i + half];
            y[i] = a * c - b * s;
            y[i + half] = a * s + b * c;
        }
    }
    return 0;
}

/* Number of threads an OpenMP region of this library runs with. */
int oracle_num_threads(int32_t threads) {
#ifdef _OPENMP
    if (threads > 0) omp_set_num_threads(threads);
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        n = omp_get_num_threads();
    }
    return n;
#else
    (void)threads;
    return 1;
#endif
}
