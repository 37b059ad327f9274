/*
 * Paged GQA attention -- the CPU oracle (test infrastructure, never product).
 *
 * Plain, slow, obviously correct fp64 C.  Only the tests, the smoke check and
 * the benchmark's CPU-baseline leg call this code; the HIP library never links
 * or includes it, and it includes nothing from the HIP library.
 *
 * Inputs are bf16 bit patterns (uint16) widened exactly to double, as the RL.cu
 * "Add Cuda Kernel" page's tests feed their CPU reference the already-rounded
 * values (section "tests/test_attention.cu", prefill test setup).  `scale` is
 * the fp32 value the GPU receives, widened.
 *
 * Every routine computes the definition directly: gather the sequence's keys
 * and values through the block table, form all scores, take the exact maximum,
 * exponentiate, normalize, weight the values.  No tiling, no online softmax,
 * no reordering beyond what the definitions state.
 *
 * Pins (tests/test_oracle.py): brute-force attention over contiguous K/V on
 * tiny inputs, closed forms (one token returns its value; equal keys or a zero
 * query return the mean of V), block-shuffle and V-scaling invariance,
 * split-equals-unsplit for the partial/merge pair, causal prefill against a
 * textbook square-causal brute force, and one-row prefill against decode.
 *
 * ORACLE_MUTANT selects a planted mistake (0 = none).  The test suite builds
 * each mutant into a scratch library and requires that some pin rejects it.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#ifndef ORACLE_MUTANT
#define ORACLE_MUTANT 0
#endif

static double bf16_to_double(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

int oracle_mutant(void) { return ORACLE_MUTANT; }

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* kv head serving query head h: consecutive query heads share one kv head,
 * the group of H_q / H_kv query heads mapping to it in order (RL.cu page,
 * the head mapping of its attention header). */
static int kv_head_of(int h, int Hq, int Hkv) {
#if ORACLE_MUTANT == 2
    return h % Hkv;
#else
    return (int)(((long)h * Hkv) / Hq);
#endif
}

/* A KV cache as the oracle reads it: bf16 bit patterns, or fp64 values (a
 * dequantized FP8 cache).  Element (block, kv head, slot, d) lives at
 *   layout 0: [num_blocks, H_kv, block_size, D]            (row-major tile)
 *   layout 1: [num_blocks, H_kv, D / 8, block_size, 8]     (x-packed K)
 *   layout 2: [num_blocks, H_kv, D, block_size]            (transposed V)
 * (layouts 1 and 2 are the BI-V100 page's key and value caches, section 3
 * "Paged K/V Gather", with x = 16 bytes / sizeof(bf16) = 8). */
#define XPACK 8
typedef struct {
    const uint16_t *bf16;
    const double *f64;
    int layout, bs, D;
} kv_cache_t;

/* Element offset of dim d of the row that starts at row-major offset `row`
 * ((block * H_kv + head) * bs + slot) * D. */
static long kv_index(kv_cache_t c, long row, int d) {
    if (c.layout == 0) return row + d;
    long tile = row / ((long)c.bs * c.D) * ((long)c.bs * c.D);
    long slot = (row / c.D) % c.bs;
    if (c.layout == 1) {
#if ORACLE_MUTANT == 19
        return tile + (long)(d % XPACK) * (c.bs * XPACK) + slot * XPACK + d / XPACK;
#else
        return tile + (long)(d / XPACK) * (c.bs * XPACK) + slot * XPACK + d % XPACK;
#endif
    }
    return tile + (long)d * c.bs + slot;
}

static double kv_elem(kv_cache_t c, long row, int d) {
    long i = kv_index(c, row, d);
    return c.bf16 ? bf16_to_double(c.bf16[i]) : c.f64[i];
}

/* Element offset of token t's row of kv head g for sequence s: the logical
 * block t / bs is looked up in the block table, the slot is t % bs (RL.cu page,
 * paged decode kernel: "logical block index -> physical block in the pool";
 * cache layout [num_blocks, H_kv, block_size, D]). */
static long kv_row(const int32_t *block_tables, int s, int t, int g, int Hkv, int bs, int D,
                   int mbps) {
    long phys = block_tables[(long)s * mbps + t / bs];
#if ORACLE_MUTANT == 4
    int slot = (t + 1) % bs;
#else
    int slot = t % bs;
#endif
    return ((phys * Hkv + g) * (long)bs + slot) * (long)D;
}

static const uint16_t *q_row(const uint16_t *q, long row, int h, int Hq, int D, long rows) {
#if ORACLE_MUTANT == 14
    (void)Hq;
    return q + ((long)h * rows + row) * D;
#else
    (void)rows;
    return q + (row * Hq + h) * (long)D;
#endif
}

/* Scaled score z_t = scale * q . k_t (BI-V100 design page, section 1
 * "Problem Definition": softmax(Q[h] K[t]^T / sqrt(d)) V[t]). */
static double score(const uint16_t *qr, kv_cache_t k, long kr, int D, double scale) {
    double acc = 0.0;
    for (int d = 0; d < D; ++d) acc += bf16_to_double(qr[d]) * kv_elem(k, kr, d);
#if ORACLE_MUTANT == 1
    (void)scale;
    return acc;
#else
    return scale * acc;
#endif
}

/* softmax over keys [t0, t1) of sequence s, weighted sum of values:
 * m = max z, l = sum exp(z - m), out = sum exp(z - m) v / l.
 * Returns m and l through the pointers (used by the partial routine). */
static void attend_range(const uint16_t *qr, kv_cache_t k_cache, kv_cache_t v_cache,
                         const int32_t *block_tables, int s, int g, int t0, int t1,
                         int Hkv, int bs, int D, int mbps, double scale,
                         double *z, double *out, double *m_out, double *l_out) {
#if ORACLE_MUTANT == 3
    t1 += 1; /* reads one slot past the end */
#endif
    int n = t1 - t0;
    double m = -INFINITY;
    for (int i = 0; i < n; ++i) {
        z[i] = score(qr, k_cache, kv_row(block_tables, s, t0 + i, g, Hkv, bs, D, mbps), D, scale);
        if (z[i] > m) m = z[i];
    }
    double l = 0.0;
    for (int i = 0; i < n; ++i) {
#if ORACLE_MUTANT == 5
        z[i] = exp(m - z[i]);
#else
        z[i] = exp(z[i] - m);
#endif
#if ORACLE_MUTANT == 7
        if (i > 0) l += z[i]; /* drops the first term of the denominator */
#else
        l += z[i];
#endif
    }
    for (int d = 0; d < D; ++d) out[d] = 0.0;
    for (int i = 0; i < n; ++i) {
        const long vr = kv_row(block_tables, s, t0 + i, g, Hkv, bs, D, mbps);
#if ORACLE_MUTANT == 6
        for (int d = 0; d < D; ++d) out[d] += z[i] * kv_elem(k_cache, vr, d);
#else
        for (int d = 0; d < D; ++d) out[d] += z[i] * kv_elem(v_cache, vr, d);
#endif
    }
    for (int d = 0; d < D; ++d) out[d] /= l;
    *m_out = m;
    *l_out = l;
}

/* O1 -- decode output.  out[s, h, :] = softmax(scale * q[s,h] . K_s) V_s over
 * the seq_lens[s] tokens of sequence s (seq_lens counts the current token,
 * RL.cu page, attention.cuh comment on seq_lens).  A zero length writes zeros. */
static int decode_impl(const uint16_t *q, kv_cache_t k_cache, kv_cache_t v_cache,
                       const int32_t *block_tables, const int32_t *seq_lens,
                       int S, int Hq, int Hkv, int D, int bs, int mbps, float scale, double *out) {
    if (Hq % Hkv != 0) return 2;
    long pairs = (long)S * Hq;
#pragma omp parallel for schedule(dynamic, 1)
    for (long i = 0; i < pairs; ++i) {
        int s = (int)(i / Hq), h = (int)(i % Hq);
        int L = seq_lens[s];
        double *o = out + i * D;
        if (L <= 0) { for (int d = 0; d < D; ++d) o[d] = 0.0; continue; }
        double *z = (double *)malloc(sizeof(double) * (size_t)(L + 1));
        double m, l;
        attend_range(q_row(q, s, h, Hq, D, S), k_cache, v_cache, block_tables, s,
                     kv_head_of(h, Hq, Hkv), 0, L, Hkv, bs, D, mbps, (double)scale, z, o, &m, &l);
        free(z);
    }
    return 0;
}

/* O2 -- decode partials.  Partition p of sequence s covers tokens
 * [p*P, min((p+1)*P, L)); it yields the exact max of its scaled scores
 * (max_logits), the sum of exp(z - max) (exp_sums) and the value average
 * weighted by exp(z - max) / exp_sum (tmp_out).  The BI-V100 design page
 * (section 2, "attention_partial") keeps the unnormalized weighted sum; the
 * normalized form stored here differs from it by the factor exp_sum, which the
 * merge multiplies back.  Partitions at or beyond ceil(L / P) are not written. */
static int partials_impl(const uint16_t *q, kv_cache_t k_cache, kv_cache_t v_cache,
                         const int32_t *block_tables, const int32_t *seq_lens,
                         int S, int Hq, int Hkv, int D, int bs, int mbps, float scale,
                         int P, int NP, double *max_logits, double *exp_sums, double *tmp_out) {
    if (Hq % Hkv != 0 || P <= 0) return 2;
    long work = (long)S * Hq * NP;
#pragma omp parallel for schedule(dynamic, 1)
    for (long i = 0; i < work; ++i) {
        int p = (int)(i % NP);
        long sh = i / NP;
        int s = (int)(sh / Hq), h = (int)(sh % Hq);
        int L = seq_lens[s];
        int nparts = (L + P - 1) / P;
        if (p >= nparts) continue;
        int t0 = p * P;
#if ORACLE_MUTANT == 9
        int t1 = (p + 1) * P + 1 < L ? (p + 1) * P + 1 : L;
#else
        int t1 = (p + 1) * P < L ? (p + 1) * P : L;
#endif
        double *z = (double *)malloc(sizeof(double) * (size_t)(t1 - t0 + 1));
        double m, l;
        double *o = tmp_out + i * D;
        attend_range(q_row(q, s, h, Hq, D, S), k_cache, v_cache, block_tables, s,
                     kv_head_of(h, Hq, Hkv), t0, t1, Hkv, bs, D, mbps, (double)scale, z, o, &m, &l);
#if ORACLE_MUTANT == 8
        for (int d = 0; d < D; ++d) o[d] *= l;
#endif
        max_logits[i] = m;
        exp_sums[i] = l;
        free(z);
    }
    return 0;
}

int oracle_decode(const uint16_t *q, const uint16_t *k_cache, const uint16_t *v_cache,
                  const int32_t *block_tables, const int32_t *seq_lens,
                  int S, int Hq, int Hkv, int D, int bs, int mbps, float scale, double *out) {
    kv_cache_t k = {k_cache, NULL, 0, bs, D}, v = {v_cache, NULL, 0, bs, D};
    return decode_impl(q, k, v, block_tables, seq_lens, S, Hq, Hkv, D, bs, mbps, scale, out);
}

int oracle_decode_partials(const uint16_t *q, const uint16_t *k_cache, const uint16_t *v_cache,
                           const int32_t *block_tables, const int32_t *seq_lens,
                           int S, int Hq, int Hkv, int D, int bs, int mbps, float scale,
                           int P, int NP, double *max_logits, double *exp_sums, double *tmp_out) {
    kv_cache_t k = {k_cache, NULL, 0, bs, D}, v = {v_cache, NULL, 0, bs, D};
    return partials_impl(q, k, v, block_tables, seq_lens, S, Hq, Hkv, D, bs, mbps, scale, P, NP,
                         max_logits, exp_sums, tmp_out);
}

/* O1 and O2 over fp64 caches: the same definitions with K and V given as
 * values (a dequantized FP8 cache, see oracle_fp8_dequant). */
int oracle_decode_f64kv(const uint16_t *q, const double *k_cache, const double *v_cache,
                        const int32_t *block_tables, const int32_t *seq_lens,
                        int S, int Hq, int Hkv, int D, int bs, int mbps, float scale, double *out) {
    kv_cache_t k = {NULL, k_cache, 0, bs, D}, v = {NULL, v_cache, 0, bs, D};
    return decode_impl(q, k, v, block_tables, seq_lens, S, Hq, Hkv, D, bs, mbps, scale, out);
}

int oracle_decode_partials_f64kv(const uint16_t *q, const double *k_cache, const double *v_cache,
                                 const int32_t *block_tables, const int32_t *seq_lens,
                                 int S, int Hq, int Hkv, int D, int bs, int mbps, float scale,
                                 int P, int NP, double *max_logits, double *exp_sums,
                                 double *tmp_out) {
    kv_cache_t k = {NULL, k_cache, 0, bs, D}, v = {NULL, v_cache, 0, bs, D};
    return partials_impl(q, k, v, block_tables, seq_lens, S, Hq, Hkv, D, bs, mbps, scale, P, NP,
                         max_logits, exp_sums, tmp_out);
}

/* O1 and O2 over the BI-V100 page's cache layouts (x-packed K, transposed
 * V; see kv_cache_t): the same definitions, only the element addresses
 * differ. */
int oracle_decode_xpacked(const uint16_t *q, const uint16_t *k_cache, const uint16_t *v_cache,
                          const int32_t *block_tables, const int32_t *seq_lens,
                          int S, int Hq, int Hkv, int D, int bs, int mbps, float scale, double *out) {
    kv_cache_t k = {k_cache, NULL, 1, bs, D}, v = {v_cache, NULL, 2, bs, D};
    return decode_impl(q, k, v, block_tables, seq_lens, S, Hq, Hkv, D, bs, mbps, scale, out);
}

int oracle_decode_partials_xpacked(const uint16_t *q, const uint16_t *k_cache,
                                   const uint16_t *v_cache, const int32_t *block_tables,
                                   const int32_t *seq_lens, int S, int Hq, int Hkv, int D, int bs,
                                   int mbps, float scale, int P, int NP, double *max_logits,
                                   double *exp_sums, double *tmp_out) {
    kv_cache_t k = {k_cache, NULL, 1, bs, D}, v = {v_cache, NULL, 2, bs, D};
    return partials_impl(q, k, v, block_tables, seq_lens, S, Hq, Hkv, D, bs, mbps, scale, P, NP,
                         max_logits, exp_sums, tmp_out);
}

/* O1 and O2 over a token-granular cache (the AstrAI page's decode with
 * page_size=1: "kv_indptr" gives each request's KV length, the page indices
 * translate logical positions to physical slots).  Sequence s has
 * L = kv_indptr[s+1] - kv_indptr[s] tokens; token t's K/V row of kv head g is
 * cache[kv_indices[kv_indptr[s] + t], g, :] in a [num_slots, H_kv, D] cache,
 * i.e. the block-table walk with one-token blocks whose table row is
 * kv_indices + kv_indptr[s]. */
static int tokens_L(const int32_t *kv_indptr, int s) {
#if ORACLE_MUTANT == 20
    return kv_indptr[s + 1]; /* the offset taken for the length */
#else
    return kv_indptr[s + 1] - kv_indptr[s];
#endif
}

int oracle_decode_tokens(const uint16_t *q, const uint16_t *k_cache, const uint16_t *v_cache,
                         const int32_t *kv_indptr, const int32_t *kv_indices, int S, int Hq,
                         int Hkv, int D, float scale, double *out) {
    if (Hq % Hkv != 0) return 2;
    kv_cache_t k = {k_cache, NULL, 0, 1, D}, v = {v_cache, NULL, 0, 1, D};
    long pairs = (long)S * Hq;
#pragma omp parallel for schedule(dynamic, 1)
    for (long i = 0; i < pairs; ++i) {
        int s = (int)(i / Hq), h = (int)(i % Hq);
        int L = tokens_L(kv_indptr, s);
        double *o = out + i * D;
        if (L <= 0) { for (int d = 0; d < D; ++d) o[d] = 0.0; continue; }
        double *z = (double *)malloc(sizeof(double) * (size_t)(L + 1));
        double m, l;
        attend_range(q_row(q, s, h, Hq, D, S), k, v, kv_indices + kv_indptr[s], 0,
                     kv_head_of(h, Hq, Hkv), 0, L, Hkv, 1, D, L, (double)scale, z, o, &m, &l);
        free(z);
    }
    return 0;
}

int oracle_decode_partials_tokens(const uint16_t *q, const uint16_t *k_cache,
                                  const uint16_t *v_cache, const int32_t *kv_indptr,
                                  const int32_t *kv_indices, int S, int Hq, int Hkv, int D,
                                  float scale, int P, int NP, double *max_logits,
                                  double *exp_sums, double *tmp_out) {
    if (Hq % Hkv != 0 || P <= 0) return 2;
    kv_cache_t k = {k_cache, NULL, 0, 1, D}, v = {v_cache, NULL, 0, 1, D};
    long work = (long)S * Hq * NP;
#pragma omp parallel for schedule(dynamic, 1)
    for (long i = 0; i < work; ++i) {
        int p = (int)(i % NP);
        long sh = i / NP;
        int s = (int)(sh / Hq), h = (int)(sh % Hq);
        int L = tokens_L(kv_indptr, s);
        if (p >= (L + P - 1) / P) continue;
        int t0 = p * P, t1 = (p + 1) * P < L ? (p + 1) * P : L;
        double *z = (double *)malloc(sizeof(double) * (size_t)(t1 - t0 + 1));
        double m, l;
        attend_range(q_row(q, s, h, Hq, D, S), k, v, kv_indices + kv_indptr[s], 0,
                     kv_head_of(h, Hq, Hkv), t0, t1, Hkv, 1, D, L, (double)scale, z,
                     tmp_out + i * D, &m, &l);
        max_logits[i] = m;
        exp_sums[i] = l;
        free(z);
    }
    return 0;
}

/* O3 -- cross-partition merge (BI-V100 design page, section 2 "combine" and
 * "Level 3: Cross-Partition Coordination"): with M = max_p m_p and weights
 * w_p = exp(m_p - M) * l_p, out = sum_p w_p * o_p / sum_p w_p over the
 * ceil(L / P) partitions that exist. */
int oracle_reduce(const double *max_logits, const double *exp_sums, const double *tmp_out,
                  const int32_t *seq_lens, int S, int Hq, int D, int P, int NP, double *out) {
    if (P <= 0) return 2;
    long pairs = (long)S * Hq;
#pragma omp parallel for schedule(dynamic, 1)
    for (long i = 0; i < pairs; ++i) {
        int s = (int)(i / Hq);
        int L = seq_lens[s];
        int nparts = (L + P - 1) / P;
        double *o = out + i * D;
        for (int d = 0; d < D; ++d) o[d] = 0.0;
        if (nparts <= 0) continue;
        const double *ml = max_logits + i * NP;
        const double *es = exp_sums + i * NP;
        double M = -INFINITY;
        for (int p = 0; p < nparts; ++p) if (ml[p] > M) M = ml[p];
        double wsum = 0.0;
        for (int p = 0; p < nparts; ++p) {
#if ORACLE_MUTANT == 10
            double w = exp(ml[p] - M);
#else
            double w = exp(ml[p] - M) * es[p];
#endif
            wsum += w;
            const double *op = tmp_out + (i * NP + p) * (long)D;
            for (int d = 0; d < D; ++d) o[d] += w * op[d];
        }
        for (int d = 0; d < D; ++d) o[d] /= wsum;
    }
    return 0;
}

/* O4 -- ragged paged prefill.  Sequence s owns query rows
 * [cu[s], cu[s+1]) of the packed [total_q, H_q, D] tensor (AstrAI page,
 * "Q Scheduling and KV Addressing": qo_indptr).  Its n = cu[s+1] - cu[s] new
 * tokens are the last n of its seq_lens[s] cached-plus-new tokens, so row j
 * sits at absolute position c + j with c = L - n, and it attends to keys
 * t <= c + j (the causal rule of the RL.cu page's prefill kernel, aligned to
 * the end of the context). */
int oracle_prefill(const uint16_t *q, const uint16_t *k_bits, const uint16_t *v_bits,
                   const int32_t *block_tables, const int32_t *seq_lens, const int32_t *cu_seqlens,
                   int S, int total_q, int Hq, int Hkv, int D, int bs, int mbps, float scale,
                   double *out) {
    if (Hq % Hkv != 0) return 2;
    kv_cache_t k_cache = {k_bits, NULL, 0, bs, D}, v_cache = {v_bits, NULL, 0, bs, D};
    long work = (long)total_q * Hq;
    for (long i = 0; i < work * D; ++i) out[i] = 0.0;
#pragma omp parallel for schedule(dynamic, 1)
    for (long w = 0; w < work; ++w) {
        long row = w / Hq;
        int h = (int)(w % Hq);
        int s = 0;
        while (s < S && !(cu_seqlens[s] <= row && row < cu_seqlens[s + 1])) ++s;
        if (s >= S) continue;
        int n = cu_seqlens[s + 1] - cu_seqlens[s];
        int L = seq_lens[s];
        int c = L - n;
        if (c < 0) continue;
        int j = (int)(row - cu_seqlens[s]);
#if ORACLE_MUTANT == 11
        int t1 = c + j;         /* drops the diagonal */
#elif ORACLE_MUTANT == 12
        int t1 = j + 1;         /* top-left alignment */
#else
        int t1 = c + j + 1;     /* keys t <= c + j */
#endif
        if (t1 <= 0) continue;
        long qrow = row;
#if ORACLE_MUTANT == 13
        qrow = (row + 1) % total_q;
#endif
        double *z = (double *)malloc(sizeof(double) * (size_t)(t1 + 1));
        double m, l;
        attend_range(q_row(q, qrow, h, Hq, D, total_q), k_cache, v_cache, block_tables, s,
                     kv_head_of(h, Hq, Hkv), 0, t1, Hkv, bs, D, mbps, (double)scale, z,
                     out + w * D, &m, &l);
        free(z);
    }
    return 0;
}

/* ---- KV cache writes ------------------------------------------------------ */

/* KV append: the cache write that comes before decode and prefill (the AstrAI
 * page's backend layer is responsible for writing and reading the cache; the B200 page's paged
 * KV cache read/write).  Sequence s owns new rows [cu[s], cu[s+1]) of k_new /
 * v_new ([num_tokens, H_kv, D]); they are the last n = cu[s+1] - cu[s] of its
 * seq_lens[s] tokens, so row j goes to position c + j with c = L - n: block
 * table entry (c + j) / bs, slot (c + j) % bs -- the placement of the prefill
 * rows above.  k_cache / v_cache are updated in place; nothing else changes.
 * Returns 2 if some sequence has fewer tokens than new rows. */
static long append_position(int c, int j) {
#if ORACLE_MUTANT == 17
    return (long)c + j + 1;
#else
    return (long)c + j;
#endif
}

static int kv_append_impl(const uint16_t *k_new, const uint16_t *v_new,
                          const int32_t *block_tables, const int32_t *seq_lens,
                          const int32_t *cu_seqlens, int S, int Hkv, int D, int bs, int mbps,
                          uint16_t *k_cache, uint16_t *v_cache, int k_layout, int v_layout) {
    kv_cache_t kl = {NULL, NULL, k_layout, bs, D}, vl = {NULL, NULL, v_layout, bs, D};
    for (int s = 0; s < S; ++s) {
        int n = cu_seqlens[s + 1] - cu_seqlens[s];
        int c = seq_lens[s] - n;
        if (c < 0) return 2;
        for (int j = 0; j < n; ++j) {
            long pos = append_position(c, j);
            if (pos / bs >= mbps) continue;
            for (int g = 0; g < Hkv; ++g) {
                long dst = kv_row(block_tables, s, (int)pos, g, Hkv, bs, D, mbps);
                long src = ((long)(cu_seqlens[s] + j) * Hkv + g) * D;
                for (int d = 0; d < D; ++d) {
                    k_cache[kv_index(kl, dst, d)] = k_new[src + d];
                    v_cache[kv_index(vl, dst, d)] = v_new[src + d];
                }
            }
        }
    }
    return 0;
}

/* KV append into the BI-V100 page's layouts (x-packed K, transposed V). */
int oracle_kv_append_xpacked(const uint16_t *k_new, const uint16_t *v_new,
                             const int32_t *block_tables, const int32_t *seq_lens,
                             const int32_t *cu_seqlens, int S, int Hkv, int D, int bs, int mbps,
                             uint16_t *k_cache, uint16_t *v_cache) {
    return kv_append_impl(k_new, v_new, block_tables, seq_lens, cu_seqlens, S, Hkv, D, bs, mbps,
                          k_cache, v_cache, 1, 2);
}

int oracle_kv_append(const uint16_t *k_new, const uint16_t *v_new, const int32_t *block_tables,
                     const int32_t *seq_lens, const int32_t *cu_seqlens, int S, int Hkv, int D,
                     int bs, int mbps, uint16_t *k_cache, uint16_t *v_cache) {
    for (int s = 0; s < S; ++s) {
        int n = cu_seqlens[s + 1] - cu_seqlens[s];
        int c = seq_lens[s] - n;
        if (c < 0) return 2;
        for (int j = 0; j < n; ++j) {
            long pos = append_position(c, j);
            if (pos / bs >= mbps) continue;
            for (int g = 0; g < Hkv; ++g) {
                long dst = kv_row(block_tables, s, (int)pos, g, Hkv, bs, D, mbps);
                long src = ((long)(cu_seqlens[s] + j) * Hkv + g) * D;
                memcpy(k_cache + dst, k_new + src, sizeof(uint16_t) * (size_t)D);
                memcpy(v_cache + dst, v_new + src, sizeof(uint16_t) * (size_t)D);
            }
        }
    }
    return 0;
}

/* ---- FP8 (E4M3) KV cache -------------------------------------------------- */

/* Value of an OCP FP8 E4M3 ("e4m3fn") code: sign bit, 4 exponent bits with
 * bias 7, 3 mantissa bits; exponent field 0 holds the subnormals m * 2^-9;
 * codes 0x7F and 0xFF are NaN; there are no infinities, so the largest finite
 * magnitude is 1.75 * 2^8 = 448. */
double oracle_e4m3_value(int code) {
    int sgn = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) {
#if ORACLE_MUTANT == 18
        v = 0.0; /* drops the subnormals */
#else
        v = m * ldexp(1.0, -9);
#endif
    } else {
        v = ldexp(1.0 + m / 8.0, e - 7);
    }
    return sgn ? -v : v;
}

/* The 256 code values, computed once from oracle_e4m3_value (a cache of the
 * definition above, filled before any parallel region reads it). */
static double e4m3_table_[256];
static int e4m3_table_ready_ = 0;
static const double *e4m3_table(void) {
    if (!e4m3_table_ready_) {
        for (int c = 0; c < 256; ++c) e4m3_table_[c] = oracle_e4m3_value(c);
        e4m3_table_ready_ = 1;
    }
    return e4m3_table_;
}

/* The non-negative E4M3 code nearest to a >= 0: every finite magnitude code
 * 0x00..0x7E is tried; on a tie the even code (even last mantissa bit) wins.
 * Magnitudes past 448 land on 448. */
static int e4m3_nearest(float a) {
    const double *val = e4m3_table_;
    int best = 0;
    double bd = INFINITY;
    for (int c = 0; c <= 0x7E; ++c) {
        double d = fabs(val[c] - (double)a);
#if ORACLE_MUTANT == 15
        if (d < bd || (d == bd && c > best)) { /* ties away from zero */
#else
        if (d < bd || (d == bd && (c & 1) == 0)) {
#endif
            bd = d;
            best = c;
        }
    }
    return best;
}

#define E4M3_MAX 448.0f

/* FP8 quantization of rows of D bf16 values, one dequant scale per row (the
 * B200 page's "FP8 KV Quantize/Dequant" with a "per-position dequant scale":
 * one scale per cached position and kv head).  For each row:
 *   amax = max_d |x_d|;  scale = fp32(amax / 448);
 *   code_d = sign(x_d) | nearest E4M3 magnitude to fp32(|x_d| / scale)
 *   (ties to the even code, saturating at 448).
 * Both divisions are single-precision, correctly rounded.  A row of zeros gets
 * scale 0 and zero codes (with the sign of each zero).  Dequantized value =
 * value(code) * scale. */
static void quantize_row(const uint16_t *xr, int D, uint8_t *codes, float *scale) {
    float amax = 0.0f;
    for (int d = 0; d < D; ++d) {
        float a = fabsf((float)bf16_to_double(xr[d]));
        if (a > amax) amax = a;
    }
#if ORACLE_MUTANT == 16
    float s = amax / 240.0f; /* another FP8 variant's largest magnitude */
#else
    float s = amax / E4M3_MAX;
#endif
    *scale = s;
    for (int d = 0; d < D; ++d) {
        float v = (float)bf16_to_double(xr[d]);
        int sgn = signbit(v) ? 0x80 : 0;
        int mag = s > 0.0f ? e4m3_nearest(fabsf(v) / s) : 0;
        codes[d] = (uint8_t)(sgn | mag);
    }
}

int oracle_quantize_fp8(const uint16_t *x, long rows, int D, uint8_t *codes, float *scales) {
    e4m3_table();
#pragma omp parallel for schedule(static)
    for (long r = 0; r < rows; ++r) quantize_row(x + r * D, D, codes + r * D, scales + r);
    return 0;
}

/* value(code) * scale for rows of D codes with one scale each. */
int oracle_fp8_dequant(const uint8_t *codes, const float *scales, long rows, int D, double *out) {
    const double *val = e4m3_table();
#pragma omp parallel for schedule(static)
    for (long r = 0; r < rows; ++r)
        for (int d = 0; d < D; ++d)
            out[r * D + d] = val[codes[r * D + d]] * (double)scales[r];
    return 0;
}

/* KV append into an FP8 cache: each new (token, kv head) row of K and of V is
 * quantized as in oracle_quantize_fp8 and written with its scale to the same
 * position oracle_kv_append uses.  Caches: codes [num_blocks, H_kv, bs, D],
 * scales [num_blocks, H_kv, bs]. */
int oracle_kv_append_fp8(const uint16_t *k_new, const uint16_t *v_new, const int32_t *block_tables,
                         const int32_t *seq_lens, const int32_t *cu_seqlens, int S, int Hkv, int D,
                         int bs, int mbps, uint8_t *k_cache, uint8_t *v_cache, float *k_scales,
                         float *v_scales) {
    e4m3_table();
    uint8_t *row = (uint8_t *)malloc((size_t)D);
    for (int s = 0; s < S; ++s) {
        int n = cu_seqlens[s + 1] - cu_seqlens[s];
        int c = seq_lens[s] - n;
        if (c < 0) { free(row); return 2; }
        for (int j = 0; j < n; ++j) {
            long pos = append_position(c, j);
            if (pos / bs >= mbps) continue;
            for (int g = 0; g < Hkv; ++g) {
                long dst = kv_row(block_tables, s, (int)pos, g, Hkv, bs, D, mbps);
                long src = ((long)(cu_seqlens[s] + j) * Hkv + g) * D;
                float sc;
                quantize_row(k_new + src, D, row, &sc);
                memcpy(k_cache + dst, row, (size_t)D);
                k_scales[dst / D] = sc;
                quantize_row(v_new + src, D, row, &sc);
                memcpy(v_cache + dst, row, (size_t)D);
                v_scales[dst / D] = sc;
            }
        }
    }
    free(row);
    return 0;
}
