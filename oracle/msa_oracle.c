/*
 * msa_oracle.c -- plain, slow, fp64 CPU oracle of the MiniMax Sparse Attention
 * (MSA) hot path and of the DSA lightning-indexer variant.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the test-suite, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no code, header, table or helper with
 * the HIP path.
 *
 * Sources (web pages; cited by title and section):
 *  [MSA-PR]  "Add MiniMax-M3 (MSA: MiniMax Sparse Attention) support",
 *            llama.cpp pull request 24908: sections "Overview",
 *            "Implementation", "Limitations", and the review thread (the
 *            RADV validation comment and the unified-KV diagnosis comment).
 *  [MSA-LOG] llama.cpp compare page (b10146), commit log entry "mtmd: Add
 *            Vision Support for Minimax-M3 (#25113)" that squashes the MSA
 *            history ("unified selection semantics", "force F32 indexer
 *            score accum", "set default cache type to F32").
 *  [DSA-PR]  "deepseek2 : GLM-DSA sparse attention (lightning indexer),
 *            --dsa off by default", ik_llama.cpp pull request 2045: sections
 *            "What this does" and "Validation of the DSA path itself".
 *
 * Everything is computed in IEEE double.  Every stored input (f32, bf16,
 * fp16) converts to double exactly, so the only rounding is that of the
 * fp64 sums and of exp().
 *
 * Readings taken where the pages leave a step open (each one is also listed
 * with its reason in the design notes of the repository):
 *  - key j is visible to a query at position p iff j <= p (self included);
 *  - a block's score is the max over its VISIBLE keys only (the causal mask
 *    is added before the max-pool, [MSA-PR] Implementation);
 *  - the "large positive bias" on the local block is read as "the local
 *    block ranks first", which equals any finite bias larger than the score
 *    range without float absorption;
 *  - ties rank the lower block (or token) id first; selected ids are
 *    reported in ascending order and padded with -1;
 *  - query head h belongs to group floor(h / heads_per_group);
 *  - softmax scale is a parameter (1/sqrt(128) in every workload), no sink,
 *    no soft-cap;
 *  - slot == position, blocks are [block*b, block*b + block) in slots;
 *  - DSA: the key rotation is the orthonormal Sylvester Hadamard transform
 *    (entries +-1/sqrt(n)), rounded once to fp16 (round to nearest, ties to
 *    even); queries are not rotated; the kept count is min(top_k, p + 1);
 *    there is no local forcing.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_API __attribute__((visibility("default")))

/* ------------------------------------------------------------------------ */
/* Exact conversions of the storage formats to double, and double -> fp16.  */
/* ------------------------------------------------------------------------ */

/* bf16 is the top 16 bits of an IEEE binary32. */
ORACLE_API double oracle_bf16_to_f64(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
ORACLE_API double oracle_f16_to_f64(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);                 /* zero or subnormal */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25);     /* 1.m * 2^(e-15) */
    return sign ? -v : v;
}

/* Round a double to binary16, round-to-nearest-even (the default IEEE mode).
 * rint() rounds half to even in the default rounding mode; every scaling
 * below is by a power of two and therefore exact. */
ORACLE_API uint16_t oracle_f64_to_f16_rne(double x) {
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (isnan(x)) return 0x7e00;
    if (a >= 65520.0) return sign | 0x7c00;        /* rounds to infinity */
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: units of 2^-24; 1024 units is the smallest normal,
         * whose encoding 0x0400 is also the integer 1024. */
        double units = rint(ldexp(a, 24));
        return sign | (uint16_t)units;
    }
    int e2;
    frexp(a, &e2);                                 /* a = f * 2^e2, f in [0.5,1) */
    int e = e2 - 1;                                /* a in [2^e, 2^(e+1)) */
    double mant = rint(ldexp(a, 10 - e));          /* in [1024, 2048] */
    if (mant == 2048.0) { mant = 1024.0; e += 1; }
    if (e > 15) return sign | 0x7c00;
    return sign | (uint16_t)(((e + 15) << 10) | ((int)mant - 1024));
}

/* ------------------------------------------------------------------------ */
/* MSA step 1+2: indexer score, causal mask, 128-token block max-pool.       */
/* [MSA-PR] Implementation: bs = maxpool_128(idx_q * idx_k^T + causal mask),  */
/* one indexer head per GQA group; [MSA-LOG] "force F32 indexer score accum" */
/* (here: accumulated in fp64, which the f32 kernels approximate).           */
/* ------------------------------------------------------------------------ */

/* Score of one key row against one query row, in double. */
static double dot_f32_f64(const float* a, const float* b, int n) {
    double s = 0.0;
    for (int d = 0; d < n; ++d) s += (double)a[d] * (double)b[d];
    return s;
}

/* Block scores of one (query, group).
 *   idx_q_g : [idx_dim] the query's indexer vector of group g
 *   idx_k_s : the stream's index-key cache, [cap][n_group][idx_dim]
 *   bs      : [p / block + 1] out; bs[b] = max over keys j of block b with
 *             j <= p of the score (every visible block has >= 1 visible key)
 */
static void block_scores_one(const float* idx_q_g, const float* idx_k_s,
                             int n_group, int idx_dim, int g, int64_t p,
                             int block, double* bs) {
    int64_t nvis = p / block + 1;
    for (int64_t b = 0; b < nvis; ++b) {
        double best = -INFINITY;
        for (int64_t j = b * block; j < (b + 1) * block && j <= p; ++j) {
            const float* krow = idx_k_s + (j * n_group + g) * (int64_t)idx_dim;
            double s = dot_f32_f64(idx_q_g, krow, idx_dim);
            if (s > best) best = s;
        }
        bs[b] = best;
    }
}

/* ------------------------------------------------------------------------ */
/* MSA step 3: top-k block selection with the local block forced in.        */
/* [MSA-PR] Overview (top-16 blocks, the query's local block always         */
/* included) and Implementation (local-force bias ranked together with bs); */
/* review thread: k = min(indexer_top_k, nblk).                             */
/* ------------------------------------------------------------------------ */

typedef struct {
    double score;
    int64_t id;
    int local;
} ranked_t;

/* Rank order: local block first, then higher score, then lower id. */
static int rank_cmp(const void* pa, const void* pb) {
    const ranked_t* a = (const ranked_t*)pa;
    const ranked_t* b = (const ranked_t*)pb;
    if (a->local != b->local) return a->local ? -1 : 1;
    if (a->score > b->score) return -1;
    if (a->score < b->score) return 1;
    return (a->id < b->id) ? -1 : (a->id > b->id);
}

static int id_cmp(const void* pa, const void* pb) {
    int32_t a = *(const int32_t*)pa, b = *(const int32_t*)pb;
    return (a > b) - (a < b);
}

/* Select from n candidates with the given scores (candidate i has id i);
 * `local` is the forced id or -1 for none.  Writes the first
 * min(top_k, n) ids of the rank order, ascending, padded with -1 to top_k. */
static int select_ranked(const double* score, int64_t n, int64_t local,
                         int top_k, int32_t* sel) {
    ranked_t* r = (ranked_t*)malloc((size_t)n * sizeof *r);
    for (int64_t i = 0; i < n; ++i) {
        r[i].score = score[i];
        r[i].id = i;
        r[i].local = (i == local);
    }
    qsort(r, (size_t)n, sizeof *r, rank_cmp);
    int k = (int)(n < top_k ? n : top_k);
    for (int i = 0; i < k; ++i) sel[i] = (int32_t)r[i].id;
    qsort(sel, (size_t)k, sizeof *sel, id_cmp);
    for (int i = k; i < top_k; ++i) sel[i] = -1;
    free(r);
    return k;
}

/* Exposed for the brute-force pins: selection over a given score vector. */
ORACLE_API int oracle_select_ranked(const double* score, int64_t n,
                                    int64_t local, int top_k, int32_t* sel) {
    return select_ranked(score, n, local, top_k, sel);
}

/*
 * MSA selection for n_q queries.
 *   idx_k  : [n_stream][cap][n_group][idx_dim] f32 index-key cache
 *   stream, pos : [n_q] each query's stream and position (slot)
 *   idx_q  : [n_q][n_group][idx_dim] f32
 *   bs_out : optional [n_q][n_group][nblk_out] fp64 block scores (unbiased;
 *            -inf for blocks past the query's local block)
 *   sel    : [n_q][n_group][top_k] ascending ids, -1 padded
 *   n_sel  : [n_q][n_group] = min(top_k, pos / block + 1)
 * Returns 0, or -1 on a position outside the cache.
 */
ORACLE_API int oracle_msa_select(int n_group, int idx_dim, int block, int top_k,
                                 int64_t cap, const float* idx_k,
                                 int64_t n_q, const int32_t* stream,
                                 const int32_t* pos, const float* idx_q,
                                 double* bs_out, int64_t nblk_out,
                                 int32_t* sel, int32_t* n_sel) {
    for (int64_t i = 0; i < n_q; ++i)
        if (pos[i] < 0 || pos[i] >= cap) return -1;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t w = 0; w < n_q * n_group; ++w) {
        int64_t i = w / n_group;
        int g = (int)(w % n_group);
        int64_t p = pos[i];
        int64_t nvis = p / block + 1;
        const float* idx_k_s = idx_k + (int64_t)stream[i] * cap * n_group * idx_dim;
        double* bs = (double*)malloc((size_t)nvis * sizeof *bs);
        block_scores_one(idx_q + (i * n_group + g) * (int64_t)idx_dim, idx_k_s,
                         n_group, idx_dim, g, p, block, bs);
        if (bs_out) {
            double* o = bs_out + (i * n_group + g) * nblk_out;
            for (int64_t b = 0; b < nblk_out; ++b) o[b] = b < nvis ? bs[b] : -INFINITY;
            if (nvis > nblk_out) {
#pragma omp atomic write
                bad = 1;
            }
        }
        int k = select_ranked(bs, nvis, p / block, top_k,
                              sel + (i * n_group + g) * (int64_t)top_k);
        n_sel[i * n_group + g] = k;
        free(bs);
    }
    return bad ? -2 : 0;
}

/* ------------------------------------------------------------------------ */
/* MSA step 4 (and DSA attention): softmax attention over the selected keys */
/* only.  [MSA-PR] Overview ("the main attention then runs only over the    */
/* selected blocks"), Implementation (decode gathers the selected blocks    */
/* and runs attention over them; prefill masks the unselected blocks).      */
/* ------------------------------------------------------------------------ */

/* out[d] = sum_j softmax_j(scale * q.k_j) v_j[d] over the token list. */
static void attend_head(const uint16_t* q, const uint16_t* k_base,
                        const uint16_t* v_base, int64_t row_stride,
                        const int64_t* tok, int64_t n_tok, int head_dim,
                        double scale, double* z, double* out) {
    double m = -INFINITY;
    for (int64_t i = 0; i < n_tok; ++i) {
        const uint16_t* krow = k_base + tok[i] * row_stride;
        double s = 0.0;
        for (int d = 0; d < head_dim; ++d)
            s += oracle_bf16_to_f64(q[d]) * oracle_bf16_to_f64(krow[d]);
        z[i] = scale * s;
        if (z[i] > m) m = z[i];
    }
    double l = 0.0;
    for (int d = 0; d < head_dim; ++d) out[d] = 0.0;
    for (int64_t i = 0; i < n_tok; ++i) {
        double w = exp(z[i] - m);
        l += w;
        const uint16_t* vrow = v_base + tok[i] * row_stride;
        for (int d = 0; d < head_dim; ++d) out[d] += w * oracle_bf16_to_f64(vrow[d]);
    }
    for (int d = 0; d < head_dim; ++d) out[d] /= l;
}

/*
 * Sparse attention for n_q queries over selected units of `unit` tokens
 * (unit = block for MSA ids, 1 for DSA token ids).
 *   k_cache, v_cache : [n_stream][cap][n_group][head_dim] bf16
 *   q     : [n_q][n_group * heads_per_group][head_dim] bf16
 *   sel   : id of entry t of (query i, group g) is
 *           sel[i * sel_q_stride + g * sel_g_stride + t], t < sel_len;
 *           negative ids are padding (sel_g_stride = 0 shares one list
 *           across the groups, as DSA does)
 *   out   : [n_q][n_group * heads_per_group][head_dim] fp64
 * Token j of a selected unit u is attended iff j <= pos[i].
 * Returns 0, -1 on a bad position or id, -3 on an empty key set.
 */
ORACLE_API int oracle_sparse_attend(int n_group, int heads_per_group, int head_dim,
                                    double scale, int64_t cap,
                                    const uint16_t* k_cache, const uint16_t* v_cache,
                                    int64_t n_q, const int32_t* stream,
                                    const int32_t* pos, const uint16_t* q,
                                    const int32_t* sel, int64_t sel_q_stride,
                                    int64_t sel_g_stride, int sel_len, int unit,
                                    double* out) {
    for (int64_t i = 0; i < n_q; ++i)
        if (pos[i] < 0 || pos[i] >= cap) return -1;
    int err = 0;
    int n_head = n_group * heads_per_group;
    int64_t row_stride = (int64_t)n_group * head_dim;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t w = 0; w < n_q * n_group; ++w) {
        int64_t i = w / n_group;
        int g = (int)(w % n_group);
        int64_t p = pos[i];
        const int32_t* ids = sel + i * sel_q_stride + g * sel_g_stride;
        int64_t* tok = (int64_t*)malloc((size_t)sel_len * unit * sizeof *tok);
        double* z = (double*)malloc((size_t)sel_len * unit * sizeof *z);
        int64_t n_tok = 0;
        for (int t = 0; t < sel_len; ++t) {
            if (ids[t] < 0) continue;
            for (int64_t j = (int64_t)ids[t] * unit; j < ((int64_t)ids[t] + 1) * unit; ++j)
                if (j <= p) tok[n_tok++] = j;
        }
        int64_t base = ((int64_t)stream[i] * cap * n_group + g) * head_dim;
        if (n_tok == 0) {
#pragma omp atomic write
            err = -3;
        } else {
            for (int hh = 0; hh < heads_per_group; ++hh) {
                int h = g * heads_per_group + hh;
                attend_head(q + (i * n_head + h) * (int64_t)head_dim, k_cache + base,
                            v_cache + base, row_stride, tok, n_tok, head_dim, scale, z,
                            out + (i * n_head + h) * (int64_t)head_dim);
            }
        }
        free(tok);
        free(z);
    }
    return err;
}

/* ------------------------------------------------------------------------ */
/* DSA lightning indexer ([DSA-PR] "What this does"): keys are Hadamard-     */
/* rotated and stored as F16 in a persistent per-layer cache; each query     */
/* keeps its top-k highest-scoring keys.                                     */
/* ------------------------------------------------------------------------ */

/* Entry (i, j) of the Sylvester Hadamard matrix: (-1)^popcount(i & j). */
static int hadamard_sign(int i, int j) {
    return (__builtin_popcount((unsigned)(i & j)) & 1) ? -1 : 1;
}

/* k_rot[r] = fp16_rne( H_n k[r] / sqrt(n) ) for n_rows rows of n (a power of
 * two) fp16 values, written as the explicit matrix product. */
ORACLE_API int oracle_dsa_rotate(int64_t n_rows, int n, const uint16_t* k_raw,
                                 uint16_t* k_rot) {
    if (n <= 0 || (n & (n - 1))) return -1;
    double inv = 1.0 / sqrt((double)n);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n_rows; ++r) {
        const uint16_t* x = k_raw + r * n;
        for (int i = 0; i < n; ++i) {
            double s = 0.0;
            for (int j = 0; j < n; ++j) s += hadamard_sign(i, j) * oracle_f16_to_f64(x[j]);
            k_rot[r * n + i] = oracle_f64_to_f16_rne(s * inv);
        }
    }
    return 0;
}

/*
 * DSA token selection for n_q queries.
 *   k_rot : [n_stream][cap][idx_dim] fp16 rotated indexer keys
 *   q_idx : [n_q][idx_dim] fp16 (not rotated)
 *   score_out : optional [n_q][cap] fp64 scores (-inf past pos)
 *   sel   : [n_q][top_k] ascending token ids of the min(top_k, pos + 1)
 *           highest scores (ties: lower id first), -1 padded
 */
ORACLE_API int oracle_dsa_select(int idx_dim, int top_k, int64_t cap,
                                 const uint16_t* k_rot, int64_t n_q,
                                 const int32_t* stream, const int32_t* pos,
                                 const uint16_t* q_idx, double* score_out,
                                 int32_t* sel, int32_t* n_sel) {
    for (int64_t i = 0; i < n_q; ++i)
        if (pos[i] < 0 || pos[i] >= cap) return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < n_q; ++i) {
        int64_t p = pos[i];
        const uint16_t* ks = k_rot + (int64_t)stream[i] * cap * idx_dim;
        const uint16_t* qv = q_idx + i * idx_dim;
        double* t = (double*)malloc((size_t)(p + 1) * sizeof *t);
        for (int64_t j = 0; j <= p; ++j) {
            double s = 0.0;
            for (int d = 0; d < idx_dim; ++d)
                s += oracle_f16_to_f64(qv[d]) * oracle_f16_to_f64(ks[j * idx_dim + d]);
            t[j] = s;
        }
        if (score_out)
            for (int64_t j = 0; j < cap; ++j) score_out[i * cap + j] = j <= p ? t[j] : -INFINITY;
        n_sel[i] = select_ranked(t, p + 1, -1, top_k, sel + i * (int64_t)top_k);
        free(t);
    }
    return 0;
}

/*
 * DSA token selection with a multi-head indexer ([DSA-PR] review thread: the
 * indexer forms one K*Q score per indexer head, n_ihead = 32 for GLM, takes
 * an element-wise product with a second matrix and reduces over the heads
 * to one score per (query, key) before the top-k).  The pages do not print
 * the reduction; it is read as the published lightning-indexer form the
 * pull request is named after:
 *     score(i, j) = sum_h w[i][h] * max(0, q[i][h] . k[j])
 * with per-query head weights w (any scale folded in by the caller).
 *   k_rot  : [n_stream][cap][idx_dim] fp16 rotated indexer keys
 *   q_idx  : [n_q][n_head][idx_dim] fp16 (not rotated)
 *   head_w : [n_q][n_head] f32
 *   score_out, sel, n_sel : as oracle_dsa_select
 */
ORACLE_API int oracle_dsa_select_heads(int idx_dim, int n_head, int top_k, int64_t cap,
                                       const uint16_t* k_rot, int64_t n_q,
                                       const int32_t* stream, const int32_t* pos,
                                       const uint16_t* q_idx, const float* head_w,
                                       double* score_out, int32_t* sel, int32_t* n_sel) {
    if (n_head < 1) return -1;
    for (int64_t i = 0; i < n_q; ++i)
        if (pos[i] < 0 || pos[i] >= cap) return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < n_q; ++i) {
        int64_t p = pos[i];
        const uint16_t* ks = k_rot + (int64_t)stream[i] * cap * idx_dim;
        double* t = (double*)malloc((size_t)(p + 1) * sizeof *t);
        for (int64_t j = 0; j <= p; ++j) {
            double total = 0.0;
            for (int h = 0; h < n_head; ++h) {
                const uint16_t* qv = q_idx + (i * n_head + h) * idx_dim;
                double s = 0.0;
                for (int d = 0; d < idx_dim; ++d)
                    s += oracle_f16_to_f64(qv[d]) * oracle_f16_to_f64(ks[j * idx_dim + d]);
                double relu = s > 0.0 ? s : 0.0;
                total += (double)head_w[i * n_head + h] * relu;
            }
            t[j] = total;
        }
        if (score_out)
            for (int64_t j = 0; j < cap; ++j) score_out[i * cap + j] = j <= p ? t[j] : -INFINITY;
        n_sel[i] = select_ranked(t, p + 1, -1, top_k, sel + i * (int64_t)top_k);
        free(t);
    }
    return 0;
}

/*
 * Indexer projection of n_tok tokens ([MSA-PR] Overview and Quantization:
 * per-group index query and key projections of the hidden state, kept in
 * F32; review thread, RADV validation comment: the layer uses a gemma-style
 * norm and RoPE on half of each head, "0.5 partial rotary").  The order of
 * the steps and the rotation convention are not printed; they are read as
 *   y  = W[g] x                          (head_dim rows of W per group)
 *   z  = y / sqrt(mean(y^2) + eps) * (1 + gamma[g])   (gemma-style RMS norm)
 *   RoPE on dims 0 .. rot_dim - 1, pairs (i, i + rot_dim / 2), angle
 *   pos * theta^(-2 i / rot_dim); dims >= rot_dim pass through.
 *   x   : [n_tok][d_model] f32        w_q, w_k : [n_group * head_dim][d_model] f32
 *   g_q, g_k : [n_group][head_dim] f32  pos : [n_tok]
 *   q_out, k_out : [n_tok][n_group][head_dim] fp64 (either may be NULL)
 */
static void project_head(const float* x, const float* w, const float* gamma, int d_model, int head_dim,
                         double eps, double theta, int rot_dim, int32_t pos, double* out) {
    double* y = (double*)malloc((size_t)head_dim * sizeof *y);
    double ss = 0.0;
    for (int i = 0; i < head_dim; ++i) {
        double s = 0.0;
        for (int d = 0; d < d_model; ++d) s += (double)w[(int64_t)i * d_model + d] * (double)x[d];
        y[i] = s;
        ss += s * s;
    }
    double inv_rms = 1.0 / sqrt(ss / head_dim + eps);
    for (int i = 0; i < head_dim; ++i) out[i] = y[i] * inv_rms * (1.0 + (double)gamma[i]);
    int half = rot_dim / 2;
    for (int i = 0; i < half; ++i) {
        double ang = (double)pos * pow(theta, -2.0 * i / rot_dim);
        double c = cos(ang), s = sin(ang);
        double a = out[i], b = out[i + half];
        out[i] = a * c - b * s;
        out[i + half] = a * s + b * c;
    }
    free(y);
}

ORACLE_API int oracle_index_project(int64_t n_tok, int d_model, int n_group, int head_dim,
                                    const float* x, const float* w_q, const float* w_k,
                                    const float* g_q, const float* g_k, double eps, double theta,
                                    int rot_dim, const int32_t* pos, double* q_out, double* k_out) {
    if (rot_dim < 0 || rot_dim > head_dim || rot_dim % 2) return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = 0; t < n_tok; ++t) {
        for (int g = 0; g < n_group; ++g) {
            const int64_t o = (t * n_group + g) * head_dim;
            const int64_t wo = (int64_t)g * head_dim * d_model;
            if (q_out)
                project_head(x + t * d_model, w_q + wo, g_q + g * head_dim, d_model, head_dim, eps, theta,
                             rot_dim, pos[t], q_out + o);
            if (k_out)
                project_head(x + t * d_model, w_k + wo, g_k + g * head_dim, d_model, head_dim, eps, theta,
                             rot_dim, pos[t], k_out + o);
        }
    }
    return 0;
}

/*
 * Quantized K/V caches ([QSA] Strata compare page, qsa_prompt_attn.hpp header
 * comment: int8 KV, and Q4_0 KV whose codes enter exactly as int8 with one
 * FP32 scale per 32 values, as int8 KV's do).  The quantizer is not printed;
 * it is read as symmetric absmax per 32 consecutive values of a row:
 *   fmt 1 (int8): s = max|x| / 127, c = rint(x / s) in -127 .. 127
 *   fmt 2 (q4_0): s = max|x| / 7,   c = rint(x / s) in -7 .. 7 (-8 unused),
 *                 stored as c + 8 in a nibble; byte j of a 32-value block
 *                 holds values j (low nibble) and j + 16 (high nibble)
 * (s = 0 gives c = 0); value = c * s.  These steps decide integers, so they
 * are taken in IEEE single precision (f32 division and rint, ties to even),
 * as the kernel takes them.
 *   x : [n_rows][row_len] bf16, row_len a multiple of 32
 *   codes : [n_rows][row_len] int8 (fmt 1) or [n_rows][row_len / 2] (fmt 2)
 *   scales : [n_rows][row_len / 32] f32
 */
ORACLE_API int oracle_kv_quantize(int64_t n_rows, int row_len, int fmt, const uint16_t* x,
                                  uint8_t* codes, float* scales) {
    if (row_len % 32 || (fmt != 1 && fmt != 2)) return -1;
    const int nb = row_len / 32;
    for (int64_t r = 0; r < n_rows; ++r) {
        for (int b = 0; b < nb; ++b) {
            float v[32];
            float amax = 0.0f;
            for (int j = 0; j < 32; ++j) {
                v[j] = (float)oracle_bf16_to_f64(x[r * row_len + 32 * b + j]);   /* exact */
                float a = fabsf(v[j]);
                if (a > amax) amax = a;
            }
            volatile float s = amax / (fmt == 1 ? 127.0f : 7.0f);
            scales[r * nb + b] = s;
            int c[32];
            for (int j = 0; j < 32; ++j) {
                volatile float t = s > 0.0f ? v[j] / s : 0.0f;
                c[j] = (int)rintf(t);
            }
            if (fmt == 1) {
                for (int j = 0; j < 32; ++j) codes[r * row_len + 32 * b + j] = (uint8_t)(int8_t)c[j];
            } else {
                uint8_t* q = codes + r * (row_len / 2) + 16 * b;
                for (int j = 0; j < 16; ++j)
                    q[j] = (uint8_t)((c[j] + 8) | ((c[j + 16] + 8) << 4));
            }
        }
    }
    return 0;
}

ORACLE_API int oracle_kv_dequantize(int64_t n_rows, int row_len, int fmt, const uint8_t* codes,
                                    const float* scales, double* out) {
    if (row_len % 32 || (fmt != 1 && fmt != 2)) return -1;
    const int nb = row_len / 32;
    for (int64_t r = 0; r < n_rows; ++r)
        for (int b = 0; b < nb; ++b)
            for (int j = 0; j < 32; ++j) {
                int c;
                if (fmt == 1) {
                    c = (int8_t)codes[r * row_len + 32 * b + j];
                } else {
                    uint8_t byte = codes[r * (row_len / 2) + 16 * b + (j & 15)];
                    c = (j < 16 ? (byte & 15) : (byte >> 4)) - 8;
                }
                out[r * row_len + 32 * b + j] = (double)c * (double)scales[r * nb + b];
            }
    return 0;
}

/* attend_head over fp64 K/V rows (dequantized caches). */
static void attend_head_f64(const uint16_t* q, const double* k_base, const double* v_base,
                            int64_t row_stride, const int64_t* tok, int64_t n_tok, int head_dim,
                            double scale, double* z, double* out) {
    double m = -INFINITY;
    for (int64_t i = 0; i < n_tok; ++i) {
        const double* krow = k_base + tok[i] * row_stride;
        double s = 0.0;
        for (int d = 0; d < head_dim; ++d) s += oracle_bf16_to_f64(q[d]) * krow[d];
        z[i] = scale * s;
        if (z[i] > m) m = z[i];
    }
    double l = 0.0;
    for (int d = 0; d < head_dim; ++d) out[d] = 0.0;
    for (int64_t i = 0; i < n_tok; ++i) {
        double w = exp(z[i] - m);
        l += w;
        const double* vrow = v_base + tok[i] * row_stride;
        for (int d = 0; d < head_dim; ++d) out[d] += w * vrow[d];
    }
    for (int d = 0; d < head_dim; ++d) out[d] /= l;
}

/* oracle_sparse_attend with fp64 K/V caches [n_stream][cap][n_group][head_dim]. */
ORACLE_API int oracle_sparse_attend_f64(int n_group, int heads_per_group, int head_dim, double scale,
                                        int64_t cap, const double* k_cache, const double* v_cache,
                                        int64_t n_q, const int32_t* stream, const int32_t* pos,
                                        const uint16_t* q, const int32_t* sel, int64_t sel_q_stride,
                                        int64_t sel_g_stride, int sel_len, int unit, double* out) {
    for (int64_t i = 0; i < n_q; ++i)
        if (pos[i] < 0 || pos[i] >= cap) return -1;
    int err = 0;
    int n_head = n_group * heads_per_group;
    int64_t row_stride = (int64_t)n_group * head_dim;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t w = 0; w < n_q * n_group; ++w) {
        int64_t i = w / n_group;
        int g = (int)(w % n_group);
        int64_t p = pos[i];
        const int32_t* ids = sel + i * sel_q_stride + g * sel_g_stride;
        int64_t* tok = (int64_t*)malloc((size_t)sel_len * unit * sizeof *tok);
        double* z = (double*)malloc((size_t)sel_len * unit * sizeof *z);
        int64_t n_tok = 0;
        for (int t = 0; t < sel_len; ++t) {
            if (ids[t] < 0) continue;
            for (int64_t j = (int64_t)ids[t] * unit; j < ((int64_t)ids[t] + 1) * unit; ++j)
                if (j <= p) tok[n_tok++] = j;
        }
        int64_t base = ((int64_t)stream[i] * cap * n_group + g) * head_dim;
        if (n_tok == 0) {
#pragma omp atomic write
            err = -3;
        } else {
            for (int hh = 0; hh < heads_per_group; ++hh) {
                int h = g * heads_per_group + hh;
                attend_head_f64(q + (i * n_head + h) * (int64_t)head_dim, k_cache + base, v_cache + base,
                                row_stride, tok, n_tok, head_dim, scale, z,
                                out + (i * n_head + h) * (int64_t)head_dim);
            }
        }
        free(tok);
        free(z);
    }
    return err;
}
