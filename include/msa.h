/*
 * msa.h -- C ABI of the MI355X (gfx950) MiniMax Sparse Attention hot path.
 *
 * What is computed (web pages cited by title and section):
 *  - "Add MiniMax-M3 (MSA: MiniMax Sparse Attention) support", llama.cpp pull
 *    request 24908 [MSA-PR]:
 *      Overview: a per-GQA-group indexer scores the visible causal context,
 *      the scores are max-pooled into 128-token key blocks, the top-16 blocks
 *      are selected with the query's own (local) block always included, and
 *      attention runs over the selected 16 x 128 = 2048 keys only.
 *      Implementation: block scores bs = maxpool_128(idx_q . idx_k^T + causal
 *      mask) plus a large positive bias on the local block, ranked together
 *      for top-k; one indexer head per group, shared by the group's 16 query
 *      heads; prefill and decode share these semantics; the index keys live in
 *      their own per-layer F32 cache beside the K/V cache; per-stream caches
 *      are slot-anchored (slot == position).
 *  - llama.cpp compare page b10146, MSA commit log [MSA-LOG]: F32 index cache
 *    by default, F32 indexer score accumulation, unified selection for
 *    prefill and decode, K/V in F16/BF16.
 *  - "deepseek2 : GLM-DSA sparse attention (lightning indexer), --dsa off by
 *    default", ik_llama.cpp pull request 2045 [DSA-PR], "What this does":
 *    indexer keys are Hadamard-rotated and cached as F16; each query keeps
 *    its top-k highest-scoring keys and the rest are masked out.
 *
 * Readings where the pages leave a step open: a key at slot j is visible to a
 * query at position p iff j <= p; a block's score is the max over its visible
 * keys; the local-block bias is "rank first"; ties rank the lower block (or
 * token) id first; query head h uses group h / heads_per_group; the softmax
 * scale is dims->scale with no sink and no soft-cap; DSA rotates keys with
 * the orthonormal Sylvester Hadamard transform and rounds once to fp16.
 *
 * Conventions common to every entry point:
 *  - All pointers named d_* are DEVICE pointers on the current HIP device;
 *    the caller owns every byte of device memory (caches, inputs, outputs,
 *    workspace).  The library keeps no state between calls, allocates
 *    nothing, never synchronises, and enqueues work only on `hip_stream`
 *    (a hipStream_t; NULL means the legacy default stream).  Outputs are
 *    valid once the stream has completed.
 *  - bf16 and fp16 values are passed as uint16_t bit patterns.
 *  - Cache layout (token-major: one row per (token, KV head)):
 *      idx_k [n_stream][cap][n_group][idx_dim] f32   (MSA index keys)
 *      dsa_k [n_stream][cap][idx_dim]          fp16  (DSA rotated keys)
 *      k, v  [n_stream][cap][n_group][head_dim] bf16
 *  - Every call validates its host-visible arguments BEFORE launching
 *    anything; on any error nothing is launched and a negative msa_status is
 *    returned.  Device-side preconditions (documented per call, not
 *    checked): every stream id is < cache->n_stream, every position is in
 *    [0, max_pos], and the keys 0..pos of a query's stream have been
 *    appended.  No exception crosses this ABI.
 *  - Device pointers must be 16-byte aligned (128-bit vector access).
 *  - n_q == 0 (or n_new == 0) is a valid empty call: MSA_OK, nothing runs.
 *  - Call sizes: at most MSA_MAX_QUERIES queries per select, block-score,
 *    top-k, attention or decode-step call, and MSA_MAX_ROWS rows (tokens)
 *    per append or projection call, so that every launch grid stays within
 *    the 2^32 work-items of one dispatch dimension; dsa_select and
 *    dsa_select_heads take at most 65535 queries (the query is the second
 *    grid dimension of their scans).  A larger call returns
 *    MSA_ERR_UNSUPPORTED (split it into several calls).
 *  - Supported geometry: n_group 4, heads_per_group 16, head_dim 128,
 *    idx_dim 128; MSA: block 128, 1 <= top_k <= 64; DSA: block 1,
 *    1 <= top_k <= 4096.  Anything else returns MSA_ERR_UNSUPPORTED.
 *  - Results are deterministic: no floating-point atomics; split partial
 *    results are combined in a fixed order.
 */
#ifndef MSA_H
#define MSA_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define MSA_API __attribute__((visibility("default")))
#else
#define MSA_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* Largest queries per select / attention / step call, rows per append or
 * projection call (see the call-size note above). */
#define MSA_MAX_QUERIES ((int64_t)1 << 18)
#define MSA_MAX_ROWS ((int64_t)1 << 24)

typedef enum msa_status {
    MSA_OK = 0,
    MSA_ERR_NULL_ARG = -1,            /* a required pointer is NULL */
    MSA_ERR_BAD_SHAPE = -2,           /* negative count, cap < 1, n_stream < 1, bad stride */
    MSA_ERR_OUT_OF_RANGE = -3,        /* max_pos / pos0 / stream outside the cache */
    MSA_ERR_MISALIGNED = -4,          /* a device pointer is not 16-byte aligned */
    MSA_ERR_WORKSPACE_TOO_SMALL = -5, /* ws_bytes < msa_workspace_bytes(...) */
    MSA_ERR_UNSUPPORTED = -6,         /* geometry outside the supported set */
    MSA_ERR_HIP = -7                  /* a kernel launch failed */
} msa_status;

/* Head geometry of one sparse attention layer. */
typedef struct msa_dims {
    int32_t n_group;          /* GQA groups = KV heads = indexer heads (4) */
    int32_t heads_per_group;  /* query heads per group (16) */
    int32_t head_dim;         /* Q/K/V head dim (128) */
    int32_t idx_dim;          /* indexer dim (128) */
    int32_t block;            /* key block for MSA (128); 1 for DSA token ids */
    int32_t top_k;            /* blocks (MSA, 16) or tokens (DSA, 2048) kept */
    float scale;              /* softmax scale (1/sqrt(head_dim)) */
} msa_dims;

/* Per-layer caches (device memory owned by the caller). */
typedef struct msa_cache {
    float* idx_k;       /* MSA index keys (f32), or NULL when unused */
    uint16_t* dsa_k;    /* DSA rotated indexer keys (fp16), or NULL */
    uint16_t* k;        /* bf16 keys */
    uint16_t* v;        /* bf16 values (not transposed) */
    int64_t cap;        /* slots per stream */
    int32_t n_stream;   /* independent streams (sequences) */
    /* MSA index keys stored as fp16 [n_stream][cap][n_group][idx_dim], or
     * NULL.  [MSA-PR] review thread, indexer precision: the index cache
     * type is a setting (F32 by default) and F16 indexer tensors were
     * tested beside F32.  msa_index_append rounds the f32 keys it receives
     * to fp16 (nearest, ties to even); scores still accumulate in f32.  The
     * index operations use whichever of idx_k / idx_k_f16 is set; setting
     * both is MSA_ERR_UNSUPPORTED.  Halves the bytes the decode scan reads. */
    uint16_t* idx_k_f16;
    /* Paged caches ([MSA-PR] review thread on per-stream caches: slot-anchored
     * per-stream caches versus a unified cache addressed through a block
     * index).  NULL: stream s owns rows s*cap .. s*cap+cap-1 of every cache
     * (slot == position).  Otherwise a DEVICE array [n_stream][table_stride]
     * of int32: logical block b (positions 128b .. 128b+127) of stream s lives
     * in page d_block_table[s*table_stride + b], i.e. cache rows
     * page*128 .. page*128+127 of idx_k / idx_k_f16 / dsa_k / k / v, which are
     * then pools of pages.  cap stays the logical capacity per stream and
     * needs table_stride*128 >= cap (MSA_ERR_BAD_SHAPE otherwise, and for
     * table_stride < 1); the table must be 4-byte aligned (MSA_ERR_MISALIGNED).
     * Device precondition (not checked): every
     * entry a call reaches (blocks 0 .. max_pos/128 of the streams it touches)
     * is a page inside all the pools the call reads or writes. */
    const int32_t* d_block_table;
    int32_t table_stride;
    /* Quantized K/V caches ([QSA] Strata compare page, qsa_prompt_attn.hpp
     * header: int8 KV, and Q4_0 KV whose codes enter as int8, with one FP32
     * scale per 32 values).  kv_format 0: k, v are bf16 as above.  1: k, v
     * hold int8 codes [rows][n_group][head_dim] (1 byte each).  2: 4-bit
     * codes [rows][n_group][head_dim / 2]; byte j of each 32-value block
     * holds values j (low nibble) and j + 16 (high nibble), stored as code + 8.
     * k_scale, v_scale: [rows][n_group][head_dim / 32] f32; value = code *
     * scale.  The append quantizes bf16 rows: s = max|x| / 127 (int8) or / 7
     * (4-bit), code = rint(x / s) in f32 (a reading: the pages give the
     * format, not the rule).  Supported by the appends and decode attention
     * (msa_attend_decode, dsa_attend_decode, msa_attend_prefill).  Other
     * values -> MSA_ERR_UNSUPPORTED. */
    int32_t kv_format;
    float* k_scale;
    float* v_scale;
} msa_cache;

/* Operations whose workspace size can be queried. */
typedef enum msa_op {
    MSA_OP_SELECT = 1,          /* msa_select */
    MSA_OP_SELECT_PREFILL = 2,  /* msa_select_prefill */
    MSA_OP_ATTEND_DECODE = 3,   /* msa_attend_decode */
    MSA_OP_ATTEND_PREFILL = 4,  /* msa_attend_prefill */
    DSA_OP_SELECT = 5,          /* dsa_select */
    DSA_OP_ATTEND_DECODE = 6,   /* dsa_attend_decode */
    MSA_OP_BLOCK_SCORES_PREFILL = 7,  /* msa_block_scores_prefill */
    MSA_OP_INDEX_PROJECT = 8,         /* msa_index_project (n_q = tokens) */
    MSA_OP_DECODE_STEP = 9            /* msa_decode_step */
} msa_op;

/* Bytes of workspace `op` needs for n_q queries whose positions are all
 * <= max_pos (msa_select_prefill / msa_attend_prefill: max_pos = pos0 +
 * n_q - 1).  Returns 0 when the op needs no workspace (always for n_q == 0,
 * an empty call) and (size_t)-1 for an unsupported geometry, op or size. */
MSA_API size_t msa_workspace_bytes(const msa_dims* dims, msa_op op, int64_t n_q, int32_t max_pos);

/* Human-readable name of a status code (static storage). */
MSA_API const char* msa_status_string(msa_status s);

/*
 * [MSA-PR] Implementation (per-layer F32 index-key cache beside K/V);
 * [DSA-PR] "What this does" (recent index keys must be written before the
 * same step's queries score).
 * Writes n_new token rows: row i goes to slot d_pos[i] of stream
 * d_stream[i] in cache->idx_k (from d_idx_k_new [n_new][n_group][idx_dim]
 * f32), cache->k and cache->v (from d_k_new / d_v_new [n_new][n_group]
 * [head_dim] bf16).  Any of the three sources may be NULL to skip that
 * cache; a non-NULL source needs its cache pointer.  Exact copies.
 * Device preconditions: d_pos[i] <= max_pos < cache->cap; the (stream, pos)
 * pairs are distinct.
 */
MSA_API msa_status msa_index_append(const msa_dims* dims, const msa_cache* cache,
                            const int32_t* d_stream, const int32_t* d_pos, int64_t n_new,
                            int32_t max_pos, const float* d_idx_k_new,
                            const uint16_t* d_k_new, const uint16_t* d_v_new,
                            void* hip_stream);

/* Indexer projection parameters (msa_index_project).  DEVICE pointers,
 * caller-owned, 16-byte aligned. */
typedef struct msa_proj {
    int32_t d_model;        /* hidden size, a positive multiple of 32 */
    const float* d_w_q;     /* [n_group * idx_dim][d_model] f32, row-major (out x in) */
    const float* d_w_k;     /* [n_group * idx_dim][d_model] f32 */
    const float* d_g_q;     /* [n_group][idx_dim] f32 norm gains (scale 1 + g) */
    const float* d_g_k;     /* [n_group][idx_dim] f32 */
    float eps;              /* RMS norm epsilon, >= 0 */
    float rope_theta;       /* RoPE base, > 0 */
    int32_t rot_dim;        /* rotated dims per head: even, 0 .. 64 */
} msa_proj;

/*
 * [MSA-PR] Overview and Quantization (per-group index query and key
 * projections of the hidden state, kept in F32); review thread, RADV
 * validation comment (gemma-style norm, RoPE over half of each head).  The
 * step order and the rotation pairs are a reading: per token t and group g
 *   y = w[g] x[t];  z = y / sqrt(mean(y^2) + eps) * (1 + gain[g]);
 *   RoPE on dims 0 .. rot_dim - 1, pairs (i, i + rot_dim / 2), angle
 *   d_pos[t] * rope_theta^(-2 i / rot_dim) (evaluated in f64).
 * Writes the queries to d_idx_q [n_tok][n_group][idx_dim] f32 and appends
 * the keys to the index cache at (d_stream[t], d_pos[t]) (f32, or fp16
 * rounded to nearest even, paged or not), i.e. it replaces the idx_k part of
 * msa_index_append.  d_x [n_tok][d_model] f32.  Products and sums in f32
 * (matrix cores), d_model split into at most 32 slices summed in a fixed
 * order.  Workspace: MSA_OP_INDEX_PROJECT with n_q = n_tok.
 * Errors: d_model not a positive multiple of 32, rot_dim odd or > 64, eps < 0
 * or rope_theta <= 0 -> MSA_ERR_UNSUPPORTED.  Device preconditions as
 * msa_index_append.
 */
MSA_API msa_status msa_index_project(const msa_dims* dims, const msa_cache* cache, const msa_proj* proj,
                             const float* d_x, const int32_t* d_stream, const int32_t* d_pos,
                             int64_t n_tok, int32_t max_pos, float* d_idx_q, void* d_ws,
                             size_t ws_bytes, void* hip_stream);

/*
 * [MSA-PR] Implementation: bs = maxpool_128(idx_q . idx_k^T + causal mask),
 * per group, F32 accumulation ([MSA-LOG]).
 * For each query i (stream d_stream[i], position d_pos[i]) and group g
 * writes d_bs[(i * n_group + g) * nblk_stride + b] for b = 0 ..
 * max_pos / block: the max over keys j in [block*b, block*b + block) with
 * j <= pos of sum_d idx_q[i][g][d] * idx_k[stream][j][g][d] (f32), and -inf
 * for blocks past pos / block.  No bias is added (the local block is forced
 * by the selection).  Requires nblk_stride >= max_pos / block + 1.  One
 * wavefront-reduced dot product per key, streamed with 128-bit loads.
 */
MSA_API msa_status msa_block_scores(const msa_dims* dims, const msa_cache* cache,
                            const float* d_idx_q, const int32_t* d_stream,
                            const int32_t* d_pos, int64_t n_q, int32_t max_pos,
                            float* d_bs, int64_t nblk_stride, void* hip_stream);

/*
 * [MSA-PR] Overview and Implementation (top-k over bs plus the local-force
 * bias; k = min(indexer_top_k, nblk) per the review thread).
 * From block scores laid out as msa_block_scores writes them, selects per
 * (query, group) k = min(top_k, pos / block + 1) blocks: the local block
 * pos / block first, then the highest scores, ties to the lower block id.
 * Writes d_sel[(i * n_group + g) * top_k + t] in ascending id order, padded
 * with -1, and d_n_sel[i * n_group + g] = k.  Only blocks <= pos / block are
 * candidates.  Requires max_pos / block + 1 <= 4096.
 */
MSA_API msa_status msa_topk_blocks(const msa_dims* dims, const float* d_bs, int64_t nblk_stride,
                           const int32_t* d_pos, int64_t n_q, int32_t max_pos,
                           int32_t* d_sel, int32_t* d_n_sel, void* hip_stream);

/*
 * msa_block_scores followed by msa_topk_blocks, with the block scores kept
 * in the workspace (size: msa_workspace_bytes(dims, MSA_OP_SELECT, n_q,
 * max_pos)).  Decode form: any mix of streams and positions.
 *   d_idx_q [n_q][n_group][idx_dim] f32; d_sel [n_q][n_group][top_k] i32;
 *   d_n_sel [n_q][n_group] i32.
 */
MSA_API msa_status msa_select(const msa_dims* dims, const msa_cache* cache, const float* d_idx_q,
                      const int32_t* d_stream, const int32_t* d_pos, int64_t n_q,
                      int32_t max_pos, int32_t* d_sel, int32_t* d_n_sel,
                      void* d_ws, size_t ws_bytes, void* hip_stream);

/* Size of the device array msa_select_static keeps its block scores in. */
#define MSA_STATIC_SCRATCH_BYTES ((size_t)4 << 20)

/*
 * For callers that cannot allocate or pass a workspace (code under HIP graph
 * capture, serving loops that forbid allocation): msa_select with its block
 * scores kept in a library-owned device array of MSA_STATIC_SCRATCH_BYTES
 * (4 MiB) instead of d_ws.  Same arguments otherwise, same results.  The
 * call allocates nothing.  Limit: n_q * n_group * (max_pos / block + 1) * 4
 * bytes must fit the array (e.g. 1024 queries at 32K context, 256 queries at
 * 128K), else MSA_ERR_WORKSPACE_TOO_SMALL and nothing is launched.  Each GPU
 * the library runs on holds its own array until the process ends; its
 * address is resolved on the first call on that device (make that first call
 * outside a stream capture).  Every call on one GPU shares that GPU's array:
 * calls that overlap on one GPU (concurrent streams, other threads) race and
 * must be ordered by the caller.  MSA_ERR_HIP if the array cannot be
 * resolved.
 */
MSA_API msa_status msa_select_static(const msa_dims* dims, const msa_cache* cache, const float* d_idx_q,
                                     const int32_t* d_stream, const int32_t* d_pos, int64_t n_q,
                                     int32_t max_pos, int32_t* d_sel, int32_t* d_n_sel, void* hip_stream);

/*
 * Prefill form of msa_block_scores ([MSA-PR] Implementation, batch path;
 * [MSA-LOG] unified selection semantics): n_q consecutive queries at
 * positions pos0 .. pos0 + n_q - 1 of stream `stream` (host values), scored
 * with matrix-core tiles.  Same output layout and values as
 * msa_block_scores (f32 sums, summation order differs).
 * Workspace: msa_workspace_bytes(dims, MSA_OP_BLOCK_SCORES_PREFILL, n_q,
 * pos0 + n_q - 1) bytes at d_ws (16-byte aligned;
 * MSA_ERR_WORKSPACE_TOO_SMALL otherwise): the index keys 0 .. pos0 + n_q - 1
 * of the stream split into bf16 high and low parts, written by the call.
 */
MSA_API msa_status msa_block_scores_prefill(const msa_dims* dims, const msa_cache* cache,
                                    const float* d_idx_q, int32_t stream, int32_t pos0,
                                    int64_t n_q, float* d_bs, int64_t nblk_stride,
                                    void* d_ws, size_t ws_bytes, void* hip_stream);

/* msa_block_scores_prefill followed by msa_topk_blocks (workspace:
 * MSA_OP_SELECT_PREFILL with max_pos = pos0 + n_q - 1). */
MSA_API msa_status msa_select_prefill(const msa_dims* dims, const msa_cache* cache,
                              const float* d_idx_q, int32_t stream, int32_t pos0, int64_t n_q,
                              int32_t* d_sel, int32_t* d_n_sel,
                              void* d_ws, size_t ws_bytes, void* hip_stream);

/*
 * [MSA-PR] Overview and Implementation, decode path: each of a group's
 * query heads attends over only the keys of the group's selected blocks.
 * For query i, head h (group g = h / heads_per_group):
 *   out[i][h][:] = sum_{j in J} softmax_j(scale * q[i][h] . k[stream][j][g])
 *                  * v[stream][j][g][:]
 * with J = { j : j / block in sel[i][g][0..top_k), j <= pos } (ids < 0 are
 * padding).  Keys are read from the cache by block id (no gather); the
 * selected blocks are split across workgroups and their partial softmax
 * states are merged in a fixed order.
 *   d_q [n_q][n_group*heads_per_group][head_dim] bf16;
 *   d_sel as msa_select writes it; d_out [n_q][n_group*heads_per_group]
 *   [head_dim] f32.  Workspace: MSA_OP_ATTEND_DECODE (sized for the same
 *   dims).
 * Token-granular ids ([DSA-PR] "What this does"): with dims->block == 1
 * (and 1 <= top_k <= 4096) d_sel [n_q][top_k] holds token ids shared by all
 * groups, as dsa_select writes them, and the call is dsa_attend_decode.
 * Device precondition: at least one selected key per (query, group) (the
 * local block always provides key pos's block start).
 */
MSA_API msa_status msa_attend_decode(const msa_dims* dims, const msa_cache* cache, const uint16_t* d_q,
                             const int32_t* d_stream, const int32_t* d_pos, int64_t n_q,
                             int32_t max_pos, const int32_t* d_sel, float* d_out,
                             void* d_ws, size_t ws_bytes, void* hip_stream);

/*
 * One decode step ([MSA-PR] Implementation, decode path: the new token's
 * index key is written before the same step's query scores the cache):
 * msa_index_append of d_idx_k_new / d_k_new / d_v_new at (d_stream[i],
 * d_pos[i]), then msa_select and msa_attend_decode of the queries at those
 * same slots, with the same outputs bit for bit (cache rows, d_sel [n_q]
 * [n_group][top_k], d_n_sel, d_out).  d_k_new and d_v_new may be NULL (that
 * cache is not written); d_idx_k_new is required.  With an f32 index
 * cache, bf16 K/V and at most 1024 blocks (max_pos < 131072) it runs three
 * kernels instead of five: the scan also writes the rows and scores the new
 * keys from d_idx_k_new, the attention ranks each (query, group)'s blocks
 * itself (and writes d_sel, d_n_sel), then the split combine; when the
 * fine scan runs (few queries over short contexts) the last attention split
 * of each (query, group) merges the partials itself, so two kernels run.
 * Other caches and longer contexts run the separate calls' kernels.
 * Device preconditions: those of the three calls ((stream, pos) pairs
 * distinct, d_pos[i] <= max_pos).  Workspace: MSA_OP_DECODE_STEP, the
 * block scores, the attention partials, then n_q * 4 arrival counters
 * (int32), each part 256-byte aligned; calls that overlap on one workspace
 * race.
 */
MSA_API msa_status msa_decode_step(const msa_dims* dims, const msa_cache* cache, const int32_t* d_stream,
                           const int32_t* d_pos, int64_t n_q, int32_t max_pos, const float* d_idx_k_new,
                           const uint16_t* d_k_new, const uint16_t* d_v_new, const float* d_idx_q,
                           const uint16_t* d_q, int32_t* d_sel, int32_t* d_n_sel, float* d_out, void* d_ws,
                           size_t ws_bytes, void* hip_stream);

/*
 * Prefill form of msa_attend_decode ([MSA-PR] Implementation, batch path:
 * block-level mask of the selection combined with the causal mask): n_q
 * consecutive queries at positions pos0 .. pos0 + n_q - 1 of `stream`.
 * Same arguments and output as msa_attend_decode.  Cache rows up to
 * pos0 + n_q - 1 must be written (the chunk's own keys included).
 * Workspace: msa_workspace_bytes(dims, MSA_OP_ATTEND_PREFILL, n_q, max_pos)
 * bytes at d_ws (16-byte aligned; MSA_ERR_WORKSPACE_TOO_SMALL otherwise),
 * the same for every cache format: per tile of 32 consecutive queries and
 * group, the ascending list of the blocks their selections hold, built on
 * the device before the sweep, and a bf16 copy of K and V of every block
 * some selection holds, rearranged into the order the matrix-core operands
 * take (64 KiB per block of 0 .. max_pos and group, so the amount grows with
 * max_pos as well as with n_q).  A quantized cache (kv_format 1, 2) is
 * dequantized into that copy: each code times its scale, formed in f32 and
 * rounded once to bf16 (decode attention keeps the codes exact instead).
 */
MSA_API msa_status msa_attend_prefill(const msa_dims* dims, const msa_cache* cache, const uint16_t* d_q,
                              int32_t stream, int32_t pos0, int64_t n_q, const int32_t* d_sel,
                              float* d_out, void* d_ws, size_t ws_bytes, void* hip_stream);

/*
 * [DSA-PR] "What this does": the indexer keys are Hadamard-rotated and kept
 * in a persistent per-layer F16 cache.
 * Row i: dsa_k[stream][pos] = fp16_rne(H x / sqrt(idx_dim)) where x is
 * d_key_new[i] ([n_new][idx_dim] fp16) and H the Sylvester Hadamard matrix
 * (H[a][b] = (-1)^popcount(a & b)); the transform is exact in fp64 and
 * rounded once (round to nearest, ties to even).  d_k_new / d_v_new (may be
 * NULL) are copied into cache->k / cache->v as in msa_index_append.
 */
MSA_API msa_status dsa_index_append(const msa_dims* dims, const msa_cache* cache,
                            const int32_t* d_stream, const int32_t* d_pos, int64_t n_new,
                            int32_t max_pos, const uint16_t* d_key_new,
                            const uint16_t* d_k_new, const uint16_t* d_v_new,
                            void* hip_stream);

/*
 * [DSA-PR] "What this does": one score per (query, key),
 * t[j] = sum_d q_idx[i][d] * dsa_k[stream][j][d] (fp16 products, f32 sums)
 * for j <= pos; keeps k = min(top_k, pos + 1) keys with the largest t, ties
 * to the lower token id, no local forcing.  Writes d_sel [n_q][top_k]
 * ascending token ids padded with -1 and d_n_sel [n_q] = k.
 *   d_q_idx [n_q][idx_dim] fp16.  Workspace: DSA_OP_SELECT, the f32 scores
 *   (one row of max_pos + 1 rounded up to 64 per query) and, for calls of at
 *   most 32 queries over 8193 .. 65536 keys, whose top-k runs over one
 *   workgroup per 8192-key chunk: the chunks' first-digit histograms, the
 *   kept ids above the boundary bin and the boundary bin's keys and ids.
 */
MSA_API msa_status dsa_select(const msa_dims* dims, const msa_cache* cache, const uint16_t* d_q_idx,
                      const int32_t* d_stream, const int32_t* d_pos, int64_t n_q,
                      int32_t max_pos, int32_t* d_sel, int32_t* d_n_sel,
                      void* d_ws, size_t ws_bytes, void* hip_stream);

/*
 * [DSA-PR] review thread (the indexer memory discussion): the GLM indexer has
 * n_ihead = 32 heads; each forms its own K*Q score, the scores take an
 * element-wise product with a second matrix and are reduced over the heads
 * to one score per (query, key) before the top-k.  The pages do not print the
 * reduction; it is read as the lightning indexer's
 *     t[j] = sum_h head_w[i][h] * max(0, sum_d q_idx_h[i][h][d] * dsa_k[stream][j][d])
 * (fp16 products, f32 sums) for j <= pos; the top-k is dsa_select's.
 *   d_q_idx_h [n_q][n_head][idx_dim] fp16, d_head_w [n_q][n_head] f32 (any
 *   scale folded in), n_head in {16, 32, 48, 64} (MSA_ERR_UNSUPPORTED
 *   otherwise).  Workspace: DSA_OP_SELECT.  A layer that shares another
 *   layer's indexer (IndexShare) passes that layer's d_sel to
 *   dsa_attend_decode instead of selecting again.
 */
MSA_API msa_status dsa_select_heads(const msa_dims* dims, const msa_cache* cache,
                            const uint16_t* d_q_idx_h, const float* d_head_w, int32_t n_head,
                            const int32_t* d_stream, const int32_t* d_pos, int64_t n_q,
                            int32_t max_pos, int32_t* d_sel, int32_t* d_n_sel,
                            void* d_ws, size_t ws_bytes, void* hip_stream);

/*
 * [DSA-PR] "What this does": attention over the kept keys only.  As
 * msa_attend_decode, but d_sel [n_q][top_k] holds token ids shared by all
 * groups (dims->block must be 1); msa_attend_decode with block 1 is this
 * call.  Workspace: DSA_OP_ATTEND_DECODE (or MSA_OP_ATTEND_DECODE with the
 * same dims: the same size).
 */
MSA_API msa_status dsa_attend_decode(const msa_dims* dims, const msa_cache* cache, const uint16_t* d_q,
                             const int32_t* d_stream, const int32_t* d_pos, int64_t n_q,
                             int32_t max_pos, const int32_t* d_sel, float* d_out,
                             void* d_ws, size_t ws_bytes, void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* MSA_H */
