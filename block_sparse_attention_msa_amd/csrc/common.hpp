// common.hpp -- device helpers shared by the gfx950 kernels of the MSA hot
// path: vector types, bf16/fp16 conversions, DPP row reductions, MFMA
// wrappers and the internal launcher declarations used by msa_api.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

// ---------------------------------------------------------------------------
// Fixed geometry of the supported layer (validated on the host).
// ---------------------------------------------------------------------------
constexpr int kGroups = 4;        // GQA groups = KV heads = indexer heads
constexpr int kHeadsPerGroup = 16;
constexpr int kHeadDim = 128;
constexpr int kIdxDim = 128;
constexpr int kBlock = 128;       // MSA key block
constexpr int kMaxTopkBlocks = 64;
constexpr int kMaxBlocks = 4096;  // candidates one top-k wave can rank (8 B of LDS each)
constexpr int kChunk = 32;        // keys per attention step (one MFMA K-depth)

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// ---------------------------------------------------------------------------
// DPP reductions inside one 16-lane row (lanes 16r .. 16r + 15).  After the
// four steps every lane of the row holds the row's result.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

__device__ __forceinline__ float row16_sum(float x) {
    x += dpp_f32<kDppQuadXor1>(x);
    x += dpp_f32<kDppQuadXor2>(x);
    x += dpp_f32<kDppRowHalfMirror>(x);
    x += dpp_f32<kDppRowMirror>(x);
    return x;
}

__device__ __forceinline__ float row16_max(float x) {
    x = fmaxf(x, dpp_f32<kDppQuadXor1>(x));
    x = fmaxf(x, dpp_f32<kDppQuadXor2>(x));
    x = fmaxf(x, dpp_f32<kDppRowHalfMirror>(x));
    x = fmaxf(x, dpp_f32<kDppRowMirror>(x));
    return x;
}

// All-lane reductions across rows with the gfx950 row-swap permutes:
// v_permlane16_swap pairs rows 0/1 and 2/3, v_permlane32_swap the two wave
// halves, so op(result[0], result[1]) combines lane l with lane l ^ 16
// (resp. l ^ 32) in every lane.
__device__ __forceinline__ float max_xor16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Order-preserving map of a finite or infinite f32 onto u32 (+0 and -0 map
// to the same key so that equal scores tie).
__device__ __forceinline__ uint32_t ordered_key(float f) {
    uint32_t u = __float_as_uint(f + 0.0f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------------------
// MFMA wrappers (gfx950 matrix cores).
//  16x16x32 bf16: lane l holds A[m = l % 16][k-slot 8 * (l / 16) + j] and
//  B[k-slot 8 * (l / 16) + j][n = l % 16] (j = 0..7), and receives
//  D[m = 4 * (l / 16) + r][n = l % 16] (r = 0..3).  Only the pairing of A and
//  B k-slots matters for correctness, so callers may permute the contraction
//  index as long as both operands use the same permutation.
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x4 mfma_16x16x32_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
//  16x16x4 f32: lane l holds A[m = l % 16][k = l / 16], B[k = l / 16][n = l % 16].
__device__ __forceinline__ f32x4 mfma_16x16x4_f32(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

}  // namespace msa

// ---------------------------------------------------------------------------
// Internal launchers (one translation unit per kernel family).  Each returns
// hipSuccess or the launch error; arguments were validated by the caller.
// ---------------------------------------------------------------------------
namespace msa {

// Token rows of the caches.  Without a block table, stream s owns rows
// s * cap .. s * cap + cap - 1 (slot == position).  With one, the caches are
// pools of 128-row pages: logical block b of stream s lives in page
// table[s * stride + b], and its 128 tokens are consecutive rows there.
struct Pager {
    const int32_t* table;      // [n_stream][stride] page of each logical block, or NULL
    int32_t stride;
    int64_t cap;
    __device__ __forceinline__ int64_t row(int64_t s, int tok) const {
        return table ? static_cast<int64_t>(table[s * stride + (tok >> 7)]) * kBlock + (tok & (kBlock - 1))
                     : s * cap + tok;
    }
    // first row of logical block b (its 128 rows follow)
    __device__ __forceinline__ int64_t block_row(int64_t s, int b) const {
        return table ? static_cast<int64_t>(table[s * stride + b]) * kBlock : s * cap + static_cast<int64_t>(b) * kBlock;
    }
    // the same for a (s, b) every lane of the wave shares: the table entry is
    // read through the scalar cache (no vector-memory load, which would be
    // counted with the copies into LDS in flight)
    __device__ __forceinline__ int64_t block_row_uniform(int64_t s, int b) const {
        if (!table) return s * cap + static_cast<int64_t>(b) * kBlock;
        const __attribute__((address_space(4))) int32_t* t =
            (const __attribute__((address_space(4))) int32_t*)(reinterpret_cast<uintptr_t>(table));
        return static_cast<int64_t>(t[s * stride + b]) * kBlock;
    }
};
static_assert(kBlock == 128, "pages are MSA blocks of 128 tokens");

struct CacheView {
    const float* idx_k;        // f32 index keys, or NULL when idx_k16 holds them
    const uint16_t* dsa_k;
    const uint16_t* k;
    const uint16_t* v;
    int64_t cap;
    const uint16_t* idx_k16;   // fp16 index keys, or NULL
    Pager pg;
};

hipError_t launch_append(float* idx_k, uint16_t* idx_k16, uint16_t* dsa_k, uint16_t* k, uint16_t* v, const Pager& pg,
                         const int32_t* stream, const int32_t* pos, int64_t n_new,
                         const float* idx_k_new, const uint16_t* dsa_key_new,
                         const uint16_t* k_new, const uint16_t* v_new, hipStream_t s);
// Quantized K/V append (kv_format 1: int8, 2: 4-bit codes; one f32 scale per
// 32 values): rows d_k_new / d_v_new (bf16) are quantized into the caches.
hipError_t launch_append_kv_quant(int kv_format, uint8_t* k, uint8_t* v, float* k_scale, float* v_scale,
                                  const Pager& pg, const int32_t* stream, const int32_t* pos, int64_t n_new,
                                  const uint16_t* k_new, const uint16_t* v_new, hipStream_t s);

hipError_t launch_block_scores_decode(const CacheView& c, const float* idx_q, const int32_t* stream,
                                      const int32_t* pos, int64_t n_q, int nblk, float* bs,
                                      int64_t nblk_stride, hipStream_t s);
// Small decode problems over an f32 index cache: each block is scanned by
// kFineSub workgroups, which write partial maxima
// bs_part[query][group][block][kFineSub]; launch_topk_blocks with
// n_sub = kFineSub ranks their maxima.  Used when scan_is_fine(n_q, nblk).
constexpr int kFineSub = 8;
constexpr int64_t kFineBelowWorkgroups = 256;   // the regular scan's grid below this size
bool scan_is_fine(int64_t n_q, int nblk);
hipError_t launch_block_scores_decode_fine(const CacheView& c, const float* idx_q, const int32_t* stream,
                                           const int32_t* pos, int64_t n_q, int nblk, float* bs_part,
                                           hipStream_t s);
// Decode step, small problems (scan_is_fine): the fine scan, which also
// writes each query's new index, K and V rows at (stream, pos), scores the
// step's new keys from idx_k_new (k_new, v_new may be NULL) and zeroes the
// attention's arrival counters arrive[n_q][kGroups].
hipError_t launch_decode_step_fine(float* idx_k, uint16_t* k, uint16_t* v, const Pager& pg, const float* idx_q,
                                   const int32_t* stream, const int32_t* pos, int64_t n_q, int nblk,
                                   const float* idx_k_new, const uint16_t* k_new, const uint16_t* v_new,
                                   float* bs_part, int32_t* arrive, hipStream_t s);

// Decode step, larger problems: the scan above (one score per block, nblk
// per (query, group)), which also appends the rows as the fine form does.
hipError_t launch_decode_step_scan(float* idx_k, uint16_t* k, uint16_t* v, const Pager& pg, const float* idx_q,
                                   const int32_t* stream, const int32_t* pos, int64_t n_q, int nblk,
                                   const float* idx_k_new, const uint16_t* k_new, const uint16_t* v_new,
                                   float* bs, hipStream_t s);

// ws: prefill_scores_ws_bytes(pos0 + n_q - 1) bytes (the split keys).
size_t prefill_scores_ws_bytes(int32_t max_pos);
hipError_t launch_block_scores_prefill(const CacheView& c, const float* idx_q, int32_t stream,
                                       int32_t pos0, int64_t n_q, int nblk, float* bs,
                                       int64_t nblk_stride, void* ws, hipStream_t s);

// n_sub > 1: block b's score is the maximum of bs[row + b * n_sub + 0 .. n_sub - 1]
// (partial maxima of a fine scan; nblk_stride = nblk * n_sub).
hipError_t launch_topk_blocks(const float* bs, int64_t nblk_stride, const int32_t* pos,
                              int64_t n_q, int nblk, int top_k, int32_t* sel, int32_t* n_sel,
                              hipStream_t s, int n_sub = 1);
// Same, for the consecutive positions pos0 .. pos0 + n_q - 1.
hipError_t launch_topk_blocks_range(const float* bs, int64_t nblk_stride, int32_t pos0, int64_t n_q,
                                    int nblk, int top_k, int32_t* sel, int32_t* n_sel, hipStream_t s);

// Attention over selected keys.  Token t of entry e of (query i, group g):
//   MSA (unit = 128): entry ids are blocks, keys id * 128 + 0..127;
//   DSA (unit = 1):   entry ids are tokens shared by all groups.
struct AttendArgs {
    const uint16_t* k;
    const uint16_t* v;
    Pager pg;
    const uint16_t* q;
    const int32_t* stream;   // per query
    const int32_t* pos;      // per query
    int64_t n_q;
    const int32_t* sel;
    int sel_len;             // entries per (query, group)
    int sel_g_stride;        // sel_len (MSA) or 0 (DSA, shared list)
    int unit;                // 128 or 1
    float scale;
    float* out;
    void* ws;
    int kv_format;           // 0 bf16; 1 int8, 2 4-bit codes with f32 scales per 32 values
    const float* k_scale;    // [rows][kGroups][kHeadDim / 32] (quantized caches)
    const float* v_scale;
    int32_t stream0;         // stream == NULL: query i is at (stream0, pos0 + i) (a prefill chunk)
    int32_t pos0;
    // Decode step (MSA blocks, at most kRankedBlocks of them; a fine scan's
    // n_sub > 1 partials only up to 512): the selection is ranked by the
    // kernel from the scan's block scores or partial maxima
    // bs_part[query][group][nblk_part][n_sub], as launch_topk_blocks ranks
    // them, instead of read from `sel`; the workgroups of split 0 write it
    // to sel_out [query][group][sel_len] and its size to n_sel_out.
    const float* bs_part = nullptr;
    int nblk_part = 0;
    int n_sub = 1;
    int32_t* sel_out = nullptr;
    int32_t* n_sel_out = nullptr;
    // Decode step: an arrival counter per (query, group), zero at launch;
    // the last split of a pair to finish merges the pair's partials (no
    // combine launch).
    int32_t* arrive = nullptr;
};
constexpr int kRankedBlocks = 1024;
int attend_num_splits(int64_t n_q, int sel_len, int unit);
size_t attend_ws_bytes(int64_t n_q, int sel_len, int unit);
hipError_t launch_attend(const AttendArgs& a, hipStream_t s);
// Indexer projection: split-K GEMM into the workspace, then norm + RoPE +
// writes (q to idx_q, k appended to the f32 or fp16 index cache).
int project_n_split(int64_t n_tok);
size_t project_ws_bytes(int64_t n_tok);
hipError_t launch_index_project(const float* x, int d_model, const float* w_q, const float* w_k,
                                const float* g_q, const float* g_k, float eps, float theta, int rot_dim,
                                const int32_t* stream, const int32_t* pos, int64_t n_tok, float* idx_q,
                                float* idx_k, uint16_t* idx_k16, const Pager& pg, void* ws, hipStream_t s);
// Prefill attention for the consecutive positions pos0 .. pos0 + n_q - 1 of
// one stream (MSA blocks); ws (prefill_attend_ws_bytes(n_q, top_k,
// pos0 + n_q - 1) bytes) holds the per-tile step lists and K and V of the
// used blocks rearranged into matrix-core operand order (bf16; a quantized
// cache, kv_format 1 int8 or 2 4-bit with its f32 scales, is dequantized
// into it).
size_t prefill_attend_ws_bytes(int64_t n_q, int top_k, int32_t max_pos);
hipError_t launch_prefill_attend(const void* k, const void* v, int kv_format, const float* k_scale,
                                 const float* v_scale, const Pager& pg, const uint16_t* q, int32_t stream,
                                 int32_t pos0, int64_t n_q, const int32_t* sel, int top_k, float scale, float* out,
                                 void* ws, hipStream_t s);

size_t dsa_select_ws_bytes(int64_t n_q, int32_t max_pos);
hipError_t launch_dsa_select(const uint16_t* dsa_k, const Pager& pg, const uint16_t* q_idx,
                             const int32_t* stream, const int32_t* pos, int64_t n_q,
                             int32_t max_pos, int top_k, int32_t* sel, int32_t* n_sel,
                             void* ws, hipStream_t s);
// Multi-head indexer form: n_head in {16, 32, 48, 64}, q_idx_h [n_q][n_head][128]
// fp16, head_w [n_q][n_head] f32; same workspace as launch_dsa_select.
hipError_t launch_dsa_select_heads(const uint16_t* dsa_k, const Pager& pg, const uint16_t* q_idx_h,
                                   const float* head_w, int n_head, const int32_t* stream,
                                   const int32_t* pos, int64_t n_q, int32_t max_pos, int top_k,
                                   int32_t* sel, int32_t* n_sel, void* ws, hipStream_t s);

}  // namespace msa
