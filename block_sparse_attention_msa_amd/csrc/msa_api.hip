// msa_api.hip -- the extern "C" entry points declared in include/msa.h:
// host-side validation (everything is checked before anything is launched),
// workspace sizing and kernel dispatch.  No allocation, no synchronisation,
// no state between calls.
#include "../../include/msa.h"
#include "common.hpp"

#include <atomic>
#include <mutex>

namespace {

using msa::kBlock;
using msa::kGroups;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

enum class Mode { Msa, Dsa };

msa_status check_dims(const msa_dims* d, Mode mode) {
    if (!d) return MSA_ERR_NULL_ARG;
    if (d->n_group != msa::kGroups || d->heads_per_group != msa::kHeadsPerGroup ||
        d->head_dim != msa::kHeadDim || d->idx_dim != msa::kIdxDim)
        return MSA_ERR_UNSUPPORTED;
    if (!(d->scale > 0.f) || !(d->scale < 1e30f)) return MSA_ERR_UNSUPPORTED;
    if (mode == Mode::Msa) {
        if (d->block != kBlock || d->top_k < 1 || d->top_k > msa::kMaxTopkBlocks) return MSA_ERR_UNSUPPORTED;
    } else {
        if (d->block != 1 || d->top_k < 1 || d->top_k > 4096) return MSA_ERR_UNSUPPORTED;
    }
    return MSA_OK;
}

msa_status check_cache(const msa_cache* c) {
    if (!c) return MSA_ERR_NULL_ARG;
    if (c->cap < 1 || c->n_stream < 1) return MSA_ERR_BAD_SHAPE;
    if (c->cap > (int64_t(1) << 31) - 1) return MSA_ERR_UNSUPPORTED;   // positions are int32
    if (c->d_block_table) {
        if (reinterpret_cast<uintptr_t>(c->d_block_table) % 4) return MSA_ERR_MISALIGNED;
        if (c->table_stride < 1 || int64_t(c->table_stride) * kBlock < c->cap) return MSA_ERR_BAD_SHAPE;
    }
    if (c->kv_format < 0 || c->kv_format > 2) return MSA_ERR_UNSUPPORTED;
    if (c->kv_format && (c->k || c->v)) {
        if (!c->k_scale || !c->v_scale) return MSA_ERR_NULL_ARG;
        if (!aligned16(c->k_scale) || !aligned16(c->v_scale)) return MSA_ERR_MISALIGNED;
    }
    return MSA_OK;
}

// n_q: 0 is an empty call, negative is a shape error, more than `limit` is
// unsupported (the launch grids would overflow a dispatch dimension); max_pos
// must lie in the cache.
msa_status check_count_pos(int64_t n, int32_t max_pos, const msa_cache* c, int64_t limit = MSA_MAX_QUERIES) {
    if (n < 0) return MSA_ERR_BAD_SHAPE;
    if (n > limit) return MSA_ERR_UNSUPPORTED;
    if (max_pos < 0 || static_cast<int64_t>(max_pos) >= c->cap) return MSA_ERR_OUT_OF_RANGE;
    return MSA_OK;
}

msa_status check_ptrs(std::initializer_list<const void*> ps) {
    for (const void* p : ps)
        if (!p) return MSA_ERR_NULL_ARG;
    for (const void* p : ps)
        if (!aligned16(p)) return MSA_ERR_MISALIGNED;
    return MSA_OK;
}

msa_status hip_status(hipError_t e) { return e == hipSuccess ? MSA_OK : MSA_ERR_HIP; }

#define MSA_TRY(expr)                    \
    do {                                 \
        const msa_status _st = (expr);   \
        if (_st != MSA_OK) return _st;   \
    } while (0)

int nblk_of(int32_t max_pos) { return max_pos / kBlock + 1; }

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// block scores of msa_select: one f32 per (query, group, block), or kFineSub
// partial maxima per block for the small problems the fine scan takes
size_t select_ws(int64_t n_q, int32_t max_pos) {
    const int nblk = nblk_of(max_pos);
    const size_t per = msa::scan_is_fine(n_q, nblk) ? msa::kFineSub : 1;
    return align256(static_cast<size_t>(n_q) * kGroups * nblk * per * sizeof(float));
}

// msa_decode_step: the block scores, the attention partials, then an
// arrival counter per (query, group).
size_t decode_step_ws(const msa_dims* dims, int64_t n_q, int32_t max_pos) {
    return select_ws(n_q, max_pos) + align256(msa::attend_ws_bytes(n_q, dims->top_k, kBlock)) +
           align256(static_cast<size_t>(n_q) * kGroups * sizeof(int32_t));
}

// msa_decode_step in three kernels (the scan appends the rows, the attention
// kernel ranks the blocks): the f32 index cache, bf16 K/V and at most
// kRankedBlocks blocks.
bool decode_step_fused(const msa_cache* c, int32_t max_pos) {
    return c->idx_k && !c->idx_k_f16 && c->kv_format == 0 && nblk_of(max_pos) <= msa::kRankedBlocks;
}

// msa_select_prefill: block scores, then the split keys of the scorer.
size_t select_prefill_ws(int64_t n_q, int32_t max_pos) {
    return select_ws(n_q, max_pos) + align256(msa::prefill_scores_ws_bytes(max_pos));
}

msa::CacheView view(const msa_cache* c) {
    return msa::CacheView{c->idx_k, c->dsa_k, c->k, c->v, c->cap, c->idx_k_f16,
                          msa::Pager{c->d_block_table, c->table_stride, c->cap}};
}

// The MSA index keys: exactly one of the f32 and fp16 caches.
msa_status check_index_cache(const msa_cache* c) {
    if (c->idx_k && c->idx_k_f16) return MSA_ERR_UNSUPPORTED;
    return check_ptrs({c->idx_k ? static_cast<const void*>(c->idx_k) : static_cast<const void*>(c->idx_k_f16)});
}

msa_status append_impl(Mode mode, const msa_dims* dims, const msa_cache* cache, const int32_t* d_stream,
                       const int32_t* d_pos, int64_t n_new, int32_t max_pos, const float* d_idx_k_new,
                       const uint16_t* d_key_new, const uint16_t* d_k_new, const uint16_t* d_v_new,
                       void* hip_stream) {
    MSA_TRY(check_dims(dims, mode));
    MSA_TRY(check_cache(cache));
    MSA_TRY(check_count_pos(n_new, max_pos, cache, MSA_MAX_ROWS));
    if (n_new == 0) return MSA_OK;
    MSA_TRY(check_ptrs({d_stream, d_pos}));
    if (d_idx_k_new) {
        MSA_TRY(check_ptrs({d_idx_k_new}));
        MSA_TRY(check_index_cache(cache));
    }
    if (d_key_new) MSA_TRY(check_ptrs({d_key_new, cache->dsa_k}));
    if (d_k_new) MSA_TRY(check_ptrs({d_k_new, cache->k}));
    if (d_v_new) MSA_TRY(check_ptrs({d_v_new, cache->v}));
    const bool quant = cache->kv_format != 0 && (d_k_new || d_v_new);
    const hipStream_t st = static_cast<hipStream_t>(hip_stream);
    if (quant) {
        MSA_TRY(hip_status(msa::launch_append_kv_quant(
            cache->kv_format, reinterpret_cast<uint8_t*>(cache->k), reinterpret_cast<uint8_t*>(cache->v),
            cache->k_scale, cache->v_scale, view(cache).pg, d_stream, d_pos, n_new, d_k_new, d_v_new, st)));
        if (!d_idx_k_new && !d_key_new) return MSA_OK;
    }
    return hip_status(msa::launch_append(cache->idx_k, cache->idx_k_f16, cache->dsa_k, cache->k, cache->v, view(cache).pg,
                                         d_stream, d_pos, n_new, d_idx_k_new, d_key_new, quant ? nullptr : d_k_new,
                                         quant ? nullptr : d_v_new, st));
}


// ---------------------------------------------------------------------------
// msa_select without a caller workspace (msa_select_static): the block scores
// live in a library-owned device array of MSA_STATIC_SCRATCH_BYTES.  Each GPU
// holds its own copy at its own address, resolved once per device with
// hipGetSymbolAddress; host code uses only that address (the array's name is
// a host-side stand-in, not a device address).  Every call on a GPU shares
// that GPU's array, so calls that overlap on one GPU race.  The block scores
// need no clearing: the scan writes every entry the top-k reads.
// ---------------------------------------------------------------------------
static __device__ __align__(256) char scratch[MSA_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 256;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

msa_status scratch_of_current_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MSA_ERR_HIP;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (!p) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MSA_ERR_HIP;
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return MSA_OK;
}

// msa_select's checks and launches; the block scores go to the workspace, or
// (use_static) to this device's scratch array.
msa_status select_impl(const msa_dims* dims, const msa_cache* cache, const float* d_idx_q,
                       const int32_t* d_stream, const int32_t* d_pos, int64_t n_q, int32_t max_pos,
                       int32_t* d_sel, int32_t* d_n_sel, void* d_ws, size_t ws_bytes, bool use_static,
                       void* hip_stream) {
    MSA_TRY(check_dims(dims, Mode::Msa));
    MSA_TRY(check_cache(cache));
    MSA_TRY(check_count_pos(n_q, max_pos, cache));
    if (n_q == 0) return MSA_OK;   // empty call: nothing to read or launch
    MSA_TRY(check_index_cache(cache));
    MSA_TRY(check_ptrs({d_idx_q, d_stream, d_pos, d_sel, d_n_sel}));
    if (nblk_of(max_pos) > msa::kMaxBlocks) return MSA_ERR_UNSUPPORTED;
    const size_t need = select_ws(n_q, max_pos);
    if (use_static) {
        if (need > MSA_STATIC_SCRATCH_BYTES) return MSA_ERR_WORKSPACE_TOO_SMALL;
        MSA_TRY(scratch_of_current_device(&d_ws));
    } else {
        MSA_TRY(check_ptrs({d_ws}));
        if (ws_bytes < need) return MSA_ERR_WORKSPACE_TOO_SMALL;
    }
    const hipStream_t s = static_cast<hipStream_t>(hip_stream);
    float* bs = static_cast<float*>(d_ws);
    const int nblk = nblk_of(max_pos);
    if (cache->idx_k && msa::scan_is_fine(n_q, nblk)) {   // few queries over a short context
        MSA_TRY(hip_status(msa::launch_block_scores_decode_fine(view(cache), d_idx_q, d_stream, d_pos, n_q, nblk,
                                                                bs, s)));
        return hip_status(msa::launch_topk_blocks(bs, int64_t(nblk) * msa::kFineSub, d_pos, n_q, nblk, dims->top_k,
                                                  d_sel, d_n_sel, s, msa::kFineSub));
    }
    MSA_TRY(hip_status(msa::launch_block_scores_decode(view(cache), d_idx_q, d_stream, d_pos, n_q, nblk,
                                                       bs, nblk, s)));
    return hip_status(msa::launch_topk_blocks(bs, nblk, d_pos, n_q, nblk, dims->top_k, d_sel, d_n_sel, s));
}

}  // namespace

extern "C" {

const char* msa_status_string(msa_status s) {
    switch (s) {
        case MSA_OK: return "MSA_OK";
        case MSA_ERR_NULL_ARG: return "MSA_ERR_NULL_ARG: a required pointer is NULL";
        case MSA_ERR_BAD_SHAPE: return "MSA_ERR_BAD_SHAPE: negative count or empty cache";
        case MSA_ERR_OUT_OF_RANGE: return "MSA_ERR_OUT_OF_RANGE: position or stream outside the cache";
        case MSA_ERR_MISALIGNED: return "MSA_ERR_MISALIGNED: device pointer not 16-byte aligned";
        case MSA_ERR_WORKSPACE_TOO_SMALL: return "MSA_ERR_WORKSPACE_TOO_SMALL";
        case MSA_ERR_UNSUPPORTED: return "MSA_ERR_UNSUPPORTED: geometry outside the supported set";
        case MSA_ERR_HIP: return "MSA_ERR_HIP: a kernel launch failed";
    }
    return "unknown msa_status";
}

size_t msa_workspace_bytes(const msa_dims* dims, msa_op op, int64_t n_q, int32_t max_pos) {
    const size_t bad = static_cast<size_t>(-1);
    if (n_q < 0 || max_pos < 0) return bad;
    if (n_q > (op == MSA_OP_INDEX_PROJECT ? MSA_MAX_ROWS : MSA_MAX_QUERIES)) return bad;
    const bool dsa = op == DSA_OP_SELECT || op == DSA_OP_ATTEND_DECODE ||
                     (op == MSA_OP_ATTEND_DECODE && dims && dims->block == 1);
    if (check_dims(dims, dsa ? Mode::Dsa : Mode::Msa) != MSA_OK) return bad;
    if (op < MSA_OP_SELECT || op > MSA_OP_DECODE_STEP) return bad;
    if (n_q == 0) return 0;   // an empty call launches nothing and needs no workspace
    switch (op) {
        case MSA_OP_SELECT:
            if (nblk_of(max_pos) > msa::kMaxBlocks) return bad;
            return select_ws(n_q, max_pos);
        case MSA_OP_SELECT_PREFILL:
            if (nblk_of(max_pos) > msa::kMaxBlocks) return bad;
            return select_prefill_ws(n_q, max_pos);
        case MSA_OP_BLOCK_SCORES_PREFILL:
            return align256(msa::prefill_scores_ws_bytes(max_pos));
        case MSA_OP_ATTEND_DECODE:
            return align256(msa::attend_ws_bytes(n_q, dims->top_k, dims->block));
        case MSA_OP_ATTEND_PREFILL:
            return align256(msa::prefill_attend_ws_bytes(n_q, dims->top_k, max_pos));
        case DSA_OP_SELECT:
            return align256(msa::dsa_select_ws_bytes(n_q, max_pos));
        case DSA_OP_ATTEND_DECODE:
            return align256(msa::attend_ws_bytes(n_q, dims->top_k, 1));
        case MSA_OP_INDEX_PROJECT:
            return align256(msa::project_ws_bytes(n_q));
        case MSA_OP_DECODE_STEP:
            if (nblk_of(max_pos) > msa::kMaxBlocks) return bad;
            return decode_step_ws(dims, n_q, max_pos);
    }
    return bad;
}

msa_status msa_index_project(const msa_dims* dims, const msa_cache* cache, const msa_proj* proj,
                             const float* d_x, const int32_t* d_stream, const int32_t* d_pos, int64_t n_tok,
                             int32_t max_pos, float* d_idx_q, void* d_ws, size_t ws_bytes, void* hip_stream) {
    MSA_TRY(check_dims(dims, Mode::Msa));
    MSA_TRY(check_cache(cache));
    if (!proj) return MSA_ERR_NULL_ARG;
    if (proj->d_model < 32 || proj->d_model % 32 || proj->rot_dim < 0 || proj->rot_dim > 64 ||
        proj->rot_dim % 2 || !(proj->eps >= 0.f) || !(proj->rope_theta > 0.f))
        return MSA_ERR_UNSUPPORTED;
    MSA_TRY(check_count_pos(n_tok, max_pos, cache, MSA_MAX_ROWS));
    if (n_tok == 0) return MSA_OK;   // empty call: nothing to read or launch
    MSA_TRY(check_ptrs({proj->d_w_q, proj->d_w_k, proj->d_g_q, proj->d_g_k, d_x, d_stream, d_pos, d_idx_q}));
    MSA_TRY(check_index_cache(cache));
    MSA_TRY(check_ptrs({d_ws}));
    if (ws_bytes < msa::project_ws_bytes(n_tok)) return MSA_ERR_WORKSPACE_TOO_SMALL;
    return hip_status(msa::launch_index_project(d_x, proj->d_model, proj->d_w_q, proj->d_w_k, proj->d_g_q,
                                                proj->d_g_k, proj->eps, proj->rope_theta, proj->rot_dim, d_stream,
                                                d_pos, n_tok, d_idx_q, cache->idx_k, cache->idx_k_f16, view(cache).pg,
                                                d_ws, static_cast<hipStream_t>(hip_stream)));
}

msa_status msa_index_append(const msa_dims* dims, const msa_cache* cache, const int32_t* d_stream,
                            const int32_t* d_pos, int64_t n_new, int32_t max_pos,
                            const float* d_idx_k_new, const uint16_t* d_k_new,
                            const uint16_t* d_v_new, void* hip_stream) {
    return append_impl(Mode::Msa, dims, cache, d_stream, d_pos, n_new, max_pos, d_idx_k_new, nullptr,
                       d_k_new, d_v_new, hip_stream);
}

msa_status dsa_index_append(const msa_dims* dims, const msa_cache* cache, const int32_t* d_stream,
                            const int32_t* d_pos, int64_t n_new, int32_t max_pos,
                            const uint16_t* d_key_new, const uint16_t* d_k_new,
                            const uint16_t* d_v_new, void* hip_stream) {
    return append_impl(Mode::Dsa, dims, cache, d_stream, d_pos, n_new, max_pos, nullptr, d_key_new,
                       d_k_new, d_v_new, hip_stream);
}

msa_status msa_block_scores(const msa_dims* dims, const msa_cache* cache, const float* d_idx_q,
                            const int32_t* d_stream, const int32_t* d_pos, int64_t n_q,
                            int32_t max_pos, float* d_bs, int64_t nblk_stride, void* hip_stream) {
    MSA_TRY(check_dims(dims, Mode::Msa));
    MSA_TRY(check_cache(cache));
    MSA_TRY(check_count_pos(n_q, max_pos, cache));
    if (n_q == 0) return MSA_OK;   // empty call: nothing to read or launch
    MSA_TRY(check_index_cache(cache));
    MSA_TRY(check_ptrs({d_idx_q, d_stream, d_pos, d_bs}));
    if (nblk_stride < nblk_of(max_pos)) return MSA_ERR_BAD_SHAPE;
    return hip_status(msa::launch_block_scores_decode(view(cache), d_idx_q, d_stream, d_pos, n_q,
                                                      nblk_of(max_pos), d_bs, nblk_stride,
                                                      static_cast<hipStream_t>(hip_stream)));
}

msa_status msa_topk_blocks(const msa_dims* dims, const float* d_bs, int64_t nblk_stride,
                           const int32_t* d_pos, int64_t n_q, int32_t max_pos, int32_t* d_sel,
                           int32_t* d_n_sel, void* hip_stream) {
    MSA_TRY(check_dims(dims, Mode::Msa));
    if (n_q < 0) return MSA_ERR_BAD_SHAPE;
    if (n_q > MSA_MAX_QUERIES) return MSA_ERR_UNSUPPORTED;
    if (max_pos < 0) return MSA_ERR_OUT_OF_RANGE;
    if (n_q == 0) return MSA_OK;   // empty call: nothing to read or launch
    MSA_TRY(check_ptrs({d_bs, d_pos, d_sel, d_n_sel}));
    if (nblk_of(max_pos) > msa::kMaxBlocks) return MSA_ERR_UNSUPPORTED;
    if (nblk_stride < nblk_of(max_pos)) return MSA_ERR_BAD_SHAPE;
    return hip_status(msa::launch_topk_blocks(d_bs, nblk_stride, d_pos, n_q, nblk_of(max_pos), dims->top_k,
                                              d_sel, d_n_sel, static_cast<hipStream_t>(hip_stream)));
}

msa_status msa_select(const msa_dims* dims, const msa_cache* cache, const float* d_idx_q,
                      const int32_t* d_stream, const int32_t* d_pos, int64_t n_q, int32_t max_pos,
                      int32_t* d_sel, int32_t* d_n_sel, void* d_ws, size_t ws_bytes,
                      void* hip_stream) {
    return select_impl(dims, cache, d_idx_q, d_stream, d_pos, n_q, max_pos, d_sel, d_n_sel, d_ws, ws_bytes,
                       false, hip_stream);
}

msa_status msa_select_static(const msa_dims* dims, const msa_cache* cache, const float* d_idx_q,
                             const int32_t* d_stream, const int32_t* d_pos, int64_t n_q, int32_t max_pos,
                             int32_t* d_sel, int32_t* d_n_sel, void* hip_stream) {
    return select_impl(dims, cache, d_idx_q, d_stream, d_pos, n_q, max_pos, d_sel, d_n_sel, nullptr, 0, true,
                       hip_stream);
}

msa_status msa_block_scores_prefill(const msa_dims* dims, const msa_cache* cache, const float* d_idx_q,
                                    int32_t stream, int32_t pos0, int64_t n_q, float* d_bs,
                                    int64_t nblk_stride, void* d_ws, size_t ws_bytes, void* hip_stream) {
    MSA_TRY(check_dims(dims, Mode::Msa));
    MSA_TRY(check_cache(cache));
    if (n_q < 0) return MSA_ERR_BAD_SHAPE;
    if (n_q > MSA_MAX_QUERIES) return MSA_ERR_UNSUPPORTED;
    if (stream < 0 || stream >= cache->n_stream || pos0 < 0 || pos0 + n_q > cache->cap)
        return MSA_ERR_OUT_OF_RANGE;
    if (n_q == 0) return MSA_OK;   // empty call: nothing to read or launch
    MSA_TRY(check_index_cache(cache));
    MSA_TRY(check_ptrs({d_idx_q, d_bs}));
    const int32_t max_pos = static_cast<int32_t>(pos0 + n_q - 1);
    if (nblk_stride < nblk_of(max_pos)) return MSA_ERR_BAD_SHAPE;
    MSA_TRY(check_ptrs({d_ws}));
    if (ws_bytes < msa::prefill_scores_ws_bytes(max_pos)) return MSA_ERR_WORKSPACE_TOO_SMALL;
    return hip_status(msa::launch_block_scores_prefill(view(cache), d_idx_q, stream, pos0, n_q,
                                                       nblk_of(max_pos), d_bs, nblk_stride, d_ws,
                                                       static_cast<hipStream_t>(hip_stream)));
}

msa_status msa_select_prefill(const msa_dims* dims, const msa_cache* cache, const float* d_idx_q,
                              int32_t stream, int32_t pos0, int64_t n_q, int32_t* d_sel,
                              int32_t* d_n_sel, void* d_ws, size_t ws_bytes, void* hip_stream) {
    MSA_TRY(check_dims(dims, Mode::Msa));
    MSA_TRY(check_cache(cache));
    if (n_q < 0) return MSA_ERR_BAD_SHAPE;
    if (n_q > MSA_MAX_QUERIES) return MSA_ERR_UNSUPPORTED;
    if (stream < 0 || stream >= cache->n_stream || pos0 < 0 || pos0 + n_q > cache->cap)
        return MSA_ERR_OUT_OF_RANGE;
    if (n_q == 0) return MSA_OK;   // empty call: nothing to read or launch
    MSA_TRY(check_index_cache(cache));
    MSA_TRY(check_ptrs({d_idx_q, d_sel, d_n_sel}));
    const int32_t max_pos = static_cast<int32_t>(pos0 + n_q - 1);
    if (nblk_of(max_pos) > msa::kMaxBlocks) return MSA_ERR_UNSUPPORTED;
    MSA_TRY(check_ptrs({d_ws}));
    if (ws_bytes < select_prefill_ws(n_q, max_pos)) return MSA_ERR_WORKSPACE_TOO_SMALL;
    // The top-k kernel reads each query's position from device memory; the
    // prefill positions pos0 + i are materialised after the block scores.
    const hipStream_t s = static_cast<hipStream_t>(hip_stream);
    const int nblk = nblk_of(max_pos);
    float* bs = static_cast<float*>(d_ws);
    void* keys_ws = static_cast<char*>(d_ws) + select_ws(n_q, max_pos);
    MSA_TRY(hip_status(msa::launch_block_scores_prefill(view(cache), d_idx_q, stream, pos0, n_q, nblk,
                                                        bs, nblk, keys_ws, s)));
    return hip_status(msa::launch_topk_blocks_range(bs, nblk, pos0, n_q, nblk, dims->top_k, d_sel,
                                                    d_n_sel, s));
}

msa_status msa_attend_decode(const msa_dims* dims, const msa_cache* cache, const uint16_t* d_q,
                             const int32_t* d_stream, const int32_t* d_pos, int64_t n_q,
                             int32_t max_pos, const int32_t* d_sel, float* d_out, void* d_ws,
                             size_t ws_bytes, void* hip_stream) {
    // block 1: token ids shared by the groups (the DSA selection)
    if (dims && dims->block == 1)
        return dsa_attend_decode(dims, cache, d_q, d_stream, d_pos, n_q, max_pos, d_sel, d_out, d_ws, ws_bytes,
                                 hip_stream);
    MSA_TRY(check_dims(dims, Mode::Msa));
    MSA_TRY(check_cache(cache));
    MSA_TRY(check_count_pos(n_q, max_pos, cache));
    if (n_q == 0) return MSA_OK;   // empty call: nothing to read or launch
    MSA_TRY(check_ptrs({cache->k, cache->v, d_q, d_stream, d_pos, d_sel, d_out}));
    const size_t need = msa::attend_ws_bytes(n_q, dims->top_k, kBlock);
    if (need) {
        MSA_TRY(check_ptrs({d_ws}));
        if (ws_bytes < need) return MSA_ERR_WORKSPACE_TOO_SMALL;
    }
    msa::AttendArgs a{cache->k, cache->v, view(cache).pg, d_q, d_stream, d_pos, n_q, d_sel,
                      dims->top_k, dims->top_k, kBlock, dims->scale, d_out, d_ws,
                      cache->kv_format, cache->k_scale, cache->v_scale};
    return hip_status(msa::launch_attend(a, static_cast<hipStream_t>(hip_stream)));
}

msa_status msa_decode_step(const msa_dims* dims, const msa_cache* cache, const int32_t* d_stream,
                           const int32_t* d_pos, int64_t n_q, int32_t max_pos, const float* d_idx_k_new,
                           const uint16_t* d_k_new, const uint16_t* d_v_new, const float* d_idx_q,
                           const uint16_t* d_q, int32_t* d_sel, int32_t* d_n_sel, float* d_out, void* d_ws,
                           size_t ws_bytes, void* hip_stream) {
    MSA_TRY(check_dims(dims, Mode::Msa));
    MSA_TRY(check_cache(cache));
    MSA_TRY(check_count_pos(n_q, max_pos, cache));
    if (n_q == 0) return MSA_OK;   // empty call: nothing to read or launch
    MSA_TRY(check_index_cache(cache));
    MSA_TRY(check_ptrs({d_stream, d_pos, d_idx_k_new, d_idx_q, d_q, d_sel, d_n_sel, d_out, d_ws, cache->k, cache->v}));
    if (d_k_new) MSA_TRY(check_ptrs({d_k_new}));
    if (d_v_new) MSA_TRY(check_ptrs({d_v_new}));
    if (nblk_of(max_pos) > msa::kMaxBlocks) return MSA_ERR_UNSUPPORTED;
    const size_t sel_bytes = select_ws(n_q, max_pos);
    const size_t att_bytes = align256(msa::attend_ws_bytes(n_q, dims->top_k, kBlock));
    if (ws_bytes < decode_step_ws(dims, n_q, max_pos)) return MSA_ERR_WORKSPACE_TOO_SMALL;
    char* att_ws = static_cast<char*>(d_ws) + sel_bytes;
    int32_t* arrive = reinterpret_cast<int32_t*>(att_ws + att_bytes);
    if (!decode_step_fused(cache, max_pos)) {
        MSA_TRY(msa_index_append(dims, cache, d_stream, d_pos, n_q, max_pos, d_idx_k_new, d_k_new, d_v_new,
                                 hip_stream));
        MSA_TRY(msa_select(dims, cache, d_idx_q, d_stream, d_pos, n_q, max_pos, d_sel, d_n_sel, d_ws, sel_bytes,
                           hip_stream));
        return msa_attend_decode(dims, cache, d_q, d_stream, d_pos, n_q, max_pos, d_sel, d_out, att_ws, att_bytes,
                                 hip_stream);
    }
    const hipStream_t s = static_cast<hipStream_t>(hip_stream);
    const int nblk = nblk_of(max_pos);
    float* bs_part = static_cast<float*>(d_ws);
    const bool fine = msa::scan_is_fine(n_q, nblk);     // few queries over a short context: partial maxima
    if (fine)
        MSA_TRY(hip_status(msa::launch_decode_step_fine(cache->idx_k, cache->k, cache->v, view(cache).pg, d_idx_q,
                                                        d_stream, d_pos, n_q, nblk, d_idx_k_new, d_k_new, d_v_new,
                                                        bs_part, arrive, s)));
    else
        MSA_TRY(hip_status(msa::launch_decode_step_scan(cache->idx_k, cache->k, cache->v, view(cache).pg, d_idx_q,
                                                        d_stream, d_pos, n_q, nblk, d_idx_k_new, d_k_new, d_v_new,
                                                        bs_part, s)));
    msa::AttendArgs a{cache->k, cache->v, view(cache).pg, d_q, d_stream, d_pos, n_q, d_sel,
                      dims->top_k, dims->top_k, kBlock, dims->scale, d_out, att_ws,
                      0, nullptr, nullptr};
    a.bs_part = bs_part;
    a.nblk_part = nblk;
    a.n_sub = fine ? msa::kFineSub : 1;
    a.sel_out = d_sel;
    a.n_sel_out = d_n_sel;
    a.arrive = fine ? arrive : nullptr;       // few queries: the last split merges (no combine launch)
    return hip_status(msa::launch_attend(a, s));
}

msa_status msa_attend_prefill(const msa_dims* dims, const msa_cache* cache, const uint16_t* d_q,
                              int32_t stream, int32_t pos0, int64_t n_q, const int32_t* d_sel,
                              float* d_out, void* d_ws, size_t ws_bytes, void* hip_stream) {
    MSA_TRY(check_dims(dims, Mode::Msa));
    MSA_TRY(check_cache(cache));
    if (n_q < 0) return MSA_ERR_BAD_SHAPE;
    if (n_q > MSA_MAX_QUERIES) return MSA_ERR_UNSUPPORTED;
    if (stream < 0 || stream >= cache->n_stream || pos0 < 0 || pos0 + n_q > cache->cap)
        return MSA_ERR_OUT_OF_RANGE;
    if (n_q == 0) return MSA_OK;   // empty call: nothing to read or launch
    if (nblk_of(static_cast<int32_t>(pos0 + n_q - 1)) > msa::kMaxBlocks) return MSA_ERR_UNSUPPORTED;
    MSA_TRY(check_ptrs({cache->k, cache->v, d_q, d_sel, d_out, d_ws}));
    if (ws_bytes < msa_workspace_bytes(dims, MSA_OP_ATTEND_PREFILL, n_q, static_cast<int32_t>(pos0 + n_q - 1)))
        return MSA_ERR_WORKSPACE_TOO_SMALL;
    // (a quantized cache is dequantized into the sweep's bf16 operand copy)
    return hip_status(msa::launch_prefill_attend(cache->k, cache->v, cache->kv_format, cache->k_scale,
                                                 cache->v_scale, view(cache).pg, d_q, stream, pos0, n_q, d_sel,
                                                 dims->top_k, dims->scale, d_out, d_ws,
                                                 static_cast<hipStream_t>(hip_stream)));
}

msa_status dsa_select(const msa_dims* dims, const msa_cache* cache, const uint16_t* d_q_idx,
                      const int32_t* d_stream, const int32_t* d_pos, int64_t n_q, int32_t max_pos,
                      int32_t* d_sel, int32_t* d_n_sel, void* d_ws, size_t ws_bytes,
                      void* hip_stream) {
    MSA_TRY(check_dims(dims, Mode::Dsa));
    MSA_TRY(check_cache(cache));
    MSA_TRY(check_count_pos(n_q, max_pos, cache));
    if (n_q == 0) return MSA_OK;   // empty call: nothing to read or launch
    MSA_TRY(check_ptrs({cache->dsa_k, d_q_idx, d_stream, d_pos, d_sel, d_n_sel}));
    if (n_q > 65535) return MSA_ERR_UNSUPPORTED;
    MSA_TRY(check_ptrs({d_ws}));
    if (ws_bytes < msa::dsa_select_ws_bytes(n_q, max_pos)) return MSA_ERR_WORKSPACE_TOO_SMALL;
    return hip_status(msa::launch_dsa_select(cache->dsa_k, view(cache).pg, d_q_idx, d_stream, d_pos, n_q,
                                             max_pos, dims->top_k, d_sel, d_n_sel, d_ws,
                                             static_cast<hipStream_t>(hip_stream)));
}

msa_status dsa_select_heads(const msa_dims* dims, const msa_cache* cache, const uint16_t* d_q_idx_h,
                            const float* d_head_w, int32_t n_head, const int32_t* d_stream,
                            const int32_t* d_pos, int64_t n_q, int32_t max_pos, int32_t* d_sel,
                            int32_t* d_n_sel, void* d_ws, size_t ws_bytes, void* hip_stream) {
    MSA_TRY(check_dims(dims, Mode::Dsa));
    MSA_TRY(check_cache(cache));
    MSA_TRY(check_count_pos(n_q, max_pos, cache));
    if (n_head < 16 || n_head > 64 || n_head % 16) return MSA_ERR_UNSUPPORTED;
    if (n_q == 0) return MSA_OK;   // empty call: nothing to read or launch
    MSA_TRY(check_ptrs({cache->dsa_k, d_q_idx_h, d_head_w, d_stream, d_pos, d_sel, d_n_sel}));
    if (n_q > 65535) return MSA_ERR_UNSUPPORTED;
    MSA_TRY(check_ptrs({d_ws}));
    if (ws_bytes < msa::dsa_select_ws_bytes(n_q, max_pos)) return MSA_ERR_WORKSPACE_TOO_SMALL;
    return hip_status(msa::launch_dsa_select_heads(cache->dsa_k, view(cache).pg, d_q_idx_h, d_head_w, n_head,
                                                   d_stream, d_pos, n_q, max_pos, dims->top_k, d_sel, d_n_sel,
                                                   d_ws, static_cast<hipStream_t>(hip_stream)));
}

msa_status dsa_attend_decode(const msa_dims* dims, const msa_cache* cache, const uint16_t* d_q,
                             const int32_t* d_stream, const int32_t* d_pos, int64_t n_q,
                             int32_t max_pos, const int32_t* d_sel, float* d_out, void* d_ws,
                             size_t ws_bytes, void* hip_stream) {
    MSA_TRY(check_dims(dims, Mode::Dsa));
    MSA_TRY(check_cache(cache));
    MSA_TRY(check_count_pos(n_q, max_pos, cache));
    if (n_q == 0) return MSA_OK;   // empty call: nothing to read or launch
    MSA_TRY(check_ptrs({cache->k, cache->v, d_q, d_stream, d_pos, d_sel, d_out}));
    const size_t need = msa::attend_ws_bytes(n_q, dims->top_k, 1);
    if (need) {
        MSA_TRY(check_ptrs({d_ws}));
        if (ws_bytes < need) return MSA_ERR_WORKSPACE_TOO_SMALL;
    }
    msa::AttendArgs a{cache->k, cache->v, view(cache).pg, d_q, d_stream, d_pos, n_q, d_sel,
                      dims->top_k, 0, 1, dims->scale, d_out, d_ws,
                      cache->kv_format, cache->k_scale, cache->v_scale};
    return hip_status(msa::launch_attend(a, static_cast<hipStream_t>(hip_stream)));
}

}  // extern "C"
