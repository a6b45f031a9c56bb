// topk.hip -- per-(query, group) top-k block selection for MSA.
//
// "Add MiniMax-M3 (MSA: MiniMax Sparse Attention) support": Overview (top-16
// blocks, the query's local block always included) and Implementation (a
// large positive bias on the local block, ranked together with the block
// scores for top-k); review thread: k = min(indexer_top_k, nblk).
//
// One wavefront per (query, group).  Every candidate block becomes one u64
// key:  bit 63 = local block, bits 62..31 = order-preserving image of the
// f32 block score, bits 30..0 = ~block id.  The maximum key is therefore the
// local block first, then the highest score, then the LOWER id on equal
// scores -- a total order, so the selection is unique and deterministic.
// Keys live in LDS (8 bytes per candidate block); each lane keeps the best key of its own slice, the wave
// takes the maximum over lanes k times and only the winning lane rescans its
// slice.  The k winners are written in ascending id order, padded with -1.
#include "common.hpp"

namespace msa {
namespace {

__device__ __forceinline__ uint64_t make_u64(uint32_t lo, uint32_t hi) {
    return (static_cast<uint64_t>(hi) << 32) | lo;
}

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t x) {
    const uint32_t lo = static_cast<uint32_t>(
        __builtin_amdgcn_update_dpp(0, static_cast<int>(static_cast<uint32_t>(x)), CTRL, 0xf, 0xf, false));
    const uint32_t hi = static_cast<uint32_t>(
        __builtin_amdgcn_update_dpp(0, static_cast<int>(static_cast<uint32_t>(x >> 32)), CTRL, 0xf, 0xf, false));
    return make_u64(lo, hi);
}

__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// Maximum over the 64 lanes, delivered to every lane: DPP inside each
// 16-lane row, then the gfx950 row swaps (v_permlane16_swap pairs rows 0/1
// and 2/3, v_permlane32_swap pairs the two halves of the wave).
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t x) {
    x = max_u64(x, dpp_u64<kDppQuadXor1>(x));
    x = max_u64(x, dpp_u64<kDppQuadXor2>(x));
    x = max_u64(x, dpp_u64<kDppRowHalfMirror>(x));
    x = max_u64(x, dpp_u64<kDppRowMirror>(x));
    {
        const auto lo = __builtin_amdgcn_permlane16_swap(static_cast<uint32_t>(x), static_cast<uint32_t>(x),
                                                         false, false);
        const auto hi = __builtin_amdgcn_permlane16_swap(static_cast<uint32_t>(x >> 32),
                                                         static_cast<uint32_t>(x >> 32), false, false);
        x = max_u64(make_u64(lo[0], hi[0]), make_u64(lo[1], hi[1]));
    }
    {
        const auto lo = __builtin_amdgcn_permlane32_swap(static_cast<uint32_t>(x), static_cast<uint32_t>(x),
                                                         false, false);
        const auto hi = __builtin_amdgcn_permlane32_swap(static_cast<uint32_t>(x >> 32),
                                                         static_cast<uint32_t>(x >> 32), false, false);
        x = max_u64(make_u64(lo[0], hi[0]), make_u64(lo[1], hi[1]));
    }
    return x;
}

__global__ __launch_bounds__(64) void topk_blocks_kernel(const float* __restrict__ bs,
                                                         int64_t nblk_stride,
                                                         const int32_t* __restrict__ q_pos,
                                                         int32_t pos0, int top_k,
                                                         int32_t* __restrict__ sel,
                                                         int32_t* __restrict__ n_sel) {
    extern __shared__ uint64_t keys[];             // [nblk] candidate keys
    __shared__ int32_t chosen[kMaxTopkBlocks];
    const int64_t qg = blockIdx.x;                 // query * kGroups + group
    const int64_t i = qg / kGroups;
    const int lane = threadIdx.x;
    const int loc = (q_pos ? q_pos[i] : pos0 + static_cast<int>(i)) / kBlock;
    const int nvis = loc + 1;
    const float* row = bs + qg * nblk_stride;

    // Build keys; lane owns blocks lane, lane + 64, ...
    uint64_t best = 0;
    for (int b = lane; b < nvis; b += 64) {
        uint64_t key = (static_cast<uint64_t>(ordered_key(row[b])) << 31) |
                       static_cast<uint64_t>(0x7fffffff - b);
        if (b == loc) key |= 1ull << 63;
        keys[b] = key;
        best = key > best ? key : best;
    }
    const int k = min(top_k, nvis);
    for (int r = 0; r < k; ++r) {
        const uint64_t w = wave_max_u64(best);
        const int b = 0x7fffffff - static_cast<int>(w & 0x7fffffff);
        if (lane == 0) chosen[r] = b;
        if ((b & 63) == lane) {                    // the owner removes it and rescans
            keys[b] = 0;
            best = 0;
            for (int bb = lane; bb < nvis; bb += 64) best = keys[bb] > best ? keys[bb] : best;
        }
    }
    __syncthreads();
    // ascending order: a winner's rank is the number of smaller winners
    int32_t* out = sel + qg * top_k;
    for (int t = lane; t < top_k; t += 64) {
        if (t < k) {
            const int b = chosen[t];
            int rank = 0;
            for (int u = 0; u < k; ++u) rank += chosen[u] < b;
            out[rank] = b;
        } else {
            out[t] = -1;
        }
    }
    if (lane == 0) n_sel[qg] = k;
}

}  // namespace

hipError_t launch_topk_blocks(const float* bs, int64_t nblk_stride, const int32_t* pos,
                              int64_t n_q, int nblk, int top_k, int32_t* sel, int32_t* n_sel,
                              hipStream_t s) {
    const size_t lds = static_cast<size_t>(nblk) * sizeof(uint64_t);
    hipLaunchKernelGGL(topk_blocks_kernel, dim3(static_cast<unsigned>(n_q * kGroups)), dim3(64), lds, s,
                       bs, nblk_stride, pos, 0, top_k, sel, n_sel);
    return hipGetLastError();
}

hipError_t launch_topk_blocks_range(const float* bs, int64_t nblk_stride, int32_t pos0, int64_t n_q,
                                    int nblk, int top_k, int32_t* sel, int32_t* n_sel, hipStream_t s) {
    const size_t lds = static_cast<size_t>(nblk) * sizeof(uint64_t);
    hipLaunchKernelGGL(topk_blocks_kernel, dim3(static_cast<unsigned>(n_q * kGroups)), dim3(64), lds, s,
                       bs, nblk_stride, nullptr, pos0, top_k, sel, n_sel);
    return hipGetLastError();
}

}  // namespace msa
