// topk_regs.hpp -- wave-level top-k of block keys held in registers, shared
// by the block top-k kernels and the decode step's attention kernel (which
// ranks its own blocks).
//
// "Add MiniMax-M3 (MSA: MiniMax Sparse Attention) support": Overview (top-16
// blocks, the query's local block always included) and Implementation (a
// large positive bias on the local block, ranked together with the block
// scores for top-k).  A candidate block is one u64 key: bit 63 = local
// block, bits 62..31 = order-preserving image of the f32 block score, bits
// 30..0 = ~block id, so the maximum key is the local block first, then the
// highest score, then the lower id on equal scores.
#pragma once
#include "common.hpp"

namespace msa {

__device__ __forceinline__ uint64_t make_u64(uint32_t lo, uint32_t hi) {
    return (static_cast<uint64_t>(hi) << 32) | lo;
}

__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// Maximum over the 64 lanes of a u32, delivered to every lane: DPP inside
// each 16-lane row (each step one max with a DPP operand), then the gfx950
// row swaps (v_permlane16_swap pairs rows 0/1 and 2/3, v_permlane32_swap the
// two halves of the wave).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
    x = max(x, dpp_u32<kDppQuadXor1>(x));
    x = max(x, dpp_u32<kDppQuadXor2>(x));
    x = max(x, dpp_u32<kDppRowHalfMirror>(x));
    x = max(x, dpp_u32<kDppRowMirror>(x));
    {
        const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
        x = max(static_cast<uint32_t>(r[0]), static_cast<uint32_t>(r[1]));
    }
    {
        const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
        x = max(static_cast<uint32_t>(r[0]), static_cast<uint32_t>(r[1]));
    }
    return x;
}

// Maximum over the 64 lanes of a u64: the maximum high word, then the
// maximum low word among the lanes holding that high word.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t x) {
    const uint32_t hi = wave_max_u32(static_cast<uint32_t>(x >> 32));
    const uint32_t lo = wave_max_u32(static_cast<uint32_t>(x >> 32) == hi ? static_cast<uint32_t>(x) : 0u);
    return make_u64(lo, hi);
}

// Writes the k winners of one (query, group) in ascending id order, padded
// with -1: a winner's slot is the number of smaller winners.
__device__ __forceinline__ void write_ascending(const int32_t* chosen, int k, int top_k, int lane, int32_t* out) {
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
}

// Candidates held in registers: lane l owns blocks l, l + 64, ..., kPer of
// them (nvis <= 64 * kPer).  Each round takes the wave maximum and every lane
// clears the key equal to it (only its owner has it), so no round waits on
// memory.  kOneSub: one score per block (no partial maxima to fold), which
// keeps the widest instantiation's key loop free of an inner loop (that would
// stop its unrolling and turn the keys into an indexed array).
// pre: the first score of each candidate, loaded by the caller (with one
// score per block, before the query's position is known).
template <int kPer, bool kOneSub>
__device__ __forceinline__ void topk_in_registers(const float* row, const float* pre, int n_sub, int nvis, int loc,
                                                  int k, int lane, int32_t* chosen) {
    uint64_t key[kPer];
    // (loads of blocks past nvis read block 0 and are masked: every load is
    // unconditional, so that they are all in flight together)
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int b = lane + 64 * j;
        const int bl = b < nvis ? b : 0;
        float sc = pre[j];
        if constexpr (!kOneSub) {
            if (n_sub > 1) {
                sc = row[bl * n_sub];
                for (int e = 1; e < n_sub; ++e) sc = fmaxf(sc, row[bl * n_sub + e]);
            }
        }
        const uint64_t kb = (static_cast<uint64_t>(ordered_key(sc)) << 31) | static_cast<uint64_t>(0x7fffffff - b) |
                            (b == loc ? 1ull << 63 : 0ull);
        key[j] = b < nvis ? kb : 0ull;
    }
#pragma unroll 1
    for (int r = 0; r < k; ++r) {
        uint64_t best = key[0];
#pragma unroll
        for (int j = 1; j < kPer; ++j) best = max_u64(best, key[j]);
        const uint64_t w = wave_max_u64(best);
        if (lane == 0) chosen[r] = 0x7fffffff - static_cast<int>(w & 0x7fffffff);
#pragma unroll
        for (int j = 0; j < kPer; ++j) key[j] = key[j] == w ? 0ull : key[j];
    }
}

}  // namespace msa
