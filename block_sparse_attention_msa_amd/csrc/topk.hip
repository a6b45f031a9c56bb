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
// Up to 1024 candidates live in registers (a lane's 16 at most; the kernel is
// instantiated for 4, 8 and 16 per lane, so that short contexts do not pay
// the register count of long ones): each of the
// k rounds is a wave maximum after which every lane clears the winner if it
// holds it.  Longer contexts (up to 4096 blocks) keep the keys in LDS; each
// lane keeps the best key of its own slice, the wave takes the maximum over
// lanes k times and only the winning lane rescans its slice.  Up to 64 blocks
// are ranked directly (a block's rank is the number of larger keys).  The k
// winners are written in ascending id order, padded with -1.
#include "common.hpp"
#include "topk_regs.hpp"

namespace msa {
namespace {

// kPer: the widest register path this instantiation holds (candidates
// 64 * kPer); it sets the kernel's register count, and with it how many
// problems share a SIMD, so a launch takes the narrowest that covers its
// contexts (0: none, longer contexts go through LDS).
template <int kPer>
__global__ __launch_bounds__(64) void topk_blocks_kernel(const float* __restrict__ bs,
                                                         int64_t nblk_stride,
                                                         const int32_t* __restrict__ q_pos,
                                                         int32_t pos0, int top_k,
                                                         int32_t* __restrict__ sel,
                                                         int32_t* __restrict__ n_sel, int n_sub) {
    extern __shared__ uint64_t keys[];             // [nblk] candidate keys
    __shared__ int32_t chosen[kMaxTopkBlocks];
    const int64_t qg = blockIdx.x;                 // query * kGroups + group
    const int64_t i = qg / kGroups;
    const int lane = threadIdx.x;
    const float* row = bs + qg * nblk_stride;
    // with one score per block, the register path's candidate scores load
    // together with the query's position (candidates past the row read
    // block 0; those past the visible blocks are masked later)
    constexpr int kPre = kPer > 0 ? kPer : 1;
    float pre[kPre];
    if (kPer > 0 && n_sub == 1) {
        const int nb_row = static_cast<int>(nblk_stride);
#pragma unroll
        for (int j = 0; j < kPre; ++j) {
            const int b = lane + 64 * j;
            pre[j] = row[b < nb_row ? b : 0];
        }
    }
    const int loc = (q_pos ? q_pos[i] : pos0 + static_cast<int>(i)) / kBlock;
    const int nvis = loc + 1;

    // (the widest register path only for one score per block; partial
    // maxima of a fine scan come with short contexts only)
    if (kPer > 0 && nvis > 64 && nvis <= 64 * kPer && (kPer <= 8 || n_sub == 1)) {
        const int k = min(top_k, nvis);
        if constexpr (kPer > 8) topk_in_registers<kPer, true>(row, pre, n_sub, nvis, loc, k, lane, chosen);
        else if constexpr (kPer > 0) topk_in_registers<kPer, false>(row, pre, n_sub, nvis, loc, k, lane, chosen);
        __syncthreads();
        write_ascending(chosen, k, top_k, lane, sel + qg * top_k);
        if (lane == 0) n_sel[qg] = k;
        return;
    }
    // Build keys; lane owns blocks lane, lane + 64, ...
    uint64_t best = 0;
    for (int b = lane; b < nvis; b += 64) {
        float sc = row[b * n_sub];
        for (int j = 1; j < n_sub; ++j) sc = fmaxf(sc, row[b * n_sub + j]);
        uint64_t key = (static_cast<uint64_t>(ordered_key(sc)) << 31) |
                       static_cast<uint64_t>(0x7fffffff - b);
        if (b == loc) key |= 1ull << 63;
        keys[b] = key;
        best = key > best ? key : best;
    }
    const int k = min(top_k, nvis);
    int32_t* out = sel + qg * top_k;
    if (nvis <= 64) {
        // short contexts: lane b holds block b's key; its rank is the number
        // of larger keys (keys are distinct), the k smallest ranks win, and a
        // winner's output slot is the number of winners with a lower id
        __syncthreads();
        const uint64_t mine = best;
        int rank = 0;
        for (int c = 0; c < nvis; ++c) rank += keys[c] > mine;
        const bool win = lane < nvis && rank < k;
        const uint64_t wins = __builtin_amdgcn_ballot_w64(win);
        if (win) out[__builtin_popcountll(wins & ((1ull << lane) - 1ull))] = lane;
        for (int t = k + lane; t < top_k; t += 64) out[t] = -1;
        if (lane == 0) n_sel[qg] = k;
        return;
    }
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
    write_ascending(chosen, k, top_k, lane, out);
    if (lane == 0) n_sel[qg] = k;
}

void launch_topk_kernel(int nblk, dim3 grid, size_t lds, hipStream_t s, const float* bs, int64_t nblk_stride,
                        const int32_t* pos, int32_t pos0, int top_k, int32_t* sel, int32_t* n_sel, int n_sub) {
    if (nblk <= 64 * 4)
        hipLaunchKernelGGL(topk_blocks_kernel<4>, grid, dim3(64), lds, s, bs, nblk_stride, pos, pos0, top_k, sel, n_sel, n_sub);
    else if (nblk <= 64 * 8)
        hipLaunchKernelGGL(topk_blocks_kernel<8>, grid, dim3(64), lds, s, bs, nblk_stride, pos, pos0, top_k, sel, n_sel, n_sub);
    else if (nblk <= 64 * 16)
        hipLaunchKernelGGL(topk_blocks_kernel<16>, grid, dim3(64), lds, s, bs, nblk_stride, pos, pos0, top_k, sel, n_sel, n_sub);
    else
        hipLaunchKernelGGL(topk_blocks_kernel<0>, grid, dim3(64), lds, s, bs, nblk_stride, pos, pos0, top_k, sel, n_sel, n_sub);
}

}  // namespace

hipError_t launch_topk_blocks(const float* bs, int64_t nblk_stride, const int32_t* pos,
                              int64_t n_q, int nblk, int top_k, int32_t* sel, int32_t* n_sel,
                              hipStream_t s, int n_sub) {
    const size_t lds = static_cast<size_t>(nblk) * sizeof(uint64_t);
    launch_topk_kernel(nblk, dim3(static_cast<unsigned>(n_q * kGroups)), lds, s, bs, nblk_stride, pos, 0, top_k, sel,
                       n_sel, n_sub);
    return hipGetLastError();
}

hipError_t launch_topk_blocks_range(const float* bs, int64_t nblk_stride, int32_t pos0, int64_t n_q,
                                    int nblk, int top_k, int32_t* sel, int32_t* n_sel, hipStream_t s) {
    const size_t lds = static_cast<size_t>(nblk) * sizeof(uint64_t);
    launch_topk_kernel(nblk, dim3(static_cast<unsigned>(n_q * kGroups)), lds, s, bs, nblk_stride, nullptr, pos0, top_k,
                       sel, n_sel, 1);
    return hipGetLastError();
}

}  // namespace msa
