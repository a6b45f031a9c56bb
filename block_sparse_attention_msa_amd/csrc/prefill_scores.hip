// prefill_scores.hip -- indexer score -> causal mask -> 128-token block
// max-pool for a prefill chunk ("Add MiniMax-M3 (MSA: MiniMax Sparse
// Attention) support", Implementation: bs = maxpool_128(idx_q . idx_k^T +
// causal mask) per group; batch and decode share these semantics).
//
// The scores of a chunk of consecutive queries of one stream form a real GEMM
// (queries x keys x 128 per group); it runs on the bf16 matrix cores with a
// three-term hi/lo split of the f32 inputs, and the causal mask and the
// max-pool are applied to the accumulator tiles in registers, so no score is
// ever written.
#include "common.hpp"

namespace msa {
namespace {

// ---------------------------------------------------------------------------
// Prefill scores on the bf16 matrix cores, three-term split
//
// Each f32 input x is split into x_hi = bf16(x) and x_lo = bf16(x - x_hi)
// (x - x_hi is exact in f32), and q.k is accumulated in f32 as
// q_hi.k_hi + q_hi.k_lo + q_lo.k_hi on v_mfma_f32_16x16x32_bf16.  The dropped
// q_lo.k_lo term and the rounding of the lo parts are ~2^-16 of each product,
// i.e. a few 1e-7 on the scaled prefill scores (std ~0.09), well inside the
// 1e-5 * max|score| near-tie band; the products are summed in f32 as the
// commit log of the MSA port requires.  Same idea as the FP16 hi/lo split in
// Strata's tensor-core prompt attention header, with bf16 for its f32 range.
// ---------------------------------------------------------------------------
constexpr int kPfWaves = 4;
constexpr int kPfSubTiles = 3;                              // 16-query sub-tiles per wave
constexpr int kPfQueriesPerWave = 16 * kPfSubTiles;         // 48
constexpr int kPfQueryTile = kPfWaves * kPfQueriesPerWave;  // 192
constexpr int kPfBlocksPerWg = 16;                          // key range of a workgroup: 2048 keys
constexpr int kPfKeyStage = 64;                             // keys per LDS stage
constexpr int kPfPitch = kIdxDim + 8;                       // bf16 per LDS key row (padding)

struct PfStage {
    __bf16 hi[kPfKeyStage * kPfPitch];
    __bf16 lo[kPfKeyStage * kPfPitch];
};

__device__ __forceinline__ void split_bf16(float x, __bf16& hi, __bf16& lo) {
    hi = static_cast<__bf16>(x);
    lo = static_cast<__bf16>(x - static_cast<float>(hi));
}

__global__ __launch_bounds__(256, 2) void block_scores_prefill_kernel(
    const float* __restrict__ idx_k, int64_t cap, const float* __restrict__ idx_q,
    int32_t stream, int32_t pos0, int64_t n_q, int nblk, int n_ranges, float* __restrict__ bs,
    int64_t nblk_stride) {
    const int g = blockIdx.y;
    const int qtile = blockIdx.x / n_ranges;
    const int range = blockIdx.x % n_ranges;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int l16 = lane & 15;
    const int l4 = lane >> 4;
    const int64_t q_first = static_cast<int64_t>(qtile) * kPfQueryTile;   // query index
    const int64_t q_wave = q_first + wave * kPfQueriesPerWave;
    const int b_begin = range * kPfBlocksPerWg;
    const int b_end = min(b_begin + kPfBlocksPerWg, nblk);
    const int64_t q_last_tile = min<int64_t>(q_first + kPfQueryTile, n_q) - 1;
    const int max_pos_tile = pos0 + static_cast<int>(q_last_tile);

    // Blocks past every query of the tile: -inf (whole range or its tail).
    const int b_vis_end = min(b_end, max_pos_tile / kBlock + 1);
    {
        const int b0 = max(b_begin, b_vis_end);
        const int nb = b_end - b0;
        for (int idx = threadIdx.x; idx < kPfQueryTile * nb; idx += 256) {
            const int64_t qi = q_first + idx / nb;
            if (qi < n_q) bs[(qi * kGroups + g) * nblk_stride + b0 + idx % nb] = -INFINITY;
        }
    }
    if (b_begin >= b_vis_end) return;

    // Query operands (A: m = query, k = dim): lane holds query
    // q_wave + 16*st + l16, dims 32*ks + 8*l4 + 0..7, as hi and lo parts.
    bf16x8 qhi[kPfSubTiles][4], qlo[kPfSubTiles][4];
#pragma unroll
    for (int st = 0; st < kPfSubTiles; ++st) {
        const int64_t qi = min<int64_t>(q_wave + 16 * st + l16, n_q - 1);
        const float* src = idx_q + (qi * kGroups + g) * kIdxDim + 8 * l4;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const f32x4 x0 = *reinterpret_cast<const f32x4*>(src + 32 * ks);
            const f32x4 x1 = *reinterpret_cast<const f32x4*>(src + 32 * ks + 4);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                __bf16 h, l;
                split_bf16(e < 4 ? x0[e] : x1[e - 4], h, l);
                qhi[st][ks][e] = h;
                qlo[st][ks][e] = l;
            }
        }
    }
    // position of the query in D-row r of sub-tile st: qpos0 + 16 * st + r
    const int qpos0 = pos0 + static_cast<int>(q_wave) + 4 * l4;

    __shared__ PfStage stage_buf[2];
    const float* kbase = idx_k + static_cast<int64_t>(stream) * cap * kGroups * kIdxDim + g * kIdxDim;
    const int key_begin = b_begin * kBlock;
    const int key_end = min(b_vis_end * kBlock, max_pos_tile + 1);   // keys past it are invisible
    const int n_stages = (key_end - key_begin + kPfKeyStage - 1) / kPfKeyStage;

    // Cooperative stage load: 64 keys x 128 floats = 2048 float4, 8 per thread,
    // split into hi / lo bf16 rows on the way into LDS.
    auto load_stage = [&](int stage, f32x4 (&reg)[8]) {
        const int kb = key_begin + stage * kPfKeyStage;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int e = threadIdx.x + 256 * j;   // float4 index within the stage
            const int kk = min(kb + (e >> 5), key_end - 1);
            reg[j] = reinterpret_cast<const f32x4*>(kbase + static_cast<int64_t>(kk) * kGroups * kIdxDim)[e & 31];
        }
    };
    auto store_stage = [&](PfStage& st_buf, const f32x4 (&reg)[8]) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int e = threadIdx.x + 256 * j;
            const int off = (e >> 5) * kPfPitch + 4 * (e & 31);
            __bf16 h[4], l[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) split_bf16(reg[j][c], h[c], l[c]);
            *reinterpret_cast<uint2*>(&st_buf.hi[off]) = __builtin_bit_cast(uint2, h);
            *reinterpret_cast<uint2*>(&st_buf.lo[off]) = __builtin_bit_cast(uint2, l);
        }
    };

    f32x4 blkmax[kPfSubTiles];
#pragma unroll
    for (int st = 0; st < kPfSubTiles; ++st) blkmax[st] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};

    f32x4 reg[8];
    load_stage(0, reg);
    store_stage(stage_buf[0], reg);
    __syncthreads();
    for (int stage = 0; stage < n_stages; ++stage) {
        const PfStage& sb = stage_buf[stage & 1];
        if (stage + 1 < n_stages) load_stage(stage + 1, reg);
        const int kb = key_begin + stage * kPfKeyStage;
#pragma unroll
        for (int kt = 0; kt < kPfKeyStage / 16; ++kt) {
            // B operand (k = dim, n = key): key kb + 16*kt + l16, dims 32*ks + 8*l4 + 0..7
            const int row = (16 * kt + l16) * kPfPitch + 8 * l4;
            const int key = kb + 16 * kt + l16;
            f32x4 acc[kPfSubTiles];
#pragma unroll
            for (int st = 0; st < kPfSubTiles; ++st) acc[st] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const bf16x8 bhi = *reinterpret_cast<const bf16x8*>(&sb.hi[row + 32 * ks]);
                const bf16x8 blo = *reinterpret_cast<const bf16x8*>(&sb.lo[row + 32 * ks]);
#pragma unroll
                for (int st = 0; st < kPfSubTiles; ++st) {
                    acc[st] = mfma_16x16x32_bf16(qhi[st][ks], bhi, acc[st]);
                    acc[st] = mfma_16x16x32_bf16(qhi[st][ks], blo, acc[st]);
                    acc[st] = mfma_16x16x32_bf16(qlo[st][ks], bhi, acc[st]);
                }
            }
#pragma unroll
            for (int st = 0; st < kPfSubTiles; ++st) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float sv = (key <= qpos0 + 16 * st + r && key < key_end) ? acc[st][r] : -INFINITY;
                    blkmax[st][r] = fmaxf(blkmax[st][r], sv);
                }
            }
            // end of a 128-key block (or of the visible keys): reduce over the
            // 16 key lanes and write; tiles wholly past key_end write nothing
            const int kend = kb + 16 * kt + 16;
            if (kend - 16 < key_end && ((kend % kBlock) == 0 || kend >= key_end)) {
                const int b = (kend - 1) / kBlock;
#pragma unroll
                for (int st = 0; st < kPfSubTiles; ++st) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float mx = row16_max(blkmax[st][r]);
                        const int64_t qi = q_wave + 16 * st + 4 * l4 + r;
                        if (l16 == r && qi < n_q) bs[(qi * kGroups + g) * nblk_stride + b] = mx;
                        blkmax[st][r] = -INFINITY;
                    }
                }
            }
        }
        if (stage + 1 < n_stages) {
            // the other buffer was last read in the previous stage, which every
            // wave finished before the barrier that ended it
            store_stage(stage_buf[(stage + 1) & 1], reg);
            __syncthreads();
        }
    }
}

}  // namespace

hipError_t launch_block_scores_prefill(const CacheView& c, const float* idx_q, int32_t stream,
                                       int32_t pos0, int64_t n_q, int nblk, float* bs,
                                       int64_t nblk_stride, hipStream_t s) {
    const int n_qtiles = static_cast<int>((n_q + kPfQueryTile - 1) / kPfQueryTile);
    const int n_ranges = (nblk + kPfBlocksPerWg - 1) / kPfBlocksPerWg;
    hipLaunchKernelGGL(block_scores_prefill_kernel, dim3(n_qtiles * n_ranges, kGroups), dim3(256), 0,
                       s, c.idx_k, c.cap, idx_q, stream, pos0, n_q, nblk, n_ranges, bs, nblk_stride);
    return hipGetLastError();
}

}  // namespace msa
