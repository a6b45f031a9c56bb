// block_scores.hip -- fused indexer score -> causal mask -> 128-token block
// max-pool for MSA ("Add MiniMax-M3 (MSA: MiniMax Sparse Attention)
// support", Implementation: bs = maxpool_128(idx_q . idx_k^T + causal mask),
// one indexer head per GQA group; the llama.cpp MSA commit log forces F32
// accumulation of the indexer score).
//
// This file holds the decode form; the prefill form (matrix cores) is in
// prefill_scores.hip.
//
// Decode: one workgroup per (query, two key blocks; eight for an fp16 cache).  The F32 index-key cache is
// streamed once with 128-bit loads; each 16-lane DPP row of a wavefront owns
// one group's 512-byte slice of a token row, so a token's four group scores
// come out of one DPP row reduction each and no scores are materialised.  An
// fp16 index cache (the review thread's F16 indexer setting) is scanned the
// same way with half the bytes: a lane's 16-byte load holds 8 keys of its
// group, widened to f32 for the products.

#include "common.hpp"

namespace msa {
namespace {

constexpr int kRowF4 = kGroups * kIdxDim / 4;   // 128 float4 per token row

// ---------------------------------------------------------------------------
// Decode scan
// ---------------------------------------------------------------------------
constexpr int kScanWaves = 8;                                        // 512 threads
constexpr int kScanWavesPerBlock = 4;
constexpr int kScanBlocksPerWg = kScanWaves / kScanWavesPerBlock;   // 2 key blocks per workgroup
constexpr int kScanTokensPerWave = kBlock / kScanWavesPerBlock;     // 32
constexpr int kScanUnroll = 8;

__device__ __forceinline__ float dot8(const f32x4& q0, const f32x4& q1, const f32x4& a,
                                      const f32x4& b) {
    float d = q0.x * a.x;
    d = fmaf(q0.y, a.y, d);
    d = fmaf(q0.z, a.z, d);
    d = fmaf(q0.w, a.w, d);
    d = fmaf(q1.x, b.x, d);
    d = fmaf(q1.y, b.y, d);
    d = fmaf(q1.z, b.z, d);
    d = fmaf(q1.w, b.w, d);
    return d;
}

// One workgroup per (query, pair of key blocks); four waves per block, 32
// tokens each.  Index keys are read once with non-temporal 128-bit loads
// (they are streamed, never re-read), 16 KiB per wave in flight.
__global__ __launch_bounds__(64 * kScanWaves) void block_scores_decode_kernel(
    const float* __restrict__ idx_k, Pager pg, const float* __restrict__ idx_q,
    const int32_t* __restrict__ q_stream, const int32_t* __restrict__ q_pos,
    float* __restrict__ bs, int64_t nblk_stride, int nblk) {
    const int64_t i = blockIdx.x;
    const int b0 = blockIdx.y * kScanBlocksPerWg;
    const int p = q_pos[i];
    const int loc = p / kBlock;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform: scalar table reads
    const int g = lane >> 4;     // the DPP row of this lane = its group
    const int c = lane & 15;     // lane's 16-byte column within the group's first/second half
    const int b = b0 + wave / kScanWavesPerBlock;   // this wave's key block
    float m = -INFINITY;
    if (b < nblk && b <= loc) {
        const f32x4* qrow = reinterpret_cast<const f32x4*>(idx_q + i * kGroups * kIdxDim);
        const f32x4 q0 = qrow[g * 32 + c];
        const f32x4 q1 = qrow[g * 32 + 16 + c];
        const f32x4* rows = reinterpret_cast<const f32x4*>(
            idx_k + pg.block_row_uniform(q_stream[i], b) * (kGroups * kIdxDim)) + g * 32 + c;
        const int t_begin = (wave % kScanWavesPerBlock) * kScanTokensPerWave;
        const int t_end = min(t_begin + kScanTokensPerWave, p - b * kBlock + 1);   // causal: tokens <= p
        int t = t_begin;
        for (; t + kScanUnroll <= t_end; t += kScanUnroll) {
            f32x4 a[kScanUnroll], bb[kScanUnroll];
#pragma unroll
            for (int u = 0; u < kScanUnroll; ++u) {
                a[u] = __builtin_nontemporal_load(rows + (t + u) * kRowF4);
                bb[u] = __builtin_nontemporal_load(rows + (t + u) * kRowF4 + 16);
            }
#pragma unroll
            for (int u = 0; u < kScanUnroll; ++u) m = fmaxf(m, row16_sum(dot8(q0, q1, a[u], bb[u])));
        }
        for (; t < t_end; ++t) {
            const f32x4 a = rows[t * kRowF4];
            const f32x4 bb = rows[t * kRowF4 + 16];
            m = fmaxf(m, row16_sum(dot8(q0, q1, a, bb)));
        }
    }
    __shared__ float red[kScanWaves][kGroups];
    if (c == 0) red[wave][g] = m;
    __syncthreads();
    if (threadIdx.x < kGroups * kScanBlocksPerWg) {
        const int gg = threadIdx.x % kGroups;
        const int bl = threadIdx.x / kGroups;
        const int bb2 = b0 + bl;
        if (bb2 < nblk) {
            float r = -INFINITY;    // stays -inf for blocks past the query's own block
#pragma unroll
            for (int w = 0; w < kScanWavesPerBlock; ++w) r = fmaxf(r, red[bl * kScanWavesPerBlock + w][gg]);
            bs[(i * kGroups + gg) * nblk_stride + bb2] = r;
        }
    }
}

// The same scan over an fp16 index cache: a token row is 4 x 128 fp16 =
// 1 KiB, lane c of DPP row g holds dims 8c .. 8c+7 of group g (one 16-byte
// load per token), 16 tokens in flight per wave (16 KiB, as above).
constexpr int kScanUnroll16 = 16;
constexpr int kRowU4h = kGroups * kIdxDim / 8;   // 64 sixteen-byte pieces per fp16 token row
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float dot8h(const f32x4& q0, const f32x4& q1, const u32x4& raw) {
    const f16x8 h = __builtin_bit_cast(f16x8, raw);
    float d = q0.x * static_cast<float>(h[0]);
    d = fmaf(q0.y, static_cast<float>(h[1]), d);
    d = fmaf(q0.z, static_cast<float>(h[2]), d);
    d = fmaf(q0.w, static_cast<float>(h[3]), d);
    d = fmaf(q1.x, static_cast<float>(h[4]), d);
    d = fmaf(q1.y, static_cast<float>(h[5]), d);
    d = fmaf(q1.z, static_cast<float>(h[6]), d);
    d = fmaf(q1.w, static_cast<float>(h[7]), d);
    return d;
}

// One wave per key block in the fp16 scan: a wave streams the block's 128
// token rows (128 KiB), a workgroup eight blocks.  With four waves per block
// (32 KiB per wave, the f32 scan's split) the scan ran 4.6 % slower at 32
// streams x 32K; the f32 scan is fastest with four.
constexpr int kScan16WavesPerBlock = 1;
constexpr int kScan16BlocksPerWg = kScanWaves / kScan16WavesPerBlock;
constexpr int kScan16TokensPerWave = kBlock / kScan16WavesPerBlock;

__global__ __launch_bounds__(64 * kScanWaves) void block_scores_decode_f16_kernel(
    const uint16_t* __restrict__ idx_k, Pager pg, const float* __restrict__ idx_q,
    const int32_t* __restrict__ q_stream, const int32_t* __restrict__ q_pos,
    float* __restrict__ bs, int64_t nblk_stride, int nblk) {
    const int64_t i = blockIdx.x;
    const int b0 = blockIdx.y * kScan16BlocksPerWg;
    const int p = q_pos[i];
    const int loc = p / kBlock;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform: scalar table reads
    const int g = lane >> 4;
    const int c = lane & 15;
    const int b = b0 + wave / kScan16WavesPerBlock;
    float m = -INFINITY;
    if (b < nblk && b <= loc) {
        const f32x4* qrow = reinterpret_cast<const f32x4*>(idx_q + i * kGroups * kIdxDim);
        const f32x4 q0 = qrow[g * 32 + 2 * c];          // dims 8c .. 8c+3 of group g
        const f32x4 q1 = qrow[g * 32 + 2 * c + 1];      // dims 8c+4 .. 8c+7
        const u32x4* rows = reinterpret_cast<const u32x4*>(
            idx_k + pg.block_row_uniform(q_stream[i], b) * (kGroups * kIdxDim)) + g * 16 + c;
        const int t_begin = (wave % kScan16WavesPerBlock) * kScan16TokensPerWave;
        const int t_end = min(t_begin + kScan16TokensPerWave, p - b * kBlock + 1);   // causal: tokens <= p
        int t = t_begin;
        for (; t + kScanUnroll16 <= t_end; t += kScanUnroll16) {
            u32x4 a[kScanUnroll16];
#pragma unroll
            for (int u = 0; u < kScanUnroll16; ++u) a[u] = __builtin_nontemporal_load(rows + (t + u) * kRowU4h);
#pragma unroll
            for (int u = 0; u < kScanUnroll16; ++u) m = fmaxf(m, row16_sum(dot8h(q0, q1, a[u])));
        }
        for (; t < t_end; ++t) m = fmaxf(m, row16_sum(dot8h(q0, q1, rows[t * kRowU4h])));
    }
    __shared__ float red[kScanWaves][kGroups];
    if (c == 0) red[wave][g] = m;
    __syncthreads();
    if (threadIdx.x < kGroups * kScan16BlocksPerWg) {
        const int gg = threadIdx.x % kGroups;
        const int bl = threadIdx.x / kGroups;
        const int bb2 = b0 + bl;
        if (bb2 < nblk) {
            float r = -INFINITY;    // stays -inf for blocks past the query's own block
#pragma unroll
            for (int w = 0; w < kScan16WavesPerBlock; ++w) r = fmaxf(r, red[bl * kScan16WavesPerBlock + w][gg]);
            bs[(i * kGroups + gg) * nblk_stride + bb2] = r;
        }
    }
}

}  // namespace

hipError_t launch_block_scores_decode(const CacheView& c, const float* idx_q, const int32_t* stream,
                                      const int32_t* pos, int64_t n_q, int nblk, float* bs,
                                      int64_t nblk_stride, hipStream_t s) {
    const unsigned ny = static_cast<unsigned>((nblk + kScanBlocksPerWg - 1) / kScanBlocksPerWg);
    const unsigned ny16 = static_cast<unsigned>((nblk + kScan16BlocksPerWg - 1) / kScan16BlocksPerWg);
    if (c.idx_k16)
        hipLaunchKernelGGL(block_scores_decode_f16_kernel, dim3(static_cast<unsigned>(n_q), ny16),
                           dim3(64 * kScanWaves), 0, s, c.idx_k16, c.pg, idx_q, stream, pos, bs, nblk_stride, nblk);
    else
        hipLaunchKernelGGL(block_scores_decode_kernel, dim3(static_cast<unsigned>(n_q), ny), dim3(64 * kScanWaves),
                           0, s, c.idx_k, c.pg, idx_q, stream, pos, bs, nblk_stride, nblk);
    return hipGetLastError();
}

}  // namespace msa
