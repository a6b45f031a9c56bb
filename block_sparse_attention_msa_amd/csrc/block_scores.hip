// block_scores.hip -- fused indexer score -> causal mask -> 128-token block
// max-pool for MSA ("Add MiniMax-M3 (MSA: MiniMax Sparse Attention)
// support", Implementation: bs = maxpool_128(idx_q . idx_k^T + causal mask),
// one indexer head per GQA group; the llama.cpp MSA commit log forces F32
// accumulation of the indexer score).
//
// Decode: one workgroup per (query, key block).  The F32 index-key cache is
// streamed once with 128-bit loads; each 16-lane DPP row of a wavefront owns
// one group's 512-byte slice of a token row, so a token's four group scores
// come out of one DPP row reduction each and no scores are materialised.
//
// Prefill: the scores of a chunk of consecutive queries form a real GEMM
// (queries x keys x 128 per group); it runs on the f32 matrix cores
// (v_mfma_f32_16x16x4_f32) with the causal mask and the max-pool applied to
// the accumulator tiles in registers.
#include "common.hpp"

namespace msa {
namespace {

constexpr int kRowF4 = kGroups * kIdxDim / 4;   // 128 float4 per token row

// ---------------------------------------------------------------------------
// Decode scan
// ---------------------------------------------------------------------------
constexpr int kScanWaves = 4;
constexpr int kScanTokensPerWave = kBlock / kScanWaves;   // 32
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

__global__ __launch_bounds__(256) void block_scores_decode_kernel(
    const float* __restrict__ idx_k, int64_t cap, const float* __restrict__ idx_q,
    const int32_t* __restrict__ q_stream, const int32_t* __restrict__ q_pos,
    float* __restrict__ bs, int64_t nblk_stride) {
    const int64_t i = blockIdx.x;
    const int b = blockIdx.y;
    const int p = q_pos[i];
    const int loc = p / kBlock;
    float* out = bs + i * kGroups * nblk_stride + b;
    if (b > loc) {
        if (threadIdx.x < kGroups) out[threadIdx.x * nblk_stride] = -INFINITY;
        return;
    }
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int g = lane >> 4;     // the DPP row of this lane = its group
    const int c = lane & 15;     // lane's 16-byte column within the group's first/second half
    const f32x4* qrow = reinterpret_cast<const f32x4*>(idx_q + i * kGroups * kIdxDim);
    const f32x4 q0 = qrow[g * 32 + c];
    const f32x4 q1 = qrow[g * 32 + 16 + c];
    const f32x4* rows = reinterpret_cast<const f32x4*>(
        idx_k + (static_cast<int64_t>(q_stream[i]) * cap + static_cast<int64_t>(b) * kBlock) *
                    (kGroups * kIdxDim)) + g * 32 + c;
    const int t_begin = wave * kScanTokensPerWave;
    const int t_end = min(t_begin + kScanTokensPerWave, p - b * kBlock + 1);
    float m = -INFINITY;
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
    __shared__ float red[kScanWaves][kGroups];
    if (c == 0) red[wave][g] = m;
    __syncthreads();
    if (threadIdx.x < kGroups) {
        const int gg = threadIdx.x;
        out[gg * nblk_stride] = fmaxf(fmaxf(red[0][gg], red[1][gg]), fmaxf(red[2][gg], red[3][gg]));
    }
}

// ---------------------------------------------------------------------------
// Prefill scores on the f32 matrix cores
// ---------------------------------------------------------------------------
constexpr int kPfWaves = 4;
constexpr int kPfSubTiles = 2;                           // 16-query sub-tiles per wave
constexpr int kPfQueriesPerWave = 16 * kPfSubTiles;      // 32
constexpr int kPfQueryTile = kPfWaves * kPfQueriesPerWave;  // 128
constexpr int kPfBlocksPerWg = 16;                       // key range of a workgroup: 2048 keys
constexpr int kPfKeyStage = 64;                          // keys per LDS stage
constexpr int kPfRowPitch = kIdxDim + 4;                 // floats; padding against bank conflicts

__global__ __launch_bounds__(256, 2) void block_scores_prefill_kernel(
    const float* __restrict__ idx_k, int64_t cap, const float* __restrict__ idx_q,
    int32_t stream, int32_t pos0, int64_t n_q, int nblk, int n_ranges, float* __restrict__ bs,
    int64_t nblk_stride) {
    const int g = blockIdx.y;
    const int qtile = blockIdx.x / n_ranges;
    const int range = blockIdx.x % n_ranges;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t q_first = static_cast<int64_t>(qtile) * kPfQueryTile;   // query index
    const int64_t q_wave = q_first + wave * kPfQueriesPerWave;
    const int b_begin = range * kPfBlocksPerWg;
    const int b_end = min(b_begin + kPfBlocksPerWg, nblk);
    const int64_t q_last_tile = min<int64_t>(q_first + kPfQueryTile, n_q) - 1;
    const int max_pos_tile = pos0 + static_cast<int>(q_last_tile);

    // Blocks past every query of the tile: -inf (whole range or its tail).
    const int b_vis_end = min(b_end, max_pos_tile / kBlock + 1);
    for (int idx = threadIdx.x; idx < kPfQueryTile * (b_end - max(b_begin, b_vis_end)); idx += 256) {
        const int nb = b_end - max(b_begin, b_vis_end);
        const int64_t qi = q_first + idx / nb;
        const int bb = max(b_begin, b_vis_end) + idx % nb;
        if (qi < n_q) bs[(qi * kGroups + g) * nblk_stride + bb] = -INFINITY;
    }
    if (b_begin >= b_vis_end) return;

    // Query operands: lane holds dims 32*(lane/16) + 0..31 of query
    // q_wave + 16*st + lane%16 (MFMA kk uses dim 32*(lane/16) + kk).
    float qa[kPfSubTiles][32];
#pragma unroll
    for (int st = 0; st < kPfSubTiles; ++st) {
        int64_t qi = q_wave + 16 * st + (lane & 15);
        qi = min(qi, n_q - 1);
        const f32x4* src = reinterpret_cast<const f32x4*>(idx_q + (qi * kGroups + g) * kIdxDim +
                                                          32 * (lane >> 4));
#pragma unroll
        for (int v4 = 0; v4 < 8; ++v4) {
            const f32x4 x = src[v4];
            qa[st][4 * v4 + 0] = x.x;
            qa[st][4 * v4 + 1] = x.y;
            qa[st][4 * v4 + 2] = x.z;
            qa[st][4 * v4 + 3] = x.w;
        }
    }
    // position of the query in D-row r of sub-tile st: qpos0 + 16 * st + r
    const int qpos0 = pos0 + static_cast<int>(q_wave) + 4 * (lane >> 4);

    __shared__ float ks[2][kPfKeyStage * kPfRowPitch];
    const float* kbase = idx_k + static_cast<int64_t>(stream) * cap * kGroups * kIdxDim + g * kIdxDim;
    const int key_begin = b_begin * kBlock;
    const int key_end = min(b_vis_end * kBlock, max_pos_tile + 1);   // keys past it are invisible
    const int n_stages = (key_end - key_begin + kPfKeyStage - 1) / kPfKeyStage;

    // Cooperative stage load: 64 keys x 128 floats = 2048 float4, 8 per thread.
    auto load_stage = [&](int stage, f32x4 (&reg)[8]) {
        const int kb = key_begin + stage * kPfKeyStage;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int e = threadIdx.x + 256 * j;   // float4 index within the stage
            const int key = e >> 5;
            const int col = e & 31;
            int kk = kb + key;
            kk = min(kk, key_end - 1);
            reg[j] = reinterpret_cast<const f32x4*>(kbase + static_cast<int64_t>(kk) * kGroups * kIdxDim)[col];
        }
    };
    auto store_stage = [&](int buf, const f32x4 (&reg)[8]) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int e = threadIdx.x + 256 * j;
            const int key = e >> 5;
            const int col = e & 31;
            *reinterpret_cast<f32x4*>(&ks[buf][key * kPfRowPitch + 4 * col]) = reg[j];
        }
    };

    f32x4 blkmax[kPfSubTiles];
#pragma unroll
    for (int st = 0; st < kPfSubTiles; ++st) blkmax[st] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};

    f32x4 reg[8];
    load_stage(0, reg);
    store_stage(0, reg);
    __syncthreads();
    for (int stage = 0; stage < n_stages; ++stage) {
        const int buf = stage & 1;
        if (stage + 1 < n_stages) load_stage(stage + 1, reg);
        const int kb = key_begin + stage * kPfKeyStage;
#pragma unroll
        for (int kt = 0; kt < kPfKeyStage / 16; ++kt) {
            // B operand: key kb + 16*kt + lane%16, dims 32*(lane/16) + 0..31
            const float* krow = &ks[buf][(16 * kt + (lane & 15)) * kPfRowPitch + 32 * (lane >> 4)];
            const int key = kb + 16 * kt + (lane & 15);
            f32x4 acc[kPfSubTiles];
#pragma unroll
            for (int st = 0; st < kPfSubTiles; ++st) acc[st] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int v4 = 0; v4 < 8; ++v4) {
                const f32x4 kv = *reinterpret_cast<const f32x4*>(krow + 4 * v4);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
#pragma unroll
                    for (int st = 0; st < kPfSubTiles; ++st)
                        acc[st] = mfma_16x16x4_f32(qa[st][4 * v4 + e], kv[e], acc[st]);
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
                        const int64_t qi = q_wave + 16 * st + 4 * (lane >> 4) + r;
                        if ((lane & 15) == r && qi < n_q) {
                            // blocks past the query's own block are -inf
                            bs[(qi * kGroups + g) * nblk_stride + b] = mx;
                        }
                        blkmax[st][r] = -INFINITY;
                    }
                }
            }
        }
        if (stage + 1 < n_stages) {
            // buf ^ 1 was last read in the previous stage, which every wave
            // finished before the barrier that ended it
            store_stage(buf ^ 1, reg);
            __syncthreads();
        }
    }
}

}  // namespace

hipError_t launch_block_scores_decode(const CacheView& c, const float* idx_q, const int32_t* stream,
                                      const int32_t* pos, int64_t n_q, int nblk, float* bs,
                                      int64_t nblk_stride, hipStream_t s) {
    hipLaunchKernelGGL(block_scores_decode_kernel, dim3(static_cast<unsigned>(n_q), nblk), dim3(256),
                       0, s, c.idx_k, c.cap, idx_q, stream, pos, bs, nblk_stride);
    return hipGetLastError();
}

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
