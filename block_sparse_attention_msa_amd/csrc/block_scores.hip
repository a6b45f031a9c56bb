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

// Decode step (kStep): the scan also appends the step's rows, as the fine
// scan of small problems does (decode_step_fine_kernel): the workgroup
// holding a query's own block writes its index, K and V rows, and the new
// keys are scored from the inputs -- the query's own token after the loop,
// and (rare: several queries of one stream) a wave whose tokens hold another
// query's new row scores its tokens one by one from wherever each lives.
struct StepRows {
    float* idx_k;               // the cache the rows go to
    uint16_t* k;
    uint16_t* v;
    int64_t n_q;
    const float* idx_k_new;     // [n_q][kGroups][kIdxDim]
    const uint16_t* k_new;      // [n_q][kGroups][kHeadDim] bf16, or NULL
    const uint16_t* v_new;
};

// One workgroup per (query, pair of key blocks); four waves per block, 32
// tokens each.  Index keys are read once with non-temporal 128-bit loads
// (they are streamed, never re-read), 16 KiB per wave in flight.
template <bool kStep>
__global__ __launch_bounds__(64 * kScanWaves) void block_scores_decode_kernel(
    const float* __restrict__ idx_k, Pager pg, const float* __restrict__ idx_q,
    const int32_t* __restrict__ q_stream, const int32_t* __restrict__ q_pos,
    float* __restrict__ bs, int64_t nblk_stride, int nblk, StepRows st) {
    const int64_t i = blockIdx.x;
    const int b0 = blockIdx.y * kScanBlocksPerWg;
    const int p = q_pos[i];
    const int loc = p / kBlock;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform: scalar table reads
    const int g = lane >> 4;     // the DPP row of this lane = its group
    const int c = lane & 15;     // lane's 16-byte column within the group's first/second half
    const int b = b0 + wave / kScanWavesPerBlock;   // this wave's key block
    if constexpr (kStep) {
        if (loc >= b0 && loc < b0 + kScanBlocksPerWg) {      // this workgroup holds the query's own token
            const int tid = threadIdx.x;
            const int64_t slot = pg.row(q_stream[i], p);
            if (tid < kGroups * kIdxDim / 4)
                reinterpret_cast<u32x4*>(st.idx_k + slot * kGroups * kIdxDim)[tid] =
                    reinterpret_cast<const u32x4*>(st.idx_k_new + i * kGroups * kIdxDim)[tid];
            if (tid < kGroups * kHeadDim / 8) {
                if (st.k_new)
                    reinterpret_cast<u32x4*>(st.k + slot * kGroups * kHeadDim)[tid] =
                        reinterpret_cast<const u32x4*>(st.k_new + i * kGroups * kHeadDim)[tid];
                if (st.v_new)
                    reinterpret_cast<u32x4*>(st.v + slot * kGroups * kHeadDim)[tid] =
                        reinterpret_cast<const u32x4*>(st.v_new + i * kGroups * kHeadDim)[tid];
            }
        }
    }
    float m = -INFINITY;
    if (b < nblk && b <= loc) {
        const f32x4* qrow = reinterpret_cast<const f32x4*>(idx_q + i * kGroups * kIdxDim);
        const f32x4 q0 = qrow[g * 32 + c];
        const f32x4 q1 = qrow[g * 32 + 16 + c];
        const f32x4* rows = reinterpret_cast<const f32x4*>(
            idx_k + pg.block_row_uniform(q_stream[i], b) * (kGroups * kIdxDim)) + g * 32 + c;
        const int t_begin = (wave % kScanWavesPerBlock) * kScanTokensPerWave;
        const int t_last = min(t_begin + kScanTokensPerWave, p - b * kBlock + 1);   // causal: tokens <= p
        int t_end = t_last;
        // step: this wave holds the query's own token (its last), scored
        // from the input after the loop
        const bool own = kStep && t_begin < t_end && b * kBlock + t_end - 1 == p;
        if (own) --t_end;
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
        if (own) {
            const f32x4* src = reinterpret_cast<const f32x4*>(st.idx_k_new + i * kGroups * kIdxDim) + g * 32 + c;
            m = fmaxf(m, row16_sum(dot8(q0, q1, src[0], src[16])));
        }
        if constexpr (kStep) {
            // Rare: another query of the launch appends into this wave's
            // tokens, so the rows read above may not hold it yet.  Checked
            // after the loop (the loop's loads need not wait for this one),
            // and the wave's tokens are then scored again one by one from
            // wherever each lives.
            const int s = q_stream[i];
            bool other = false;
            for (int64_t j0 = 0; j0 < st.n_q; j0 += 64) {
                const int64_t j = j0 + lane;
                bool hit = false;
                if (j < st.n_q && j != i && q_stream[j] == s) {
                    const int pj = q_pos[j] - b * kBlock;
                    hit = pj >= t_begin && pj < t_last;
                }
                other = other || __builtin_amdgcn_ballot_w64(hit) != 0;
            }
            if (other) {
                m = -INFINITY;
                for (int tt = t_begin; tt < t_last; ++tt) {
                    const int tok = b * kBlock + tt;
                    int64_t src_q = tok == p ? i : -1;
                    for (int64_t j0 = 0; j0 < st.n_q && src_q < 0; j0 += 64) {
                        const int64_t j = j0 + lane;
                        const bool hit = j < st.n_q && q_stream[j] == s && q_pos[j] == tok;
                        const uint64_t mk = __builtin_amdgcn_ballot_w64(hit);
                        if (mk) src_q = j0 + __builtin_ctzll(mk);
                    }
                    const f32x4* src = src_q >= 0
                                           ? reinterpret_cast<const f32x4*>(st.idx_k_new + src_q * kGroups * kIdxDim) + g * 32 + c
                                           : rows + tt * kRowF4;
                    m = fmaxf(m, row16_sum(dot8(q0, q1, src[0], src[16])));
                }
            }
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

// Small problems (a few queries over a short context: fewer workgroups than
// compute units in the scan above) split every block over kFineSub
// workgroups of four waves, four tokens per wave, so that the whole scan is
// one round of loads in flight; each workgroup writes the partial maximum
// of its 16 tokens per group, and the top-k takes the maximum of a block's
// kFineSub partials (a max is exact in any order, so the block scores are
// those of the scan above, bit for bit).
constexpr int kFineWaves = 4;
constexpr int kFineTokPerWave = kBlock / (kFineSub * kFineWaves);   // 4

__global__ __launch_bounds__(64 * kFineWaves) void block_scores_decode_fine_kernel(
    const float* __restrict__ idx_k, Pager pg, const float* __restrict__ idx_q,
    const int32_t* __restrict__ q_stream, const int32_t* __restrict__ q_pos,
    float* __restrict__ bs_part, int nblk) {
    const int64_t i = blockIdx.x;
    const int b = blockIdx.y;
    const int sub = blockIdx.z;
    const int p = q_pos[i];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4;
    const int c = lane & 15;
    float m = -INFINITY;
    const int t_begin = (sub * kFineWaves + wave) * kFineTokPerWave;
    const int t_end = min(t_begin + kFineTokPerWave, p - b * kBlock + 1);   // causal: tokens <= p
    if (t_begin < t_end) {
        const f32x4* qrow = reinterpret_cast<const f32x4*>(idx_q + i * kGroups * kIdxDim);
        const f32x4 q0 = qrow[g * 32 + c];
        const f32x4 q1 = qrow[g * 32 + 16 + c];
        const f32x4* rows = reinterpret_cast<const f32x4*>(
            idx_k + pg.block_row_uniform(q_stream[i], b) * (kGroups * kIdxDim)) + g * 32 + c;
        f32x4 a[kFineTokPerWave], bb[kFineTokPerWave];
#pragma unroll
        for (int u = 0; u < kFineTokPerWave; ++u) {
            const int t = min(t_begin + u, t_end - 1);           // past the query: its last visible token again
            a[u] = __builtin_nontemporal_load(rows + t * kRowF4);
            bb[u] = __builtin_nontemporal_load(rows + t * kRowF4 + 16);
        }
#pragma unroll
        for (int u = 0; u < kFineTokPerWave; ++u) m = fmaxf(m, row16_sum(dot8(q0, q1, a[u], bb[u])));
    }
    __shared__ float red[kFineWaves][kGroups];
    if (c == 0) red[wave][g] = m;
    __syncthreads();
    if (threadIdx.x < kGroups) {
        float r = red[0][threadIdx.x];
#pragma unroll
        for (int w = 1; w < kFineWaves; ++w) r = fmaxf(r, red[w][threadIdx.x]);
        bs_part[((i * kGroups + threadIdx.x) * nblk + b) * kFineSub + sub] = r;
    }
}

// Decode step, small problems: the fine scan of the step's queries, which
// also appends the step's rows.  The new index keys are scored from the
// inputs (a row this launch writes cannot be read back by it): the query's
// own token, and any token of its stream that another query of the launch
// appends (found by a ballot over the launch's (stream, position) pairs,
// 64 per round; rows loaded from the cache for such a token are replaced).
// The workgroup holding a query's own token writes its index, K and V rows,
// which later kernels read.  The dot products, and with them the partial
// maxima, are those of the fine scan, bit for bit.
struct StepScanArgs {
    float* idx_k;
    uint16_t* k;
    uint16_t* v;
    Pager pg;
    const float* idx_q;
    const int32_t* stream;
    const int32_t* pos;
    int64_t n_q;
    const float* idx_k_new;     // [n_q][kGroups][kIdxDim]
    const uint16_t* k_new;      // [n_q][kGroups][kHeadDim] bf16, or NULL
    const uint16_t* v_new;
    float* bs_part;
    int nblk;
    int32_t* arrive;            // [n_q][kGroups], zeroed here for the attention that follows
};

__global__ __launch_bounds__(64 * kFineWaves) void decode_step_fine_kernel(StepScanArgs a) {
    const int64_t i = blockIdx.x;
    const int b = blockIdx.y;
    const int sub = blockIdx.z;
    const int p = a.pos[i];
    const int s = a.stream[i];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4;
    const int c = lane & 15;
    constexpr int kTokPerWg = kFineWaves * kFineTokPerWave;                // 16
    const f32x4* new_row = reinterpret_cast<const f32x4*>(a.idx_k_new + i * kGroups * kIdxDim);
    if (b == 0 && sub == 0 && tid < kGroups) a.arrive[i * kGroups + tid] = 0;
    if (b == p / kBlock && sub == (p % kBlock) / kTokPerWg) {
        const int64_t slot = a.pg.row(s, p);
        if (tid < kGroups * kIdxDim / 4)   // 128 x 16 B
            reinterpret_cast<u32x4*>(a.idx_k + slot * kGroups * kIdxDim)[tid] =
                reinterpret_cast<const u32x4*>(new_row)[tid];
        if (tid < kGroups * kHeadDim / 8) {   // 64 x 16 B each
            if (a.k_new)
                reinterpret_cast<u32x4*>(a.k + slot * kGroups * kHeadDim)[tid] =
                    reinterpret_cast<const u32x4*>(a.k_new + i * kGroups * kHeadDim)[tid];
            if (a.v_new)
                reinterpret_cast<u32x4*>(a.v + slot * kGroups * kHeadDim)[tid] =
                    reinterpret_cast<const u32x4*>(a.v_new + i * kGroups * kHeadDim)[tid];
        }
    }
    float m = -INFINITY;
    const int t_begin = (sub * kFineWaves + wave) * kFineTokPerWave;
    const int t_end = min(t_begin + kFineTokPerWave, p - b * kBlock + 1);   // causal: tokens <= p
    if (t_begin < t_end) {
        const f32x4* qrow = reinterpret_cast<const f32x4*>(a.idx_q + i * kGroups * kIdxDim);
        const f32x4 q0 = qrow[g * 32 + c];
        const f32x4 q1 = qrow[g * 32 + 16 + c];
        const f32x4* rows = reinterpret_cast<const f32x4*>(
            a.idx_k + a.pg.block_row_uniform(s, b) * (kGroups * kIdxDim)) + g * 32 + c;
        f32x4 ka[kFineTokPerWave], kb[kFineTokPerWave];
        int tok[kFineTokPerWave];
#pragma unroll
        for (int u = 0; u < kFineTokPerWave; ++u) {
            tok[u] = b * kBlock + min(t_begin + u, t_end - 1);            // past the query: its last visible token again
            const f32x4* src = tok[u] == p ? new_row + g * 32 + c : rows + (tok[u] - b * kBlock) * kRowF4;
            ka[u] = __builtin_nontemporal_load(src);
            kb[u] = __builtin_nontemporal_load(src + 16);
        }
        // tokens of this wave that other queries of the launch append
        const int tok_lo = b * kBlock + t_begin, tok_hi = b * kBlock + t_end;   // [lo, hi)
        for (int64_t j0 = 0; j0 < a.n_q; j0 += 64) {
            const int64_t j = j0 + lane;
            bool hit = false;
            if (j < a.n_q && j != i && a.stream[j] == s) {
                const int pj = a.pos[j];
                hit = pj >= tok_lo && pj < tok_hi;
            }
            uint64_t mask = __builtin_amdgcn_ballot_w64(hit);
            while (mask) {                                               // wave-uniform
                const int64_t jj = j0 + __builtin_ctzll(mask);
                mask &= mask - 1;
                const int pj = a.pos[jj];
                const f32x4* src = reinterpret_cast<const f32x4*>(a.idx_k_new + jj * kGroups * kIdxDim) + g * 32 + c;
#pragma unroll
                for (int u = 0; u < kFineTokPerWave; ++u) {
                    if (tok[u] == pj) {
                        ka[u] = src[0];
                        kb[u] = src[16];
                    }
                }
            }
        }
#pragma unroll
        for (int u = 0; u < kFineTokPerWave; ++u) m = fmaxf(m, row16_sum(dot8(q0, q1, ka[u], kb[u])));
    }
    __shared__ float red[kFineWaves][kGroups];
    if (c == 0) red[wave][g] = m;
    __syncthreads();
    if (tid < kGroups) {
        float r = red[0][tid];
#pragma unroll
        for (int w = 1; w < kFineWaves; ++w) r = fmaxf(r, red[w][tid]);
        a.bs_part[((i * kGroups + tid) * a.nblk + b) * kFineSub + sub] = r;
    }
}

}  // namespace

bool scan_is_fine(int64_t n_q, int nblk) {
    return n_q * ((nblk + kScanBlocksPerWg - 1) / kScanBlocksPerWg) < kFineBelowWorkgroups;
}

hipError_t launch_block_scores_decode_fine(const CacheView& c, const float* idx_q, const int32_t* stream,
                                           const int32_t* pos, int64_t n_q, int nblk, float* bs_part,
                                           hipStream_t s) {
    hipLaunchKernelGGL(block_scores_decode_fine_kernel, dim3(static_cast<unsigned>(n_q), nblk, kFineSub),
                       dim3(64 * kFineWaves), 0, s, c.idx_k, c.pg, idx_q, stream, pos, bs_part, nblk);
    return hipGetLastError();
}

hipError_t launch_decode_step_fine(float* idx_k, uint16_t* k, uint16_t* v, const Pager& pg, const float* idx_q,
                                   const int32_t* stream, const int32_t* pos, int64_t n_q, int nblk,
                                   const float* idx_k_new, const uint16_t* k_new, const uint16_t* v_new,
                                   float* bs_part, int32_t* arrive, hipStream_t s) {
    StepScanArgs a{idx_k, k, v, pg, idx_q, stream, pos, n_q, idx_k_new, k_new, v_new, bs_part, nblk, arrive};
    hipLaunchKernelGGL(decode_step_fine_kernel, dim3(static_cast<unsigned>(n_q), nblk, kFineSub),
                       dim3(64 * kFineWaves), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_decode_step_scan(float* idx_k, uint16_t* k, uint16_t* v, const Pager& pg, const float* idx_q,
                                   const int32_t* stream, const int32_t* pos, int64_t n_q, int nblk,
                                   const float* idx_k_new, const uint16_t* k_new, const uint16_t* v_new,
                                   float* bs, hipStream_t s) {
    const unsigned ny = static_cast<unsigned>((nblk + kScanBlocksPerWg - 1) / kScanBlocksPerWg);
    hipLaunchKernelGGL(block_scores_decode_kernel<true>, dim3(static_cast<unsigned>(n_q), ny), dim3(64 * kScanWaves),
                       0, s, idx_k, pg, idx_q, stream, pos, bs, static_cast<int64_t>(nblk), nblk,
                       StepRows{idx_k, k, v, n_q, idx_k_new, k_new, v_new});
    return hipGetLastError();
}

hipError_t launch_block_scores_decode(const CacheView& c, const float* idx_q, const int32_t* stream,
                                      const int32_t* pos, int64_t n_q, int nblk, float* bs,
                                      int64_t nblk_stride, hipStream_t s) {
    const unsigned ny = static_cast<unsigned>((nblk + kScanBlocksPerWg - 1) / kScanBlocksPerWg);
    const unsigned ny16 = static_cast<unsigned>((nblk + kScan16BlocksPerWg - 1) / kScan16BlocksPerWg);
    if (c.idx_k16)
        hipLaunchKernelGGL(block_scores_decode_f16_kernel, dim3(static_cast<unsigned>(n_q), ny16),
                           dim3(64 * kScanWaves), 0, s, c.idx_k16, c.pg, idx_q, stream, pos, bs, nblk_stride, nblk);
    else
        hipLaunchKernelGGL(block_scores_decode_kernel<false>, dim3(static_cast<unsigned>(n_q), ny),
                           dim3(64 * kScanWaves), 0, s, c.idx_k, c.pg, idx_q, stream, pos, bs, nblk_stride, nblk,
                           StepRows{});
    return hipGetLastError();
}

}  // namespace msa
