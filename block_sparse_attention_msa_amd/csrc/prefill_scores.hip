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
//
// The keys are split once, by a pre-pass, into 512-byte rows [hi | lo] per
// (group, key) in the workspace; the GEMM kernel then copies them straight
// into LDS (global_load_lds, no registers, no conversion) through a ring of
// two 128-key stages while the matrix cores work on the previous stage.
// ---------------------------------------------------------------------------
constexpr int kScWaves = 8;
constexpr int kScThreads = 64 * kScWaves;
constexpr int kScSub = 2;                                   // 16-query sub-tiles per wave
constexpr int kScQueryTile = kScWaves * 16 * kScSub;        // 256 queries per workgroup
constexpr int kScBlocksPerWg = 16;                          // key range of a workgroup: 2048 keys
constexpr int kScStageKeys = 128;                           // keys per LDS stage
constexpr int kScRowBytes = 2 * kIdxDim * 2;                // one key's [hi | lo] row: 512 B
constexpr int kScStageBytes = kScStageKeys * kScRowBytes;   // 64 KiB
constexpr int kScCopies = kScStageBytes / 16 / kScThreads;  // 16-byte copies per thread and stage

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

// Rows are stored with their 16-byte segments permuted by seg ^ f(row & 15),
// f one-to-one on 16 rows, so the 16 rows an operand read touches at one
// segment fall in 16 different bank groups.
__device__ __forceinline__ int sc_rowperm(int row) { return ((row & 7) << 1) | ((row >> 3) & 1); }

__device__ __forceinline__ void split_bf16(float x, __bf16& hi, __bf16& lo) {
    hi = static_cast<__bf16>(x);
    lo = static_cast<__bf16>(x - static_cast<float>(hi));
}

// s_waitcnt immediate: at most n vector-memory operations of this wave
// outstanding (expcnt and lgkmcnt left at their maxima).
constexpr unsigned sc_waitcnt_vm(int n) {
    return static_cast<unsigned>((n & 15) | (((n >> 4) & 3) << 14) | (7 << 4) | (15 << 8));
}

// Barrier ordering LDS accesses only: copies into LDS still in flight are not
// waited for.
__device__ __forceinline__ void sc_lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);        // vmcnt 63, expcnt 7, lgkmcnt 0
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Pre-pass: keys 0 .. n_keys-1 of `stream` -> khl[g][key][0..127 hi, 128..255 lo],
// from the f32 index cache or (idx_k16 non-NULL) the fp16 one, whose values
// widen to f32 exactly.
__global__ __launch_bounds__(256) void split_keys_kernel(const float* __restrict__ idx_k,
                                                         const uint16_t* __restrict__ idx_k16, Pager pg,
                                                         int32_t stream, int64_t n_keys,
                                                         uint16_t* __restrict__ khl) {
    const int64_t n8 = n_keys * kGroups * (kIdxDim / 8);   // 8-key pieces
    for (int64_t e = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; e < n8;
         e += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        const int64_t key = e / (kGroups * (kIdxDim / 8));
        const int g = static_cast<int>((e / (kIdxDim / 8)) % kGroups);
        const int d8 = static_cast<int>(e % (kIdxDim / 8));
        const int64_t off = (pg.row(stream, static_cast<int>(key)) * kGroups + g) * kIdxDim + 8 * d8;
        f32x4 x0, x1;
        if (idx_k16) {
            typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
            const f16x8 h = __builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4*>(idx_k16 + off));
            x0 = f32x4{static_cast<float>(h[0]), static_cast<float>(h[1]), static_cast<float>(h[2]), static_cast<float>(h[3])};
            x1 = f32x4{static_cast<float>(h[4]), static_cast<float>(h[5]), static_cast<float>(h[6]), static_cast<float>(h[7])};
        } else {
            x0 = *reinterpret_cast<const f32x4*>(idx_k + off);
            x1 = *reinterpret_cast<const f32x4*>(idx_k + off + 4);
        }
        __bf16 h[8], l[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) split_bf16(c < 4 ? x0[c] : x1[c - 4], h[c], l[c]);
        uint16_t* row = khl + (static_cast<int64_t>(g) * n_keys + key) * (2 * kIdxDim);
        *reinterpret_cast<u32x4*>(row + 8 * d8) = __builtin_bit_cast(u32x4, h);
        *reinterpret_cast<u32x4*>(row + kIdxDim + 8 * d8) = __builtin_bit_cast(u32x4, l);
    }
}

struct ScArgs {
    const uint16_t* khl;   // [g][n_keys][256] bf16
    int64_t n_keys;
    const float* idx_q;
    int32_t pos0;
    int64_t n_q;
    int nblk;
    int n_ranges;
    float* bs;
    int64_t nblk_stride;
};

__global__ __launch_bounds__(kScThreads, 1) void block_scores_prefill_kernel(ScArgs a) {
    const int g = blockIdx.y;
    const int qtile = blockIdx.x / a.n_ranges;
    const int range = blockIdx.x % a.n_ranges;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l16 = lane & 15;
    const int l4 = lane >> 4;
    const int64_t q_first = static_cast<int64_t>(qtile) * kScQueryTile;   // query index
    const int64_t q_wave = q_first + wave * (16 * kScSub);
    const int b_begin = range * kScBlocksPerWg;
    const int b_end = min(b_begin + kScBlocksPerWg, a.nblk);
    const int64_t q_last_tile = (q_first + kScQueryTile < a.n_q ? q_first + kScQueryTile : a.n_q) - 1;
    const int max_pos_tile = a.pos0 + static_cast<int>(q_last_tile);

    // Blocks past every query of the tile: -inf (whole range or its tail).
    const int b_vis_end = min(b_end, max_pos_tile / kBlock + 1);
    {
        const int b0 = max(b_begin, b_vis_end);
        const int nb = b_end - b0;
        for (int idx = threadIdx.x; idx < kScQueryTile * nb; idx += kScThreads) {
            const int64_t qi = q_first + idx / nb;
            if (qi < a.n_q) a.bs[(qi * kGroups + g) * a.nblk_stride + b0 + idx % nb] = -INFINITY;
        }
    }
    if (b_begin >= b_vis_end) return;   // workgroup-uniform

    __shared__ __attribute__((aligned(16))) char sbuf0[kScStageBytes];
    __shared__ __attribute__((aligned(16))) char sbuf1[kScStageBytes];
    // the tile's block maxima, written to bs as one 64-byte row per query at
    // the end (a store per (query, block) would land 4 KiB from the next)
    __shared__ __attribute__((aligned(16))) float bs_tile[kScQueryTile][kScBlocksPerWg];
    for (int idx = threadIdx.x; idx < kScQueryTile * kScBlocksPerWg; idx += kScThreads)
        bs_tile[idx / kScBlocksPerWg][idx % kScBlocksPerWg] = -INFINITY;

    // Query operands (A: m = query, k = dim): lane holds query
    // q_wave + 16*st + l16, dims 32*ks + 8*l4 + 0..7, as hi and lo parts.
    bf16x8 qhi[kScSub][4], qlo[kScSub][4];
#pragma unroll
    for (int st = 0; st < kScSub; ++st) {
        const int64_t qn = q_wave + 16 * st + l16;
        const int64_t qi = qn < a.n_q ? qn : a.n_q - 1;
        const float* src = a.idx_q + (qi * kGroups + g) * kIdxDim + 8 * l4;
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
    const int qpos0 = a.pos0 + static_cast<int>(q_wave) + 4 * l4;
    const int wave_min_pos = a.pos0 + static_cast<int>(q_wave);

    const uint16_t* kg = a.khl + static_cast<int64_t>(g) * a.n_keys * (2 * kIdxDim);
    const int key_begin = b_begin * kBlock;
    const int key_end = min(b_vis_end * kBlock, max_pos_tile + 1);   // keys past it are invisible
    // an even number of stages, so the two buffers alternate in a loop with
    // no conditional copies or waits (a stage past key_end copies the last
    // visible key and is fully masked; the loop's last two copies refill
    // buffers nobody reads again)
    int n_stages = (key_end - key_begin + kScStageKeys - 1) / kScStageKeys;
    n_stages += n_stages & 1;

    // B operand offsets (k = dim, n = key): key row 16*kt + l16, hi segment
    // 4*ks + l4 (dims 32*ks + 8*l4 ..), lo segment 16 + 4*ks + l4.
    const int rp = sc_rowperm(l16);
    int hoff[4], loff[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        hoff[ks] = l16 * kScRowBytes + (((4 * ks + l4) ^ rp) << 4);
        loff[ks] = l16 * kScRowBytes + (((16 + 4 * ks + l4) ^ rp) << 4);
    }
    // Copies of stage s: slot c = 256*j + thread holds segment (c % 32) ^ f(row)
    // of key row c / 32.
    auto stage = [&](int s_idx, char* dst) {
        const int kb = key_begin + s_idx * kScStageKeys;
#pragma unroll
        for (int j = 0; j < kScCopies; ++j) {
            const int c = kScThreads * j + static_cast<int>(threadIdx.x);
            const int row = c >> 5;
            const int seg = (c & 31) ^ sc_rowperm(row);
            const int key = min(kb + row, key_end - 1);
            __builtin_amdgcn_global_load_lds(kg + static_cast<int64_t>(key) * (2 * kIdxDim) + 8 * seg,
                                             LDS_PTR(void, dst + (kScThreads * j + 64 * wave) * 16), 16, 0, 0);
        }
    };

    f32x4 blkmax[kScSub];
#pragma unroll
    for (int st = 0; st < kScSub; ++st) blkmax[st] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};

    // B operands of one 16-key tile: hi and lo parts for the four dim steps
    auto load_b = [&](const char* sb, int kt, bf16x8 (&bh)[4], bf16x8 (&bl)[4]) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            bh[ks] = *reinterpret_cast<const bf16x8*>(sb + 16 * kt * kScRowBytes + hoff[ks]);
            bl[ks] = *reinterpret_cast<const bf16x8*>(sb + 16 * kt * kScRowBytes + loff[ks]);
        }
    };
    auto compute = [&](int s_idx, const char* sb) {
        const int kb = key_begin + s_idx * kScStageKeys;
        bf16x8 bh[2][4], bl[2][4];                 // this tile's operands and the next one's
        load_b(sb, 0, bh[0], bl[0]);
#pragma unroll
        for (int kt = 0; kt < kScStageKeys / 16; ++kt) {
            if (kt + 1 < kScStageKeys / 16) load_b(sb, kt + 1, bh[(kt + 1) & 1], bl[(kt + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);     // the next tile's reads stay ahead of these products
            // one accumulation chain per (sub-tile, product), issued round
            // robin, so that consecutive products never wait on each other
            f32x4 acc3[3][kScSub];
#pragma unroll
            for (int pr = 0; pr < 3; ++pr)
#pragma unroll
                for (int st = 0; st < kScSub; ++st) acc3[pr][st] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const bf16x8 bhi = bh[kt & 1][ks];
                const bf16x8 blo = bl[kt & 1][ks];
#pragma unroll
                for (int st = 0; st < kScSub; ++st) acc3[0][st] = mfma_16x16x32_bf16(qhi[st][ks], bhi, acc3[0][st]);
#pragma unroll
                for (int st = 0; st < kScSub; ++st) acc3[1][st] = mfma_16x16x32_bf16(qhi[st][ks], blo, acc3[1][st]);
#pragma unroll
                for (int st = 0; st < kScSub; ++st) acc3[2][st] = mfma_16x16x32_bf16(qlo[st][ks], bhi, acc3[2][st]);
            }
            f32x4 acc[kScSub];
#pragma unroll
            for (int st = 0; st < kScSub; ++st) acc[st] = acc3[0][st] + (acc3[1][st] + acc3[2][st]);
            const int key = kb + 16 * kt + l16;
            const int tile_last = kb + 16 * kt + 15;
            if (tile_last <= wave_min_pos && tile_last < key_end) {   // wave-uniform: no masking
#pragma unroll
                for (int st = 0; st < kScSub; ++st)
#pragma unroll
                    for (int r = 0; r < 4; ++r) blkmax[st][r] = fmaxf(blkmax[st][r], acc[st][r]);
            } else {
#pragma unroll
                for (int st = 0; st < kScSub; ++st)
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
                for (int st = 0; st < kScSub; ++st) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float mx = row16_max(blkmax[st][r]);
                        if (l16 == r) bs_tile[wave * 16 * kScSub + 16 * st + 4 * l4 + r][b - b_begin] = mx;
                        blkmax[st][r] = -INFINITY;
                    }
                }
            }
        }
    };

    // Two-stage ring: stage s + 1 streams in while stage s is computed.
    stage(0, sbuf0);
    stage(1, sbuf1);
    for (int s_idx = 0; s_idx < n_stages; s_idx += 2) {
        __builtin_amdgcn_s_waitcnt(sc_waitcnt_vm(kScCopies));
        sc_lds_barrier();                          // stage s is in LDS
        compute(s_idx, sbuf0);
        sc_lds_barrier();                          // every wave is done with buffer 0
        stage(s_idx + 2, sbuf0);
        __builtin_amdgcn_s_waitcnt(sc_waitcnt_vm(kScCopies));
        sc_lds_barrier();                          // stage s + 1 is in LDS
        compute(s_idx + 1, sbuf1);
        sc_lds_barrier();
        stage(s_idx + 3, sbuf1);
    }
    __builtin_amdgcn_s_waitcnt(sc_waitcnt_vm(0));   // the last two copies land before the exit
    __syncthreads();
    // blocks b_begin .. b_vis_end - 1 of the tile's queries (the rest was
    // written as -inf above): a thread writes 4 consecutive blocks of a query
    const int nbv = b_vis_end - b_begin;
    for (int idx = threadIdx.x; idx < kScQueryTile * (kScBlocksPerWg / 4); idx += kScThreads) {
        const int ql = idx / (kScBlocksPerWg / 4);
        const int b4 = 4 * (idx % (kScBlocksPerWg / 4));
        const int64_t qi = q_first + ql;
        if (qi >= a.n_q || b4 >= nbv) continue;
        float* dst = a.bs + (qi * kGroups + g) * a.nblk_stride + b_begin + b4;
        if (b4 + 4 <= nbv && (reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
            *reinterpret_cast<f32x4*>(dst) = *reinterpret_cast<const f32x4*>(&bs_tile[ql][b4]);
        } else {
            for (int e = 0; e < 4 && b4 + e < nbv; ++e) dst[e] = bs_tile[ql][b4 + e];
        }
    }
}

}  // namespace

size_t prefill_scores_ws_bytes(int32_t max_pos) {
    return static_cast<size_t>(max_pos + 1) * kGroups * kScRowBytes;
}

hipError_t launch_block_scores_prefill(const CacheView& c, const float* idx_q, int32_t stream,
                                       int32_t pos0, int64_t n_q, int nblk, float* bs,
                                       int64_t nblk_stride, void* ws, hipStream_t s) {
    const int64_t n_keys = pos0 + n_q;             // keys 0 .. pos0 + n_q - 1
    uint16_t* khl = static_cast<uint16_t*>(ws);
    const int64_t n8 = n_keys * kGroups * (kIdxDim / 8);
    const int64_t want = (n8 + 255) / 256;
    const unsigned split_grid = static_cast<unsigned>(want < 8192 ? want : 8192);
    hipLaunchKernelGGL(split_keys_kernel, dim3(split_grid), dim3(256), 0, s, c.idx_k, c.idx_k16, c.pg, stream,
                       n_keys, khl);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    ScArgs a;
    a.khl = khl;
    a.n_keys = n_keys;
    a.idx_q = idx_q;
    a.pos0 = pos0;
    a.n_q = n_q;
    a.nblk = nblk;
    a.n_ranges = (nblk + kScBlocksPerWg - 1) / kScBlocksPerWg;
    a.bs = bs;
    a.nblk_stride = nblk_stride;
    const int n_qtiles = static_cast<int>((n_q + kScQueryTile - 1) / kScQueryTile);
    hipLaunchKernelGGL(block_scores_prefill_kernel, dim3(n_qtiles * a.n_ranges, kGroups), dim3(kScThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace msa
