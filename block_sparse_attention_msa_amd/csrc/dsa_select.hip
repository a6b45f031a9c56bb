// dsa_select.hip -- DSA lightning-indexer token selection.
//
// "deepseek2 : GLM-DSA sparse attention (lightning indexer), --dsa off by
// default", What this does: each query is scored against every (Hadamard-
// rotated, F16-cached) indexer key and keeps its top-k highest-scoring keys.
// Readings: one score per (query, key) = fp16 dot product accumulated in f32;
// keys j <= pos only; k = min(top_k, pos + 1); ties to the lower token id.
//
// Kernel 1 streams the fp16 key cache once with 128-bit loads (a 16-lane DPP
// row per 256-byte key row, v_dot2 on fp16 pairs) and writes the f32 scores.
// Its multi-head form (same pull request, review thread: one score per
// indexer head, an element-wise product with the head weights and a
// reduction over the heads before the top-k; the reduction is read as the
// lightning indexer's sum over heads of weight x ReLU(q_h . k)) contracts 16
// keys at a time against all heads on the fp16 matrix cores.
// Kernel 2 is an exact radix select on order-preserving u32 keys (digits of
// 12, 12 and 8 bits) that finds the k-th largest key T, then an order-
// preserving compaction writes every key > T and the lowest-id keys == T, so
// the output is already in ascending id order and unique.
#include "common.hpp"

namespace msa {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

constexpr int kScoreKeysPerWg = 1024;
constexpr int kScoreUnroll = 8;
constexpr int kSelThreads = 1024;

__device__ __forceinline__ float dot8_f16(const u32x4& q, const u32x4& k) {
    float d = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        // copy the element out first: a bit-cast of a vector-element lvalue
        // reads element 0 whatever the index
        const uint32_t qe = q[e], ke = k[e];
        d = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, qe), __builtin_bit_cast(half2_t, ke), d, false);
    }
    return d;
}

__global__ __launch_bounds__(256) void dsa_score_kernel(const uint16_t* __restrict__ dsa_k, Pager pg,
                                                        const uint16_t* __restrict__ q_idx,
                                                        const int32_t* __restrict__ q_stream,
                                                        const int32_t* __restrict__ q_pos,
                                                        float* __restrict__ scores, int64_t stride) {
    const int64_t i = blockIdx.y;
    const int p = q_pos[i];
    const int j_wg = blockIdx.x * kScoreKeysPerWg;
    if (j_wg > p) return;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform: scalar table reads
    const int r = lane >> 4;     // key row within a group of four
    const int c = lane & 15;     // 16-byte column (8 fp16 dims)
    const u32x4 q = *reinterpret_cast<const u32x4*>(q_idx + i * kIdxDim + 8 * c);
    const int64_t s = q_stream[i];
    float* out = scores + i * stride;
    const int j_begin = j_wg + wave * (kScoreKeysPerWg / 4);
    const int j_end = min(j_begin + kScoreKeysPerWg / 4, p + 1);
    static_assert(kBlock % (4 * kScoreUnroll) == 0, "an iteration's keys lie in one 128-key block");
    for (int j0 = j_begin; j0 < j_end; j0 += 4 * kScoreUnroll) {
        // keys j0 .. j0 + 31 (and p >= j0) share one block: one row lookup
        const int64_t rb = pg.block_row_uniform(s, j0 / kBlock);
        const int jb = j0 & ~(kBlock - 1);
        u32x4 kr[kScoreUnroll];
#pragma unroll
        for (int u = 0; u < kScoreUnroll; ++u) {
            int j = j0 + 4 * u + r;
            j = min(j, p);                                   // rows past p are never written
            kr[u] = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4*>(dsa_k + (rb + (j - jb)) * kIdxDim + 8 * c));
        }
#pragma unroll
        for (int u = 0; u < kScoreUnroll; ++u) {
            const float d = row16_sum(dot8_f16(q, kr[u]));
            const int j = j0 + 4 * u + r;
            if (c == 0 && j < j_end) out[j] = d;
        }
    }
}

// Multi-head scores, H = 16 * kTiles heads.  Per 16-key group a wave forms
// D[head][key] = Q K^T with v_mfma_f32_16x16x32_f16 (heads are the M side,
// keys the N side; four 32-dim slices per head tile), applies ReLU and the
// head weights to its 4 rows per tile in registers, and sums the heads with
// two cross-row swaps, after which every lane holds its key's score.  A lane
// reads 4 x 16 bytes of one key row (dims 32c + 8 * (lane / 16) ..), so one
// load instruction covers a contiguous 64-byte piece of 16 rows.  A wave
// walks 1024 keys, 64 (16 KiB) per step, with the next step's keys loading
// while the current step's products run (one workgroup of 4 waves per 4096
// keys of a query).  Measured on 16 x 65536 keys, 32 heads: 48 us, as fast as
// a plain read of the same 268 MB (45-50 us); shorter waves (64-512 keys) or
// no prefetch ran 49-60 us.
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
constexpr int kMhWaves = 4;
constexpr int kMhKeysPerWave = 1024;
constexpr int kMhKeysPerWg = kMhWaves * kMhKeysPerWave;
constexpr int kMhGroups = 4;                 // 16-key groups per step
constexpr int kMhStep = 16 * kMhGroups;
static_assert(kBlock % kMhStep == 0, "a step's keys lie in one 128-key block");

template <int kTiles>
__global__ __launch_bounds__(64 * kMhWaves) void dsa_score_heads_kernel(
    const uint16_t* __restrict__ dsa_k, Pager pg, const uint16_t* __restrict__ q_idx_h,
    const float* __restrict__ head_w, const int32_t* __restrict__ q_stream,
    const int32_t* __restrict__ q_pos, float* __restrict__ scores, int64_t stride) {
    constexpr int kHeads = 16 * kTiles;
    const int64_t i = blockIdx.y;
    const int p = q_pos[i];
    const int j_wg = blockIdx.x * kMhKeysPerWg;
    if (j_wg > p) return;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform: scalar table reads
    const int l16 = lane & 15;
    const int l4 = lane >> 4;
    // A operand: head 16t + l16, dims 32c + 8 * l4 .. + 7
    f16x8 qa[kTiles][4];
    // weights of the D rows this lane holds: heads 16t + 4 * l4 + r
    f32x4 wr[kTiles];
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
        const uint16_t* qh = q_idx_h + (i * kHeads + 16 * t + l16) * kIdxDim + 8 * l4;
#pragma unroll
        for (int c = 0; c < 4; ++c) qa[t][c] = *reinterpret_cast<const f16x8*>(qh + 32 * c);
        wr[t] = *reinterpret_cast<const f32x4*>(head_w + i * kHeads + 16 * t + 4 * l4);
    }
    const int64_t s = q_stream[i];
    float* out = scores + i * stride;
    const int j_begin = j_wg + wave * kMhKeysPerWave;
    const int j_end = min(j_begin + kMhKeysPerWave, p + 1);

    auto load = [&](f16x8 (&kb)[kMhGroups][4], int j0) __attribute__((always_inline)) {
        const int64_t rb = pg.block_row_uniform(s, j0 / kBlock);
        const int jb = j0 & ~(kBlock - 1);
#pragma unroll
        for (int u = 0; u < kMhGroups; ++u) {
            const int j = min(j0 + 16 * u + l16, p);           // rows past p are never written
            const f16x8* row = reinterpret_cast<const f16x8*>(dsa_k + (rb + (j - jb)) * kIdxDim + 8 * l4);
#pragma unroll
            for (int c = 0; c < 4; ++c) kb[u][c] = __builtin_nontemporal_load(row + 4 * c);
        }
    };
    auto compute = [&](const f16x8 (&kb)[kMhGroups][4], int j0) __attribute__((always_inline)) {
        float tot[kMhGroups];
#pragma unroll
        for (int u = 0; u < kMhGroups; ++u) {
            float acc = 0.f;
#pragma unroll
            for (int t = 0; t < kTiles; ++t) {
                f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int c = 0; c < 4; ++c) d = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[t][c], kb[u][c], d, 0, 0, 0);
#pragma unroll
                for (int r = 0; r < 4; ++r) acc = __builtin_fmaf(wr[t][r], fmaxf(d[r], 0.f), acc);
            }
            tot[u] = sum_xor32(sum_xor16(acc));               // all heads: key j0 + 16u + l16
        }
        // lane (l16, l4) writes key j0 + 16 * l4 + l16: 256 contiguous bytes
        float v = tot[0];
#pragma unroll
        for (int u = 1; u < kMhGroups; ++u) v = l4 == u ? tot[u] : v;
        const int j = j0 + 16 * l4 + l16;
        if (j < j_end) out[j] = v;
    };
    // Two register sets: the next step's keys load while this step computes.
    // Each branch holds its load and the products after it, so the wait
    // before the products leaves the prefetch in flight (a load issued on
    // one path only would make the wait at the join drain every load).
    if (j_begin >= j_end) return;
    f16x8 ka[kMhGroups][4], kn[kMhGroups][4];
    load(ka, j_begin);
    for (int j0 = j_begin;; j0 += 2 * kMhStep) {
        if (j0 + kMhStep < j_end) {
            load(kn, j0 + kMhStep);
            __builtin_amdgcn_sched_barrier(0);                // loads issued before the products
            compute(ka, j0);
        } else {
            compute(ka, j0);
            break;
        }
        if (j0 + 2 * kMhStep < j_end) {
            load(ka, j0 + 2 * kMhStep);
            __builtin_amdgcn_sched_barrier(0);
            compute(kn, j0 + kMhStep);
        } else {
            compute(kn, j0 + kMhStep);
            break;
        }
    }
}

// Inclusive prefix sum over the 1024 threads of the workgroup.
__device__ int block_inclusive_scan(int v, int* wave_sums) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(v, o, 64);
        if (lane >= o) v += y;
    }
    if (lane == 63) wave_sums[wave] = v;
    __syncthreads();
    if (wave == 0) {
        int sum = lane < kSelThreads / 64 ? wave_sums[lane] : 0;
#pragma unroll
        for (int o = 1; o < kSelThreads / 64; o <<= 1) {
            const int y = __shfl_up(sum, o, 64);
            if (lane >= o) sum += y;
        }
        if (lane < kSelThreads / 64) wave_sums[lane] = sum;
    }
    __syncthreads();
    if (wave > 0) v += wave_sums[wave - 1];
    __syncthreads();
    return v;
}

// Digits of the radix select, most significant first: 12 + 12 + 8 bits.
// Wide first digits spread the (exponent-concentrated) f32 scores over many
// histogram bins, which keeps LDS atomic collisions rare.
constexpr int kDigitBits[3] = {12, 12, 8};
constexpr int kBins = 4096;
constexpr int kBinsPerThread = kBins / kSelThreads;   // 4

// One workgroup of 1024 threads per query, three streaming passes over the
// query's scores (16-byte loads, coalesced across the workgroup):
//  1. histogram of the top 12 key bits -> the digit d1 of the top_k-th
//     largest key T, and how many keys equal to T's prefix are still needed;
//  2. the keys whose top 12 bits equal d1 (the boundary bin, typically ~1% of
//     the keys) are copied with their ids into an LDS candidate list, whose
//     remaining 12 + 8 bits are resolved there;
//  3. an order-preserving compaction in rounds of 16384 consecutive keys emits
//     every key > T and the lowest-id keys == T, ascending.
// A boundary bin larger than the LDS list (heavily tied scores) takes the
// general path, which re-reads the scores for the last two digits.
constexpr int kCandCap = 4096;

// Visits every score j < n as (j, ordered key).  Each thread issues four
// 16-byte loads per batch (j = 4 * (tid + 1024 * r) + c, coalesced across the
// workgroup) before using any of them.
constexpr int kBatch = 4;

template <typename F>
__device__ __forceinline__ void for_each_score(const float* t, int n, F&& f) {
    const int full = n & ~3;
    for (int base = 4 * threadIdx.x; base < full; base += 4 * kSelThreads * kBatch) {
        f32x4 x[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int j = base + 4 * kSelThreads * u;
            x[u] = j < full ? *reinterpret_cast<const f32x4*>(t + j) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int j = base + 4 * kSelThreads * u;
            if (j < full) {
                f(j, ordered_key(x[u].x));
                f(j + 1, ordered_key(x[u].y));
                f(j + 2, ordered_key(x[u].z));
                f(j + 3, ordered_key(x[u].w));
            }
        }
    }
    if (static_cast<int>(threadIdx.x) < n - full) f(full + threadIdx.x, ordered_key(t[full + threadIdx.x]));
}

// Finds the digit (bits `bits` wide) of the rank-`remaining` largest among
// the histogram counts; returns it through s_digit / s_remaining.
__device__ __forceinline__ void pick_digit(const int* hist, int bits, int remaining, int* wave_sums,
                                           uint32_t* s_digit, int* s_remaining) {
    const int nb = 1 << bits;
    int c[kBinsPerThread];
    int csum = 0;
#pragma unroll
    for (int e = 0; e < kBinsPerThread; ++e) {
        const int dd = kBinsPerThread * threadIdx.x + e;    // descending bin order
        c[e] = dd < nb ? hist[nb - 1 - dd] : 0;
        csum += c[e];
    }
    const int incl = block_inclusive_scan(csum, wave_sums);
    if (incl >= remaining && incl - csum < remaining) {
        int before = incl - csum;
#pragma unroll
        for (int e = 0; e < kBinsPerThread; ++e) {
            if (before + c[e] >= remaining) {
                *s_digit = static_cast<uint32_t>(nb - 1 - (kBinsPerThread * threadIdx.x + e));
                *s_remaining = remaining - before;
                break;
            }
            before += c[e];
        }
    }
    __syncthreads();
}

__global__ __launch_bounds__(kSelThreads) void dsa_topk_kernel(const float* __restrict__ scores,
                                                               int64_t stride,
                                                               const int32_t* __restrict__ q_pos,
                                                               int top_k, int32_t* __restrict__ sel,
                                                               int32_t* __restrict__ n_sel) {
    __shared__ int hist[kBins];
    __shared__ uint32_t cand_key[kCandCap];
    __shared__ int32_t cand_id[kCandCap];
    __shared__ int wave_sums[kSelThreads / 64];
    __shared__ uint32_t s_digit;
    __shared__ int s_remaining;
    __shared__ int s_ncand;
    const int64_t i = blockIdx.x;
    const int tid = threadIdx.x;
    const int n = q_pos[i] + 1;
    const float* t = scores + i * stride;
    int32_t* out = sel + i * top_k;
    if (n <= top_k) {                                   // every visible key is kept
        for (int j = tid; j < top_k; j += kSelThreads) out[j] = j < n ? j : -1;
        if (tid == 0) n_sel[i] = n;
        return;
    }
    // ---- pass 1: top 12 bits over all keys
    for (int b = tid; b < kBins; b += kSelThreads) hist[b] = 0;
    if (tid == 0) s_ncand = 0;
    __syncthreads();
    for_each_score(t, n, [&](int, uint32_t key) { atomicAdd(&hist[key >> 20], 1); });
    __syncthreads();
    pick_digit(hist, 12, top_k, wave_sums, &s_digit, &s_remaining);
    const uint32_t d1 = s_digit;
    int remaining = s_remaining;
    const int bin_count = hist[d1];
    uint32_t prefix = d1 << 20, mask = 0xfff00000u;
    __syncthreads();
    if (bin_count <= kCandCap) {
        // ---- pass 2: gather the boundary bin, resolve the low 20 bits in LDS
        for_each_score(t, n, [&](int j, uint32_t key) {
            if ((key & mask) == prefix) {
                const int slot = atomicAdd(&s_ncand, 1);
                cand_key[slot] = key;
                cand_id[slot] = j;
            }
        });
        __syncthreads();
        const int nc = s_ncand;
#pragma unroll
        for (int pass = 1; pass < 3; ++pass) {
            const int bits = kDigitBits[pass];
            const int shift = pass == 1 ? 8 : 0;
            const uint32_t dmask = (1u << bits) - 1;
            for (int b = tid; b < kBins; b += kSelThreads) hist[b] = 0;
            __syncthreads();
            for (int c = tid; c < nc; c += kSelThreads) {
                const uint32_t key = cand_key[c];
                if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & dmask], 1);
            }
            __syncthreads();
            pick_digit(hist, bits, remaining, wave_sums, &s_digit, &s_remaining);
            prefix |= s_digit << shift;
            mask |= dmask << shift;
            remaining = s_remaining;
            __syncthreads();
        }
    } else {
        // ---- general path: the last two digits over all keys
#pragma unroll
        for (int pass = 1; pass < 3; ++pass) {
            const int bits = kDigitBits[pass];
            const int shift = pass == 1 ? 8 : 0;
            const uint32_t dmask = (1u << bits) - 1;
            for (int b = tid; b < kBins; b += kSelThreads) hist[b] = 0;
            __syncthreads();
            for_each_score(t, n, [&](int, uint32_t key) {
                if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & dmask], 1);
            });
            __syncthreads();
            pick_digit(hist, bits, remaining, wave_sums, &s_digit, &s_remaining);
            prefix |= s_digit << shift;
            mask |= dmask << shift;
            remaining = s_remaining;
            __syncthreads();
        }
    }
    const uint32_t T = prefix;          // the top_k-th largest key; `remaining` keys equal to it are kept
    // ---- pass 3: order-preserving compaction; thread tid takes 16 consecutive
    // keys of each round of 16384
    constexpr int kPer = 16;
    int written = 0, eq_seen = 0;       // running totals over the rounds (uniform)
    for (int base = 0; base < n; base += kPer * kSelThreads) {
        const int j = base + kPer * tid;
        uint32_t key[kPer];
#pragma unroll
        for (int v = 0; v < kPer / 4; ++v) {
            const int jj = j + 4 * v;
            if (jj + 3 < n) {
                const f32x4 x = *reinterpret_cast<const f32x4*>(t + jj);
                key[4 * v] = ordered_key(x.x);
                key[4 * v + 1] = ordered_key(x.y);
                key[4 * v + 2] = ordered_key(x.z);
                key[4 * v + 3] = ordered_key(x.w);
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c) key[4 * v + c] = jj + c < n ? ordered_key(t[jj + c]) : 0u;
            }
        }
        int n_eq = 0;
#pragma unroll
        for (int c = 0; c < kPer; ++c) n_eq += (j + c < n) && key[c] == T;
        const int eq_incl = block_inclusive_scan(n_eq, wave_sums);
        int eq_rank = eq_seen + eq_incl - n_eq;      // equal keys before this thread's keys
        uint32_t take = 0;
        int n_take = 0;
#pragma unroll
        for (int c = 0; c < kPer; ++c) {
            const bool in = j + c < n;
            const bool eq = in && key[c] == T;
            const bool tk = (in && key[c] > T) || (eq && eq_rank < remaining);
            eq_rank += eq;
            take |= static_cast<uint32_t>(tk) << c;
            n_take += tk;
        }
        const int take_incl = block_inclusive_scan(n_take, wave_sums);
        int w = written + take_incl - n_take;
#pragma unroll
        for (int c = 0; c < kPer; ++c) {
            if ((take >> c) & 1) {
                if (w < top_k) out[w] = j + c;      // exactly top_k keys qualify; the bound is defensive
                ++w;
            }
        }
        // round totals: the last thread's inclusive values, via the scan's LDS
        if (tid == kSelThreads - 1) {
            wave_sums[0] = eq_incl;
            wave_sums[1] = take_incl;
        }
        __syncthreads();
        eq_seen += wave_sums[0];
        written += wave_sums[1];
        __syncthreads();
    }
    if (tid == 0) n_sel[i] = top_k;
}

int64_t score_stride(int32_t max_pos) {
    return ((static_cast<int64_t>(max_pos) + 1 + 63) / 64) * 64;
}

}  // namespace

size_t dsa_select_ws_bytes(int64_t n_q, int32_t max_pos) {
    return static_cast<size_t>(n_q) * score_stride(max_pos) * sizeof(float);
}

hipError_t launch_dsa_select(const uint16_t* dsa_k, const Pager& pg, const uint16_t* q_idx,
                             const int32_t* stream, const int32_t* pos, int64_t n_q,
                             int32_t max_pos, int top_k, int32_t* sel, int32_t* n_sel, void* ws,
                             hipStream_t s) {
    float* scores = static_cast<float*>(ws);
    const int64_t stride = score_stride(max_pos);
    const unsigned nx = static_cast<unsigned>((max_pos + kScoreKeysPerWg) / kScoreKeysPerWg);
    hipLaunchKernelGGL(dsa_score_kernel, dim3(nx, static_cast<unsigned>(n_q)), dim3(256), 0, s, dsa_k,
                       pg, q_idx, stream, pos, scores, stride);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(dsa_topk_kernel, dim3(static_cast<unsigned>(n_q)), dim3(kSelThreads), 0, s, scores,
                       stride, pos, top_k, sel, n_sel);
    return hipGetLastError();
}

hipError_t launch_dsa_select_heads(const uint16_t* dsa_k, const Pager& pg, const uint16_t* q_idx_h,
                                   const float* head_w, int n_head, const int32_t* stream,
                                   const int32_t* pos, int64_t n_q, int32_t max_pos, int top_k,
                                   int32_t* sel, int32_t* n_sel, void* ws, hipStream_t s) {
    float* scores = static_cast<float*>(ws);
    const int64_t stride = score_stride(max_pos);
    const dim3 grid(static_cast<unsigned>((max_pos + kMhKeysPerWg) / kMhKeysPerWg), static_cast<unsigned>(n_q));
    const dim3 block(64 * kMhWaves);
    switch (n_head) {
        case 16: hipLaunchKernelGGL(dsa_score_heads_kernel<1>, grid, block, 0, s, dsa_k, pg, q_idx_h, head_w,
                                    stream, pos, scores, stride); break;
        case 32: hipLaunchKernelGGL(dsa_score_heads_kernel<2>, grid, block, 0, s, dsa_k, pg, q_idx_h, head_w,
                                    stream, pos, scores, stride); break;
        case 48: hipLaunchKernelGGL(dsa_score_heads_kernel<3>, grid, block, 0, s, dsa_k, pg, q_idx_h, head_w,
                                    stream, pos, scores, stride); break;
        case 64: hipLaunchKernelGGL(dsa_score_heads_kernel<4>, grid, block, 0, s, dsa_k, pg, q_idx_h, head_w,
                                    stream, pos, scores, stride); break;
        default: return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(dsa_topk_kernel, dim3(static_cast<unsigned>(n_q)), dim3(kSelThreads), 0, s, scores,
                       stride, pos, top_k, sel, n_sel);
    return hipGetLastError();
}

}  // namespace msa
